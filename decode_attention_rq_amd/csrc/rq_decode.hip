// rq_decode.hip -- decode launches for a BF16 reference, the split/tail
// merge kernel, and the dispatch over reference kinds (gfx950).  The kernel
// template and its description are in rq_decode_kernel.hpp.

#include "rq_decode_kernel.hpp"

namespace rq {

// Kernel M: one workgroup per (batch*head, loop slot).  Its waves share the
// BF16 tail of the slot's loop (original domain) with the decode kernel's
// lane mapping: D/8 lanes per row, 8 dims per lane, 64/(D/8) rows side by
// side, kTailRows rows per lane per batch (one 128-bit load per row and
// lane, row sums by DPP inside the row's lanes, no LDS traffic).  Every lane
// keeps the online softmax of its row; rows, then waves (through LDS), are
// merged by log-sum-exp.  Wave 0 then merges the splits' records with the
// tail state and finishes the row.
constexpr int kTailRows = 4;
constexpr int kMergeWaves = 4;
// Split records read per batch of loads: the merge issues the loads of this
// many records before it uses any of them, so a merge over S records waits
// for ceil(S / kRecBatch) memory round trips, not S.
constexpr int kRecBatch = 8;

template <int D>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(const DecodeArgs a, int n_res) {
  constexpr int E = D / 64;
  constexpr int REC = 2 * D + 2;
  constexpr int LANES = D / 8;                 // lanes per tail row
  constexpr int ROWS = kWave / LANES;          // rows side by side in a wave
  const int bh = blockIdx.x, s = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const bool residual = s < n_res;
  if (!((a.out_mask >> a.qloop[s]) & 1u)) return;   // a chain link computed, not asked for

  // split records of this (slot, batch*head): their maximum, and the first
  // batch of records, are loaded before the tail walk so that those loads
  // overlap it
  const size_t stride = (size_t)kMaxSlots * a.bh * REC;
  const float *rec0 = a.ws + ((size_t)s * a.bh + bh) * REC;
  float M = -FLT_MAX;
  float rm[kRecBatch], rl[kRecBatch], ro[kRecBatch][E], rr[kRecBatch][E];
  // records [sp0, sp0 + kRecBatch) into rm/rl/ro/rr; indices past the last
  // record re-read the last one (and are not used)
  auto load_recs = [&](int sp0) {
#pragma unroll
    for (int i = 0; i < kRecBatch; ++i) {
      const float *rec = rec0 + (size_t)min(sp0 + i, a.n_splits - 1) * stride;
      rm[i] = rec[0];
      rl[i] = rec[1];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ro[i][e] = rec[2 + lane + 64 * e];
        rr[i][e] = residual ? rec[2 + D + lane + 64 * e] : 0.0f;
      }
    }
  };
  if (wave == 0) {
    for (int sp = lane; sp < a.n_splits; sp += 64) M = fmaxf(M, rec0[sp * stride]);
    if (a.n_splits > 0) load_recs(0);    // none when only the tail is attended
  }

  float mt = -FLT_MAX, lt = 0.0f, ot[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ot[e] = 0.0f;
  if (a.n_tail > 0) {
    const int j = lane % LANES, r = lane / LANES;
    const uint16_t *tk = a.tk[s] + (size_t)bh * a.tcap * D;
    const uint16_t *tv = a.tv[s] + (size_t)bh * a.tcap * D;
    const uint4 qw = *reinterpret_cast<const uint4 *>(a.q + ((size_t)a.qloop[s] * a.bh + bh) * D + 8 * j);
    float o8[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) o8[p] = 0.0f;
    for (int t0 = wave * ROWS * kTailRows; t0 < a.n_tail; t0 += nw * ROWS * kTailRows) {
      uint4 kw[kTailRows], vw[kTailRows];
#pragma unroll
      for (int i = 0; i < kTailRows; ++i) {
        const uint32_t t = (uint32_t)min(t0 + i * ROWS + r, a.n_tail - 1);
        kw[i] = ldg_nt<uint4>(tk, t * (2 * D) + 16 * j);
        vw[i] = ldg_nt<uint4>(tv, t * (2 * D) + 16 * j);
      }
      float sc[kTailRows];
      float mb = -FLT_MAX;
#pragma unroll
      for (int i = 0; i < kTailRows; ++i) {
        float dp = dot2bf0(qw.x, kw[i].x);
        dp = dot2bf(qw.y, kw[i].y, dp);
        dp = dot2bf(qw.z, kw[i].z, dp);
        dp = dot2bf(qw.w, kw[i].w, dp);
        sc[i] = group_sum_dpp<LANES>(dp) * a.qscale;
        if (t0 + i * ROWS + r >= a.n_tail) sc[i] = -INFINITY;
        mb = fmaxf(mb, sc[i]);
      }
      if (mb > mt) {
        const float f = fexp2(mt - mb);
        lt *= f;
#pragma unroll
        for (int p = 0; p < 8; ++p) o8[p] *= f;
        mt = mb;
      }
#pragma unroll
      for (int i = 0; i < kTailRows; ++i) {
        const float pw = fexp2(sc[i] - mt);
        lt += pw;
        const uint32_t w4[4] = {vw[i].x, vw[i].y, vw[i].z, vw[i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          o8[2 * c] = __builtin_fmaf(pw, bf16lo(w4[c]), o8[2 * c]);
          o8[2 * c + 1] = __builtin_fmaf(pw, bf16hi(w4[c]), o8[2 * c + 1]);
        }
      }
    }
    // rows of the wave (lane distances LANES, 2 LANES, ...), then waves
    auto merge_with = [&](float mo, float lo, const float (&oo)[8]) {
      const float Mx = fmaxf(mt, mo);
      const float fa = fexp2(mt - Mx), fb = fexp2(mo - Mx);
      lt = lt * fa + lo * fb;
#pragma unroll
      for (int p = 0; p < 8; ++p) o8[p] = o8[p] * fa + oo[p] * fb;
      mt = Mx;
    };
    auto merge_lanes = [&](auto mask_t) {
      constexpr int MASK = decltype(mask_t)::value;
      float oo[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) oo[p] = xor_lane<MASK>(o8[p]);
      merge_with(xor_lane<MASK>(mt), xor_lane<MASK>(lt), oo);
    };
    if constexpr (ROWS >= 2) merge_lanes(std::integral_constant<int, LANES>{});
    if constexpr (ROWS >= 4) merge_lanes(std::integral_constant<int, LANES * 2>{});
    if constexpr (ROWS >= 8) merge_lanes(std::integral_constant<int, LANES * 4>{});
    __shared__ float sm[kMergeWaves][2 + D];
    if (r == 0) {
      if (j == 0) { sm[wave][0] = mt; sm[wave][1] = lt; }
#pragma unroll
      for (int p = 0; p < 8; ++p) sm[wave][2 + 8 * j + p] = o8[p];
    }
    __syncthreads();
    if (wave != 0) return;
    mt = sm[0][0];
    for (int w = 1; w < nw; ++w) mt = fmaxf(mt, sm[w][0]);
    lt = 0.0f;
    for (int w = 0; w < nw; ++w) {
      const float f = fexp2(sm[w][0] - mt);
      lt = __builtin_fmaf(f, sm[w][1], lt);
#pragma unroll
      for (int e = 0; e < E; ++e) ot[e] = __builtin_fmaf(f, sm[w][2 + lane + 64 * e], ot[e]);
    }
  }

  M = group_max<64>(M);
  const float Mall = fmaxf(M, mt);

  float L = 0.0f, o[E], q[E];
#pragma unroll
  for (int e = 0; e < E; ++e) { o[e] = 0.0f; q[e] = 0.0f; }
  for (int sp0 = 0;;) {
#pragma unroll
    for (int i = 0; i < kRecBatch; ++i) {
      if (sp0 + i < a.n_splits) {
        const float f = fexp2(rm[i] - Mall);
        L = __builtin_fmaf(f, rl[i], L);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          o[e] = __builtin_fmaf(f, ro[i][e], o[e]);
          q[e] = __builtin_fmaf(f, rr[i][e], q[e]);
        }
      }
    }
    sp0 += kRecBatch;
    if (sp0 >= a.n_splits) break;
    load_recs(sp0);
  }
  const float ft = fexp2(mt - Mall);
  L = __builtin_fmaf(ft, lt, L);
#pragma unroll
  for (int e = 0; e < E; ++e) ot[e] *= ft;
  finish_row<D>(a, bh, s, residual, lane, L, o, q, ot);
}

hipError_t launch_merge(const DecodeArgs &a, int head_dim, int n_res, int n_slots, hipStream_t st) {
  // one wave unless there is a tail to share out
  const dim3 grid(a.bh, n_slots), block(a.n_tail > 0 ? 64 * kMergeWaves : 64);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(decode_merge_kernel<64>, grid, block, 0, st, a, n_res); break;
    case 128: hipLaunchKernelGGL(decode_merge_kernel<128>, grid, block, 0, st, a, n_res); break;
    case 256: hipLaunchKernelGGL(decode_merge_kernel<256>, grid, block, 0, st, a, n_res); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Instantiated in rq_decode_inst.hip, one object file per combination.
#define RQ_DECODE_EXTERN(D, AQ, CHAIN) \
  extern template hipError_t launch_decode_d<D, AQ, CHAIN>(const DecodeArgs &, int, bool, hipStream_t);
#define RQ_DECODE_EXTERN_D(AQ, CHAIN) \
  RQ_DECODE_EXTERN(64, AQ, CHAIN) RQ_DECODE_EXTERN(128, AQ, CHAIN) RQ_DECODE_EXTERN(256, AQ, CHAIN)
RQ_DECODE_EXTERN_D(0, 0)
RQ_DECODE_EXTERN_D(2, 0)
RQ_DECODE_EXTERN_D(4, 0)
RQ_DECODE_EXTERN_D(0, 1)
RQ_DECODE_EXTERN_D(4, 1)
RQ_DECODE_EXTERN_D(0, 2)
RQ_DECODE_EXTERN_D(4, 2)
extern template int decode_blocks_per_cu_d<64>();
extern template int decode_blocks_per_cu_d<128>();
extern template int decode_blocks_per_cu_d<256>();

int decode_blocks_per_cu(int head_dim) {
  switch (head_dim) {
    case 64: return decode_blocks_per_cu_d<64>();
    case 128: return decode_blocks_per_cu_d<128>();
    case 256: return decode_blocks_per_cu_d<256>();
    default: return -1;
  }
}

// One decode pass with reference kind AQ (0: BF16 rows; 2, 4: anchor bits),
// chained references or not.
template <int AQ, int CHAIN>
static hipError_t launch_decode_aq(const DecodeArgs &a, int head_dim, int n_res, bool ref, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_decode_d<64, AQ, CHAIN>(a, n_res, ref, st);
    case 128: return launch_decode_d<128, AQ, CHAIN>(a, n_res, ref, st);
    case 256: return launch_decode_d<256, AQ, CHAIN>(a, n_res, ref, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs &a, int head_dim, int n_res, bool ref, int anchor_bits,
                         int chain, hipStream_t st) {
  if (chain == 1 || chain == 2) {
    switch (anchor_bits) {
      case 0: return chain == 1 ? launch_decode_aq<0, 1>(a, head_dim, n_res, ref, st)
                                : launch_decode_aq<0, 2>(a, head_dim, n_res, ref, st);
      case 4: return chain == 1 ? launch_decode_aq<4, 1>(a, head_dim, n_res, ref, st)
                                : launch_decode_aq<4, 2>(a, head_dim, n_res, ref, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (chain != 0) return hipErrorInvalidValue;
  switch (anchor_bits) {
    case 0: return launch_decode_aq<0, 0>(a, head_dim, n_res, ref, st);
    case 2: return launch_decode_aq<2, 0>(a, head_dim, n_res, ref, st);
    case 4: return launch_decode_aq<4, 0>(a, head_dim, n_res, ref, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rq
