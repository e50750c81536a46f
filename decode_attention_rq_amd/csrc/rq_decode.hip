// rq_decode.hip -- decode launches for a BF16 reference, the split/tail
// merge kernel, and the dispatch over reference kinds (gfx950).  The kernel
// template and its description are in rq_decode_kernel.hpp.

#include "rq_decode_kernel.hpp"

namespace rq {

// Kernel M: one workgroup per (batch*head, loop slot).  Its waves share the
// BF16 tail of the slot's loop (original domain): each wave takes batches of
// kTailBatch tokens (loads issued together, reductions interleaved) with its
// own online softmax; the waves' states meet in LDS.  Wave 0 then merges the
// splits' records with the tail state by log-sum-exp and finishes the row.
constexpr int kTailBatch = 16;
constexpr int kMergeWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(const DecodeArgs a, int n_res) {
  constexpr int E = D / 64;
  constexpr int REC = 2 * D + 2;
  const int bh = blockIdx.x, s = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const bool residual = s < n_res;
  if (!((a.out_mask >> a.qloop[s]) & 1u)) return;   // a chain link computed, not asked for

  // split records of this (slot, batch*head): their maximum first, so the
  // record loads overlap the tail walk
  const size_t stride = (size_t)kMaxSlots * a.bh * REC;
  const float *rec0 = a.ws + ((size_t)s * a.bh + bh) * REC;
  float M = -FLT_MAX;
  if (wave == 0)
    for (int sp = lane; sp < a.n_splits; sp += 64) M = fmaxf(M, rec0[sp * stride]);

  float mt = -FLT_MAX, lt = 0.0f, ot[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ot[e] = 0.0f;
  if (a.n_tail > 0) {
    const uint16_t *qrow = a.q + ((size_t)a.qloop[s] * a.bh + bh) * D;
    const uint16_t *tk = a.tk[s] + (size_t)bh * a.tcap * D;
    const uint16_t *tv = a.tv[s] + (size_t)bh * a.tcap * D;
    float qv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) qv[e] = bf16lo(qrow[lane + 64 * e]);
    for (int t0 = wave * kTailBatch; t0 < a.n_tail; t0 += nw * kTailBatch) {
      float kk[kTailBatch][E], vv[kTailBatch][E];
#pragma unroll
      for (int i = 0; i < kTailBatch; ++i) {
        const size_t row = (size_t)min(t0 + i, a.n_tail - 1) * D;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          kk[i][e] = bf16lo(tk[row + lane + 64 * e]);
          vv[i][e] = bf16lo(tv[row + lane + 64 * e]);
        }
      }
      float sc[kTailBatch];
#pragma unroll
      for (int i = 0; i < kTailBatch; ++i) {
        float dp = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) dp = __builtin_fmaf(qv[e], kk[i][e], dp);
        sc[i] = group_sum<64>(dp) * a.qscale;
      }
      float mb = -FLT_MAX;
#pragma unroll
      for (int i = 0; i < kTailBatch; ++i) {
        if (t0 + i >= a.n_tail) sc[i] = -INFINITY;
        mb = fmaxf(mb, sc[i]);
      }
      if (mb > mt) {
        const float f = fexp2(mt - mb);
        lt *= f;
#pragma unroll
        for (int e = 0; e < E; ++e) ot[e] *= f;
        mt = mb;
      }
#pragma unroll
      for (int i = 0; i < kTailBatch; ++i) {
        const float p = fexp2(sc[i] - mt);
        lt += p;
#pragma unroll
        for (int e = 0; e < E; ++e) ot[e] = __builtin_fmaf(p, vv[i][e], ot[e]);
      }
    }
  }
  __shared__ float sm[kMergeWaves][2 + D];
  if (nw > 1) {
    if (lane == 0) { sm[wave][0] = mt; sm[wave][1] = lt; }
#pragma unroll
    for (int e = 0; e < E; ++e) sm[wave][2 + lane + 64 * e] = ot[e];
    __syncthreads();
    if (wave != 0) return;
    mt = sm[0][0];
    for (int w = 1; w < nw; ++w) mt = fmaxf(mt, sm[w][0]);
    lt = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) ot[e] = 0.0f;
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
  for (int sp = 0; sp < a.n_splits; ++sp) {
    const float *rec = rec0 + sp * stride;
    const float f = fexp2(rec[0] - Mall);
    L = __builtin_fmaf(f, rec[1], L);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(f, rec[2 + lane + 64 * e], o[e]);
    if (residual) {
#pragma unroll
      for (int e = 0; e < E; ++e) q[e] = __builtin_fmaf(f, rec[2 + D + lane + 64 * e], q[e]);
    }
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

template <int D>
static int blocks_per_cu_d() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, decode_kernel<D, kMaxRes, true, 0, kTilesPerIter, kWaves, 0, false>, 64 * kWaves, 0) != hipSuccess)
    return -1;
  return n;
}

int decode_blocks_per_cu(int head_dim) {
  switch (head_dim) {
    case 64: return blocks_per_cu_d<64>();
    case 128: return blocks_per_cu_d<128>();
    case 256: return blocks_per_cu_d<256>();
    default: return -1;
  }
}

template hipError_t launch_decode_aq<0, false>(const DecodeArgs &, int, int, bool, hipStream_t);
// instantiated in rq_decode_anchor{2,4}.hip and rq_decode_chain{0,4}.hip
extern template hipError_t launch_decode_aq<2, false>(const DecodeArgs &, int, int, bool, hipStream_t);
extern template hipError_t launch_decode_aq<4, false>(const DecodeArgs &, int, int, bool, hipStream_t);
extern template hipError_t launch_decode_aq<0, true>(const DecodeArgs &, int, int, bool, hipStream_t);
extern template hipError_t launch_decode_aq<4, true>(const DecodeArgs &, int, int, bool, hipStream_t);

hipError_t launch_decode(const DecodeArgs &a, int head_dim, int n_res, bool ref, int anchor_bits,
                         bool chain, hipStream_t st) {
  if (chain) {
    switch (anchor_bits) {
      case 0: return launch_decode_aq<0, true>(a, head_dim, n_res, ref, st);
      case 4: return launch_decode_aq<4, true>(a, head_dim, n_res, ref, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (anchor_bits) {
    case 0: return launch_decode_aq<0, false>(a, head_dim, n_res, ref, st);
    case 2: return launch_decode_aq<2, false>(a, head_dim, n_res, ref, st);
    case 4: return launch_decode_aq<4, false>(a, head_dim, n_res, ref, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rq
