// rq_decode.hip -- fused decode attention over a ResidualQuant cache (gfx950).
//
// ResidualQuant page ("ResidualQuant: KV Cache Quantization for Looped
// Transformers with 2-Bit Residuals"), Abstract: decode reads each loop's
// compressed cache (BF16 reference + low-bit residual) and the smaller
// traffic is what speeds it up.  For loop l and token t, with y the
// reference vector and u = z + s*code the rotated, quantized residual:
//   key    k_t = aK_t y_t + H_n u_t        value  v_t = aV_t y_t + H_n u'_t
// Because H_n is symmetric and orthonormal the rotation is folded:
//   q . k_t      = aK_t (q . y_t) + sum_k [ s_k (q'_k . code_k) + z_k sum(q'_k) ]
//   sum_t p_t v_t = sum_t (p_t aV_t) y_t + H_n sum_t p_t u'_t
// with q' = H_n q, so the per-token work is the reference dot product, the
// code dot products and FMA accumulation; H_n is applied once per output.
//
// One kernel per call (per pass of up to three residual loops): a workgroup
// per (token split, batch*head); 4 waves, each taking every 4th tile of
// ROWS*TR tokens.  Lanes: D/8 lanes per token, 8 consecutive dims per lane,
// ROWS = 64/(D/8) tokens side by side, so one 128-bit load per lane reads ROWS
// consecutive reference rows, and every loop of the pass shares that load.
// Online softmax per (row, loop) in the exp2 domain; rows, then waves
// (through LDS), are merged by log-sum-exp into one record per (split, loop,
// batch*head) in the workspace.  The last workgroup of a batch*head to finish
// (an atomic counter in the workspace, reset by that workgroup) merges the
// splits, un-rotates the residual accumulator and normalises.

#include <float.h>

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
__device__ __forceinline__ void merge_splits(const DecodeArgs &a, int bh, int s, bool residual, int lane);

// Merge the online-softmax states of rows at lane distance MASK.
template <int MASK, int NS, int NR>
__device__ __forceinline__ void merge_rows(float (&m)[NS], float (&l)[NS], float (&oref)[NS][8],
                                           float (&ores)[NR > 0 ? NR : 1][8]) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float mo = xor_lane<MASK>(m[s]);
    const float M = fmaxf(m[s], mo);
    const float fa = fexp2(m[s] - M), fb = fexp2(mo - M);
    l[s] = l[s] * fa + xor_lane<MASK>(l[s]) * fb;
#pragma unroll
    for (int p = 0; p < 8; ++p) oref[s][p] = oref[s][p] * fa + xor_lane<MASK>(oref[s][p]) * fb;
    if (s < NR) {
#pragma unroll
      for (int p = 0; p < 8; ++p) ores[s][p] = ores[s][p] * fa + xor_lane<MASK>(ores[s][p]) * fb;
    }
    m[s] = M;
  }
}

template <int D, int NR, bool REF, int TR>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
  constexpr int LANES = D / 8;
  constexpr int ROWS = kWave / LANES;
  constexpr int NS = NR + (REF ? 1 : 0);
  constexpr int NRA = NR > 0 ? NR : 1;
  constexpr int TILE = ROWS * TR;
  constexpr int REC = 2 * D + 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane % LANES, r = lane / LANES;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int t_begin = split * a.tps;
  const int t_end = min(t_begin + a.tps, a.n_ctx);
  const int gl = a.group / 8;
  const int G = D / a.group;
  const int k = j / gl;

  // ---- prologue: queries of every loop in the pass -------------------------
  uint32_t qb[NS][4];
  float qr[NRA][8], sig[NRA];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint4 w = *reinterpret_cast<const uint4 *>(a.q + ((size_t)a.qloop[s] * a.bh + bh) * D + 8 * j);
    qb[s][0] = w.x; qb[s][1] = w.y; qb[s][2] = w.z; qb[s][3] = w.w;
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float f[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) { f[2 * p] = bf16lo(qb[i][p]); f[2 * p + 1] = bf16hi(qb[i][p]); }
    if (a.rotate) wht8<D>(f, lane);
    float sacc = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p) { qr[i][p] = f[p] * (a.rot_c * a.qscale); sacc += qr[i][p]; }
    sig[i] = sacc;
  }

  float m[NS], l[NS], oref[NS][8], ores[NRA][8], zacc[NRA];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    m[s] = -FLT_MAX; l[s] = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p) oref[s][p] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NRA; ++i) {
    zacc[i] = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p) ores[i][p] = 0.0f;
  }

  // ---- token tiles ----------------------------------------------------------
  for (int base = t_begin + wave * TILE; base < t_end; base += 4 * TILE) {
    uint4 yk[TR], yv[TR];
    uint32_t kcw[TR][NRA], kmw[TR][NRA], kaw[TR][NRA], vcw[TR][NRA], vmw[TR][NRA], vaw[TR][NRA];
    bool valid[TR];
#pragma unroll
    for (int u = 0; u < TR; ++u) {
      const int t = base + u * ROWS + r;
      valid[u] = t < t_end;
      const size_t slot = (size_t)bh * a.cap + (size_t)(valid[u] ? t : t_end - 1);
      yk[u] = *reinterpret_cast<const uint4 *>(a.kref + slot * D + 8 * j);
      yv[u] = *reinterpret_cast<const uint4 *>(a.vref + slot * D + 8 * j);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (a.bits[i] == 2) {
          kcw[u][i] = reinterpret_cast<const uint16_t *>(a.kc[i] + slot * (D / 4))[j];
          vcw[u][i] = reinterpret_cast<const uint16_t *>(a.vc[i] + slot * (D / 4))[j];
        } else {
          kcw[u][i] = reinterpret_cast<const uint32_t *>(a.kc[i] + slot * (D / 2))[j];
          vcw[u][i] = reinterpret_cast<const uint32_t *>(a.vc[i] + slot * (D / 2))[j];
        }
        kmw[u][i] = a.km[i][slot * G + k];
        vmw[u][i] = a.vm[i][slot * G + k];
        kaw[u][i] = a.ka[i][slot];
        vaw[u][i] = a.va[i][slot];
      }
    }

    // scores
    float sc[TR][NS];
#pragma unroll
    for (int u = 0; u < TR; ++u) {
      float part[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float dy = dot2bf(qb[s][0], yk[u].x, 0.0f);
        dy = dot2bf(qb[s][1], yk[u].y, dy);
        dy = dot2bf(qb[s][2], yk[u].z, dy);
        dy = dot2bf(qb[s][3], yk[u].w, dy);
        part[s] = dy;
      }
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int bits = a.bits[i];
        const uint32_t mask = (1u << bits) - 1u;
        float dc = 0.0f;
#pragma unroll
        for (int p = 0; p < 8; ++p)
          dc = __builtin_fmaf(qr[i][p], (float)((kcw[u][i] >> (bits * p)) & mask), dc);
        const float sK = f16_to_f32(kmw[u][i] & 0xffffu), zK = f16_to_f32(kmw[u][i] >> 16);
        const float aK = f16_to_f32(kaw[u][i]);
        part[i] = __builtin_fmaf(aK * a.qscale, part[i], __builtin_fmaf(sK, dc, zK * sig[i]));
      }
      if (REF) part[NR] *= a.qscale;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float tot = group_sum<LANES>(part[s]);
        sc[u][s] = valid[u] ? tot : -INFINITY;
      }
    }

    // online softmax: one rescale per tile
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float mt = sc[0][s];
#pragma unroll
      for (int u = 1; u < TR; ++u) mt = fmaxf(mt, sc[u][s]);
      const float mn = fmaxf(m[s], mt);
      const float f = fexp2(m[s] - mn);
      m[s] = mn;
      l[s] *= f;
#pragma unroll
      for (int p = 0; p < 8; ++p) oref[s][p] *= f;
      if (s < NR) {
        zacc[s] *= f;
#pragma unroll
        for (int p = 0; p < 8; ++p) ores[s][p] *= f;
      }
    }

    // values
#pragma unroll
    for (int u = 0; u < TR; ++u) {
      const float y[8] = {bf16lo(yv[u].x), bf16hi(yv[u].x), bf16lo(yv[u].y), bf16hi(yv[u].y),
                          bf16lo(yv[u].z), bf16hi(yv[u].z), bf16lo(yv[u].w), bf16hi(yv[u].w)};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float pr = fexp2(sc[u][s] - m[s]);
        l[s] += pr;
        if (s < NR) {
          const int bits = a.bits[s];
          const uint32_t mask = (1u << bits) - 1u;
          const float sV = f16_to_f32(vmw[u][s] & 0xffffu), zV = f16_to_f32(vmw[u][s] >> 16);
          const float wr = pr * f16_to_f32(vaw[u][s]);
          const float wq = pr * sV;
          zacc[s] = __builtin_fmaf(pr, zV, zacc[s]);
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            oref[s][p] = __builtin_fmaf(wr, y[p], oref[s][p]);
            ores[s][p] = __builtin_fmaf(wq, (float)((vcw[u][s] >> (bits * p)) & mask), ores[s][p]);
          }
        } else {
#pragma unroll
          for (int p = 0; p < 8; ++p) oref[s][p] = __builtin_fmaf(pr, y[p], oref[s][p]);
        }
      }
    }
  }

  // ---- merge rows, then waves -----------------------------------------------
#pragma unroll
  for (int i = 0; i < NR; ++i) {
#pragma unroll
    for (int p = 0; p < 8; ++p) ores[i][p] += zacc[i];
  }
  if constexpr (ROWS >= 2) merge_rows<LANES, NS, NR>(m, l, oref, ores);
  if constexpr (ROWS >= 4) merge_rows<LANES * 2, NS, NR>(m, l, oref, ores);
  if constexpr (ROWS >= 8) merge_rows<LANES * 4, NS, NR>(m, l, oref, ores);

  __shared__ float sm[4][NS][REC];
  if (r == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (j == 0) { sm[wave][s][0] = m[s]; sm[wave][s][1] = l[s]; }
#pragma unroll
      for (int p = 0; p < 8; ++p) sm[wave][s][2 + 8 * j + p] = oref[s][p];
      if (s < NR) {
#pragma unroll
        for (int p = 0; p < 8; ++p) sm[wave][s][2 + D + 8 * j + p] = ores[s][p];
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NS * REC; e += 256) {
    const int s = e / REC, c = e - s * REC;
    if (s >= NR && c >= 2 + D) continue;             // the reference loop has no residual part
    const float M = fmaxf(fmaxf(sm[0][s][0], sm[1][s][0]), fmaxf(sm[2][s][0], sm[3][s][0]));
    float v;
    if (c == 0) {
      v = M;
    } else {
      v = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v = __builtin_fmaf(fexp2(sm[w][s][0] - M), sm[w][s][c], v);
    }
    a.ws[(((size_t)split * kMaxSlots + s) * a.bh + bh) * REC + c] = v;
  }

  // ---- the last split of this batch*head merges all splits -----------------
  __shared__ int last;
  __threadfence();                                   // release this split's record
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(a.counters + bh, 1u) == (unsigned)(a.n_splits - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();                                   // acquire the other splits' records
  if (wave < NS) merge_splits<D>(a, bh, wave, wave < NR, lane);
  if (threadIdx.x == 0) a.counters[bh] = 0u;         // ready for the next call
}

// Log-sum-exp over the splits' records of one (batch*head, slot), then
// o = (o_ref + H_n o_res) / l.  One wave; lane holds dims lane + 64*e.
template <int D>
__device__ __forceinline__ void merge_splits(const DecodeArgs &a, int bh, int s, bool residual, int lane) {
  constexpr int E = D / 64;
  constexpr int REC = 2 * D + 2;
  const size_t stride = (size_t)kMaxSlots * a.bh * REC;
  const float *rec0 = a.ws + ((size_t)s * a.bh + bh) * REC;

  float M = -FLT_MAX;
  for (int sp = lane; sp < a.n_splits; sp += 64) M = fmaxf(M, rec0[sp * stride]);
  M = group_max<64>(M);

  float L = 0.0f, o[E], w[E];
#pragma unroll
  for (int e = 0; e < E; ++e) { o[e] = 0.0f; w[e] = 0.0f; }
  for (int sp = 0; sp < a.n_splits; ++sp) {
    const float *rec = rec0 + sp * stride;
    const float f = fexp2(rec[0] - M);
    L = __builtin_fmaf(f, rec[1], L);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(f, rec[2 + lane + 64 * e], o[e]);
    if (residual) {
#pragma unroll
      for (int e = 0; e < E; ++e) w[e] = __builtin_fmaf(f, rec[2 + D + lane + 64 * e], w[e]);
    }
  }
  if (residual) {
    if (a.rotate) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        w[e] = wht_stage<1>(w[e], lane);
        w[e] = wht_stage<2>(w[e], lane);
        w[e] = wht_stage<4>(w[e], lane);
        w[e] = wht_stage<8>(w[e], lane);
        w[e] = wht_stage<16>(w[e], lane);
        w[e] = wht_stage<32>(w[e], lane);
      }
#pragma unroll
      for (int h = 1; h < E; h *= 2) {
#pragma unroll
        for (int e0 = 0; e0 < E; e0 += 2 * h) {
#pragma unroll
          for (int e = e0; e < e0 + h; ++e) {
            const float x = w[e], y = w[e + h];
            w[e] = x + y;
            w[e + h] = x - y;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) w[e] *= a.rot_c;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] += w[e];
  }
  const float invL = 1.0f / L;
  float *out = a.out + ((size_t)a.qloop[s] * a.bh + bh) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) out[lane + 64 * e] = o[e] * invL;
}

template <int D, int NR, bool REF>
static hipError_t launch_partial(const DecodeArgs &a, hipStream_t st) {
  constexpr int TR = 2;
  const dim3 grid(a.n_splits, a.bh), block(256);
  hipLaunchKernelGGL((decode_kernel<D, NR, REF, TR>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs &a, int n_res, bool ref, hipStream_t st) {
  if (ref) {
    switch (n_res) {
      case 0: return launch_partial<D, 0, true>(a, st);
      case 1: return launch_partial<D, 1, true>(a, st);
      case 2: return launch_partial<D, 2, true>(a, st);
      case 3: return launch_partial<D, 3, true>(a, st);
    }
  } else {
    switch (n_res) {
      case 1: return launch_partial<D, 1, false>(a, st);
      case 2: return launch_partial<D, 2, false>(a, st);
      case 3: return launch_partial<D, 3, false>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a, int head_dim, int n_res, bool ref, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_decode_d<64>(a, n_res, ref, st);
    case 128: return launch_decode_d<128>(a, n_res, ref, st);
    case 256: return launch_decode_d<256>(a, n_res, ref, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rq
