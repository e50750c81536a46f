// rq_decode_kernel.hpp -- fused decode attention over a ResidualQuant cache
// (gfx950): the kernel template, instantiated by rq_decode_inst.hip once per
// (head_dim, reference kind, chain mode) and dispatched from rq_decode.hip,
// which also holds the split merge (kernel M).
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
// Kernel P, one launch per pass of up to three residual loops: a workgroup
// of W waves per (token split, batch*head), each wave taking every W-th tile
// of ROWS*TR tokens.  Lanes: D/8 lanes per token, 8 consecutive dims per
// lane, ROWS = 64/(D/8) tokens side by side, so one 128-bit load per lane
// reads ROWS consecutive reference rows, and every loop of the pass shares
// that load.  Online softmax per (row, loop) in the exp2 domain; rows, then
// waves (through LDS), are merged by log-sum-exp.  The splits also attend
// the BF16 tail rows, an equal share each.  With one split the workgroup
// finishes the output itself (un-rotation of the residual accumulator,
// normalisation); with several it writes one record per (split, loop,
// batch*head) to the workspace and kernel M merges the records.  (Kernel M
// alone attends a tail with no cache tokens before it.)

#pragma once

#include <float.h>

#include <type_traits>

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Value of x in lane 4*(lane/4) + S (DPP quad_perm broadcast).
__device__ __forceinline__ float quad_bcast(float x, int s) {
  switch (s) {
    case 0: return dpp<0x00>(x);
    case 1: return dpp<0x55>(x);
    case 2: return dpp<0xAA>(x);
    default: return dpp<0xFF>(x);
  }
}

// Lane j of a row owns loop slot j mod NP, NP = the pass's slot count
// rounded up to 1, 2 or 4 (so the four lanes of a quad own slots 0..3).
template <int NSC>
constexpr int own_slots() { return NSC <= 1 ? 1 : NSC <= 2 ? 2 : 4; }

// The row total of the partial scores of every slot, returned on each lane
// for its own slot only: a reduce-scatter over the row's LANES lanes.  Lanes
// j and j^1 swap half of the slots and add the half each keeps, lanes j and
// j^2 the same with what is left; then the lanes that own the same slot
// (j, j^4, j^8, ...) add theirs.  For four slots over 16 lanes that is 11
// VALU instructions, where four all-lane butterflies (every lane receiving
// every total) take 16.  All lanes that own a slot receive the same bits
// (each addition pairs the same two values, IEEE addition commutes).
template <int LANES, int NSC>
__device__ __forceinline__ float own_slot_total(const float (&part)[NSC], int j) {
  constexpr int NP = own_slots<NSC>();
  if constexpr (NP == 1) {
    return group_sum_dpp<LANES>(part[0]);
  } else {
    const bool b0 = (j & 1) != 0;
    float x;
    if constexpr (NP == 2) {
      const float keep = b0 ? part[1] : part[0], send = b0 ? part[0] : part[1];
      x = keep + dpp<kDppQuadXor1>(send);
      x += dpp<kDppQuadXor2>(x);
    } else {
      float p3 = 0.0f;
      if constexpr (NSC > 3) p3 = part[3];
      const float ka = b0 ? part[1] : part[0], sa = b0 ? part[0] : part[1];
      const float kb = b0 ? p3 : part[2], sb = b0 ? part[2] : p3;
      const float A = ka + dpp<kDppQuadXor1>(sa);
      const float B = kb + dpp<kDppQuadXor1>(sb);
      const bool b1 = (j & 2) != 0;
      const float keep = b1 ? B : A, send = b1 ? A : B;
      x = keep + dpp<kDppQuadXor2>(send);
    }
    if constexpr (LANES == 8) {
      x += xor_lane<4>(x);
    } else {
      x += dpp<kDppRowRor4>(x);
      x += dpp<kDppRowRor8>(x);
      if constexpr (LANES == 32) x += xor_lane<16>(x);
    }
    return x;
  }
}

// First product of a dot chain: the three-operand v_dot2_f32_bf16 with an
// inline zero accumulator (the builtin would zero a register first).
__device__ __forceinline__ float dot2bf0(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }


// Merge the online-softmax states of rows at lane distance MASK.  The lane's
// running sum l_own belongs to loop slot `own` (lane index mod 4).
// Slots below OREF_FROM carry no reference accumulator (with a quantized
// anchor the residual slots fold the anchor into their residual one).
template <int MASK, int NS, int NR, int OREF_FROM>
__device__ __forceinline__ void merge_rows(float (&m)[NS], float &l_own, int own, float (&oref)[NS][8],
                                           float (&ores)[NR > 0 ? NR : 1][8]) {
  const float lo = xor_lane<MASK>(l_own);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float mo = xor_lane<MASK>(m[s]);
    const float M = fmaxf(m[s], mo);
    const float fa = fexp2(m[s] - M), fb = fexp2(mo - M);
    if (own == s) l_own = l_own * fa + lo * fb;
    if (s >= OREF_FROM) {
#pragma unroll
      for (int p = 0; p < 8; ++p) oref[s][p] = oref[s][p] * fa + xor_lane<MASK>(oref[s][p]) * fb;
    }
    if (s < NR) {
#pragma unroll
      for (int p = 0; p < 8; ++p) ores[s][p] = ores[s][p] * fa + xor_lane<MASK>(ores[s][p]) * fb;
    }
    m[s] = M;
  }
}

// Output row of one (loop slot, batch*head), lane holding dims lane + 64*e:
// out = (o_ref + H_n o_res + t) / l, where o_ref accumulates the reference
// (BF16 rows, or the anchor), o_res the residual codes and t the BF16 tail
// rows.  When the anchor is itself rotated, o_ref joins o_res before the
// un-rotation.  H_n runs as butterflies across lanes (distances 1..32) and
// across the lane's E = D/64 elements.
template <int D>
__device__ __forceinline__ void finish_row(const DecodeArgs &a, int bh, int s, bool residual, int lane,
                                           float L, float (&o)[D / 64], float (&w)[D / 64],
                                           const float (&t)[D / 64]) {
  constexpr int E = D / 64;
  if (!((a.out_mask >> a.qloop[s]) & 1u)) return;   // a chain link computed, not asked for
  const bool ref_rot = a.ref_rotated != 0;
  if (residual || ref_rot) {
    if (ref_rot) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        w[e] = residual ? w[e] + o[e] : o[e];
        o[e] = 0.0f;
      }
    }
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
  for (int e = 0; e < E; ++e) out[lane + 64 * e] = (o[e] + t[e]) * invL;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// fma(a, h, c) where h is one half of `w` read as an FP16 number (v_fma_mix_f32
// takes the half directly, no conversion instruction).
template <int HI>
__device__ __forceinline__ float fma_half(float a, uint32_t w, float c) {
  const half2_t h = __builtin_bit_cast(half2_t, w);
  return __builtin_fmaf(a, (float)h[HI], c);
}

// The 8 codes of one lane as 8 FP16 halves, each holding one code in its
// mantissa bits: a half whose bit pattern is c << b (b + width <= 10) is the
// subnormal number c * 2^(b-24), exact.  Code p lands in half (p / 4) of word
// w[p % 4] at mantissa bit position pos(p) = 2 * (p % 4), for INT2 and INT4
// alike, so one set of 2^(24 - pos) factors serves every loop:
//   INT2 (the lane's 16 code bits, code p at bits 2p, in the aligned 32-bit
//   word x that holds them, selected by sel): its bytes c0..c3 and c4..c7
//   are spread to the two halves, then masked per code.
//   INT4 (32-bit word x, code p at bits 4p): the halves already hold c0..c3
//   and c4..c7; code q of each half is shifted down by 2q bits, then masked.
template <bool INT4>
__device__ __forceinline__ void code_halves(uint32_t x, uint32_t (&w)[4], uint32_t sel) {
  if constexpr (INT4) {
    w[0] = x & 0x000F000Fu;
    w[1] = (x >> 2) & 0x003C003Cu;
    w[2] = (x >> 4) & 0x00F000F0u;
    w[3] = (x >> 6) & 0x03C003C0u;
  } else {
    const uint32_t X = __builtin_amdgcn_perm(0u, x, sel);             // [b_lo, 0, b_hi, 0]
    w[0] = X & 0x00030003u;
    w[1] = X & 0x000C000Cu;
    w[2] = X & 0x00300030u;
    w[3] = X & 0x00C000C0u;
  }
}

// An INT2 lane reads the aligned 32-bit word holding its 2 code bytes (lanes
// 2i and 2i+1 share one word): the byte-permute selector that spreads the
// lane's own bytes, [b0, 0, b1, 0] for an even lane and [b2, 0, b3, 0] for an
// odd one.  A full-word load keeps the value 32 bits wide through the tile
// registers, so no mask is needed before the permute.
__device__ __forceinline__ uint32_t int2_sel(int j) { return (j & 1) ? 0x0c030c02u : 0x0c010c00u; }

// Mantissa bit position of code p in its half (so its half reads c * 2^(pos-24)).
__host__ __device__ constexpr int code_pos(int p) { return 2 * (p & 3); }

// Sum over the lane's 8 codes (as halves w) of coef[p] * half_p (coef
// pre-multiplied by 2^(24 - pos) makes this sum_p coef'[p] * c_p).
__device__ __forceinline__ float code_dot_h(const uint32_t (&w)[4], const float (&coef)[8], float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = fma_half<0>(coef[q], w[q], acc);
    acc = fma_half<1>(coef[q + 4], w[q], acc);
  }
  return acc;
}

// acc[p] += wgt * half_p  (the accumulator then carries 2^(pos-24)).
__device__ __forceinline__ void code_axpy_h(const uint32_t (&w)[4], float wgt, float (&acc)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[q] = fma_half<0>(wgt, w[q], acc[q]);
    acc[q + 4] = fma_half<1>(wgt, w[q], acc[q + 4]);
  }
}

// The low / high FP16 half of a 32-bit word, for use as an fma operand
// (v_fma_mix_f32 reads it in place).
__device__ __forceinline__ float h_lo(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[0]; }
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[1]; }

// Load from a uniform base plus a 32-bit byte offset (global_load with an
// SGPR base and a 32-bit VGPR offset; no 64-bit address arithmetic per lane).
template <typename T>
__device__ __forceinline__ T ldg(const void *base, uint32_t byte_off) {
  return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}

// The same with the non-temporal hint, for the planes every byte of which is
// read exactly once per step by one load instruction (reference rows and
// code words).  On MI355X it lifts a plain 128-bit read stream from about
// 6.0 to 6.8 TB/s and the int2-8k decode step by ~9%.  The meta and alpha
// planes keep the default policy: consecutive tiles share their cache lines,
// and streaming them too made the step slower (300 against 285 us).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ T ldg_nt(const void *base, uint32_t byte_off);
template <>
__device__ __forceinline__ uint4 ldg_nt<uint4>(const void *base, uint32_t byte_off) {
  const u32x4_t v = __builtin_nontemporal_load(
      reinterpret_cast<const u32x4_t *>(reinterpret_cast<const char *>(base) + byte_off));
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <>
__device__ __forceinline__ uint32_t ldg_nt<uint32_t>(const void *base, uint32_t byte_off) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(base) + byte_off));
}

// Reference part of a token tile: BF16 rows (AQ = 0), or a quantized
// anchor's code word and (scale, zero) word per lane (AQ = its bit width).
template <int TR, int AQ>
struct RefTile {
  uint32_t ak[TR], av[TR], amk[TR], amv[TR];
};
template <int TR>
struct RefTile<TR, 0> {
  uint4 yk[TR], yv[TR];
};

template <int TR, int NRA, int AQ>
struct Tile : RefTile<TR, AQ> {
  uint32_t kc[TR][NRA], km[TR][NRA], ka[TR][NRA], vc[TR][NRA], vm[TR][NRA], va[TR][NRA];
};

// Scores above the running max by more than this (log2 units) trigger a
// rescale; below it, weights exp2(s - m) stay <= 2^8 and no rescale is done.
constexpr float kRescaleSlack = 8.0f;

// CHAIN (1, 2): chained references (each residual loop's reference is the
// next slot's reconstruction, the last residual slot's is the pass's
// reference).  Slot i then scores q_i . K_i with K_i = a_i K_{i+1} + r_i
// unrolled down the chain, and accumulates p_i (prod a) r_m for every m >= i
// into its residual sum.  CHAIN == 2 computes slot 0 alone (the other slots
// are links whose outputs are not asked for).
template <int D, int NR, bool REF, int B4, int TR, int W, int AQ, int CHAIN>
__global__ __launch_bounds__(64 * W) void decode_kernel(const DecodeArgs a) {
  constexpr int LANES = D / 8;
  constexpr int ROWS = kWave / LANES;
  constexpr int NS = NR + (REF ? 1 : 0);
  constexpr int NRA = NR > 0 ? NR : 1;
  // Slots computed: every slot of the pass, or with CHAIN == 2 only slot 0
  // (a call for one loop along a chain reads every link's planes but wants
  // none of the links' own outputs).
  constexpr int NSC = CHAIN == 2 ? 1 : NS;
  constexpr int NRS = CHAIN == 2 ? 1 : NR;     // residual slots computed
  constexpr int NRSA = NRS > 0 ? NRS : 1;
  constexpr int TILE = ROWS * TR;
  constexpr int STEP = W * TILE;
  constexpr int REC = 2 * D + 2;
  static_assert(W >= NSC, "one merging wave per loop slot");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane % LANES, r = lane / LANES;
  const uint32_t sel2 = int2_sel(j);                // INT2 code bytes in the loaded word
  const int split = blockIdx.x, bh = blockIdx.y;
  const int t_begin = split * a.tps;
  const int t_end = min(t_begin + a.tps, a.n_ctx);
  const int G = D / a.group;
  const int gshift = __builtin_ctz((unsigned)G);     // meta words per token = 2^gshift
  const int k = j / (a.group / 8);
  constexpr bool AINT4 = AQ == 4;
  const int ashift = __builtin_ctz((unsigned)(D / a.agroup));   // anchor meta words per token
  const int ka_ = j / (a.agroup / 8);                           // this lane's anchor group

  // Plane bases of this (batch, head): uniform, so they live in SGPRs and
  // every load is base + 32-bit lane offset.
  const size_t row0 = (size_t)bh * a.cap;
  const uint16_t *kref = a.kref + row0 * D;
  const uint16_t *vref = a.vref + row0 * D;
  const uint8_t *kac = a.kac + row0 * (D * (AQ > 0 ? AQ : 1) / 8);
  const uint8_t *vac = a.vac + row0 * (D * (AQ > 0 ? AQ : 1) / 8);
  const uint32_t *kam = a.kam + (row0 << ashift);
  const uint32_t *vam = a.vam + (row0 << ashift);
  const uint8_t *kc[NRA], *vc[NRA];
  const uint32_t *km[NRA], *vm[NRA];
  const uint16_t *ka[NRA], *va[NRA];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int cb = ((B4 >> i) & 1) ? D / 2 : D / 4;
    kc[i] = a.kc[i] + row0 * cb;
    vc[i] = a.vc[i] + row0 * cb;
    km[i] = a.km[i] + row0 * G;
    vm[i] = a.vm[i] + row0 * G;
    ka[i] = a.ka[i] + row0;
    va[i] = a.va[i] + row0;
  }

  auto load = [&](Tile<TR, NRA, AQ> &T, int base) {
#pragma unroll
    for (int u = 0; u < TR; ++u) {
      const uint32_t t = (uint32_t)min(base + u * ROWS + r, t_end - 1);
      if constexpr (AQ == 0) {
        T.yk[u] = ldg_nt<uint4>(kref, t * (2 * D) + 16 * j);
        T.yv[u] = ldg_nt<uint4>(vref, t * (2 * D) + 16 * j);
      } else {
        if constexpr (AINT4) {
          T.ak[u] = ldg_nt<uint32_t>(kac, t * (D / 2) + 4 * j);
          T.av[u] = ldg_nt<uint32_t>(vac, t * (D / 2) + 4 * j);
        } else {
          T.ak[u] = ldg_nt<uint32_t>(kac, t * (D / 4) + 4 * (j >> 1));
          T.av[u] = ldg_nt<uint32_t>(vac, t * (D / 4) + 4 * (j >> 1));
        }
        T.amk[u] = ldg<uint32_t>(kam, ((t << ashift) + ka_) * 4);
        T.amv[u] = ldg<uint32_t>(vam, ((t << ashift) + ka_) * 4);
      }
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if ((B4 >> i) & 1) {
          T.kc[u][i] = ldg_nt<uint32_t>(kc[i], t * (D / 2) + 4 * j);
          T.vc[u][i] = ldg_nt<uint32_t>(vc[i], t * (D / 2) + 4 * j);
        } else {
          T.kc[u][i] = ldg_nt<uint32_t>(kc[i], t * (D / 4) + 4 * (j >> 1));
          T.vc[u][i] = ldg_nt<uint32_t>(vc[i], t * (D / 4) + 4 * (j >> 1));
        }
        T.km[u][i] = ldg<uint32_t>(km[i], ((t << gshift) + k) * 4);
        T.vm[u][i] = ldg<uint32_t>(vm[i], ((t << gshift) + k) * 4);
        T.ka[u][i] = ldg<uint16_t>(ka[i], t * 2);
        T.va[u][i] = ldg<uint16_t>(va[i], t * 2);
      }
    }
  };

  // ---- prologue: queries of every loop in the pass -------------------------
  // The query rows, the first token tile and the first tail rows are loaded
  // before any of them is used, so their memory latencies overlap.  (The
  // first tile is loaded even by a wave with no tile in the split: its token
  // indices are clamped into the split.)
  uint4 qraw[NSC];
#pragma unroll
  for (int s = 0; s < NSC; ++s)
    qraw[s] = *reinterpret_cast<const uint4 *>(a.q + ((size_t)a.qloop[s] * a.bh + bh) * D + 8 * j);
  int base = t_begin + wave * TILE;
  Tile<TR, NRA, AQ> ta, tb;
  load(ta, base);

  // BF16 tail rows: split s attends rows [tail0, tail1), an equal share of the
  // tail per split (as more tokens of its own), so that no split's chain of
  // work is longer than the others'.  Each wave takes every W-th group of
  // ROWS rows of the share, TG groups per chunk, every loop slot's rows at
  // once.  Slots whose loop is not asked for (chain links) have no tail.
  constexpr int TG = 2;
  const int tshare = a.tail_in ? (a.n_tail + (int)gridDim.x - 1) / (int)gridDim.x : 0;
  const int tail0 = split * tshare, tail1 = min(tail0 + tshare, a.n_tail);
  uint4 tkw[TG][NSC], tvw[TG][NSC];
  auto load_tail = [&](int t0) {
#pragma unroll
    for (int g = 0; g < TG; ++g) {
      const uint32_t t = (uint32_t)min(t0 + g * W * ROWS + r, tail1 - 1);
#pragma unroll
      for (int s = 0; s < NSC; ++s) {
        if (!((a.out_mask >> a.qloop[s]) & 1u)) continue;
        const size_t o = (size_t)bh * a.tcap * D;
        tkw[g][s] = ldg_nt<uint4>(a.tk[s] + o, t * (2 * D) + 16 * j);
        tvw[g][s] = ldg_nt<uint4>(a.tv[s] + o, t * (2 * D) + 16 * j);
      }
    }
  };
  const bool tail_here = a.tail_in && tail0 < tail1;
  if (tail_here) load_tail(tail0 + wave * ROWS);

  // BF16 reference: its dots use the BF16 query pairs as stored (qb).
  // Code dots (residual loops, and with a quantized anchor the anchor too)
  // use q' = H_n q in FP32 (just q without rotation), each element
  // pre-multiplied by 2^(24 - pos) for its code's position in code_halves
  // (qr); sig is the lane's sum of q' for the offsets.  Scores are scaled by
  // sm_scale*log2(e) after the row sum.
  constexpr int NQB = AQ ? 1 : NSC;
  constexpr int NQR = AQ ? NSC : NRSA;
  uint32_t qb[NQB][4];
  float qr[NQR][8], sig[NQR];
#pragma unroll
  for (int s = 0; s < NSC; ++s) {
    const uint4 w = qraw[s];
    const uint32_t wq[4] = {w.x, w.y, w.z, w.w};
    if constexpr (!AQ) {
#pragma unroll
      for (int p = 0; p < 4; ++p) qb[s][p] = wq[p];
    }
    if (AQ || s < NRS) {
      const int i = s < NQR ? s : 0;
      float f[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) { f[2 * p] = bf16lo(wq[p]); f[2 * p + 1] = bf16hi(wq[p]); }
      if (a.rotate) wht8<D>(f, lane);
      float tot = 0.0f;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float v = f[p] * a.rot_c;
        tot += v;
        qr[i][p] = v * (float)(1 << (24 - code_pos(p)));
      }
      sig[i] = tot;
    }
  }

  // Softmax state: m per loop slot (uniform across a row); the running sum of
  // loop slot own = j % 4 only, kept by the lanes that compute that slot's
  // exponentials (lane j of a quad computes slot j's weight; the quad shares
  // the four weights through DPP).
  const int own = j & (own_slots<NSC>() - 1);
  // With a quantized anchor the residual slots fold the anchor's values into
  // their residual accumulator (both are code sums in the same domain), so
  // only the anchor's own slot keeps a reference accumulator (with offset
  // share zref).
  constexpr int OREF_FROM = AQ ? NRS : 0;
  float m[NSC], l_own = 0.0f, oref[NSC][8], ores[NRSA][8], zacc[NRSA], zref = 0.0f;
#pragma unroll
  for (int s = 0; s < NSC; ++s) {
    m[s] = -FLT_MAX;
#pragma unroll
    for (int p = 0; p < 8; ++p) oref[s][p] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NRSA; ++i) {
    zacc[i] = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p) ores[i][p] = 0.0f;
  }

  // The running max of the lane's own slot.  The tail section below keeps
  // the max of every slot (m); the token tiles keep only the own slot's, and
  // every lane reads another slot's max from the lane of its quad that owns
  // it (a slot's max is the same on all lanes of a row that own it).
  float m_own = -FLT_MAX;

  // ---- the tail rows.  Scores use the BF16 query; values go to the
  // accumulator the output is finished from: the reference sums (original
  // domain) with a BF16 reference, or with a quantized anchor the code sums,
  // which live in the rotated domain and carry the 2^(pos-24) code factors,
  // so those rows enter as c H v times those factors (finish_row un-rotates
  // them back).
  if (tail_here) {
    for (int t0 = tail0 + wave * ROWS; t0 < tail1; t0 += TG * W * ROWS) {
      if (t0 != tail0 + wave * ROWS) load_tail(t0);
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        const bool valid = t0 + g * W * ROWS + r < tail1;
#pragma unroll
        for (int s = 0; s < NSC; ++s) {
          if (!((a.out_mask >> a.qloop[s]) & 1u)) continue;   // a chain link not asked for
          const uint4 kw = tkw[g][s], vw = tvw[g][s], qw = qraw[s];
          float dp = dot2bf0(qw.x, kw.x);
          dp = dot2bf(qw.y, kw.y, dp);
          dp = dot2bf(qw.z, kw.z, dp);
          dp = dot2bf(qw.w, kw.w, dp);
          const float tot = group_sum_dpp<LANES>(dp) * a.qscale;
          const float sc = valid ? tot : -INFINITY;
          if (own == s) m_own = fmaxf(m_own, sc);
          if (sc > m[s]) {
            const float f = fexp2(m[s] - sc);
            m[s] = sc;
            if (own == s) l_own *= f;
            if (s >= OREF_FROM) {
#pragma unroll
              for (int p = 0; p < 8; ++p) oref[s][p] *= f;
              if (AQ) zref *= f;
            }
            if (s < NRS) {
              zacc[s] *= f;
#pragma unroll
              for (int p = 0; p < 8; ++p) ores[s][p] *= f;
            }
          }
          const float pw = fexp2(sc - m[s]);
          if (own == s) l_own += pw;
          float y[8];
          y[0] = bf16lo(vw.x); y[1] = bf16hi(vw.x);
          y[2] = bf16lo(vw.y); y[3] = bf16hi(vw.y);
          y[4] = bf16lo(vw.z); y[5] = bf16hi(vw.z);
          y[6] = bf16lo(vw.w); y[7] = bf16hi(vw.w);
          if constexpr (AQ == 0) {
#pragma unroll
            for (int p = 0; p < 8; ++p) oref[s][p] = __builtin_fmaf(pw, y[p], oref[s][p]);
          } else {
            if (a.rotate) {
              wht8<D>(y, lane);
#pragma unroll
              for (int p = 0; p < 8; ++p) y[p] *= a.rot_c;
            }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              const float yp = y[p] * (1.0f / (float)(1 << (24 - code_pos(p))));
              if (s < NRS) ores[s][p] = __builtin_fmaf(pw, yp, ores[s][p]);
              else oref[s][p] = __builtin_fmaf(pw, yp, oref[s][p]);
            }
          }
        }
      }
    }
  }

  auto process = [&](const Tile<TR, NRA, AQ> &T, int base, auto full_tile) {
    constexpr bool FULL = decltype(full_tile)::value;
    // scores (log2 units) of the lane's own slot
    float sc[TR];
#pragma unroll
    for (int u = 0; u < TR; ++u) {
      // Partial scores of this lane's 8 dims, in units of 1/qscale: the
      // reference dots are exact BF16 products; the residual dots and their
      // offset terms carry q' without the softmax scale, and the FP16 scale,
      // zero and LS coefficient enter v_fma_mix_f32 as stored.
      float part[NSC];
      if constexpr (AQ == 0) {
#pragma unroll
        for (int s = 0; s < NSC; ++s) {
          float dy = dot2bf0(qb[s][0], T.yk[u].x);
          dy = dot2bf(qb[s][1], T.yk[u].y, dy);
          dy = dot2bf(qb[s][2], T.yk[u].z, dy);
          part[s] = dot2bf(qb[s][3], T.yk[u].w, dy);
        }
      } else {
        // anchor dot per slot: s_a (q' . code) + z_a sum(q'), codes as halves
        uint32_t hk[4];
        code_halves<AINT4>(T.ak[u], hk, sel2);
        const uint32_t mw = T.amk[u];
#pragma unroll
        for (int s = 0; s < NSC; ++s) {
          const float dc = code_dot_h(hk, qr[s], 0.0f);
          part[s] = __builtin_fmaf(h_lo(mw), dc, __builtin_fmaf(h_hi(mw), sig[s], 0.0f));
        }
      }
      uint32_t hk[NRA][4];
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        if ((B4 >> m) & 1) code_halves<true>(T.kc[u][m], hk[m], sel2);
        else code_halves<false>(T.kc[u][m], hk[m], sel2);
      }
#pragma unroll
      for (int i = 0; i < NRS; ++i) {
        // K_i = a_i K_{i+1} + r_i: from the reference (part) down to loop i
        float acc = part[i];
#pragma unroll
        for (int m = NR - 1; m >= i; --m) {
          if (!CHAIN && m != i) continue;
          const float dc = code_dot_h(hk[m], qr[i], 0.0f);
          const uint32_t mw = T.km[u][m];
          const float t = __builtin_fmaf(h_lo(mw), dc, __builtin_fmaf(h_hi(mw), sig[i], 0.0f));
          acc = __builtin_fmaf(h_lo(T.ka[u][m]), acc, t);
        }
        part[i] = acc;
      }
      const bool valid = (FULL || base + u * ROWS + r < t_end) && own < NSC;
      const float tot = own_slot_total<LANES, NSC>(part, j) * a.qscale;
      sc[u] = (FULL && own_slots<NSC>() == NSC) ? tot : (valid ? tot : -INFINITY);
    }

    // online softmax; rescale only when the max grows by more than the slack.
    // Each lane tests its own slot; the rescale (rarely taken) runs on the
    // whole wave when any lane's slot grew, every lane taking each slot's
    // new max from the lane of its quad that owns the slot (the slot's max
    // is the same on every such lane of the row).
    float mt = sc[0];
#pragma unroll
    for (int u = 1; u < TR; ++u) mt = fmaxf(mt, sc[u]);
    if (__builtin_amdgcn_ballot_w64(mt > m_own + kRescaleSlack) != 0) {
#pragma unroll
      for (int s = 0; s < NSC; ++s) {
        const float mts = own_slots<NSC>() == 1 ? mt : quad_bcast(mt, s);
        const float mos = own_slots<NSC>() == 1 ? m_own : quad_bcast(m_own, s);
        if (mts > mos + kRescaleSlack) {
          const float f = fexp2(mos - mts);
          if (own == s) l_own *= f;
          if (s >= OREF_FROM) {
#pragma unroll
            for (int p = 0; p < 8; ++p) oref[s][p] *= f;
            if (AQ) zref *= f;
          }
          if (s < NRS) {
            zacc[s] *= f;
#pragma unroll
            for (int p = 0; p < 8; ++p) ores[s][p] *= f;
          }
        }
      }
      m_own = mt > m_own + kRescaleSlack ? mt : m_own;
    }

    // values
#pragma unroll
    for (int u = 0; u < TR; ++u) {
      float y[8];
      uint32_t hv[4];
      if constexpr (AQ == 0) {
        y[0] = bf16lo(T.yv[u].x); y[1] = bf16hi(T.yv[u].x);
        y[2] = bf16lo(T.yv[u].y); y[3] = bf16hi(T.yv[u].y);
        y[4] = bf16lo(T.yv[u].z); y[5] = bf16hi(T.yv[u].z);
        y[6] = bf16lo(T.yv[u].w); y[7] = bf16hi(T.yv[u].w);
      } else {
        code_halves<AINT4>(T.av[u], hv, sel2);
      }
      // one exponential per lane (slot own), shared across the quad
      const float p_own = fexp2(sc[u] - m_own);
      l_own += p_own;
      float pq[NSC];
#pragma unroll
      for (int s = 0; s < NSC; ++s) pq[s] = NSC == 1 ? p_own : quad_bcast(p_own, s);
      uint32_t hvc[NRA][4];
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        if ((B4 >> m) & 1) code_halves<true>(T.vc[u][m], hvc[m], sel2);
        else code_halves<false>(T.vc[u][m], hvc[m], sel2);
      }
#pragma unroll
      for (int s = 0; s < NSC; ++s) {
        const float pr = pq[s];
        if (s < NRS) {
          // p (s_m code + z_m) for loop s (and, chained, every loop after it,
          // each weighted by the alphas on the way), then the reference's part
          float w = pr;
#pragma unroll
          for (int m = s; m < NR; ++m) {
            if (!CHAIN && m != s) continue;
            const uint32_t mw = T.vm[u][m];
            zacc[s] = __builtin_fmaf(h_hi(mw), w, zacc[s]);
            code_axpy_h(hvc[m], __builtin_fmaf(h_lo(mw), w, 0.0f), ores[s]);
            w = __builtin_fmaf(h_lo(T.va[u][m]), w, 0.0f);
          }
          if constexpr (AQ == 0) {
#pragma unroll
            for (int p = 0; p < 8; ++p) oref[s][p] = __builtin_fmaf(w, y[p], oref[s][p]);
          } else {
            // alpha_V p (s_a code + z_a), into the residual accumulator
            const uint32_t am = T.amv[u];
            zacc[s] = __builtin_fmaf(h_hi(am), w, zacc[s]);
            code_axpy_h(hv, __builtin_fmaf(h_lo(am), w, 0.0f), ores[s]);
          }
        } else if constexpr (AQ == 0) {
#pragma unroll
          for (int p = 0; p < 8; ++p) oref[s][p] = __builtin_fmaf(pr, y[p], oref[s][p]);
        } else {
          const uint32_t am = T.amv[u];
          zref = __builtin_fmaf(h_hi(am), pr, zref);
          code_axpy_h(hv, __builtin_fmaf(h_lo(am), pr, 0.0f), oref[s]);
        }
      }
    }
  };

  // ---- token tiles: two tile buffers, the next one loading while the other
  // is processed.  The next tile is always loaded (its token indices clamped
  // into the split), so the loads are straight-line code and the wait before
  // processing a tile covers only that tile's loads.
  if (base < t_end) {
    while (true) {
      load(tb, base + STEP);
      if (base + TILE <= t_end) process(ta, base, std::true_type{});
      else process(ta, base, std::false_type{});
      base += STEP;
      if (base >= t_end) break;
      load(ta, base + STEP);
      if (base + TILE <= t_end) process(tb, base, std::true_type{});
      else process(tb, base, std::false_type{});
      base += STEP;
      if (base >= t_end) break;
    }
  }

  // undo the 2^(pos-24) factors of the value codes, add the offsets' share
#pragma unroll
  for (int i = 0; i < NRS; ++i) {
#pragma unroll
    for (int p = 0; p < 8; ++p) ores[i][p] = __builtin_fmaf(ores[i][p], (float)(1 << (24 - code_pos(p))), zacc[i]);
  }
  if constexpr (AQ > 0 && REF) {
#pragma unroll
    for (int p = 0; p < 8; ++p) oref[NRS][p] = __builtin_fmaf(oref[NRS][p], (float)(1 << (24 - code_pos(p))), zref);
  }

  // every slot's running max on every lane, for the merges
#pragma unroll
  for (int s = 0; s < NSC; ++s) m[s] = own_slots<NSC>() == 1 ? m_own : quad_bcast(m_own, s);

  // ---- merge rows, then waves -----------------------------------------------
  if constexpr (ROWS >= 2) merge_rows<LANES, NSC, NRS, OREF_FROM>(m, l_own, own, oref, ores);
  if constexpr (ROWS >= 4) merge_rows<LANES * 2, NSC, NRS, OREF_FROM>(m, l_own, own, oref, ores);
  if constexpr (ROWS >= 8) merge_rows<LANES * 4, NSC, NRS, OREF_FROM>(m, l_own, own, oref, ores);

  __shared__ float sm[W][NSC][REC];
  if (r == 0) {
#pragma unroll
    for (int s = 0; s < NSC; ++s) {
      if (j == 0) sm[wave][s][0] = m[s];
      if (j == s) sm[wave][s][1] = l_own;
#pragma unroll
      for (int p = 0; p < 8; ++p) sm[wave][s][2 + 8 * j + p] = s >= OREF_FROM ? oref[s][p] : 0.0f;
      if (s < NRS) {
#pragma unroll
        for (int p = 0; p < 8; ++p) sm[wave][s][2 + D + 8 * j + p] = ores[s][p];
      }
    }
  }
  __syncthreads();
  // wave s combines loop slot s over the W waves
  if (wave < NSC) {
    const int s = wave;
    const bool residual = s < NRS;
    float M = sm[0][s][0];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, sm[w][s][0]);
    float f[W];
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) { f[w] = fexp2(sm[w][s][0] - M); L = __builtin_fmaf(f[w], sm[w][s][1], L); }
    constexpr int E = D / 64;
    float o[E], q[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      o[e] = 0.0f; q[e] = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        o[e] = __builtin_fmaf(f[w], sm[w][s][2 + lane + 64 * e], o[e]);
        if (residual) q[e] = __builtin_fmaf(f[w], sm[w][s][2 + D + lane + 64 * e], q[e]);
      }
    }
    if (!a.records) {
      float none[E];
#pragma unroll
      for (int e = 0; e < E; ++e) none[e] = 0.0f;
      finish_row<D>(a, bh, s, residual, lane, L, o, q, none);
    } else {
      float *rec = a.ws + (((size_t)split * kMaxSlots + s) * a.bh + bh) * REC;
      if (lane == 0) { rec[0] = M; rec[1] = L; }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        rec[2 + lane + 64 * e] = o[e];
        if (residual) rec[2 + D + lane + 64 * e] = q[e];
      }
    }
  }
}


// Tiles per wave iteration and waves per workgroup.  Four waves (the fewest
// that give every loop slot its own merging wave) let two workgroups share a
// compute unit, so one workgroup's merge overlaps the other's streaming.
// A single-slot pass (one loop alone) moves few bytes per token, so its waves
// keep four tiles in flight instead of two.
constexpr int kTilesPerIter = 2;
constexpr int kWaves = 4;
template <int NS>
constexpr int tiles_per_iter() { return NS == 1 ? 4 : kTilesPerIter; }

// Waves of the wide form's workgroup.  A single-slot pass over a quantized
// anchor (a per-loop call of an INT2 residual loop, or of the anchor loop)
// or over BF16 rows alone fits three waves per SIMD (at most 168 VGPRs, no
// spills), so its one workgroup per batch*head runs 12 waves: interleaved
// A/B, per-loop anchored step 383.0 -> 374.8 us at batch 16, 8k, identical
// within 6e-5.  Every other pass keeps 8 (two per SIMD).
template <int NR, bool REF, int B4, int AQ, int CHAIN>
constexpr int wide_waves() {
  return (CHAIN == 0 && ((AQ > 0 && NR == 1 && !REF && B4 == 0) || (NR == 0 && REF))) ? 12 : 2 * kWaves;
}

// Workgroup shape (decided on the host): a call of two splits with no tail
// whose batch*heads fill the compute units once (a.wide) runs as one 8-wave
// workgroup per batch*head instead: the same waves over the same tokens, two
// per SIMD as before, with no split records and no merge launch.  Splits
// that fit one workgroup per compute unit (a.waves8) run 8 waves each.
template <int D, int NR, bool REF, int B4, int AQ, int CHAIN>
static hipError_t launch_kernel(const DecodeArgs &a, hipStream_t st) {
  constexpr int NS = NR + (REF ? 1 : 0);
  constexpr int TR = tiles_per_iter<NS>();
  if (a.wide) {
    DecodeArgs b = a;
    b.n_splits = 1;
    b.tps = a.n_ctx;
    b.records = 0;
    constexpr int WW = wide_waves<NR, REF, B4, AQ, CHAIN>();
    hipLaunchKernelGGL((decode_kernel<D, NR, REF, B4, TR, WW, AQ, CHAIN>), dim3(1, a.bh), dim3(64 * WW), 0, st, b);
    return hipGetLastError();
  }
  const dim3 grid(a.n_splits, a.bh);
  if (a.waves8)
    hipLaunchKernelGGL((decode_kernel<D, NR, REF, B4, TR, 2 * kWaves, AQ, CHAIN>), grid, dim3(64 * 2 * kWaves), 0, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, NR, REF, B4, TR, kWaves, AQ, CHAIN>), grid, dim3(64 * kWaves), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.records) return e;
  DecodeArgs m = a;
  if (a.tail_in) m.n_tail = 0;        // already in the splits' records
  if constexpr (CHAIN == 2) return launch_merge(m, D, 1, 1, st);
  return launch_merge(m, D, NR, NR + (REF ? 1 : 0), st);
}

// Bit widths of the pass's residual loops as a mask (bit i: loop i is INT4).
template <int D, int NR, bool REF, int AQ, int CHAIN>
static hipError_t launch_bits(const DecodeArgs &a, hipStream_t st) {
  int b4 = 0;
  for (int i = 0; i < NR; ++i) b4 |= (a.bits[i] == 4) << i;
  switch (b4) {
    case 0: return launch_kernel<D, NR, REF, 0, AQ, CHAIN>(a, st);
    case 1: if constexpr (NR >= 1) return launch_kernel<D, NR, REF, 1, AQ, CHAIN>(a, st); break;
    case 2: if constexpr (NR >= 2) return launch_kernel<D, NR, REF, 2, AQ, CHAIN>(a, st); break;
    case 3: if constexpr (NR >= 2) return launch_kernel<D, NR, REF, 3, AQ, CHAIN>(a, st); break;
    case 4: if constexpr (NR >= 3) return launch_kernel<D, NR, REF, 4, AQ, CHAIN>(a, st); break;
    case 5: if constexpr (NR >= 3) return launch_kernel<D, NR, REF, 5, AQ, CHAIN>(a, st); break;
    case 6: if constexpr (NR >= 3) return launch_kernel<D, NR, REF, 6, AQ, CHAIN>(a, st); break;
    case 7: if constexpr (NR >= 3) return launch_kernel<D, NR, REF, 7, AQ, CHAIN>(a, st); break;
  }
  return hipErrorInvalidValue;
}

// One decode pass at head_dim D with reference kind AQ (0: BF16 rows; 2, 4:
// anchor bits), chained references or not.  Each (D, AQ, CHAIN) is
// instantiated in an object file of its own (rq_decode_inst.hip).
template <int D, int AQ, int CHAIN>
hipError_t launch_decode_d(const DecodeArgs &a, int n_res, bool ref, hipStream_t st) {
  if constexpr (CHAIN == 2) {       // slot 0 alone: never the reference slot
    switch (ref ? -1 : n_res) {
      case 1: return launch_bits<D, 1, false, AQ, CHAIN>(a, st);
      case 2: return launch_bits<D, 2, false, AQ, CHAIN>(a, st);
      case 3: return launch_bits<D, 3, false, AQ, CHAIN>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if (ref) {
    switch (n_res) {
      case 0: return launch_bits<D, 0, true, AQ, CHAIN>(a, st);
      case 1: return launch_bits<D, 1, true, AQ, CHAIN>(a, st);
      case 2: return launch_bits<D, 2, true, AQ, CHAIN>(a, st);
      case 3: return launch_bits<D, 3, true, AQ, CHAIN>(a, st);
    }
  } else {
    switch (n_res) {
      case 1: return launch_bits<D, 1, false, AQ, CHAIN>(a, st);
      case 2: return launch_bits<D, 2, false, AQ, CHAIN>(a, st);
      case 3: return launch_bits<D, 3, false, AQ, CHAIN>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

// Resident workgroups per compute unit of the main decode kernel at head_dim
// D (4-wave workgroups, a full pass over a BF16 reference), or -1 on a HIP
// error.
template <int D>
int decode_blocks_per_cu_d() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, decode_kernel<D, kMaxRes, true, 0, kTilesPerIter, kWaves, 0, 0>, 64 * kWaves, 0) != hipSuccess)
    return -1;
  return n;
}

}  // namespace rq
