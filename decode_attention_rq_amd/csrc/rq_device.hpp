// rq_device.hpp -- device helpers shared by the gfx950 kernels of librq.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

// Low / high bf16 of a packed pair, widened exactly to fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default
// rounding mode), saturating an infinite result to +-65504.
__device__ __forceinline__ uint32_t f32_to_f16_sat(float x) {
  uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)x);
  if ((h & 0x7fffu) == 0x7c00u) h = (h & 0x8000u) | 0x7bffu;
  return h;
}

// ---------------------------------------------------------------------------
// lane exchange
// ---------------------------------------------------------------------------

// DPP lane moves inside a 16-lane row (VALU only, no LDS traffic).  Every
// control used here is a full permutation or broadcast within each row, so
// no lane reads an invalid source and the destination needs no old value
// (no zero-initialising move; a move feeding an add fuses into it).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;    // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

constexpr int kDppQuadReverse = 0x1B;    // quad_perm [3,2,1,0]
constexpr int kDppRowRor4 = 0x124;       // lane i <- lane (i - 4) mod 16 within each 16 lanes
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane (i - 8) mod 16

// Value of `x` in lane (lane ^ mask).  Masks 1 and 2 are one DPP quad
// permutation; 4 is the half-row mirror (i -> 7-i) after a quad reversal
// (4a+b -> 4a+3-b), 8 the row mirror (i -> 15-i) after the half-row mirror:
// VALU moves, no LDS traffic.  16 uses ds_swizzle (bitmask mode, no LDS
// allocation) and 32 ds_bpermute.
template <int MASK>
__device__ __forceinline__ float xor_lane(float x) {
  static_assert(MASK > 0 && MASK < 64 && (MASK & (MASK - 1)) == 0, "power-of-two lane mask");
  if constexpr (MASK == 1) {
    return dpp<kDppQuadXor1>(x);
  } else if constexpr (MASK == 2) {
    return dpp<kDppQuadXor2>(x);
  } else if constexpr (MASK == 4) {
    return dpp<kDppHalfMirror>(dpp<kDppQuadReverse>(x));
  } else if constexpr (MASK == 8) {
    return dpp<kDppRowMirror>(dpp<kDppHalfMirror>(x));
  } else if constexpr (MASK < 32) {
    // offset[15] = 0: and_mask = 0x1f, or_mask = 0, xor_mask = MASK
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x),
                                                                  0x1f | (MASK << 10)));
  } else {
    int src = (int)(__lane_id() ^ MASK) << 2;
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, x)));
  }
}

template <int MASK>
__device__ __forceinline__ uint32_t xor_lane_u(uint32_t x) {
  return __builtin_bit_cast(uint32_t, xor_lane<MASK>(__builtin_bit_cast(float, x)));
}

// Sum over aligned groups of N lanes (N a power of two <= 64), every lane of
// the group receiving the total (xor butterfly).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += xor_lane<1>(x);
  if constexpr (N >= 4) x += xor_lane<2>(x);
  if constexpr (N >= 8) x += xor_lane<4>(x);
  if constexpr (N >= 16) x += xor_lane<8>(x);
  if constexpr (N >= 32) x += xor_lane<16>(x);
  if constexpr (N >= 64) x += xor_lane<32>(x);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, xor_lane<1>(x));
  if constexpr (N >= 4) x = fmaxf(x, xor_lane<2>(x));
  if constexpr (N >= 8) x = fmaxf(x, xor_lane<4>(x));
  if constexpr (N >= 16) x = fmaxf(x, xor_lane<8>(x));
  if constexpr (N >= 32) x = fmaxf(x, xor_lane<16>(x));
  if constexpr (N >= 64) x = fmaxf(x, xor_lane<32>(x));
  return x;
}

template <int N>
__device__ __forceinline__ float group_min(float x) {
  if constexpr (N >= 2) x = fminf(x, xor_lane<1>(x));
  if constexpr (N >= 4) x = fminf(x, xor_lane<2>(x));
  if constexpr (N >= 8) x = fminf(x, xor_lane<4>(x));
  if constexpr (N >= 16) x = fminf(x, xor_lane<8>(x));
  if constexpr (N >= 32) x = fminf(x, xor_lane<16>(x));
  if constexpr (N >= 64) x = fminf(x, xor_lane<32>(x));
  return x;
}

// Sum over aligned groups of N in {8, 16, 32} lanes, every lane receiving
// the total.  After the quad sums, a mirror pairs each lane with one in the
// other half of its 8 (then 16) lanes.
template <int N>
__device__ __forceinline__ float group_sum_dpp(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "group of 8, 16 or 32 lanes");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N >= 32) x += xor_lane<16>(x);
  return x;
}

// One cross-lane butterfly stage of the Walsh-Hadamard transform: element i
// of this lane pairs with element i of lane (lane ^ MASK).  The lane with the
// MASK bit clear holds the lower index a and keeps a + b; its partner, holding
// b, keeps a - b.  Both are the partner's value plus this lane's value, the
// upper lane's sign flipped: b + a = a + b (IEEE addition is commutative) and
// a + (-b) = a - b, so the results are those of the sequential definition.
template <int MASK>
__device__ __forceinline__ float wht_stage(float own, int lane) {
  const float other = xor_lane<MASK>(own);
  const uint32_t flip = (lane & MASK) ? 0x80000000u : 0u;
  return other + __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, own) ^ flip);
}

// In-register Walsh-Hadamard transform (unnormalized) of a D-vector spread
// over D/8 consecutive lanes, 8 consecutive elements per lane (element
// 8*(lane % (D/8)) + p in v[p]).  Stages run h = 1, 2, 4 inside the lane,
// then h = 8, 16, ... across lanes.
template <int D>
__device__ __forceinline__ void wht8(float (&v)[8], int lane) {
#pragma unroll
  for (int h = 1; h < 8; h *= 2) {
#pragma unroll
    for (int j = 0; j < 8; j += 2 * h) {
#pragma unroll
      for (int i = j; i < j + h; ++i) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  constexpr int LANES = D / 8;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if constexpr (LANES >= 2) v[p] = wht_stage<1>(v[p], lane);
    if constexpr (LANES >= 4) v[p] = wht_stage<2>(v[p], lane);
    if constexpr (LANES >= 8) v[p] = wht_stage<4>(v[p], lane);
    if constexpr (LANES >= 16) v[p] = wht_stage<8>(v[p], lane);
    if constexpr (LANES >= 32) v[p] = wht_stage<16>(v[p], lane);
  }
}

}  // namespace rq
