// rq_encode.hip -- ResidualQuant encoder for gfx950.
//
// ResidualQuant page ("ResidualQuant: KV Cache Quantization for Looped
// Transformers with 2-Bit Residuals"), Fig. 1 steps 2-5: every earlier loop's
// K/V vector becomes a least-squares-scaled residual against the final loop,
// is rotated, and is quantized per group of g dims at that loop's bit width.
// With a quantized anchor (Fig. 3 caption, "Ascending [2,2,2,4]"; Table 8
// caption) the final loop is first quantized the same way (no LS
// coefficient) and the residuals are taken against its dequantized value.
//
// Mapping: one head_dim vector per D/8 consecutive lanes, 8 consecutive dims
// per lane (one 128-bit load), 64/(D/8) tokens per wave.  A wave handles all
// residual loops of its tokens, so each reference vector is read once.  The
// FP32 arithmetic is the library's bit-exact contract: the same IEEE
// operations in the same order as the sequential definition, no contraction
// (fp contract off below), explicit fma where the contract has one.

#pragma clang fp contract(off)

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {

// Dot-product term sum in the contract order: pairwise halving inside the
// lane's block of 8, then pairwise halving over the D/8 lanes (largest
// distance first).  Every lane of the vector receives the same bits, since
// IEEE addition is commutative.
template <int LANES>
__device__ __forceinline__ float dot_sum(float (&t)[8]) {
  float a0 = t[0] + t[4], a1 = t[1] + t[5], a2 = t[2] + t[6], a3 = t[3] + t[7];
  float b0 = a0 + a2, b1 = a1 + a3;
  float s = b0 + b1;
  if constexpr (LANES >= 32) s = s + xor_lane<16>(s);
  if constexpr (LANES >= 16) s = s + xor_lane<8>(s);
  if constexpr (LANES >= 8) s = s + xor_lane<4>(s);
  if constexpr (LANES >= 4) s = s + xor_lane<2>(s);
  if constexpr (LANES >= 2) s = s + xor_lane<1>(s);
  return s;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 w, float (&f)[8]) {
  f[0] = bf16lo(w.x); f[1] = bf16hi(w.x);
  f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
  f[4] = bf16lo(w.z); f[5] = bf16hi(w.z);
  f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
}

// Group quantization of the lane's 8 values (already rotated if the layout
// rotates): canonicalise -0 to +0, group min/max over the gl lanes of the
// group, FP16 scale and offset, codes by round-half-even of (u - z) * (1/s)
// clamped to the grid.  Returns the packed code word (code p at bits
// [bits*p, +bits)); q receives the codes as floats.
__device__ __forceinline__ uint32_t quantize8(float (&u)[8], int bits, int gl, uint32_t &s16,
                                              uint32_t &z16, float (&q)[8]) {
#pragma unroll
  for (int p = 0; p < 8; ++p) u[p] = u[p] + 0.0f;   // -0 -> +0
  float mn = u[0], mx = u[0];
#pragma unroll
  for (int p = 1; p < 8; ++p) { mn = fminf(mn, u[p]); mx = fmaxf(mx, u[p]); }
  if (gl == 4) { mn = group_min<4>(mn); mx = group_max<4>(mx); }
  else         { mn = group_min<2>(mn); mx = group_max<2>(mx); }
  const float levels = (float)((1 << bits) - 1);
  s16 = f32_to_f16_sat((mx - mn) / levels);
  z16 = f32_to_f16_sat(mn);
  const float s = f16_to_f32(s16);
  const float z = f16_to_f32(z16);
  uint32_t word = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) q[p] = 0.0f;
  if (s != 0.0f) {
    const float inv = 1.0f / s;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      float c = __builtin_rintf((u[p] - z) * inv);
      c = fminf(fmaxf(c, 0.0f), levels);
      q[p] = c;
      word |= (uint32_t)c << (bits * p);
    }
  }
  return word;
}

template <int D>
__device__ __forceinline__ void store_codes(uint8_t *plane, size_t slot, int j, int bits, uint32_t word) {
  if (bits == 2)
    reinterpret_cast<uint16_t *>(plane + slot * (D / 4))[j] = (uint16_t)word;
  else
    reinterpret_cast<uint32_t *>(plane + slot * (D / 2))[j] = word;
}

template <int D>
__global__ __launch_bounds__(256) void encode_kernel(const EncodeArgs a) {
  constexpr int LANES = D / 8;
  constexpr int VPW = kWave / LANES;
  const int lane = threadIdx.x & 63;
  const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= 2 * a.tasks_per_side) return;          // whole wave
  const int side = task >= a.tasks_per_side ? 1 : 0;
  const int tk = task - side * a.tasks_per_side;
  const int bh = tk / a.chunks;
  const int chunk = tk - bh * a.chunks;
  const int j = lane % LANES;
  const int tl = chunk * VPW + lane / LANES;         // token within [0, n)
  const bool valid = tl < a.n;
  const int tlc = valid ? tl : a.n - 1;              // in-bounds stand-in for loads
  const size_t slot = (size_t)bh * a.cap + (size_t)(a.t0 + tlc);
  const EncodeSide &S = a.side[side];
  const int G = D / a.group;
  const int gl = a.group / 8;                        // lanes per group

  float y[8];
  if (a.abits == 0) {
    unpack_bf16x8(*reinterpret_cast<const uint4 *>(S.ref + slot * D + 8 * j), y);
  } else {
    // the anchor: loop L-1 of the input, quantized like a residual (groups of
    // agroup, no LS coefficient); y becomes its dequantized value
    const uint16_t *yp = S.xin[a.n_res] + ((size_t)bh * a.n + tlc) * D + 8 * j;
    unpack_bf16x8(*reinterpret_cast<const uint4 *>(yp), y);
    if (a.rotate) {
      wht8<D>(y, lane);
#pragma unroll
      for (int p = 0; p < 8; ++p) y[p] = y[p] * a.rot_c;
    }
    uint32_t s16, z16;
    float q[8];
    const int agl = a.agroup / 8;
    const uint32_t word = quantize8(y, a.abits, agl, s16, z16, q);
    if (valid) {
      const size_t oslot = (size_t)bh * a.cap + (size_t)(a.t0 + tl);
      store_codes<D>(S.codes[a.n_res], oslot, j, a.abits, word);
      if (j % agl == 0) S.meta[a.n_res][oslot * (D / a.agroup) + j / agl] = s16 | (z16 << 16);
    }
    const float s = f16_to_f32(s16), z = f16_to_f32(z16);
#pragma unroll
    for (int p = 0; p < 8; ++p) y[p] = __builtin_fmaf(q[p], s, z);
    if (a.rotate) {
      wht8<D>(y, lane);
#pragma unroll
      for (int p = 0; p < 8; ++p) y[p] = y[p] * a.rot_c;
    }
  }
  float t[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) t[p] = y[p] * y[p];    // exact for a BF16 y
  const float den = dot_sum<LANES>(t);

  for (int l = 0; l < a.n_res; ++l) {
    const uint16_t *xp = S.xin[l] + ((size_t)bh * a.n + tlc) * D + 8 * j;
    float x[8];
    unpack_bf16x8(*reinterpret_cast<const uint4 *>(xp), x);
    float alpha32;
    if (a.alpha_mode == 1) {
      alpha32 = 1.0f;
    } else if (a.alpha_mode == 2) {                    // ||x|| / ||y||
#pragma unroll
      for (int p = 0; p < 8; ++p) t[p] = x[p] * x[p];
      const float nx = dot_sum<LANES>(t);
      alpha32 = den > 0.0f ? __builtin_sqrtf(nx) / __builtin_sqrtf(den) : 0.0f;
    } else {                                           // <x,y> / <y,y>
#pragma unroll
      for (int p = 0; p < 8; ++p) t[p] = x[p] * y[p];
      const float num = dot_sum<LANES>(t);
      alpha32 = den > 0.0f ? num / den : 0.0f;
    }
    const uint32_t a16 = f32_to_f16_sat(alpha32);
    const float af = f16_to_f32(a16);

    float u[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) u[p] = __builtin_fmaf(-af, y[p], x[p]);
    if (a.rotate) {
      wht8<D>(u, lane);
#pragma unroll
      for (int p = 0; p < 8; ++p) u[p] = u[p] * a.rot_c;
    }
    const int bits = a.bits[l];
    uint32_t s16, z16;
    float q[8];
    const uint32_t word = quantize8(u, bits, gl, s16, z16, q);
    if (valid) {
      const size_t oslot = (size_t)bh * a.cap + (size_t)(a.t0 + tl);
      store_codes<D>(S.codes[l], oslot, j, bits, word);
      if (j % gl == 0) S.meta[l][oslot * G + j / gl] = s16 | (z16 << 16);
      if (j == 0) S.alpha[l][oslot] = (uint16_t)a16;
    }
  }
}

hipError_t launch_encode(const EncodeArgs &a, int head_dim, hipStream_t s) {
  const int tasks = 2 * a.tasks_per_side;
  const dim3 grid((tasks + 3) / 4), block(256);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(encode_kernel<64>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(encode_kernel<128>, grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL(encode_kernel<256>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rq
