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
// Mapping: one head_dim vector per D/32 consecutive lanes, 32 consecutive dims
// per lane, 64/(D/32) tokens per wave.  A wave handles all residual loops of
// its tokens, so each reference vector is read once.  The
// FP32 arithmetic is the library's bit-exact contract: the same IEEE
// operations in the same order as the sequential definition, no contraction
// (fp contract off below), explicit fma where the contract has one.

#pragma clang fp contract(off)

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {

// Lane mapping: 32 consecutive dims of one vector per lane (four 128-bit
// loads), D/32 lanes per vector, 64/(D/32) vectors per wave.  With this many
// dims in a lane, 5 of the 7 butterfly stages of a 128-point Hadamard
// transform, the group min/max (g <= 32) and most of each dot product stay in
// the lane.
constexpr int EPL = kEncodeElemsPerLane;

__device__ __forceinline__ void load_bf16x32(const uint16_t *p, float (&f)[EPL]) {
  const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
  for (int k = 0; k < EPL / 8; ++k) {
    const uint4 w = q[k];
    f[8 * k + 0] = bf16lo(w.x); f[8 * k + 1] = bf16hi(w.x);
    f[8 * k + 2] = bf16lo(w.y); f[8 * k + 3] = bf16hi(w.y);
    f[8 * k + 4] = bf16lo(w.z); f[8 * k + 5] = bf16hi(w.z);
    f[8 * k + 6] = bf16lo(w.w); f[8 * k + 7] = bf16hi(w.w);
  }
}

// sum_i a[i] * b[i] over the whole vector in the contract order: each block
// of 8 consecutive products by pairwise halving (distances 4, 2, 1), then the
// D/8 block sums by pairwise halving from the largest distance.  The lane
// holds blocks 4j..4j+3, so the block tree first pairs lanes (block distance
// 4m is lane distance m), then finishes in the lane.  Both lanes of a pair
// add the same two values (IEEE addition is commutative), so every lane of
// the vector ends with the same bits.
template <int LANES>
__device__ __forceinline__ float dot_sum32(const float (&a)[EPL], const float (&b)[EPL]) {
  float bs[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float t[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) t[p] = a[8 * k + p] * b[8 * k + p];
    const float a0 = t[0] + t[4], a1 = t[1] + t[5], a2 = t[2] + t[6], a3 = t[3] + t[7];
    bs[k] = (a0 + a2) + (a1 + a3);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (LANES >= 8) bs[k] = bs[k] + xor_lane<4>(bs[k]);
    if constexpr (LANES >= 4) bs[k] = bs[k] + xor_lane<2>(bs[k]);
    if constexpr (LANES >= 2) bs[k] = bs[k] + xor_lane<1>(bs[k]);
  }
  return (bs[0] + bs[2]) + (bs[1] + bs[3]);
}

// Unnormalized Walsh-Hadamard transform of the vector: butterflies
// h = 1, ..., 16 inside the lane, then h = 32, 64, 128 across lanes at lane
// distances 1, 2, 4, ascending as in the sequential definition.
template <int LANES>
__device__ __forceinline__ void fwht32(float (&v)[EPL], int lane) {
#pragma unroll
  for (int h = 1; h < EPL; h *= 2) {
#pragma unroll
    for (int j = 0; j < EPL; j += 2 * h) {
#pragma unroll
      for (int i = j; i < j + h; ++i) {
        const float x = v[i], y = v[i + h];
        v[i] = x + y;
        v[i + h] = x - y;
      }
    }
  }
#pragma unroll
  for (int p = 0; p < EPL; ++p) {
    if constexpr (LANES >= 2) v[p] = wht_stage<1>(v[p], lane);
    if constexpr (LANES >= 4) v[p] = wht_stage<2>(v[p], lane);
    if constexpr (LANES >= 8) v[p] = wht_stage<4>(v[p], lane);
  }
}

// Quantize one group of N values of the lane (rotated if the layout rotates,
// and -0 already canonicalised to +0): min/max, FP16 scale and offset, codes
// by round-half-even of (u - z) * (1/s) clamped to the grid (all 0 if the
// stored scale is 0).  q receives the codes as floats.
template <int N>
__device__ __forceinline__ void quantize_group(float *u, int bits, uint32_t &s16, uint32_t &z16, float *q) {
  float mn = u[0], mx = u[0];
#pragma unroll
  for (int p = 1; p < N; ++p) { mn = fminf(mn, u[p]); mx = fmaxf(mx, u[p]); }
  const float levels = (float)((1 << bits) - 1);
  s16 = f32_to_f16_sat((mx - mn) / levels);
  z16 = f32_to_f16_sat(mn);
  const float s = f16_to_f32(s16);
  const float z = f16_to_f32(z16);
  if (s != 0.0f) {
    const float inv = 1.0f / s;
#pragma unroll
    for (int p = 0; p < N; ++p) q[p] = __builtin_amdgcn_fmed3f(__builtin_rintf((u[p] - z) * inv), 0.0f, levels);
  } else {
#pragma unroll
    for (int p = 0; p < N; ++p) q[p] = 0.0f;
  }
}

// The values a group quantizer sees: c * H u when rotating, u otherwise, with
// -0 turned into +0.  fma(v, c, +0) is the rounded product c*v except that a
// zero product comes out +0, so one instruction scales and canonicalises.
template <int LANES>
__device__ __forceinline__ void rotate_canonical(float (&v)[EPL], int rotate, float rot_c, int lane) {
  if (rotate) {
    fwht32<LANES>(v, lane);
#pragma unroll
    for (int p = 0; p < EPL; ++p) v[p] = __builtin_fmaf(v[p], rot_c, 0.0f);
  } else {
#pragma unroll
    for (int p = 0; p < EPL; ++p) v[p] = v[p] + 0.0f;
  }
}

// Quantize the lane's 32 values in groups of `group` (16 or 32), store the
// packed codes (code p of the lane at bits [bits*p, +bits) of its
// 32*bits/8-byte slice, LSB first) and the (scale | zero << 16) words of its
// groups.  q receives the codes.
template <int D>
__device__ __forceinline__ void quantize_store(float (&u)[EPL], int bits, int group, float (&q)[EPL],
                                               uint32_t (&sz)[2], uint8_t *codes, uint32_t *meta,
                                               size_t oslot, int j, bool valid) {
  uint32_t s16[2], z16[2];
  int ng;
  if (group == 32) {
    quantize_group<32>(u, bits, s16[0], z16[0], q);
    ng = 1;
  } else {
    quantize_group<16>(u, bits, s16[0], z16[0], q);
    quantize_group<16>(u + 16, bits, s16[1], z16[1], q + 16);
    ng = 2;
  }
  sz[0] = s16[0] | (z16[0] << 16);
  sz[1] = ng == 2 ? (s16[1] | (z16[1] << 16)) : sz[0];
  if (!valid) return;
  if (bits == 2) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      w0 |= (uint32_t)q[p] << (2 * p);
      w1 |= (uint32_t)q[16 + p] << (2 * p);
    }
    *reinterpret_cast<uint2 *>(codes + oslot * (D / 4) + 8 * j) = make_uint2(w0, w1);
  } else {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < EPL; ++p) w[p / 8] |= (uint32_t)q[p] << (4 * (p % 8));
    *reinterpret_cast<uint4 *>(codes + oslot * (D / 2) + 16 * j) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  const int G = D / group;
  if (ng == 1) meta[oslot * G + j] = sz[0];
  else *reinterpret_cast<uint2 *>(meta + oslot * G + 2 * j) = make_uint2(sz[0], sz[1]);
}

template <int D>
__global__ __launch_bounds__(256) void encode_kernel(const EncodeArgs a) {
  constexpr int LANES = D / EPL;
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
  const size_t oslot = (size_t)bh * a.cap + (size_t)(a.t0 + tl);
  const EncodeSide &S = a.side[side];
  const size_t xrow = ((size_t)bh * a.n + tlc) * D + EPL * j;

  float y[EPL];
  if (a.abits == 0) {
    load_bf16x32(S.ref + slot * D + EPL * j, y);
  } else {
    // the anchor: its input (index n_res) quantized like a residual (groups
    // of agroup, no LS coefficient); y becomes its dequantized value
    load_bf16x32(S.xin[a.n_res] + xrow, y);
    rotate_canonical<LANES>(y, a.rotate, a.rot_c, lane);
    float q[EPL];
    uint32_t sz[2];
    quantize_store<D>(y, a.abits, a.agroup, q, sz, S.codes[a.n_res], S.meta[a.n_res], oslot, j, valid);
#pragma unroll
    for (int p = 0; p < EPL; ++p) {
      const uint32_t w = (a.agroup == 32 || p < 16) ? sz[0] : sz[1];
      y[p] = __builtin_fmaf(q[p], f16_to_f32(w & 0xffffu), f16_to_f32(w >> 16));
    }
    if (a.rotate) {
      fwht32<LANES>(y, lane);
#pragma unroll
      for (int p = 0; p < EPL; ++p) y[p] = y[p] * a.rot_c;
    }
  }
  float den = dot_sum32<LANES>(y, y);                // exact products for a BF16 y

  for (int l = 0; l < a.n_res; ++l) {
    float x[EPL];
    load_bf16x32(S.xin[l] + xrow, x);
    float alpha32;
    if (a.alpha_mode == 1) {
      alpha32 = 1.0f;
    } else if (a.alpha_mode == 2) {                    // ||x|| / ||y||
      const float nx = dot_sum32<LANES>(x, x);
      alpha32 = den > 0.0f ? __builtin_sqrtf(nx) / __builtin_sqrtf(den) : 0.0f;
    } else {                                           // <x,y> / <y,y>
      const float num = dot_sum32<LANES>(x, y);
      alpha32 = den > 0.0f ? num / den : 0.0f;
    }
    const uint32_t a16 = f32_to_f16_sat(alpha32);
    const float af = f16_to_f32(a16);
#pragma unroll
    for (int p = 0; p < EPL; ++p) x[p] = __builtin_fmaf(-af, y[p], x[p]);
    rotate_canonical<LANES>(x, a.rotate, a.rot_c, lane);
    float q[EPL];
    uint32_t sz[2];
    quantize_store<D>(x, a.bits[l], a.group, q, sz, S.codes[l], S.meta[l], oslot, j, valid);
    if (valid && j == 0) S.alpha[l][oslot] = (uint16_t)a16;
    if (a.chain && l + 1 < a.n_res) {
      // chained references: the next loop's reference is this loop's
      // reconstruction, y <- fma(alpha, y, r_hat), r_hat = c*H(fma(code, s, z))
#pragma unroll
      for (int p = 0; p < EPL; ++p) {
        const uint32_t w = (a.group == 32 || p < 16) ? sz[0] : sz[1];
        x[p] = __builtin_fmaf(q[p], f16_to_f32(w & 0xffffu), f16_to_f32(w >> 16));
      }
      if (a.rotate) {
        fwht32<LANES>(x, lane);
#pragma unroll
        for (int p = 0; p < EPL; ++p) x[p] = x[p] * a.rot_c;
      }
#pragma unroll
      for (int p = 0; p < EPL; ++p) y[p] = __builtin_fmaf(af, y[p], x[p]);
      den = dot_sum32<LANES>(y, y);
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
