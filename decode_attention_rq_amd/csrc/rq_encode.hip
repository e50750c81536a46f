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
// its tokens, so each reference vector is read once.  The FP32 arithmetic is
// the library's bit-exact contract: the results of the sequential
// definition's IEEE operations in its order, no contraction (fp contract off
// below), explicit fma where the contract has one.  Two quotients (a group's
// scale, its code factor) are formed without a divide instruction, by fma
// identities that give the IEEE quotient's bits for every input they see.

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

// One cross-lane stage of the sign-folded transform at lane distance M (1 or
// 2): w = dpp(w) * s + w for every value, one v_fmac_f32 with a DPP source
// each (s = -1 on the lane whose bit M is set, +1 on its partner; the
// product is exact, so the sum is rounded once, as an add).  Written as
// assembly because the compiler does not combine a lane move into an FMA.
// Each block begins with two wait states (a DPP instruction must not read a
// register the previous VALU instruction wrote); inside a block every
// instruction reads only its own value, written before the block.
template <int M>
__device__ __forceinline__ void fmac_dpp_stage(float (&v)[EPL], float s) {
  static_assert(M == 1 || M == 2, "quad_perm lane distances");
#pragma unroll
  for (int o = 0; o < EPL; o += 16) {
    if constexpr (M == 1) {
      asm volatile(
        "s_nop 1\n"
        "v_fmac_f32_dpp %0, %0, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %1, %1, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %2, %2, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %3, %3, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %4, %4, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %5, %5, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %6, %6, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %7, %7, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %8, %8, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %9, %9, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %10, %10, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %11, %11, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %12, %12, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %13, %13, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %14, %14, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %15, %15, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        : "+v"(v[o + 0]), "+v"(v[o + 1]), "+v"(v[o + 2]), "+v"(v[o + 3]), "+v"(v[o + 4]), "+v"(v[o + 5]), "+v"(v[o + 6]), "+v"(v[o + 7]), "+v"(v[o + 8]), "+v"(v[o + 9]), "+v"(v[o + 10]), "+v"(v[o + 11]), "+v"(v[o + 12]), "+v"(v[o + 13]), "+v"(v[o + 14]), "+v"(v[o + 15])
        : "v"(s));
    } else {
      asm volatile(
        "s_nop 1\n"
        "v_fmac_f32_dpp %0, %0, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %1, %1, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %2, %2, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %3, %3, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %4, %4, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %5, %5, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %6, %6, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %7, %7, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %8, %8, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %9, %9, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %10, %10, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %11, %11, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %12, %12, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %13, %13, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %14, %14, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %15, %15, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        : "+v"(v[o + 0]), "+v"(v[o + 1]), "+v"(v[o + 2]), "+v"(v[o + 3]), "+v"(v[o + 4]), "+v"(v[o + 5]), "+v"(v[o + 6]), "+v"(v[o + 7]), "+v"(v[o + 8]), "+v"(v[o + 9]), "+v"(v[o + 10]), "+v"(v[o + 11]), "+v"(v[o + 12]), "+v"(v[o + 13]), "+v"(v[o + 14]), "+v"(v[o + 15])
        : "v"(s));
    }
  }
}

// Unnormalized Walsh-Hadamard transform of the vector: butterflies
// h = 1, ..., 16 inside the lane, then h = 32, 64, 128 across lanes at lane
// distances 1, 2, 4, ascending as in the sequential definition.  In each
// cross-lane stage the partner's value enters multiplied by s, the lane's
// own as is (lane distances 1 and 2 as above, 4 through the lane moves of
// xor_lane), instead of flipping the sign of the own value on the lane that
// subtracts (one instruction per value, not two).  The lane whose bit of the
// stage is set then holds its butterfly output negated (partner - own =
// -(own's output), rounded alike), and later stages keep that sign, since
// both lanes of a pair carry the same one.  Returns the lane's resulting
// sign (+-1) for the caller to fold into its scaling.  A zero may come out
// with the other sign, so only a caller that turns zeros into +0 afterwards
// may use it.
template <int LANES>
__device__ __forceinline__ float fwht32_signed(float (&v)[EPL], int lane) {
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
  float sign = 1.0f;
  if constexpr (LANES >= 2) {
    const float s = (lane & 1) ? -1.0f : 1.0f;
    fmac_dpp_stage<1>(v, s);
    sign *= s;
  }
  if constexpr (LANES >= 4) {
    const float s = (lane & 2) ? -1.0f : 1.0f;
    fmac_dpp_stage<2>(v, s);
    sign *= s;
  }
  if constexpr (LANES >= 8) {
    const float s = (lane & 4) ? -1.0f : 1.0f;
#pragma unroll
    for (int p = 0; p < EPL; ++p) v[p] = __builtin_fmaf(xor_lane<4>(v[p]), s, v[p]);
    sign *= s;
  }
  return sign;
}

// Raw buffer access: a wave-uniform base address and byte count in SGPRs, a
// 32-bit byte offset per lane (no 64-bit address registers).  Accesses at or
// beyond the byte count are dropped by the hardware (loads return 0).  Word 3
// selects the untyped 32-bit data format of plain buffer_load/store_dword*.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void load_raw32(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t (&w)[EPL / 8]) {
#pragma unroll
  for (int k = 0; k < EPL / 8; ++k) w[k] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 16 * k, 0);
}

__device__ __forceinline__ void unpack_raw32(const u32x4_t (&w)[EPL / 8], float (&f)[EPL]) {
#pragma unroll
  for (int k = 0; k < EPL / 8; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[8 * k + 2 * e] = bf16lo(w[k][e]);
      f[8 * k + 2 * e + 1] = bf16hi(w[k][e]);
    }
  }
}

// c * H v for a reconstruction (the dequantized anchor, a chain link's
// residual).  Its inputs fma(code, s, z) are never -0 (code, s >= 0 and z is
// the min of values whose zeros are +0), so every zero of the sequential
// transform, and of its product with c > 0, is +0; the sign-folded transform
// followed by fma(v, +-c, +0), which turns any zero into +0, therefore gives
// the same bits.
template <int LANES>
__device__ __forceinline__ void rotate_rebuilt(float (&v)[EPL], float rot_c, int lane) {
  const float c = rot_c * fwht32_signed<LANES>(v, lane);
#pragma unroll
  for (int p = 0; p < EPL; ++p) v[p] = __builtin_fmaf(v[p], c, 0.0f);
}

// The values a group quantizer sees: c * H u when rotating, u otherwise, with
// -0 turned into +0.  fma(v, c, +0) is the rounded product c*v except that a
// zero product comes out +0, so one instruction scales and canonicalises.
template <int LANES>
__device__ __forceinline__ void rotate_canonical(float (&v)[EPL], int rotate, float rot_c, int lane) {
  if (rotate) {
    const float c = rot_c * fwht32_signed<LANES>(v, lane);   // exact: the sign is +-1
#pragma unroll
    for (int p = 0; p < EPL; ++p) v[p] = __builtin_fmaf(v[p], c, 0.0f);
  } else {
#pragma unroll
    for (int p = 0; p < EPL; ++p) v[p] = v[p] + 0.0f;
  }
}

// range / L for the level count L = 2^b - 1 (3 or 15) of a group's range
// x >= 0, bit-identical to the IEEE quotient without a divide sequence:
// q = RN(x * RN(1/L)) is within an ulp of x / L, the residual x - q*L is exact
// in one fma, and one fma correction rounds to the quotient.  The identity
// holds for every float x in [0, 2^120] and both level counts (an exhaustive
// host check in the test suite); a larger range, infinite included, is
// clamped to 2^120 first, whose quotient saturates binary16 as the IEEE one
// does.
template <int L>
__device__ __forceinline__ float div_levels(float x) {
  constexpr float r = 1.0f / (float)L;
  x = fminf(x, 0x1p120f);
  const float q = x * r;
  const float e = __builtin_fmaf(-q, (float)L, x);
  return __builtin_fmaf(e, r, q);
}

// 1/s for a stored binary16 scale s > 0, bit-identical to the IEEE quotient:
// v_rcp_f32 is within an ulp of 1/s, and one fma Newton step from any value
// within 2 ulp rounds to 1/s for every positive finite binary16 s (an
// exhaustive host check in the test suite).
__device__ __forceinline__ float recip_f16_value(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-r0, s, 1.0f);
  return __builtin_fmaf(e, r0, r0);
}

// One group of N values of the lane (rotated if the layout rotates, -0
// already canonicalised to +0): min/max, then the FP16 scale s = (max-min)/
// (2^b - 1) and offset z = min as stored, and the factor the codes use, 1/s
// (0 when the stored scale is 0, which makes every code 0).  Both conversions
// round to nearest even and saturate at +-65504: clamping to +-65504 first and
// converting gives the same half as converting and replacing an infinity.
template <int N, int L>
__device__ __forceinline__ void group_params(const float *u, uint32_t &sz, float &s, float &z, float &inv) {
  float mn = u[0], mx = u[0];
#pragma unroll
  for (int p = 1; p < N; ++p) { mn = fminf(mn, u[p]); mx = fmaxf(mx, u[p]); }
  const uint32_t s16 = __builtin_bit_cast(uint16_t, (_Float16)fminf(div_levels<L>(mx - mn), 65504.0f));
  const uint32_t z16 = __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_fmed3f(mn, -65504.0f, 65504.0f));
  s = f16_to_f32(s16);
  z = f16_to_f32(z16);
  inv = s != 0.0f ? recip_f16_value(s) : 0.0f;
  sz = s16 | (z16 << 16);
}

// Quantize the lane's 32 values in groups of `group` (16 or 32): code =
// round-half-even of (u - z) * (1/s), clamped to [0, 2^b - 1].  Stores the
// packed codes (code p of the lane at bits [b*p, +b) of its 32*b/8-byte
// slice, LSB first) and the (scale | zero << 16) words of its groups.  With
// DEQ, u becomes the dequantized values fma(code, s, z) (for a reference
// that a later step rebuilds).
//
// Clamping before rounding gives the same code as rounding first, as both
// bounds are integers.  v_cvt_pk_u8_f32 rounds to nearest even (the default
// mode) and writes the code into a chosen byte of a word, so one instruction
// per code rounds and places it: byte i of plane word m collects the codes
// that land in byte i of an output word, and shifted ORs of the planes
// interleave them into 2- or 4-bit fields.  cr / mr address the code and meta
// planes from the wave's first token; tok is the lane's token relative to it.
template <int D, int BITS, bool DEQ>
__device__ __forceinline__ void quantize_pack(float (&u)[EPL], int group, __amdgpu_buffer_rsrc_t cr,
                                              __amdgpu_buffer_rsrc_t mr, uint32_t tok, int j, bool valid) {
  constexpr int L = (1 << BITS) - 1;
  constexpr int PER_BYTE = 8 / BITS;                  // codes per output byte
  constexpr int NW = EPL * BITS / 32;                 // output words per lane
  uint32_t sz[2];
  float sc[2], z[2], inv[2];
  if (group == 32) {
    group_params<32, L>(u, sz[0], sc[0], z[0], inv[0]);
    sz[1] = sz[0]; sc[1] = sc[0]; z[1] = z[0]; inv[1] = inv[0];
  } else {
    group_params<16, L>(u, sz[0], sc[0], z[0], inv[0]);
    group_params<16, L>(u + 16, sz[1], sc[1], z[1], inv[1]);
  }
  // plane[k][m], byte i = code 32*k/BITS + PER_BYTE*i + m of the lane
  uint32_t plane_w[NW][PER_BYTE];
#pragma unroll
  for (int p = 0; p < EPL; ++p) {
    const int g = p / 16;
    const int k = p / (32 / BITS), i = (p % (32 / BITS)) / PER_BYTE, m = p % PER_BYTE;
    float c = __builtin_amdgcn_fmed3f((u[p] - z[g]) * inv[g], 0.0f, (float)L);
    if constexpr (DEQ) {
      c = __builtin_rintf(c);
      u[p] = __builtin_fmaf(c, sc[g], z[g]);
    }
    plane_w[k][m] = __builtin_amdgcn_cvt_pk_u8_f32(c, i, i == 0 ? 0u : plane_w[k][m]);
  }
  if (!valid) return;
  uint32_t w[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    w[k] = plane_w[k][0];
#pragma unroll
    for (int m = 1; m < PER_BYTE; ++m) w[k] = (plane_w[k][m] << (BITS * m)) | w[k];
  }
  if constexpr (BITS == 2) {
    const u32x2_t v = {w[0], w[1]};
    __builtin_amdgcn_raw_buffer_store_b64(v, cr, tok * (D / 4) + 8 * j, 0, 0);
  } else {
    const u32x4_t v = {w[0], w[1], w[2], w[3]};
    __builtin_amdgcn_raw_buffer_store_b128(v, cr, tok * (D / 2) + 16 * j, 0, 0);
  }
  const uint32_t G = D / group;
  if (group == 32) {
    __builtin_amdgcn_raw_buffer_store_b32(sz[0], mr, 4 * (tok * G + j), 0, 0);
  } else {
    const u32x2_t v = {sz[0], sz[1]};
    __builtin_amdgcn_raw_buffer_store_b64(v, mr, 4 * (tok * G + 2 * j), 0, 0);
  }
}

// quantize_pack for a bit width known at run time, onto the planes of one
// loop (codes / meta at the wave's first output slot row0, nw valid tokens).
template <int D, bool DEQ>
__device__ __forceinline__ void quantize_loop(float (&u)[EPL], int bits, int group, uint8_t *codes, uint32_t *meta,
                                              size_t row0, int nw, uint32_t tok, int j, bool valid) {
  const int G = D / group;
  const __amdgpu_buffer_rsrc_t mr = plane(meta + row0 * G, (uint32_t)nw * 4 * G);
  if (bits == 2)
    quantize_pack<D, 2, DEQ>(u, group, plane(codes + row0 * (D / 4), (uint32_t)nw * (D / 4)), mr, tok, j, valid);
  else
    quantize_pack<D, 4, DEQ>(u, group, plane(codes + row0 * (D / 2), (uint32_t)nw * (D / 2)), mr, tok, j, valid);
}

// One wave encodes VPW tokens of one (side, batch*head): the reference (the
// BF16 final loop, or a quantized anchor: quantized like a residual without
// the LS coefficient, then dequantized and rotated back as the residuals'
// reference), then each residual loop in turn.  With chains each loop's
// reconstruction becomes the next loop's reference.
//
// Everything that depends only on the wave is wave-uniform, so every plane
// is a buffer at the wave's first token addressed by 32-bit lane offsets.
// Each loop's input is loaded when the loop starts, with no prefetch of the
// next loop's rows: that buffer cost 16 VGPRs, and without it the kernel
// fits 128 (four waves per SIMD), whose other waves cover the load latency
// (anchored prefill 4% faster, [4,2,2] prefill unchanged).  CHAIN (chained
// references) is a template parameter: without it y is fixed over the
// loops, and the loop carries no copies of it around its back edge.
template <int D, bool CHAIN>
__global__ __launch_bounds__(256) void encode_kernel(const EncodeArgs a) {
  constexpr int LANES = D / EPL;
  constexpr int VPW = kWave / LANES;
  const int lane = threadIdx.x & 63;
  const int task = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (task >= 2 * a.tasks_per_side) return;          // whole wave
  const int side = task >= a.tasks_per_side ? 1 : 0;
  const int tk = task - side * a.tasks_per_side;
  const int bh = tk / a.chunks;
  const int chunk = tk - bh * a.chunks;
  const int j = lane % LANES;
  const int t_first = chunk * VPW;                   // the wave's first token in [0, n)
  const int nw = min(VPW, a.n - t_first);            // the wave's valid tokens
  const uint32_t tok = (uint32_t)(lane / LANES);     // relative to t_first
  const bool valid = (int)tok < nw;
  const uint32_t tokc = valid ? tok : (uint32_t)(nw - 1);   // in-bounds stand-in for loads
  const EncodeSide &S = a.side[side];
  const size_t row0 = (size_t)bh * a.cap + (size_t)(a.t0 + t_first);   // output slot of t_first
  const size_t xrow0 = (size_t)bh * a.n + (size_t)t_first;            // input row of t_first
  const uint32_t xoff = 2 * (tokc * D + EPL * j);
  const uint32_t rows = (uint32_t)nw * (2 * D);
  auto input = [&](int i) { return plane(S.xin[i] + xrow0 * D, rows); };

  float y[EPL];
  {
    u32x4_t yr[EPL / 8];
    load_raw32(a.abits == 0 ? plane(S.ref + row0 * D, rows) : input(a.n_res), xoff, yr);
    unpack_raw32(yr, y);
  }
  if (a.abits != 0) {
    rotate_canonical<LANES>(y, a.rotate, a.rot_c, lane);
    quantize_loop<D, true>(y, a.abits, a.agroup, S.codes[a.n_res], S.meta[a.n_res], row0, nw, tok, j, valid);
    if (a.rotate) rotate_rebuilt<LANES>(y, a.rot_c, lane);
  }
  float den = dot_sum32<LANES>(y, y);                // exact products for a BF16 y

  for (int l = 0; l < a.n_res; ++l) {
    float x[EPL];
    {
      u32x4_t raw[EPL / 8];
      load_raw32(input(l), xoff, raw);
      unpack_raw32(raw, x);
    }
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
    const bool link = CHAIN && l + 1 < a.n_res;       // the next loop refers to this one
    if (link)
      quantize_loop<D, true>(x, a.bits[l], a.group, S.codes[l], S.meta[l], row0, nw, tok, j, valid);
    else
      quantize_loop<D, false>(x, a.bits[l], a.group, S.codes[l], S.meta[l], row0, nw, tok, j, valid);
    if (valid && j == 0)
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)a16, plane(S.alpha[l] + row0, (uint32_t)nw * 2), 2 * tok, 0, 0);
    if constexpr (CHAIN) {
      if (link) {
        // chained references: y <- fma(alpha, y, r_hat), r_hat = c * H(fma(code, s, z))
        if (a.rotate) rotate_rebuilt<LANES>(x, a.rot_c, lane);
#pragma unroll
        for (int p = 0; p < EPL; ++p) y[p] = __builtin_fmaf(af, y[p], x[p]);
        den = dot_sum32<LANES>(y, y);
      }
    }
  }
}

hipError_t launch_encode(const EncodeArgs &a, int head_dim, hipStream_t s) {
  const int tasks = 2 * a.tasks_per_side;
  const dim3 grid((tasks + 3) / 4), block(256);
  switch (head_dim) {
    case 64:
      if (a.chain) hipLaunchKernelGGL((encode_kernel<64, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((encode_kernel<64, false>), grid, block, 0, s, a);
      break;
    case 128:
      if (a.chain) hipLaunchKernelGGL((encode_kernel<128, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((encode_kernel<128, false>), grid, block, 0, s, a);
      break;
    case 256:
      if (a.chain) hipLaunchKernelGGL((encode_kernel<256, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((encode_kernel<256, false>), grid, block, 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rq
