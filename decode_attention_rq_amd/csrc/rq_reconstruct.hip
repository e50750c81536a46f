// rq_reconstruct.hip -- explicit dequantization of one loop (gfx950).
//
// ResidualQuant page, Abstract: a residual loop is rebuilt from the reference
// and its codes, x_hat = alpha*y + H_n (z + s*code).  With a quantized anchor
// y is the anchor's own dequantized value H_n (z_a + s_a*code_a), which is
// also what the anchor loop itself reconstructs to.  Same lane mapping as the
// encoder (8 consecutive dims per lane, D/8 lanes per vector); FP32.

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {

// The lane's 8 values of a quantized vector: z + s*code per element (FP32),
// then H_n / sqrt(D) when rotated.  The rotation's cross-lane stages run in
// every lane of the wave, so callers keep all lanes active here.
template <int D>
__device__ __forceinline__ void dequant8(const uint8_t *codes, const uint32_t *meta, size_t slot, int j,
                                         int bits, int group, int rotate, float rot_c, int lane,
                                         float (&u)[8]) {
  const uint32_t word = (bits == 2)
      ? (uint32_t)reinterpret_cast<const uint16_t *>(codes + slot * (D / 4))[j]
      : reinterpret_cast<const uint32_t *>(codes + slot * (D / 2))[j];
  const uint32_t mz = meta[slot * (D / group) + j / (group / 8)];
  const float s = f16_to_f32(mz & 0xffffu), z = f16_to_f32(mz >> 16);
  const uint32_t mask = (1u << bits) - 1u;
#pragma unroll
  for (int p = 0; p < 8; ++p) u[p] = __builtin_fmaf(s, (float)((word >> (bits * p)) & mask), z);
  if (rotate) {
    wht8<D>(u, lane);
#pragma unroll
    for (int p = 0; p < 8; ++p) u[p] *= rot_c;
  }
}

template <int D>
__global__ __launch_bounds__(256) void reconstruct_kernel(const ReconArgs a) {
  constexpr int LANES = D / 8;
  constexpr int VPW = kWave / LANES;
  const int lane = threadIdx.x & 63;
  const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= a.bh * a.chunks) return;               // whole wave
  const int bh = task / a.chunks;
  const int chunk = task - bh * a.chunks;
  const int j = lane % LANES;
  const int tl = chunk * VPW + lane / LANES;
  const bool valid = tl < a.n;
  const int tlc = valid ? tl : a.n - 1;
  const size_t slot = (size_t)bh * a.cap + (size_t)(a.t0 + tlc);

  float y[8];
  if (a.abits == 0) {
    const uint4 yw = *reinterpret_cast<const uint4 *>(a.ref + slot * D + 8 * j);
    y[0] = bf16lo(yw.x); y[1] = bf16hi(yw.x); y[2] = bf16lo(yw.y); y[3] = bf16hi(yw.y);
    y[4] = bf16lo(yw.z); y[5] = bf16hi(yw.z); y[6] = bf16lo(yw.w); y[7] = bf16hi(yw.w);
  } else {
    dequant8<D>(a.acodes, a.ameta, slot, j, a.abits, a.agroup, a.rotate, a.rot_c, lane, y);
  }
  for (int k = 0; k < a.npre; ++k) {   // chained references: the links from the root
    float u[8];
    dequant8<D>(a.pcodes[k], a.pmeta[k], slot, j, a.pbits[k], a.group, a.rotate, a.rot_c, lane, u);
    const float ak = f16_to_f32(a.palpha[k][slot]);
#pragma unroll
    for (int p = 0; p < 8; ++p) y[p] = __builtin_fmaf(ak, y[p], u[p]);
  }
  if (a.codes == nullptr) {            // the anchor loop itself
    if (valid) {
      float4 *o = reinterpret_cast<float4 *>(a.out + ((size_t)bh * a.n + tl) * D + 8 * j);
      o[0] = make_float4(y[0], y[1], y[2], y[3]);
      o[1] = make_float4(y[4], y[5], y[6], y[7]);
    }
    return;
  }
  float u[8];
  dequant8<D>(a.codes, a.meta, slot, j, a.bits, a.group, a.rotate, a.rot_c, lane, u);
  const float af = f16_to_f32(a.alpha[slot]);
  if (valid) {
    float4 *o = reinterpret_cast<float4 *>(a.out + ((size_t)bh * a.n + tl) * D + 8 * j);
    o[0] = make_float4(__builtin_fmaf(af, y[0], u[0]), __builtin_fmaf(af, y[1], u[1]),
                       __builtin_fmaf(af, y[2], u[2]), __builtin_fmaf(af, y[3], u[3]));
    o[1] = make_float4(__builtin_fmaf(af, y[4], u[4]), __builtin_fmaf(af, y[5], u[5]),
                       __builtin_fmaf(af, y[6], u[6]), __builtin_fmaf(af, y[7], u[7]));
  }
}

hipError_t launch_reconstruct(const ReconArgs &a, int head_dim, hipStream_t s) {
  const int tasks = a.bh * a.chunks;
  const dim3 grid((tasks + 3) / 4), block(256);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(reconstruct_kernel<64>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(reconstruct_kernel<128>, grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL(reconstruct_kernel<256>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rq
