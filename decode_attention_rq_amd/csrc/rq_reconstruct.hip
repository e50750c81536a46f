// rq_reconstruct.hip -- explicit dequantization of one residual loop (gfx950).
//
// ResidualQuant page, Abstract: a residual loop is rebuilt from the reference
// and its codes, x_hat = alpha*y + H_n (z + s*code).  Same lane mapping as the
// encoder (8 consecutive dims per lane, D/8 lanes per vector); FP32.

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {

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
  const int G = D / a.group;
  const int k = j / (a.group / 8);

  uint32_t word = (a.bits == 2)
      ? (uint32_t)reinterpret_cast<const uint16_t *>(a.codes + slot * (D / 4))[j]
      : reinterpret_cast<const uint32_t *>(a.codes + slot * (D / 2))[j];
  const uint32_t mz = a.meta[slot * G + k];
  const float s = f16_to_f32(mz & 0xffffu), z = f16_to_f32(mz >> 16);
  const uint32_t mask = (1u << a.bits) - 1u;
  float u[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) u[p] = __builtin_fmaf(s, (float)((word >> (a.bits * p)) & mask), z);
  if (a.rotate) {
    wht8<D>(u, lane);
#pragma unroll
    for (int p = 0; p < 8; ++p) u[p] *= a.rot_c;
  }
  const float af = f16_to_f32(a.alpha[slot]);
  const uint4 yw = *reinterpret_cast<const uint4 *>(a.ref + slot * D + 8 * j);
  const float y[8] = {bf16lo(yw.x), bf16hi(yw.x), bf16lo(yw.y), bf16hi(yw.y),
                      bf16lo(yw.z), bf16hi(yw.z), bf16lo(yw.w), bf16hi(yw.w)};
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
