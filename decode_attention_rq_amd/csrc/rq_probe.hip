// rq_probe.hip -- a plain 128-bit HBM read stream (gfx950): the attainable
// read bandwidth that the decode kernel's achieved rate is compared with.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rq.h"
#include "rq_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4_t load16(const u32x4_t *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

__device__ __forceinline__ uint32_t fold(u32x4_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Grid-stride pattern: every lane reads elements i, i + stride, ... of the
// buffer (stride = all lanes of the grid), four independent loads per
// iteration, and writes the XOR of everything it read.
template <bool NT>
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4_t *p, uint64_t n16, uint32_t *sink) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = load16<NT>(p + i), b = load16<NT>(p + i + stride);
    const u32x4_t c = load16<NT>(p + i + 2 * stride), d = load16<NT>(p + i + 3 * stride);
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n16; i += stride) acc ^= fold(load16<NT>(p + i));
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Chunked pattern: workgroup b reads the b-th of gridDim.x contiguous
// chunks of the buffer, 16 KiB per iteration (four consecutive 4 KiB
// segments, one 128-bit load per lane each), the way a decode workgroup
// walks one (batch, head)'s token rows.
template <bool NT>
__global__ __launch_bounds__(256) void read_chunk_kernel(const u32x4_t *p, uint64_t n16, uint32_t *sink) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t begin = (uint64_t)blockIdx.x * per;
  const uint64_t end = begin + per < n16 ? begin + per : n16;
  uint64_t i = begin + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * 256 < end; i += 4 * 256) {
    const u32x4_t a = load16<NT>(p + i), b = load16<NT>(p + i + 256);
    const u32x4_t c = load16<NT>(p + i + 512), d = load16<NT>(p + i + 768);
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < end; i += 256) acc ^= fold(load16<NT>(p + i));
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Planes pattern: the buffer is cut into kProbePlanes equal planes and
// workgroup b walks the b-th chunk of every plane at once, as a decode
// workgroup walks one (batch, head)'s rows of every plane it reads (an
// int2-8k step: the reference K and V, and each residual loop's codes,
// scale/zero words and alphas, K and V: 20).  Four 128-bit loads per lane
// per iteration, taking the planes in turn.
constexpr int kProbePlanes = 20;
template <bool NT>
__global__ __launch_bounds__(256) void read_planes_kernel(const u32x4_t *p, uint64_t n16, uint32_t *sink) {
  const uint64_t plane = n16 / kProbePlanes;
  const uint64_t per = (plane / gridDim.x) & ~(uint64_t)255;   // whole 4 KiB segments per plane
  const uint64_t b0 = (uint64_t)blockIdx.x * per;
  const uint64_t nseg = per / 256 * kProbePlanes;               // segment s: plane s % P, row s / P
  uint32_t acc = 0;
  uint64_t s = 0;
  for (; s + 3 < nseg; s += 4) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t ss = s + u;
      v[u] = load16<NT>(p + (ss % kProbePlanes) * plane + b0 + (ss / kProbePlanes) * 256 + threadIdx.x);
    }
    acc ^= fold(v[0]) ^ fold(v[1]) ^ fold(v[2]) ^ fold(v[3]);
  }
  for (; s < nseg; ++s)
    acc ^= fold(load16<NT>(p + (s % kProbePlanes) * plane + b0 + (s / kProbePlanes) * 256 + threadIdx.x));
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" rq_status rq_probe_read_stream(const void *buf, size_t bytes, int32_t nontemporal, int32_t pattern,
                                          int32_t n_blocks, uint32_t *sink, void *hip_stream) {
  if (!aligned16(buf) || !aligned16(sink) || bytes < 16 || bytes % 16 != 0) return RQ_ERR_INVALID_ARG;
  if (n_blocks < 1 || n_blocks > 65535 || (nontemporal != 0 && nontemporal != 1)) return RQ_ERR_INVALID_ARG;
  if (pattern < 0 || pattern > 2) return RQ_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const u32x4_t *p = static_cast<const u32x4_t *>(buf);
  const uint64_t n16 = bytes / 16;
  const dim3 grid(n_blocks), block(256);
  if (pattern == 0) {
    if (nontemporal) hipLaunchKernelGGL(read_stream_kernel<true>, grid, block, 0, st, p, n16, sink);
    else hipLaunchKernelGGL(read_stream_kernel<false>, grid, block, 0, st, p, n16, sink);
  } else if (pattern == 1) {
    if (nontemporal) hipLaunchKernelGGL(read_chunk_kernel<true>, grid, block, 0, st, p, n16, sink);
    else hipLaunchKernelGGL(read_chunk_kernel<false>, grid, block, 0, st, p, n16, sink);
  } else {
    if (nontemporal) hipLaunchKernelGGL(read_planes_kernel<true>, grid, block, 0, st, p, n16, sink);
    else hipLaunchKernelGGL(read_planes_kernel<false>, grid, block, 0, st, p, n16, sink);
  }
  return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_DEVICE;
}
