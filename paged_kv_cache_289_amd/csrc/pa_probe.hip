// A plain streaming read of one device buffer: the measured HBM read ceiling
// that the paged kernels' bandwidth figures are set against (the published
// 8 TB/s peak stays the roofline).
#include "pa_common.h"

namespace pa {

// Every thread reads 16-byte vectors kUnroll at a time (independent loads in
// flight), striding over the buffer by the whole grid; the xor of everything
// read is stored only if it equals a value no input produces by chance, which
// keeps every load live without writing per thread.
template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p,
                                                          size_t n16, unsigned* sink) {
  constexpr int kUnroll = 8;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* sink, int workgroups,
                              int nontemporal, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(workgroups), dim3(256), 0, st,
                       static_cast<const u32x4_t*>(buf), n16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(workgroups), dim3(256), 0, st,
                       static_cast<const u32x4_t*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace pa
