// Plain streaming reads of one device buffer: the measured HBM read ceiling
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

// Each wave streams its own contiguous share of the buffer in 8 KiB steps by
// direct-to-LDS loads (non-temporal) into two 8 KiB stages, the next step in
// flight while one word of the current is read back; the bytes past the waves'
// shares are read by a grid-stride loop.  (Whole runs per wave read faster than
// the grid-stride pattern above, which spreads each wave over the buffer.)
__global__ __launch_bounds__(256) void stream_read_lds_kernel(const u32x4_t* __restrict__ p,
                                                              size_t n16, unsigned* sink) {
  __shared__ __attribute__((aligned(16))) char st[4][2][8192];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t wave = (size_t)blockIdx.x * 4 + w;
  const size_t waves = (size_t)gridDim.x * 4;
  const size_t per = n16 / waves / 512 * 512;      // 16-byte units per wave, whole steps
  const char* q = reinterpret_cast<const char*>(p + wave * per);
  const size_t steps = per / 512;
  unsigned acc = 0;
  auto issue = [&](size_t step, int b) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      __builtin_amdgcn_global_load_lds(q + step * 8192 + u * 1024 + lane * 16,
                                       (__attribute__((address_space(3))) void*)&st[w][b][u * 1024],
                                       16, 0, kCpolNt);
  };
  if (steps > 0) issue(0, 0);
  for (size_t k = 0; k < steps; ++k) {
    if (k + 1 < steps) {
      issue(k + 1, (int)((k + 1) & 1));
      __builtin_amdgcn_s_waitcnt(0x0F78);            // vmcnt(8): step k has landed
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
    }
    const unsigned addr =
        (unsigned)(size_t)(__attribute__((address_space(3))) char*)&st[w][k & 1][lane * 16];
    unsigned x;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
    acc ^= x;
  }
  for (size_t i = waves * per + (size_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * 256) {
    const u32x4_t v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* sink, int workgroups,
                              int mode, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const u32x4_t* p = static_cast<const u32x4_t*>(buf);
  if (mode == 2)
    hipLaunchKernelGGL(stream_read_lds_kernel, dim3(workgroups), dim3(256), 0, st, p, n16, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(workgroups), dim3(256), 0, st, p, n16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(workgroups), dim3(256), 0, st, p, n16, sink);
  return hipGetLastError();
}

}  // namespace pa
