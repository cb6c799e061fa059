// Reference kernels for measuring the decode product against what the hardware gives at the same
// size: a plain read of a weight's bytes in the decode kernel's launch shape, and an empty launch.
// They compute nothing of the method; the benchmark times them beside the product.  Built into a
// library of their own (libnvfp4_ceiling.so), outside the product's C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 8;  // 16-byte loads per lane in flight at once

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The two regions are read as one range (a's bytes, then b's): workgroup w reads the w-th
// contiguous share of it, 16 bytes per lane per load, with every load of a batch issued before
// any is used; the bytes are folded by XOR so the loads stay live, and each wavefront writes one
// word.  (Reading each region's share separately issues twice the load instructions and took
// 4.5 us against 4.1 us for one 14.75 MB weight.)
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ a, int64_t na,
                                                               const u32x4* __restrict__ b, int64_t nb,
                                                               uint32_t* __restrict__ out) {
  const int64_t n = na + nb, g = gridDim.x;
  const int64_t lo = n * blockIdx.x / g, hi = n * (blockIdx.x + 1) / g;
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + u * kThreads;
      v[u] = j < hi ? __builtin_nontemporal_load(j < na ? a + j : b + (j - na)) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = acc;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// Read `na` bytes at `a` and `nb` bytes at `b` (both 16-byte aligned, sizes multiples of 16) with
// `blocks` workgroups of 512 lanes; `out` receives blocks * 8 words.  Returns a hipError_t code.
int nvfp4_ceiling_stream_read(const void* a, int64_t na, const void* b, int64_t nb, uint32_t* out,
                              int blocks, void* stream) {
  if (blocks <= 0 || na < 0 || nb < 0 || (na % 16) || (nb % 16) || !out ||
      (reinterpret_cast<uintptr_t>(a) % 16) || (reinterpret_cast<uintptr_t>(b) % 16) ||
      (na && !a) || (nb && !b))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const u32x4*>(a), na / 16, reinterpret_cast<const u32x4*>(b),
                     nb / 16, out);
  return (int)hipGetLastError();
}

// One launch of a kernel that does nothing (one wavefront).
int nvfp4_ceiling_empty_launch(void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

}  // extern "C"
