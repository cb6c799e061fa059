// Reference kernels for measuring the decode product against what the hardware gives at the same
// size: a plain read of a weight's bytes in the decode kernel's launch shape, and an empty launch.
// They compute nothing of the method; the benchmark times them beside the product.  Built into a
// library of their own (libnvfp4_ceiling.so), outside the product's C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 8;  // 16-byte loads per lane and region in flight at once

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup w reads the w-th contiguous share of each region, 16 bytes per lane per load, with every
// load of a batch issued before any is used; the bytes are folded by XOR so the loads stay live, and
// each wavefront writes one word.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ a, int64_t na,
                                                               const u32x4* __restrict__ b, int64_t nb,
                                                               uint32_t* __restrict__ out) {
  const int64_t g = gridDim.x;
  const int64_t sa = (na + g - 1) / g, sb = (nb + g - 1) / g;
  const int64_t a0 = blockIdx.x * sa, a1 = min(na, a0 + sa);
  const int64_t b0 = blockIdx.x * sb, b1 = min(nb, b0 + sb);
  uint32_t acc = 0;
  for (int64_t i = threadIdx.x; a0 + i < a1 || b0 + i < b1; i += kUnroll * kThreads) {
    u32x4 va[kUnroll], vb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t ia = a0 + i + u * kThreads, ib = b0 + i + u * kThreads;
      va[u] = ia < a1 ? __builtin_nontemporal_load(a + ia) : u32x4{0, 0, 0, 0};
      vb[u] = ib < b1 ? __builtin_nontemporal_load(b + ib) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      acc ^= va[u].x ^ va[u].y ^ va[u].z ^ va[u].w ^ vb[u].x ^ vb[u].y ^ vb[u].z ^ vb[u].w;
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
