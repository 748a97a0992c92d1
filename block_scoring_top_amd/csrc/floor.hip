// Floor launches for the benchmark: an empty kernel, a plain streaming read of
// a byte range, optionally followed by the arrival counter of the fused select
// (relaxed agent-scope ticket after the workgroup's loads complete; the last
// arriver returns it to zero), and back-to-back bf16 matrix products on
// register operands. Nothing of the method is computed here.
#include <hip/hip_runtime.h>

#include "idx.h"
#include "idx_floor.h"

namespace idxk {

__global__ __launch_bounds__(64) void floor_empty_kernel() {}

template <int NT>
__global__ __launch_bounds__(NT) void floor_read_kernel(const uint4* __restrict__ src,
                                                        size_t n16, float* __restrict__ sink,
                                                        uint32_t* __restrict__ ticket) {
  // workgroup g reads 16-byte words [g * per, min((g + 1) * per, n16))
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  // four loads in flight per thread
  for (; i + 3 * NT < hi; i += 4 * NT) {
    const uint4 a = src[i], b = src[i + NT], c = src[i + 2 * NT], d = src[i + 3 * NT];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < hi; i += NT) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0;
  __syncthreads();
  atomicXor(&red, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = __uint_as_float(red);
  if (ticket == nullptr) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

typedef __bf16 fbf16x8 __attribute__((ext_vector_type(8)));
typedef float ff32x16 __attribute__((ext_vector_type(16)));

// Four independent accumulator chains per wave, so that no product waits on
// the one before it; the operands cycle through eight A and eight B fragments.
__global__ __launch_bounds__(256, 2) void floor_mfma_kernel(const uint4* __restrict__ frags,
                                                            int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  fbf16x8 a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = __builtin_bit_cast(fbf16x8, frags[k * 64 + lane]);
    b[k] = __builtin_bit_cast(fbf16x8, frags[(8 + k) * 64 + lane]);
  }
  ff32x16 acc[4];
  for (int c = 0; c < 4; ++c)
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b[(r + c) & 7], acc[c], 0, 0, 0);
  }
  float s = 0.f;
  for (int c = 0; c < 4; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace idxk

extern "C" int idx_floor_mfma(const void* frags, int blocks, int iters, float* sink,
                              void* stream) {
  if (frags == nullptr || sink == nullptr || blocks < 1 || blocks > 65536 || iters < 8 ||
      iters > 16384 || iters % 8 != 0 || reinterpret_cast<uintptr_t>(frags) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return IDX_ERR_INVALID_ARG;
  hipLaunchKernelGGL(idxk::floor_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(frags), iters,
                     sink);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_ERR_HIP;
}

extern "C" int idx_floor_empty(int blocks, void* stream) {
  if (blocks < 1 || blocks > 65536) return IDX_ERR_INVALID_ARG;
  hipLaunchKernelGGL(idxk::floor_empty_kernel, dim3((unsigned)blocks), dim3(64), 0,
                     static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_ERR_HIP;
}

extern "C" int idx_floor_read(const void* src, size_t bytes, float* sink, uint32_t* ticket,
                              int blocks, int threads, void* stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 || blocks < 1 ||
      blocks > 65536 || (threads != 256 && threads != 1024) ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(ticket) % 4 != 0)
    return IDX_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* p = static_cast<const uint4*>(src);
  if (threads == 256)
    hipLaunchKernelGGL(idxk::floor_read_kernel<256>, dim3((unsigned)blocks), dim3(256), 0, s, p,
                       bytes / 16, sink, ticket);
  else
    hipLaunchKernelGGL(idxk::floor_read_kernel<1024>, dim3((unsigned)blocks), dim3(1024), 0, s,
                       p, bytes / 16, sink, ticket);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_ERR_HIP;
}
