// Block centroids from the keys of a request ("Round 15 Track C Audit",
// section 2: the pooled keys are one of the indexer's stages checked for
// parity; "Iterate Centroids Score": the scorer reads one centroid per block of
// the paged cache). Reading: a block's pooled key is the mean of its tokens'
// keys.
//
//   c[b,n,:] = mean of k[b,s,:] over the tokens s of block n that the request
//              holds: s in [n*page, min((n+1)*page, seq_len[b])),
// for the blocks n < n_valid = min(N_pad, ceil(seq_len / page)); rows past
// n_valid are not written. Sums run in fp32 in token order; bf16 output is the
// round-to-nearest-even of the fp32 mean.
//
// A streaming reduction, HBM-bound: 16 lanes own one block row (8 dims each, 16
// bytes of bf16), load the block's tokens back to back (all loads in flight
// before the adds) and write one 16-byte row of the centroid.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.h"

namespace idxk {

constexpr int kPoolNT = 256;               // 16 block rows per workgroup step
constexpr int kPoolRowsPerWG = kPoolNT / 16;

__device__ __forceinline__ uint32_t pool_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool BF16, int PAGE>
__global__ __launch_bounds__(kPoolNT) void pool_keys_kernel(const void* __restrict__ k,
                                                            const int32_t* __restrict__ seq_len,
                                                            void* __restrict__ c, int S_pad,
                                                            int N_pad, int page_size,
                                                            int blocks_per_b) {
  const int b = blockIdx.x / blocks_per_b;
  const int n = (blockIdx.x - b * blocks_per_b) * kPoolRowsPerWG + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  const int64_t sl = min((int64_t)max(seq_len[b], 0), (int64_t)S_pad);
  const int nv = (int)min((int64_t)N_pad, (sl + page_size - 1) / page_size);
  if (n >= nv) return;
  const int s0 = n * page_size;
  const int cnt = (int)min((int64_t)page_size, sl - s0);  // >= 1 since n < nv
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // PAGE > 0: the page size is known here, every token load is issued before
  // the adds; PAGE == 0: any page size, one token at a time
  constexpr int UNROLL = PAGE > 0 ? PAGE : 1;
  for (int base = 0; base < cnt; base += UNROLL) {
    float x[UNROLL][8];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int s = s0 + min(base + u, cnt - 1);  // clamp: a duplicate read, discarded
      const size_t row = (size_t)b * S_pad + s;
      if constexpr (BF16) {
        const uint4 v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k) +
                                                       row * kHeadDim)[l16];
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[u][2 * e] = bf16_lo(wd[e]);
          x[u][2 * e + 1] = bf16_hi(wd[e]);
        }
      } else {
        const float4* p =
            reinterpret_cast<const float4*>(static_cast<const float*>(k) + row * kHeadDim) +
            2 * l16;
        const float4 a = p[0], bb = p[1];
        x[u][0] = a.x; x[u][1] = a.y; x[u][2] = a.z; x[u][3] = a.w;
        x[u][4] = bb.x; x[u][5] = bb.y; x[u][6] = bb.z; x[u][7] = bb.w;
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (base + u < cnt)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[u][e];
  }
  float m[8];  // correctly rounded fp32 division (exact for whole pages of 2^j tokens)
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = acc[e] / (float)cnt;
  const size_t orow = (size_t)b * N_pad + n;
  if constexpr (BF16) {
    uint4 o;
    o.x = pool_bf16_rne(m[0]) | (pool_bf16_rne(m[1]) << 16);
    o.y = pool_bf16_rne(m[2]) | (pool_bf16_rne(m[3]) << 16);
    o.z = pool_bf16_rne(m[4]) | (pool_bf16_rne(m[5]) << 16);
    o.w = pool_bf16_rne(m[6]) | (pool_bf16_rne(m[7]) << 16);
    reinterpret_cast<uint4*>(static_cast<uint16_t*>(c) + orow * kHeadDim)[l16] = o;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(c) + orow * kHeadDim) + 2 * l16;
    p[0] = make_float4(m[0], m[1], m[2], m[3]);
    p[1] = make_float4(m[4], m[5], m[6], m[7]);
  }
}

int launch_pool_keys(const void* k, const int32_t* seq_len, void* c, int B, int S_pad, int N_pad,
                     int page_size, bool bf16, void* stream) {
  const int blocks_per_b = (N_pad + kPoolRowsPerWG - 1) / kPoolRowsPerWG;
  const int64_t grid = (int64_t)B * blocks_per_b;
  if (grid > 0x7FFFFFFF) return (int)hipErrorInvalidConfiguration;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)grid), blk(kPoolNT);
#define IDX_POOL(BF, PG)                                                                   \
  hipLaunchKernelGGL((pool_keys_kernel<BF, PG>), g, blk, 0, s, k, seq_len, c, S_pad, N_pad, \
                     page_size, blocks_per_b)
  if (page_size == 16) {
    if (bf16) IDX_POOL(true, 16); else IDX_POOL(false, 16);
  } else {
    if (bf16) IDX_POOL(true, 0); else IDX_POOL(false, 0);
  }
#undef IDX_POOL
  return (int)hipGetLastError();
}

}  // namespace idxk
