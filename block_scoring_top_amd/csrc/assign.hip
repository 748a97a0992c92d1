// Nearest-centroid k-means assignment on the matrix cores ("Export Cake KMeans
// plan-runtime suite", Summary: assignment of bf16 points to centroids with the
// centroid norms computed inside the call).
//
//   assign[i] = argmax_j ( x_i . c_j - |c_j|^2 / 2 ),  ties to the lower j,
//
// which has the same maximiser as 2 x.c - |c|^2. The contraction X . C^T is a
// dense bf16 GEMM with fp32 accumulation, so it runs on v_mfma_f32_32x32x16_bf16;
// the bias -|c|^2/2 is loaded into the accumulators before the products are
// added, and the argmax is a running max in registers, so the score matrix is
// never written anywhere.
//
// Layout: the MFMA's A operand is a 32-centroid x 16-dim slice of C (from LDS),
// the B operand a 16-dim x 32-point slice of X^T (registers, loaded once). The
// 32x32 result tile then has one point per lane column (lane % 32) and 16
// centroid rows per lane, so the max over centroids is mostly in-lane; lanes l
// and l^32 hold disjoint centroid rows of the same point and are merged once.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.h"

namespace idxk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAsgNT = 256;          // 4 waves
constexpr int kAsgPtsPerWave = 64;   // two 32-point column blocks
constexpr int kAsgPts = kAsgPtsPerWave * (kAsgNT / kWave);
constexpr int kAsgTileC = 64;        // centroids per LDS tile: two 32-row blocks
constexpr int kChunks = kHeadDim * 2 / 16;  // 16-byte chunks per bf16 row (16)

// -|c_j|^2 / 2 in fp32 (squares of bf16 values are exact in fp32)
__global__ __launch_bounds__(256) void cnorm_kernel(const uint16_t* __restrict__ c, int C,
                                                    float* __restrict__ cn) {
  const int lane = threadIdx.x & (kWave - 1);
  const int l16 = lane & 15;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= C) return;
  const uint4 v = reinterpret_cast<const uint4*>(c + (size_t)row * kHeadDim)[l16];
  float s = 0.f;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = bf16_lo(w[k]), b = bf16_hi(w[k]);
    s = fmaf(a, a, s);
    s = fmaf(b, b, s);
  }
  s = sum16(s);
  if (l16 == 0) cn[row] = -0.5f * s;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// row r of a centroid tile: its 16-byte chunk k sits at chunk position k ^ (r & 15)
__device__ __forceinline__ int swz(int r, int k) { return r * kChunks + (k ^ (r & 15)); }

__global__ __launch_bounds__(kAsgNT) void assign_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ c,
                                                        const float* __restrict__ cn,
                                                        int32_t* __restrict__ assign,
                                                        float* __restrict__ best_out, int64_t N,
                                                        int C) {
  __shared__ uint4 ctile[kAsgTileC * kChunks];  // 16 KiB
  __shared__ float ctn[kAsgTileC];
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int lane = t & (kWave - 1);
  const int col = lane & 31;  // point within a 32-point block; centroid row for A
  const int half = lane >> 5; // which 8 dims of a 16-dim k-step this lane carries
  const int64_t p0 = (int64_t)blockIdx.x * kAsgPts + w * kAsgPtsPerWave;

  // B operand: this lane's point rows, all 128 dims, as 8 k-steps of 8 bf16
  uint4 xb[2][8];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    int64_t p = p0 + cb * 32 + col;
    p = p < N ? p : N - 1;  // clamp: a valid duplicate row, never stored
    const uint4* xr = reinterpret_cast<const uint4*>(x + p * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) xb[cb][ks] = xr[2 * ks + half];
  }

  float best[2] = {-__builtin_inff(), -__builtin_inff()};
  int bidx[2] = {0, 0};

  for (int j0 = 0; j0 < C; j0 += kAsgTileC) {
    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int i = 0; i < kAsgTileC * kChunks / kAsgNT; ++i) {
      const int g = t + i * kAsgNT;
      const int r = g / kChunks, k = g % kChunks;
      const int j = j0 + r < C ? j0 + r : C - 1;  // clamp; rows past C are never winners
      ctile[swz(r, k)] = reinterpret_cast<const uint4*>(c + (size_t)j * kHeadDim)[k];
    }
    if (t < kAsgTileC) ctn[t] = (j0 + t < C) ? cn[j0 + t] : -__builtin_inff();
    __syncthreads();

    f32x16 acc[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float bias = ctn[rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3)];
        acc[rb][0][r] = bias;
        acc[rb][1][r] = bias;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8 a = as_bf16x8(ctile[swz(rb * 32 + col, 2 * ks + half)]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(xb[cb][ks]),
                                                               acc[rb][cb], 0, 0, 0);
      }
    }
    // running argmax; centroid index increases with (rb, r) for a fixed lane, so
    // a strict comparison keeps the lowest index among equal values
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = acc[rb][cb][r];
          const int j = j0 + rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (v > best[cb]) {
            best[cb] = v;
            bidx[cb] = j;
          }
        }
      }
    }
  }

  // merge the two lanes that share a point (l and l^32)
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float ov = __shfl_xor(best[cb], 32, kWave);
    const int oi = __shfl_xor(bidx[cb], 32, kWave);
    if (ov > best[cb] || (ov == best[cb] && oi < bidx[cb])) {
      best[cb] = ov;
      bidx[cb] = oi;
    }
    const int64_t p = p0 + cb * 32 + col;
    if (half == 0 && p < N) {
      assign[p] = bidx[cb];
      if (best_out != nullptr) best_out[p] = best[cb];
    }
  }
}

int launch_assign(const void* x, const void* c, int32_t* assign, float* best, int64_t N, int C,
                  float* cnorm, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(cnorm_kernel, dim3((unsigned)((C + 15) / 16)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(c), C, cnorm);
  int e = (int)hipGetLastError();
  if (e != 0) return e;
  const int64_t nblk = (N + kAsgPts - 1) / kAsgPts;
  hipLaunchKernelGGL(assign_kernel, dim3((unsigned)nblk), dim3(kAsgNT), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(c), cnorm,
                     assign, best, N, C);
  return (int)hipGetLastError();
}

}  // namespace idxk
