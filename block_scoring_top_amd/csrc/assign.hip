// Nearest-centroid k-means assignment on the matrix cores ("Export Cake KMeans
// plan-runtime suite", Summary: assignment of bf16 points to centroids with the
// centroid norms computed inside the call).
//
//   assign[i] = argmax_j ( x_i . c_j - |c_j|^2 / 2 ),  ties to the lower j,
//
// which has the same maximiser as 2 x.c - |c|^2. The contraction X . C^T is a
// dense bf16 GEMM with fp32 accumulation, so it runs on v_mfma_f32_32x32x16_bf16.
// The bias -|c|^2/2 (computed once per call by a small kernel into the
// workspace) is loaded into the accumulators before the products are added, and
// the argmax is a running max in registers: the score matrix is never written.
//
// Layout: the MFMA's A operand is a 32-centroid x 16-dim slice of C (from a
// double-buffered LDS tile of 64 centroids, filled by direct-to-LDS loads that
// overlap the previous tile's products), the B operand a 16-dim x 32-point
// slice of X^T (registers, loaded once). The 32x32 result tile then has one
// point per lane column (lane % 32) and 16 centroid rows per lane, so the max
// over centroids is mostly in-lane; lanes l and l^32 hold disjoint centroid rows
// of the same point and are merged once at the end.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.h"

namespace idxk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAsgNT = 256;          // 4 waves
constexpr int kAsgPtsPerWave = 64;   // two 32-point column blocks
constexpr int kCB = kAsgPtsPerWave / 32;  // 32-point column blocks per wave
constexpr int kAsgPts = kAsgPtsPerWave * (kAsgNT / kWave);
constexpr int kAsgTileC = 64;        // centroids per LDS tile: two 32-row blocks
constexpr int kChunks = kHeadDim * 2 / 16;                // 16-byte chunks per bf16 row (16)
constexpr int kTileLoads = kAsgTileC * kChunks / kAsgNT;  // 16-byte loads per thread per tile
static_assert(kTileLoads * kAsgNT == kAsgTileC * kChunks, "whole loads per thread");

// -|c_j|^2 / 2 in fp32, once per call (squares of bf16 values are exact in fp32),
// padded with -inf up to a whole number of centroid tiles
__global__ __launch_bounds__(256) void cnorm_kernel(const uint16_t* __restrict__ c, int C,
                                                    float* __restrict__ cn) {
  const int l16 = threadIdx.x & 15;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int rows = (C + kAsgTileC - 1) / kAsgTileC * kAsgTileC;
  if (row >= rows) return;  // whole 16-lane groups leave together
  const uint4 v = reinterpret_cast<const uint4*>(c + (size_t)(row < C ? row : C - 1) * kHeadDim)[l16];
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = bf16_lo(wd[k]), b = bf16_hi(wd[k]);
    s = fmaf(a, a, s);
    s = fmaf(b, b, s);
  }
  s = sum16(s);
  if (l16 == 0) cn[row] = row < C ? -0.5f * s : -__builtin_inff();
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// row r of a centroid tile: its 16-byte chunk k sits at chunk position k ^ (r & 15),
// so the 32 lanes reading one chunk column of 32 rows hit distinct banks
__device__ __forceinline__ int swz(int r, int k) { return r * kChunks + (k ^ (r & 15)); }

// Global -> LDS without a trip through registers (16-byte direct-to-LDS loads).
// Load i of wave w fills the 64 consecutive 16-byte LDS slots p = 64 (4w + i) +
// lane; slot p holds chunk (p & 15) ^ (row & 15) of tile row p >> 4, which is
// the swizzled layout the MFMA operand reads expect. Rows past C repeat row C-1
// (their bias is -inf, so they never win). Each wave also brings 16 of the
// tile's biases from the -inf-padded norm buffer, so every wave issues the same
// kLoadsPerTile loads per tile.
constexpr int kBiasPerWave = kAsgTileC / (kAsgNT / kWave);
constexpr int kLoadsPerTile = kTileLoads + 1;
__device__ __forceinline__ void load_ctile_lds(const uint16_t* __restrict__ c,
                                               const float* __restrict__ cn, int C, int j0,
                                               uint4* tile, float* tn) {
  const int t = threadIdx.x;
  const int w = t >> 6, lane = t & (kWave - 1);
#pragma unroll
  for (int i = 0; i < kTileLoads; ++i) {
    const int slot0 = (w * kTileLoads + i) * kWave;  // wave-uniform LDS base
    const int p = slot0 + lane;
    const int row = p >> 4;
    const int k = (p & 15) ^ (row & 15);
    const int j = j0 + row < C ? j0 + row : C - 1;
    __builtin_amdgcn_global_load_lds(c + (size_t)j * kHeadDim + k * 8, tile + slot0, 16, 0, 0);
  }
  if (lane < kBiasPerWave)
    __builtin_amdgcn_global_load_lds(cn + j0 + w * kBiasPerWave + lane, tn + w * kBiasPerWave, 4,
                                     0, 0);
}

// s_waitcnt with only the vector-memory count (expcnt and lgkmcnt left at
// their maxima, i.e. not waited for)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The workgroup barrier of the tile pipeline. The builtin alone is not a memory
// operation to the compiler, which could then move LDS reads or the direct-to-
// LDS refills across it; the empty asm statements with a memory clobber keep
// them on their side without the vmcnt(0) that a workgroup fence would add.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct ArgmaxState {
  float best[kCB];
  int bidx[kCB];
};

// One centroid tile: A fragments and biases from LDS tile `cur`, then (once
// they are in registers) the direct-to-LDS load of tile `tile + 2` into `nxt`,
// the products, the running argmax, and the wait for tile `tile + 1`.
__device__ __forceinline__ void assign_tile(const uint16_t* __restrict__ c,
                                            const float* __restrict__ cn, int C, int tile,
                                            int ntiles, const uint4* cur, const float4* curn,
                                            uint4* nxt, float* nxtn, const uint4 (&xb)[kCB][8],
                                            ArgmaxState& st) {
  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int j0 = tile * kAsgTileC;
  bf16x8 a[8][2];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    a[ks][0] = as_bf16x8(cur[swz(col, 2 * ks + half)]);
    a[ks][1] = as_bf16x8(cur[swz(32 + col, 2 * ks + half)]);
  }
  float4 bias[2][4];  // rows 8g + 4*half + 0..3 of 32-row block rb
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int g = 0; g < 4; ++g) bias[rb][g] = curn[rb * 8 + 2 * g + half];
  const bool refill = tile + 2 < ntiles;
  if (refill) load_ctile_lds(c, cn, C, j0 + 2 * kAsgTileC, nxt, nxtn);

  // independent accumulator chains: 2 centroid blocks x kCB point blocks
  f32x16 acc[2][kCB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[rb][cb][4 * g + 0] = bias[rb][g].x;
        acc[rb][cb][4 * g + 1] = bias[rb][g].y;
        acc[rb][cb][4 * g + 2] = bias[rb][g].z;
        acc[rb][cb][4 * g + 3] = bias[rb][g].w;
      }
    }
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const bf16x8 b = as_bf16x8(xb[cb][ks]);
      acc[0][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][0], b, acc[0][cb], 0, 0, 0);
      acc[1][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][1], b, acc[1][cb], 0, 0, 0);
    }
  }
  // Running argmax. The 16 values of a lane are reduced with 3-input maxes;
  // only when some lane of the wave finds a strictly larger value is the index
  // of its first (lowest-index) occurrence searched. For a fixed lane the
  // centroid index increases with (tile, rb, r), so strict comparisons keep
  // the lowest index among equal values.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const f32x16& v = acc[rb][cb];
      float m = v[0];
#pragma unroll
      for (int r = 1; r < 15; r += 2)  // a chain of 3-input maxes
        m = __builtin_fmaxf(__builtin_fmaxf(m, v[r]), v[r + 1]);
      m = __builtin_fmaxf(m, v[15]);
      const bool better = m > st.best[cb];
      if (__builtin_amdgcn_ballot_w64(better) != 0) {
        int rr = 15;
#pragma unroll
        for (int r = 14; r >= 0; --r) rr = (v[r] == m) ? r : rr;
        if (better) {
          st.best[cb] = m;
          st.bidx[cb] = j0 + rb * 32 + 8 * (rr >> 2) + 4 * half + (rr & 3);
        }
      }
    }
  }
  // Tile `tile + 1` has landed once at most the loads just issued for tile
  // `tile + 2` are outstanding in this wave, and in every wave after the
  // barrier; the barrier also frees `cur` for the refill issued next step.
  // (A plain barrier: the fence of __syncthreads would wait for every load.)
  if (refill) wait_vmcnt<kLoadsPerTile>();
  else wait_vmcnt<0>();
  tile_barrier();
}

__global__ __launch_bounds__(kAsgNT, 2) void assign_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ c,
                                                           const float* __restrict__ cn,
                                                           int32_t* __restrict__ assign,
                                                           float* __restrict__ best_out,
                                                           int64_t N, int C) {
  // three LDS tiles of 64 centroids (16 KiB each) and their biases, as
  // separate objects: tile t+2 streams in while tile t is multiplied
  __shared__ uint4 ct0[kAsgTileC * kChunks], ct1[kAsgTileC * kChunks], ct2[kAsgTileC * kChunks];
  __shared__ float4 cn0[kAsgTileC / 4], cn1[kAsgTileC / 4], cn2[kAsgTileC / 4];
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int lane = t & (kWave - 1);
  const int col = lane & 31;   // point within a 32-point block; centroid row for A
  const int half = lane >> 5;  // which 8 dims of a 16-dim k-step this lane carries
  const int64_t p0 = (int64_t)blockIdx.x * kAsgPts + w * kAsgPtsPerWave;

  // B operand: this lane's point rows, all 128 dims, as 8 k-steps of 8 bf16
  uint4 xb[kCB][8];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    int64_t p = p0 + cb * 32 + col;
    p = p < N ? p : N - 1;  // clamp: a valid duplicate row, never stored
    const uint4* xr = reinterpret_cast<const uint4*>(x + p * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) xb[cb][ks] = xr[2 * ks + half];
  }

  ArgmaxState st;
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    st.best[cb] = -__builtin_inff();
    st.bidx[cb] = 0;
  }
  const int ntiles = (C + kAsgTileC - 1) / kAsgTileC;
  load_ctile_lds(c, cn, C, 0, ct0, reinterpret_cast<float*>(cn0));
  if (ntiles > 1) {
    load_ctile_lds(c, cn, C, kAsgTileC, ct1, reinterpret_cast<float*>(cn1));
    wait_vmcnt<kLoadsPerTile>();
  } else {
    wait_vmcnt<0>();
  }
  tile_barrier();

  // unrolled by three so that every LDS access names its buffer at compile time
  for (int tile = 0; tile < ntiles; tile += 3) {
    assign_tile(c, cn, C, tile, ntiles, ct0, cn0, ct2, reinterpret_cast<float*>(cn2), xb, st);
    if (tile + 1 >= ntiles) break;
    assign_tile(c, cn, C, tile + 1, ntiles, ct1, cn1, ct0, reinterpret_cast<float*>(cn0), xb, st);
    if (tile + 2 >= ntiles) break;
    assign_tile(c, cn, C, tile + 2, ntiles, ct2, cn2, ct1, reinterpret_cast<float*>(cn1), xb, st);
  }
  float* best = st.best;
  int* bidx = st.bidx;

  // merge the two lanes that share a point (l and l^32)
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
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
  const int rows = (C + kAsgTileC - 1) / kAsgTileC * kAsgTileC;
  hipLaunchKernelGGL(cnorm_kernel, dim3((unsigned)(rows / 16)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(c), C, cnorm);
  const int e = (int)hipGetLastError();
  if (e != 0) return e;
  const int64_t nblk = (N + kAsgPts - 1) / kAsgPts;
  hipLaunchKernelGGL(assign_kernel, dim3((unsigned)nblk), dim3(kAsgNT), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(c), cnorm,
                     assign, best, N, C);
  return (int)hipGetLastError();
}

}  // namespace idxk
