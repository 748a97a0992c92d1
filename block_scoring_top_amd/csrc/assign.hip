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
// triple-buffered LDS tile of 64 centroids, filled by direct-to-LDS loads that
// overlap the products of the tiles before it), the B operand a 16-dim x
// 32-point slice of X^T (registers, loaded once). The 32x32 result tile then
// has one point per lane column (lane % 32) and 16 centroid rows per lane, so
// the max over centroids is mostly in-lane; lanes l and l^32 hold disjoint
// centroid rows of the same point and are merged once at the end.
//
// Software pipeline: two accumulator sets alternate between tiles. While the
// products of tile t accumulate into one set, the running argmax of tile t-1
// is taken from the other, half of one accumulator per k-step, so that its
// vector instructions issue in the shadow of that k-step's matrix products
// (each k-step is a scheduling region of its own; it also reads the next
// k-step's A fragments from LDS).
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
// (their bias is -inf, so they never win). Each wave also writes all 64 of the
// tile's biases (the same values in every wave, from the -inf-padded norm
// buffer), so every wave issues the same kLoadsPerTile loads per tile and none
// branches. A tile past the last one (loaded by the pipeline's last steps and
// never read) takes its rows from row C-1 and its biases from the last tile.
constexpr int kLoadsPerTile = kTileLoads + 1;
// Byte offset of load i of this lane within a tile of whole rows.
__device__ __forceinline__ int refill_off(int i) {
  const int t = threadIdx.x;
  const int w = t >> 6, lane = t & (kWave - 1);
  const int p = (w * kTileLoads + i) * kWave + lane;
  const int row = p >> 4;
  const int k = (p & 15) ^ (row & 15);
  return row * kHeadDim * 2 + k * 16;
}
// roff[i] = refill_off(i), computed once: a tile of 64 whole rows is loaded
// from the tile's base plus these offsets; a partial last tile (and a tile
// past the end) clamps each row to C - 1.
__device__ __forceinline__ void load_ctile_lds(const uint16_t* __restrict__ c,
                                               const float* __restrict__ cn, int C, int j0,
                                               uint4* tile, float* tn,
                                               const int (&roff)[kTileLoads]) {
  const int t = threadIdx.x;
  const int w = t >> 6, lane = t & (kWave - 1);
  const int jb = min(j0, (C - 1) / kAsgTileC * kAsgTileC);
  if (j0 + kAsgTileC <= C) {
    const char* base = reinterpret_cast<const char*>(c + (size_t)j0 * kHeadDim);
#pragma unroll
    for (int i = 0; i < kTileLoads; ++i)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(base + roff[i]),
                                       tile + (w * kTileLoads + i) * kWave, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(cn + jb + lane, tn, 4, 0, 0);
    return;
  }
#pragma unroll
  for (int i = 0; i < kTileLoads; ++i) {
    const int slot0 = (w * kTileLoads + i) * kWave;  // wave-uniform LDS base
    const int p = slot0 + lane;
    const int row = p >> 4;
    const int k = (p & 15) ^ (row & 15);
    const int j = j0 + row < C ? j0 + row : C - 1;
    __builtin_amdgcn_global_load_lds(c + (size_t)j * kHeadDim + k * 8, tile + slot0, 16, 0, 0);
  }
  __builtin_amdgcn_global_load_lds(cn + jb + lane, tn, 4, 0, 0);
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

// Running argmax of one 32x32 accumulator tile, without branches: the lane's
// 16 rows are centroids jbase + 8 (r >> 2) + (r & 3), r = 0..15 (jbase
// includes the lane's 4 * half). Part 0 takes the max m and searches rows
// 15..8 for it, part 1 searches rows 7..0 and updates the running best. The
// search keeps the lowest row holding m, and a strictly larger m replaces the
// best, so among equal values the lowest centroid index wins (tiles and row
// blocks are visited in increasing index order).
__device__ __forceinline__ void argmax_part0(const f32x16& v, float& m, int& rr) {
  m = v[0];
#pragma unroll
  for (int r = 1; r < 15; r += 2)  // a chain of 3-input maxes
    m = __builtin_fmaxf(__builtin_fmaxf(m, v[r]), v[r + 1]);
  m = __builtin_fmaxf(m, v[15]);
  rr = 8 * 3 + 3;  // the row offset of r = 15
#pragma unroll
  for (int r = 14; r >= 8; --r) rr = (v[r] == m) ? (8 * (r >> 2) + (r & 3)) : rr;
}
__device__ __forceinline__ void argmax_part1(const f32x16& v, float m, int rr, int jbase,
                                             float& best, int& bidx) {
#pragma unroll
  for (int r = 7; r >= 0; --r) rr = (v[r] == m) ? (8 * (r >> 2) + (r & 3)) : rr;
  const bool better = m > best;
  best = better ? m : best;
  bidx = better ? jbase + rr : bidx;
}

// One tile step: the products of tile `tile` (LDS tile cur) into accumulator
// set `acc`, the direct-to-LDS refill of tile + 2 into nxt (the tile read two
// steps ago, which every wave has finished: the previous step ended with a
// barrier), and, with EPI, the argmax of the previous tile from `prev`,
// interleaved with the products. aoff[ks] is the byte offset of this lane's A
// fragment of k-step ks within a tile (the second 32-row block is 8 KiB on).
template <bool EPI>
__device__ __forceinline__ void tile_step(const uint16_t* __restrict__ c,
                                          const float* __restrict__ cn, int C, int tile,
                                          const uint4* cur, const float4* curn, uint4* nxt,
                                          float* nxtn, const uint4 (&xb)[kCB][8],
                                          f32x16 (&acc)[2][kCB], const f32x16 (&prev)[2][kCB],
                                          ArgmaxState& st, const int (&aoff)[8],
                                          const int (&roff)[kTileLoads]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int half = lane >> 5;
  const int j0 = tile * kAsgTileC;
  const char* curb = reinterpret_cast<const char*>(cur);
  auto afrag = [&](int ks, int rb) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(curb + aoff[ks] + rb * 32 * kChunks * 16));
  };
  // The biases (rows 8g + 4 half + 0..3 of each 32-row block) go straight into
  // the last point block's accumulators: the first k-step's products of every
  // point block start from them.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 b4 = curn[rb * 8 + 2 * g + half];
      acc[rb][kCB - 1][4 * g + 0] = b4.x;
      acc[rb][kCB - 1][4 * g + 1] = b4.y;
      acc[rb][kCB - 1][4 * g + 2] = b4.z;
      acc[rb][kCB - 1][4 * g + 3] = b4.w;
    }
  bf16x8 a0 = afrag(0, 0);
  bf16x8 a1 = afrag(0, 1);
  load_ctile_lds(c, cn, C, j0 + 2 * kAsgTileC, nxt, nxtn, roff);
  __builtin_amdgcn_sched_barrier(0);
  const int jp = j0 - kAsgTileC + 4 * half;  // the previous tile's rows of this lane
  float m = 0.f;
  int rr = 0;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bf16x8 n0 = a0, n1 = a1;
    if (ks < 7) {  // the next k-step's fragments
      n0 = afrag(ks + 1, 0);
      n1 = afrag(ks + 1, 1);
    }
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const bf16x8 b = as_bf16x8(xb[cb][ks]);
      acc[0][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          a0, b, ks == 0 ? acc[0][kCB - 1] : acc[0][cb], 0, 0, 0);
      acc[1][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          a1, b, ks == 0 ? acc[1][kCB - 1] : acc[1][cb], 0, 0, 0);
    }
    if constexpr (EPI) {  // k-steps 2i, 2i+1: accumulator (cb, rb) = (i >> 1, i & 1)
      const int cb = ks >> 2, rb = (ks >> 1) & 1;
      if ((ks & 1) == 0) argmax_part0(prev[rb][cb], m, rr);
      else argmax_part1(prev[rb][cb], m, rr, jp + 32 * rb, st.best[cb], st.bidx[cb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    a0 = n0;
    a1 = n1;
  }
  // Tile + 1 has landed once at most this step's refill loads are outstanding
  // in this wave, and in every wave after the barrier, which also frees `cur`
  // for the next step's refill.
  wait_vmcnt<kLoadsPerTile>();
  tile_barrier();
}

__global__ __launch_bounds__(kAsgNT, 2) void assign_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ c,
                                                           const float* __restrict__ cn,
                                                           int32_t* __restrict__ assign,
                                                           float* __restrict__ best_out,
                                                           int64_t N, int C) {
  // three LDS tiles of 64 centroids (16 KiB each) and their biases, as separate
  // objects: the compiler then tells a refill's target from the tile being
  // read, and the reads do not wait for the refill
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
  // A fragment and refill offsets, computed once and kept opaque (otherwise
  // the compiler recomputes them per buffer and step, and spills)
  int aoff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    aoff[ks] = swz(col, 2 * ks + half) * 16;
    asm volatile("" : "+v"(aoff[ks]));
  }
  int roff[kTileLoads];
#pragma unroll
  for (int i = 0; i < kTileLoads; ++i) {
    roff[i] = refill_off(i);
    asm volatile("" : "+v"(roff[i]));
  }
  const int ntiles = (C + kAsgTileC - 1) / kAsgTileC;
  load_ctile_lds(c, cn, C, 0, ct0, reinterpret_cast<float*>(cn0), roff);
  load_ctile_lds(c, cn, C, kAsgTileC, ct1, reinterpret_cast<float*>(cn1), roff);
  wait_vmcnt<kLoadsPerTile>();
  tile_barrier();

  // Tile tl + PH uses LDS tile (tl + PH) % 3 and accumulator set (tl + PH) % 2:
  // the loop is unrolled by six so that both are fixed at compile time.
  f32x16 accA[2][kCB], accB[2][kCB];
#define IDX_STEP(PH, EPI_, CUR, CURN, NXT, NXTN)                                              \
  tile_step<EPI_>(c, cn, C, tl + (PH), CUR, CURN, NXT, reinterpret_cast<float*>(NXTN), xb,    \
                  ((PH) % 2) ? accB : accA, ((PH) % 2) ? accA : accB, st, aoff, roff)
  int tl = 0;
  IDX_STEP(0, false, ct0, cn0, ct2, cn2);
  for (tl = 0; tl + 1 < ntiles; tl += 6) {
    IDX_STEP(1, true, ct1, cn1, ct0, cn0);
    if (tl + 2 >= ntiles) break;
    IDX_STEP(2, true, ct2, cn2, ct1, cn1);
    if (tl + 3 >= ntiles) break;
    IDX_STEP(3, true, ct0, cn0, ct2, cn2);
    if (tl + 4 >= ntiles) break;
    IDX_STEP(4, true, ct1, cn1, ct0, cn0);
    if (tl + 5 >= ntiles) break;
    IDX_STEP(5, true, ct2, cn2, ct1, cn1);
    if (tl + 6 >= ntiles) break;
    IDX_STEP(6, true, ct0, cn0, ct2, cn2);
  }
#undef IDX_STEP
  // the last tile's argmax
  {
    const int last = ntiles - 1;
    const int jp = last * kAsgTileC + 4 * half;
    auto epi = [&](const f32x16 (&pa)[2][kCB]) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float m;
          int rr;
          argmax_part0(pa[rb][cb], m, rr);
          argmax_part1(pa[rb][cb], m, rr, jp + 32 * rb, st.best[cb], st.bidx[cb]);
        }
    };
    if (last & 1) epi(accB);
    else epi(accA);
  }
  wait_vmcnt<0>();  // no direct-to-LDS load may outlive the workgroup
  float* best = st.best;
  int* bidx = st.bidx;

  // The point indices are derived again from an opaque copy of the thread
  // index: kept from the start, they would hold registers across the loop.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int64_t q0 = (int64_t)blockIdx.x * kAsgPts + (tid >> 6) * kAsgPtsPerWave + (tid & 31);
  // merge the two lanes that share a point (l and l^32)
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const float ov = __shfl_xor(best[cb], 32, kWave);
    const int oi = __shfl_xor(bidx[cb], 32, kWave);
    if (ov > best[cb] || (ov == best[cb] && oi < bidx[cb])) {
      best[cb] = ov;
      bidx[cb] = oi;
    }
    const int64_t p = q0 + cb * 32;
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
