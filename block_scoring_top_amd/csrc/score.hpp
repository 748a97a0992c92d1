// Block scoring: s[b,n] = sum_h q[b,h,:] . c[b,n,:] over one chunk of a request's
// centroid table ("Iterate Centroids Score": the indexer's centroid scorer;
// "Round 18 Track C", section 1 Target 2: query heads held in registers, keys
// streamed with lane-contiguous loads).
//
// MI355X mapping: 16 lanes cover one 128-dim centroid row, each lane owning 8
// consecutive dims (16 B of bf16 or 32 B of fp32), so a wave reads 4 whole rows
// per load step and every load instruction is fully coalesced. The query heads
// are summed once per workgroup into qsum[d] = sum_h q[h,d] (fp32) held in
// registers: the exact score is unchanged, only the fp32 rounding differs, and
// the per-row work drops from H*8 to 8 FMAs per lane.
#pragma once

#include "common.hpp"

namespace idxk {

template <bool BF16>
struct RowLoad;

// 8 consecutive bf16 values = one 16-byte load
template <>
struct RowLoad<true> {
  uint4 v;
  __device__ __forceinline__ void load(const void* base, size_t row, int l16) {
    v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * kHeadDim)[l16];
  }
  __device__ __forceinline__ void to_f32(float (&x)[8]) const {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
};

// 8 consecutive fp32 values = two 16-byte loads
template <>
struct RowLoad<false> {
  float4 a, b;
  __device__ __forceinline__ void load(const void* base, size_t row, int l16) {
    const float4* p =
        reinterpret_cast<const float4*>(static_cast<const float*>(base) + row * kHeadDim) + 2 * l16;
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void to_f32(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

// qsum[k] = sum_{h<H} q[b,h, 8*l16 + k], accumulated in head order.
template <bool BF16>
__device__ __forceinline__ void load_qsum(const void* q, int b, int H, int l16, float (&qs)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) qs[k] = 0.f;
  for (int h = 0; h < H; ++h) {
    RowLoad<BF16> r;
    r.load(q, (size_t)b * H + h, l16);
    float x[8];
    r.to_f32(x);
#pragma unroll
    for (int k = 0; k < 8; ++k) qs[k] += x[k];
  }
}

// Where score row r of a request reads its centroid. Dense tables: row
// row_base + r. Paged tables: the request's page list holds the row, and a
// slot whose entry lies outside [0, n_rows) (or past the list) is not a
// candidate: it scores -inf and its centroid is never read.
struct DenseRows {
  size_t row_base;
  __device__ __forceinline__ int64_t operator()(int r) const { return (int64_t)(row_base + r); }
};
struct PagedRows {
  const int32_t* indices;  // the request's page list starts at indices[0]
  int64_t avail;           // entries of the list that exist in memory
  int n_rows;              // rows of the centroid pool
  __device__ __forceinline__ int64_t operator()(int r) const {
    if (r >= avail) return -1;
    const int j = indices[r];
    return (unsigned)j < (unsigned)n_rows ? (int64_t)j : -1;
  }
};

// Scores rows [r0, r1) of one request into dst[r] (dst = that request's score row).
// Rows are spread over the workgroup: wave w, lane group g = lane/16 takes rows
// r0 + 16*NWAVES*... in steps; U row-steps are loaded before any is reduced so
// that several loads per lane are in flight (for paged tables the U page
// entries are read first, then the U rows).
// With COHERENT the scores are written with agent-scope stores, which are
// visible to every XCD once complete (see the hand-off in the fused kernel).
template <bool BF16, int NT, bool COHERENT = false, int U = 4, typename RowOf>
__device__ __forceinline__ void score_rows(const void* c, const RowOf& row_of, const float (&qs)[8],
                                           int r0, int r1, float* dst) {
  constexpr int NW = NT / kWave;
  constexpr int ROWS_PER_STEP = NW * 4;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int l16 = lane & 15;
  const int my = (t >> 6) * 4 + (lane >> 4);  // row offset inside one step
  if (r1 <= r0) return;
  for (int base = r0; base < r1; base += ROWS_PER_STEP * U) {
    int64_t j[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int r = base + u * ROWS_PER_STEP + my;
      r = r < r1 ? r : r1 - 1;  // clamp: a duplicate in-range read, result discarded
      j[u] = row_of(r);
    }
    RowLoad<BF16> ld[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ld[u].load(c, (size_t)(j[u] < 0 ? 0 : j[u]), l16);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[8];
      ld[u].to_f32(x);
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc = fmaf(qs[k], x[k], acc);
      acc = sum16(acc);
      if (j[u] < 0) acc = -__builtin_inff();
      const int r = base + u * ROWS_PER_STEP + my;
      if (l16 == 0 && r < r1) {
        if constexpr (COHERENT) {
          __hip_atomic_store(dst + r, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          dst[r] = acc;
        }
      }
    }
  }
}

__device__ __forceinline__ void fill_neg_inf(float* dst, int r0, int r1) {
  for (int r = r0 + (int)threadIdx.x; r < r1; r += (int)blockDim.x) dst[r] = -__builtin_inff();
}

}  // namespace idxk
