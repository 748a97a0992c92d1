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

// Query heads, summed per dim: qsum[k] = sum_{h<H} q[b,h, 8*l16 + k]. The four
// 16-lane groups of a wave split the heads (group g takes h = g, g + 4, ...),
// G of them per round trip (G loads in flight: the first group before the
// caller's first centroid rows, the rest while those rows are in flight), and
// two lane swaps add the four partial sums. Addition is commutative, so every
// group ends with the same bits: ((p0 + p2) + (p1 + p3)) in each.
template <bool BF16>
struct QHeads {
  static constexpr int G = BF16 ? 4 : 2;  // 16-byte loads: 4 or 8 VGPRs per head
  RowLoad<BF16> r[G];
  __device__ __forceinline__ static int head(int g4, int h0, int i) { return h0 + 4 * i + g4; }
  __device__ __forceinline__ void issue(const void* q, int b, int H, int h0, int l16, int g4) {
#pragma unroll
    for (int i = 0; i < G; ++i) r[i].load(q, (size_t)b * H + min(head(g4, h0, i), H - 1), l16);
  }
  // heads past H (clamped duplicate loads) add zero; no branch, so that no
  // load is deferred to its use
  __device__ __forceinline__ void add(int H, int h0, int g4, float (&qs)[8]) const {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const bool live = head(g4, h0, i) < H;
      float x[8];
      r[i].to_f32(x);
#pragma unroll
      for (int k = 0; k < 8; ++k) qs[k] += live ? x[k] : 0.f;
    }
  }
  // qs from this (first, issued) group and the remaining groups
  __device__ __forceinline__ void sum(const void* q, int b, int H, int l16, int g4,
                                      float (&qs)[8]) const {
#pragma unroll
    for (int k = 0; k < 8; ++k) qs[k] = 0.f;
    add(H, 0, g4, qs);
    for (int h0 = 4 * G; h0 < H; h0 += 4 * G) {
      QHeads<BF16> g;
      g.issue(q, b, H, h0, l16, g4);
      g.add(H, h0, g4, qs);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      qs[k] += __uint_as_float(lane_xor<32>(__float_as_uint(qs[k])));
      qs[k] += __uint_as_float(lane_xor<16>(__float_as_uint(qs[k])));
    }
  }
};

// Where score row r of a request reads its centroid, as a row of the table c
// the caller passes. Dense tables (c = the request's own table): row r. Paged
// tables (c = the pool): the request's page list holds the row, and a
// slot whose entry lies outside [0, n_rows) (or past the list) is not a
// candidate: it scores -inf and its centroid is never read.
struct DenseRows {
  __device__ __forceinline__ int operator()(int r) const { return r; }
};
struct PagedRows {
  const int32_t* indices;  // the request's page list starts at indices[0]
  int64_t avail;           // entries of the list that exist in memory
  int n_rows;              // rows of the centroid pool
  __device__ __forceinline__ int operator()(int r) const {
    if (r >= avail) return -1;
    const int j = indices[r];
    return (unsigned)j < (unsigned)n_rows ? j : -1;
  }
};

// Paged rows whose validated table rows (or -1) were staged in LDS: slot r of
// the request is staged[r - base].
struct StagedRows {
  const int32_t* staged;
  int base;
  __device__ __forceinline__ int operator()(int r) const { return staged[r - base]; }
};

// The centroid table that starts `rows` rows into c.
template <bool BF16>
__device__ __forceinline__ const void* table_of(const void* c, size_t rows) {
  return static_cast<const char*>(c) + rows * kHeadDim * (BF16 ? 2 : 4);
}

// One row-step batch: U row-steps of the workgroup, one row per 16 lanes each.
template <bool BF16, int NT, int U>
struct RowBatch {
  static constexpr int ROWS_PER_STEP = NT / kWave * 4;
  int j[U];  // table row of each of the lane group's rows, -1 when not a candidate
  RowLoad<BF16> ld[U];
  template <typename RowOf>
  __device__ __forceinline__ void issue(const void* c, const RowOf& row_of, int base, int r1,
                                        int my, int l16) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int r = base + u * ROWS_PER_STEP + my;
      r = r < r1 ? r : r1 - 1;  // clamp: a duplicate in-range read, result discarded
      j[u] = row_of(r);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) ld[u].load(c, (size_t)(j[u] < 0 ? 0 : j[u]), l16);
  }
};

// Scores rows [r0, r1) of one request into dst[r] (dst = that request's score row).
// Rows are spread over the workgroup: wave w, lane group g = lane/16 takes row
// 4w + g of each row-step; a batch is U row-steps. The first batch is requested
// before the query heads are summed (qh: its first group already requested by
// the caller), and each next batch before the current one is reduced, so that
// row loads stay in flight (for paged tables a batch reads its U page entries
// first, then the U rows).
// With COHERENT the scores are written with agent-scope stores, which are
// visible to every XCD once complete (see the hand-off in the fused kernel).
template <bool BF16, int NT, bool COHERENT = false, int U = 4, typename RowOf>
__device__ __forceinline__ void score_rows(const void* c, const RowOf& row_of,
                                           const QHeads<BF16>& qh, const void* q, int b, int H,
                                           int r0, int r1, float* dst) {
  using Batch = RowBatch<BF16, NT, U>;
  constexpr int STEP = Batch::ROWS_PER_STEP * U;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int l16 = lane & 15;
  const int my = (t >> 6) * 4 + (lane >> 4);  // row offset inside one step
  if (r1 <= r0) return;
  Batch cur;
  cur.issue(c, row_of, r0, r1, my, l16);
  __builtin_amdgcn_sched_barrier(0);  // the rows are requested before the query is summed
  float qs[8];
  qh.sum(q, b, H, l16, lane >> 4, qs);
  for (int base = r0; base < r1; base += STEP) {
    Batch nxt;
    if (base + STEP < r1) nxt.issue(c, row_of, base + STEP, r1, my, l16);
    // every load of the next batch is issued before the current one is used
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[8];
      cur.ld[u].to_f32(x);
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc = fmaf(qs[k], x[k], acc);
      acc = sum16(acc);
      if (cur.j[u] < 0) acc = -__builtin_inff();
      const int r = base + u * Batch::ROWS_PER_STEP + my;
      if (l16 == 0 && r < r1) {
        if constexpr (COHERENT) {
          __hip_atomic_store(dst + r, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          dst[r] = acc;
        }
      }
    }
    cur = nxt;
  }
}

__device__ __forceinline__ void fill_neg_inf(float* dst, int r0, int r1) {
  for (int r = r0 + (int)threadIdx.x; r < r1; r += (int)blockDim.x) dst[r] = -__builtin_inff();
}

}  // namespace idxk
