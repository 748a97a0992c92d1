// Multi-token (prefill) scoring on the matrix cores ("Round 15 Track C Audit",
// section 1 Target 1: the prompt path scores 16-token tiles of query rows
// against the block keys with one matrix product per tile before the top-K;
// "Round 18 Track C", section 3: the score stage grows with the number of
// query tokens).
//
//   s[b,t,n] = sum_h q[b,t,h,:] . c[b,n,:]   for n < n_valid(pos0[b] + t + 1),
//   n_valid(p) = min(N_pad, ceil(p / page_size)), and -inf elsewhere:
// token t of request b sits at position pos0[b] + t and sees blocks up to the
// one holding itself.
//
// MI355X mapping: the heads are summed once per token in fp32 (q_bar), and
// q_bar is split into bf16 hi + lo parts (hi = bf16(q_bar), lo = bf16(q_bar -
// hi); the remainder is below 2^-16 |q_bar|). Each part goes through
// v_mfma_f32_32x32x16_bf16 against the bf16 centroids with fp32 accumulation:
// A = 32 tokens x 16 dims (registers, built by every wave), B = 16 dims x 32
// centroid rows (16-byte loads straight from HBM, no reuse to stage). A
// workgroup covers 32 tokens x 256 centroid rows (32 per wave: the heads of
// the 32 tokens are summed once for 256 rows; with 128 rows per workgroup
// the prompt-token call measured 17.2 against 16.8 us); the output
// tile has one centroid per lane column, so each store writes two 128-byte
// runs. Column blocks past the last token's visible blocks are not read.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.h"

namespace idxk {

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pf_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfNT = 512;    // 8 waves
constexpr int kPfTok = 32;    // tokens per workgroup (MFMA rows)
constexpr int kPfCols = 256;  // centroid rows per workgroup (32 per wave)

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int prefill_n_valid(int p0, int t, int page_size, int N_pad) {
  const int64_t p = (int64_t)p0 + t + 1;  // tokens visible to token t
  const int64_t nb = (p + page_size - 1) / page_size;
  return (int)(nb < N_pad ? nb : N_pad);
}

__global__ __launch_bounds__(kPfNT) void prefill_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ c,
    const int32_t* __restrict__ pos0, float* __restrict__ scores, int64_t row_stride,
    int32_t* __restrict__ n_valid_out, int T, int H, int N_pad, int page_size, int n_ttiles,
    int n_ctiles, bool fill_dead) {
  const int per_b = n_ttiles * n_ctiles;
  const int b = blockIdx.x / per_b;
  const int rem = blockIdx.x - b * per_b;
  const int tt = rem / n_ctiles;
  const int ct = rem - tt * n_ctiles;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int t0 = tt * kPfTok;
  const int n0 = ct * kPfCols + w * 32;
  const int p0 = max(pos0[b], 0);

  if (ct == 0 && w == 0 && half == 0 && t0 + col < T)
    n_valid_out[(size_t)b * T + t0 + col] = prefill_n_valid(p0, t0 + col, page_size, N_pad);

  // blocks visible to the tile's last token bound every token of the tile
  const int nv_max = prefill_n_valid(p0, min(t0 + kPfTok, T) - 1, page_size, N_pad);
  float* out = scores + (size_t)b * T * row_stride;
  // columns no token of the tile sees get -inf when the scores are the
  // caller's output (staged scores past a token's count are never read); a
  // workgroup with none visible at all leaves at once (the condition is the
  // same for all its waves)
  auto fill_dead_cols = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (t < T && n0 + col < N_pad) out[(size_t)t * row_stride + n0 + col] = -__builtin_inff();
    }
  };
  if (ct * kPfCols >= nv_max) {
    if (fill_dead) fill_dead_cols();
    return;
  }
  const bool live = n0 < nv_max;  // this wave's 32 columns hold a visible block

  // B operand: centroid row n0 + col (clamped in range; discarded past N_pad),
  // 8 dims of each 16-dim k-step; issued first, it lands while q_bar is built
  uint4 cb[8];
  if (live) {
    const int n = min(n0 + col, N_pad - 1);
    const uint4* cr = reinterpret_cast<const uint4*>(c + ((size_t)b * N_pad + n) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) cb[ks] = cr[2 * ks + half];
  }

  // A operand, built once per workgroup in LDS: item (token u, 16-byte chunk k)
  // of the tile sums the token's H heads over 8 dims (16 consecutive lanes read
  // one head row of a token: 256 contiguous bytes), splits the sum into bf16
  // hi + lo, and stores both at slot k * 32 + u, so that a wave's operand read
  // (32 tokens, one chunk) is 512 contiguous bytes.
  __shared__ uint4 a_hi[16 * kPfTok], a_lo[16 * kPfTok];
  constexpr int kItems = 16 * kPfTok / kPfNT;  // items per thread
  // the first four heads of every item are requested before any is added
  // (tokens past T read token T - 1 and add nothing; heads past H add nothing)
  uint4 v[kItems][4];
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int item = it * kPfNT + threadIdx.x;
    const int t = min(t0 + (item >> 4), T - 1);
    const uint4* qt = reinterpret_cast<const uint4*>(q + ((size_t)b * T + t) * H * kHeadDim) + (item & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[it][i] = qt[(size_t)min(i, H - 1) * 16];
  }
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int item = it * kPfNT + threadIdx.x;
    const int u = item >> 4, k = item & 15;
    const bool live_t = t0 + u < T;
    const uint4* qt =
        reinterpret_cast<const uint4*>(q + ((size_t)b * T + min(t0 + u, T - 1)) * H * kHeadDim) + k;
    float sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = 0.f;
    auto add4 = [&](const uint4 (&w4)[4], int h0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = live_t && h0 + i < H;
        const uint32_t wd[4] = {w4[i].x, w4[i].y, w4[i].z, w4[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[2 * e] += live ? bf16_lo(wd[e]) : 0.f;
          sum[2 * e + 1] += live ? bf16_hi(wd[e]) : 0.f;
        }
      }
    };
    add4(v[it], 0);
    // more heads: four per step, their loads in flight together
    for (int h0 = 4; h0 < H; h0 += 4) {
      uint4 w4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w4[i] = qt[(size_t)min(h0 + i, H - 1) * 16];
      add4(w4, h0);
    }
    uint32_t h4[4], l4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h0 = bf16_rne_bits(sum[2 * e]), h1 = bf16_rne_bits(sum[2 * e + 1]);
      const float r0 = sum[2 * e] - __uint_as_float(h0 << 16);
      const float r1 = sum[2 * e + 1] - __uint_as_float(h1 << 16);
      h4[e] = h0 | (h1 << 16);
      l4[e] = bf16_rne_bits(r0) | (bf16_rne_bits(r1) << 16);
    }
    a_hi[k * kPfTok + u] = make_uint4(h4[0], h4[1], h4[2], h4[3]);
    a_lo[k * kPfTok + u] = make_uint4(l4[0], l4[1], l4[2], l4[3]);
  }
  __syncthreads();

  if (!live) {
    if (fill_dead) fill_dead_cols();
    return;
  }
  pf_f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const pf_bf16x8 bv = __builtin_bit_cast(pf_bf16x8, cb[ks]);
    const pf_bf16x8 ah = __builtin_bit_cast(pf_bf16x8, a_hi[(2 * ks + half) * kPfTok + col]);
    const pf_bf16x8 al = __builtin_bit_cast(pf_bf16x8, a_lo[(2 * ks + half) * kPfTok + col]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bv, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bv, acc, 0, 0, 0);
  }

  // value r of this lane: token t0 + 8(r/4) + 4 half + r%4, centroid n0 + col.
  // Block n is visible to token t iff it starts at or before the token:
  // n * page_size <= pos0 + t (the same as n < ceil((pos0 + t + 1) / page_size)).
  const int n = n0 + col;
  const int64_t start = (int64_t)n * page_size - p0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (t < T && n < N_pad && (fill_dead || start <= t))
      out[(size_t)t * row_stride + n] = start <= t ? acc[r] : -__builtin_inff();
  }
}

int launch_prefill_score(const void* q, const void* c, const int32_t* pos0, float* scores,
                         int64_t row_stride, int32_t* n_valid, int B, int T, int H, int N_pad,
                         int page_size, bool fill_dead, void* stream) {
  const int n_ttiles = (T + kPfTok - 1) / kPfTok;
  const int n_ctiles = (N_pad + kPfCols - 1) / kPfCols;
  const int64_t grid = (int64_t)B * n_ttiles * n_ctiles;
  if (grid > 0x7FFFFFFF) return (int)hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_score_kernel, dim3((unsigned)grid), dim3(kPfNT), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(c), pos0, scores, row_stride, n_valid, T, H,
                     N_pad, page_size, n_ttiles, n_ctiles, fill_dead);
  return (int)hipGetLastError();
}

}  // namespace idxk
