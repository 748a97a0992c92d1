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
// workgroup covers 32 tokens x 128 centroid rows (32 per wave); the output
// tile has one centroid per lane column, so each store writes two 128-byte
// runs. Column blocks past the last token's visible blocks are not read.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.h"

namespace idxk {

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pf_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfNT = 256;    // 4 waves
constexpr int kPfTok = 32;    // tokens per workgroup (MFMA rows)
constexpr int kPfCols = 128;  // centroid rows per workgroup (32 per wave)

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
    int n_ctiles) {
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
  if (n0 >= N_pad) return;
  if (n0 >= nv_max) {  // nothing visible in this column block: -inf for every token
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
      const int n = n0 + col;
      if (t < T && n < N_pad) out[(size_t)t * row_stride + n] = -__builtin_inff();
    }
    return;
  }

  // B operand: centroid row n0 + col (clamped in range; discarded past N_pad),
  // 8 dims of each 16-dim k-step
  uint4 cb[8];
  {
    const int n = min(n0 + col, N_pad - 1);
    const uint4* cr = reinterpret_cast<const uint4*>(c + ((size_t)b * N_pad + n) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) cb[ks] = cr[2 * ks + half];
  }

  // A operand: q_bar of token t0 + col (zero past T), split into bf16 hi + lo
  uint32_t hi[8][4], lo[8][4];
  {
    const int t = t0 + col;
    float s[8][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[ks][e] = 0.f;
    if (t < T) {
      const uint16_t* qt = q + ((size_t)b * T + t) * H * kHeadDim;
      for (int h = 0; h < H; ++h) {
        const uint4* qr = reinterpret_cast<const uint4*>(qt + (size_t)h * kHeadDim);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const uint4 v = qr[2 * ks + half];
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            s[ks][2 * k] += bf16_lo(wd[k]);
            s[ks][2 * k + 1] += bf16_hi(wd[k]);
          }
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t h0 = bf16_rne_bits(s[ks][2 * k]), h1 = bf16_rne_bits(s[ks][2 * k + 1]);
        const float r0 = s[ks][2 * k] - __uint_as_float(h0 << 16);
        const float r1 = s[ks][2 * k + 1] - __uint_as_float(h1 << 16);
        hi[ks][k] = h0 | (h1 << 16);
        lo[ks][k] = bf16_rne_bits(r0) | (bf16_rne_bits(r1) << 16);
      }
    }
  }

  pf_f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const pf_bf16x8 bv = __builtin_bit_cast(pf_bf16x8, cb[ks]);
    const pf_bf16x8 ah = __builtin_bit_cast(pf_bf16x8, make_uint4(hi[ks][0], hi[ks][1], hi[ks][2], hi[ks][3]));
    const pf_bf16x8 al = __builtin_bit_cast(pf_bf16x8, make_uint4(lo[ks][0], lo[ks][1], lo[ks][2], lo[ks][3]));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bv, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bv, acc, 0, 0, 0);
  }

  // value r of this lane: token t0 + 8(r/4) + 4 half + r%4, centroid n0 + col
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
    const int n = n0 + col;
    if (t < T && n < N_pad) {
      const int nv = prefill_n_valid(p0, t, page_size, N_pad);
      out[(size_t)t * row_stride + n] = n < nv ? acc[r] : -__builtin_inff();
    }
  }
}

int launch_prefill_score(const void* q, const void* c, const int32_t* pos0, float* scores,
                         int64_t row_stride, int32_t* n_valid, int B, int T, int H, int N_pad,
                         int page_size, void* stream) {
  const int n_ttiles = (T + kPfTok - 1) / kPfTok;
  const int n_ctiles = (N_pad + kPfCols - 1) / kPfCols;
  const int64_t grid = (int64_t)B * n_ttiles * n_ctiles;
  if (grid > 0x7FFFFFFF) return (int)hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_score_kernel, dim3((unsigned)grid), dim3(kPfNT), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(c), pos0, scores, row_stride, n_valid, T, H,
                     N_pad, page_size, n_ttiles, n_ctiles);
  return (int)hipGetLastError();
}

}  // namespace idxk
