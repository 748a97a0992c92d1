// Kernels of the indexer path: score, top-K, fused score + top-K.
#include <hip/hip_runtime.h>

#include <mutex>

#include "idx.h"
#include "indexer_kernels.hpp"

namespace idxk {

constexpr int kScoreNT = 256;   // idx_score workgroup: 4 waves

// ---- idx_score ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kScoreNT) void score_kernel(const void* __restrict__ q,
                                                         const void* __restrict__ c,
                                                         const int32_t* __restrict__ seq_len,
                                                         float* __restrict__ scores, int H,
                                                         int N_pad, int page_size, int chunk,
                                                         int nchunk) {
  const int b = blockIdx.x / nchunk;
  const int ch = blockIdx.x - b * nchunk;
  const int nv = n_valid_blocks(seq_len[b], page_size, N_pad);
  const int r0 = ch * chunk;
  const int r_end = min(r0 + chunk, N_pad);
  const int r1 = min(r_end, nv);
  float* dst = scores + (size_t)b * N_pad;
  if (r1 > r0) {
    QHeads<BF16> qh;
    qh.issue(q, b, H, 0, threadIdx.x & 15, (threadIdx.x >> 4) & 3);
    score_rows<BF16, kScoreNT>(table_of<BF16>(c, (size_t)b * N_pad), DenseRows{}, qh, q, b, H,
                               r0, r1, dst);
  }
  fill_neg_inf(dst, max(r0, nv), r_end);
}

// ---- launchers ---------------------------------------------------------------------------
int launch_score(const void* q, const void* c, const int32_t* seq_len, float* scores, int B,
                 int H, int N_pad, int page_size, bool bf16, int chunk, void* stream) {
  const int nchunk = (N_pad + chunk - 1) / chunk;
  const dim3 grid((unsigned)B * nchunk), block(kScoreNT);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    hipLaunchKernelGGL(score_kernel<true>, grid, block, 0, s, q, c, seq_len, scores, H, N_pad,
                       page_size, chunk, nchunk);
  else
    hipLaunchKernelGGL(score_kernel<false>, grid, block, 0, s, q, c, seq_len, scores, H, N_pad,
                       page_size, chunk, nchunk);
  return (int)hipGetLastError();
}

// bf16 rows (any distribution, adaptive bins): the same shapes as the fp32
// rows, without the dot-product instances.
int launch_topk_bf16(const void* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
                     int B, int N, int K, bool sorted, void* split_ws, void* stream) {
  const dim3 grid((unsigned)B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int S = split_ws != nullptr ? topk_segments(B, N, K) : 1;
  if (S > 1) {
    const int L = ((N + S - 1) / S + 3) / 4 * 4;
    const int cstride = (S * K + 3) / 4 * 4;
    char* w = static_cast<char*>(split_ws);
    uint32_t* tickets = reinterpret_cast<uint32_t*>(w);
    float* cs = reinterpret_cast<float*>(w + topk_cand_offset());
    int32_t* ci = reinterpret_cast<int32_t*>(w + topk_cand_offset() + (size_t)B * cstride * 4);
    const dim3 g2((unsigned)((int64_t)B * S));
    const bool merge2 = (int64_t)S * K <= kTopkNT * 2 * 4;
#define IDX_LAUNCH_SPLIT16(SO, MS)                                                             \
  hipLaunchKernelGGL((topk_split_kernel<SO, MS, true>), g2, dim3(kTopkNT),                     \
                     SO ? sort_lds_bytes(K) : 0, s, scores, n_valid, ids, counts, N, K, S, L,  \
                     tickets, cs, ci, cstride)
    if (sorted) {
      if (merge2) IDX_LAUNCH_SPLIT16(true, 2);
      else IDX_LAUNCH_SPLIT16(true, kTopkSlots);
    } else {
      IDX_LAUNCH_SPLIT16(false, 0);
    }
#undef IDX_LAUNCH_SPLIT16
    return (int)hipGetLastError();
  }
  const bool narrow = B >= 512 && N <= 2048 && (!sorted || K <= 1024);
#define IDX_LAUNCH_TOPK16(SO, NT_, SL_)                                                       \
  hipLaunchKernelGGL((topk_kernel<SO, NT_, SL_, true, true>), grid, dim3(NT_),               \
                     SO ? sort_lds_bytes(K) : 0, s, scores, n_valid, ids, counts, N, K)
  if (narrow) {
    if (sorted) IDX_LAUNCH_TOPK16(true, 256, 2);
    else IDX_LAUNCH_TOPK16(false, 256, 2);
  } else if (N <= kTopkNT * 2 * 4) {
    if (sorted) IDX_LAUNCH_TOPK16(true, kTopkNT, 2);
    else IDX_LAUNCH_TOPK16(false, kTopkNT, 2);
  } else {
    if (sorted) IDX_LAUNCH_TOPK16(true, kTopkNT, kTopkSlots);
    else IDX_LAUNCH_TOPK16(false, kTopkNT, kTopkSlots);
  }
#undef IDX_LAUNCH_TOPK16
  return (int)hipGetLastError();
}

int launch_topk(const void* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
                int B, int N, int K, bool sorted, void* split_ws, void* stream, bool dot_scores,
                bool bf16, bool radix8) {
  if (bf16) return launch_topk_bf16(scores, n_valid, ids, counts, B, N, K, sorted, split_ws, stream);
  if (radix8)
    return launch_topk_radix8(scores, n_valid, ids, counts, B, N, K, sorted, split_ws, stream,
                              dot_scores);
  return launch_topk_f32<false>(scores, n_valid, ids, counts, B, N, K, sorted, split_ws, stream,
                                dot_scores);
}

size_t topk_split_workspace_bytes(int B, int N, int K) {
  const int S = topk_segments(B, N, K);
  if (S <= 1) return 0;
  const size_t cstride = ((size_t)S * K + 3) / 4 * 4;
  return topk_cand_offset() + (size_t)B * cstride * 8;
}

int launch_select(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                  int32_t* counts, float* scores_out, int B, int H, int N_pad, int page_size,
                  int K, bool bf16, bool sorted, int chunk, bool wide, uint32_t* tickets,
                  float* stage, int stage_stride, const int32_t* indptr, const int32_t* indices,
                  int64_t n_indices, int n_rows, void* stream, bool radix8) {
  if (radix8)
    return launch_select_radix8(q, c, seq_len, ids, counts, scores_out, B, H, N_pad, page_size,
                                K, bf16, sorted, chunk, wide, tickets, stage, stage_stride, indptr,
                                indices, n_indices, n_rows, stream);
  return launch_select_t<false>(q, c, seq_len, ids, counts, scores_out, B, H, N_pad, page_size,
                                K, bf16, sorted, chunk, wide, tickets, stage, stage_stride, indptr,
                                indices, n_indices, n_rows, stream);
}

int launch_select_tokens(const void* q, const void* c, const int32_t* pos0, int32_t* ids,
                         int32_t* counts, float* scores_out, int B, int tokens, int H, int N_pad,
                         int page_size, int K, bool bf16, bool sorted, int chunk, bool wide,
                         uint32_t* tickets, float* stage, int stage_stride, void* stream) {
  if (tokens < 1) return (int)hipErrorInvalidValue;
  return launch_select_t<false>(q, c, pos0, ids, counts, scores_out, B, H, N_pad, page_size, K,
                                bf16, sorted, chunk, wide, tickets, stage, stage_stride, nullptr,
                                nullptr, 0, 0, stream, tokens);
}

// ---- static scratch of idx_select_noalloc ------------------------------------------------
// Arrival lines, then score staging. Each GPU the library runs on holds its own
// copy until the process ends. In host code `scratch` is only a stand-in for the
// symbol: the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[IDX_NOALLOC_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

int noalloc_scratch(void** out, void* stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    // arrival lines start at zero (a fill kernel, so that the clear is also
    // correct when the first call is captured into a graph)
    const int words = (int)(IDX_NOALLOC_TICKET_BYTES / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3(128), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return 0;
}

}  // namespace idxk
