// Host-side launchers of the indexer kernels (defined in the .hip files).
// Plain C++ declarations, no HIP types: the stream travels as void*.
// Each returns 0 on success or the hipError_t of a failed launch.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace idxk {

int launch_score(const void* q, const void* c, const int32_t* seq_len, float* scores, int B,
                 int H, int N_pad, int page_size, bool bf16, int chunk, void* stream);

// split_ws: NULL (one workgroup per row), or at least topk_split_workspace_bytes
// of zero-filled workspace (long rows are then cut into segments selected by
// several workgroups, merged by the last one; the workspace is left zeroed).
// dot_scores: rows of dot-product scores (value bins in the linear pass of
// rows up to 8192 entries); otherwise rows of any distribution (bins chosen
// per row).
// bf16: the scores are bf16 (raw 16-bit patterns, any distribution).
// radix8: fp32 rows selected with four 8-bit radix passes and no linear-bin
// pass (the same results; for comparison).
int launch_topk(const void* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
                int B, int N, int K, bool sorted, void* split_ws, void* stream,
                bool dot_scores = false, bool bf16 = false, bool radix8 = false);
int launch_topk_bf16(const void* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
                     int B, int N, int K, bool sorted, void* split_ws, void* stream);
int launch_topk_radix8(const void* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
                       int B, int N, int K, bool sorted, void* split_ws, void* stream,
                       bool dot_scores);
size_t topk_split_workspace_bytes(int B, int N, int K);

// indptr == nullptr: dense tables (c is [B, N_pad, 128], seq_len gives the
// valid rows). Otherwise paged: c is a pool of n_rows centroids, request b's
// slots are indices[indptr[b] .. indptr[b+1]) (n_indices entries exist), N_pad
// is the longest page list, and seq_len / page_size are unused.
// radix8 (dense tables only): four 8-bit radix passes, no linear-bin pass.
int launch_select(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                  int32_t* counts, float* scores_out, int B, int H, int N_pad, int page_size,
                  int K, bool bf16, bool sorted, int chunk, bool wide, uint32_t* tickets,
                  float* stage, int stage_stride, const int32_t* indptr, const int32_t* indices,
                  int64_t n_indices, int n_rows, void* stream, bool radix8 = false);
// launch_select over prompt tokens: row b is token b % tokens of request
// b / tokens (q rows [B, H, D] with B = requests * tokens, c tables per
// request), seq_len the requests' first positions.
int launch_select_tokens(const void* q, const void* c, const int32_t* pos0, int32_t* ids,
                         int32_t* counts, float* scores_out, int B, int tokens, int H, int N_pad,
                         int page_size, int K, bool bf16, bool sorted, int chunk, bool wide,
                         uint32_t* tickets, float* stage, int stage_stride, void* stream);
int launch_select_radix8(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                         int32_t* counts, float* scores_out, int B, int H, int N_pad,
                         int page_size, int K, bool bf16, bool sorted, int chunk, bool wide,
                         uint32_t* tickets, float* stage, int stage_stride, const int32_t* indptr,
                         const int32_t* indices, int64_t n_indices, int n_rows, void* stream);

// The calling device's copy of the static scratch of idx_select_noalloc
// (IDX_NOALLOC_SCRATCH_BYTES). The first call on a device looks up its address
// and clears the arrival lines with a fill kernel on `stream`.
int noalloc_scratch(void** scratch, void* stream);

int launch_assign(const void* x, const void* c, int32_t* assign, float* best, int64_t N, int C,
                  float* cnorm, void* stream);

// Block means of the keys: c[b,n,:] = mean of k[b, tokens of block n, :].
int launch_pool_keys(const void* k, const int32_t* seq_len, void* c, int B, int S_pad, int N_pad,
                     int page_size, bool bf16, void* stream);

// Prefill scores of T tokens per request into scores[(b*T + t) * row_stride + n]
// (row_stride >= N_pad) and each token's visible block count into n_valid[b*T + t].
int launch_prefill_score(const void* q, const void* c, const int32_t* pos0, float* scores,
                         int64_t row_stride, int32_t* n_valid, int B, int T, int H, int N_pad,
                         int page_size, bool fill_dead, void* stream);

}  // namespace idxk
