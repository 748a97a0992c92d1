// The indexer's selects with four 8-bit radix passes and no linear-bin pass:
// the radix of the proposal seed in "Iterate Topk" (section 6) and of the
// four-pass loop in "Round 18 Track C" (section 1, Target 1). The results are
// those of the library's own selects; the launches exist to measure that
// design against them (IDX_RADIX8).
#include "indexer_kernels.hpp"

namespace idxk {

int launch_topk_radix8(const void* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
                       int B, int N, int K, bool sorted, void* split_ws, void* stream,
                       bool dot_scores) {
  return launch_topk_f32<true>(scores, n_valid, ids, counts, B, N, K, sorted, split_ws, stream,
                               dot_scores);
}

int launch_select_radix8(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                         int32_t* counts, float* scores_out, int B, int H, int N_pad,
                         int page_size, int K, bool bf16, bool sorted, int chunk, bool wide,
                         uint32_t* tickets, float* stage, int stage_stride, const int32_t* indptr,
                         const int32_t* indices, int64_t n_indices, int n_rows, void* stream) {
  return launch_select_t<true>(q, c, seq_len, ids, counts, scores_out, B, H, N_pad, page_size, K,
                               bf16, sorted, chunk, wide, tickets, stage, stage_stride, indptr,
                               indices, n_indices, n_rows, stream);
}

}  // namespace idxk
