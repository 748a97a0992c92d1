// C ABI of the indexer: host-side argument validation, workspace layout and
// dispatch to the kernel launchers. Validation makes no HIP call, so every
// error path runs (and is tested) on a machine without a GPU.
#include <stdint.h>
#include <string.h>

#include <new>

#include "idx.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Blocks scored per workgroup: a power of two in [lo, 256] chosen so that the
// grid holds about `target` workgroups over the padded tables; or the caller's
// choice from the flags.
int chunk_rows(int B, int N_pad, uint32_t flags, int lo, int target) {
  const uint32_t l = (flags & IDX_CHUNK_MASK) >> IDX_CHUNK_SHIFT;
  if (l != 0) return 1 << l;
  const int64_t total = (int64_t)B * N_pad;
  int c = lo;
  while (c < 256 && total / (2 * c) >= target) c *= 2;
  return c;
}
// idx_score: 256-thread workgroups, 16 rows per step, ~1024 of them (4 per CU)
constexpr int kScoreChunkMin = 16, kScoreTarget = 1024;
// idx_select: many requests -> 512-thread workgroups (16 rows per step, ~1024)
constexpr int kWideMaxRequests = 32;
// largest score-ordered K that the many-request workgroups (512 threads) sort
// (kept at four ids per thread of a 256-thread workgroup)
constexpr int kNarrowMaxSortedK = 1024;
// idx_select, few requests: 1024-thread workgroups, which score 64 rows per
// step. A chunk of 32 rows leaves half of one idle, so it pays only while it
// spreads the call over more CUs (the tiny score-ordered call of 1024 blocks:
// 7.8 us with 64-row chunks, 7.55 with 32, 7.9 with 16). The chunk is the
// smallest (32..256 rows) whose grid fits one workgroup per CU: with two per
// CU two requests of 7501 blocks took 13.3 us (32-row chunks, 469 workgroups)
// against 10.4 (64 rows, 235), and eight such requests in bf16 13.1 us against
// 11.9 (128 and 256 rows).
constexpr int kWideChunkMin = 32, kWideMaxGrid = 256;
int chunk_rows_wide(int B, int N_pad, uint32_t flags) {
  const uint32_t l = (flags & IDX_CHUNK_MASK) >> IDX_CHUNK_SHIFT;
  if (l != 0) return 1 << l;
  int c = kWideChunkMin;
  while (c < 256 && (int64_t)B * ((N_pad + c - 1) / c) > kWideMaxGrid) c *= 2;
  return c;
}

int check_chunk_flag(uint32_t flags) {
  const uint32_t l = (flags & IDX_CHUNK_MASK) >> IDX_CHUNK_SHIFT;
  if (l != 0 && (l < 4 || l > 14)) return IDX_ERR_INVALID_ARG;
  if (flags & ~(IDX_SORTED | IDX_RADIX8 | IDX_CHUNK_MASK)) return IDX_ERR_INVALID_ARG;
  return IDX_OK;
}

int check_scoring_args(const void* q, const void* c, const int32_t* seq_len, int B, int H, int D,
                       int N_pad, int page_size, idx_dtype dt) {
  if (q == nullptr || c == nullptr || seq_len == nullptr) return IDX_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(c, 16) || !aligned(seq_len, 4)) return IDX_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || D < 1 || N_pad < 1 || page_size < 1) return IDX_ERR_INVALID_ARG;
  if (dt != IDX_F32 && dt != IDX_BF16) return IDX_ERR_INVALID_ARG;
  if ((int64_t)B * N_pad > kMaxRows) return IDX_ERR_INVALID_ARG;
  if (H > IDX_MAX_HEADS || D != IDX_HEAD_DIM) return IDX_ERR_UNSUPPORTED;
  return IDX_OK;
}

int hip_status(int e) { return e == 0 ? IDX_OK : IDX_ERR_HIP; }

// idx_select workspace: [arrival counters: a fixed 2 MiB, one 128-byte line per
// request][staging: B rows of round_up(N_pad, 4) floats]. Every call returns all
// of it to zero, so one workspace can serve calls of any shape that fits.
constexpr int kMaxRequests = 16384;
constexpr size_t kTicketBytes = kMaxRequests * size_t(128);
int stage_stride(int N_pad) { return (int)round_up((size_t)N_pad, 4); }

}  // namespace

extern "C" {

const char* idx_status_string(int status) {
  switch (status) {
    case IDX_OK: return "ok";
    case IDX_ERR_INVALID_ARG: return "invalid argument";
    case IDX_ERR_UNSUPPORTED: return "unsupported configuration";
    case IDX_ERR_WORKSPACE: return "workspace missing or too small";
    case IDX_ERR_HIP: return "HIP launch failed";
    case IDX_ERR_SCRATCH: return "shape exceeds the static scratch of idx_select_noalloc";
    case IDX_ERR_NO_MEMORY: return "host memory for the plan could not be allocated";
    default: return "unknown status";
  }
}

int idx_score(const void* q, const void* c, const int32_t* seq_len, float* scores, int B, int H,
              int D, int N_pad, int page_size, idx_dtype dt, void* stream) {
  int st = check_scoring_args(q, c, seq_len, B, H, D, N_pad, page_size, dt);
  if (st != IDX_OK) return st;
  if (scores == nullptr || !aligned(scores, 4)) return IDX_ERR_INVALID_ARG;
  return hip_status(idxk::launch_score(q, c, seq_len, scores, B, H, N_pad, page_size,
                                       dt == IDX_BF16,
                                       chunk_rows(B, N_pad, 0, kScoreChunkMin, kScoreTarget),
                                       stream));
}

size_t idx_topk_workspace_bytes(int B, int N, int K, uint32_t flags) {
  (void)flags;
  if (B < 1 || N < 1 || K < 1) return 0;
  return idxk::topk_split_workspace_bytes(B, N, K);
}

}  // extern "C"

namespace {

// idx_topk and idx_topk_bf16: the scores are fp32 (16-byte aligned) or bf16
// (8-byte aligned).
int topk_checked(const void* scores, bool bf16, const int32_t* n_valid, int32_t* ids,
                 int32_t* counts, int B, int N, int K, uint32_t flags, void* ws, size_t ws_bytes,
                 void* stream) {
  if (scores == nullptr || ids == nullptr) return IDX_ERR_INVALID_ARG;
  if (!aligned(scores, bf16 ? 8 : 16) || !aligned(ids, 4) || !aligned(n_valid, 4) ||
      !aligned(counts, 4))
    return IDX_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || K < 1) return IDX_ERR_INVALID_ARG;
  if (flags & ~(IDX_SORTED | IDX_RADIX8)) return IDX_ERR_INVALID_ARG;
  if (bf16 && (flags & IDX_RADIX8) != 0) return IDX_ERR_UNSUPPORTED;
  if ((int64_t)B * N > (int64_t(1) << 40) || (int64_t)B * K > kMaxRows) return IDX_ERR_INVALID_ARG;
  const bool sorted = (flags & IDX_SORTED) != 0;
  if (sorted && K > IDX_MAX_SORTED_K) return IDX_ERR_UNSUPPORTED;
  const size_t need = idx_topk_workspace_bytes(B, N, K, flags);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 256)))
    return IDX_ERR_WORKSPACE;
  return hip_status(idxk::launch_topk(scores, n_valid, ids, counts, B, N, K, sorted,
                                      need > 0 ? ws : nullptr, stream, false, bf16,
                                      (flags & IDX_RADIX8) != 0));
}

}  // namespace

extern "C" {

int idx_topk(const float* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts, int B,
             int N, int K, uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  return topk_checked(scores, false, n_valid, ids, counts, B, N, K, flags, ws, ws_bytes, stream);
}

int idx_topk_bf16(const uint16_t* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
                  int B, int N, int K, uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  return topk_checked(scores, true, n_valid, ids, counts, B, N, K, flags, ws, ws_bytes, stream);
}

size_t idx_workspace_bytes(int B, int N_pad, int H, int K, uint32_t flags) {
  (void)H; (void)K; (void)flags;
  if (B < 1 || N_pad < 1) return 0;
  return kTicketBytes + (size_t)B * stage_stride(N_pad) * sizeof(float);
}

}  // extern "C"

namespace {

// The shape of an idx_select call (everything that a plan fixes).
int check_select_shape(int B, int H, int D, int N_pad, int page_size, int K, idx_dtype dt,
                       uint32_t flags) {
  if (B < 1 || H < 1 || D < 1 || N_pad < 1 || page_size < 1) return IDX_ERR_INVALID_ARG;
  if (dt != IDX_F32 && dt != IDX_BF16) return IDX_ERR_INVALID_ARG;
  if ((int64_t)B * N_pad > kMaxRows) return IDX_ERR_INVALID_ARG;
  if (K < 1 || (int64_t)B * K > kMaxRows) return IDX_ERR_INVALID_ARG;
  int st;
  if ((st = check_chunk_flag(flags)) != IDX_OK) return st;
  if (H > IDX_MAX_HEADS || D != IDX_HEAD_DIM) return IDX_ERR_UNSUPPORTED;
  if (B > kMaxRequests) return IDX_ERR_UNSUPPORTED;
  if ((flags & IDX_SORTED) != 0 && K > IDX_MAX_SORTED_K) return IDX_ERR_UNSUPPORTED;
  return IDX_OK;
}

// The pointers of an idx_select call.
int check_select_ptrs(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                      int32_t* counts, float* scores_out) {
  if (q == nullptr || c == nullptr || seq_len == nullptr || ids == nullptr)
    return IDX_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(c, 16) || !aligned(seq_len, 4) || !aligned(ids, 4) ||
      !aligned(counts, 4) || !aligned(scores_out, 4))
    return IDX_ERR_INVALID_ARG;
  return IDX_OK;
}

// Argument checks shared by idx_select and idx_select_noalloc (everything but
// the workspace).
int check_select_args(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                      int32_t* counts, float* scores_out, int B, int H, int D, int N_pad,
                      int page_size, int K, idx_dtype dt, uint32_t flags) {
  const int st = check_select_shape(B, H, D, N_pad, page_size, K, dt, flags);
  if (st != IDX_OK) return st;
  return check_select_ptrs(q, c, seq_len, ids, counts, scores_out);
}

// The launch of a fused select, resolved from its shape: 1024-thread
// workgroups for a few requests, 512-thread ones for many (the score order of
// more than 1024 ids is sorted by 1024-thread workgroups only), and the rows
// scored per workgroup.
struct SelectLaunch {
  int B, H, N_pad, page_size, K;
  bool bf16, sorted, wide;
  int chunk;
  bool radix8;
};

SelectLaunch resolve_select(int B, int H, int N_pad, int page_size, int K, idx_dtype dt,
                            uint32_t flags) {
  const bool sorted = (flags & IDX_SORTED) != 0;
  const bool wide = B <= kWideMaxRequests || (sorted && K > kNarrowMaxSortedK);
  const int chunk = wide ? chunk_rows_wide(B, N_pad, flags)
                         : chunk_rows(B, N_pad, flags, kScoreChunkMin, kScoreTarget);
  return SelectLaunch{B,     H,      N_pad, page_size, K, dt == IDX_BF16, sorted, wide, chunk,
                      (flags & IDX_RADIX8) != 0};
}

int launch_resolved(const SelectLaunch& L, const void* q, const void* c, const int32_t* seq_len,
                    int32_t* ids, int32_t* counts, float* scores_out, uint32_t* tickets,
                    float* stage, void* stream) {
  return hip_status(idxk::launch_select(q, c, seq_len, ids, counts, scores_out, L.B, L.H,
                                        L.N_pad, L.page_size, L.K, L.bf16, L.sorted, L.chunk,
                                        L.wide, tickets, stage, stage_stride(L.N_pad), nullptr,
                                        nullptr, 0, 0, stream, L.radix8));
}

int dispatch_select(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                    int32_t* counts, float* scores_out, int B, int H, int N_pad, int page_size,
                    int K, idx_dtype dt, uint32_t flags, uint32_t* tickets, float* stage,
                    void* stream) {
  return launch_resolved(resolve_select(B, H, N_pad, page_size, K, dt, flags), q, c, seq_len,
                         ids, counts, scores_out, tickets, stage, stream);
}

}  // namespace

extern "C" {

int idx_select(const void* q, const void* c, const int32_t* seq_len, int32_t* ids, int32_t* counts,
               float* scores_out, int B, int H, int D, int N_pad, int page_size, int K,
               idx_dtype dt, uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  const int st = check_select_args(q, c, seq_len, ids, counts, scores_out, B, H, D, N_pad,
                                   page_size, K, dt, flags);
  if (st != IDX_OK) return st;
  const size_t need = idx_workspace_bytes(B, N_pad, H, K, flags);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return IDX_ERR_WORKSPACE;
  uint32_t* tickets = static_cast<uint32_t*>(ws);
  float* stage = reinterpret_cast<float*>(static_cast<char*>(ws) + kTicketBytes);
  return dispatch_select(q, c, seq_len, ids, counts, scores_out, B, H, N_pad, page_size, K, dt,
                         flags, tickets, stage, stream);
}

int idx_select_noalloc(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                       int32_t* counts, float* scores_out, int B, int H, int D, int N_pad,
                       int page_size, int K, idx_dtype dt, uint32_t flags, void* stream) {
  const int st = check_select_args(q, c, seq_len, ids, counts, scores_out, B, H, D, N_pad,
                                   page_size, K, dt, flags);
  if (st != IDX_OK) return st;
  if (B > IDX_NOALLOC_MAX_REQUESTS) return IDX_ERR_SCRATCH;
  if (scores_out == nullptr &&
      (size_t)B * stage_stride(N_pad) * sizeof(float) > (size_t)IDX_NOALLOC_STAGE_BYTES)
    return IDX_ERR_SCRATCH;
  void* scratch = nullptr;
  if (idxk::noalloc_scratch(&scratch, stream) != 0) return IDX_ERR_HIP;
  uint32_t* tickets = static_cast<uint32_t*>(scratch);
  float* stage =
      reinterpret_cast<float*>(static_cast<char*>(scratch) + IDX_NOALLOC_TICKET_BYTES);
  return dispatch_select(q, c, seq_len, ids, counts, scores_out, B, H, N_pad, page_size, K, dt,
                         flags, tickets, stage, stream);
}

}  // extern "C"

// A resolved idx_select launch for one call signature (host memory only).
struct idx_plan {
  SelectLaunch launch;
  size_t ws_bytes;
};

extern "C" {

int idx_plan_create(idx_plan** plan, int B, int H, int D, int N_pad, int page_size, int K,
                    idx_dtype dt, uint32_t flags) {
  if (plan == nullptr) return IDX_ERR_INVALID_ARG;
  *plan = nullptr;
  const int st = check_select_shape(B, H, D, N_pad, page_size, K, dt, flags);
  if (st != IDX_OK) return st;
  idx_plan* p = new (std::nothrow) idx_plan{resolve_select(B, H, N_pad, page_size, K, dt, flags),
                                            idx_workspace_bytes(B, N_pad, H, K, flags)};
  if (p == nullptr) return IDX_ERR_NO_MEMORY;
  *plan = p;
  return IDX_OK;
}

size_t idx_plan_workspace_bytes(const idx_plan* plan) {
  return plan == nullptr ? 0 : plan->ws_bytes;
}

int idx_plan_select(const idx_plan* plan, const void* q, const void* c, const int32_t* seq_len,
                    int32_t* ids, int32_t* counts, float* scores_out, void* ws, size_t ws_bytes,
                    void* stream) {
  if (plan == nullptr) return IDX_ERR_INVALID_ARG;
  const int st = check_select_ptrs(q, c, seq_len, ids, counts, scores_out);
  if (st != IDX_OK) return st;
  if (ws == nullptr || ws_bytes < plan->ws_bytes || !aligned(ws, 256)) return IDX_ERR_WORKSPACE;
  uint32_t* tickets = static_cast<uint32_t*>(ws);
  float* stage = reinterpret_cast<float*>(static_cast<char*>(ws) + kTicketBytes);
  return launch_resolved(plan->launch, q, c, seq_len, ids, counts, scores_out, tickets, stage,
                         stream);
}

void idx_plan_destroy(idx_plan* plan) { delete plan; }

int idx_select_paged(const void* q, const void* c_pool, const int32_t* kv_indptr,
                     const int32_t* kv_indices, int32_t* ids, int32_t* counts, float* scores_out,
                     int B, int H, int D, int n_rows, int64_t n_indices, int max_pages, int K,
                     idx_dtype dt, uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  if (q == nullptr || c_pool == nullptr || kv_indptr == nullptr || ids == nullptr)
    return IDX_ERR_INVALID_ARG;
  if (kv_indices == nullptr && n_indices > 0) return IDX_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(c_pool, 16) || !aligned(kv_indptr, 4) ||
      !aligned(kv_indices, 4) || !aligned(ids, 4) || !aligned(counts, 4) ||
      !aligned(scores_out, 4))
    return IDX_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || D < 1 || n_rows < 1 || n_indices < 0 || max_pages < 1 || K < 1)
    return IDX_ERR_INVALID_ARG;
  if (dt != IDX_F32 && dt != IDX_BF16) return IDX_ERR_INVALID_ARG;
  if ((int64_t)B * max_pages > kMaxRows || (int64_t)B * K > kMaxRows) return IDX_ERR_INVALID_ARG;
  if (H > IDX_MAX_HEADS || D != IDX_HEAD_DIM) return IDX_ERR_UNSUPPORTED;
  int st;
  if ((st = check_chunk_flag(flags)) != IDX_OK) return st;
  if ((flags & IDX_RADIX8) != 0) return IDX_ERR_UNSUPPORTED;
  if (B > kMaxRequests) return IDX_ERR_UNSUPPORTED;
  const bool sorted = (flags & IDX_SORTED) != 0;
  if (sorted && K > IDX_MAX_SORTED_K) return IDX_ERR_UNSUPPORTED;
  const size_t need = idx_workspace_bytes(B, max_pages, H, K, flags);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return IDX_ERR_WORKSPACE;
  uint32_t* tickets = static_cast<uint32_t*>(ws);
  float* stage = reinterpret_cast<float*>(static_cast<char*>(ws) + kTicketBytes);
  const bool wide = B <= kWideMaxRequests || (sorted && K > kNarrowMaxSortedK);
  const int chunk = wide ? chunk_rows_wide(B, max_pages, flags)
                         : chunk_rows(B, max_pages, flags, kScoreChunkMin, kScoreTarget);
  return hip_status(idxk::launch_select(q, c_pool, nullptr, ids, counts, scores_out, B, H,
                                        max_pages, 1, K, dt == IDX_BF16, sorted, chunk, wide,
                                        tickets, stage, stage_stride(max_pages), kv_indptr,
                                        kv_indices, n_indices, n_rows, stream));
}

int idx_pool_keys(const void* k, const int32_t* seq_len, void* c, int B, int S_pad, int D,
                  int N_pad, int page_size, idx_dtype dt, void* stream) {
  if (k == nullptr || seq_len == nullptr || c == nullptr) return IDX_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(c, 16) || !aligned(seq_len, 4)) return IDX_ERR_INVALID_ARG;
  if (B < 1 || S_pad < 1 || D < 1 || N_pad < 1 || page_size < 1) return IDX_ERR_INVALID_ARG;
  if (dt != IDX_F32 && dt != IDX_BF16) return IDX_ERR_INVALID_ARG;
  if ((int64_t)B * S_pad > kMaxRows || (int64_t)B * N_pad > kMaxRows) return IDX_ERR_INVALID_ARG;
  if (D != IDX_HEAD_DIM) return IDX_ERR_UNSUPPORTED;
  return hip_status(idxk::launch_pool_keys(k, seq_len, c, B, S_pad, N_pad, page_size,
                                           dt == IDX_BF16, stream));
}

// Prompt-token calls of a few tokens over few rows run as one fused select per
// token row (each row reads its request's table; the heads are not summed
// first); longer prompts go through the matrix-core scores and a top-K.
constexpr int kPrefillFusedMaxTokens = 8;
constexpr int kPrefillFusedMaxRows = 256;
// arrival lines of the fused rows, at a fixed place so that calls of any shape
// can share one workspace; then the per-token counts, then the score staging
constexpr size_t kPrefillTicketBytes = kPrefillFusedMaxRows * size_t(128);

size_t idx_prefill_workspace_bytes(int B, int T, int N_pad, int K, uint32_t flags) {
  (void)K; (void)flags;
  if (B < 1 || T < 1 || N_pad < 1) return 0;
  const size_t rows = (size_t)B * T;
  return kPrefillTicketBytes + round_up(rows * sizeof(int32_t), 256) +
         rows * stage_stride(N_pad) * sizeof(float);
}

int idx_select_prefill(const void* q, const void* c, const int32_t* pos0, int32_t* ids,
                       int32_t* counts, float* scores_out, int B, int T, int H, int D, int N_pad,
                       int page_size, int K, idx_dtype dt, uint32_t flags, void* ws,
                       size_t ws_bytes, void* stream) {
  if (q == nullptr || c == nullptr || pos0 == nullptr || ids == nullptr)
    return IDX_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(c, 16) || !aligned(pos0, 4) || !aligned(ids, 4) ||
      !aligned(counts, 4) || !aligned(scores_out, 16))
    return IDX_ERR_INVALID_ARG;
  if (B < 1 || T < 1 || H < 1 || D < 1 || N_pad < 1 || page_size < 1 || K < 1)
    return IDX_ERR_INVALID_ARG;
  if (dt != IDX_F32 && dt != IDX_BF16) return IDX_ERR_INVALID_ARG;
  if (flags & ~(IDX_SORTED | IDX_RADIX8)) return IDX_ERR_INVALID_ARG;
  if ((flags & IDX_RADIX8) != 0) return IDX_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)B * T;
  if (rows > kMaxRows || rows * N_pad > (int64_t(1) << 40) || rows * K > kMaxRows ||
      (int64_t)B * N_pad > kMaxRows)
    return IDX_ERR_INVALID_ARG;
  // a few tokens over few rows: one fused select over the token rows
  const bool fused =
      T <= kPrefillFusedMaxTokens && rows <= kPrefillFusedMaxRows && rows * N_pad <= kMaxRows;
  if ((dt != IDX_BF16 && !fused) || H > IDX_MAX_HEADS || D != IDX_HEAD_DIM)
    return IDX_ERR_UNSUPPORTED;
  const bool sorted = (flags & IDX_SORTED) != 0;
  if (sorted && K > IDX_MAX_SORTED_K) return IDX_ERR_UNSUPPORTED;
  const size_t need = idx_prefill_workspace_bytes(B, T, N_pad, K, flags);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return IDX_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  int32_t* n_valid = reinterpret_cast<int32_t*>(w + kPrefillTicketBytes);
  float* stage = reinterpret_cast<float*>(w + kPrefillTicketBytes +
                                          round_up((size_t)rows * sizeof(int32_t), 256));
  if (fused) {
    const SelectLaunch L = resolve_select((int)rows, H, N_pad, page_size, K, dt,
                                          flags & IDX_SORTED);
    return hip_status(idxk::launch_select_tokens(
        q, c, pos0, ids, counts, scores_out, (int)rows, T, H, N_pad, page_size, K, L.bf16,
        sorted, L.chunk, L.wide, reinterpret_cast<uint32_t*>(w), stage, stage_stride(N_pad),
        stream));
  }
  float* scores = scores_out;
  int64_t stride = N_pad;
  if (scores == nullptr) {  // staged in the workspace, rows 16-byte aligned
    scores = stage;
    stride = stage_stride(N_pad);
  }
  // staged scores are read only up to each token's count: no -inf fill
  int e = idxk::launch_prefill_score(q, c, pos0, scores, stride, n_valid, B, T, H, N_pad,
                                     page_size, scores_out != nullptr, stream);
  if (e != 0) return IDX_ERR_HIP;
  return hip_status(idxk::launch_topk(scores, n_valid, ids, counts, (int)rows, (int)stride, K,
                                      sorted, nullptr, stream, /*dot_scores=*/true));
}

// -|c|^2/2 per centroid, padded with -inf to a multiple of 128 (a whole number of
// centroid tiles)
size_t idx_assign_workspace_bytes(int C, int D) {
  (void)D;
  if (C < 1) return 0;
  return round_up(round_up((size_t)C, 128) * sizeof(float), 256);
}

int idx_assign(const void* x, const void* c, int32_t* assign, float* best, int64_t N, int C, int D,
               idx_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  if (x == nullptr || c == nullptr || assign == nullptr) return IDX_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(c, 16) || !aligned(assign, 4) || !aligned(best, 4))
    return IDX_ERR_INVALID_ARG;
  if (N < 1 || N > kMaxRows || C < 1 || C > 65536 || D < 1) return IDX_ERR_INVALID_ARG;
  if (dt != IDX_F32 && dt != IDX_BF16) return IDX_ERR_INVALID_ARG;
  if (D != IDX_HEAD_DIM || dt != IDX_BF16) return IDX_ERR_UNSUPPORTED;
  const size_t need = idx_assign_workspace_bytes(C, D);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 16)) return IDX_ERR_WORKSPACE;
  return hip_status(idxk::launch_assign(x, c, assign, best, N, C, static_cast<float*>(ws), stream));
}

}  // extern "C"
