/*
 * idx.h -- C ABI of the block-scoring + top-K indexer for AMD MI355X (gfx950).
 *
 * The indexer of a block-sparse attention layer scores every block (page) of a
 * request's KV cache by comparing the block's centroid with the request's query
 * heads, masks blocks past the request's length, and keeps the K best blocks.
 * Sources (web pages; cited by title and section):
 *   [CS]  "Iterate Centroids Score" -- the centroid-scoring kernel of a
 *         block-sparse-attention indexer: query rows against a table of block
 *         centroids, scoring each request's candidate pages for the top-K stage;
 *         the scorer writes into a caller-provided output buffer.
 *   [TK]  "Iterate Topk" -- the top-K kernel: per-segment scores in, top-K
 *         indices out; an 8-bit radix seed design.
 *   [QS]  "Round 18 Track C: qsa_topk2 Register-Cached Keys & Barrier Reduction
 *         + qsa_score Query Hoisting & Unrolling" -- section 1 (score kernel
 *         with query heads hoisted into registers; 4-pass 8-bit radix select
 *         over unsigned order keys with a 256-bin histogram), section 2 (ids
 *         compared bitwise, ties and signed zeros included).
 *   [KM]  "Export Cake KMeans plan-runtime suite" -- Summary: the k-means
 *         assignment call on bf16 points and centroids, norms fused into it.
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller; arrays are
 *     dense, row-major, C-contiguous. The library never allocates, frees,
 *     copies between host and device, or synchronises: each call validates its
 *     arguments on the host, enqueues kernels on `stream` and returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). The
 *     kernels run on the device that is current on the calling thread.
 *   - On a validation failure a call returns a negative status and enqueues
 *     nothing, so no output byte is written. IDX_ERR_HIP reports a failed
 *     launch; faults inside a kernel surface at the caller's next synchronise.
 *   - Pointers read with 16-byte vector loads must be 16-byte aligned (stated
 *     per argument). Integer arrays must be 4-byte aligned.
 *   - bf16 data is passed as raw 16-bit patterns (uint16_t storage).
 *   - Workspace: a caller-owned device buffer of at least the size the
 *     matching *_workspace_bytes() returns. A workspace must be zero-filled
 *     once before its first use: it holds arrival counters, which every call
 *     returns to zero, and scratch, which calls overwrite before reading. One
 *     workspace may serve any sequence of calls on one stream whose sizes come
 *     from the same *_workspace_bytes() function (idx_select, idx_select_paged
 *     and plans share one layout, idx_topk and idx_topk_bf16 another,
 *     idx_select_prefill a third; the layouts differ, so a buffer used under
 *     one must be zero-filled again
 *     before it serves another). Calls that may overlap (other streams) need
 *     distinct workspaces.
 */
#ifndef IDX_H
#define IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { IDX_F32 = 0, IDX_BF16 = 1 } idx_dtype;

enum {
  IDX_OK = 0,
  IDX_ERR_INVALID_ARG = -1, /* null / misaligned pointer, size out of range   */
  IDX_ERR_UNSUPPORTED = -2, /* legal but not built: head_dim != 128, K > 4096 sorted */
  IDX_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required      */
  IDX_ERR_HIP = -4,         /* the HIP runtime refused the launch              */
  IDX_ERR_SCRATCH = -5,     /* idx_select_noalloc: the shape needs more than its
                               static scratch holds                              */
  IDX_ERR_NO_MEMORY = -6    /* idx_plan_create: no host memory for the plan      */
};

/* flags */
#define IDX_SORTED 0x1u /* ids ordered by (score descending, id ascending);
                           default: ascending block id                        */
/* IDX_RADIX8: find the threshold with four 8-bit radix passes and no
 * linear-bin pass: the radix of the proposal seed in [TK] section 6 and of the
 * four-pass select loop in [QS] section 1 Target 1. The outputs are the same
 * as without it (same selection rule, same order); it exists to measure that
 * design against the library's own select (a linear-bin pass, then 11 + 11 +
 * 10-bit digits). Accepted by idx_topk (fp32 scores), idx_select,
 * idx_select_noalloc and idx_plan_create; idx_topk_bf16, idx_select_paged and
 * idx_select_prefill return IDX_ERR_UNSUPPORTED for it. */
#define IDX_RADIX8 0x2u
/* Bits 8..12 of `flags` optionally fix log2 of the number of blocks scored by
 * one workgroup (4..14); 0 lets the library choose. Results do not depend on it. */
#define IDX_CHUNK_SHIFT 8
#define IDX_CHUNK_MASK (0x1Fu << IDX_CHUNK_SHIFT)
#define IDX_CHUNK_LOG2(l) ((uint32_t)(l) << IDX_CHUNK_SHIFT)

/* Limits of this build. */
#define IDX_HEAD_DIM 128     /* D: the only head dimension compiled            */
#define IDX_MAX_HEADS 64     /* H                                              */
#define IDX_MAX_SORTED_K 4096
#define IDX_MAX_REQUESTS 16384 /* B of one idx_select call */

/*
 * Number of blocks of request b that hold tokens, used by every scoring call:
 *     n_valid[b] = min(N_pad, ceil(seq_len[b] / page_size)).
 * The partly filled last page is a candidate ([QS] section 1 counts a block for
 * every started group of tokens: 8193 tokens in 4-token blocks are 2049 blocks).
 */

/*
 * idx_score -- block scores ([CS]; [QS] section 1, Target 2).
 *   scores[b,n] = sum_{h<H} sum_{d<D} q[b,h,d] * c[b,n,d]   for n <  n_valid[b]
 *   scores[b,n] = -inf (bit pattern 0xFF800000)             for n >= n_valid[b]
 * accumulated in fp32. Centroid rows at or past n_valid[b] are never read, so
 * their contents are irrelevant (they may hold NaN).
 *   q        [B,H,D]      dtype dt, 16-byte aligned
 *   c        [B,N_pad,D]  dtype dt, 16-byte aligned
 *   seq_len  [B] int32    tokens per request, 0 <= seq_len[b] <= N_pad*page_size
 *                         (values are read on the device; an out-of-range value
 *                         is clamped to that range, not reported)
 *   scores   [B,N_pad] float32 output
 * B >= 1, 1 <= H <= IDX_MAX_HEADS, D == IDX_HEAD_DIM, N_pad >= 1, page_size >= 1.
 */
int idx_score(const void* q, const void* c, const int32_t* seq_len, float* scores,
              int B, int H, int D, int N_pad, int page_size, idx_dtype dt, void* stream);

/*
 * idx_topk -- row-wise top-K of given scores ([TK]; [QS] section 1 Target 1).
 *   For each row b, candidates are the entries n < n_valid[b] (all N entries if
 *   n_valid is NULL) whose score is not -inf. The selected set is the m =
 *   min(K, #candidates) candidates with the largest scores; equal scores
 *   (-0.0 == +0.0) go to the lower index. NaN scores are outside the contract.
 *   ids[b, 0..m-1] receive the selected indices, in ascending index order by
 *   default or by (score desc, index asc) with IDX_SORTED; ids[b, m..K-1] = -1.
 *   counts[b] = m when counts is not NULL.
 *   scores  [B,N] float32 (16-byte aligned)      n_valid [B] int32 or NULL
 *   ids     [B,K] int32 output                    counts  [B] int32 output or NULL
 * B >= 1, N >= 1, K >= 1 (K <= IDX_MAX_SORTED_K with IDX_SORTED).
 * ws / ws_bytes: workspace of at least idx_topk_workspace_bytes() bytes
 * (256-byte aligned; may be NULL when that is 0). It is nonzero when rows are
 * few and long: each row is then cut into segments selected by several
 * workgroups and merged by the last to finish (arrival counters and segment
 * candidates live in the workspace). It must be zero-filled before first use;
 * every call returns its arrival counters to zero (the candidates are scratch),
 * so it may serve any later call that fits it. Calls that may overlap (other
 * streams) need distinct workspaces.
 */
size_t idx_topk_workspace_bytes(int B, int N, int K, uint32_t flags);
int idx_topk(const float* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
             int B, int N, int K, uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * idx_topk_bf16 -- idx_topk over bf16 scores ("Iterate Topk", section 6: a
 * 16-bit radix for bf16 scores, whose fp32 patterns have a zero low half).
 * The same selection rule, outputs, workspace (idx_topk_workspace_bytes) and
 * errors as idx_topk; scores compare as the exact fp32 values of the bf16
 * patterns (-0.0 == +0.0, -inf never selected). Half the bytes of fp32 scores
 * are read, and a key is resolved by at most two radix digits (11 + 5 bits).
 *   scores [B,N] bf16 as raw 16-bit patterns, 8-byte aligned (rows of N % 4 != 0
 *          are read entry by entry)
 */
int idx_topk_bf16(const uint16_t* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
                  int B, int N, int K, uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * idx_select -- fused score + mask + top-K ([CS] scorer feeding the top-K
 * stage; [QS] section 1, "combined" = score then select). Same inputs as
 * idx_score and the same selection rule as idx_topk applied to the scores that
 * idx_score would produce; the ids do not depend on whether scores_out is given.
 *   ids        [B,K] int32 output; counts [B] int32 output or NULL
 *   scores_out [B,N_pad] float32 output or NULL: when given it receives exactly
 *              what idx_score writes (for parity checks and debugging)
 * K >= 1 (K <= IDX_MAX_SORTED_K with IDX_SORTED).
 * B <= IDX_MAX_REQUESTS.
 * ws / ws_bytes: workspace of at least idx_workspace_bytes(B, N_pad, H, K, flags)
 * bytes, zero-filled before first use: 2 MiB of per-request arrival counters
 * (one 128-byte line each), which every call returns to zero, and staging for
 * the scores (scratch), so one workspace may serve calls of any shape that fits
 * it.
 */
size_t idx_workspace_bytes(int B, int N_pad, int H, int K, uint32_t flags);
int idx_select(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
               int32_t* counts, float* scores_out, int B, int H, int D, int N_pad,
               int page_size, int K, idx_dtype dt, uint32_t flags, void* ws,
               size_t ws_bytes, void* stream);

/*
 * idx_select_noalloc -- idx_select with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, results and errors as
 * idx_select (the ids are identical), minus ws / ws_bytes.
 *   Scratch: the arrival counters and the score staging live in one static
 *   device array of IDX_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held until the
 *   process ends: arrival lines for up to IDX_NOALLOC_MAX_REQUESTS requests,
 *   then IDX_NOALLOC_STAGE_BYTES of staging. The first call on a device looks
 *   up that device's copy of the array and clears its arrival lines (a fill
 *   kernel on `stream`); every call returns them to zero.
 *   Limits: B <= IDX_NOALLOC_MAX_REQUESTS and, when scores_out is NULL,
 *   B * round_up(N_pad, 4) * 4 <= IDX_NOALLOC_STAGE_BYTES; beyond them the call
 *   returns IDX_ERR_SCRATCH and enqueues nothing.
 *   The call makes no hipMalloc / hipFree and no other allocating call.
 *   All calls on one GPU share its array: calls that may overlap on one GPU
 *   (other streams, or other threads) race and must not be issued.
 */
#define IDX_NOALLOC_SCRATCH_BYTES (16u << 20)
#define IDX_NOALLOC_MAX_REQUESTS 4096
#define IDX_NOALLOC_TICKET_BYTES (IDX_NOALLOC_MAX_REQUESTS * 128u)
#define IDX_NOALLOC_STAGE_BYTES (IDX_NOALLOC_SCRATCH_BYTES - IDX_NOALLOC_TICKET_BYTES)
int idx_select_noalloc(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                       int32_t* counts, float* scores_out, int B, int H, int D, int N_pad,
                       int page_size, int K, idx_dtype dt, uint32_t flags, void* stream);

/*
 * Plans -- a resolved idx_select launch for one call signature ("Export Cake
 * KMeans plan-runtime suite", Summary: a per-signature launch plan resolved
 * once, then called many times; the plan's calls may be captured into a HIP
 * graph, which the library leaves to the caller's stream capture).
 *   idx_plan_create validates the shape (B, H, D, N_pad, page_size, K, dt,
 *   flags: the rules and errors of idx_select) and resolves the launch (kernel
 *   instance, workgroup size, blocks scored per workgroup) into a plan held in
 *   host memory, owned by the caller until idx_plan_destroy; it makes no HIP
 *   call. *plan is NULL on failure (IDX_ERR_NO_MEMORY: host allocation failed).
 *   idx_plan_workspace_bytes: the workspace its calls need (that of idx_select).
 *   idx_plan_select: idx_select with the plan's shape. Only the pointers, their
 *   alignment and the workspace are checked; the ids, counts and scores are
 *   those idx_select writes. A plan is read-only after creation and may be used
 *   from several threads; calls that may overlap need distinct workspaces.
 *   idx_plan_destroy(NULL) is a no-op.
 */
typedef struct idx_plan idx_plan;
int idx_plan_create(idx_plan** plan, int B, int H, int D, int N_pad, int page_size, int K,
                    idx_dtype dt, uint32_t flags);
size_t idx_plan_workspace_bytes(const idx_plan* plan);
int idx_plan_select(const idx_plan* plan, const void* q, const void* c, const int32_t* seq_len,
                    int32_t* ids, int32_t* counts, float* scores_out, void* ws, size_t ws_bytes,
                    void* stream);
void idx_plan_destroy(idx_plan* plan);

/*
 * idx_select_paged -- idx_select over a paged centroid pool ([CS] submission
 * contract and benchmark protocol: the scorer reads each request's pages
 * through its context (page lists cut into work tiles) from a pool of block
 * centroids, n_blocks = 16384 in the benchmark sweep).
 *   c_pool     [n_rows, D] centroids (16-byte aligned), shared by all requests
 *   kv_indptr  [B+1] int32 device array; request b's score slots are
 *              i = 0 .. kv_indptr[b+1] - kv_indptr[b] - 1, slot i reading the
 *              pool row kv_indices[kv_indptr[b] + i]
 *   kv_indices [n_indices] int32 device array of pool rows
 *   s[b,i] = sum_h q[b,h,:] . c_pool[kv_indices[kv_indptr[b] + i], :]
 * A request's slot count is clamped to [0, max_pages]. A slot whose list entry
 * does not exist (position outside [0, n_indices)) or names a row outside
 * [0, n_rows) is not a candidate: it scores -inf and nothing is read for it.
 * ids, counts and the selection rule are those of idx_select, with slot
 * positions i as the ids (the caller maps them to pool rows through its lists).
 *   scores_out [B, max_pages] float32 output or NULL (-inf past a request's slots)
 * Workspace: idx_workspace_bytes(B, max_pages, H, K, flags), with the same
 * zero-fill rule as idx_select.
 * B >= 1, n_rows >= 1, n_indices >= 0, max_pages >= 1, K >= 1; other limits as
 * idx_select.
 */
int idx_select_paged(const void* q, const void* c_pool, const int32_t* kv_indptr,
                     const int32_t* kv_indices, int32_t* ids, int32_t* counts, float* scores_out,
                     int B, int H, int D, int n_rows, int64_t n_indices, int max_pages, int K,
                     idx_dtype dt, uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * idx_pool_keys -- block centroids from the keys ("Round 15 Track C Audit",
 * section 2: the pooled keys are a stage of the indexer checked for parity;
 * [CS]: the scorer reads one centroid per block). Reading: a block's pooled
 * key is the mean of the keys of its tokens.
 *   k       [B,S_pad,D] keys (16-byte aligned), token s of request b in row s
 *   seq_len [B] int32 device array: request b holds tokens 0 .. seq_len[b]-1
 *           (clamped to [0, S_pad])
 *   c       [B,N_pad,D] output, same dtype as k (16-byte aligned)
 *   c[b,n,:] = mean of k[b,s,:] over s in [n*page_size, min((n+1)*page_size,
 *              seq_len[b])), for n < min(N_pad, ceil(seq_len[b]/page_size));
 * rows past that count are not written. Sums in fp32 in token order, then a
 * correctly rounded division; bf16 output rounds the fp32 mean to nearest even.
 * D == IDX_HEAD_DIM, dt IDX_F32 or IDX_BF16. No workspace.
 */
int idx_pool_keys(const void* k, const int32_t* seq_len, void* c, int B, int S_pad, int D,
                  int N_pad, int page_size, idx_dtype dt, void* stream);

/*
 * idx_select_prefill -- per-token scores and top-K for T prompt tokens per
 * request ("Round 15 Track C Audit", section 1 Target 1: the prompt path
 * scores tiles of query tokens against the block keys with a matrix product,
 * every token before its top-K; "Round 18 Track C", section 3: the score
 * stage grows with the number of query tokens).
 *   q    [B,T,H,D] (16-byte aligned): token t of request b sits at position
 *        pos0[b] + t
 *   c    [B,N_pad,D] (16-byte aligned): the request's block centroids
 *   pos0 [B] int32 device array (negative values count as 0)
 * Token t sees the blocks n < n_valid = min(N_pad, ceil((pos0[b] + t + 1) /
 * page_size)) (the blocks up to the one holding itself), and
 *   s[b,t,n] = sum_h q[b,t,h,:] . c[b,n,:] for those blocks, -inf past them.
 * Each (b, t) row then gets the selection of idx_topk:
 *   ids        [B,T,K] int32 output;  counts [B,T] int32 output or NULL
 *   scores_out [B,T,N_pad] float32 output or NULL (16-byte aligned)
 * Calls with T <= 8, B*T <= 256 and B*T*N_pad < 2^31 score each token row as
 * idx_select does (one fused launch; products and head sums in fp32), with
 * fp32 or bf16 inputs. Longer prompts (bf16 only) sum the heads per token in
 * fp32 and split the sum into two bf16 parts for the matrix cores (the
 * dropped remainder is below 2^-16 of each summed value), products
 * accumulated in fp32; the top-K follows in a second launch.
 * dt == IDX_BF16 (or IDX_F32 on the short route), D == IDX_HEAD_DIM,
 * H <= IDX_MAX_HEADS, K >= 1 (K <= IDX_MAX_SORTED_K with IDX_SORTED).
 * ws / ws_bytes: at least idx_prefill_workspace_bytes(B, T, N_pad, K, flags)
 * bytes, zero-filled before first use: arrival lines (left zeroed by each
 * call), then per-token block counts and score staging.
 */
size_t idx_prefill_workspace_bytes(int B, int T, int N_pad, int K, uint32_t flags);
int idx_select_prefill(const void* q, const void* c, const int32_t* pos0, int32_t* ids,
                       int32_t* counts, float* scores_out, int B, int T, int H, int D, int N_pad,
                       int page_size, int K, idx_dtype dt, uint32_t flags, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * idx_assign -- nearest-centroid k-means assignment ([KM] Summary): the select
 * step with K = 1 over a dense score matrix.
 *   assign[i] = argmax_j ( 2 * x[i,:].c[j,:] - |c[j,:]|^2 ), ties to the lower j,
 * products of bf16 values accumulated in fp32 on the matrix cores. The centroid
 * norms are computed inside the call (the workspace holds them).
 *   x      [N,D] bf16 (16-byte aligned)    c [C,D] bf16 (16-byte aligned)
 *   assign [N] int32 output
 *   best   [N] float32 output or NULL: the winning value of dot(x,c) - |c|^2/2
 *          (half the score above), for parity checks
 * N >= 1, 1 <= C <= 65536, D == IDX_HEAD_DIM, dt == IDX_BF16.
 */
size_t idx_assign_workspace_bytes(int C, int D);
int idx_assign(const void* x, const void* c, int32_t* assign, float* best, int64_t N,
               int C, int D, idx_dtype dt, void* ws, size_t ws_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* idx_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H */
