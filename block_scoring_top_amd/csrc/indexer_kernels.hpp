// Kernels of the indexer path's selects (top-K of given rows, fused score +
// top-K) and their launch templates, shared by the two translation units that
// instantiate them: indexer.hip (the library's selects) and
// indexer_radix8.hip (the same launches with four 8-bit radix passes).
#pragma once

#include <hip/hip_runtime.h>

#include "launch.h"
#include "score.hpp"
#include "select.hpp"

namespace idxk {

// One arrival counter per request, each on its own 128-byte line: the atomics of
// one line are serialised where they are performed, so requests must not share.
constexpr int kTicketStride = 32;
// arrival lines of B rows, rounded to 256 bytes
inline size_t topk_ticket_bytes(int B) {
  return ((size_t)B * kTicketStride * 4 + 255) / 256 * 256;
}
// Rows are cut into segments only when there are at most kTopkSplitMaxRows of
// them (topk_segments). Their arrival counters take the workspace's first
// topk_ticket_bytes(kTopkSplitMaxRows) bytes whatever the row count, and the
// candidates follow: a later call with more rows then never finds an earlier
// call's candidates where its own counters lie.
constexpr int kTopkSplitMaxRows = 256;
inline size_t topk_cand_offset() { return topk_ticket_bytes(kTopkSplitMaxRows); }
constexpr int kTopkNT = 1024;   // top-K workgroup: 16 waves
constexpr int kTopkSlots = 8;   // register tile: 1024*8*4 = 32768 keys
constexpr int kSplitRep = 4;    // histogram copies of the split top-K merges' linear passes

// ---- idx_topk ----------------------------------------------------------------------------
// One workgroup of NT threads per row; rows longer than NT*SLOTS*4 keys are
// streamed through the register tile. ADAPTIVE (rows of any distribution):
// the linear pass chooses its bins per row; otherwise value bins (dot-product
// scores).
// BF16IN: the scores are bf16 (raw 16-bit patterns), selected with 16-bit keys.
// R8: 8-bit radix digits, no linear-bin pass (fp32 rows; the same results).
template <bool BF16IN>
__device__ __forceinline__ const void* score_row(const void* scores, size_t off) {
  return BF16IN ? static_cast<const void*>(static_cast<const uint16_t*>(scores) + off)
                : static_cast<const void*>(static_cast<const float*>(scores) + off);
}

template <bool SORTED, int NT, int SLOTS, bool ADAPTIVE = true, bool BF16IN = false,
          bool R8 = false>
__global__ __launch_bounds__(NT) void topk_kernel(const void* __restrict__ scores,
                                                  const int32_t* __restrict__ n_valid,
                                                  int32_t* __restrict__ ids,
                                                  int32_t* __restrict__ counts, int N, int K) {
  __shared__ SelectSmem<NT, SLOTS> sm;
  extern __shared__ uint64_t sort_lds[];  // sort_lds_bytes(K) when SORTED
  const int b = blockIdx.x;
  int n = N;
  if (n_valid != nullptr) n = max(0, min(n_valid[b], N));
  select_row<NT, SLOTS, SORTED, false, false, IdsOut, ADAPTIVE, BF16IN, BF16IN, R8>(
      score_row<BF16IN>(scores, (size_t)b * N), n, N, K, IdsOut{ids + (size_t)b * K},
      counts ? counts + b : nullptr, sm, sort_lds);
}

// Long rows, few of them: each row is cut into S segments of L entries (L a
// multiple of 4), one workgroup per segment. A segment's workgroup selects its
// own top-K and hands them over as (score, index) candidates; the last of the
// row's segments to arrive selects the row's top-K from the S*K candidates.
// The global top-K is inside the union of the segments' top-Ks (the same total
// order on each side), and candidates are laid out in segment order, each
// segment's in ascending index order, so candidate order is index order and
// the lower-index tie-break carries over.
// Workspace per row: an arrival line, and cstride >= S*K candidate scores and
// ids (cstride a multiple of 4). MS: key slots of the merge, 2 when the S*K
// candidates fit one 2-slot tile, else 8, chosen on the host for score-ordered
// merges (one merge per kernel keeps the registers of the 8-slot sort
// unspilled); 0: chosen per call inside one kernel (index-order merges).
template <bool SORTED, int MS, bool BF16IN = false, bool R8 = false>
__global__ __launch_bounds__(kTopkNT) void topk_split_kernel(
    const void* __restrict__ scores, const int32_t* __restrict__ n_valid,
    int32_t* __restrict__ ids, int32_t* __restrict__ counts, int N, int K, int S, int L,
    uint32_t* tickets, float* cand_score, int32_t* cand_id, int cstride) {
  // segments and index-order merges of at most 8192 keys use 2 key slots (one
  // register tile; the merge loads the candidate ids beside the scores), longer
  // ones 8
  __shared__ union {
    SelectSmem<kTopkNT, kTopkSlots> s8;
    SelectSmem<kTopkNT, 2> s2;
  } smu;
  SelectSmem<kTopkNT, kTopkSlots>& sm = smu.s8;
  // The merges count their linear pass into kSplitRep histogram copies:
  // quantised rows hand over candidates of two or three values, which put most
  // lanes of a wave on the LDS words of two or three bins. (With the sort
  // buffer of a score-ordered merge the workgroup takes 67-83 KB of LDS.)
  constexpr int HR = R8 ? 1 : kSplitRep;
  __shared__ __attribute__((aligned(16))) uint32_t s_rep[HR > 1 ? HR * kRepStride : 4];
  __shared__ int s_last;
  extern __shared__ uint64_t sort_lds[];  // sort_lds_bytes(K) when SORTED
  const int b = blockIdx.x / S;
  const int seg = blockIdx.x - b * S;
  int n = N;
  if (n_valid != nullptr) n = max(0, min(n_valid[b], N));
  const int lo = seg * L;
  const int seg_n = max(0, min(lo + L, n) - lo);
  float* rs = cand_score + (size_t)b * cstride;
  int32_t* ri = cand_id + (size_t)b * cstride;
  const CandOut cand{rs + (size_t)seg * K, ri + (size_t)seg * K, lo};
  if (L <= kTopkNT * 2 * 4 && K <= kBins) {
    // The candidates are staged in the histogram LDS, free once the
    // threshold is known, and then written out contiguously: whole lines,
    // where the emit's own stores would cover only its taken lanes.
    float* st_s = reinterpret_cast<float*>(smu.s2.hist[0]);
    int32_t* st_i = reinterpret_cast<int32_t*>(smu.s2.hist[1]);
    select_row<kTopkNT, 2, false, false, false, StagedCandOut, true, BF16IN, BF16IN, R8>(
        score_row<BF16IN>(scores, (size_t)b * N + lo), seg_n, max(N - lo, 0), K,
        StagedCandOut{st_s, st_i, lo}, nullptr, smu.s2, sort_lds);
    __syncthreads();
    for (int k = threadIdx.x; k < K; k += kTopkNT) {
      __hip_atomic_store(cand.score + k, st_s[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(cand.id + k, st_i[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (L <= kTopkNT * 2 * 4) {
    select_row<kTopkNT, 2, false, false, false, CandOut, true, BF16IN, BF16IN, R8>(
        score_row<BF16IN>(scores, (size_t)b * N + lo), seg_n, max(N - lo, 0), K, cand, nullptr,
        smu.s2, sort_lds);
  } else {
    select_row<kTopkNT, kTopkSlots, false, false, false, CandOut, true, BF16IN, BF16IN, R8>(
        score_row<BF16IN>(scores, (size_t)b * N + lo), seg_n, max(N - lo, 0), K, cand, nullptr,
        sm, sort_lds);
  }
  // hand-off: as in the fused select (agent-scope stores, all memory operations
  // of the workgroup complete, one relaxed agent-scope ticket)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&tickets[(size_t)b * kTicketStride], 1u,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == (uint32_t)(S - 1));
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0)
    __hip_atomic_store(&tickets[(size_t)b * kTicketStride], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  const MappedIdsOut out{ids + (size_t)b * K, ri};
  // the candidates of bf16 rows are bf16 values (in fp32): 16-bit keys
  if (MS == 2 || (MS == 0 && S * K <= kTopkNT * 2 * 4))
    select_row<kTopkNT, 2, SORTED, true, false, MappedIdsOut, true, false, BF16IN, R8, HR>(
        rs, S * K, cstride, K, out, counts ? counts + b : nullptr, smu.s2, sort_lds, s_rep);
  else
    select_row<kTopkNT, kTopkSlots, SORTED, true, false, MappedIdsOut, true, false, BF16IN, R8,
               HR>(rs, S * K, cstride, K, out, counts ? counts + b : nullptr, sm, sort_lds, s_rep);
}

// ---- idx_select: score chunks, the last-arriving workgroup of a request selects ---------
constexpr int kPageStage = 256;  // page-list entries a paged chunk stages in LDS (default chunks <= 256)
// NT threads per workgroup, select tile NT*SLOTS*4 keys.
// PAGED: request b's score slots are its page list indices[indptr[b] ..
// indptr[b+1]) (at most N_pad of them) into a shared pool of n_rows centroids;
// otherwise its N_pad rows of c, the first n_valid(seq_len[b]) of them scored.
// tokens > 0 (query tokens of a prompt): row b is token b % tokens of request
// b / tokens, whose table it scores; seq_len then holds each request's first
// position pos0, and the token at pos0 + t sees the blocks n < n_valid(pos0 +
// t + 1) (negative pos0 counts as 0).
// R8: 8-bit radix digits, no linear-bin pass (dense tables; the same results).
template <bool BF16, bool SORTED, int NT, int SLOTS, bool BLOCKED, bool PAGED, bool R8 = false>
__global__ __launch_bounds__(NT) void select_fused_kernel(
    const void* __restrict__ q, const void* __restrict__ c, const int32_t* __restrict__ seq_len,
    int32_t* __restrict__ ids, int32_t* __restrict__ counts, float* __restrict__ scores_out,
    int H, int N_pad, int page_size, int K, int chunk, int nchunk, uint32_t* tickets,
    float* stage, int stage_stride, const int32_t* __restrict__ indptr,
    const int32_t* __restrict__ indices, int64_t n_indices, int n_rows, int tokens) {
  __shared__ SelectSmem<NT, SLOTS> sm;
  __shared__ int s_last;
  __shared__ int32_t s_pages[PAGED ? kPageStage : 1];
  extern __shared__ uint64_t sort_lds[];  // sort_lds_bytes(K) when SORTED
  const int b = blockIdx.x / nchunk;
  const int ch = blockIdx.x - b * nchunk;
  // the first query heads are requested with the request length, and summed
  // while the first centroid rows are in flight
  QHeads<BF16> qh;
  qh.issue(q, b, H, 0, threadIdx.x & 15, (threadIdx.x >> 4) & 3);
  int nv;
  int64_t pbase = 0, avail = 0;
  int tb = b;  // the centroid table this row scores
  if constexpr (PAGED) {
    const int lo = indptr[b], hi = indptr[b + 1];
    nv = min(max(hi - lo, 0), N_pad);
    pbase = lo;
    avail = (lo >= 0 && (int64_t)lo < n_indices) ? n_indices - lo : 0;
  } else if (tokens > 0) {
    tb = b / tokens;
    const int64_t seen = (int64_t)max(seq_len[tb], 0) + (b - tb * tokens) + 1;
    const int64_t nb = (seen + page_size - 1) / page_size;
    nv = (int)(nb < N_pad ? nb : N_pad);
  } else {
    nv = n_valid_blocks(seq_len[b], page_size, N_pad);
  }
  const int n_part = max(1, (nv + chunk - 1) / chunk);
  const int r0 = ch * chunk;
  const int r_end = min(r0 + chunk, N_pad);
  if (ch >= n_part) {  // nothing to score here
    if (scores_out != nullptr) fill_neg_inf(scores_out + (size_t)b * N_pad, r0, r_end);
    return;
  }
  float* row = scores_out != nullptr ? scores_out + (size_t)b * N_pad
                                     : stage + (size_t)b * stage_stride;
  const int row_cap = scores_out != nullptr ? N_pad : stage_stride;
  const int r1 = min(r_end, nv);
  if (r1 > r0) {
    constexpr int U = NT >= 1024 ? 2 : 4;
    if constexpr (PAGED) {
      // The chunk's page-list entries, validated, are staged in LDS (one round
      // trip per kPageStage of them), so that a row load waits on an LDS read
      // only: a list load would also wait for every row load issued before it.
      const PagedRows pages{indices + (avail > 0 ? pbase : 0), avail, n_rows};
      for (int s0 = r0; s0 < r1; s0 += kPageStage) {
        const int s1 = min(s0 + kPageStage, r1);
        if (s0 > r0) __syncthreads();  // the previous piece's entries are read
        for (int i = threadIdx.x; i < s1 - s0; i += NT) s_pages[i] = pages(s0 + i);
        __syncthreads();
        score_rows<BF16, NT, true, U>(c, StagedRows{s_pages, s0}, qh, q, b, H, s0, s1, row);
      }
    } else
      score_rows<BF16, NT, true, U>(table_of<BF16>(c, (size_t)tb * N_pad), DenseRows{}, qh, q, b,
                                    H, r0, r1, row);
  }
  if (scores_out != nullptr) fill_neg_inf(row, max(r0, nv), r_end);

  // Hand-off without cache-wide fences: the scores above were written with
  // agent-scope (write-through) stores; waiting for every outstanding memory
  // operation of this wave, then a workgroup barrier, means all of them have
  // completed before the ticket is taken. The last of the request's n_part
  // chunks to take a ticket reads the row with agent-scope loads (the staged
  // row is scratch: every call writes the entries it reads).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&tickets[(size_t)b * kTicketStride], 1u,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == (uint32_t)(n_part - 1));
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0)  // ready for the next call on this workspace
    __hip_atomic_store(&tickets[(size_t)b * kTicketStride], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  select_row<NT, SLOTS, SORTED, true, BLOCKED, IdsOut, (!BLOCKED && SLOTS >= 8), false, false, R8>(
      row, nv, row_cap, K, IdsOut{ids + (size_t)b * K}, counts ? counts + b : nullptr, sm,
      sort_lds);
}

// ---- launch templates ----------------------------------------------------------------
inline int topk_segments(int B, int N, int K) {
  // more workgroups while a row's segments stay long (at least 4096 entries and
  // twice K) and the candidates fit one register tile of the merge
  int S = 1;
  while (S < 8 && B <= kTopkSplitMaxRows && (int64_t)B * S * 2 <= 512 && N / (S * 2) >= 4096 && N / (S * 2) >= 2 * K &&
         (int64_t)(S * 2) * K <= kTopkNT * kTopkSlots * 4)
    S *= 2;
  return S;
}

// fp32 rows; R8: 8-bit radix digits
template <bool R8>
int launch_topk_f32(const void* scores, const int32_t* n_valid, int32_t* ids, int32_t* counts,
                    int B, int N, int K, bool sorted, void* split_ws, void* stream,
                    bool dot_scores) {
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
#define IDX_LAUNCH_SPLIT(SO, MS)                                                            \
  hipLaunchKernelGGL((topk_split_kernel<SO, MS, false, R8>), g2, dim3(kTopkNT), SO ? sort_lds_bytes(K) : 0, \
                     s, scores, n_valid, ids, counts, N, K, S, L, tickets, cs, ci, cstride)
    if (sorted) {
      if (merge2) IDX_LAUNCH_SPLIT(true, 2);
      else IDX_LAUNCH_SPLIT(true, kTopkSlots);
    } else {
      IDX_LAUNCH_SPLIT(false, 0);
    }
#undef IDX_LAUNCH_SPLIT
    return (int)hipGetLastError();
  }
  // Rows come from HBM here, so they are read in the striped layout (every load
  // fully coalesced). Many short rows (several rows per CU, each within one
  // 256-thread register tile of 2048 keys) take 256-thread workgroups, so that
  // several selects share a CU; otherwise 1024 threads per row, in a 2-slot
  // tile for rows of at most 8192 entries (no dead slots), else in 8 slots.
  // 256-thread workgroups order at most 1024 ids.
  const bool narrow = B >= 512 && N <= 2048 && (!sorted || K <= 1024);
#define IDX_LAUNCH_TOPK(SO, NT_, SL_, AD)                                                  \
  hipLaunchKernelGGL((topk_kernel<SO, NT_, SL_, AD, false, R8>), grid, dim3(NT_), SO ? sort_lds_bytes(K) : 0, \
                     s, scores, n_valid, ids, counts, N, K)
  if (narrow) {
    // index-order dot-product rows (the prompt-token select) in 512-thread
    // workgroups with one key slot (prompt tokens 16.7 -> 16.4 us; in score
    // order 16.8 -> 18.0 us, so those keep 256 threads); rows of any
    // distribution in 256-thread ones with two (1024 rows x 2048: 10.1 us,
    // against 10.8 in 512-thread workgroups)
    if (sorted) {
      if (dot_scores) IDX_LAUNCH_TOPK(true, 256, 2, false);
      else IDX_LAUNCH_TOPK(true, 256, 2, true);
    } else {
      if (dot_scores) IDX_LAUNCH_TOPK(false, 512, 1, false);
      else IDX_LAUNCH_TOPK(false, 256, 2, true);
    }
  } else if (N <= kTopkNT * 2 * 4) {
    // rows within one 2-slot tile of a 1024-thread workgroup
    if (sorted) {
      if (dot_scores) IDX_LAUNCH_TOPK(true, kTopkNT, 2, false);
      else IDX_LAUNCH_TOPK(true, kTopkNT, 2, true);
    } else {
      if (dot_scores) IDX_LAUNCH_TOPK(false, kTopkNT, 2, false);
      else IDX_LAUNCH_TOPK(false, kTopkNT, 2, true);
    }
  } else if (sorted) {
    hipLaunchKernelGGL((topk_kernel<true, kTopkNT, kTopkSlots, true, false, R8>), grid, dim3(kTopkNT),
                       sort_lds_bytes(K), s, scores, n_valid, ids, counts, N, K);
  } else {
    hipLaunchKernelGGL((topk_kernel<false, kTopkNT, kTopkSlots, true, false, R8>), grid, dim3(kTopkNT), 0, s,
                       scores, n_valid, ids, counts, N, K);
  }
#undef IDX_LAUNCH_TOPK
  return (int)hipGetLastError();
}

// R8: 8-bit radix digits (dense tables only)
template <bool R8>
int launch_select_t(const void* q, const void* c, const int32_t* seq_len, int32_t* ids,
                    int32_t* counts, float* scores_out, int B, int H, int N_pad, int page_size,
                    int K, bool bf16, bool sorted, int chunk, bool wide, uint32_t* tickets,
                    float* stage, int stage_stride, const int32_t* indptr, const int32_t* indices,
                    int64_t n_indices, int n_rows, void* stream, int tokens = 0) {
  const int nchunk = (N_pad + chunk - 1) / chunk;
  const dim3 grid((unsigned)B * nchunk);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // wide: 1024-thread workgroups (16 waves keep the selecting workgroup's SIMDs
  // busy; for a few long requests); otherwise 512 threads (many requests)
  // blocked: every row fits the select's register tile (1024*2*4 = 512*4*4 = 8192;
  // 512-thread workgroups use 1 slot, 512*1*4 = 2048, when that is enough)
  const bool blocked = N_pad <= 8192;
  const bool short_rows = N_pad <= 2048;
  const bool paged = indptr != nullptr;
  if (R8 && paged) return (int)hipErrorInvalidValue;
#define IDX_LAUNCH_FUSED(BF, SO, NT_, SL_, BL)                                                  \
  do {                                                                                         \
    if constexpr (!R8) {                                                                       \
      if (paged) {                                                                             \
        hipLaunchKernelGGL((select_fused_kernel<BF, SO, NT_, SL_, BL, true>), grid, dim3(NT_), \
                           SO ? sort_lds_bytes(K) : 0, s, q, c, seq_len, ids, counts,          \
                           scores_out, H, N_pad, page_size, K, chunk, nchunk, tickets, stage,  \
                           stage_stride, indptr, indices, n_indices, n_rows, 0);               \
        break;                                                                                 \
      }                                                                                        \
    }                                                                                          \
    hipLaunchKernelGGL((select_fused_kernel<BF, SO, NT_, SL_, BL, false, R8>), grid,           \
                       dim3(NT_), SO ? sort_lds_bytes(K) : 0, s, q, c, seq_len, ids, counts,   \
                       scores_out, H, N_pad, page_size, K, chunk, nchunk, tickets, stage,      \
                       stage_stride, indptr, indices, n_indices, n_rows, tokens);              \
  } while (0)
#define IDX_LAUNCH_FUSED_NT(BF, SO)                                                  \
  if (wide) {                                                                        \
    if (blocked) IDX_LAUNCH_FUSED(BF, SO, 1024, 2, true);                            \
    else IDX_LAUNCH_FUSED(BF, SO, 1024, 2, false);                                   \
  } else {                                                                           \
    if (short_rows) IDX_LAUNCH_FUSED(BF, SO, 512, 1, true);                          \
    else if (blocked) IDX_LAUNCH_FUSED(BF, SO, 512, 4, true);                        \
    else IDX_LAUNCH_FUSED(BF, SO, 512, 4, false);                                    \
  }
  if (bf16) {
    if (sorted) { IDX_LAUNCH_FUSED_NT(true, true); }
    else { IDX_LAUNCH_FUSED_NT(true, false); }
  } else {
    if (sorted) { IDX_LAUNCH_FUSED_NT(false, true); }
    else { IDX_LAUNCH_FUSED_NT(false, false); }
  }
#undef IDX_LAUNCH_FUSED_NT
#undef IDX_LAUNCH_FUSED
  return (int)hipGetLastError();
}

}  // namespace idxk
