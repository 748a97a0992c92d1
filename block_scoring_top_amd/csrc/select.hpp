// Exact row top-K by radix select ("Iterate Topk": radix top-K over order keys;
// "Round 18 Track C", section 1 Target 1: passes over unsigned order keys, each
// a histogram of the next digit scanned from the top bin down to find the bin
// that holds the K-th key and how many keys of that bin are still needed, keys
// cached in registers for short rows). Ties are taken in ascending index order,
// which the pages' bitwise id checks with adversarial ties require.
//
// One workgroup of NT threads selects one row. Keys live in registers, in one
// of two layouts. Striped: slot i of thread t holds the 4 consecutive entries
// starting at 4*(i*NT + t), so every load is a coalesced 16-byte vector load
// and rows longer than one register tile (NT*SLOTS*4 entries) are streamed
// tile by tile each pass. Blocked: thread t holds one run of consecutive
// entries, which makes the emit a single scan (rows that fit one tile).
//
// The select is bound by the issue of its per-key vector instructions (up to
// 16 waves share one CU) and by its barriers, so it is built to touch each key
// as few times, with as few instructions, as it can:
//  - Linear first pass (rows held in registers, except the 8-slot instances):
//    keys are counted in 2048 bins spread linearly over the row's value range.
//    On spread-out scores the K-th key's bin then holds a few keys: taken
//    whole, its smallest key is the threshold; otherwise up to 64 of them are
//    gathered in LDS and ranked. Rows where this fails (range not finite,
//    clustered or tied rows) fall back to:
//  - Radix passes: digits of 11, 11 and 10 bits (three passes instead of the
//    pages' four 8-bit ones; a 2048-bin histogram is 8 KiB of LDS). A pass
//    stops early when the chosen bin is taken whole, or when every key still
//    in play is the same value.
// Histograms: two 2048-bin LDS histograms, alternating by pass, so one is
// cleared while the other is searched; the search runs in all waves. Histogram
// adds peel off lanes that share a bin (a whole wave, or 16 or more lanes with
// the first active lane's digit) into one atomic, which removes the
// same-address atomic serialisation of degenerate rows.
//
// Emit: the taken keys are given by two bounds on a class value (the key, or
// the linear bin): above the upper bound taken, between the bounds the first
// `need` in index order. Output positions come from in-wave counts plus one
// workgroup scan, so ids are written in ascending index order without atomics
// (deterministic). The score order (score desc, id asc) orders the selected
// (key, ~id) pairs as 64-bit words: when the linear pass settled the row with a
// simple threshold, each taken key goes straight to its bin's segment of the
// output (counts of the bins above it, plus a slot from one LDS atomic) and
// ranks itself among the few keys of its bin; otherwise a bitonic sort.
#pragma once

#include "common.hpp"

namespace idxk {

constexpr int kMaxSortedK = 4096;
// threshold bins of more than 64 keys are refined by a bitonic sort (below)
constexpr bool kRefineBitonic = true;

// Radix digits of the order keys. 32-bit keys: 11 + 11 + 10 bits. Keys of
// bf16 scores (kDigits16) carry only 16 bits of information: the low half of
// the fp32 pattern is zero, so the low half of the key is 0x0000 for
// non-negative scores and 0xFFFF for negative ones; two digits of 11 + 5 bits
// resolve them ("Iterate Topk", section 6: a 16-bit radix for the bottom-zero
// bf16 keys). kDigits8: four 8-bit digits, the radix of the proposal seed in
// "Iterate Topk" (section 6) and of the four-pass loop in "Round 18 Track C"
// (section 1, Target 1), kept for comparison.
enum DigitScheme : int { kDigits11 = 0, kDigits16 = 1, kDigits8 = 2 };
constexpr int kResolved = 4;  // a `level` above every scheme's pass count: the whole key
template <int DS>
__device__ __forceinline__ int n_passes() {
  return DS == kDigits8 ? 4 : (DS == kDigits16 ? 2 : 3);
}
template <int DS>
__device__ __forceinline__ int digit_shift(int p) {
  if (DS == kDigits8) return 24 - 8 * p;
  return p == 0 ? kDigit0Shift : (DS == kDigits16 ? 16 : (p == 1 ? 10 : 0));
}
template <int DS>
__device__ __forceinline__ int digit_bits(int p) {
  if (DS == kDigits8) return 8;
  return p == 0 ? 11 : (DS == kDigits16 ? 5 : (p == 1 ? 11 : 10));
}
// the whole key of a bf16 score from its 16 significant bits
__device__ __forceinline__ uint32_t key16_full(uint32_t top) {
  return (top << 16) | ((top & 0x8000u) ? 0u : 0xFFFFu);
}

template <int NT, int SLOTS>
struct SelectSmem {
  static constexpr int NW = NT / kWave;
  static constexpr int E = SLOTS * NW;  // emit-count entries per tile
  alignas(16) uint32_t hist[2][kBins];
  uint32_t wpack[NW];  // per-wave counts of the blocked emit
  uint32_t wmin[NW], wmax[NW];  // per-wave min / max of the keys in play
  float wsum[NW];               // per-wave sums and counts of the scored entries
  uint32_t wcnt[NW];            // (the mapping choice of the 8-slot linear pass)
  uint32_t bin_max;             // max key of the linear threshold bin
  uint32_t sel_bin, sel_need, sel_tot, n_cand, all_same, same_key;
  uint32_t n_gather, gather[kWave];  // the keys of a small threshold bin
  uint32_t wtot[NW];                 // per-wave bin totals of the bin search
  uint32_t cgt[E], ceq[E];
  uint32_t tot_gt, tot_eq;
};

// Copies of the linear pass's histogram (select_row's HREP > 1, for rows with
// few distinct scores, whose lanes would otherwise queue on a few LDS words):
// lane l adds to copy l % HREP, and copy r starts r * kRepStride words after
// copy 0, so one bin of different copies sits in different LDS banks (kBins
// is a multiple of the 32 banks; 8 more words move each copy by 8 banks).
constexpr int kRepStride = kBins + 8;

// Loads one register tile of keys. Every load of the tile is issued before any
// is used (no branch between them), so the tile costs one memory round trip.
// `cap` is the number of floats that may be read at `row` (>= n): when the row
// is 16-byte aligned and cap is a multiple of 4, whole 4-float groups are read
// up to round_up(n, 4) <= cap and entries at or past n become kKeyNegInf
// (never candidates); otherwise entries are read one by one.
// With COHERENT every entry is read with an agent-scope load, which sees data
// that other workgroups wrote with agent-scope stores, on any XCD.
// BF16IN: the row holds bf16 scores (raw 16-bit patterns); every group of 4 is
// one 8-byte load when the row is 8-byte aligned, and each value is widened to
// its exact fp32 bits before the key transform.
template <int NT, int SLOTS, bool COHERENT, bool BF16IN = false>
__device__ __forceinline__ void load_keys(const void* row_v, int n, int cap, int base,
                                          uint32_t (&keys)[SLOTS][4]) {
  static_assert(!(COHERENT && BF16IN), "bf16 rows are caller inputs, not staged rows");
  const int t = threadIdx.x;
  const float* row = static_cast<const float*>(row_v);
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(row);
  if constexpr (BF16IN) {
    const uint16_t* h = static_cast<const uint16_t*>(row_v);
    const bool aligned4h = (((uintptr_t)h & 7) == 0) && (cap & 3) == 0;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (base + i * NT * 4 < n) {  // uniform: some thread of the workgroup has data here
        const int e0 = base + (i * NT + t) * 4;
        if (aligned4h) {
          const uint2 v = *reinterpret_cast<const uint2*>(h + (e0 < n ? e0 : 0));
          keys[i][0] = v.x << 16;
          keys[i][1] = v.x & 0xFFFF0000u;
          keys[i][2] = v.y << 16;
          keys[i][3] = v.y & 0xFFFF0000u;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) keys[i][j] = (uint32_t)h[e0 + j < n ? e0 + j : 0] << 16;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = base + (i * NT + t) * 4 + j;
        keys[i][j] = e < n ? order_key(__uint_as_float(keys[i][j])) : kKeyNegInf;
      }
    }
    return;
  }
  const bool aligned4 = (((uintptr_t)row & 15) == 0) && (cap & 3) == 0;
  if (COHERENT && aligned4) {
    // 16-byte buffer loads with the device-scope cache policy (sc1); the buffer
    // bounds are the row's readable bytes, past which a load returns zeros
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), (short)0, cap * 4, kBufferDword3);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (base + i * NT * 4 < n) {
        const int e0 = base + (i * NT + t) * 4;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, e0 * 4, 0, kCachePolicySc1);
        keys[i][0] = v[0];
        keys[i][1] = v[1];
        keys[i][2] = v[2];
        keys[i][3] = v[3];
      }
    }
  } else if (!COHERENT && aligned4) {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (base + i * NT * 4 < n) {  // uniform: some thread of the workgroup has data here
        const int e0 = base + (i * NT + t) * 4;
        const uint4 v = *reinterpret_cast<const uint4*>(bits + (e0 < n ? e0 : 0));
        keys[i][0] = v.x;
        keys[i][1] = v.y;
        keys[i][2] = v.z;
        keys[i][3] = v.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (base + i * NT * 4 < n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = base + (i * NT + t) * 4 + j;
          if constexpr (COHERENT)
            keys[i][j] = __hip_atomic_load(const_cast<uint32_t*>(bits) + (e < n ? e : 0),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            keys[i][j] = bits[e < n ? e : 0];
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = base + (i * NT + t) * 4 + j;
      keys[i][j] = e < n ? order_key(__uint_as_float(keys[i][j])) : kKeyNegInf;
    }
  }
}

// Loads the entries of `src` (written by other workgroups: agent-scope loads)
// at the places load_keys reads the keys of the same tile, as raw bits; entries
// past n are not read (their lanes are never emitted).
template <int NT, int SLOTS>
__device__ __forceinline__ void load_payload(const int32_t* src, int n, int cap, int base,
                                             uint32_t (&pay)[SLOTS][4]) {
  const int t = threadIdx.x;
  const bool aligned4 = (((uintptr_t)src & 15) == 0) && (cap & 3) == 0;
  if (aligned4) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(src), (short)0, cap * 4, kBufferDword3);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (base + i * NT * 4 < n) {
        const int e0 = base + (i * NT + t) * 4;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, e0 * 4, 0, kCachePolicySc1);
        pay[i][0] = v[0];
        pay[i][1] = v[1];
        pay[i][2] = v[2];
        pay[i][3] = v[3];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (base + i * NT * 4 < n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = base + (i * NT + t) * 4 + j;
          pay[i][j] = (uint32_t)__hip_atomic_load(const_cast<int32_t*>(src) + (e < n ? e : 0),
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// Loads a whole row (n <= NT * SLOTS * 4) in the blocked layout: thread t holds
// the kpt4 consecutive entries starting at t * kpt4 (kpt4 a multiple of 4, the
// same for every thread), so its keys are in ascending index order. Entries at
// or past n become kKeyNegInf. Loads are issued before any is used.
template <int NT, int SLOTS, bool COHERENT>
__device__ __forceinline__ void load_keys_blocked(const float* row, int n, int cap, int kpt4,
                                                  uint32_t (&keys)[SLOTS][4],
                                                  uint32_t (&raw)[SLOTS][4]) {
  const int t = threadIdx.x;
  const int e_base = t * kpt4;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(row);
  const bool aligned4 = (((uintptr_t)row & 15) == 0) && (cap & 3) == 0;
  if (aligned4) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), (short)0, cap * 4, kBufferDword3);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (4 * i < kpt4) {  // uniform
        // buffer loads: bounds-checked (zeros past cap); sc1 when the row was
        // written by other workgroups in this kernel
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (e_base + 4 * i) * 4, 0,
                                                             COHERENT ? kCachePolicySc1 : 0);
        keys[i][0] = v[0];
        keys[i][1] = v[1];
        keys[i][2] = v[2];
        keys[i][3] = v[3];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (4 * i < kpt4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = e_base + 4 * i + j;
          if constexpr (COHERENT)
            keys[i][j] = __hip_atomic_load(const_cast<uint32_t*>(bits) + (e < n ? e : 0),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            keys[i][j] = bits[e < n ? e : 0];
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < SLOTS; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[i][j] = keys[i][j];
  if (e_base + kpt4 <= n) {  // every entry of the thread is in the row (all but the last threads)
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        keys[i][j] = 4 * i < kpt4 ? order_key(__uint_as_float(keys[i][j])) : kKeyNegInf;
    }
  } else {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e_base + 4 * i + j;
        keys[i][j] = (4 * i < kpt4 && e < n) ? order_key(__uint_as_float(keys[i][j])) : kKeyNegInf;
      }
    }
  }
}

// Adds one count per active lane to h[digit]. When the first active lane's
// digit is shared by at least 16 lanes (all-equal, sorted or quantised rows),
// that lane adds the whole group's count and the group's other lanes add
// nothing, in the same atomic instruction as the lanes of other digits;
// otherwise every lane adds its own count.
__device__ __forceinline__ void hist_add(uint32_t* h, bool act, uint32_t digit) {
  const uint64_t m = ballot(act);
  if (m == 0) return;
  const uint32_t d0 = readlane<uint32_t>(digit, __builtin_ctzll(m));
  const uint64_t same = ballot(digit == d0) & m;
  const uint32_t ns = popc64(same);
  if (ns >= 16) {
    // the group's other lanes skip; its first lane adds the group's count
    const uint64_t lead = m & (~m + 1);
    if (__builtin_amdgcn_inverse_ballot_w64((m & ~same) | lead))
      atomicAdd(&h[digit], __builtin_amdgcn_inverse_ballot_w64(lead) ? ns : 1u);
  } else if (act) {
    atomicAdd(&h[digit], 1u);
  }
}

// Exclusive scan, in place, of a[0..E) and b[0..E) by wave 0; totals to *ta, *tb.
template <int E>
__device__ __forceinline__ void wave0_scan2(uint32_t* a, uint32_t* b, uint32_t* ta, uint32_t* tb) {
  constexpr int R = (E + kWave - 1) / kWave;
  const int lane = lane_id();
  uint32_t va[R], vb[R], sa = 0, sb = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int k = lane * R + r;
    va[r] = k < E ? a[k] : 0u;
    vb[r] = k < E ? b[k] : 0u;
    sa += va[r];
    sb += vb[r];
  }
  const uint32_t ia = wave_incl_scan(sa), ib = wave_incl_scan(sb);
  uint32_t ea = ia - sa, eb = ib - sb;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int k = lane * R + r;
    if (k < E) {
      a[k] = ea;
      b[k] = eb;
    }
    ea += va[r];
    eb += vb[r];
  }
  if (lane == kWave - 1) {
    *ta = ia;
    *tb = ib;
  }
}

// Bytes of dynamic LDS the score-ordered output needs for up to K ids: one
// 64-bit word per id, K rounded up to a power of two (at least 4).
__host__ __device__ inline int sort_lds_bytes(int K) {
  int p = 4;
  while (p < K) p <<= 1;
  return p * 8;
}

template <int M>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t v) {
  return (uint64_t)lane_xor<M>((uint32_t)(v >> 32)) << 32 | lane_xor<M>((uint32_t)v);
}

// One compare-exchange stage of a descending bitonic sort over elements held E
// per thread (element i = E*t + e in v[e]): partner i ^ J, and the pair is in
// descending order when bit k of i is clear. J < E pairs registers of one
// thread, E <= J < 64E lanes of one wave.
template <int E, int J>
__device__ __forceinline__ void bitonic_stage(uint64_t (&v)[E], int t, int k) {
  if constexpr (J < E) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & J) == 0) {
        const bool desc = ((E * t + e) & k) == 0;
        const uint64_t a = v[e], b = v[e | J];
        const bool sw = desc ? a < b : a > b;
        v[e] = sw ? b : a;
        v[e | J] = sw ? a : b;
      }
    }
  } else {
    constexpr int M = J / E;  // lane distance
    const bool lower = (t & M) == 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t u = lane_xor64<M>(v[e]);
      const bool keep_max = lower == (((E * t + e) & k) == 0);
      v[e] = (keep_max == (u > v[e])) ? u : v[e];
    }
  }
}

// the in-wave tail of a merge of size k: stages J, J/2, ..., 1
template <int E, int J>
__device__ __forceinline__ void bitonic_merge_tail(uint64_t (&v)[E], int t, int k) {
  bitonic_stage<E, J>(v, t, k);
  if constexpr (J > 1) bitonic_merge_tail<E, J / 2>(v, t, k);
}

// Bitonic sort into descending order of P 64-bit words (P a power of two,
// 64E <= P <= E * NT, or P < 64E with E == 1), E per thread: thread t < P / E
// holds elements E*t .. E*t+E-1 in v[0..E); the other threads hold nothing
// and skip the work, but take part in every barrier. Merges of up to 64E
// elements stay inside one wave (registers and cross-lane moves, no LDS); the
// stages of larger merges whose partners sit in another wave go through
// `xbuf` (P words of LDS), two barriers each.
template <int NT, int E>
__device__ __forceinline__ void bitonic_desc(uint64_t (&v)[E], int P, uint64_t* xbuf) {
  const int t = threadIdx.x;
  const bool live = E * t < P;
  const bool wave_live = E * (t & ~(kWave - 1)) < P;  // uniform per wave
  if (wave_live) {
#define IDX_BITONIC_RUN(KK, JJ)                                   \
  if constexpr (64 * E >= KK) {                                   \
    if (P >= KK) bitonic_merge_tail<E, JJ>(v, t, KK);             \
  }
    IDX_BITONIC_RUN(2, 1)
    IDX_BITONIC_RUN(4, 2)
    IDX_BITONIC_RUN(8, 4)
    IDX_BITONIC_RUN(16, 8)
    IDX_BITONIC_RUN(32, 16)
    IDX_BITONIC_RUN(64, 32)
    IDX_BITONIC_RUN(128, 64)
    IDX_BITONIC_RUN(256, 128)
#undef IDX_BITONIC_RUN
  }
  for (int k = 128 * E; k <= P; k <<= 1) {
    for (int j = k >> 1; j >= 64 * E; j >>= 1) {
      __syncthreads();  // earlier readers of xbuf are done
      if (live) {
#pragma unroll
        for (int e = 0; e < E; ++e) xbuf[E * t + e] = v[e];
      }
      __syncthreads();
      if (live) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = E * t + e;
          const uint64_t u = xbuf[i ^ j];
          const bool keep_max = ((i & j) == 0) == ((i & k) == 0);
          v[e] = (keep_max == (u > v[e])) ? u : v[e];
        }
      }
    }
    if (wave_live) bitonic_merge_tail<E, 32 * E>(v, t, k);
  }
}

// Where select_row puts its result: put(pos, id, key) for the pos-th selected
// entry (its index in the row and its order key), pad(k) for the unused slots
// k in [m, K).
//
// IdsOut: the ids themselves, -1 in unused slots.
struct IdsOut {
  static constexpr bool kUsesKey = false;  // put() ignores its key argument
  static constexpr bool kPayload = false;
  int32_t* ids;
  __device__ __forceinline__ void put(int pos, int id, uint32_t) const { ids[pos] = id; }
  __device__ __forceinline__ void pad(int k) const { ids[k] = -1; }
};

// score of an order key (the inverse of order_key; -0.0 comes back as +0.0)
__device__ __forceinline__ float key_to_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// CandOut: the candidates of one segment of a row, as (score, row index) pairs,
// written with agent-scope stores for the workgroup that merges the segments;
// unused slots hold -inf (never selected).
struct CandOut {
  static constexpr bool kUsesKey = true;  // the score is written beside the id
  static constexpr bool kPayload = false;
  float* score;
  int32_t* id;
  int base;  // the segment's first index in the row
  __device__ __forceinline__ void put(int pos, int i, uint32_t key) const {
    __hip_atomic_store(score + pos, key_to_score(key), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(id + pos, base + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ void pad(int k) const {
    __hip_atomic_store(score + k, -__builtin_inff(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(id + k, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

// StagedCandOut: CandOut's (score, row index) pairs written to LDS arrays of K
// entries (the caller copies them out once the select has returned); unused
// slots hold -inf and -1. The emit must not touch the LDS they occupy.
struct StagedCandOut {
  static constexpr bool kUsesKey = true;
  static constexpr bool kPayload = false;
  float* score;
  int32_t* id;
  int base;  // the segment's first index in the row
  __device__ __forceinline__ void put(int pos, int i, uint32_t key) const {
    score[pos] = key_to_score(key);
    id[pos] = base + i;
  }
  __device__ __forceinline__ void pad(int k) const {
    score[k] = -__builtin_inff();
    id[k] = -1;
  }
};

// MappedIdsOut: selecting over a candidate list, the id of candidate i is
// map[i] (written by other workgroups: read with agent-scope loads). Striped
// rows of 1 or 2 key slots load the map beside the keys (kPayload), in the same layout, so the
// index-order emit writes each id from a register (put_payload); the score
// order looks ids up (put).
struct MappedIdsOut {
  static constexpr bool kUsesKey = false;
  static constexpr bool kPayload = true;
  int32_t* ids;
  const int32_t* map;
  __device__ __forceinline__ void put(int pos, int i, uint32_t) const {
    ids[pos] = __hip_atomic_load(map + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ void put_payload(int pos, uint32_t v) const { ids[pos] = (int32_t)v; }
  __device__ __forceinline__ void pad(int k) const { ids[k] = -1; }
};

// Sorts the m pairs in sortbuf[0..m) into descending order and hands each
// entry (its position i in the order, its row index from the inverted low
// word) to out.put: E = 1 up to NT pairs (one per thread), else P / NT per
// thread.
template <int NT, int E, typename Out>
__device__ __forceinline__ void sort_pairs_desc(uint64_t* sortbuf, int m, int P, const Out& out) {
  const int t = threadIdx.x;
  __syncthreads();  // every pair is in sortbuf
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = E * t + e;
    v[e] = i < m ? sortbuf[i] : 0ull;
  }
  bitonic_desc<NT, E>(v, P, sortbuf);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = E * t + e;
    if (i < m) out.put(i, (int32_t)~(uint32_t)v[e], (uint32_t)(v[e] >> 32));
  }
}

// The linear bin of a key: the same float arithmetic as the linear pass (the
// key's score, scaled and shifted, clamped to [0, kBins - 1]).
// Value bins: x = score * scale + off (one fma). Key bins: x = (key - klo) *
// scale in the order-key domain, whose spacing grows with the magnitude
// (sign, exponent, mantissa), for rows of one sign that span many octaves.
// Both are monotone in the key and clamp to [0, kBins - 1].
struct BinMap {
  float scale, off;
  uint32_t klo;
  bool by_key;
  __device__ __forceinline__ uint32_t bin(uint32_t key, float score) const {
    const float x = by_key ? (float)(key - klo) * scale : __builtin_fmaf(score, scale, off);
    return (uint32_t)__builtin_amdgcn_fmed3f(x, 0.f, (float)(kBins - 1));
  }
  __device__ __forceinline__ uint32_t operator()(uint32_t key) const {
    return bin(key, key_to_score(key));
  }
};

// Finishes the score order of m pairs that sit in sortbuf[0..m) grouped by
// linear bin, highest bin first: bin b's pairs fill [sfx[b], sfx[b] + cnt[b]) in
// no particular order. Each thread takes the pairs at positions t + e * NT,
// ranks each among the pairs of its bin (one or two on spread-out scores; four
// reads in flight at a time) and hands the final position to out.put.
template <int NT, int E, typename Out>
__device__ __forceinline__ void rank_in_bins(uint64_t* sortbuf, int m, const BinMap& bin_of,
                                             const uint32_t* cnt, const uint32_t* sfx,
                                             const Out& out) {
  const int t = threadIdx.x;
  __syncthreads();  // every pair is in place
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = t + e * NT;
    if (i < m) {
      const uint64_t v = sortbuf[i];
      const uint32_t key = (uint32_t)(v >> 32), b = bin_of(key);
      const uint32_t base = sfx[b], c = cnt[b];
      uint32_t rank = 0;
      for (uint32_t r0 = 0; r0 < c; r0 += 4) {
        uint64_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = sortbuf[min(base + r0 + u, (uint32_t)m - 1u)];
#pragma unroll
        for (int u = 0; u < 4; ++u) rank += (r0 + u < c && x[u] > v) ? 1u : 0u;
      }
      out.put((int)(base + rank), (int32_t)~(uint32_t)v, key);
    }
  }
}

// Radix -> bitonic refinement of the linear pass's threshold bin ("Iterate
// Topk", section 6: a hybrid whose threshold bin is refined by a bitonic sort).
// When that bin holds more keys than the rank gather takes (64) but at most
// refine_cap<NT>() of them, not all equal, its keys are gathered into the
// histogram LDS (one reservation per wave and key slot), sorted in descending
// order, and the key at position bneed - 1 is the threshold; the keys of the
// bin above it are counted, which gives how many copies of the threshold to
// take. This replaces up to three radix passes over the whole row.
// 256-thread workgroups keep the radix passes (their four-word-per-thread sort
// measured slower: 1024 score-ordered rows of 2048 clustered scores, 16.6
// against 16.0 us).
template <int NT>
constexpr int refine_e() { return NT >= 1024 ? 2 : 4; }   // sorted words per thread
template <int NT>
constexpr int refine_cap() { return NT >= 512 ? refine_e<NT>() * NT : 0; }  // <= 2048 words

template <int NT, int SLOTS, class SM, class LiveFn>
__device__ __forceinline__ uint32_t refine_bin_bitonic(const uint32_t (&keys)[SLOTS][4],
                                                       const uint32_t (&bins)[SLOTS][4],
                                                       uint32_t sb, uint32_t btot, uint32_t bneed,
                                                       SM& sm, const LiveFn& slot_live,
                                                       uint32_t* need_eq) {
  constexpr int E = refine_e<NT>();
  static_assert(E * NT * 8 <= sizeof(sm.hist), "the sort fits the histogram LDS");
  uint64_t* buf = reinterpret_cast<uint64_t*>(&sm.hist[0][0]);
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  if (t == 0) sm.tot_gt = 0u;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    if (!slot_live(0, i)) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool g = keys[i][j] != kKeyNegInf && bins[i][j] == sb;
      const uint64_t m = ballot(g);
      if (m == 0) continue;  // uniform over the wave
      uint32_t base = 0u;
      if (lane == 0) base = atomicAdd(&sm.n_gather, popc64(m));
      base = readlane<uint32_t>(base, 0);
      if (g) buf[base + mbcnt(m)] = (uint64_t)keys[i][j] << 32;
    }
  }
  __syncthreads();
  int P = 64 * E;
  while (P < (int)btot) P <<= 1;
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = E * t + e;
    v[e] = i < (int)btot ? buf[i] : 0ull;  // zero sorts below every key
  }
  bitonic_desc<NT, E>(v, P, buf);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (E * t + e == (int)bneed - 1) sm.same_key = (uint32_t)(v[e] >> 32);
  __syncthreads();
  const uint32_t T = sm.same_key;
  uint32_t c = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) c += (uint32_t)(v[e] >> 32) > T ? 1u : 0u;
  c = readlane<uint32_t>(wave_incl_scan(c), kWave - 1);
  if (lane == 0 && c != 0u) atomicAdd(&sm.tot_gt, c);
  __syncthreads();
  *need_eq = bneed - sm.tot_gt;
  return T;
}

// All NW waves find the bin of h that holds the need-th largest of the counted
// keys, bins ranked from the top (kBins - 1) down: sm.sel_bin, sm.sel_need
// (need minus the keys in higher bins), sm.sel_tot (the bin's count) and
// sm.n_cand (the histogram's total). Wave w covers the kBins / NW bins below
// kBins - w * kBins / NW, each lane a run of BPL consecutive bins read as one
// vector (consecutive lanes, consecutive runs: no bank conflicts); a wave scan
// gives the counts above each lane within the wave, and after one barrier a
// scan of the per-wave totals gives the counts above each wave. The lane whose
// run holds the need-th key then walks its bins. Ends with a barrier; the
// results are read after the caller's next barrier. `clear` (may be null),
// kBins words, is zeroed on the way. With `sfx` (kBins words, may be null),
// sfx[b] gets the count of the bins above b and h is zeroed (for reuse as
// per-bin counters). R > 1: h holds R copies of the histogram, copy r at
// h + r * kRepStride, and a bin's count is the sum over the copies (only copy
// 0 is zeroed for sfx).
template <int NT, class SM, int R = 1>
__device__ __forceinline__ void find_bin(uint32_t* h, uint32_t need, SM& sm, uint32_t* clear,
                                         uint32_t* sfx = nullptr) {
  constexpr int NW = NT / kWave;
  constexpr int BPL = kBins / NT;  // bins per lane: 2, 4 or 8
  static_assert(BPL == 2 || BPL == 4 || BPL == 8, "2048 bins over 256..1024 threads");
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int top = kBins - (w * kWave + lane) * BPL;  // this lane's bins: [top - BPL, top)
  uint32_t c[BPL];  // c[k] = h[top - 1 - k]: descending
#pragma unroll
  for (int k = 0; k < BPL; ++k) c[k] = 0u;
#pragma unroll
  for (int cp = 0; cp < R; ++cp) {
    const uint32_t* hc = h + cp * kRepStride;
    if constexpr (BPL == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(hc + top - 2);
      c[0] += v.y; c[1] += v.x;
    } else {
#pragma unroll
      for (int r = 0; r < BPL / 4; ++r) {
        const uint4 v = *reinterpret_cast<const uint4*>(hc + top - 4 * (r + 1));
        c[4 * r] += v.w; c[4 * r + 1] += v.z; c[4 * r + 2] += v.y; c[4 * r + 3] += v.x;
      }
    }
  }
  uint32_t loc = 0;
#pragma unroll
  for (int k = 0; k < BPL; ++k) loc += c[k];
  const uint32_t incl = wave_incl_scan(loc);
  if (lane == kWave - 1) sm.wtot[w] = incl;
  if (clear != nullptr) {
#pragma unroll
    for (int k = 0; k < BPL; ++k) clear[threadIdx.x * BPL + k] = 0u;
  }
  if (sfx != nullptr) {  // this lane's own bins, already read
#pragma unroll
    for (int k = 0; k < BPL; ++k) h[top - 1 - k] = 0u;
  }
  __syncthreads();
  const uint32_t ws = wave_incl_scan(lane < NW ? sm.wtot[lane] : 0u);
  const uint32_t above = w > 0 ? readlane<uint32_t>(ws, w - 1) : 0u;
  if (w == 0 && lane == 0) sm.n_cand = readlane<uint32_t>(ws, NW - 1);
  uint32_t cum = above + incl - loc;
  if (sfx != nullptr) {
    uint32_t run = cum;
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
      sfx[top - 1 - k] = run;
      run += c[k];
    }
  }
  if (cum < need && need <= cum + loc) {  // one lane: the need-th key is in its bins
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
      if (cum < need && need <= cum + c[k]) {
        sm.sel_bin = (uint32_t)(top - 1 - k);
        sm.sel_need = need - cum;
        sm.sel_tot = c[k];
      }
      cum += c[k];
    }
  }
}

// BLOCKED: the caller guarantees n <= NT * SLOTS * 4; the row is held in the
// blocked layout. Otherwise any n, in the striped layout (streamed tile by tile
// when it does not fit one register tile). ADAPTIVE: the linear pass of a
// striped row chooses value or key bins from the mean of its scores.
// BF16IN: the row holds bf16 scores (striped rows only). KEY16: every key is
// that of a bf16 score (bf16 rows, or candidates taken from them), so two
// radix digits resolve a key. RADIX8: four 8-bit radix passes, no linear-bin
// pass (the same results, for comparison).
// HREP > 1: the linear pass counts into HREP copies of its histogram at hrep
// (HREP * kRepStride words of LDS).
template <int NT, int SLOTS, bool SORTED, bool COHERENT, bool BLOCKED, typename Out = IdsOut,
          bool ADAPTIVE = (!BLOCKED && SLOTS >= 8), bool BF16IN = false, bool KEY16 = BF16IN,
          bool RADIX8 = false, int HREP = 1>
__device__ __attribute__((always_inline)) void select_row(const void* row, int n, int cap, int K,
                                                         const Out& out, int32_t* count_out,
                                                         SelectSmem<NT, SLOTS>& sm,
                                                         uint64_t* sortbuf,
                                                         uint32_t* hrep = nullptr) {
  static_assert(HREP == 1 || HREP == 2 || HREP == 4 || HREP == 8, "1, 2, 4 or 8 copies");
  constexpr int NW = NT / kWave;
  constexpr int TILE = NT * SLOTS * 4;
  constexpr int E = SLOTS * NW;
  static_assert(NT >= 256 && NT <= 1024 && NT % 256 == 0,
                "256 to 1024 threads: the bin search gives each thread 2 to 8 bins");
  static_assert(!(BF16IN && BLOCKED), "bf16 rows use the striped layout");
  static_assert(!(RADIX8 && KEY16), "8-bit digits are built for 32-bit keys only");
  // RADIX8: four 8-bit radix passes and no linear-bin pass (for comparison)
  constexpr int kDS = RADIX8 ? kDigits8 : (KEY16 ? kDigits16 : kDigits11);
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int lane = t & (kWave - 1);
  const int ntiles = BLOCKED ? 1 : (n + TILE - 1) / TILE;
  const bool cached = ntiles <= 1;
  // blocked layout: thread t owns kpt4 consecutive entries
  const int kpt4 = BLOCKED ? ((n + NT - 1) / NT + 3) / 4 * 4 : 0;
  // slots that hold no entry of the row, for any thread, are skipped
  auto slot_live = [&](int base, int i) {
    return BLOCKED ? 4 * i < kpt4 : base + i * NT * 4 < n;
  };

  constexpr bool kPay = Out::kPayload && !BLOCKED && SLOTS <= 2;  // (registers: 4 per slot)
  uint32_t keys[SLOTS][4];
  uint32_t raw[BLOCKED ? SLOTS : 1][4];  // blocked rows: the scores' bits as loaded
  uint32_t pay[kPay ? SLOTS : 1][4];     // striped rows with a payload: out.map's entries
  if constexpr (BLOCKED) {
    load_keys_blocked<NT, SLOTS, COHERENT>(static_cast<const float*>(row), n, cap, kpt4, keys,
                                          raw);
  } else if (cached) {
    load_keys<NT, SLOTS, COHERENT, BF16IN>(row, n, cap, 0, keys);
    if constexpr (kPay) load_payload<NT, SLOTS>(out.map, n, cap, 0, pay);
  }

  // The linear bins and the all-equal exits need the min and max of the keys
  // in play: after the first pass those of the row (rows that try the linear
  // bins take them here, once, others during the first pass; the max may
  // include inactive keys: kKeyNegInf is below every active key but negative
  // NaNs, so min == max still means all active keys are equal), and for
  // striped rows (idx_topk inputs: quantised, heavy-tailed or tied rows) after
  // the second pass those of the keys left in the chosen bins. The blocked
  // rows of the fused select (dot-product scores) skip that second range: its
  // cost on every row outweighs the pass it saves on tied rows, and the third
  // pass resolves every remaining bit either way.
  // Rows held in registers first try one pass over linear bins (below): the
  // blocked and the 1- and 2-slot instances, and the 8-slot instances (few
  // long idx_topk rows, any distribution), which choose the bins per row from
  // the mean of the scores (kAdaptive). Not the 4-slot striped instances
  // (rows longer than one tile of the fused select, held in registers only
  // when a request is shorter than its table).
  constexpr bool kAdaptive = ADAPTIVE && !BLOCKED;
  constexpr bool kLinear = (BLOCKED || SLOTS <= 2 || kAdaptive) && !RADIX8;
  const bool upfront = kLinear && cached;  // the range is taken before the passes
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (upfront) {
    float fsum = 0.f;
    uint32_t fcnt = 0u;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (!slot_live(0, i)) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t key = keys[i][j];
        kmin = min(kmin, key == kKeyNegInf ? 0xFFFFFFFFu : key);
        kmax = max(kmax, key);
        if constexpr (kAdaptive) {
          const bool act = key != kKeyNegInf;
          fsum += act ? key_to_score(key) : 0.f;
          fcnt += act ? 1u : 0u;
        }
      }
    }
    kmin = wave_reduce_minmax<true>(kmin);
    kmax = wave_reduce_minmax<false>(kmax);
    if constexpr (kAdaptive) {
      fsum = wave_sum_f32(fsum);
      fcnt = readlane<uint32_t>(wave_incl_scan(fcnt), kWave - 1);
    }
    if (lane == 0) {
      sm.wmin[w] = kmin;
      sm.wmax[w] = kmax;
      if constexpr (kAdaptive) {
        sm.wsum[w] = fsum;
        sm.wcnt[w] = fcnt;
      }
    }
  }
  for (int i = t; i < 2 * kBins; i += NT) (&sm.hist[0][0])[i] = 0u;
  if constexpr (HREP > 1) {
    static_assert(kRepStride % 4 == 0, "the copies are cleared as 16-byte words");
    if (upfront)
      for (int i = t; i < HREP * kRepStride / 4; i += NT)
        reinterpret_cast<uint4*>(hrep)[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  uint32_t prefix = 0, need = (uint32_t)K, ncand = 0;
  int level = 0;  // digits resolved (kResolved = the whole key)
  bool take_all = false, resolved = false;
  // simple threshold: exactly the keys whose class value (the key, or its
  // linear bin) is at least t_lo are taken, with no partial tie
  bool simple = false;
  uint32_t t_lo = 0u;
  int boff = 0;  // histogram buffer of the first radix pass
  // score order from the linear bins (SORTED rows the linear pass settles
  // with a simple threshold): histogram 1 holds the count of the keys in
  // higher bins, histogram 0 per-bin counters
  bool by_bins = false;
  uint32_t bins[SLOTS][4];
  BinMap bin_map{0.f, 0.f, 0u, false};  // the linear pass's bins

  // The linear pass: with the row's range [lo, hi], key x goes to bin
  // floor((x - lo) * kBins / (hi - lo)), clamped to the last bin (monotone in
  // x, so a higher bin never holds a smaller key, and equal scores share a
  // bin). On spread-out scores the bin of the K-th key then holds a few keys,
  // where the first 11-bit digit (sign, exponent, two mantissa bits) leaves
  // tens to hundreds, and a second radix pass would follow. A bin taken whole
  // gives a simple threshold; a bin of at most 64 keys is gathered in LDS and
  // wave 0 ranks them, which gives an exact threshold key. Otherwise (ranges
  // that are not finite, clustered or tied rows) the radix passes below
  // resolve the row.
  if (upfront) {
    uint32_t lo = lane < NW ? sm.wmin[lane] : 0xFFFFFFFFu;
    uint32_t hi = lane < NW ? sm.wmax[lane] : 0u;
    lo = wave_reduce_minmax<true>(lo);
    hi = wave_reduce_minmax<false>(hi);
    const float flo = key_to_score(lo), fhi = key_to_score(hi);
    const float span = fhi - flo;
    const float scale = (float)kBins / span;
    // the same values in every wave: the branches are uniform over the workgroup
    const bool value_ok = lo < hi && __builtin_isfinite(flo) && __builtin_isfinite(fhi) &&
                          __builtin_isfinite(span) && span > 0.f && __builtin_isfinite(scale);
    bool by_key = false;
    if constexpr (kAdaptive) {
      // Rows of one sign whose mean sits in the outer 1/32 of [lo, hi]
      // (heavy-tailed rows: most scores crowd one end, where value bins would
      // put the K-th score in a bin of hundreds) take key bins.
      float fs = lane < NW ? sm.wsum[lane] : 0.f;
      uint32_t fc = lane < NW ? sm.wcnt[lane] : 0u;
      fs = wave_sum_f32(fs);
      fc = readlane<uint32_t>(wave_incl_scan(fc), kWave - 1);
      const float pos = (fs / (float)fc - flo) / span;  // NaN or inf when degenerate
      const bool one_sign = lo >= 0x80000000u || hi < 0x80000000u;
      by_key = lo < hi && one_sign && !(pos >= 1.f / 32.f && pos <= 31.f / 32.f);
    }
    if (value_ok || by_key) {
      const BinMap bm{by_key ? (float)kBins / (float)(hi - lo) : scale, by_key ? 0.f : -flo * scale,
                      lo, by_key};
      bin_map = bm;
      uint32_t* h = sm.hist[0];
      // this lane's copy of the histogram
      uint32_t* hl = HREP > 1 ? hrep + (lane & (HREP - 1)) * kRepStride : h;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (!slot_live(0, i)) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // unscored entries (kKeyNegInf, or past the row with arbitrary
          // bits) go to bin 0 and are not counted
          const bool act = keys[i][j] != kKeyNegInf;
          float f;
          if constexpr (BLOCKED)
            f = __uint_as_float(raw[i][j]);
          else
            f = key_to_score(keys[i][j]);
          const uint32_t bin = act ? bm.bin(keys[i][j], f) : 0u;
          bins[i][j] = bin;
          // Linear bins are spread out by construction, so every lane adds
          // its own count: independent atomics, with no per-key wave test.
          // Rows whose scores all share one bin except an outlier's, and
          // quantised rows, measured the same as with merged adds of shared
          // bins.
          if (act) atomicAdd(&hl[bin], 1u);
        }
      }
      if (t == 0) {
        sm.n_gather = 0u;
        sm.same_key = 0xFFFFFFFFu;
        sm.bin_max = 0u;
      }
      __syncthreads();
      // with copies, histogram 0 stays zero (as find_bin leaves it for the
      // score-ordered counters, and as the radix passes expect it)
      if constexpr (SORTED)
        find_bin<NT, SelectSmem<NT, SLOTS>, HREP>(HREP > 1 ? hrep : h, need, sm, nullptr,
                                                  sm.hist[1]);
      else
        find_bin<NT, SelectSmem<NT, SLOTS>, HREP>(HREP > 1 ? hrep : h, need, sm, sm.hist[1]);
      __syncthreads();
      ncand = sm.n_cand;
      const uint32_t sb = sm.sel_bin, bneed = sm.sel_need, btot = sm.sel_tot;
      if (ncand <= (uint32_t)K) {
        take_all = true;
        resolved = true;
        by_bins = SORTED;
      } else if (btot == bneed && !SORTED && !Out::kUsesKey && sb > 0) {
        // the bin is taken whole and only ids are written: the keys of bins
        // sb and above are taken, so the bins become the class values (scored
        // keys below the bin, and unscored ones in bin 0, stay below sb)
#pragma unroll
        for (int i = 0; i < SLOTS; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) keys[i][j] = bins[i][j];
        simple = true;
        t_lo = sb;
        resolved = true;
      } else if (btot == bneed) {
        // the bin is taken whole: the threshold is its smallest key, and every
        // key at or above it is taken (they make K)
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
          if (!slot_live(0, i)) continue;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (keys[i][j] != kKeyNegInf && bins[i][j] == sb) atomicMin(&sm.same_key, keys[i][j]);
        }
        __syncthreads();
        simple = true;
        t_lo = sm.same_key;
        resolved = true;
        by_bins = SORTED;
      } else if (btot <= (uint32_t)kWave) {
        // gather the bin's keys into LDS
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
          if (!slot_live(0, i)) continue;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // at most 64 keys of the row match: one slot per key from an LDS
            // atomic, with no per-key wave test (the rank below does not
            // depend on the order)
            if (keys[i][j] != kKeyNegInf && bins[i][j] == sb)
              sm.gather[atomicAdd(&sm.n_gather, 1u)] = keys[i][j];
          }
        }
        __syncthreads();
        if (w == 0) {
          // lane l ranks gathered key c: gt keys above it, eq equal to it; the
          // threshold is the key with gt < bneed <= gt + eq
          const uint32_t c = (uint32_t)lane < btot ? sm.gather[lane] : 0u;
          uint32_t gt = 0, eq = 0;
          for (uint32_t j = 0; j < btot; ++j) {
            const uint32_t x = readlane<uint32_t>(c, (int)j);
            gt += x > c ? 1u : 0u;
            eq += x == c ? 1u : 0u;
          }
          const uint64_t hm = ballot((uint32_t)lane < btot && gt < bneed && bneed <= gt + eq);
          const int l0 = hm != 0 ? __builtin_ctzll(hm) : 0;  // hm != 0: 1 <= bneed <= btot
          const uint32_t tkey = readlane<uint32_t>(c, l0);
          const uint32_t tgt = readlane<uint32_t>(gt, l0);
          const uint32_t teq = readlane<uint32_t>(eq, l0);
          if (lane == 0) {
            sm.same_key = tkey;
            sm.sel_need = bneed - tgt;
            sm.all_same = teq == bneed - tgt ? 1u : 0u;  // every copy of the threshold taken
          }
        }
        __syncthreads();
        prefix = sm.same_key;
        need = sm.sel_need;
        level = kResolved;
        resolved = true;
        if (sm.all_same) {
          simple = true;
          t_lo = prefix;
          by_bins = SORTED;
        }
      } else {
        // too many to gather: when every key of the bin is the same
        // (quantised or tied rows), that key is the threshold
        uint32_t bmin = 0xFFFFFFFFu, bmax = 0u;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
          if (!slot_live(0, i)) continue;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool g = keys[i][j] != kKeyNegInf && bins[i][j] == sb;
            bmin = g ? min(bmin, keys[i][j]) : bmin;
            bmax = g ? max(bmax, keys[i][j]) : bmax;
          }
        }
        bmin = wave_reduce_minmax<true>(bmin);
        bmax = wave_reduce_minmax<false>(bmax);
        if (lane == 0 && bmin <= bmax) {
          atomicMin(&sm.same_key, bmin);
          atomicMax(&sm.bin_max, bmax);
        }
        __syncthreads();
        if (sm.same_key == sm.bin_max) {
          prefix = sm.same_key;
          need = bneed;
          level = kResolved;
          resolved = true;
        } else if (kRefineBitonic && btot <= (uint32_t)refine_cap<NT>()) {
          uint32_t neq;
          prefix = refine_bin_bitonic<NT, SLOTS>(keys, bins, sb, btot, bneed, sm, slot_live, &neq);
          need = neq;
          level = kResolved;
          resolved = true;
        } else {
          // the linear counts are in histogram 0 and histogram 1 is clear, or
          // (score-ordered rows) histogram 0 was zeroed for counters
          boff = SORTED ? 0 : 1;
        }
      }
    }
  }

  // Each pass histograms the next digit of the keys that still match the
  // resolved prefix, then finds the bin holding the need-th largest of them
  // (wave 0, find_bin above).
  for (int p = 0; p < (resolved ? 0 : n_passes<kDS>()); ++p) {
    const int buf = (p + boff) & 1;
    uint32_t* h = sm.hist[buf];
    const int shift = digit_shift<kDS>(p);
    const uint32_t dmask = (1u << digit_bits<kDS>(p)) - 1u;
    const int hshift = p == 0 ? 0 : digit_shift<kDS>(p - 1);  // the resolved bits sit above this
    // this pass takes the range of its keys
    const bool track = (p == 0 && !upfront) || (!BLOCKED && p == 1);
    if (p == 1) {
      kmin = 0xFFFFFFFFu;
      kmax = 0u;
    }
    for (int tile = 0; tile < ntiles; ++tile) {
      if (!cached) load_keys<NT, SLOTS, COHERENT, BF16IN>(row, n, cap, tile * TILE, keys);
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (!slot_live(tile * TILE, i)) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t key = keys[i][j];
          const bool act = key != kKeyNegInf && (p == 0 || (key >> hshift) == prefix);
          hist_add(h, act, (key >> shift) & dmask);
          if (track) {
            kmin = act && key < kmin ? key : kmin;
            kmax = act && key > kmax ? key : kmax;
          }
        }
      }
    }
    if (track) {
      kmin = wave_reduce_minmax<true>(kmin);
      kmax = wave_reduce_minmax<false>(kmax);
      if (lane == 0) {
        sm.wmin[w] = kmin;
        sm.wmax[w] = kmax;
      }
    }
    __syncthreads();
    // All waves find the bin and clear the next pass's histogram; where a pass
    // has a key range (above), wave 0 also reduces the per-wave ranges.
    find_bin<NT>(h, need, sm, sm.hist[buf ^ 1]);
    if (w == 0) {
      if (p == 0 || (!BLOCKED && p == 1)) {
        uint32_t lo = lane < NW ? sm.wmin[lane] : 0xFFFFFFFFu;
        uint32_t hi = lane < NW ? sm.wmax[lane] : 0u;
        lo = wave_reduce_minmax<true>(lo);
        hi = wave_reduce_minmax<false>(hi);
        if (lane == 0) sm.all_same = lo == hi ? 1u : 0u;
        if (lane == 0) sm.same_key = lo;
      }
    }
    __syncthreads();
    if (p == 0) {
      ncand = sm.n_cand;
      if (ncand <= (uint32_t)K) {
        take_all = true;
        break;
      }
    }
    // every key in play is the same value: the threshold is that key, of which
    // `need` are taken (identical keys would only fill one bin per later pass)
    if ((p == 0 || (!BLOCKED && p == 1)) && sm.all_same) {
      prefix = sm.same_key;
      level = kResolved;
      break;
    }
    prefix = (prefix << digit_bits<kDS>(p)) | sm.sel_bin;
    need = sm.sel_need;
    level = p + 1;
    if (KEY16 && p == 1) {  // the 16 significant bits fix the whole key
      prefix = key16_full(prefix);
      level = kResolved;
    }
    if (sm.sel_tot == need) {  // the whole bin is taken: every key from its lowest on
      simple = true;
      t_lo = level == kResolved ? prefix : prefix << digit_shift<kDS>(p);
      break;
    }
  }

  // ---- emit --------------------------------------------------------------------------
  // The taken keys as two class bounds: a key above hi_b is taken; a key in
  // [lo_b, hi_b] is a threshold copy, of which the first need_e in index order
  // are taken. A simple threshold t_lo is hi_b = t_lo - 1 with an empty copy
  // range. Every scored key is above kKeyNegInf (NaN scores are outside the
  // contract), so take_all is the simple threshold kKeyNegInf + 1.
  if (take_all) {
    simple = true;
    t_lo = kKeyNegInf + 1u;
  }
  // the bits below the resolved digits (KEY16 rows: level 1 or kResolved)
  const int shiftL = (level <= 0 || level >= kResolved) ? 0 : digit_shift<kDS>(level - 1);
  const uint32_t lo_b = simple ? t_lo : prefix << shiftL;
  const uint32_t hi_b = simple ? t_lo - 1u : lo_b | ((1u << shiftL) - 1u);
  const uint32_t need_e = simple ? 0u : need;
  const uint32_t m_out = take_all ? ncand : (uint32_t)K;
  if constexpr (SORTED) {
    if (by_bins) {
      // Score order from the linear bins, no sorting network: histogram 1
      // holds sfx[b], the count of the taken keys in bins above b, and
      // histogram 0 is zero. A taken key of bin b goes to slot sfx[b] +
      // atomicAdd(cnt[b], 1) (every atomic of the thread issued before the
      // first return is used); rank_in_bins then orders each bin's keys.
      uint32_t* cnt = sm.hist[0];
      const uint32_t* sfx = sm.hist[1];
      uint32_t dst[SLOTS][4];
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (!slot_live(0, i)) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dst[i][j] = 0u;
          if (keys[i][j] >= t_lo) dst[i][j] = atomicAdd(&cnt[bins[i][j]], 1u) + sfx[bins[i][j]];
        }
      }
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (!slot_live(0, i)) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int id = BLOCKED ? t * kpt4 + 4 * i + j : (i * NT + t) * 4 + j;
          if (keys[i][j] >= t_lo && dst[i][j] < m_out)  // dst < m_out always holds
            sortbuf[dst[i][j]] = (uint64_t)keys[i][j] << 32 | (uint32_t)~id;
        }
      }
    }
  }
  if (BLOCKED && !by_bins) {
    // Blocked layout: each thread counts its taken-for-sure (gt) and threshold
    // (eq) keys, one workgroup scan of the counts gives the keys before the
    // thread, and the thread then writes its taken ids in ascending order.
    auto count_before = [&](uint32_t mine) {  // workgroup exclusive scan
      const uint32_t incl = wave_incl_scan(mine);
      if (lane == kWave - 1) sm.wpack[w] = incl;
      __syncthreads();
      // counts of the waves before this one: a scan over the per-wave totals
      const uint32_t wscan = wave_incl_scan(lane < NW ? sm.wpack[lane] : 0u);
      const int wu = __builtin_amdgcn_readfirstlane(w);
      return incl - mine + (wu > 0 ? readlane<uint32_t>(wscan, wu - 1) : 0u);
    };
    if (simple) {
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (!slot_live(0, i)) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) cnt += keys[i][j] >= t_lo ? 1u : 0u;
      }
      uint32_t g = count_before(cnt);
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (!slot_live(0, i)) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool take = keys[i][j] >= t_lo;
          if (take && g < m_out) {  // g < m_out always holds; the test only bounds the store
            const int id = t * kpt4 + 4 * i + j;
            if constexpr (SORTED) {
              sortbuf[g] = (uint64_t)keys[i][j] << 32 | (uint32_t)~id;
            } else {
              out.put((int)g, id, keys[i][j]);
            }
          }
          g += take ? 1u : 0u;
        }
      }
    } else {
      // threshold copies: packed counts (eq << 16 | gt; both fit 16 bits since
      // n <= 32768)
      uint32_t ngt = 0, nge = 0;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (!slot_live(0, i)) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ngt += keys[i][j] > hi_b ? 1u : 0u;
          nge += keys[i][j] >= lo_b ? 1u : 0u;
        }
      }
      const uint32_t packed = ngt + ((nge - ngt) << 16);
      const uint32_t before = count_before(packed);
      uint32_t gb = before & 0xFFFFu, eb = before >> 16;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (!slot_live(0, i)) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool gt = keys[i][j] > hi_b;
          const bool eq = !gt && keys[i][j] >= lo_b;
          const bool take = gt || (eq && eb < need_e);
          const uint32_t pos = gb + min(eb, need_e);
          if (take && pos < m_out) {  // pos < m_out always holds; the test only bounds the store
            const int id = t * kpt4 + 4 * i + j;
            if constexpr (SORTED) {
              sortbuf[pos] = (uint64_t)keys[i][j] << 32 | (uint32_t)~id;
            } else {
              out.put((int)pos, id, keys[i][j]);
            }
          }
          gb += gt ? 1u : 0u;
          eb += eq ? 1u : 0u;
        }
      }
    }
  }
  uint32_t carry_gt = 0, carry_eq = 0;
  for (int tile = 0; tile < ((BLOCKED || by_bins) ? 0 : ntiles); ++tile) {
    if (!cached) {
      __syncthreads();  // the previous tile's counts have been read
      load_keys<NT, SLOTS, COHERENT, BF16IN>(row, n, cap, tile * TILE, keys);
      if constexpr (kPay) load_payload<NT, SLOTS>(out.map, n, cap, tile * TILE, pay);
    }
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      uint32_t g = 0, e = 0;
      if (slot_live(tile * TILE, i)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t key = keys[i][j];
          const bool gt = key > hi_b;
          g += popc64(ballot(gt));
          e += popc64(ballot(!gt && key >= lo_b));
        }
      }
      if (lane == 0) {
        sm.cgt[i * NW + w] = g;
        sm.ceq[i * NW + w] = e;
      }
    }
    __syncthreads();
    if (w == 0) wave0_scan2<E>(sm.cgt, sm.ceq, &sm.tot_gt, &sm.tot_eq);
    __syncthreads();
    const int tbase = tile * TILE;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (!slot_live(tbase, i)) continue;
      bool gt[4], eq[4];
      uint32_t gb = carry_gt + sm.cgt[i * NW + w];
      uint32_t eb = carry_eq + sm.ceq[i * NW + w];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t key = keys[i][j];
        gt[j] = key > hi_b;
        eq[j] = !gt[j] && key >= lo_b;
        gb += mbcnt(ballot(gt[j]));
        eb += mbcnt(ballot(eq[j]));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool take = gt[j] || (eq[j] && eb < need_e);
        const uint32_t pos = gb + min(eb, need_e);
        if (take && pos < m_out) {  // pos < m_out always holds; the test only bounds the store
          const int id = tbase + (i * NT + t) * 4 + j;
          if constexpr (SORTED) {
            sortbuf[pos] = (uint64_t)keys[i][j] << 32 | (uint32_t)~id;
          } else if constexpr (kPay) {
            out.put_payload((int)pos, pay[i][j]);
          } else {
            out.put((int)pos, id, keys[i][j]);
          }
        }
        gb += gt[j] ? 1u : 0u;
        eb += eq[j] ? 1u : 0u;
      }
    }
    carry_gt += sm.tot_gt;
    carry_eq += sm.tot_eq;
  }

  // Every taken key is the one threshold key (no key above a one-key band):
  // the pairs were placed in index order, which for equal keys is the score
  // order (ties to the lower id), so they need no sort.
  const bool one_key = !BLOCKED && !by_bins && !simple && lo_b == hi_b && carry_gt == 0u;

  for (int k = (int)m_out + t; k < K; k += NT) out.pad(k);
  if (count_out != nullptr && t == 0) *count_out = (int32_t)m_out;

  if constexpr (SORTED) {
    // (key << 32 | ~id) is unique per pair and orders by key, then by lower id
    int P = 2;
    while (P < (int)m_out) P <<= 1;
    // P <= 4 * NT: callers give 256- and 512-thread workgroups at most 1024 ids
    // to order (1024-thread ones take up to kMaxSortedK = 4 * 1024)
    if (by_bins) {
      if (P <= NT) {
        rank_in_bins<NT, 1>(sortbuf, (int)m_out, bin_map, sm.hist[0], sm.hist[1], out);
      } else if (P == 2 * NT) {
        rank_in_bins<NT, 2>(sortbuf, (int)m_out, bin_map, sm.hist[0], sm.hist[1], out);
      } else {
        rank_in_bins<NT, 4>(sortbuf, (int)m_out, bin_map, sm.hist[0], sm.hist[1], out);
      }
    } else if (one_key) {
      __syncthreads();  // every pair is in sortbuf
      for (int i = t; i < (int)m_out; i += NT) {
        const uint64_t v = sortbuf[i];
        out.put(i, (int32_t)~(uint32_t)v, (uint32_t)(v >> 32));
      }
    } else {
      // zero (below every key) pads the sort up to a power of two
      if (P <= NT) {
        sort_pairs_desc<NT, 1>(sortbuf, (int)m_out, P, out);
      } else if (P == 2 * NT) {
        sort_pairs_desc<NT, 2>(sortbuf, (int)m_out, P, out);
      } else {
        sort_pairs_desc<NT, 4>(sortbuf, (int)m_out, P, out);
      }
    }
  }
}

}  // namespace idxk
