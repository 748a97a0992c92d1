// Exact row top-K by 4-pass 8-bit radix select ("Iterate Topk": 8-bit radix
// top-K; "Round 18 Track C", section 1 Target 1: four passes over uint order
// keys, a 256-bin histogram scanned from the top bin down to find the bin that
// holds the K-th key and how many keys of that bin are still needed, keys
// cached in registers for short rows). Ties are taken in ascending index order,
// which the pages' bitwise id checks with adversarial ties require.
//
// One workgroup of NT threads selects one row. Keys live in registers in a
// striped layout: slot i of thread t holds the 4 consecutive entries starting
// at 4*(i*NT + t), so every load is a coalesced 16-byte vector load and, for a
// fixed slot, the workgroup holds one contiguous index range. Rows longer than
// one register tile (NT*SLOTS*4 entries) are streamed tile by tile each pass.
//
// Histogram: per-wave 256-bin sub-histograms in LDS. Before the LDS atomics a
// wave peels off the group of lanes that share the first active lane's digit
// and adds that group with one atomic; on degenerate rows (all equal, few
// distinct values) this removes the same-address atomic serialisation.
//
// Emit: a key is taken if its resolved digits exceed the threshold prefix, or
// equal it and fewer than `need` equal keys precede it. Output positions come
// from ballot/mbcnt counts inside a wave plus one workgroup scan over
// (slot, wave) counts, so ids are written in ascending index order without any
// atomics (deterministic). The sorted order (score desc, id asc) is then a rank
// count over the selected (key, id) pairs in LDS.
#pragma once

#include "common.hpp"

namespace idxk {

constexpr int kMaxSortedK = 4096;

constexpr int kPasses = 3;
__device__ __forceinline__ int digit_shift(int p) {
  return p == 0 ? kDigit0Shift : (p == 1 ? 10 : 0);
}
__device__ __forceinline__ uint32_t digit_mask(int p) { return p == 2 ? 0x3FFu : 0x7FFu; }

template <int NT, int SLOTS, bool SORTED>
struct SelectSmem {
  static constexpr int NW = NT / kWave;
  static constexpr int E = SLOTS * NW;  // emit-count entries per tile
  uint32_t hist[2][kBins];
  uint32_t wsum[4];
  uint32_t wpack[NW];  // per-wave packed (eq << 16 | gt) counts of the blocked emit
  uint32_t wmin[NW], wmax[NW];  // per-wave min / max of a pass's active keys
  uint32_t sel_bin, sel_need, sel_tot, n_cand;
  uint32_t cgt[E], ceq[E];
  uint32_t tot_gt, tot_eq;
  alignas(16) uint32_t skey[SORTED ? kMaxSortedK + 4 : 1];
  int32_t sid[SORTED ? kMaxSortedK : 1];
};

// Loads one register tile of keys. Every load of the tile is issued before any
// is used (no branch between them), so the tile costs one memory round trip.
// `cap` is the number of floats that may be read at `row` (>= n): when the row
// is 16-byte aligned and cap is a multiple of 4, whole 4-float groups are read
// up to round_up(n, 4) <= cap and entries at or past n become kKeyNegInf
// (never candidates); otherwise entries are read one by one.
// With COHERENT every entry is read with an agent-scope load, which sees data
// that other workgroups wrote with agent-scope stores, on any XCD.
template <int NT, int SLOTS, bool COHERENT>
__device__ __forceinline__ void load_keys(const float* row, int n, int cap, int base,
                                          uint32_t (&keys)[SLOTS][4]) {
  const int t = threadIdx.x;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(row);
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

// Loads a whole row (n <= NT * SLOTS * 4) in the blocked layout: thread t holds
// the kpt4 consecutive entries starting at t * kpt4 (kpt4 a multiple of 4, the
// same for every thread), so its keys are in ascending index order. Entries at
// or past n become kKeyNegInf. Loads are issued before any is used.
template <int NT, int SLOTS, bool COHERENT>
__device__ __forceinline__ void load_keys_blocked(const float* row, int n, int cap, int kpt4,
                                                  uint32_t (&keys)[SLOTS][4]) {
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
  for (int i = 0; i < SLOTS; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e_base + 4 * i + j;
      keys[i][j] = (4 * i < kpt4 && e < n) ? order_key(__uint_as_float(keys[i][j])) : kKeyNegInf;
    }
  }
}

// Adds one count per active lane to h[digit]. When every active lane of the
// wave has the same digit (all-equal or sorted rows) the wave adds them with one
// atomic; when the first active lane's digit is shared by at least 16 lanes that
// group is added with one atomic and the rest one by one; otherwise every lane
// adds its own count (distinct digits do not serialise).
__device__ __forceinline__ void hist_add(uint32_t* h, bool act, uint32_t digit) {
  const uint64_t m = ballot(act);
  if (m == 0) return;
  const int leader = __builtin_ctzll(m);
  const uint32_t d0 = readlane<uint32_t>(digit, leader);
  const uint64_t same = ballot(act && digit == d0);
  const uint32_t ns = popc64(same);
  if (ns >= 16) {
    if (lane_id() == leader) atomicAdd(&h[d0], ns);
    if (same != m && act && digit != d0) atomicAdd(&h[digit], 1u);
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

// Counts, for element i of keys[0..m) (LDS, zero-padded to a multiple of 4),
//   gt = #{j : keys[j] > keys[i]}  and  tie = #{j < i : keys[j] == keys[i]}
//   (or, with TIES_ALL, eq = #{j : keys[j] == keys[i]}).
// Four adjacent lanes share one element, each counting a quarter of the groups
// of 4 keys, and their counts are summed across the quad; every loop is uniform
// across the wave. fn(i, key_i, gt, tie_or_eq) is called by the quad's first lane.
template <int NT, bool TIES_ALL, typename Fn>
__device__ __forceinline__ void quad_rank(const uint32_t* keys, int m, Fn fn) {
  const int t = threadIdx.x;
  const int part = t & 3;
  const int ng = (m + 3) / 4;
  const uint4* k4 = reinterpret_cast<const uint4*>(keys);
  for (int i0 = 0; i0 < m; i0 += NT / 4) {
    const int i = i0 + (t >> 2);
    const uint32_t ki = i < m ? keys[i] : 0xFFFFFFFFu;
    uint32_t gt = 0, tie = 0;
    // groups part, part+4, ...: four groups are read before any is compared
    for (int g0 = 0; g0 < ng; g0 += 16) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = g0 + 4 * u + part;
        v[u] = k4[g < ng ? g : 0];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = g0 + 4 * u + part;
        if (g < ng) {
          const uint32_t kv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            gt += kv[c] > ki ? 1u : 0u;
            tie += (kv[c] == ki && (TIES_ALL || 4 * g + c < i)) ? 1u : 0u;
          }
        }
      }
    }
    gt += dpp_u32<kDppQuadXor1>(gt);
    gt += dpp_u32<kDppQuadXor2>(gt);
    tie += dpp_u32<kDppQuadXor1>(tie);
    tie += dpp_u32<kDppQuadXor2>(tie);
    if (part == 0 && i < m) fn(i, ki, gt, tie);
  }
}

// stage_zero (may be null): the row is returned to zero at the end.
// BLOCKED: the caller guarantees n <= NT * SLOTS * 4; the row is held in the
// blocked layout. Otherwise any n, in the striped layout (streamed tile by tile
// when it does not fit one register tile).
template <int NT, int SLOTS, bool SORTED, bool COHERENT, bool BLOCKED>
__device__ __attribute__((always_inline)) void select_row(const float* row, int n, int cap, int K,
                                                         int32_t* ids_out, int32_t* count_out,
                                                         SelectSmem<NT, SLOTS, SORTED>& sm,
                                                         float* stage_zero = nullptr) {
  constexpr int NW = NT / kWave;
  constexpr int TILE = NT * SLOTS * 4;
  constexpr int E = SLOTS * NW;
  static_assert(NT >= 256 && NT % 256 == 0, "the bin scan uses the first 256 threads");
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

  uint32_t keys[SLOTS][4];
  if constexpr (BLOCKED)
    load_keys_blocked<NT, SLOTS, COHERENT>(row, n, cap, kpt4, keys);
  else if (cached)
    load_keys<NT, SLOTS, COHERENT>(row, n, cap, 0, keys);

  for (int i = t; i < 2 * kBins; i += NT) (&sm.hist[0][0])[i] = 0u;
  __syncthreads();

  // Each pass histograms the next digit of the keys that still match the
  // resolved prefix, then finds the bin holding the need-th largest of them:
  // thread t < 256 owns bins [kBins - 8(t+1), kBins - 8t), scanned from the top.
  uint32_t prefix = 0, need = (uint32_t)K, ncand = 0;
  int level = 0;  // digits resolved (kPasses = the whole key)
  bool take_all = false;
  for (int p = 0; p < kPasses; ++p) {
    const int buf = p & 1;
    uint32_t* h = sm.hist[buf];
    const int shift = digit_shift(p);
    const uint32_t dmask = digit_mask(p);
    const int hshift = p == 0 ? 0 : digit_shift(p - 1);  // the resolved bits sit above this
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;  // over this pass's active keys
    for (int tile = 0; tile < ntiles; ++tile) {
      if (!cached) load_keys<NT, SLOTS, COHERENT>(row, n, cap, tile * TILE, keys);
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (!slot_live(tile * TILE, i)) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t key = keys[i][j];
          const bool act = key != kKeyNegInf && (p == 0 || (key >> hshift) == prefix);
          hist_add(h, act, (key >> shift) & dmask);
          kmin = act && key < kmin ? key : kmin;
          kmax = act && key > kmax ? key : kmax;
        }
      }
    }
    kmin = wave_reduce_minmax<true>(kmin);
    kmax = wave_reduce_minmax<false>(kmax);
    if (lane == 0) {
      sm.wmin[w] = kmin;
      sm.wmax[w] = kmax;
    }
    __syncthreads();
    // read before the next barrier: the next pass rewrites these slots
    for (int ww = 0; ww < NW; ++ww) {
      kmin = sm.wmin[ww] < kmin ? sm.wmin[ww] : kmin;
      kmax = sm.wmax[ww] > kmax ? sm.wmax[ww] : kmax;
    }
    uint32_t c8[8], loc = 0, incl = 0;
    if (t < 256) {
      const uint4* hv = reinterpret_cast<const uint4*>(h + kBins - 8 * (t + 1));
      const uint4 lo = hv[0], hi = hv[1];
      c8[0] = hi.w; c8[1] = hi.z; c8[2] = hi.y; c8[3] = hi.x;  // descending bins
      c8[4] = lo.w; c8[5] = lo.z; c8[6] = lo.y; c8[7] = lo.x;
#pragma unroll
      for (int k = 0; k < 8; ++k) loc += c8[k];
      incl = wave_incl_scan(loc);
      if (lane == kWave - 1) sm.wsum[w] = incl;
    }
    for (int i = t; i < kBins; i += NT) sm.hist[buf ^ 1][i] = 0u;
    __syncthreads();
    if (t < 256) {
      for (int ww = 0; ww < w; ++ww) incl += sm.wsum[ww];
      uint32_t cum = incl - loc;
      if (p == 0 && t == 255) sm.n_cand = incl;
      if (cum < need && need <= incl) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (cum < need && need <= cum + c8[k]) {
            sm.sel_bin = (uint32_t)(kBins - 1 - 8 * t - k);
            sm.sel_need = need - cum;
            sm.sel_tot = c8[k];
          }
          cum += c8[k];
        }
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
    // every active key is the same value: the threshold is that key, of which
    // `need` are taken (identical keys would only fill one bin per later pass)
    if (kmin == kmax) {
      prefix = kmin;
      level = kPasses;
      break;
    }
    prefix = (prefix << (p == 2 ? 10 : 11)) | sm.sel_bin;
    need = sm.sel_need;
    level = p + 1;
    if (sm.sel_tot == need) break;  // the whole bin is taken: nothing left to resolve
  }

  // ---- emit --------------------------------------------------------------------------
  const int shiftL = take_all ? 0 : (level == 1 ? 21 : (level == 2 ? 10 : 0));
  const uint32_t m_out = take_all ? ncand : (uint32_t)K;
  auto classify = [&](uint32_t key, bool& gt, bool& eq) {
    const bool act = key != kKeyNegInf;
    const uint32_t hi = take_all ? 0u : (key >> shiftL);
    gt = act && (take_all || hi > prefix);
    eq = act && !take_all && hi == prefix;
  };
  if constexpr (BLOCKED) {
    // Blocked layout: each thread counts its taken-for-sure (gt) and threshold
    // (eq) keys, one workgroup scan of the packed counts (eq << 16 | gt; both
    // fit 16 bits since n <= 32768) gives the keys before the thread, and the
    // thread then writes its taken ids in ascending order.
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (!slot_live(0, i)) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bool gt, eq;
        classify(keys[i][j], gt, eq);
        packed += (gt ? 1u : 0u) + (eq ? 0x10000u : 0u);
      }
    }
    const uint32_t incl = wave_incl_scan(packed);
    if (lane == kWave - 1) sm.wpack[w] = incl;
    __syncthreads();
    uint32_t before = incl - packed;
    for (int ww = 0; ww < w; ++ww) before += sm.wpack[ww];
    uint32_t gb = before & 0xFFFFu, eb = before >> 16;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (!slot_live(0, i)) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bool gt, eq;
        classify(keys[i][j], gt, eq);
        const bool take = gt || (eq && eb < need);
        const uint32_t pos = gb + (eb < need ? eb : need);
        if (take && pos < m_out) {  // pos < m_out always holds; the test only bounds the store
          const int id = t * kpt4 + 4 * i + j;
          if constexpr (SORTED) {
            sm.skey[pos] = keys[i][j];
            sm.sid[pos] = id;
          } else {
            ids_out[pos] = id;
          }
        }
        gb += gt ? 1u : 0u;
        eb += eq ? 1u : 0u;
      }
    }
  }
  uint32_t carry_gt = 0, carry_eq = 0;
  for (int tile = 0; tile < (BLOCKED ? 0 : ntiles); ++tile) {
    if (!cached) {
      __syncthreads();  // the previous tile's counts have been read
      load_keys<NT, SLOTS, COHERENT>(row, n, cap, tile * TILE, keys);
    }
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      uint32_t g = 0, e = 0;
      if (slot_live(tile * TILE, i)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t key = keys[i][j];
          const bool act = key != kKeyNegInf;
          const uint32_t hi = take_all ? 0u : (key >> shiftL);
          const bool gt = act && (take_all || hi > prefix);
          const bool eq = act && !take_all && hi == prefix;
          g += popc64(ballot(gt));
          e += popc64(ballot(eq));
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
        const bool act = key != kKeyNegInf;
        const uint32_t hi = take_all ? 0u : (key >> shiftL);
        gt[j] = act && (take_all || hi > prefix);
        eq[j] = act && !take_all && hi == prefix;
        gb += mbcnt(ballot(gt[j]));
        eb += mbcnt(ballot(eq[j]));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool take = gt[j] || (eq[j] && eb < need);
        const uint32_t pos = gb + (eb < need ? eb : need);
        if (take && pos < m_out) {  // pos < m_out always holds; the test only bounds the store
          const int id = tbase + (i * NT + t) * 4 + j;
          if constexpr (SORTED) {
            sm.skey[pos] = keys[i][j];
            sm.sid[pos] = id;
          } else {
            ids_out[pos] = id;
          }
        }
        gb += gt[j] ? 1u : 0u;
        eb += eq[j] ? 1u : 0u;
      }
    }
    carry_gt += sm.tot_gt;
    carry_eq += sm.tot_eq;
  }

  for (int k = (int)m_out + t; k < K; k += NT) ids_out[k] = -1;
  if (count_out != nullptr && t == 0) *count_out = (int32_t)m_out;

  if constexpr (SORTED) {
    if (t < 4) sm.skey[m_out + t] = 0u;  // padding: below every key, never counted
    __syncthreads();
    // rank of pair i = number of pairs with a larger key, or an equal key and a
    // smaller id (pairs are stored in ascending id order)
    quad_rank<NT, false>(sm.skey, (int)m_out, [&](int i, uint32_t, uint32_t gt, uint32_t tie) {
      ids_out[gt + tie] = sm.sid[i];
    });
  }
  if (stage_zero != nullptr) {
    if (!cached) __syncthreads();  // streamed rows: every read of the row is done
    for (int i = t; i < n; i += NT) stage_zero[i] = 0.f;
  }
}

}  // namespace idxk
