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

// Radix digits of the 32-bit keys, most significant first: 11 + 11 + 10 bits,
// so a row is resolved in at most three histogram passes over 2048 bins.
constexpr int kPasses = 3;
constexpr int kCandCap = 512;  // threshold-bin keys resolved by counting instead of passes
constexpr int kBins = 2048;
__device__ __forceinline__ int digit_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int p) { return p == 2 ? 0x3FFu : 0x7FFu; }

template <int NT, int SLOTS, bool SORTED>
struct SelectSmem {
  static constexpr int NW = NT / kWave;
  static constexpr int E = SLOTS * NW;  // emit-count entries per tile
  uint32_t hist[2][kBins];
  uint32_t wsum[4];
  uint32_t sel_bin, sel_need, sel_tot, n_cand;
  uint32_t cgt[E], ceq[E];
  uint32_t tot_gt, tot_eq;
  uint32_t n_in_bin, thr_key, thr_need;
  alignas(16) uint32_t cand[kCandCap + 8];
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
  const bool vec = !COHERENT && (((uintptr_t)row & 15) == 0) && (cap & 3) == 0;
  if (vec) {
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

// add one count per active lane to h[digit]
__device__ __forceinline__ void hist_add(uint32_t* h, bool act, uint32_t digit) {
  const uint64_t m = ballot(act);
  if (m == 0) return;
  const int leader = __builtin_ctzll(m);
  const uint32_t d0 = readlane<uint32_t>(digit, leader);
  const bool same = act && digit == d0;
  const uint64_t sm = ballot(same);
  if (lane_id() == leader) atomicAdd(&h[d0], popc64(sm));
  if (act && !same) atomicAdd(&h[digit], 1u);
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

// Select the top-K of row[0..n) into ids_out[0..K); *count_out = number selected.
// row[0..cap) may be read (cap >= n).
// All NT threads of the workgroup must call this together.
template <int NT, int SLOTS, bool SORTED, bool COHERENT = false>
__device__ __attribute__((always_inline)) void select_row(const float* row, int n, int cap, int K,
                                                         int32_t* ids_out, int32_t* count_out,
                                                         SelectSmem<NT, SLOTS, SORTED>& sm) {
  constexpr int NW = NT / kWave;
  constexpr int TILE = NT * SLOTS * 4;
  constexpr int E = SLOTS * NW;
  static_assert(NT >= 256 && NT % 256 == 0, "the bin scan uses the first 256 threads");
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int lane = t & (kWave - 1);
  const int ntiles = (n + TILE - 1) / TILE;
  const bool cached = ntiles <= 1;
  // slots of a tile that hold no entry of the row, for any thread, are skipped
  auto slot_live = [&](int base, int i) { return base + i * NT * 4 < n; };

  uint32_t keys[SLOTS][4];
  if (cached) load_keys<NT, SLOTS, COHERENT>(row, n, cap, 0, keys);

  for (int i = t; i < 2 * kBins; i += NT) (&sm.hist[0][0])[i] = 0u;
  if (t == 0) sm.n_in_bin = 0u;
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
        }
      }
    }
    __syncthreads();
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
    prefix = (prefix << (p == 2 ? 10 : 11)) | sm.sel_bin;
    need = sm.sel_need;
    level = p + 1;
    const uint32_t in_bin = sm.sel_tot;
    if (in_bin == need) break;  // the whole bin is taken: nothing left to resolve
    if (p == 0 && in_bin <= (uint32_t)kCandCap && ntiles <= 1) {
      // Few keys share the threshold bin: gather them in LDS and find the
      // need-th largest directly by counting, instead of two more passes.
      uint32_t cnt[SLOTS * 4], tot = 0;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t key = keys[i][j];
          const uint64_t m = slot_live(0, i) ? ballot(key != kKeyNegInf && (key >> 21) == prefix)
                                             : 0ull;
          cnt[i * 4 + j] = (uint32_t)(m != 0);  // reuse: 1 if any lane of the wave is in the bin
          tot += popc64(m);
        }
      }
      uint32_t base = 0;
      if (tot != 0) {
        if (lane == 0) base = atomicAdd(&sm.n_in_bin, tot);
        base = readlane<uint32_t>(base, 0);
      }
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cnt[i * 4 + j] == 0u) continue;
          const uint32_t key = keys[i][j];
          const bool inb = key != kKeyNegInf && (key >> 21) == prefix;
          const uint64_t m = ballot(inb);
          if (inb) sm.cand[base + mbcnt(m)] = key;
          base += popc64(m);
        }
      }
      if (t < 4) sm.cand[in_bin + t] = 0u;  // padding: 0 is below every key
      __syncthreads();
      // the need-th largest candidate key T, and how many keys equal to T to take
      const uint4* c4 = reinterpret_cast<const uint4*>(sm.cand);
      for (int i = t; i < (int)in_bin; i += NT) {
        const uint32_t ki = sm.cand[i];
        uint32_t gt = 0, ge = 0;
        const int ng = (int)(in_bin + 3) / 4;
#pragma unroll 8
        for (int j = 0; j < ng; ++j) {
          const uint4 v = c4[j];
          gt += (v.x > ki) + (v.y > ki) + (v.z > ki) + (v.w > ki);
          ge += (v.x >= ki) + (v.y >= ki) + (v.z >= ki) + (v.w >= ki);
        }
        if (gt < need && need <= ge) {  // every candidate equal to T writes the same
          sm.thr_key = ki;
          sm.thr_need = need - gt;
        }
      }
      __syncthreads();
      prefix = sm.thr_key;
      need = sm.thr_need;
      level = kPasses;
      break;
    }
  }

  // ---- emit --------------------------------------------------------------------------
  const int shiftL = take_all ? 0 : (level == 1 ? 21 : (level == 2 ? 10 : 0));
  const uint32_t m_out = take_all ? ncand : (uint32_t)K;
  uint32_t carry_gt = 0, carry_eq = 0;
  for (int tile = 0; tile < ntiles; ++tile) {
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
    const uint4* k4 = reinterpret_cast<const uint4*>(sm.skey);
    for (int i = t; i < (int)m_out; i += NT) {
      const uint32_t ki = sm.skey[i];
      uint32_t r = 0;
      const int full = i / 4;  // groups entirely below i: ties count
#pragma unroll 8
      for (int j = 0; j < full; ++j) {
        const uint4 v = k4[j];
        r += (v.x >= ki) + (v.y >= ki) + (v.z >= ki) + (v.w >= ki);
      }
      {
        const uint4 v = k4[full];  // the group holding i
        const uint32_t kv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = full * 4 + c;
          r += (kv[c] > ki || (kv[c] == ki && j < i)) ? 1u : 0u;
        }
      }
      const int ng = (int)(m_out + 3) / 4;
#pragma unroll 8
      for (int j = full + 1; j < ng; ++j) {
        const uint4 v = k4[j];
        r += (v.x > ki) + (v.y > ki) + (v.z > ki) + (v.w > ki);
      }
      ids_out[r] = sm.sid[i];
    }
  }
}

}  // namespace idxk
