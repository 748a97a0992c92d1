// Device helpers shared by the indexer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxk {

constexpr int kWave = 64;
constexpr int kHeadDim = 128;

// ---- bf16 -------------------------------------------------------------------------------
// A bf16 value is the upper half of an fp32 value; widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- order keys -------------------------------------------------------------------------
// Unsigned keys whose integer order is the numeric order of the fp32 scores
// ("Round 18 Track C", section 1 Target 1: the radix passes run over uint keys).
// Negative values have all bits flipped, non-negative ones get the sign bit set;
// -0.0 is first mapped to +0.0 so that equal scores have equal keys.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;  // order_key(-inf): never a candidate

// Radix digits of the keys, most significant first: 11 + 11 + 10 bits, so a row
// is resolved in at most three histogram passes over 2048 bins.
constexpr int kBins = 2048;
constexpr int kDigit0Shift = 21;  // the first digit is key >> 21

// ---- buffer loads ----------------------------------------------------------------------
// Fourth dword of a raw buffer resource (32-bit data format) and the cache
// policy bit that makes a load device-coherent (sc1: bypasses stale L2 lines of
// other XCDs).
constexpr int kBufferDword3 = 0x00020000;
constexpr int kCachePolicySc1 = 16;

// ---- wave primitives --------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of m in lanes below the calling lane
__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

template <typename T>
__device__ __forceinline__ T readlane(T v, int l);
template <>
__device__ __forceinline__ uint32_t readlane<uint32_t>(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Data-parallel-primitive lane moves (DPP, GFX9 encodings): each reads another
// lane's register inside the VALU, with no trip through LDS.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowShl1 = 0x101;    // row_shl:n = 0x100 + n: lane l <- lane l + n of its row
constexpr int kDppRowShr1 = 0x111;    // row_shr:n = 0x110 + n: lane l <- lane l - n of its row
constexpr int kDppRowRor1 = 0x121;    // row_ror:n = 0x120 + n: rotation within the row
constexpr int kDppRowMirror = 0x140;  // lane i <- lane 15-i of its row
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i of its half row
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of a row -> the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> rows 2 and 3

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  // lanes whose source is outside the row, or whose row is masked off, read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// The value of lane (lane ^ M) for M a power of two below 64, without LDS:
// DPP within a 16-lane row (quad permutes, row shifts, row rotation) and the
// gfx950 row-swap permutes across rows.
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (M == 1) {
    return dpp_u32<kDppQuadXor1>(v);
  } else if constexpr (M == 2) {
    return dpp_u32<kDppQuadXor2>(v);
  } else if constexpr (M == 4) {
    const uint32_t up = dpp_u32<kDppRowShl1 + 3>(v);  // lane l + 4
    const uint32_t dn = dpp_u32<kDppRowShr1 + 3>(v);  // lane l - 4
    return (lane_id() & 4) ? dn : up;
  } else if constexpr (M == 8) {
    return dpp_u32<kDppRowRor1 + 7>(v);  // rotation by 8 within the row
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane_id() & 16) ? r[0] : r[1];
  } else {
    static_assert(M == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane_id() & 32) ? r[0] : r[1];
  }
}

// inclusive prefix sum over the 64 lanes of a wave (row scans, then the row
// totals carried across rows by broadcasts)
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_u32<kDppRowShr1>(v);
  v += dpp_u32<kDppRowShr1 + 1>(v);
  v += dpp_u32<kDppRowShr1 + 3>(v);  // row_shr:4 (lanes 0..3 see 0)
  v += dpp_u32<kDppRowShr1 + 7>(v);  // row_shr:8
  v += dpp_u32<kDppRowBcast15, 0xA>(v);
  v += dpp_u32<kDppRowBcast31, 0xC>(v);
  return v;
}

// min / max over the 64 lanes of a wave (returned in every lane)
template <bool IS_MIN>
__device__ __forceinline__ uint32_t wave_reduce_minmax(uint32_t v) {
  const int ident = IS_MIN ? -1 : 0;  // lanes without a source keep the identity
  auto op = [](uint32_t a, uint32_t b) { return IS_MIN ? (a < b ? a : b) : (a > b ? a : b); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, kDppRowShr1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, kDppRowShr1 + 1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, kDppRowShr1 + 3, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, kDppRowShr1 + 7, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, kDppRowBcast15, 0xA, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, kDppRowBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// sum over groups of 16 consecutive lanes; every lane of a group gets the same
// value (the pairings are symmetric, so each lane adds the same operands)
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  return v;
}

// sum over the 64 lanes of a wave (returned in every lane)
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = sum16(v);
  v += __uint_as_float(lane_xor<16>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<32>(__float_as_uint(v)));
  return v;
}

__device__ __forceinline__ int n_valid_blocks(int seq_len, int page_size, int n_pad) {
  long long s = seq_len < 0 ? 0 : seq_len;
  long long nv = (s + page_size - 1) / page_size;
  return (int)(nv < n_pad ? nv : n_pad);
}

}  // namespace idxk
