// Lane exchanges inside one wave64 without going through LDS.
#pragma once

#include <type_traits>

#include "fva_common.h"

namespace fva {

// Value of lane l ^ M (M a power of two below 64) without going through
// LDS: DPP quad permutations for 1 and 2; for 4 the half-row mirror (l ^ 7)
// then l ^ 3, for 8 the row mirror (l ^ 15) then the half-row mirror; for 16
// and 32 the permlane swaps of x with itself, whose two results hold this
// lane's and its partner's values in some order (so their sum minus x, in
// wrapping integer arithmetic, is the partner's).
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
  const int v = (int)x;
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, false);
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, false);
  } else if constexpr (M == 4) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, false), 0x1B, 0xf, 0xf,
                                              false);
  } else if constexpr (M == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x140, 0xf, 0xf, false), 0x141, 0xf,
                                              0xf, false);
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return r[0] + r[1] - x;
  } else {
    static_assert(M == 32, "lane xor below 64");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return r[0] + r[1] - x;
  }
}

template <int M>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t x) {
  return ((uint64_t)xor_lane<M>((uint32_t)(x >> 32)) << 32) | xor_lane<M>((uint32_t)x);
}

// Inclusive prefix sums over the wave's 64 lanes (lane order): DPP row
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes (a lane whose source
// lies before its row's start adds 0), then the totals of rows 0..2, read
// from lanes 15, 31 and 47, added to every lane of the rows after them.
template <int S>
__device__ __forceinline__ uint32_t dpp_row_shr(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x110 + S, 0xf, 0xf, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
  x += dpp_row_shr<1>(x);
  x += dpp_row_shr<2>(x);
  x += dpp_row_shr<4>(x);
  x += dpp_row_shr<8>(x);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  return x + (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
}
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x, int lane) {
  auto shr = [](uint64_t v, auto s) {
    constexpr int S = decltype(s)::value;
    return ((uint64_t)dpp_row_shr<S>((uint32_t)(v >> 32)) << 32) | dpp_row_shr<S>((uint32_t)v);
  };
  x += shr(x, std::integral_constant<int, 1>{});
  x += shr(x, std::integral_constant<int, 2>{});
  x += shr(x, std::integral_constant<int, 4>{});
  x += shr(x, std::integral_constant<int, 8>{});
  auto lane_value = [&](int l) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  };
  const uint64_t r0 = lane_value(15), r1 = lane_value(31), r2 = lane_value(47);
  return x + (lane >= 16 ? r0 : 0ull) + (lane >= 32 ? r1 : 0ull) + (lane >= 48 ? r2 : 0ull);
}

// One bitonic compare-exchange of a 64-bit key with the key of lane l ^ M:
// the larger of the two where keep_larger, else the smaller.  For M = 16 and
// 32 the permlane swaps of the key's two halves with themselves leave both
// keys in every lane (the two results of each swap come from the same pair of
// lanes, in an order that depends on the lane), and the larger or smaller of
// a pair does not depend on that order.
template <int M>
__device__ __forceinline__ uint64_t exchange_keep(uint64_t a, bool keep_larger) {
  if constexpr (M == 16 || M == 32) {
    const uint32_t hi = (uint32_t)(a >> 32), lo = (uint32_t)a;
    const auto h = M == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                           : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const auto l = M == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                           : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const uint64_t x0 = ((uint64_t)h[0] << 32) | l[0], x1 = ((uint64_t)h[1] << 32) | l[1];
    return ((x0 > x1) == keep_larger) ? x0 : x1;
  } else {
    const uint64_t b = xor_lane_u64<M>(a);
    return ((a > b) == keep_larger) ? a : b;
  }
}

}  // namespace fva
