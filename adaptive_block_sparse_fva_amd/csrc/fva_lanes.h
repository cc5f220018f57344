// Lane exchanges inside one wave64 without going through LDS.
#pragma once

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

}  // namespace fva
