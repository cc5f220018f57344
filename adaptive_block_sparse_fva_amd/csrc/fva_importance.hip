// Precise block importance, phase 2 (GSRS S5.3, A.1-A.3).
//
// After an attention call that recorded, for every kept (row, key block) pair,
// each query's log-sum-exp over that block's keys (phase 1, inside the
// attention kernel), the importance of kept block j for row (h, i) is the
// mean over the row's queries of exp(block LSE - row LSE): the share of each
// query's attention weight that falls on j's keys.  Blocks not kept get 0,
// and each row sums to 1.
#include "fva_common.h"
#include "fva_lanes.h"

namespace fva {

// One workgroup per (head, query block) row.  The row's block LSEs are one
// contiguous run of (kept pairs) x BLK floats; the workgroup streams it with
// 16-byte loads, BLK/4 lanes per pair, PF passes of pairs with their loads
// in flight together, and reduces each pair inside its lane group with DPP /
// permlane exchanges.
template <int BLK>
__global__ __launch_bounds__(256) void block_importance_kernel(const int32_t* __restrict__ order,
                                                              const int32_t* __restrict__ row_ptr,
                                                              const int32_t* __restrict__ col_idx,
                                                              const float* __restrict__ lse,
                                                              const float* __restrict__ block_lse, int n, int nb,
                                                              float* __restrict__ importance) {
  constexpr int LPP = BLK / 4;    // lanes per pair
  constexpr int PPI = 256 / LPP;  // pairs per pass
  constexpr int PF = 8;           // passes per batch of loads
  __shared__ float row_lse[BLK];
  const int t = blockIdx.x, h = t / nb, i = t - h * nb;
  const int tid = threadIdx.x;
  const int c0 = row_ptr[t], c1 = row_ptr[t + 1];
  const int g = tid / LPP, r = (tid % LPP) * 4;
  // the first batch of block LSEs is loaded before (and independently of)
  // the row LSE gather
  f32x4 x[PF];
  auto load_batch = [&](int cb) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int c = cb + k * PPI + g;
      x[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c < c1) x[k] = *reinterpret_cast<const f32x4*>(block_lse + (int64_t)c * BLK + r);
    }
  };
  load_batch(c0);
  for (int qq = tid; qq < BLK; qq += 256) {
    const int tok = order[i * BLK + qq];
    row_lse[qq] = tok >= 0 ? lse[(int64_t)h * n + tok] : INFINITY;  // exp(x - inf) = 0 for slots past N
  }
  float* out = importance + (int64_t)t * nb;
  for (int j = tid; j < nb; j += 256) out[j] = 0.f;
  __syncthreads();
  const float inv_rows = 1.0f / (float)min(BLK, n - i * BLK);
  // exp(x - l) as 2^(x log2 e - l log2 e): one FMA and one exp2 per element
  constexpr float LOG2E = 1.44269504088896341f;
  const float l0 = row_lse[r] * LOG2E, l1 = row_lse[r + 1] * LOG2E, l2 = row_lse[r + 2] * LOG2E,
              l3 = row_lse[r + 3] * LOG2E;
  for (int cb = c0; cb < c1; cb += PF * PPI) {
    if (cb > c0) load_batch(cb);
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int c = cb + k * PPI + g;  // the same for the LPP lanes of a pair
      float acc = __builtin_amdgcn_exp2f(fmaf(x[k][0], LOG2E, -l0)) + __builtin_amdgcn_exp2f(fmaf(x[k][1], LOG2E, -l1)) +
                  __builtin_amdgcn_exp2f(fmaf(x[k][2], LOG2E, -l2)) + __builtin_amdgcn_exp2f(fmaf(x[k][3], LOG2E, -l3));
      static_for<0, __builtin_ctz(LPP)>([&](auto sl) {
        constexpr int M = LPP >> (decltype(sl)::value + 1);
        acc += __uint_as_float(xor_lane<M>(__float_as_uint(acc)));
      });
      if (c < c1 && tid % LPP == 0) out[col_idx[c]] = acc * inv_rows;
    }
  }
}

int launch_block_importance(const fva_problem& p, int nb, const int32_t* order, const int32_t* row_ptr,
                            const int32_t* col_idx, const float* lse, const float* block_lse,
                            float* importance, hipStream_t stream) {
  const int rows = p.num_heads * nb;
  if (p.block == 128)
    block_importance_kernel<128><<<rows, 256, 0, stream>>>(order, row_ptr, col_idx, lse, block_lse, p.seq_len, nb,
                                                           importance);
  else
    block_importance_kernel<64><<<rows, 256, 0, stream>>>(order, row_ptr, col_idx, lse, block_lse, p.seq_len, nb,
                                                          importance);
  return record_hip_error(hipGetLastError(), "block_importance launch");
}

}  // namespace fva
