// Plan kernels: one-GPU slack refill, CSR block mask, heaviest-first tile order.
//
// FVAttn paper S3.2: once the mask is materialised the per-head work is known
// and the placement of work is repaired without changing which blocks are
// computed.  On one GPU the placement is the order in which (head, query-block)
// tiles are handed to compute units: longest first, so that the heavy heads do
// not finish last.  S3.3: slack is turned into extra blocks taken, in the
// routing's own ranking, after the ones already kept (no re-sort, no
// re-scoring); here every row gets e_i = min(nb - k_i, k_i * refill / 1000).
#include "fva_common.h"

namespace fva {

constexpr int PLAN_THREADS = 1024;

__device__ __forceinline__ int refill_count(int k, int nb, int refill_per_mille) {
  return k + min(nb - k, (k * refill_per_mille) / 1000);
}

// One workgroup: final counts, CSR row offsets, per-head totals, LPT order,
// queue reset.  Rows (tiles) are at most FVA_MAX_TILES = 16384.
__global__ __launch_bounds__(PLAN_THREADS) void plan_scan_kernel(
    const int32_t* __restrict__ row_count, int rows, int rpad, int nb,
    int refill_per_mille, int32_t* __restrict__ row_ptr,
    int32_t* __restrict__ head_count_final, int32_t* __restrict__ tile_order,
    uint32_t* __restrict__ tile_counter) {
  __shared__ uint32_t keys[FVA_MAX_TILES];
  __shared__ int32_t wave_tot[PLAN_THREADS / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // per-thread contiguous chunk of rows
  const int per = (rows + PLAN_THREADS - 1) / PLAN_THREADS;
  const int r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
  int local = 0;
  for (int r = r0; r < r1; ++r) local += refill_count(row_count[r], nb, refill_per_mille);

  // exclusive scan of the chunk sums across the workgroup
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  int run = base + incl - local;

  // row offsets, sort keys ((2048 - k') << 14 | tile) and per-head totals
  int head_acc = 0, head_cur = (r0 < r1) ? r0 / nb : -1;
  for (int r = r0; r < r1; ++r) {
    const int kp = refill_count(row_count[r], nb, refill_per_mille);
    row_ptr[r] = run;
    run += kp;
    keys[r] = ((uint32_t)(FVA_MAX_BLOCKS - kp) << 14) | (uint32_t)r;
    const int hh = r / nb;
    if (hh != head_cur) {
      atomicAdd(&head_count_final[head_cur], head_acc);
      head_cur = hh;
      head_acc = 0;
    }
    head_acc += kp;
  }
  if (head_cur >= 0 && head_acc > 0) atomicAdd(&head_count_final[head_cur], head_acc);
  if (r1 == rows && r0 < r1) row_ptr[rows] = run;
  if (rows == 0 && tid == 0) row_ptr[0] = 0;
  for (int r = rows + tid; r < rpad; r += PLAN_THREADS) keys[r] = 0xffffffffu;
  __syncthreads();

  // bitonic sort, ascending keys = k' descending, then tile id ascending
  for (int kk = 2; kk <= rpad; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < (rpad >> 1); i += PLAN_THREADS) {
        const int lo = ((i & ~(jj - 1)) << 1) | (i & (jj - 1));
        const int hi = lo | jj;
        const uint32_t a = keys[lo], b = keys[hi];
        const bool asc = (lo & kk) == 0;
        if ((a > b) == asc) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < rows; r += PLAN_THREADS) tile_order[r] = (int32_t)(keys[r] & 0x3fffu);
  if (tid == 0) {
    atomicExch(&tile_counter[0], 0u);
    atomicExch(&tile_counter[1], 0u);
  }
}

// Clears the per-head totals before plan_scan accumulates into them.
__global__ void plan_clear_kernel(int32_t* __restrict__ head_count_final, int num_heads) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < num_heads; i += gridDim.x * blockDim.x)
    head_count_final[i] = 0;
}

// One workgroup per row: mark the first k'_i ranked key blocks in an LDS
// bitmap, then emit their ids in ascending order at the row's CSR offset.
__global__ __launch_bounds__(256) void plan_fill_kernel(
    const int16_t* __restrict__ ranked, const int32_t* __restrict__ row_ptr, int nb,
    int32_t* __restrict__ col_idx) {
  __shared__ uint32_t bits[FVA_MAX_BLOCKS / 32];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int start = row_ptr[row];
  const int kp = row_ptr[row + 1] - start;
  int32_t* out = col_idx + start;
  if (kp >= nb) {
    for (int j = tid; j < nb; j += 256) out[j] = j;
    return;
  }
  const int nwords = (nb + 31) >> 5;
  for (int w = tid; w < nwords; w += 256) bits[w] = 0u;
  __syncthreads();
  const int16_t* rk = ranked + (int64_t)row * nb;
  for (int r = tid; r < kp; r += 256) {
    const int j = rk[r];
    atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  if (tid < 64) {
    // each lane owns words lane, lane+64, ... ; nwords <= 64 for nb <= 2048
    const uint32_t word = (tid < nwords) ? bits[tid] : 0u;
    const int cnt = __popc(word);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (tid >= off) incl += y;
    }
    int pos = incl - cnt;
    uint32_t w = word;
    while (w) {
      const int b = __ffs(w) - 1;
      out[pos++] = tid * 32 + b;
      w &= w - 1;
    }
  }
}

int launch_plan(const fva_problem& p, int nb, const int16_t* ranked,
                const int32_t* row_count, int32_t* row_ptr, int32_t* col_idx,
                int32_t* head_count_final, int32_t* tile_order,
                uint32_t* tile_counter, hipStream_t stream) {
  const int rows = p.num_heads * nb;
  int rpad = 2;
  while (rpad < rows) rpad <<= 1;
  plan_clear_kernel<<<(p.num_heads + 255) / 256, 256, 0, stream>>>(head_count_final, p.num_heads);
  int st = record_hip_error(hipGetLastError(), "plan_clear launch");
  if (st) return st;
  plan_scan_kernel<<<1, PLAN_THREADS, 0, stream>>>(row_count, rows, rpad, nb, p.refill_per_mille,
                                                   row_ptr, head_count_final, tile_order,
                                                   tile_counter);
  st = record_hip_error(hipGetLastError(), "plan_scan launch");
  if (st) return st;
  plan_fill_kernel<<<rows, 256, 0, stream>>>(ranked, row_ptr, nb, col_idx);
  return record_hip_error(hipGetLastError(), "plan_fill launch");
}

}  // namespace fva
