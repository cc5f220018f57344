// Plan kernels: one-GPU slack refill, CSR block mask, heaviest-first work list.
//
// FVAttn paper S3.2: once the mask is materialised the per-head work is known
// and the placement of work is repaired without changing which blocks are
// computed.  On one GPU the placement is the order in which (head, query-block)
// tiles are handed to compute units: longest first, so that the heavy heads do
// not finish last.  S3.3: slack is turned into extra blocks taken, in the
// routing's own ranking, after the ones already kept (no re-sort, no
// re-scoring); here every row gets e_i = min(nb - k_i, k_i * f / 1000), with
// f one value for the call or one per head (a budget turned into a refill).
#include "fva_common.h"
#include "fva_lanes.h"

namespace fva {

constexpr int PLAN_THREADS = 1024;
constexpr int FILL_WGS_MAX = 1024;  // CSR fill workgroups of the plan launch

__device__ __forceinline__ int refill_count(int k, int nb, int f) {
  return k + (int)min((int64_t)(nb - k), (int64_t)k * f / 1000);
}

// refill per mille of the head that row r belongs to
__device__ __forceinline__ int row_refill(const int32_t* __restrict__ head_refill, int r, int nb,
                                          int refill_per_mille) {
  if (!head_refill) return refill_per_mille;
  return min(max(head_refill[r / nb], 0), FVA_MAX_HEAD_REFILL);
}

// Sort key of a work item: length descending, then tile, then part.
__device__ __forceinline__ uint32_t item_key(int len, int tile, int part) {
  return ((uint32_t)(FVA_MAX_BLOCKS - len) << 15) | ((uint32_t)tile << 1) | (uint32_t)part;
}

// NS consecutive stages of bitonic merge level kk, compare distances jj,
// jj/2, .., jj >> (NS-1), done as one round: the 2^NS elements whose indices
// differ only in those NS bits form a group that the stages never leave, and
// they share the level's direction bit (kk lies above jj), so a thread loads
// a group into registers, applies the NS stages in order and writes it back.
// Same compare-exchanges as the stage-by-stage network, one LDS round trip
// and one barrier per round.
template <int NS>
__device__ __forceinline__ void sort_round(uint32_t* keys, int ipad, int kk, int jj, int tid) {
  constexpr int G = 1 << NS;
  const int low = jj >> (NS - 1);
  for (int g = tid; g < (ipad >> NS); g += PLAN_THREADS) {
    const int base = ((g & ~(low - 1)) << NS) | (g & (low - 1));
    const bool asc = (base & kk) == 0;
    uint32_t v[G];
#pragma unroll
    for (int m = 0; m < G; ++m) v[m] = keys[base + m * low];
#pragma unroll
    for (int st = NS - 1; st >= 0; --st)
#pragma unroll
      for (int m = 0; m < G; ++m)
        if (!(m & (1 << st))) {
          const uint32_t a = v[m], b = v[m | (1 << st)];
          const uint32_t lo = a < b ? a : b, hi = a < b ? b : a;
          v[m] = asc ? lo : hi;
          v[m | (1 << st)] = asc ? hi : lo;
        }
#pragma unroll
    for (int m = 0; m < G; ++m) keys[base + m * low] = v[m];
  }
  __syncthreads();
}

// Stages J0, J0/2, .., 1 of bitonic merge level kk on one wave's chunk of
// 128 keys at offset base, held two per lane (chunk slot 64e + lane in
// v[e]): distance 64 pairs a lane's two keys, smaller distances pair lanes
// (DPP / permlane exchanges).  Every such stage stays inside the chunk.
template <int J0>
__device__ __forceinline__ void chunk_stages(uint32_t (&v)[2], int lane, int base, int kk) {
  static_for<0, __builtin_ctz(J0) + 1>([&](auto sl) {
    constexpr int JJ = J0 >> decltype(sl)::value;
    if constexpr (JJ == 64) {
      const bool asc = ((base + lane) & kk) == 0;
      const uint32_t x = v[0], y = v[1];
      const bool keep = (x < y) == asc;  // the pair is already in this chunk's order
      v[0] = keep ? x : y;
      v[1] = keep ? y : x;
    } else {
      const bool lower = (lane & JJ) == 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool asc = ((base + 64 * e + lane) & kk) == 0;
        const uint32_t a = v[e], b = xor_lane<JJ>(a);
        // the lower side of an ascending pair keeps the smaller key: one
        // compare picks between a and b
        v[e] = ((a < b) == (lower == asc)) ? a : b;
      }
    }
  });
}

// One workgroup: final counts, CSR row offsets, per-head totals, the split
// decision, the heaviest-first work list, queue reset.  Rows (tiles) are at
// most FVA_MAX_TILES = 16384, work items at most rows + FVA_MAX_SPLITS.
//
// Placement on one GPU: with a = ceil(sum k' / split_s) and split_s = half
// the compute units (a / 2 is then about the mean load of one unit), a tile
// with k' >= 2 and 2 k' > a is cut into two work items (its first ceil(k'/2)
// kept blocks, then the rest), since no ordering can balance a single item
// larger than a unit's mean load.  Split tiles get slots 0, 1, ... in tile-id
// order.  Fewer than 2 * split_s tiles can qualify, and
// split_s <= FVA_MAX_SPLITS / 2.
__device__ __forceinline__ void plan_scan(
    const int32_t* __restrict__ row_count, const int32_t* __restrict__ head_refill, int rows, int nb,
    int refill_per_mille, int split_s,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ head_count_final,
    int32_t* __restrict__ work_order, int32_t* __restrict__ plan_meta,
    uint32_t* __restrict__ tile_counter) {
  // at most FVA_MAX_TILES + FVA_MAX_SPLITS - 1 items, padded to a power of two
  static_assert(FVA_MAX_SPLITS <= FVA_MAX_TILES, "item list fits the padded sort");
  extern __shared__ uint32_t keys[];  // sized by the launch to the padded item count
  __shared__ int32_t wave_tot[PLAN_THREADS / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // exclusive scan across the workgroup; *total gets the sum
  auto block_scan = [&](int x, int* total) {
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < PLAN_THREADS / 64; ++w) {
      if (w < wave) base += wave_tot[w];
      tot += wave_tot[w];
    }
    __syncthreads();
    *total = tot;
    return base + incl - x;
  };

  auto kept = [&](int r) {
    return refill_count(row_count[r], nb, row_refill(head_refill, r, nb, refill_per_mille));
  };

  // per-thread contiguous chunk of rows
  const int per = (rows + PLAN_THREADS - 1) / PLAN_THREADS;
  const int r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
  int local = 0;
  for (int r = r0; r < r1; ++r) local += kept(r);
  int total = 0;
  int run = block_scan(local, &total);

  // row offsets, then per-head totals from them (the stores are complete and
  // visible to the workgroup after the barrier inside the next scan)
  for (int r = r0; r < r1; ++r) {
    row_ptr[r] = run;
    run += kept(r);
  }
  if (r1 == rows && r0 < r1) row_ptr[rows] = run;

  // split decision and slots
  const int mean = (total + split_s - 1) / split_s;
  auto is_split = [&](int kp) { return kp >= 2 && 2 * kp > mean; };
  int nsp = 0;
  for (int r = r0; r < r1; ++r) nsp += is_split(kept(r)) ? 1 : 0;
  int nsplit = 0;
  int sp = block_scan(nsp, &nsplit);
  for (int hh = tid; hh < rows / nb; hh += PLAN_THREADS)
    head_count_final[hh] = row_ptr[(hh + 1) * nb] - row_ptr[hh * nb];

  // work items: tile r's items start at r + (split tiles before r)
  for (int r = r0; r < r1; ++r) {
    const int kp = kept(r);
    const int pos = r + sp;
    if (is_split(kp)) {
      plan_meta[2 + r] = sp;
      plan_meta[2 + rows + sp] = r;
      keys[pos] = item_key((kp + 1) >> 1, r, 0);
      keys[pos + 1] = item_key(kp >> 1, r, 1);
      ++sp;
    } else {
      plan_meta[2 + r] = -1;
      keys[pos] = item_key(kp, r, 0);
    }
  }
  const int nitems = rows + nsplit;
  int ipad = 128;
  while (ipad < nitems) ipad <<= 1;
  for (int x = nitems + tid; x < ipad; x += PLAN_THREADS) keys[x] = 0xffffffffu;
  __syncthreads();

  // bitonic sort of the item keys, ascending.  Merge levels 2 .. 128 stay
  // inside 128-key chunks: each wave sorts its chunks in registers.  Every
  // later level kk runs its stages of distance >= 128 over the whole list in
  // LDS rounds (sort_round, up to three stages each) and the rest inside the
  // chunks again, so that the workgroup synchronises only between those.
  const int nchunks = ipad >> 7;
  for (int c = wave; c < nchunks; c += PLAN_THREADS / 64) {
    uint32_t v[2] = {keys[128 * c + lane], keys[128 * c + 64 + lane]};
    static_for<1, 8>([&](auto kl) {
      constexpr int KK = 1 << decltype(kl)::value;
      chunk_stages<KK / 2>(v, lane, 128 * c, KK);
    });
    keys[128 * c + lane] = v[0];
    keys[128 * c + 64 + lane] = v[1];
  }
  __syncthreads();
  for (int kk = 256; kk <= ipad; kk <<= 1) {
    int jj = kk >> 1;
    for (; jj >= 512; jj >>= 3) sort_round<3>(keys, ipad, kk, jj, tid);
    if (jj == 256) sort_round<2>(keys, ipad, kk, 256, tid);
    else if (jj == 128) sort_round<1>(keys, ipad, kk, 128, tid);
    for (int c = wave; c < nchunks; c += PLAN_THREADS / 64) {
      uint32_t v[2] = {keys[128 * c + lane], keys[128 * c + 64 + lane]};
      chunk_stages<64>(v, lane, 128 * c, kk);
      keys[128 * c + lane] = v[0];
      keys[128 * c + 64 + lane] = v[1];
    }
    __syncthreads();
  }
  for (int x = tid; x < nitems; x += PLAN_THREADS) work_order[x] = (int32_t)(keys[x] & 0x7fffu);
  if (tid == 0) {
    plan_meta[0] = nitems;
    plan_meta[1] = nsplit;
    atomicExch(&tile_counter[0], 0u);
    atomicExch(&tile_counter[1], 0u);
  }
}

// CSR column fill, four rows per workgroup (a quarter of it per row): mark
// the first k'_i ranked key blocks in an LDS bitmap, then emit their ids in
// ascending order at the row's CSR offset.  The workgroup computes the
// offsets itself, the sum of k' over the rows before its first row (the same
// integers the scan adds), so it does not wait for the scan.
__device__ __forceinline__ void plan_fill(const int16_t* __restrict__ ranked, const int32_t* __restrict__ row_count,
                                          const int32_t* __restrict__ head_refill, int rows, int nb,
                                          int refill_per_mille, int first, int last,
                                          int32_t* __restrict__ col_idx) {
  __shared__ uint32_t bits[4][FVA_MAX_BLOCKS / 32];
  __shared__ int32_t wave_sum[PLAN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qr = tid >> 8, qt = tid & 255;  // quarter (row) and thread in it
  auto kept = [&](int r) {
    return refill_count(row_count[r], nb, row_refill(head_refill, r, nb, refill_per_mille));
  };
  int part = 0;
  for (int r = tid; r < first; r += PLAN_THREADS) part += kept(r);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
  if (lane == 0) wave_sum[wave] = part;
  __syncthreads();
  int base = 0;  // CSR offset of row r0 below
#pragma unroll
  for (int w = 0; w < PLAN_THREADS / 64; ++w) base += wave_sum[w];
  const int nwords = (nb + 31) >> 5;
  for (int r0 = first; r0 < last; r0 += 4) {
    const int row = r0 + qr;
    int start = base, kp = 0;
    for (int r = r0; r < r0 + 4 && r < rows; ++r) {
      const int k = kept(r);
      if (r < row) start += k;
      if (r == row) kp = k;
      base += k;
    }
    const bool live = row < last;
    const bool full = kp >= nb;
    for (int w = qt; w < nwords; w += 256) bits[qr][w] = 0u;
    __syncthreads();
    if (live && !full) {
      const int16_t* rk = ranked + (int64_t)row * nb;
      for (int r = qt; r < kp; r += 256) {
        const int j = rk[r];
        atomicOr(&bits[qr][j >> 5], 1u << (j & 31));
      }
    }
    __syncthreads();
    int32_t* out = col_idx + start;
    if (live && full) {
      for (int j = qt; j < nb; j += 256) out[j] = j;
    } else if (live && qt < 64) {
      // each lane owns one word; nwords <= 64 for nb <= 2048
      const uint32_t word = (qt < nwords) ? bits[qr][qt] : 0u;
      const int cnt = __popc(word);
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (qt >= off) incl += y;
      }
      int pos = incl - cnt;
      uint32_t w = word;
      while (w) {
        const int bb = __ffs(w) - 1;
        out[pos++] = qt * 32 + bb;
        w &= w - 1;
      }
    }
    __syncthreads();  // every quarter is done with its bitmap
  }
}

// One launch: workgroup 0 runs the scans, the split rule and the sorted work
// list; workgroups 1, 2, ... fill the CSR columns of four rows each.
__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(
    const int16_t* __restrict__ ranked, const int32_t* __restrict__ row_count,
    const int32_t* __restrict__ head_refill, int rows, int nb, int refill_per_mille, int split_s,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx, int32_t* __restrict__ head_count_final,
    int32_t* __restrict__ work_order, int32_t* __restrict__ plan_meta, uint32_t* __restrict__ tile_counter) {
  if (blockIdx.x == 0) {
    plan_scan(row_count, head_refill, rows, nb, refill_per_mille, split_s, row_ptr, head_count_final, work_order,
              plan_meta, tile_counter);
  } else {
    // fill workgroup f of F takes the rows [f * per, (f + 1) * per), per a
    // multiple of four
    const int nf = (int)gridDim.x - 1, f = (int)blockIdx.x - 1;
    const int per = ((rows + nf - 1) / nf + 3) & ~3;
    const int first = min(rows, f * per);
    plan_fill(ranked, row_count, head_refill, rows, nb, refill_per_mille, first, min(rows, first + per), col_idx);
  }
}

int launch_plan(const fva_problem& p, int nb, int split_s, const int16_t* ranked,
                const int32_t* row_count, const int32_t* head_refill, int32_t* row_ptr,
                int32_t* col_idx, int32_t* head_count_final, int32_t* work_order,
                int32_t* plan_meta, uint32_t* tile_counter, hipStream_t stream) {
  const int rows = p.num_heads * nb;
  // the sort's LDS: the item count padded to a power of two (>= 128)
  const int cap = rows + (rows < FVA_MAX_SPLITS ? rows : FVA_MAX_SPLITS);
  int ipad = 128;
  while (ipad < cap) ipad <<= 1;
  const int fill_wgs = (rows + 3) / 4 < FILL_WGS_MAX ? (rows + 3) / 4 : FILL_WGS_MAX;
  plan_kernel<<<1 + fill_wgs, PLAN_THREADS, ipad * sizeof(uint32_t), stream>>>(ranked, row_count, head_refill, rows, nb,
                                                               p.refill_per_mille, split_s, row_ptr, col_idx,
                                                               head_count_final, work_order, plan_meta, tile_counter);
  return record_hip_error(hipGetLastError(), "plan launch");
}

}  // namespace fva
