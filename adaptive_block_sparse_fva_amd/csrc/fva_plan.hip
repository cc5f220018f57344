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
//
// FROM_CSR: the row lengths come from a given row_ptr (fva_schedule) instead
// of the refill of row_count; row_ptr and head_count_final are then inputs /
// unused and only the work list, plan_meta and the counter are written.
template <bool FROM_CSR>
__device__ __forceinline__ void plan_scan(
    const int32_t* __restrict__ row_count, const int32_t* __restrict__ head_refill, int rows, int nb,
    int refill_per_mille, int split_s,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ head_count_final,
    int32_t* __restrict__ work_order, int32_t* __restrict__ plan_meta,
    uint32_t* __restrict__ tile_counter) {
  // at most FVA_MAX_TILES + FVA_MAX_SPLITS - 1 items
  static_assert(FVA_MAX_SPLITS <= FVA_MAX_TILES, "item count bound");
  extern __shared__ uint32_t keys[];  // two item buffers and the sort's count table, sized by the launch
  __shared__ int32_t wave_tot[PLAN_THREADS / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // exclusive scan across the workgroup; *total gets the sum
  auto block_scan = [&](int x, int* total) {
    const int incl = (int)wave_incl_scan((uint32_t)x, lane);
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
    if constexpr (FROM_CSR) return row_ptr[r + 1] - row_ptr[r];
    else return refill_count(row_count[r], nb, row_refill(head_refill, r, nb, refill_per_mille));
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
  if constexpr (!FROM_CSR) {
    for (int r = r0; r < r1; ++r) {
      row_ptr[r] = run;
      run += kept(r);
    }
    if (r1 == rows && r0 < r1) row_ptr[rows] = run;
  }

  // split decision and slots
  const int mean = (total + split_s - 1) / split_s;
  auto is_split = [&](int kp) { return kp >= 2 && 2 * kp > mean; };
  // no row can be cut when even a full row (nb blocks) stays within half the
  // mean load: then the slot scan is skipped (one barrier still publishes
  // the row offsets read below)
  int nsplit = 0, sp = 0;
  if (2 * nb > mean) {
    int nsp = 0;
    for (int r = r0; r < r1; ++r) nsp += is_split(kept(r)) ? 1 : 0;
    sp = block_scan(nsp, &nsplit);
  } else {
    __syncthreads();
  }
  if constexpr (!FROM_CSR)
    for (int hh = tid; hh < rows / nb; hh += PLAN_THREADS)
      head_count_final[hh] = row_ptr[(hh + 1) * nb] - row_ptr[hh * nb];

  // work items: tile r's items start at r + (split tiles before r); the
  // range of their length fields bounds the radix passes below
  __shared__ uint32_t key_lo, key_hi;
  if (tid == 0) {
    key_lo = 0xffffffffu;
    key_hi = 0u;
  }
  __syncthreads();
  uint32_t my_lo = 0xffffffffu, my_hi = 0u;
  for (int r = r0; r < r1; ++r) {
    const int kp = kept(r);
    const int pos = r + sp;
    if (is_split(kp)) {
      plan_meta[2 + r] = sp;
      plan_meta[2 + rows + sp] = r;
      keys[pos] = item_key((kp + 1) >> 1, r, 0);
      keys[pos + 1] = item_key(kp >> 1, r, 1);
      my_lo = min(my_lo, (uint32_t)(FVA_MAX_BLOCKS - ((kp + 1) >> 1)));
      my_hi = max(my_hi, (uint32_t)(FVA_MAX_BLOCKS - (kp >> 1)));
      ++sp;
    } else {
      plan_meta[2 + r] = -1;
      keys[pos] = item_key(kp, r, 0);
      my_lo = min(my_lo, (uint32_t)(FVA_MAX_BLOCKS - kp));
      my_hi = max(my_hi, (uint32_t)(FVA_MAX_BLOCKS - kp));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    my_lo = min(my_lo, (uint32_t)__shfl_xor((int)my_lo, off, 64));
    my_hi = max(my_hi, (uint32_t)__shfl_xor((int)my_hi, off, 64));
  }
  if (lane == 0) {
    atomicMin(&key_lo, my_lo);
    atomicMax(&key_hi, my_hi);
  }
  const int nitems = rows + nsplit;
  __syncthreads();

  // Stable LSD radix sort of the items on their length field (key bits
  // 15 .. 26, up to three 4-bit digits).  Items enter in index order, which is
  // (tile, part) order, so items of equal length keep that order, as the full
  // key order demands.  Per pass: each wave takes 64-item slots, ranks its
  // items among the slot's items with the same digit from four ballots, and
  // writes per-digit slot counts; an exclusive scan over (digit, slot) gives
  // every item its destination.
  {
    const int cap = rows + (rows < FVA_MAX_SPLITS ? rows : FVA_MAX_SPLITS);
    uint32_t* src = keys;
    uint32_t* dst = keys + cap;
    uint32_t* tab = keys + 2 * cap;
    const int nslots = (nitems + 63) >> 6;
    const int ntab = 16 * nslots;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    // lanes of this slot whose item digit equals e, from the four digit-bit
    // ballots b[k] and the valid lanes vm
    auto lanes_with = [&](const uint64_t (&b)[4], uint64_t vm, uint32_t e) {
      uint64_t m = vm;
#pragma unroll
      for (int k = 0; k < 4; ++k) m &= ((e >> k) & 1u) ? b[k] : ~b[k];
      return m;
    };
    // digits above the highest bit in which the length fields differ are the
    // same for every item: those passes would leave the order as it is
    const uint32_t diff = key_lo ^ key_hi;
    const int sig = diff ? 32 - __builtin_clz(diff) : 0;
    const int end_shift = 15 + ((sig + 3) & ~3);
    for (int shift = 15; shift < end_shift; shift += 4) {
      for (int s = wave; s < nslots; s += PLAN_THREADS / 64) {
        const int i = (s << 6) + lane;
        const bool valid = i < nitems;
        const uint32_t d = valid ? (src[i] >> shift) & 15u : 0u;
        uint64_t b[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) b[k] = __ballot(valid && ((d >> k) & 1u));
        // lane e < 16 counts the slot's items with digit e
        const uint64_t cnt = lanes_with(b, __ballot(valid), (uint32_t)lane);
        if (lane < 16) tab[lane * nslots + s] = (uint32_t)__popcll(cnt);
      }
      __syncthreads();
      if (ntab <= 16 * 64) {
        // small table: wave 0 scans it (up to 16 entries per lane)
        if (wave == 0) {
          const int per_l = (ntab + 63) >> 6;
          const int t0 = min(ntab, lane * per_l), t1 = min(ntab, t0 + per_l);
          int loc = 0;
          for (int x = t0; x < t1; ++x) loc += (int)tab[x];
          const int incl = (int)wave_incl_scan((uint32_t)loc, lane);
          int ex = incl - loc;
          for (int x = t0; x < t1; ++x) {
            const int c = (int)tab[x];
            tab[x] = (uint32_t)ex;
            ex += c;
          }
        }
      } else {
        const int per_t = (ntab + PLAN_THREADS - 1) / PLAN_THREADS;
        const int t0 = min(ntab, tid * per_t), t1 = min(ntab, t0 + per_t);
        int loc = 0;
        for (int x = t0; x < t1; ++x) loc += (int)tab[x];
        int tot = 0;
        int ex = block_scan(loc, &tot);
        for (int x = t0; x < t1; ++x) {
          const int c = (int)tab[x];
          tab[x] = (uint32_t)ex;
          ex += c;
        }
      }
      __syncthreads();
      for (int s = wave; s < nslots; s += PLAN_THREADS / 64) {
        const int i = (s << 6) + lane;
        const bool valid = i < nitems;
        const uint32_t v = valid ? src[i] : 0u;
        const uint32_t d = (v >> shift) & 15u;
        uint64_t b[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) b[k] = __ballot(valid && ((d >> k) & 1u));
        const uint64_t same = lanes_with(b, __ballot(valid), d);
        if (valid) dst[tab[d * nslots + s] + __popcll(same & below)] = v;
      }
      __syncthreads();
      uint32_t* t = src;
      src = dst;
      dst = t;
    }
    for (int x = tid; x < nitems; x += PLAN_THREADS) work_order[x] = (int32_t)(src[x] & 0x7fffu);
  }
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
      const int incl = (int)wave_incl_scan((uint32_t)cnt, qt);
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
    plan_scan<false>(row_count, head_refill, rows, nb, refill_per_mille, split_s, row_ptr, head_count_final,
                     work_order, plan_meta, tile_counter);
  } else {
    // fill workgroup f of F takes the rows [f * per, (f + 1) * per), per a
    // multiple of four
    const int nf = (int)gridDim.x - 1, f = (int)blockIdx.x - 1;
    const int per = ((rows + nf - 1) / nf + 3) & ~3;
    const int first = min(rows, f * per);
    plan_fill(ranked, row_count, head_refill, rows, nb, refill_per_mille, first, min(rows, first + per), col_idx);
  }
}

// The placement step alone, from a given CSR mask (fva_schedule).
__global__ __launch_bounds__(PLAN_THREADS) void schedule_kernel(
    const int32_t* __restrict__ row_ptr, int rows, int nb, int split_s, int32_t* __restrict__ work_order,
    int32_t* __restrict__ plan_meta, uint32_t* __restrict__ tile_counter) {
  plan_scan<true>(nullptr, nullptr, rows, nb, 0, split_s, const_cast<int32_t*>(row_ptr), nullptr, work_order,
                  plan_meta, tile_counter);
}

// LDS of the work-list sort: two buffers of the largest item count and the
// (digit, 64-item slot) count table.
static size_t sort_lds_bytes(int rows) {
  const int cap = rows + (rows < FVA_MAX_SPLITS ? rows : FVA_MAX_SPLITS);
  return (size_t)(2 * cap + 16 * ((cap + 63) / 64)) * sizeof(uint32_t);
}

int launch_schedule(const fva_problem& p, int nb, int split_s, const int32_t* row_ptr,
                    int32_t* work_order, int32_t* plan_meta, uint32_t* tile_counter,
                    hipStream_t stream) {
  const int rows = p.num_heads * nb;
  schedule_kernel<<<1, PLAN_THREADS, sort_lds_bytes(rows), stream>>>(row_ptr, rows, nb, split_s, work_order,
                                                                      plan_meta, tile_counter);
  return record_hip_error(hipGetLastError(), "schedule launch");
}

int launch_plan(const fva_problem& p, int nb, int split_s, const int16_t* ranked,
                const int32_t* row_count, const int32_t* head_refill, int32_t* row_ptr,
                int32_t* col_idx, int32_t* head_count_final, int32_t* work_order,
                int32_t* plan_meta, uint32_t* tile_counter, hipStream_t stream) {
  const int rows = p.num_heads * nb;
  const int fill_wgs = (rows + 3) / 4 < FILL_WGS_MAX ? (rows + 3) / 4 : FILL_WGS_MAX;
  plan_kernel<<<1 + fill_wgs, PLAN_THREADS, sort_lds_bytes(rows), stream>>>(ranked, row_count, head_refill, rows, nb,
                                                               p.refill_per_mille, split_s, row_ptr, col_idx,
                                                               head_count_final, work_order, plan_meta, tile_counter);
  return record_hip_error(hipGetLastError(), "plan launch");
}

}  // namespace fva
