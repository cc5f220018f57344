// Routing frontend kernels: video-aware order, pooled block representatives,
// block scores, ranking and the Top-p cutoff with a Top-k floor.
//
// FVAttn paper S3.1: blocks are reorganised along a locality-preserving order,
// block similarity comes from pooled Q/K, a Top-p CDF threshold per query
// block decides how many key blocks to keep, a Top-k floor keeps a minimum,
// and the same pass yields the per-head density and the importance order.
// GSRS paper S5.3 / A.4: importance is normalised over the key blocks of a
// query block; Top-p takes the shortest descending prefix reaching p.
#include "fva_common.h"
#include "fva_lanes.h"

namespace fva {

// ---------------------------------------------------------------------------
// 1. Pooling and re-layout.  One workgroup per (block b, head h): the mean
// of the block's Q rows and of its K rows, accumulated in fp32, and the K
// rows written in position order (kp).  V is
// re-laid out (transposed per 64-position sub-block, vt) by extra workgroups
// of the select launch, where its memory traffic overlaps the latency-bound
// ranking; the layouts are those described with vt_key.  Memory bound: every
// byte of Q, K and V is read exactly once with 16-byte loads, a row's 16-byte
// chunks spread over consecutive lanes, all of a block's loads in flight
// together.  The workgroups of head 0 also publish the order table, and
// workgroup (0,0) clears the per-head counters for the select kernel.
// ---------------------------------------------------------------------------

// Where the V re-layout workgroups read and write.
struct VRelayout {
  const bf16_t* v;
  int64_t stride_head, stride_token;
  const int32_t* order;  // position -> token, -1 past the end (written by the pool kernel)
  bf16_t* vt;
  int block, nb, n;
};

// V of one block, transposed per 64-position sub-block: a thread gathers the
// 16-byte chunk dc (features 8dc .. 8dc+7) of the 8 keys that make up output
// chunk jc (columns 8jc .. 8jc+7), transposes the 8 x 8 bf16 block in
// registers and writes 8 rows of 16 bytes.  The 8 keys of chunk jc are
// vt_key(8jc + e) = 16(jc/2) + 4(jc%2) + 8(e/4) + e%4.  256 threads; tok
// holds the block's tokens in LDS (rb real ones), x points at the head's V,
// dst_blk at the block's first V^T sub-tile.
template <int D>
__device__ __forceinline__ void vt_transpose_block(const bf16_t* __restrict__ x, int64_t stride_token,
                                                   const int32_t* tok, int rb, int block,
                                                   bf16_t* __restrict__ dst_blk) {
  const int tid = threadIdx.x;
  constexpr int DCH = D / 8;
  constexpr int PER_SB = (VT_KEYS / 8) * DCH;
  for (int w = tid; w < (block / VT_KEYS) * PER_SB; w += 256) {
    const int sb = w / PER_SB, rem = w % PER_SB;
    // output chunk fastest: the eight lanes of one feature chunk dc write a
    // whole 128-byte V^T row (64 keys) in one store instruction
    const int jc = rem % (VT_KEYS / 8), dc = rem / (VT_KEYS / 8);
    const int k0 = sb * VT_KEYS + 16 * (jc >> 1) + 4 * (jc & 1);
    u32x4 in[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = k0 + 8 * (e >> 2) + (e & 3);
      in[e] = u32x4{0u, 0u, 0u, 0u};
      if (key < rb) in[e] = *reinterpret_cast<const u32x4*>(x + (int64_t)tok[key] * stride_token + dc * 8);
    }
    bf16_t* dst = dst_blk + (int64_t)(sb * VT_KEYS) * D + (8 * dc) * VT_KEYS + jc * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // feature 8dc + i of keys e = 0..7: the low (i even) or high (i odd)
      // half of dword i/2 of each key's chunk, paired two keys per dword
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      uint32_t o[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr)
        o[pr] = __builtin_amdgcn_perm(in[2 * pr + 1][i >> 1], in[2 * pr][i >> 1], sel);
      *reinterpret_cast<u32x4*>(dst + i * VT_KEYS) = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

// V re-layout of block b of head h inside the select launch (the order
// table has been written by the pooling launch).  tok is 128 ints of LDS.
template <int D>
__device__ __forceinline__ void vt_relayout_block(const VRelayout& r, int b, int h, int32_t* tok) {
  const int tid = threadIdx.x;
  const int block = r.block;
  if (tid < block) tok[tid] = r.order[b * block + tid];
  __syncthreads();
  const int rb = min(block, r.n - b * block);
  const int64_t npad = (int64_t)r.nb * block;
  vt_transpose_block<D>(r.v + (int64_t)h * r.stride_head, r.stride_token, tok, rb, block,
                        r.vt + ((int64_t)h * npad + (int64_t)b * block) * D);
}

// K and V of block b of head h in the attention's layout, from the caller's
// tensors alone (fva_kv_layout): the block's tokens from the closed-form
// order, K rows copied in position order (zero rows past the end, all loads
// in flight before the stores), V transposed as above.  Workgroups of head 0
// also publish the order table.
template <int D>
__global__ __launch_bounds__(256) void kv_layout_kernel(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, int64_t stride_head,
    int64_t stride_token, OrderGeo geo, int block, int nb, int32_t* __restrict__ order,
    bf16_t* __restrict__ kp, bf16_t* __restrict__ vt) {
  constexpr int CH = D / 8;
  constexpr int MAXIT = 128 * CH / 256;
  __shared__ int32_t tok[128];
  const int b = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int rb = min(block, geo.n - b * block);
  if (tid < block) {
    const int t = geo.token(b * block + tid);
    tok[tid] = t;
    if (h == 0) order[b * block + tid] = t;
  }
  __syncthreads();
  const int64_t npad = (int64_t)nb * block;
  const bf16_t* xk = k + (int64_t)h * stride_head;
  u32x4 rows[MAXIT];
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int x = tid + it * 256, r = x / CH, c = x % CH;
    rows[it] = u32x4{0u, 0u, 0u, 0u};
    if (r < rb) rows[it] = *reinterpret_cast<const u32x4*>(xk + (int64_t)tok[r] * stride_token + c * 8);
  }
  bf16_t* dst = kp + ((int64_t)h * npad + (int64_t)b * block) * D;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int x = tid + it * 256, r = x / CH, c = x % CH;
    if (r < block) *reinterpret_cast<u32x4*>(dst + (int64_t)r * D + c * 8) = rows[it];
  }
  vt_transpose_block<D>(v + (int64_t)h * stride_head, stride_token, tok, rb, block,
                        vt + ((int64_t)h * npad + (int64_t)b * block) * D);
}
// (at least 5 workgroups per compute unit, so that a 5-head problem's
// workgroups are all resident at once)
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void route_pool_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    int64_t stride_head, int64_t stride_token, OrderGeo geo, int block,
    int nb, int num_heads, float* __restrict__ qbar, float* __restrict__ kbar,
    int32_t* __restrict__ order, int32_t* __restrict__ head_count,
    bf16_t* __restrict__ kp) {
  constexpr int CH = D / 8;      // 16-byte chunks per row
  constexpr int RG = 256 / CH;   // rows in flight per pass
  constexpr int MAXIT = 128 / RG;
  __shared__ int32_t tok[128];
  __shared__ float part[2][RG][D];

  const int b = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int rb = min(block, geo.n - b * block);
  if (tid < block) {
    const int t = geo.token(b * block + tid);
    tok[tid] = t;
    if (h == 0) order[b * block + tid] = t;
  }
  if (b == 0 && h == 0)
    for (int i = tid; i < num_heads; i += 256) head_count[i] = 0;
  __syncthreads();

  const int64_t npad = (int64_t)nb * block;
  const int c = tid % CH, rg = tid / CH;

  // every row of the block's Q and K in flight at once
  const bf16_t* xq = q + (int64_t)h * stride_head;
  const bf16_t* xk = k + (int64_t)h * stride_head;
  u32x4 qrows[MAXIT], krows[MAXIT];
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int r = rg + it * RG;
    qrows[it] = krows[it] = u32x4{0u, 0u, 0u, 0u};
    if (r < rb) {
      const int64_t off = (int64_t)tok[r] * stride_token + c * 8;
      qrows[it] = *reinterpret_cast<const u32x4*>(xq + off);
      krows[it] = *reinterpret_cast<const u32x4*>(xk + off);
    }
  }
  // K rows in position order, zero rows past the end (when the caller asked
  // for the attention's K/V layout)
  if (kp != nullptr) {
    bf16_t* dst = kp + ((int64_t)h * npad + (int64_t)b * block) * D;
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int r = rg + it * RG;
      if (r < block) *reinterpret_cast<u32x4*>(dst + (int64_t)r * D + c * 8) = krows[it];
    }
  }
  auto column_sums = [&](const u32x4(&rows)[MAXIT], float(&pt)[RG][D]) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      acc[0] += bf16_lo(rows[it].x); acc[1] += bf16_hi(rows[it].x);
      acc[2] += bf16_lo(rows[it].y); acc[3] += bf16_hi(rows[it].y);
      acc[4] += bf16_lo(rows[it].z); acc[5] += bf16_hi(rows[it].z);
      acc[6] += bf16_lo(rows[it].w); acc[7] += bf16_hi(rows[it].w);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) pt[rg][c * 8 + e] = acc[e];
  };
  column_sums(qrows, part[0]);
  column_sums(krows, part[1]);
  __syncthreads();
  if (tid < 2 * D) {
    const int which = tid / D, col = tid % D;
    float sum = 0.f;
#pragma unroll 8
    for (int g = 0; g < RG; ++g) sum += part[which][g][col];
    float* out = (which == 0 ? qbar : kbar) + ((int64_t)h * nb + b) * D;
    out[col] = sum / (float)rb;
  }
}

// ---------------------------------------------------------------------------
// 2. Block scores S_h = sm_scale * Qbar_h Kbar_h^T with fp32 MFMA
// (v_mfma_f32_32x32x2f32).  A workgroup owns a 32 x 32 tile of S and its
// four waves split the contraction over d into quarters, so that the short
// dependent MFMA chains of many tiles run on all compute units at once; the
// partial tiles are added in LDS in wave order.  Operands are staged in LDS
// with one float of row padding so that the 32 rows a wave reads at one
// column hit 32 banks.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void route_scores_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nb,
    float sm_scale, float* __restrict__ scores) {
  constexpr int LD = D + 1;
  constexpr int KQ = D / 4;  // contraction slice of one wave
  __shared__ float qs[32 * LD];
  __shared__ float ks[32 * LD];
  __shared__ float part[4][32 * 33];
  const int h = blockIdx.z;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int tid = threadIdx.x;
  const float* qh = qbar + (int64_t)h * nb * D;
  const float* kh = kbar + (int64_t)h * nb * D;
  for (int idx = tid; idx < 32 * D / 4; idx += 256) {
    const int r = idx / (D / 4), c4 = idx % (D / 4);
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    if (i0 + r < nb) a = *reinterpret_cast<const f32x4*>(qh + (int64_t)(i0 + r) * D + c4 * 4);
    if (j0 + r < nb) b = *reinterpret_cast<const f32x4*>(kh + (int64_t)(j0 + r) * D + c4 * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qs[r * LD + c4 * 4 + e] = a[e];
      ks[r * LD + c4 * 4 + e] = b[e];
    }
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hf = lane >> 5;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const float* qrow = qs + l32 * LD + hf + wave * KQ;
  const float* krow = ks + l32 * LD + hf + wave * KQ;
#pragma unroll
  for (int kk = 0; kk < KQ; kk += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qrow[kk], krow[kk], acc, 0, 0, 0);
  // acc[r] holds this wave's part of S[i0 + 8*(r/4) + 4*hf + r%4][j0 + l32]
#pragma unroll
  for (int r = 0; r < 16; ++r) part[wave][(8 * (r >> 2) + 4 * hf + (r & 3)) * 33 + l32] = acc[r];
  __syncthreads();
  for (int x = tid; x < 32 * 32; x += 256) {
    const int ii = x >> 5, jj = x & 31;
    const int i = i0 + ii, j = j0 + jj;
    const int o = ii * 33 + jj;
    const float sum = ((part[0][o] + part[1][o]) + part[2][o]) + part[3][o];
    if (i < nb && j < nb) scores[(int64_t)h * nb * nb + (int64_t)i * nb + j] = sm_scale * sum;
  }
}

// Order-preserving map float -> uint32 (larger float -> larger key), with
// -0.0 folded onto +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of orderable (with -0.0 already folded onto +0.0).
__device__ __forceinline__ float from_orderable(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// ---------------------------------------------------------------------------
// 3. Ranking and cutoff.  One wave per (query block i, head h) row at a time,
// SEL_ROWS consecutive rows per wave and four waves per workgroup; the sort
// and the scan use no LDS and no barriers (rows of more than 256 blocks take
// two waves each, see sort_desc_rows):
//   - keys (orderable(s_j) << 32) | (2^32-1-j), slot x = E lane + e held
//     in register e of the lane, sorted descending by a bitonic network
//     (strides below E between the lane's registers, larger strides between
//     lanes): score descending, equal scores by lower id;
//   - weights w_r = rint(exp(s_(r) - s_(0)) * 2^40) in fp64, an exact integer
//     inclusive scan along the ranking (within each lane's registers, then
//     across lanes by DPP row shifts and the row totals), target
//     T = fl(p * W);
//   - k_p = 1 + #{r : prefix_r < ceil(T)}, k_i = max(k_p, min(k_min, nb)).
// Integer prefix sums make the cutoff independent of summation order.  The
// per-head sums of k_i are accumulated per wave and per workgroup before one
// atomic add per head touched (same-address atomics from many workgroups
// serialise, about 10 ns each).
// ---------------------------------------------------------------------------
constexpr int SEL_ROWS = 1;

// Bitonic sort of the wave's 64 E keys, descending over slot x = E lane + e:
// each lane holds E consecutive slots, so the strides below E (which occur in
// the most stages) compare two registers of one lane, and a stride JJ >= E
// exchanges between lanes l and l ^ (JJ / E).
template <int E>
__device__ __forceinline__ void sort_desc(uint64_t (&key)[E], int lane) {
  constexpr int LOG = __builtin_ctz(64 * E);
  static_for<1, LOG + 1>([&](auto kl) {
    constexpr int KK = 1 << decltype(kl)::value;
    static_for<0, decltype(kl)::value>([&](auto jl) {
      constexpr int JJ = KK >> (decltype(jl)::value + 1);
      if constexpr (JJ < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & JJ) == 0) {
            const bool desc = ((lane * E + e) & KK) == 0;
            const uint64_t a = key[e], b = key[e | JJ];
            if ((a < b) == desc) {
              key[e] = b;
              key[e | JJ] = a;
            }
          }
        }
      } else {
        constexpr int LJ = JJ / E;
        // KK > JJ >= E, so the direction is the same for all of the lane's
        // slots; the slot keeps the larger key where its side and direction
        // agree, else the smaller
        const bool keep_larger = ((lane & LJ) == 0) == (((lane * E) & KK) == 0);
#pragma unroll
        for (int e = 0; e < E; ++e) key[e] = exchange_keep<LJ>(key[e], keep_larger);
      }
    });
  });
}

// Inclusive scan of the weights w[e] of slots x = E lane + e (a running sum
// over the lane's registers, then one scan of the lane totals across the
// wave); total = the wave's sum.
template <int E>
__device__ __forceinline__ void scan_slots(const uint64_t (&w)[E], uint64_t (&prefix)[E], uint64_t& total,
                                           int lane) {
  uint64_t run = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    run += w[e];
    prefix[e] = run;
  }
  const uint64_t incl = wave_incl_scan_u64(run, lane);
  const uint64_t before = incl - run;
#pragma unroll
  for (int e = 0; e < E; ++e) prefix[e] += before;
  const uint32_t tlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)incl, 63);
  const uint32_t thi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(incl >> 32), 63);
  total = ((uint64_t)thi << 32) | tlo;
}

// Exact integer inclusive scan of the weights along the ranking; returns
// #{slots with a weight-bearing entry whose prefix stays below ceil(p * W)},
// W = the sum of all weights.  (Slots with zero weight past the ranked
// entries are never below the target once the prefix has reached W.)
template <int E>
__device__ __forceinline__ int count_below_target(const uint64_t (&w)[E], const bool (&live)[E],
                                                  float p, int lane) {
  uint64_t prefix[E];
  uint64_t carry;
  scan_slots<E>(w, prefix, carry, lane);
  const double target = (double)p * (double)carry;
  const uint64_t tint = (uint64_t)ceil(target);
  // the count over the wave, from one ballot per register
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(live[e] && prefix[e] < tint));
  return cnt;
}

template <int E>  // keys per lane: the row padded to 64 E >= nb slots
__device__ __forceinline__ int select_row(const float* __restrict__ scores, int nb, int row, float top_p,
                                          int k_min, int16_t* __restrict__ ranked, int lane) {
  const float* s = scores + (int64_t)row * nb;

  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = lane * E + e;
    key[e] = x < nb ? (((uint64_t)orderable(s[x]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)x)) : 0ull;
  }
  sort_desc<E>(key, lane);

  int16_t* rk = ranked + (int64_t)row * nb;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = lane * E + e;
    if (x < nb) rk[x] = (int16_t)(0xffffffffu - (uint32_t)(key[e] & 0xffffffffull));
  }

  int kp;
  const float p = top_p;
  if (p >= 1.0f) {
    kp = nb;
  } else if (!(p > 0.0f)) {
    kp = 0;
  } else {
    // weights along the ranking (pad slots weigh 0), exact integer scan
    const uint32_t top = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key[0] >> 32), 0);
    const double smax = (double)from_orderable(top);
    uint64_t w[E];
    bool live[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int x = lane * E + e;
      const double sr = (double)from_orderable((uint32_t)(key[e] >> 32));
      live[e] = x < nb;
      w[e] = live[e] ? (uint64_t)rint(exp(sr - smax) * 1099511627776.0) : 0ull;  // 2^40
    }
    kp = min(nb, count_below_target<E>(w, live, p, lane) + 1);
  }
  return max(kp, min(k_min, nb));
}

// Rows of more than 256 blocks are ranked by W = 2 waves together (one wave
// alone would take 16 or 32 keys per lane through the whole network), two
// rows per workgroup.  Slot x = 64 EL v + EL lane + e of a row is register e
// of lane `lane` of the row's wave v (v = 0 .. W-1, EL = E / W keys per
// lane); the bitonic stages of stride below EL compare registers of one lane,
// strides EL .. 32 EL exchange between lanes, and stride 64 EL -- the widest
// stage of the last merge level -- between the row's two waves through LDS.
constexpr int RANK_WAVES = 2;  // waves per row for rows of more than 256 blocks

template <int EL>
struct RowRankLds {
  uint64_t xbuf[RANK_WAVES * EL * 64];
  uint64_t wave_total[RANK_WAVES];
  int wave_count[RANK_WAVES];
  uint32_t top;
};

template <int EL>
__device__ __forceinline__ void sort_desc_rows(uint64_t (&key)[EL], int lane, int v, uint64_t* xbuf) {
  constexpr int LOG = __builtin_ctz(64 * EL * RANK_WAVES);
  const int x0 = v * EL * 64 + lane * EL;  // slot of register 0
  static_for<1, LOG + 1>([&](auto kl) {
    constexpr int KK = 1 << decltype(kl)::value;
    static_for<0, decltype(kl)::value>([&](auto jl) {
      constexpr int JJ = KK >> (decltype(jl)::value + 1);
      if constexpr (JJ >= 64 * EL) {
        constexpr int WJ = JJ / (64 * EL);
#pragma unroll
        for (int e = 0; e < EL; ++e) xbuf[(v * EL + e) * 64 + lane] = key[e];
        __syncthreads();
        const bool keep_larger = ((v & WJ) == 0) == ((x0 & KK) == 0);
#pragma unroll
        for (int e = 0; e < EL; ++e) {
          const uint64_t a = key[e], b = xbuf[((v ^ WJ) * EL + e) * 64 + lane];
          key[e] = ((a > b) == keep_larger) ? a : b;
        }
        __syncthreads();
      } else if constexpr (JJ < EL) {
#pragma unroll
        for (int e = 0; e < EL; ++e) {
          if ((e & JJ) == 0) {
            const bool desc = ((x0 + e) & KK) == 0;
            const uint64_t a = key[e], b = key[e | JJ];
            if ((a < b) == desc) {
              key[e] = b;
              key[e | JJ] = a;
            }
          }
        }
      } else {
        constexpr int LJ = JJ / EL;
        // KK > JJ >= EL, so the direction is the same for all of the lane's
        // slots; the slot keeps the larger key where its side and direction
        // agree, else the smaller
        const bool keep_larger = ((lane & LJ) == 0) == ((x0 & KK) == 0);
#pragma unroll
        for (int e = 0; e < EL; ++e) key[e] = exchange_keep<LJ>(key[e], keep_larger);
      }
    });
  });
}

// select_row for one row ranked by RANK_WAVES waves (same keys, weights,
// target and count; the weights' inclusive scan runs per wave and is carried
// across the row's waves in slot order).  `live_row` is false for the second
// row slot of the last workgroup when the row count is odd: its waves take
// part in the barriers only.
template <int EL>
__device__ __forceinline__ int select_row_waves(const float* __restrict__ scores, int nb, int row, bool live_row,
                                                float top_p, int k_min, int16_t* __restrict__ ranked, int lane,
                                                int v, RowRankLds<EL>& sh) {
  const float* s = scores + (int64_t)row * nb;
  const int x0 = v * EL * 64 + lane * EL;
  uint64_t key[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    const int x = x0 + e;
    key[e] = (live_row && x < nb) ? (((uint64_t)orderable(s[x]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)x))
                                  : 0ull;
  }
  sort_desc_rows<EL>(key, lane, v, sh.xbuf);

  if (live_row) {
    int16_t* rk = ranked + (int64_t)row * nb;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int x = x0 + e;
      if (x < nb) rk[x] = (int16_t)(0xffffffffu - (uint32_t)(key[e] & 0xffffffffull));
    }
  }

  int kp;
  const float p = top_p;
  if (p >= 1.0f) {
    kp = nb;
  } else if (!(p > 0.0f)) {
    kp = 0;
  } else {
    if (v == 0 && lane == 0) sh.top = (uint32_t)(key[0] >> 32);
    __syncthreads();
    const double smax = (double)from_orderable(sh.top);
    uint64_t w[EL], prefix[EL];
    bool live[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int x = x0 + e;
      const double sr = (double)from_orderable((uint32_t)(key[e] >> 32));
      live[e] = live_row && x < nb;
      w[e] = live[e] ? (uint64_t)rint(exp(sr - smax) * 1099511627776.0) : 0ull;  // 2^40
    }
    uint64_t carry;
    scan_slots<EL>(w, prefix, carry, lane);
    if (lane == 0) sh.wave_total[v] = carry;
    __syncthreads();
    uint64_t before = 0, total = 0;
#pragma unroll
    for (int u = 0; u < RANK_WAVES; ++u) {
      const uint64_t t = sh.wave_total[u];
      total += t;
      if (u < v) before += t;
    }
    const uint64_t tint = (uint64_t)ceil((double)p * (double)total);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < EL; ++e) cnt += __popcll(__ballot(live[e] && before + prefix[e] < tint));
    if (lane == 0) sh.wave_count[v] = cnt;
    __syncthreads();
    int c = 1;
#pragma unroll
    for (int u = 0; u < RANK_WAVES; ++u) c += sh.wave_count[u];
    kp = min(nb, c);
  }
  return max(kp, min(k_min, nb));
}

// Re-selection inside an evaluated set (growing sparsity with reduced
// search): the row's evaluated blocks (its CSR entries) are ranked by their
// precise importance, descending, equal values by lower id, and the other
// blocks follow by ascending id; the weights are rint(importance * 2^40) of
// the evaluated blocks, the cutoff the shortest prefix reaching p of their
// sum, the floor min(k_min, evaluated count).  `bits` is this wave's LDS
// membership bitmap (nb bits).
template <int E>
__device__ __forceinline__ int reselect_row(const float* __restrict__ importance, const int32_t* __restrict__ row_ptr,
                                            const int32_t* __restrict__ col_idx, int nb, int row, float top_p,
                                            int k_min, int16_t* __restrict__ ranked, uint32_t* bits, int lane) {
  const int nwords = (nb + 31) >> 5;
  if (lane < nwords) bits[lane] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int c0 = row_ptr[row], c = row_ptr[row + 1] - c0;
  for (int j = lane; j < c; j += 64) {
    const int b = col_idx[c0 + j];
    atomicOr(&bits[b >> 5], 1u << (b & 31));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float* v = importance + (int64_t)row * nb;
  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = lane * E + e;
    const uint64_t id = (uint64_t)(0xffffffffu - (uint32_t)x);
    if (x >= nb)
      key[e] = 0ull;
    else if ((bits[x >> 5] >> (x & 31)) & 1u)
      key[e] = ((uint64_t)orderable(v[x]) << 32) | id;  // >= 2^63 for importance >= 0
    else
      key[e] = id;
  }
  sort_desc<E>(key, lane);

  int16_t* rk = ranked + (int64_t)row * nb;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = lane * E + e;
    if (x < nb) rk[x] = (int16_t)(0xffffffffu - (uint32_t)(key[e] & 0xffffffffull));
  }

  int kp;
  const float p = top_p;
  if (p >= 1.0f) {
    kp = c;
  } else if (!(p > 0.0f)) {
    kp = 0;
  } else {
    // the first c ranks are the evaluated blocks
    uint64_t w[E];
    bool live[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      live[e] = lane * E + e < c;
      const double imp = fmax((double)from_orderable((uint32_t)(key[e] >> 32)), 0.0);
      w[e] = live[e] ? (uint64_t)rint(imp * 1099511627776.0) : 0ull;  // 2^40
    }
    kp = min(c, count_below_target<E>(w, live, p, lane) + 1);
  }
  return max(kp, min(k_min, c));
}

// The launch also carries the V re-layout: workgroups sel_wgs .. sel_wgs +
// H*nb - 1 each transpose one (head, block) of V (vt_relayout_block), so that
// the memory traffic overlaps the latency-bound ranking.
template <int E, int D>
__global__ __launch_bounds__(256) void route_select_kernel(
    const float* __restrict__ scores, int nb, int rows, float top_p, int k_min,
    int16_t* __restrict__ ranked, int32_t* __restrict__ row_count,
    int32_t* __restrict__ head_count, int sel_wgs, VRelayout vr) {
  if ((int)blockIdx.x >= sel_wgs) {
    __shared__ int32_t tok[128];
    const int w = blockIdx.x - sel_wgs;
    vt_relayout_block<D>(vr, w % vr.nb, w / vr.nb, tok);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if constexpr (E >= 8) {
    // two rows per workgroup, RANK_WAVES waves per row
    constexpr int RPW = 4 / RANK_WAVES;
    __shared__ RowRankLds<E / RANK_WAVES> sh[RPW];
    const int slot = wave / RANK_WAVES, v = wave % RANK_WAVES;
    const int row = blockIdx.x * RPW + slot;
    const bool live_row = row < rows;
    const int ki = select_row_waves<E / RANK_WAVES>(scores, nb, live_row ? row : 0, live_row, top_p, k_min,
                                                    ranked, lane, v, sh[slot]);
    // the workgroup's rows are summed per head before one atomic add per
    // head touched (one add per row made these launches 8 us slower at
    // 2,955 rows)
    __shared__ int row_k[RPW];
    if (v == 0 && lane == 0) {
      if (live_row) row_count[row] = ki;
      row_k[slot] = live_row ? ki : 0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const int r0 = blockIdx.x * RPW;  // < rows: the grid has ceil(rows / RPW) ranking workgroups
      int head = r0 / nb, sum = 0;
      for (int sl = 0; sl < RPW && r0 + sl < rows; ++sl) {
        const int hs = (r0 + sl) / nb;
        if (hs != head) {
          atomicAdd(&head_count[head], sum);
          head = hs;
          sum = 0;
        }
        sum += row_k[sl];
      }
      atomicAdd(&head_count[head], sum);
    }
    return;
  }
  __shared__ int wave_sum[4];
  const int first = blockIdx.x * 4 * SEL_ROWS;
  const int last = min(rows, first + 4 * SEL_ROWS) - 1;
  const bool one_head = first / nb == last / nb;  // the common case: pool the workgroup's sum
  int head = -1, sum = 0;
  for (int j = 0; j < SEL_ROWS; ++j) {
    const int row = first + wave * SEL_ROWS + j;
    if (row >= rows) break;  // uniform per wave
    const int ki = select_row<E>(scores, nb, row, top_p, k_min, ranked, lane);
    if (lane == 0) row_count[row] = ki;
    const int h = row / nb;
    if (h != head) {
      if (head >= 0 && lane == 0) atomicAdd(&head_count[head], sum);
      head = h;
      sum = 0;
    }
    sum += ki;
  }
  // every wave leaves its sum in its own LDS word (0 without rows), so the
  // words need no clearing and the workgroup one barrier
  if (lane == 0) {
    if (one_head) wave_sum[wave] = head >= 0 ? sum : 0;
    else if (head >= 0) atomicAdd(&head_count[head], sum);
  }
  __syncthreads();
  if (threadIdx.x == 0 && one_head)
    atomicAdd(&head_count[first / nb], (wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3]));
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int n, int v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int E>
__global__ __launch_bounds__(256) void reselect_kernel(
    const float* __restrict__ importance, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int nb, int rows, float top_p, int k_min,
    int16_t* __restrict__ ranked, int32_t* __restrict__ row_count, int32_t* __restrict__ head_count) {
  __shared__ uint32_t bits[4][FVA_MAX_BLOCKS / 32];
  __shared__ int wg_sum;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int first = blockIdx.x * 4;
  const int last = min(rows, first + 4) - 1;
  const bool one_head = first / nb == last / nb;
  if (threadIdx.x == 0) wg_sum = 0;
  __syncthreads();
  const int row = first + wave;
  if (row < rows) {  // uniform per wave
    const int ki = reselect_row<E>(importance, row_ptr, col_idx, nb, row, top_p, k_min, ranked,
                                   bits[wave], lane);
    if (lane == 0) {
      row_count[row] = ki;
      if (one_head) atomicAdd(&wg_sum, ki);
      else atomicAdd(&head_count[row / nb], ki);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && one_head) atomicAdd(&head_count[first / nb], wg_sum);
}

int launch_reselect(const fva_problem& p, int nb, const int32_t* row_ptr, const int32_t* col_idx,
                    const float* importance, int16_t* ranked, int32_t* row_count,
                    int32_t* head_count, hipStream_t stream) {
  fill_i32_kernel<<<(p.num_heads + 255) / 256, 256, 0, stream>>>(head_count, p.num_heads, 0);
  int st = record_hip_error(hipGetLastError(), "fill launch");
  if (st) return st;
  const int rows = p.num_heads * nb;
  const int grid = (rows + 3) / 4;
  int e = 1;
  while (64 * e < nb) e <<= 1;
#define FVA_RESELECT(E_)                                                                    \
  reselect_kernel<E_><<<grid, 256, 0, stream>>>(importance, row_ptr, col_idx, nb, rows, p.top_p, \
                                                p.k_min, ranked, row_count, head_count)
  switch (e) {
    case 1: FVA_RESELECT(1); break;
    case 2: FVA_RESELECT(2); break;
    case 4: FVA_RESELECT(4); break;
    case 8: FVA_RESELECT(8); break;
    case 16: FVA_RESELECT(16); break;
    default: FVA_RESELECT(32); break;
  }
#undef FVA_RESELECT
  return record_hip_error(hipGetLastError(), "reselect launch");
}

int launch_route(const fva_problem& p, int nb, const void* q, const void* k, const void* v,
                 float* scores, int16_t* ranked, int32_t* row_count,
                 int32_t* head_count, int32_t* order, void* kv, float* qbar, float* kbar,
                 float sm_scale, hipStream_t stream) {
  const OrderGeo geo = make_order_geo(p);
  const dim3 pool_grid(nb, p.num_heads);
  // kv == nullptr: routing only (Q and K read, nothing re-laid out)
  bf16_t* kp = (bf16_t*)kv;
  bf16_t* vt = kp ? kp + (int64_t)p.num_heads * nb * p.block * p.head_dim : nullptr;
  if (p.head_dim == 128)
    route_pool_kernel<128><<<pool_grid, 256, 0, stream>>>(
        (const bf16_t*)q, (const bf16_t*)k, p.stride_head, p.stride_token, geo, p.block, nb,
        p.num_heads, qbar, kbar, order, head_count, kp);
  else
    route_pool_kernel<64><<<pool_grid, 256, 0, stream>>>(
        (const bf16_t*)q, (const bf16_t*)k, p.stride_head, p.stride_token, geo, p.block, nb,
        p.num_heads, qbar, kbar, order, head_count, kp);
  int st = record_hip_error(hipGetLastError(), "route_pool launch");
  if (st) return st;

  const dim3 sc_grid((nb + 31) / 32, (nb + 31) / 32, p.num_heads);
  if (p.head_dim == 128)
    route_scores_kernel<128><<<sc_grid, 256, 0, stream>>>(qbar, kbar, nb, sm_scale, scores);
  else
    route_scores_kernel<64><<<sc_grid, 256, 0, stream>>>(qbar, kbar, nb, sm_scale, scores);
  st = record_hip_error(hipGetLastError(), "route_scores launch");
  if (st) return st;

  // with kv, the select launch also carries the V re-layout, one workgroup
  // per (head, block); a share of it in the scores launch was slower (those
  // workgroups would hold the score tiles' 66 KB of LDS each)
  const int rows = p.num_heads * nb;
  const VRelayout vr{(const bf16_t*)v, p.stride_head, p.stride_token, order, vt, p.block, nb, p.seq_len};
  int e = 1;
  while (64 * e < nb) e <<= 1;
  // ranking workgroups: four rows each (one wave per row), or two rows each
  // (two waves per row) when a row has more than 256 blocks (E >= 8)
  const int sel_wgs = e >= 8 ? (rows + 1) / 2 : (rows + 4 * SEL_ROWS - 1) / (4 * SEL_ROWS);
  const int grid = sel_wgs + (kv ? rows : 0);
#define FVA_SELECT(E_)                                                                               \
  do {                                                                                               \
    if (p.head_dim == 128)                                                                           \
      route_select_kernel<E_, 128><<<grid, 256, 0, stream>>>(scores, nb, rows, p.top_p, p.k_min, ranked, \
                                                             row_count, head_count, sel_wgs, vr);    \
    else                                                                                             \
      route_select_kernel<E_, 64><<<grid, 256, 0, stream>>>(scores, nb, rows, p.top_p, p.k_min, ranked,  \
                                                            row_count, head_count, sel_wgs, vr);    \
  } while (0)
  switch (e) {
    case 1: FVA_SELECT(1); break;
    case 2: FVA_SELECT(2); break;
    case 4: FVA_SELECT(4); break;
    case 8: FVA_SELECT(8); break;
    case 16: FVA_SELECT(16); break;
    default: FVA_SELECT(32); break;
  }
#undef FVA_SELECT
  return record_hip_error(hipGetLastError(), "route_select launch");
}

int launch_kv_layout(const fva_problem& p, int nb, const void* k, const void* v, int32_t* order,
                     void* kv, hipStream_t stream) {
  const OrderGeo geo = make_order_geo(p);
  const dim3 grid(nb, p.num_heads);
  bf16_t* kp = (bf16_t*)kv;
  bf16_t* vt = kp + (int64_t)p.num_heads * nb * p.block * p.head_dim;
  if (p.head_dim == 128)
    kv_layout_kernel<128><<<grid, 256, 0, stream>>>((const bf16_t*)k, (const bf16_t*)v, p.stride_head,
                                                    p.stride_token, geo, p.block, nb, order, kp, vt);
  else
    kv_layout_kernel<64><<<grid, 256, 0, stream>>>((const bf16_t*)k, (const bf16_t*)v, p.stride_head,
                                                   p.stride_token, geo, p.block, nb, order, kp, vt);
  return record_hip_error(hipGetLastError(), "kv_layout launch");
}

}  // namespace fva
