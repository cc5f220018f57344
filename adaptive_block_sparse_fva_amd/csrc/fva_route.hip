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

namespace fva {

// ---------------------------------------------------------------------------
// 1. Pooling and re-layout.  One workgroup per (block b, head h, tensor
// Q|K|V).  Q and K workgroups take the mean of the block's rows, accumulated
// in fp32; the K workgroups also write the rows in position order (kp), and
// the V workgroups write V transposed per 64-position sub-block (vt); the
// layouts are those described with vt_key.  Memory bound: every byte of Q, K
// and V is read exactly once with 16-byte loads, a row's 16-byte chunks
// spread over consecutive lanes.  The Q workgroups of head 0 also publish the
// order table, and workgroup (0,0,0) clears the per-head counters for the
// select kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void route_pool_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    int64_t stride_head, int64_t stride_token, OrderGeo geo, int block,
    int nb, int num_heads, float* __restrict__ qbar, float* __restrict__ kbar,
    int32_t* __restrict__ order, int32_t* __restrict__ head_count,
    bf16_t* __restrict__ kp, bf16_t* __restrict__ vt) {
  constexpr int CH = D / 8;      // 16-byte chunks per row
  constexpr int RG = 256 / CH;   // rows in flight per pass
  constexpr int MAXIT = 128 / RG;
  constexpr int VP = D + 8;      // padded LDS row of the V transpose
  __shared__ int32_t tok[128];
  __shared__ float part[RG][D];
  __shared__ __attribute__((aligned(16))) bf16_t vs[VT_KEYS * VP];

  const int b = blockIdx.x, h = blockIdx.y, which = blockIdx.z;
  const int tid = threadIdx.x;
  const int rb = min(block, geo.n - b * block);
  if (tid < block) {
    const int t = geo.token(b * block + tid);
    tok[tid] = t;
    if (which == 0 && h == 0) order[b * block + tid] = t;
  }
  if (b == 0 && h == 0 && which == 0)
    for (int i = tid; i < num_heads; i += 256) head_count[i] = 0;
  __syncthreads();

  const int64_t npad = (int64_t)nb * block;
  const int c = tid % CH, rg = tid / CH;
  if (which == 2) {
    // V: per 64-position sub-block, rows into LDS, then columns out
    const bf16_t* x = v + (int64_t)h * stride_head;
    for (int sb = 0; sb < block; sb += VT_KEYS) {
      for (int r = rg; r < VT_KEYS; r += RG) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (sb + r < rb) w = *reinterpret_cast<const u32x4*>(x + (int64_t)tok[sb + r] * stride_token + c * 8);
        *reinterpret_cast<u32x4*>(&vs[r * VP + c * 8]) = w;
      }
      __syncthreads();
      bf16_t* dst = vt + ((int64_t)h * npad + (int64_t)b * block + sb) * D;
      for (int i = tid; i < D * (VT_KEYS / 8); i += 256) {
        const int row = i / (VT_KEYS / 8), jc = i % (VT_KEYS / 8);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)vs[vt_key(jc * 8 + 2 * e) * VP + row] |
                 ((uint32_t)vs[vt_key(jc * 8 + 2 * e + 1) * VP + row] << 16);
        *reinterpret_cast<u32x4*>(dst + row * VT_KEYS + jc * 8) = u32x4{w[0], w[1], w[2], w[3]};
      }
      __syncthreads();
    }
    return;
  }

  const bf16_t* x = (which == 0 ? q : k) + (int64_t)h * stride_head;
  u32x4 rows[MAXIT];
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int r = rg + it * RG;
    if (r < rb)
      rows[it] = *reinterpret_cast<const u32x4*>(x + (int64_t)tok[r] * stride_token + c * 8);
    else
      rows[it] = u32x4{0u, 0u, 0u, 0u};
  }
  if (which == 1) {
    // K rows in position order, zero rows past the end
    bf16_t* dst = kp + ((int64_t)h * npad + (int64_t)b * block) * D;
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int r = rg + it * RG;
      if (r < block) *reinterpret_cast<u32x4*>(dst + (int64_t)r * D + c * 8) = rows[it];
    }
  }
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
  for (int e = 0; e < 8; ++e) part[rg][c * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll 8
    for (int g = 0; g < RG; ++g) s += part[g][tid];
    float* out = (which == 0 ? qbar : kbar) + ((int64_t)h * nb + b) * D;
    out[tid] = s / (float)rb;
  }
}

// ---------------------------------------------------------------------------
// 2. Block scores S_h = sm_scale * Qbar_h Kbar_h^T with fp32 MFMA
// (v_mfma_f32_32x32x2f32).  A workgroup owns a 64 x 64 tile of S; each of its
// four waves a 32 x 32 quarter.  Operands are staged in LDS with one float of
// row padding so that the 32 rows a wave reads at one column hit 32 banks.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void route_scores_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nb,
    float sm_scale, float* __restrict__ scores) {
  constexpr int LD = D + 1;
  __shared__ float qs[64 * LD];
  __shared__ float ks[64 * LD];
  const int h = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  const float* qh = qbar + (int64_t)h * nb * D;
  const float* kh = kbar + (int64_t)h * nb * D;
  for (int idx = tid; idx < 64 * D / 4; idx += 256) {
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
  const int wm = wave & 1, wn = wave >> 1;
  const int l32 = lane & 31, hf = lane >> 5;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const float* qrow = qs + (wm * 32 + l32) * LD + hf;
  const float* krow = ks + (wn * 32 + l32) * LD + hf;
#pragma unroll 8
  for (int kk = 0; kk < D; kk += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qrow[kk], krow[kk], acc, 0, 0, 0);
  // acc[r] holds S[i0 + wm*32 + 8*(r/4) + 4*hf + r%4][j0 + wn*32 + l32]
  const int j = j0 + wn * 32 + l32;
  if (j < nb) {
    float* out = scores + (int64_t)h * nb * nb + j;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + wm * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (i < nb) out[(int64_t)i * nb] = sm_scale * acc[r];
    }
  }
}

// Order-preserving map float -> uint32 (larger float -> larger key), with
// -0.0 folded onto +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroup-wide exclusive scan of one uint64 per thread (256 threads).
__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t x, uint64_t* wave_tot,
                                                             uint64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint64_t base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) base += wave_tot[w];
    all += wave_tot[w];
  }
  *total = all;
  return base + incl - x;
}

// ---------------------------------------------------------------------------
// 3. Ranking and cutoff.  One workgroup per (query block i, head h) row:
//   - keys (orderable(s_j) << 32) | (2^32-1-j) sorted descending with a
//     bitonic network in LDS: score descending, equal scores by lower id;
//   - weights w_r = rint(exp(s_(r) - s_(0)) * 2^40) in fp64, an exact integer
//     inclusive scan along the ranking, target T = fl(p * W);
//   - k_p = 1 + #{r : prefix_r < ceil(T)}, k_i = max(k_p, min(k_min, nb)).
// Integer prefix sums make the cutoff independent of summation order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_select_kernel(
    const float* __restrict__ scores, int nb, int npad, float top_p, int k_min,
    int16_t* __restrict__ ranked, int32_t* __restrict__ row_count,
    int32_t* __restrict__ head_count) {
  __shared__ uint64_t keys[FVA_MAX_BLOCKS];
  __shared__ float srow[FVA_MAX_BLOCKS];
  __shared__ uint64_t wave_tot[4];
  __shared__ int32_t wave_cnt[4];

  const int h = blockIdx.y;
  const int row = h * nb + blockIdx.x;
  const int tid = threadIdx.x;
  const float* s = scores + (int64_t)row * nb;

  for (int j = tid; j < npad; j += 256) {
    if (j < nb) {
      const float f = s[j];
      srow[j] = f;
      keys[j] = ((uint64_t)orderable(f) << 32) | (uint64_t)(0xffffffffu - (uint32_t)j);
    } else {
      keys[j] = 0ull;
    }
  }
  __syncthreads();

  for (int kk = 2; kk <= npad; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < (npad >> 1); i += 256) {
        const int lo = ((i & ~(jj - 1)) << 1) | (i & (jj - 1));
        const int hi = lo | jj;
        const uint64_t a = keys[lo], b = keys[hi];
        const bool desc = (lo & kk) == 0;
        if ((a < b) == desc) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  int16_t* rk = ranked + (int64_t)row * nb;
  for (int r = tid; r < nb; r += 256)
    rk[r] = (int16_t)(0xffffffffu - (uint32_t)(keys[r] & 0xffffffffull));

  int kp;
  const float p = top_p;
  if (p >= 1.0f) {
    kp = nb;
  } else if (!(p > 0.0f)) {
    kp = 0;
  } else {
    // weights along the ranking (pad slots weigh 0)
    const double smax = (double)srow[0xffffffffu - (uint32_t)(keys[0] & 0xffffffffull)];
    __syncthreads();  // every thread has read keys[0]; keys[] is reused for weights
    for (int r = tid; r < nb; r += 256) {
      const double sr = (double)srow[0xffffffffu - (uint32_t)(keys[r] & 0xffffffffull)];
      keys[r] = (uint64_t)rint(exp(sr - smax) * 1099511627776.0);  // 2^40
    }
    __syncthreads();
    // contiguous segment of the ranking per thread, exact integer scan
    const int ept = (nb + 255) / 256;
    const int r0 = min(nb, tid * ept), r1 = min(nb, r0 + ept);
    uint64_t local = 0;
    for (int r = r0; r < r1; ++r) local += keys[r];
    uint64_t total;
    uint64_t prefix = block_exclusive_scan_u64(local, wave_tot, &total);
    const double target = (double)p * (double)total;
    const uint64_t tint = (uint64_t)ceil(target);
    int cnt = 0;
    for (int r = r0; r < r1; ++r) {
      prefix += keys[r];
      cnt += (prefix < tint) ? 1 : 0;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if ((tid & 63) == 0) wave_cnt[tid >> 6] = cnt;
    __syncthreads();
    cnt = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    kp = min(nb, cnt + 1);
  }
  if (tid == 0) {
    const int ki = max(kp, min(k_min, nb));
    row_count[row] = ki;
    atomicAdd(&head_count[h], ki);
  }
}

// ---------------------------------------------------------------------------
// Launch sequence for fva_route.
// ---------------------------------------------------------------------------
int launch_route(const fva_problem& p, int nb, const void* q, const void* k, const void* v,
                 float* scores, int16_t* ranked, int32_t* row_count,
                 int32_t* head_count, int32_t* order, void* kv, float* qbar, float* kbar,
                 float sm_scale, hipStream_t stream) {
  const OrderGeo geo = make_order_geo(p);
  const dim3 pool_grid(nb, p.num_heads, 3);
  bf16_t* kp = (bf16_t*)kv;
  bf16_t* vt = kp + (int64_t)p.num_heads * nb * p.block * p.head_dim;
  if (p.head_dim == 128)
    route_pool_kernel<128><<<pool_grid, 256, 0, stream>>>(
        (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, p.stride_head, p.stride_token, geo,
        p.block, nb, p.num_heads, qbar, kbar, order, head_count, kp, vt);
  else
    route_pool_kernel<64><<<pool_grid, 256, 0, stream>>>(
        (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, p.stride_head, p.stride_token, geo,
        p.block, nb, p.num_heads, qbar, kbar, order, head_count, kp, vt);
  int st = record_hip_error(hipGetLastError(), "route_pool launch");
  if (st) return st;

  const dim3 sc_grid((nb + 63) / 64, (nb + 63) / 64, p.num_heads);
  if (p.head_dim == 128)
    route_scores_kernel<128><<<sc_grid, 256, 0, stream>>>(qbar, kbar, nb, sm_scale, scores);
  else
    route_scores_kernel<64><<<sc_grid, 256, 0, stream>>>(qbar, kbar, nb, sm_scale, scores);
  st = record_hip_error(hipGetLastError(), "route_scores launch");
  if (st) return st;

  int npad = 1;
  while (npad < nb) npad <<= 1;
  const dim3 sel_grid(nb, p.num_heads);
  route_select_kernel<<<sel_grid, 256, 0, stream>>>(scores, nb, npad, p.top_p, p.k_min,
                                                    ranked, row_count, head_count);
  return record_hip_error(hipGetLastError(), "route_select launch");
}

}  // namespace fva
