// Block-sparse attention forward over the kept key blocks of each
// (head, query-block) tile, run from a persistent heaviest-first tile queue.
//
// GSRS paper S3.2: block-sparse FlashAttention walks only the selected key
// blocks inside its tiling loop, skipping the others' compute and memory
// traffic.  GSRS A.1: online softmax keeps a running maximum and denominator,
// rescales what was accumulated when the maximum grows, and has the true
// log-sum-exp only after the last block.  FVAttn S3.2: the order in which work
// is placed changes where it runs, never what is computed.
//
// Layout of one workgroup (BLK/32 waves, one tile of BLK query rows):
//   - wave w owns query rows 32w .. 32w+31 of the tile; lane l holds query
//     32w + (l % 32), the two half-waves (l / 32) split every 32-key group;
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows from LDS,
//     B = Q fragments kept in registers for the whole tile, so every lane owns
//     one query column and the softmax row statistics stay in-lane (one
//     cross-half shuffle for the maximum per block);
//   - O^T += V^T P^T: A = V^T from LDS (V is transposed while staging),
//     B = P converted to bf16 straight from the S^T accumulators; the key
//     permutation implied by the accumulator layout is applied to the V^T
//     reads, so no register shuffles are needed;
//   - K and V rows are gathered through the order table (position -> token).
#include "fva_common.h"

namespace fva {

struct AttnArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  float* lse;
  const int32_t* order;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* tile_order;
  uint32_t* tile_counter;
  int64_t stride_head, stride_token;
  int n, nb, num_tiles;
  float scale_log2;  // sm_scale * log2(e)
};

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void sparse_attn_fwd_kernel(AttnArgs a) {
  constexpr int NW = BLK / 32;  // waves per workgroup
  constexpr int NT = NW * 64;   // threads per workgroup
  constexpr int KS = BLK / 32;  // 32-key sub-tiles of S^T
  constexpr int DS = D / 16;    // k-steps of S^T = K Q^T
  constexpr int DO = D / 32;    // 32-row sub-tiles of O^T
  constexpr int PS = BLK / 16;  // k-steps of O^T += V^T P^T
  constexpr int KLD = D + 8;    // LDS row stride of K (elements)
  constexpr int VLD = BLK + 4;  // LDS row stride of V^T (elements)
  constexpr int CH = D / 8;     // 16-byte chunks per K/V row
  constexpr int GPI = NT / CH;  // 4-row groups staged per pass
  constexpr int ITS = (BLK / 4) / GPI;
  static_assert(ITS >= 1 && (BLK / 4) % GPI == 0, "staging layout");

  __shared__ __attribute__((aligned(16))) bf16_t ks[BLK * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t vt[D * VLD];
  __shared__ int s_tile;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  for (;;) {
    if (tid == 0) s_tile = (int)atomicAdd(&a.tile_counter[0], 1u);
    __syncthreads();
    const int idx = s_tile;
    __syncthreads();
    if (idx >= a.num_tiles) break;

    const int t = a.tile_order[idx];
    const int h = t / a.nb;
    const int i = t - h * a.nb;
    const int64_t hoff = (int64_t)h * a.stride_head;
    const bf16_t* kh = a.k + hoff;
    const bf16_t* vh = a.v + hoff;

    // Q fragments of this lane's query row (zeros past the end of the sequence)
    const int qtok = a.order[i * BLK + wave * 32 + l32];
    bf16x8 qf[DS];
    {
      const bf16_t* qrow = a.q + hoff + (int64_t)(qtok < 0 ? 0 : qtok) * a.stride_token + hf * 8;
#pragma unroll
      for (int d = 0; d < DS; ++d) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qtok >= 0) w = *reinterpret_cast<const u32x4*>(qrow + d * 16);
        qf[d] = __builtin_bit_cast(bf16x8, w);
      }
    }

    f32x16 acc_o[DO];
#pragma unroll
    for (int d = 0; d < DO; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[d][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int c0 = a.row_ptr[t], c1 = a.row_ptr[t + 1];
    for (int c = c0; c < c1; ++c) {
      const int j = a.col_idx[c];
      __syncthreads();  // all waves are done reading the previous K/V tile

      // ---- stage K (row-major) and V (transposed) of key block j in LDS ----
#pragma unroll
      for (int it = 0; it < ITS; ++it) {
        const int g = tid / CH + it * GPI;  // rows 4g .. 4g+3 of the block
        const int ch = tid % CH;
        const int32_t* tp = a.order + j * BLK + 4 * g;
        const int t0 = tp[0], t1 = tp[1], t2 = tp[2], t3 = tp[3];
        const int toks[4] = {t0, t1, t2, t3};
        u32x4 kr[4], vr[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          kr[rr] = u32x4{0u, 0u, 0u, 0u};
          vr[rr] = u32x4{0u, 0u, 0u, 0u};
          if (toks[rr] >= 0) {
            const int64_t off = (int64_t)toks[rr] * a.stride_token + ch * 8;
            kr[rr] = *reinterpret_cast<const u32x4*>(kh + off);
            vr[rr] = *reinterpret_cast<const u32x4*>(vh + off);
          }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<u32x4*>(&ks[(4 * g + rr) * KLD + ch * 8]) = kr[rr];
        // transpose 4 keys x 8 features into 8 rows of V^T, 4 keys each
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t w0 = vr[0][m], w1 = vr[1][m], w2 = vr[2][m], w3 = vr[3][m];
          const u32x2 even = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
          const u32x2 odd = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
          *reinterpret_cast<u32x2*>(&vt[(ch * 8 + 2 * m) * VLD + 4 * g]) = even;
          *reinterpret_cast<u32x2*>(&vt[(ch * 8 + 2 * m + 1) * VLD + 4 * g]) = odd;
        }
      }
      __syncthreads();

      // ---- S^T = K Q^T for this wave's 32 queries ----
      f32x16 s[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kk][r] = 0.f;
#pragma unroll
        for (int d = 0; d < DS; ++d) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(&ks[(kk * 32 + l32) * KLD + d * 16 + hf * 8]);
          s[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), qf[d], s[kk],
                                                          0, 0, 0);
        }
      }
      // s[kk][r] = q . k for key kk*32 + 8*(r/4) + 4*hf + r%4 of block j

      // keys past the end of the sequence (only in the last block) get -inf
      const int valid = min(BLK, a.n - j * BLK);
      if (valid < BLK) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kk * 32 + 8 * (r >> 2) + 4 * hf + (r & 3) >= valid) s[kk][r] = -INFINITY;
      }

      // ---- online softmax (base 2), row statistics per lane ----
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kk][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(fmaf(s[kk][r], a.scale_log2, -m_new));
          s[kk][r] = p;
          rs += p;
        }
      l_run = fmaf(l_run, alpha, rs);
#pragma unroll
      for (int d = 0; d < DO; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[d][r] *= alpha;

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (__bf16)s[ps >> 1][(ps & 1) * 8 + e];
#pragma unroll
        for (int d = 0; d < DO; ++d) {
          const bf16_t* vrow = &vt[(d * 32 + l32) * VLD + ps * 16 + hf * 4];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
          acc_o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf, acc_o[d],
                                                             0, 0, 0);
        }
      }
    }

    // ---- normalise and store O (and LSE) for this lane's query ----
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (qtok >= 0) {
      const float inv = 1.0f / l_tot;
      bf16_t* orow = a.o + hoff + (int64_t)qtok * a.stride_token;
#pragma unroll
      for (int d = 0; d < DO; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 w = {pack_bf16x2(acc_o[d][4 * g] * inv, acc_o[d][4 * g + 1] * inv),
                           pack_bf16x2(acc_o[d][4 * g + 2] * inv, acc_o[d][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d * 32 + 8 * g + 4 * hf) = w;
        }
      if (hf == 0 && a.lse != nullptr)
        a.lse[(int64_t)h * a.n + qtok] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
    }
  }

  // Queue drain: the last workgroup to leave resets the counters, so the
  // buffer is {0, 0} again for the next call.
  if (tid == 0) {
    const uint32_t done = atomicAdd(&a.tile_counter[1], 1u);
    if (done == gridDim.x - 1) {
      atomicExch(&a.tile_counter[0], 0u);
      atomicExch(&a.tile_counter[1], 0u);
    }
  }
}

template <int D, int BLK>
static int launch_attn_t(const AttnArgs& args, int grid, hipStream_t stream) {
  sparse_attn_fwd_kernel<D, BLK><<<grid, BLK * 2, 0, stream>>>(args);
  return record_hip_error(hipGetLastError(), "sparse_attn_fwd launch");
}

template <int D, int BLK>
static int occupancy_t(int* blocks) {
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, sparse_attn_fwd_kernel<D, BLK>,
                                                           BLK * 2, 0);
}

// Resident workgroups per CU for the (d, B) instantiation, or -1 on error.
int attn_blocks_per_cu(int d, int block) {
  int b = 0;
  hipError_t e;
  if (d == 128 && block == 128) e = (hipError_t)occupancy_t<128, 128>(&b);
  else if (d == 128) e = (hipError_t)occupancy_t<128, 64>(&b);
  else if (block == 128) e = (hipError_t)occupancy_t<64, 128>(&b);
  else e = (hipError_t)occupancy_t<64, 64>(&b);
  if (e != hipSuccess) return -1;
  return b < 1 ? 1 : b;
}

int launch_attn(const fva_problem& p, int nb, int grid, const void* q, const void* k,
                const void* v, const int32_t* order, const int32_t* row_ptr,
                const int32_t* col_idx, const int32_t* tile_order, uint32_t* tile_counter,
                void* o, float* lse, float sm_scale, hipStream_t stream) {
  AttnArgs a;
  a.q = (const bf16_t*)q;
  a.k = (const bf16_t*)k;
  a.v = (const bf16_t*)v;
  a.o = (bf16_t*)o;
  a.lse = lse;
  a.order = order;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.tile_order = tile_order;
  a.tile_counter = tile_counter;
  a.stride_head = p.stride_head;
  a.stride_token = p.stride_token;
  a.n = p.seq_len;
  a.nb = nb;
  a.num_tiles = p.num_heads * nb;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  if (p.head_dim == 128 && p.block == 128) return launch_attn_t<128, 128>(a, grid, stream);
  if (p.head_dim == 128) return launch_attn_t<128, 64>(a, grid, stream);
  if (p.block == 128) return launch_attn_t<64, 128>(a, grid, stream);
  return launch_attn_t<64, 64>(a, grid, stream);
}

}  // namespace fva
