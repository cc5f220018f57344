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
//   - O^T += V^T P^T: A = V^T fragments, one 16-byte LDS load each from a
//     V^T sub-tile whose columns are already in the order the S^T
//     accumulators hold their keys; B = P converted to bf16 straight from
//     the S^T accumulators, so no register shuffles are needed;
//   - K and V come re-laid out in the video-aware order by the routing pass
//     or by fva_kv_layout (K row-major per position, V transposed per
//     64-position sub-block with its columns in the order the S^T
//     accumulators hold their keys), so the kernel streams contiguous
//     sub-tiles into a ring of LDS slots with direct buffer -> LDS loads
//     whose addresses are per-lane constants plus one scalar offset, and
//     reads its V^T operands with plain 16-byte LDS loads.
#include <type_traits>

#ifndef FVA_KB
#define FVA_KB 64
#endif
#ifndef FVA_NBUF
#define FVA_NBUF 2
#endif

#include "fva_common.h"

namespace fva {

struct AttnArgs {
  const bf16_t* q;
  const bf16_t* kp;  // [H][npad][d], K in position order (zero rows past N)
  const bf16_t* vt;  // [H][npad/64][d][64], V^T per 64-position sub-block
  bf16_t* o;
  float* lse;
  float* block_lse;  // optional: per kept (row, block) pair, B per-query block LSEs
  const int32_t* order;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* work_order;  // tile * 2 + part
  const int32_t* plan_meta;   // [0] items, [1] split tiles, [2 + t] split slot of tile t
  uint32_t* tile_counter;
  float* partial;             // per split slot and part: O^T (unnormalised), max, denominator
  int64_t stride_head, stride_token;
  int n, nb, num_tiles;
  int npad;          // nb * B
  float scale_log2;  // sm_scale * log2(e)
  int64_t* item_trace;        // traced launches only: FVA_TRACE_FIELDS per work item
};

// Buffer resource over one head's rows of the re-laid-out K or V: raw byte
// addressing, num_records = bytes (loads beyond return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const bf16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits until at most n vector memory operations are
// outstanding and leaves the other counters alone (GFX9 encoding).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Direct buffer -> LDS load of 16 bytes per lane from byte offset
// voff + soff: lane l's bytes land at lds_base + 16*l (lds_base and soff
// wave-uniform).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, bf16_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, (int)voff, soff, 0, 0);
}

// Reductions over the two half-waves (lanes l and l ^ 32), in every lane,
// without going through LDS: v_permlane32_swap of x with itself leaves x's
// own and other-half values in the two results, in some order per lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_total(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Chunk swizzle of the LDS tiles: logical 16-byte chunk c of row r is stored
// at position c ^ swz(r).  For 16 chunks per row (K, d = 128) swz swaps the
// two 2-bit halves of r mod 16, a bijection on any 16 consecutive rows (the
// K operand reads 32 rows at one logical chunk).  For 8 chunks per row (K at
// d = 64, and every V^T tile: 64 keys per row) rows alternate between the two
// bank halves, so swz uses r / 2.
template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 1) & 7;
}

// Placement of the calling wave: XCC id (hardware register 20 on this
// family) in bits 32.., the hardware id register (wave, SIMD, CU, shader
// array and engine fields) below.
__device__ __forceinline__ int64_t wave_placement() {
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
  const uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20);
  return ((int64_t)xcc << 32) | hw;
}

// One workgroup = one (head, query block) tile at a time; KB = keys per
// sub-block (a kept key block of BLK keys is processed as BLK/KB sub-blocks,
// numbered u = 0 .. nsub-1 along the tile's kept list).  K and V^T sub-tiles
// stream through a ring of NBUF LDS slots: sub-block u+NBUF-1 is issued while
// u is computed.  Two waves per SIMD; the B = 64, d = 128 shape, whose
// 74 KB of LDS allows one wave per SIMD anyway, asks for one.
template <int D, int BLK, int KB, int NBUF, bool TRACE>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(BLK == 64 && D == 128 ? 1 : 2,
                                                                          BLK == 64 && D == 128 ? 1 : 2)))
void sparse_attn_fwd_kernel(AttnArgs a) {
  constexpr int NW = BLK / 32;   // waves per workgroup (32 query rows each)
  constexpr int SUB = BLK / KB;  // sub-blocks per kept key block
  constexpr int KS = KB / 32;    // 32-key sub-tiles of S^T per sub-block
  constexpr int DS = D / 16;     // k-steps of S^T = K Q^T
  constexpr int DO = D / 32;     // 32-row sub-tiles of O^T
  constexpr int PS = KB / 16;    // k-steps of O^T += V^T P^T
  constexpr int CH = D / 8;      // 16-byte chunks per K/V row
  constexpr int RW = 64 / CH;    // K rows written by one wave-wide LDS-DMA load
  constexpr int RPW = KB / NW;   // K rows each wave stages per sub-block
  constexpr int NI = RPW / RW;   // K LDS-DMA loads per wave per sub-block
  constexpr int VCH = KB / 8;    // 16-byte chunks per V^T row
  constexpr int VRW = 64 / VCH;  // V^T rows written by one LDS-DMA load
  constexpr int VRPW = D / NW;   // V^T rows each wave stages
  constexpr int NIV = VRPW / VRW;  // V^T LDS-DMA loads per wave per sub-block
  constexpr int TILE = KB * D;   // elements of one K or V^T sub-tile
  static_assert(NW * 32 == BLK && SUB * KB == BLK && NI >= 1 && NI * RW == RPW, "tiling");
  static_assert(KB == 64 && NIV >= 1 && NIV * VRW == VRPW, "V^T tiling (64-key sub-blocks)");
  static_assert(NBUF == 2, "two K and two V^T slots");
  constexpr int DA = DS < 2 ? DS : 2;  // k-steps of S^T(u+1) issued with the row maximum

  // K sub-tiles: KB rows (keys) of D elements; V^T sub-tiles: D rows of KB
  // keys; 16-byte chunk c of row r stored at position c ^ swz(r).  The ring slots are separate LDS
  // objects and the loop is unrolled by NBUF, so the compiler can tell that
  // loads into one slot never alias reads of another and does not wait for
  // them.
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds2[NBUF > 2 ? TILE : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds2[NBUF > 2 ? TILE : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds3[NBUF > 3 ? TILE : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds3[NBUF > 3 ? TILE : 8];
  __shared__ int s_tile;
  auto kslot = [&](auto b) -> bf16_t* {
    constexpr int B = decltype(b)::value;
    if constexpr (B == 0) return k_lds0;
    else if constexpr (B == 1) return k_lds1;
    else if constexpr (B == 2) return k_lds2;
    else return k_lds3;
  };
  auto vslot = [&](auto b) -> bf16_t* {
    constexpr int B = decltype(b)::value;
    if constexpr (B == 0) return v_lds0;
    else if constexpr (B == 1) return v_lds1;
    else if constexpr (B == 2) return v_lds2;
    else return v_lds3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  // LDS-DMA: byte offset (inside one sub-block's contiguous K or V^T
  // sub-tile) of the logical chunk that lands at this lane's position
  uint32_t kdma[NI], vdma[NIV];
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int row = wave * RPW + m * RW + lane / CH;
    kdma[m] = (uint32_t)(row * D + ((lane % CH) ^ swz<CH>(row)) * 8) * 2u;
  }
#pragma unroll
  for (int m = 0; m < NIV; ++m) {
    const int row = wave * VRPW + m * VRW + lane / VCH;
    vdma[m] = (uint32_t)(row * KB + ((lane % VCH) ^ swz<VCH>(row)) * 8) * 2u;
  }
  const uint32_t head_bytes = (uint32_t)a.npad * D * 2u;
  const int num_items = a.plan_meta[0];

  // Work items: workgroup w starts with item w (so the workgroups do not all
  // hit the counter at launch); later items come from the queue counter,
  // offset by the grid size, claimed when a workgroup becomes free (claiming
  // earlier would reserve items for busy workgroups and unbalance the tail).
  int idx = blockIdx.x;
  while (idx < num_items) {

    int64_t rt0 = 0, clk0 = 0;
    if constexpr (TRACE) {
      rt0 = (int64_t)__builtin_amdgcn_s_memrealtime();
      clk0 = (int64_t)__builtin_amdgcn_s_memtime();
    }
    // work item: a whole tile, or one part of a split tile's kept list
    const int item = a.work_order[idx];
    const int t = item >> 1;
    const int part = item & 1;
    const int slot = a.plan_meta[2 + t];
    const int h = t / a.nb;
    const int i = t - h * a.nb;
    const int64_t hoff = (int64_t)h * a.stride_head;
    const int64_t ph = (int64_t)h * a.npad * D;
    const __amdgpu_buffer_rsrc_t rk = head_rsrc(a.kp + ph, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = head_rsrc(a.vt + ph, head_bytes);

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
    float blk_l = 0.f;  // this lane's share of the current key block's denominator

    // Per-lane LDS operand offsets (elements).  The swizzle depends on the row
    // modulo 16 only, which is the same for every 32-key sub-tile (K) and
    // every 16-key k-step (V), so sub-tiles and k-steps differ by constants.
    int koff[DS];
#pragma unroll
    for (int d = 0; d < DS; ++d) koff[d] = l32 * D + ((2 * d + hf) ^ swz<CH>(l32)) * 8;
    // V^T operand of k-step ps: row 32dt + l32, logical chunk 2ps + hf (its 8
    // columns are the keys of this lane's P^T operand); the swizzle of rows
    // 32dt + l32 does not depend on dt
    int voff[PS];
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) voff[ps] = l32 * KB + ((2 * ps + hf) ^ swz<VCH>(l32)) * 8;

    int c0 = a.row_ptr[t];
    int ncols = a.row_ptr[t + 1] - c0;
    if (slot >= 0) {
      const int first = (ncols + 1) >> 1;
      if (part) {
        c0 += first;
        ncols -= first;
      } else {
        ncols = first;
      }
    }
    const int nsub = ncols * SUB;
    // first sequence position of sub-block u; the kept key-block ids come
    // through the scalar cache (uniform addresses in the constant address
    // space: the list is not written while the kernel runs), so no LDS copy
    // of the list and no vector load stands before a step's first MFMA
    typedef const __attribute__((address_space(4))) int32_t* const_i32p;
    const const_i32p cols = (const_i32p)(a.col_idx + c0);
    auto sub_pos = [&](int u) { return cols[u / SUB] * BLK + (u % SUB) * KB; };

    // K and V^T sub-tiles of sub-block u: both start at byte pos * D * 2 of
    // their head's re-laid-out buffer
    auto issue_k = [&](bf16_t* kt, int u) {
      const int soff = __builtin_amdgcn_readfirstlane(sub_pos(u) * D * 2);
#pragma unroll
      for (int m = 0; m < NI; ++m) lds_dma16(rk, kdma[m], soff, kt + (wave * RPW + m * RW) * D);
    };
    auto issue_v = [&](bf16_t* vt, int u) {
      const int soff = __builtin_amdgcn_readfirstlane(sub_pos(u) * D * 2);
#pragma unroll
      for (int m = 0; m < NIV; ++m) lds_dma16(rv, vdma[m], soff, vt + (wave * VRPW + m * VRW) * KB);
    };
    // k-step d of S^T = K Q^T for the KS 32-key sub-tiles of one sub-block
    // (the KS accumulation chains are independent, so their MFMAs interleave)
    auto s_kstep = [&](f32x16(&sacc)[KS], const bf16_t* ks, int d) {
      u32x4 kf[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) kf[kk] = *reinterpret_cast<const u32x4*>(&ks[kk * 32 * D + koff[d]]);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        sacc[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[kk]), qf[d], sacc[kk],
                                                           0, 0, 0);
    };

    // Software pipeline over the sub-blocks: the S^T MFMAs of sub-block u+1
    // run while this wave's softmax of sub-block u is on the vector unit, so
    // a wave keeps the matrix unit fed through its own vector work.  K runs
    // one sub-block ahead of V: during step u the LDS ring holds K(u+1) and
    // V(u) and receives K(u+2) and V(u+1).
    issue_k(k_lds0, 0);
    issue_v(v_lds0, 0);
    if (nsub > 1) issue_k(k_lds1, 1);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 sa[KS], sb[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[kk][r] = 0.f;
#pragma unroll
    for (int d = 0; d < DS; ++d) s_kstep(sa, k_lds0, d);
    __syncthreads();  // every wave has read K slot 0, which receives K(2)

    // step u: sc holds S^T(u) (raw q.k); sn receives S^T(u+1).  At the last
    // step the S^T of a sub-block past the end is computed from whatever the
    // K slot holds and never used.
    auto step = [&](auto cur_tag, f32x16(&sc)[KS], f32x16(&sn)[KS], int u) {
      constexpr int CUR = decltype(cur_tag)::value;
      constexpr int NXT = CUR ^ 1;
      const bf16_t* kn = kslot(std::integral_constant<int, NXT>{});
      const bf16_t* vs = vslot(std::integral_constant<int, CUR>{});
      const int pos = sub_pos(u);
      if (u + 2 < nsub) issue_k(kslot(std::integral_constant<int, CUR>{}), u + 2);
      if (u + 1 < nsub) issue_v(vslot(std::integral_constant<int, NXT>{}), u + 1);

      // keys past the end of the sequence (only in the last block) get -inf
      // (a real branch: the empty asm keeps the compiler from turning it
      // into selects that would run on every sub-block)
      const int valid = a.n - pos;
      if (__builtin_expect(valid < KB, 0)) {
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kk * 32 + 8 * (r >> 2) + 4 * hf + (r & 3) >= valid) sc[kk][r] = -INFINITY;
      }

      // ---- phase A: the first k-steps of S^T(u+1) with the row maximum of
      // S^T(u).  The running maximum m_run is only raised when a sub-block's
      // maximum exceeds it by more than 8 (a factor 2^8), so most sub-blocks
      // skip the rescale of the accumulators; weights then stay below 2^8,
      // and the final division by the matching denominator makes the result
      // exact.
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[kk][r] = 0.f;
#pragma unroll
      for (int d = 0; d < DA; ++d) s_kstep(sn, kn, d);
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kk][r]);
      mx = halves_max(mx) * a.scale_log2;
      if (__any(mx > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        blk_l *= alpha;
#pragma unroll
        for (int d = 0; d < DO; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[d][r] *= alpha;
      }

      // ---- phase B: the remaining k-steps of S^T(u+1), the weights of
      // S^T(u) (base 2), and O^T += V^T P^T for sub-block u ----
#pragma unroll
      for (int d = DA; d < DS; ++d) s_kstep(sn, kn, d);
      float rs = 0.f;
      bf16x8 pf[PS];
#pragma unroll
      for (int ps = 0; ps < PS; ++ps)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[ps >> 1][(ps & 1) * 8 + e], a.scale_log2, -m_run));
          rs += p;
          pf[ps][e] = (__bf16)p;
        }
      l_run += rs;
      blk_l += rs;
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        u32x4 vf[DO];
#pragma unroll
        for (int d = 0; d < DO; ++d) vf[d] = *reinterpret_cast<const u32x4*>(&vs[d * 32 * KB + voff[ps]]);
#pragma unroll
        for (int d = 0; d < DO; ++d)
          acc_o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[d]), pf[ps], acc_o[d],
                                                             0, 0, 0);
      }

      // GSRS S5.3 phase 1: after the last sub-block of a kept key block,
      // each query's log-sum-exp over that block's keys (natural log, same
      // scale as the row LSE); normalised by the final row LSE later
      const bool rec = a.block_lse != nullptr && (u % SUB) == SUB - 1;
      float blk_lse = 0.f;
      if (rec) {
        const float tot = halves_total(blk_l);
        blk_lse = (m_run + __log2f(tot)) * 0.69314718055994531f;
        blk_l = 0.f;
      }

      // K(u+2) and V(u+1) have landed for every wave and every wave is done
      // with K(u+1) and V(u)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
      // stored after the wait, so that the store completes behind the next
      // sub-block's work instead of stalling this one
      if (rec && hf == 0) a.block_lse[(int64_t)(c0 + u / SUB) * BLK + wave * 32 + l32] = blk_lse;
    };
    for (int u = 0; u < nsub; u += 2) {
      step(std::integral_constant<int, 0>{}, sa, sb, u);
      if (u + 1 < nsub) step(std::integral_constant<int, 1>{}, sb, sa, u + 1);
    }

    // ---- normalise and store O (and LSE) for this lane's query, or leave
    // the part's partial result for the merge ----
    const float l_tot = halves_total(l_run);
    if (slot >= 0) {
      float* pp = a.partial + ((int64_t)slot * 2 + part) * (BLK * D + 2 * BLK);
      const int qrow = wave * 32 + l32;
#pragma unroll
      for (int d = 0; d < DO; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(pp + qrow * D + d * 32 + 8 * g + 4 * hf) =
              f32x4{acc_o[d][4 * g], acc_o[d][4 * g + 1], acc_o[d][4 * g + 2], acc_o[d][4 * g + 3]};
      if (hf == 0) {
        pp[BLK * D + qrow] = m_run;
        pp[BLK * D + BLK + qrow] = l_tot;
      }
    } else if (qtok >= 0) {
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
    if constexpr (TRACE) {
      if (tid == 0) {
        const int64_t clk1 = (int64_t)__builtin_amdgcn_s_memtime();
        const int64_t rt1 = (int64_t)__builtin_amdgcn_s_memrealtime();
        int64_t* tr = a.item_trace + (int64_t)idx * FVA_TRACE_FIELDS;
        tr[0] = rt0;
        tr[1] = rt1;
        tr[2] = clk0;
        tr[3] = clk1;
        tr[4] = wave_placement();
        tr[5] = blockIdx.x;
      }
    }
    if (tid == 0) s_tile = (int)gridDim.x + (int)atomicAdd(&a.tile_counter[0], 1u);
    __syncthreads();  // s_tile is set
    idx = s_tile;
    __syncthreads();
  }
}

constexpr int KEYS_PER_STEP = FVA_KB;
constexpr int RING_SLOTS = FVA_NBUF;

template <int D, int BLK>
static int launch_attn_t(const AttnArgs& args, int grid, hipStream_t stream) {
  if (args.item_trace)
    sparse_attn_fwd_kernel<D, BLK, KEYS_PER_STEP, RING_SLOTS, true><<<grid, BLK * 2, 0, stream>>>(args);
  else
    sparse_attn_fwd_kernel<D, BLK, KEYS_PER_STEP, RING_SLOTS, false><<<grid, BLK * 2, 0, stream>>>(args);
  return record_hip_error(hipGetLastError(), "sparse_attn_fwd launch");
}

// Merge of split tiles (BLK/32 workgroups per split slot, 32 query rows each;
// groups of them stride over the slots), run after the attention launch
// (this launch also resets the queue counter):
// the two parts' partial results combine as in the online softmax (GSRS A.1):
// with
// m = max(m0, m1) and weights a_p = 2^(m_p - m), O = (a0 O0 + a1 O1) /
// (a0 l0 + a1 l1) and LSE = (m + log2(a0 l0 + a1 l1)) ln 2.  Part 0 and part 1
// enter the formula in that order whichever finished last, so the result does
// not depend on the order the queue handed them out.
template <int D, int BLK>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ partial,
                                                        const int32_t* __restrict__ plan_meta,
                                                        const int32_t* __restrict__ order, int rows, int nb,
                                                        int n, int64_t stride_head, int64_t stride_token,
                                                        bf16_t* __restrict__ o, float* __restrict__ lse,
                                                        uint32_t* __restrict__ tile_counter) {
  // a thread takes 4 output columns of NP rows and issues all its loads
  // before any arithmetic
  constexpr int WPS = BLK / 32;      // workgroups per slot
  constexpr int CPR = D / 4;         // 4-float chunks per row
  constexpr int RPP = 256 / CPR;     // rows per pass
  constexpr int NP = 32 / RPP;       // passes
  const int r0 = (blockIdx.x % WPS) * 32;
  // the attention launch has finished: reset the queue for the next call
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    atomicExch(&tile_counter[0], 0u);
    atomicExch(&tile_counter[1], 0u);
  }
  // split slots in a grid-stride loop: the grid is sized by the device, not
  // by the number of split tiles, which only the device knows
  const int ns = plan_meta[1];
  for (int s = blockIdx.x / WPS; s < ns; s += gridDim.x / WPS) {
    const int t = plan_meta[2 + rows + s];
    const int h = t / nb, i = t - h * nb;
    constexpr int PART = BLK * D + 2 * BLK;
    const float* p0 = partial + (int64_t)s * 2 * PART;
    const float* p1 = p0 + PART;
    const int c = (threadIdx.x % CPR) * 4;
    int tok[NP];
    float m0[NP], m1[NP], l0[NP], l1[NP];
    f32x4 x0[NP], x1[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int q = r0 + j * RPP + threadIdx.x / CPR;
      tok[j] = order[i * BLK + q];
      m0[j] = p0[BLK * D + q];
      m1[j] = p1[BLK * D + q];
      l0[j] = p0[BLK * D + BLK + q];
      l1[j] = p1[BLK * D + BLK + q];
      x0[j] = *reinterpret_cast<const f32x4*>(p0 + q * D + c);
      x1[j] = *reinterpret_cast<const f32x4*>(p1 + q * D + c);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (tok[j] < 0) continue;
      const float m = fmaxf(m0[j], m1[j]);
      const float a0 = __builtin_amdgcn_exp2f(m0[j] - m), a1 = __builtin_amdgcn_exp2f(m1[j] - m);
      const float l = a0 * l0[j] + a1 * l1[j];
      const float inv = 1.0f / l;
      const u32x2 w = {pack_bf16x2((a0 * x0[j][0] + a1 * x1[j][0]) * inv, (a0 * x0[j][1] + a1 * x1[j][1]) * inv),
                       pack_bf16x2((a0 * x0[j][2] + a1 * x1[j][2]) * inv, (a0 * x0[j][3] + a1 * x1[j][3]) * inv)};
      *reinterpret_cast<u32x2*>(o + (int64_t)h * stride_head + (int64_t)tok[j] * stride_token + c) = w;
      if (c == 0 && lse != nullptr) lse[(int64_t)h * n + tok[j]] = (m + __log2f(l)) * 0.69314718055994531f;
    }
  }
}

template <int D, int BLK>
static int occupancy_t(int* blocks) {
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks, sparse_attn_fwd_kernel<D, BLK, KEYS_PER_STEP, RING_SLOTS, false>, BLK * 2, 0);
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

template <int D, int BLK>
static int launch_merge_t(const AttnArgs& a, int rows, hipStream_t stream) {
  // one group of BLK/32 workgroups per split slot, up to one group per
  // compute unit; more split tiles than groups are taken in turn
  int slots = rows < FVA_MAX_SPLITS ? rows : FVA_MAX_SPLITS;
  const int cus = device_cu_count();
  if (cus > 0 && cus < slots) slots = cus;
  const int grid = slots * (BLK / 32);
  attn_merge_kernel<D, BLK><<<grid, 256, 0, stream>>>(a.partial, a.plan_meta, a.order, rows, a.nb, a.n,
                                                      a.stride_head, a.stride_token, a.o, a.lse,
                                                      a.tile_counter);
  return record_hip_error(hipGetLastError(), "attn_merge launch");
}

int launch_attn(const fva_problem& p, int nb, int grid, const void* q, const void* kv,
                const int32_t* order, const int32_t* row_ptr, const int32_t* col_idx,
                const int32_t* work_order, const int32_t* plan_meta, uint32_t* tile_counter,
                void* o, float* lse, float* block_lse, void* workspace, float sm_scale,
                int64_t* item_trace, hipStream_t stream) {
  const int npad = nb * p.block;
  const bf16_t* kp = (const bf16_t*)kv;
  const bf16_t* vt = kp + (int64_t)p.num_heads * npad * p.head_dim;
  AttnArgs a;
  a.q = (const bf16_t*)q;
  a.kp = kp;
  a.vt = vt;
  a.npad = npad;
  a.o = (bf16_t*)o;
  a.lse = lse;
  a.block_lse = block_lse;
  a.order = order;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.work_order = work_order;
  a.plan_meta = plan_meta;
  a.tile_counter = tile_counter;
  a.partial = (float*)workspace;
  a.item_trace = item_trace;
  a.stride_head = p.stride_head;
  a.stride_token = p.stride_token;
  a.n = p.seq_len;
  a.nb = nb;
  a.num_tiles = p.num_heads * nb;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  const int rows = p.num_heads * nb;
  int st;
  if (p.head_dim == 128 && p.block == 128) {
    if ((st = launch_attn_t<128, 128>(a, grid, stream))) return st;
    return launch_merge_t<128, 128>(a, rows, stream);
  }
  if (p.head_dim == 128) {
    if ((st = launch_attn_t<128, 64>(a, grid, stream))) return st;
    return launch_merge_t<128, 64>(a, rows, stream);
  }
  if (p.block == 128) {
    if ((st = launch_attn_t<64, 128>(a, grid, stream))) return st;
    return launch_merge_t<64, 128>(a, rows, stream);
  }
  if ((st = launch_attn_t<64, 64>(a, grid, stream))) return st;
  return launch_merge_t<64, 64>(a, rows, stream);
}

}  // namespace fva
