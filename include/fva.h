/*
 * fva.h -- C ABI of the adaptive block-sparse attention library (libfva.so)
 * for video diffusion transformers on AMD Instinct MI355X (gfx950).
 *
 * One call of the hot path is three stream-ordered entry points:
 *
 *   fva_route            video-aware order, pooled Q/K block scores, ranking,
 *                        Top-p cutoff with a Top-k floor, per-head counts;
 *                        optionally also K and V re-laid out in the order
 *   fva_plan             refill of next-ranked blocks, CSR block mask,
 *                        heaviest-first (LPT) tile order, queue reset
 *   fva_sparse_attn_fwd  block-sparse attention forward over the kept blocks,
 *                        run from a persistent tile queue
 *
 * Attention over a mask the caller already holds (a reused or hand-built
 * CSR) needs no routing: fva_kv_layout puts the caller's K and V into the
 * layout the attention reads, and fva_schedule builds the work list of any
 * CSR mask.
 *
 * Sources (page title, section) for what each call computes:
 *   "FVAttn: Adaptive Sparse Attention with Runtime Load Balancing for Video
 *    Generation": S2.1 (scores s_{h,i,j}, mask M_{h,i,j}, Top-p, Top-k floor),
 *    S2.2 Eq 1 (per-head workload), S3.1 (reordering, pooled Q/K similarity,
 *    density and ranking from the same routing pass), S3.2 (runtime load
 *    balancing moves work without changing it), S3.3 (slack-aware
 *    augmentation adds next-ranked blocks without re-sorting).
 *   "Sparse Attention for Video Generation Acceleration via Growing Sparsity
 *    and Reduced Search": S3.2 (block-sparse FlashAttention skips unselected
 *    key blocks), S5.3 (importance normalised per query block), A.1 (online
 *    softmax), A.4 (shortest descending prefix reaching p), A.6 (reordering).
 *
 * Conventions
 *   - Every buffer is allocated, owned and freed by the caller.  The library
 *     never allocates, frees or synchronises; all work is enqueued on
 *     `stream` (a hipStream_t, NULL = the default stream) and results are
 *     valid once the caller has synchronised that stream.
 *   - "device" pointers must point to memory of the current HIP device; the
 *     problem struct is read on the host during the call only.
 *   - Tensors q, k, v, o are bf16, element (h, n, c) at
 *     h*stride_head + n*stride_token + c, in natural token order
 *     n = t*grid_h*grid_w + y*grid_w + x.  They must be 16-byte aligned with
 *     stride_token and stride_head multiples of 8 elements.
 *   - Notation: H heads, N tokens, d head_dim, B block, nb = ceil(N/B) query
 *     blocks = key blocks, H*nb (head, query-block) rows = tiles.
 *   - Every entry point returns FVA_OK or an error code and never throws.
 *     Argument checks run on the host before anything is enqueued; on an
 *     error nothing is enqueued.  FVA_ERR_HIP means a launch failed; the
 *     text is available from fva_last_error().
 *   - The functions keep no state between calls and may be called from
 *     several host threads; calls that share output buffers or the tile
 *     counter must be ordered by the caller.
 */
#ifndef FVA_H_
#define FVA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fva_status {
  FVA_OK = 0,
  FVA_ERR_ARG = 1,          /* null pointer, inconsistent sizes, NaN p, ... */
  FVA_ERR_UNSUPPORTED = 2,  /* head_dim or block not in {64, 128}; size limits */
  FVA_ERR_HIP = 3,          /* a HIP launch or device query failed */
  FVA_ERR_WORKSPACE = 4     /* workspace smaller than fva_sizes() asks for */
};

/* Largest supported nb (key blocks per row) and H*nb (rows / tiles), and the
 * most tiles one call cuts into two work items. */
#define FVA_MAX_BLOCKS 2048
#define FVA_MAX_TILES 16384
#define FVA_MAX_SPLITS 1024
/* Largest per-head refill per mille (fills every row that keeps >= 1 block). */
#define FVA_MAX_HEAD_REFILL (1000 * (FVA_MAX_BLOCKS - 1))

/*
 * The problem statement (FVAttn S2.1: per head h, query block i, key block j;
 * Top-p threshold p and Top-k floor; S3.1: video-aware block organisation).
 */
typedef struct fva_problem {
  int32_t num_heads;         /* H >= 1 */
  int32_t seq_len;           /* N, must equal grid_t * grid_h * grid_w */
  int32_t head_dim;          /* d in {64, 128} */
  int32_t grid_t, grid_h, grid_w; /* latent video grid, each >= 1 */
  int32_t block;             /* B in {64, 128}; query and key blocks alike */
  int32_t tile_h, tile_w;    /* spatial tile of the order; both 0 = raster order */
  float top_p;               /* p; >= 1 keeps every block, <= 0 keeps only the floor */
  int32_t k_min;             /* Top-k floor >= 1 (clamped to nb) */
  int32_t refill_per_mille;  /* one-GPU slack refill, 0..1000 (0 = off) */
  float sm_scale;            /* softmax scale; 0 = 1/sqrt(d) */
  int64_t stride_head;       /* elements between heads in q, k, v, o */
  int64_t stride_token;      /* elements between tokens (>= d) */
  int32_t order_kind;        /* FVA_ORDER_TILES (default) or FVA_ORDER_HILBERT */
  int32_t reserved;          /* must be 0 */
} fva_problem;

/*
 * Token orders (FVAttn S3.1, GSRS A.6; both frame-major):
 *   FVA_ORDER_TILES    tile_h x tile_w spatial tiles in raster order, raster
 *                      inside a tile, edge tiles cut at the border
 *                      (tile_h = tile_w = 0: natural order);
 *   FVA_ORDER_HILBERT  each frame along a generalised Hilbert curve from
 *                      (x, y) = (0, 0), primary direction x (tile ignored):
 *                      for a w x h rectangle walked from its origin along
 *                      primary a, secondary b, a 1-high strip is walked along
 *                      a and a 1-wide one along b; if w > 2h the two halves
 *                      of a (first ceil(w/2)) are walked in turn; if h > 2w
 *                      the first ceil(w/2) columns are walked with a and b
 *                      swapped, then the rest from the far corner with both
 *                      reversed; otherwise the quadrants (first ceil(w/2)
 *                      columns, first ceil(h/2) rows) are walked in
 *                      Hilbert's U (first transposed, last transposed and
 *                      reversed).  For 2^k x 2^k frames: Hilbert's curve.
 */
#define FVA_ORDER_TILES 0
#define FVA_ORDER_HILBERT 1

/* Sizes derived from a problem (element counts unless named _bytes). */
typedef struct fva_sizes_t {
  int32_t num_blocks;        /* nb */
  int32_t num_rows;          /* H*nb: row_count, tile_order, row_ptr - 1 */
  int64_t order_elems;       /* nb*B int32 (order) */
  int64_t scores_elems;      /* H*nb*nb float (scores) */
  int64_t ranked_elems;      /* H*nb*nb int16 (ranked) */
  int64_t col_idx_capacity;  /* H*nb*nb int32 (col_idx, worst case) */
  int64_t workspace_bytes;   /* fva_route workspace (pooled means, and the
                                scores when the caller passes none) */
  int32_t tile_counter_elems;/* 2 uint32 */
  int64_t kv_elems;          /* 2*H*nb*B*d bf16 (kv) */
  int64_t work_order_elems;  /* H*nb + min(H*nb, FVA_MAX_SPLITS) int32 (work_order) */
  int64_t plan_meta_elems;   /* 2 + H*nb + FVA_MAX_SPLITS int32 (plan_meta) */
  int64_t attn_workspace_bytes; /* fva_sparse_attn_fwd workspace */
  int64_t block_lse_capacity;/* H*nb*nb*B float: block_lse for any mask
                                (row_ptr[H*nb] * B suffices for a given one) */
} fva_sizes_t;

/* Host only: validate a problem and report buffer sizes.  Makes no HIP call. */
int fva_sizes(const fva_problem* prob, fva_sizes_t* out);

/* Number of persistent workgroups fva_sparse_attn_fwd launches for this
 * problem on the current device (compute units x resident workgroups per
 * unit, at most H*nb).  Queries the device; FVA_ERR_HIP without one. */
int fva_attn_workgroups(const fva_problem* prob, int32_t* out);

/* Compute units of the current device: the count C that fva_plan's split
 * rule uses.  Queries the device; FVA_ERR_HIP without one, FVA_ERR_ARG for a
 * null out. */
int fva_compute_units(int32_t* out);

/*
 * Routing frontend (FVAttn S3.1; GSRS S5.3, A.4, A.6).
 *   q, k        device bf16 [H][N][d] (strided as above), read only.
 *   v           device bf16 [H][N][d] or NULL; given exactly when kv is.
 *   scores      device float [H][nb][nb] or NULL, written: s_{h,i,j} =
 *               sm_scale * <mean of Q_h over query block i, mean of K_h over
 *               key block j>, blocks taken in the video-aware order.  With
 *               NULL the scores live in the workspace and are not returned.
 *   ranked      device int16 [H][nb][nb], written: per row, key-block ids by
 *               float32 score descending, equal scores by lower id.
 *   row_count   device int32 [H*nb], written: k_i = max(k_p, min(k_min, nb))
 *               where k_p is the shortest ranked prefix whose importance
 *               (softmax of the row's scores, as exact 2^-40 fixed-point
 *               weights) reaches p.
 *   head_count  device int32 [H], written: sum of row_count over the head's
 *               rows (Eq 1: L_h = head_count[h] / nb).
 *   order       device int32 [nb*B], written: natural token index of every
 *               position of the video-aware order, -1 past N (frame-major,
 *               tile_h x tile_w tiles in raster order, raster inside a tile,
 *               edge tiles cut at the border).
 *   kv          device bf16 [2][H][nb*B][d] (fva_sizes().kv_elems), 16-byte
 *               aligned, or NULL: when given, the routing pass also writes
 *               exactly what fva_kv_layout(k, v) writes (K is read once for
 *               both the pooling and the re-layout).  NULL makes the call
 *               routing only: it reads Q and K and nothing else.
 *   workspace   device scratch of workspace_bytes >= fva_sizes().workspace_bytes
 *               (pooled block means, and the scores when scores is NULL);
 *               contents are not needed after the call.
 * FVA_ERR_ARG also when exactly one of v and kv is NULL.
 */
int fva_route(const fva_problem* prob, const void* q, const void* k,
              const void* v, float* scores, int16_t* ranked,
              int32_t* row_count, int32_t* head_count, int32_t* order,
              void* kv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fva_route for callers that cannot allocate device memory (code under HIP
 * stream capture, serving loops or harnesses that forbid allocation): the
 * same arguments without the workspace, which lives instead in a static
 * device array of FVA_NOALLOC_SCRATCH_BYTES that each GPU the library runs
 * on holds until the process ends.  The call allocates and frees nothing.
 * Problems whose fva_sizes().workspace_bytes exceed the array return
 * FVA_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU uses
 * that GPU's one array: calls that may overlap on one GPU (other streams,
 * other host threads) race on it and must be ordered by the caller.
 * Outputs exactly as fva_route's.
 */
#define FVA_NOALLOC_SCRATCH_BYTES (32 << 20)
int fva_route_noalloc(const fva_problem* prob, const void* q, const void* k,
                      const void* v, float* scores, int16_t* ranked,
                      int32_t* row_count, int32_t* head_count, int32_t* order,
                      void* kv, void* stream);

/*
 * K and V in the layout fva_sparse_attn_fwd reads (GSRS A.6: the token
 * permutation that makes every block a contiguous run of positions).
 *   k, v        device bf16 [H][N][d] (strided as above), read only.
 *   order       device int32 [nb*B], written: as fva_route's order.
 *   kv          device bf16 [2][H][nb*B][d] (fva_sizes().kv_elems), 16-byte
 *               aligned, written.  Part 0: row p of head h = K row of token
 *               order[p]; part 1: V transposed per 64-position sub-block s,
 *               [h][s][c][j] = V of token order[64 s + key(j)] at feature c,
 *               with key(j) = 16(j/16) + 8((j%8)/4) + 4((j/8)%2) + j%4 (the
 *               order in which the attention's score accumulators hold their
 *               keys, so that its V operand is one 16-byte load).  Rows of
 *               positions past N are zero.
 * Depends only on K, V and the problem's geometry: a caller that keeps a
 * mask across calls (GSRS S5.1 mask reuse) calls this instead of fva_route.
 */
int fva_kv_layout(const fva_problem* prob, const void* k, const void* v,
                  int32_t* order, void* kv, void* stream);

/*
 * Plan (FVAttn S3.2-S3.3 on one GPU: the placement step becomes a
 * heaviest-first work queue, slack augmentation a per-row refill).
 *   ranked, row_count   as written by fva_route, read only.
 *   head_refill  device int32 [H] or NULL: refill per mille of each head,
 *                replacing prob->refill_per_mille (for budgets from
 *                fva_sasa_refill); values are clamped to
 *                [0, FVA_MAX_HEAD_REFILL].
 *   row_ptr      device int32 [H*nb + 1], written: CSR row offsets of the
 *                final mask; row (h, i) keeps k'_i = k_i + e_i blocks with
 *                e_i = min(nb - k_i, floor(k_i * f_h / 1000)), f_h =
 *                head_refill[h], or refill_per_mille without head_refill.
 *   col_idx      device int32 [>= row_ptr[H*nb]] (capacity H*nb*nb always
 *                suffices), written: the first k'_i ranked key blocks of each
 *                row, ascending.
 *   head_count_final  device int32 [H], written: sum of k'_i per head.
 *   work_order   device int32 [work_order_elems], written: the work items,
 *                entries tile * 2 + part (tile id h*nb + i), longest first,
 *                then tile, then part.  With C = fva_compute_units(),
 *                S = min(max(C / 2, 1), FVA_MAX_SPLITS / 2) and
 *                a = ceil(sum k' / S) (so a / 2 is about the mean load of
 *                one compute unit), a
 *                tile with k' >= 2 and 2 k' > a is two items: part 0 = its
 *                first ceil(k'/2) kept blocks, part 1 = the rest; any other
 *                tile is one item (part 0, all its blocks).  Splitting only
 *                moves work between compute units; what is computed is the
 *                same.
 *   plan_meta    device int32 [plan_meta_elems], written: [0] number of work
 *                items, [1] number of split tiles ns, [2 + t] split slot of
 *                tile t (its rank among split tiles by tile id) or -1,
 *                [2 + H*nb + s] tile of split slot s (s < ns).
 *   tile_counter device uint32 [2], written: reset to {0, 0}.
 * Queries the device for C (FVA_ERR_HIP without one).
 */
int fva_plan(const fva_problem* prob, const int16_t* ranked,
             const int32_t* row_count, const int32_t* head_refill,
             int32_t* row_ptr, int32_t* col_idx,
             int32_t* head_count_final, int32_t* work_order,
             int32_t* plan_meta, uint32_t* tile_counter, void* stream);

/*
 * The placement step of fva_plan on its own, for a CSR mask the caller
 * already holds (FVAttn S3.2: placement changes where work runs, never which
 * blocks are computed).
 *   row_ptr      device int32 [H*nb + 1], read only: CSR row offsets, each
 *                row keeping between 1 and nb blocks.
 *   work_order, plan_meta, tile_counter   written exactly as fva_plan writes
 *                them for a mask with these row lengths (same split rule,
 *                same heaviest-first order).
 * Queries the device for C (FVA_ERR_HIP without one).
 */
int fva_schedule(const fva_problem* prob, const int32_t* row_ptr,
                 int32_t* work_order, int32_t* plan_meta,
                 uint32_t* tile_counter, void* stream);

/*
 * Block-sparse attention forward (GSRS S3.2, A.1): for every query token of
 * query block i of head h, softmax(sm_scale * q.k) over the tokens of the kept
 * key blocks col_idx[row_ptr[h*nb+i] .. row_ptr[h*nb+i+1]) only, times V.
 *   q            device bf16 [H][N][d] (strided as above), read only.
 *   kv           K and V as written by fva_kv_layout (or by fva_route
 *                with a kv buffer), read only.
 *   order        device int32 [nb*B] as written by fva_route or fva_kv_layout.
 *   row_ptr, col_idx   CSR mask: each row keeps between 1 and nb blocks,
 *                ids in [0, nb).  A mask outside this contract gives
 *                unspecified o and lse (the K/V loads stay inside the kv
 *                buffer whatever the ids).
 *   work_order, plan_meta   as written by fva_plan or fva_schedule (for
 *                this row_ptr); the queue hands the
 *                work items out in work_order's order.  Any permutation of
 *                the first plan_meta[0] entries gives bitwise the same o and
 *                lse.  The two parts of a split tile each leave their
 *                partial result (unnormalised output, running maximum and
 *                denominator) in the workspace, and a second kernel merges
 *                them and writes that tile's o and lse.
 *   tile_counter device uint32 [2], must be {0, 0} on entry (fva_plan leaves
 *                it so); the kernel leaves it {0, 0} again on exit.  Calls
 *                that may run at the same time (other streams) need their
 *                own tile_counter and workspace.
 *   o            device bf16 [H][N][d] (strided like q), written.
 *   lse          device float [H][N] or NULL, written: natural-log
 *                log-sum-exp of each query's kept logits.
 *   block_lse    device float [row_ptr[H*nb] * B] or NULL (requires lse),
 *                written: GSRS S5.3 phase 1, for kept pair c of the CSR mask
 *                (row t, key block col_idx[c]) and query slot r of the row's
 *                query block (position t%nb * B + r), the natural-log
 *                log-sum-exp of that query's logits over the block's keys, at
 *                [c * B + r].  Slots past N hold unspecified values.
 *   workspace    device scratch of workspace_bytes >=
 *                fva_sizes().attn_workspace_bytes, 16-byte aligned: the
 *                partial results of split tiles; contents are not needed
 *                after the call.
 */
int fva_sparse_attn_fwd(const fva_problem* prob, const void* q, const void* kv,
                        const int32_t* order, const int32_t* row_ptr,
                        const int32_t* col_idx, const int32_t* work_order,
                        const int32_t* plan_meta, uint32_t* tile_counter,
                        void* o, float* lse, float* block_lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * fva_sparse_attn_fwd with a per-work-item trace, for measuring how the
 * persistent queue spreads work over the compute units (the one-GPU form of
 * FVAttn S2.2 Eq 2's imbalance factor).  Same arguments and outputs, plus:
 *   item_trace   device int64 [plan_meta[0]][FVA_TRACE_FIELDS], written: for
 *                the work item at queue position x, [x][0] and [x][1] the
 *                constant-rate clock (100 MHz) when its workgroup started and
 *                finished it, [x][2] and [x][3] the compute unit's own cycle
 *                counter at the same two points, [x][4] the hardware placement
 *                of the workgroup (XCC id << 32 | hardware id register), and
 *                [x][5] the workgroup index.
 * The trace stores are the only difference from fva_sparse_attn_fwd: o, lse
 * and block_lse are bitwise the same.
 */
#define FVA_TRACE_FIELDS 6
int fva_sparse_attn_fwd_traced(const fva_problem* prob, const void* q, const void* kv,
                               const int32_t* order, const int32_t* row_ptr,
                               const int32_t* col_idx, const int32_t* work_order,
                               const int32_t* plan_meta, uint32_t* tile_counter,
                               void* o, float* lse, float* block_lse, void* workspace,
                               size_t workspace_bytes, int64_t* item_trace, void* stream);

/*
 * Precise block importance (GSRS S5.3 phase 2, A.2): after an attention call
 * that recorded block_lse and lse, the importance of kept key block j for
 * query block i of head h is the mean over the block's queries of
 * exp(block LSE - row LSE), i.e. the average share of a query's attention
 * weight (softmax over the row's kept keys) that falls on j; it sums to 1
 * over the row's kept blocks.
 *   order, row_ptr, col_idx, lse, block_lse   as used / written above.
 *   importance   device float [H][nb][nb], written (0 for blocks not kept).
 */
int fva_block_importance(const fva_problem* prob, const int32_t* order,
                         const int32_t* row_ptr, const int32_t* col_idx,
                         const float* lse, const float* block_lse,
                         float* importance, void* stream);

/*
 * Re-selection inside an evaluated set (GSRS S5.1 reduced search, S5.2 and
 * A.4 Top-p, A.2 importance over the evaluated blocks): after an attention
 * call over a mask with block_lse and fva_block_importance, choose each
 * row's new kept blocks from among that mask's blocks.
 *   row_ptr, col_idx  device, the evaluated mask (the one the importance was
 *                computed over), read only; each row non-empty, ids < nb,
 *                no repeats.
 *   importance   device float [H][nb][nb] as written by fva_block_importance
 *                for that mask, read only.
 *   prob->top_p, prob->k_min   the search's threshold and floor (the rest of
 *                prob as for the other calls).
 *   ranked       device int16 [H][nb][nb], written: per row the evaluated
 *                blocks by importance descending (equal values by lower id),
 *                then the remaining blocks by ascending id.
 *   row_count    device int32 [H*nb], written: k = max(k_p, min(k_min, c)),
 *                c = the row's evaluated count, k_p = the shortest ranked
 *                prefix whose weights rint(max(importance, 0) * 2^40) reach
 *                fl(p * their sum) (1 if p reaches it with one block; c for
 *                p >= 1; 0 for p <= 0).
 *   head_count   device int32 [H], written: sum of row_count per head.
 * fva_plan(ranked, row_count) then materialises the new mask, which is a
 * subset of the evaluated one whenever refill is off.
 */
int fva_reselect(const fva_problem* prob, const int32_t* row_ptr,
                 const int32_t* col_idx, const float* importance,
                 int16_t* ranked, int32_t* row_count, int32_t* head_count,
                 void* stream);

/*
 * Step schedule of growing sparsity with reduced search (GSRS S5.1, A.5;
 * S6.1's default: 50 steps, 10 warm-up steps, searches at 10, 20, 30, 40
 * with p = 0.95, 0.9, 0.85, 0.8).  Host only.
 *   FVA_GSRS_DENSE             full attention (warm-up, or before any search)
 *   FVA_GSRS_FULL_SEARCH       attention over every block with block LSEs,
 *                              importance, re-selection with *top_p; at the
 *                              first search past the warm-up (or every
 *                              search when reduced = 0); its mask is the
 *                              candidate set of the later searches
 *   FVA_GSRS_CANDIDATE_SEARCH  the same over the candidate set only
 *   FVA_GSRS_REUSE             attention over the latest selected mask
 * A search step's output is its attention over the evaluated blocks.
 * FVA_ERR_ARG for null pointers, step outside [0, num_steps), search steps
 * not strictly increasing inside [0, num_steps), a NaN p, more than
 * FVA_GSRS_MAX_SEARCHES searches or reduced not 0/1.
 */
#define FVA_GSRS_MAX_SEARCHES 16
#define FVA_GSRS_DENSE 0
#define FVA_GSRS_FULL_SEARCH 1
#define FVA_GSRS_CANDIDATE_SEARCH 2
#define FVA_GSRS_REUSE 3

typedef struct fva_gsrs_schedule {
  int32_t num_steps;      /* >= 1 */
  int32_t warmup_steps;   /* >= 0 */
  int32_t num_searches;   /* 0 .. FVA_GSRS_MAX_SEARCHES */
  int32_t reduced;        /* 1: later searches over the candidate set only */
  int32_t search_step[FVA_GSRS_MAX_SEARCHES];  /* strictly increasing */
  float top_p[FVA_GSRS_MAX_SEARCHES];          /* p of each search */
} fva_gsrs_schedule;

int fva_gsrs_action(const fva_gsrs_schedule* schedule, int32_t step,
                    int32_t* action, float* top_p);

/*
 * Measurement aid, outside the hot path: enqueue a kernel that runs only
 * bf16 MFMAs (v_mfma_f32_32x32x16_bf16, four independent chains per wave,
 * two 256-thread workgroups per compute unit) for `iters` rounds, with zero
 * operands (random_operands = 0) or N(0,1)-like ones (1).  The caller times
 * it on `stream`; *flops receives the FLOPs it performs.  The clock a device
 * sustains under MFMA load depends on the operand data, so this gives the
 * matrix-unit rate actually reachable with realistic data, next to the
 * nominal peak.
 *   sink         device float [sink_elems >= 512 * compute units], written.
 * Returns FVA_ERR_ARG for iters < 1 or null pointers, FVA_ERR_WORKSPACE for a
 * short sink.
 */
int fva_mfma_probe(int32_t iters, int32_t random_operands, float* sink,
                   int64_t sink_elems, double* flops, void* stream);

/*
 * Runtime load balancing and slack-aware augmentation across ranks
 * (FVAttn S3.2 Eq 5-6, S3.3 Eq 7-10 and the rho gating; S4.1 defaults).
 * Host only: these two calls make no HIP call and touch no device memory.
 *
 * R ranks each hold Hl heads, rank r the heads r*Hl .. r*Hl+Hl-1, with
 * integer workloads (kept query-block x key-block tiles, head_count from
 * fva_route).  Rank loads L_r are sums over the rank's heads and
 * rho = max L / mean L (Eq 2).
 *
 * Gating: rho < k1 -> FVA_BALANCE_NONE; k1 <= rho < k2 -> FVA_BALANCE_SASA;
 * rho >= k2 -> FVA_BALANCE_RLB_SASA, compared exactly as
 * 1000 * R * max L >= k * sum L.  All-zero loads gate to NONE.
 *
 * RLB (only under FVA_BALANCE_RLB_SASA): a plan is a permutation sigma of the
 * ranks; a rank with sigma(r) != r sends one of its heads, send_head[r], to
 * sigma(r) and receives one from sigma^-1(r), so every rank moves at most one
 * head out and one in (Eq 5: L_new_r = L_r - sent + received).  Candidates:
 *   FVA_RLB_PAIRS  every involution (disjoint pairs of ranks, each pair swaps
 *                  one head each way), R <= FVA_RLB_MAX_PAIR_RANKS;
 *   FVA_RLB_RING   the identity and the cycle r -> r+1 mod R in which every
 *                  rank sends one head, R <= FVA_RLB_MAX_RANKS.
 * The chosen plan minimises, in order: max_r L_new_r; sum_r L_new_r^2 (the
 * variance of Eq 6, since the total is fixed); the number of moved heads;
 * sigma as a vector; send_head as a vector (-1 for ranks that send none).
 * The result is a deterministic function of the inputs, so every rank can run
 * the search on the same all-gathered loads and read off its own partners.
 *
 * SASA (under SASA and RLB_SASA): slack[r] = max L_new - L_new_r (Eq 7),
 * budget[r] = floor(n1 * slack[r] / 1000) where 1000 * slack[r] >
 * n2 * max L_new, else 0 (Eq 8 and the trigger); budget is 0 under NONE.
 * With n1 <= 1000 no budget lifts a rank past max L_new (Eq 10's first term
 * is 0).
 */
#define FVA_RLB_PAIRS 0
#define FVA_RLB_RING 1
#define FVA_BALANCE_NONE 0
#define FVA_BALANCE_SASA 1
#define FVA_BALANCE_RLB_SASA 2
#define FVA_RLB_MAX_PAIR_RANKS 12
#define FVA_RLB_MAX_RANKS 64
#define FVA_RLB_MAX_HEADS 64
#define FVA_RLB_MAX_HEAD_LOAD (1 << 22)  /* nb^2 at nb = 2048 */
#define FVA_RLB_MAX_PER_MILLE 1000000

typedef struct fva_balance_params {
  int32_t num_ranks;       /* R >= 1 */
  int32_t heads_per_rank;  /* Hl, 1 .. FVA_RLB_MAX_HEADS */
  int32_t topology;        /* FVA_RLB_PAIRS or FVA_RLB_RING */
  int32_t k1_per_mille;    /* SASA threshold on rho (1050) */
  int32_t k2_per_mille;    /* RLB threshold on rho (1100), >= k1 */
  int32_t n1_per_mille;    /* budget coefficient (800), 0 .. 1000 */
  int32_t n2_per_mille;    /* trigger threshold on the slack (70) */
  int32_t reserved;        /* must be 0 */
} fva_balance_params;

typedef struct fva_balance_info {
  int32_t mode;              /* FVA_BALANCE_* chosen by the gating */
  int32_t moves;             /* heads migrated (ranks with sigma(r) != r) */
  int32_t rho_per_mille;     /* floor(1000 * rho) before, after RLB: */
  int32_t rho_new_per_mille;
  int64_t load_total;        /* sum L (unchanged by migration) */
  int64_t load_max;          /* max L */
  int64_t load_new_max;      /* max L_new: the critical path after RLB */
  int64_t load_aug_max;      /* max (L_new + budget) (Eq 9) */
} fva_balance_info;

/*
 *   prm          host, read during the call.
 *   head_load    host int32 [R][Hl], each 0 .. FVA_RLB_MAX_HEAD_LOAD.
 *   sigma, send_head   host int32 [R], written (send_head -1 = no move).
 *   load_new, slack, budget   host int64 [R], written.
 *   info         host, written.
 * FVA_ERR_ARG for null pointers, loads out of range, reserved != 0, k1 > k2,
 * n1 outside 0 .. 1000 or per-mille values outside 0 .. FVA_RLB_MAX_PER_MILLE;
 * FVA_ERR_UNSUPPORTED for R or Hl past the limits above.
 */
int fva_balance(const fva_balance_params* prm, const int32_t* head_load,
                int32_t* sigma, int32_t* send_head, int64_t* load_new,
                int64_t* slack, int64_t* budget, fva_balance_info* info);

/*
 * One-GPU form of the augmentation (FVAttn S3.3: extra blocks follow the
 * routing's ranking and skip the heads migrated out): turns each rank's block
 * budget into one refill per mille f_r for the rank's heads that did not move
 * (moved heads get 0).  With e_i = min(nb - k_i, floor(k_i f / 1000)) summed
 * over the eligible rows as A(f), A* is the most blocks any f in
 * [0, 1000 (nb - 1)] adds without exceeding budget[r], and f_r is the
 * smallest f with A(f) = A*.
 *   row_count    host int32 [R*Hl][nb] (fva_route's row_count per head),
 *                each 0 .. nb.
 *   send_head, budget   host, as written by fva_balance (budget >= 0).
 *   head_refill  host int32 [R*Hl], written: f_r per head (fva_plan's
 *                head_refill after a copy to the device).
 *   added        host int64 [R], written: A* per rank.
 * Errors as fva_balance, plus FVA_ERR_ARG for nb outside 1 .. FVA_MAX_BLOCKS.
 */
int fva_sasa_refill(const fva_balance_params* prm, int32_t nb,
                    const int32_t* row_count, const int32_t* send_head,
                    const int64_t* budget, int32_t* head_refill,
                    int64_t* added);

/* Static text for a status code. */
const char* fva_status_string(int status);

/* Text of the last FVA_ERR_HIP on the calling thread ("" if none). */
const char* fva_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fva_version(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* FVA_H_ */
