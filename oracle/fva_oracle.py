"""Oracle: adaptive block-sparse self-attention for video DiTs, step by step.

TEST INFRASTRUCTURE ONLY -- imported by tests/, the smoke check and the bench's
CPU-baseline leg, never by the product path.  Everything is NumPy float64
unless a step is defined on float32 scores; it shares no code with the HIP
library.

Sources (page title, section):
  [FVA]  "FVAttn: Adaptive Sparse Attention with Runtime Load Balancing for
         Video Generation" (full paper text, translated):
         S2.1 block mask M_{h,i,j} from scores s_{h,i,j}; Top-p keeps the
              smallest set of key blocks whose cumulative normalised importance
              reaches p; a Top-k floor keeps a minimum budget per query block.
         S2.2 Eq 1 per-head workload L_h = mean_i sum_j M_{h,i,j}; Eq 2 load
              imbalance rho = max_r L_r / mean_r L_r.
         S3.1 video-aware block reordering, block similarity from pooled Q/K,
              the same routing pass yields per-head density and the
              block-importance ordering.
         S3.2 load balancing moves work, never changes the selected blocks.
         S3.3 SASA adds not-yet-selected blocks in the routing's priority order
              (no re-sort, no re-scoring).
  [GSRS] "Sparse Attention for Video Generation Acceleration via Growing
         Sparsity and Reduced Search":
         S3.1/A.1 online softmax; S3.2 block-sparse FlashAttention skips
         unselected key blocks; S5.3 block importance is normalised over the
         key blocks of a query block (sums to 1); A.4 Top-p takes the shortest
         descending prefix whose cumulative sum reaches p; A.6 token reordering
         so that nearby space-time tokens share blocks; S5.3/A.2 precise block
         importance: the mean over a query block's queries of the attention
         weight on each key block, normalised over the evaluated keys.

Readings where the pages are silent (each also listed in the design notes):
  * ordering: frame-major, spatial tiles tile_h x tile_w in raster order,
    raster inside a tile, ragged edge tiles truncated; blocks are runs of B
    consecutive positions (they may straddle tiles or frames);
  * pooling: mean over the real tokens of a block (a short last block divides
    by its own size);
  * score: s_{h,i,j} = sm_scale * <qbar_{h,i}, kbar_{h,j}>, sm_scale = 1/sqrt(d);
    importance = row softmax over j;
  * ranking: scores compared as float32, descending, ties -> lower j first,
    -0.0 == +0.0;
  * cutoff arithmetic: importance weights are exp(s - s_max) in float64,
    quantised to integers w = rint(e * 2^40) so that every cumulative sum is
    exact; k_p = min{k : sum_{r<k} w_(r) >= fl(p * W)} with p taken as the
    float32 value; p >= 1 keeps every block, p <= 0 keeps none before the floor;
  * floor: k_i = max(k_p, min(k_min, nb)), per (head, query block) row;
  * one-GPU SASA: every row gets e_i = min(nb - k_i, floor(k_i * refill / 1000))
    more blocks, the next ones in the ranking;
  * tile order: tiles sorted by kept count descending, then head, then query
    block (longest-processing-time first);
  * one-GPU placement with split tiles (our adaptation of S3.2's "move work,
    never change it" to the compute units of one GPU; no page defines it):
    with S = min(workgroups, MAX_SPLITS / 2) and a = ceil(sum_t k'_t / S), a
    tile with k'_t >= 2 and 2 k'_t > a is cut into two work items, its first
    ceil(k'/2) kept blocks and the rest; the work list is every item sorted by
    item length descending, then tile, then part.
"""

from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

FIXED_POINT_BITS = 40
MAX_SPLITS = 1024  # split tiles one call can hold partial results for


# --------------------------------------------------------------------------
# Geometry and the video-aware order  ([FVA] S3.1, [GSRS] A.6)
# --------------------------------------------------------------------------

def num_blocks(n_tokens: int, block: int) -> int:
    return -(-n_tokens // block)


def block_sizes(n_tokens: int, block: int) -> np.ndarray:
    """r_b: number of real positions in block b (only the last may be short)."""
    nb = num_blocks(n_tokens, block)
    starts = np.arange(nb) * block
    return np.minimum(block, n_tokens - starts).astype(np.int64)


def token_order(grid: Tuple[int, int, int], tile: Tuple[int, int]) -> np.ndarray:
    """pi: position -> natural token index, by explicit enumeration.

    Frames in time order; inside a frame the spatial tiles in raster order
    (tile rows top to bottom, tile columns left to right), edge tiles cut at the
    frame border; inside a tile its tokens in raster order.  tile == (0, 0)
    means no reordering.
    """
    T, H, W = grid
    th, tw = tile
    if th == 0 and tw == 0:
        return np.arange(T * H * W, dtype=np.int64)
    out = []
    for t in range(T):
        for a in range(-(-H // th)):
            for c in range(-(-W // tw)):
                for y in range(a * th, min(H, (a + 1) * th)):
                    for x in range(c * tw, min(W, (c + 1) * tw)):
                        out.append(t * H * W + y * W + x)
    return np.asarray(out, dtype=np.int64)


def _hilbert_walk(o, da, db, w, h, out):
    """Append the cells o + i*da + j*db (0 <= i < w along the primary vector da,
    0 <= j < h along the secondary db) in generalised Hilbert order, starting
    at o and, except in the single-column case, ending at o + (w-1)*da."""
    if h == 1:
        for i in range(w):
            out.append((o[0] + i * da[0], o[1] + i * da[1]))
        return
    if w == 1:
        for j in range(h):
            out.append((o[0] + j * db[0], o[1] + j * db[1]))
        return
    if w > 2 * h:
        # long along the primary: two halves walked one after the other
        w0 = (w + 1) // 2
        _hilbert_walk(o, da, db, w0, h, out)
        _hilbert_walk((o[0] + w0 * da[0], o[1] + w0 * da[1]), da, db, w - w0, h, out)
        return
    if h > 2 * w:
        # long along the secondary: up over the first ceil(w/2) columns, then
        # down over the rest from the far corner, ending at o + (w-1)*da
        w0 = (w + 1) // 2
        _hilbert_walk(o, db, da, h, w0, out)
        o1 = (o[0] + (w - 1) * da[0] + (h - 1) * db[0], o[1] + (w - 1) * da[1] + (h - 1) * db[1])
        _hilbert_walk(o1, (-db[0], -db[1]), (-da[0], -da[1]), h, w - w0, out)
        return
    # the four quadrants in Hilbert's U: first one transposed, last one
    # transposed and reversed, so every quadrant starts next to the previous end
    w0, h0 = (w + 1) // 2, (h + 1) // 2
    w1, h1 = w - w0, h - h0
    _hilbert_walk(o, db, da, h0, w0, out)
    o1 = (o[0] + h0 * db[0], o[1] + h0 * db[1])
    _hilbert_walk(o1, da, db, w0, h1, out)
    _hilbert_walk((o1[0] + w0 * da[0], o1[1] + w0 * da[1]), da, db, w1, h1, out)
    o3 = (o[0] + (w - 1) * da[0] + (h0 - 1) * db[0], o[1] + (w - 1) * da[1] + (h0 - 1) * db[1])
    _hilbert_walk(o3, (-db[0], -db[1]), (-da[0], -da[1]), h0, w1, out)


def hilbert_order(grid: Tuple[int, int, int]) -> np.ndarray:
    """pi for the Hilbert-curve reordering ([FVA] S3.1, [GSRS] A.6), by explicit
    enumeration: frames in time order; inside a frame the grid_h x grid_w
    cells along a generalised Hilbert curve that starts at (x, y) = (0, 0)
    with its primary direction along x.  The generalisation to any width w
    (along the primary) and height h: a strip of height 1 (or width 1) is
    walked straight; if w > 2h the two halves of the primary are walked one
    after the other; if h > 2w the first ceil(w/2) columns are walked up and
    the others down from the far corner; otherwise the four quadrants (first
    ceil(w/2) columns, first ceil(h/2) rows) are visited as in Hilbert's
    curve.  For 2^k x 2^k frames this is Hilbert's curve itself."""
    T, H, W = grid
    cells = []
    _hilbert_walk((0, 0), (1, 0), (0, 1), W, H, cells)
    frame = np.array([y * W + x for x, y in cells], dtype=np.int64)
    return np.concatenate([t * H * W + frame for t in range(T)])


def padded_order(order: np.ndarray, block: int) -> np.ndarray:
    """The order as nb*B slots, -1 in the slots past the end of the sequence."""
    nb = num_blocks(len(order), block)
    out = np.full(nb * block, -1, dtype=np.int64)
    out[: len(order)] = order
    return out


# --------------------------------------------------------------------------
# Pooled block representatives and block scores  ([FVA] S2.1, S3.1)
# --------------------------------------------------------------------------

def pool(x: np.ndarray, order: np.ndarray, block: int) -> np.ndarray:
    """Mean of the rows of each block, in float64.  x: [H][N][d] -> [H][nb][d]."""
    H, N, d = x.shape
    nb = num_blocks(N, block)
    out = np.zeros((H, nb, d))
    for b in range(nb):
        toks = order[b * block: min(N, (b + 1) * block)]
        out[:, b, :] = x[:, toks, :].mean(axis=1)
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray, sm_scale: float) -> np.ndarray:
    """s_{h,i,j} = sm_scale * <qbar_{h,i}, kbar_{h,j}>, float64 [H][nb][nb]."""
    return sm_scale * np.einsum("hid,hjd->hij", qbar, kbar)


def block_importance(scores: np.ndarray) -> np.ndarray:
    """Normalised importance: softmax over key blocks j (each row sums to 1)."""
    s = np.asarray(scores, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# Ranking, Top-p with a Top-k floor  ([FVA] S2.1, S3.1; [GSRS] S5.2, A.4)
# --------------------------------------------------------------------------

def ranking(s_row: np.ndarray) -> np.ndarray:
    """Key-block ids by float32 score descending, ties to the lower id."""
    s = np.asarray(s_row, dtype=np.float32)
    idx = np.arange(len(s))
    return np.lexsort((idx, -s.astype(np.float64)))


def fixed_point_weights(s_sorted: np.ndarray) -> np.ndarray:
    """w_r = rint(exp(s_(r) - s_(0)) * 2^40) as exact integers (uint64)."""
    s = np.asarray(s_sorted, dtype=np.float32).astype(np.float64)
    e = np.exp(s - s[0])
    return np.rint(e * float(2 ** FIXED_POINT_BITS)).astype(np.uint64)


def topp_count(s_row: np.ndarray, top_p: float) -> int:
    """k_p: length of the shortest ranked prefix whose cumulative weight reaches p."""
    nb = len(s_row)
    p = np.float32(top_p)
    if p >= 1.0:
        return nb
    if p <= 0.0:
        return 0
    s_sorted = np.asarray(s_row, dtype=np.float32)[ranking(s_row)]
    w = fixed_point_weights(s_sorted)
    prefix = np.cumsum(w, dtype=np.uint64)  # exact: total < 2^51
    target = float(p) * float(prefix[-1])
    reached = np.flatnonzero(prefix.astype(np.float64) >= target)
    return int(reached[0]) + 1 if len(reached) else nb


def select_counts(scores32: np.ndarray, top_p: float, k_min: int):
    """Per (head, query block) kept counts k_i and per-head totals.

    scores32: float32 [H][nb][nb].  Returns (row_count int64 [H*nb],
    head_count int64 [H]).
    """
    H, nqb, nkb = scores32.shape
    floor = min(k_min, nkb)
    rc = np.zeros(H * nqb, dtype=np.int64)
    for h in range(H):
        for i in range(nqb):
            rc[h * nqb + i] = max(topp_count(scores32[h, i], top_p), floor)
    return rc, rc.reshape(H, nqb).sum(axis=1)


def kept_blocks(s_row: np.ndarray, count: int) -> np.ndarray:
    """The first `count` ranked key blocks, as ascending ids."""
    return np.sort(ranking(s_row)[:count])


# --------------------------------------------------------------------------
# Plan: one-GPU SASA refill, CSR mask, LPT tile order  ([FVA] S2.2, S3.2, S3.3)
# --------------------------------------------------------------------------

def refill_counts(row_count: np.ndarray, nb: int, refill_per_mille) -> np.ndarray:
    """k'_i = k_i + min(nb - k_i, floor(k_i * f / 1000)); f is one value, or
    one per row (a per-head refill repeated over the head's rows)."""
    rc = np.asarray(row_count, dtype=np.int64)
    f = np.asarray(refill_per_mille, dtype=np.int64)
    extra = np.minimum(nb - rc, (rc * f) // 1000)
    return rc + extra


def plan(scores32: np.ndarray, row_count: np.ndarray, refill_per_mille: int,
         head_refill: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """head_refill: optional refill per mille per head, replacing the single
    value (the slack-driven budget of one-GPU SASA)."""
    H, nqb, nkb = scores32.shape
    if head_refill is not None:
        refill_per_mille = np.repeat(np.asarray(head_refill, dtype=np.int64), nqb)
    kept = refill_counts(row_count, nkb, refill_per_mille)
    row_ptr = np.zeros(H * nqb + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(kept)
    col_idx = np.zeros(int(row_ptr[-1]), dtype=np.int64)
    for h in range(H):
        for i in range(nqb):
            r = h * nqb + i
            col_idx[row_ptr[r]: row_ptr[r + 1]] = kept_blocks(scores32[h, i], int(kept[r]))
    tiles = np.arange(H * nqb)
    tile_order = np.array(sorted(tiles, key=lambda t: (-int(kept[t]), t // nqb, t % nqb)), dtype=np.int64)
    return {
        "kept": kept,
        "row_ptr": row_ptr,
        "col_idx": col_idx,
        "head_count": kept.reshape(H, nqb).sum(axis=1),
        "tile_order": tile_order,
    }


def work_items(kept: np.ndarray, compute_units: int, max_splits: int = MAX_SPLITS):
    """One-GPU placement of the tiles ([FVA] S3.2 adapted to one GPU).

    A tile heavier than the mean load of one compute unit cannot be balanced
    by ordering alone, so each tile with k' >= 2 and 2 k' > ceil(total / S) is
    cut into two work items (the first ceil(k'/2) of its kept blocks, then the
    rest), S = min(max(compute_units // 2, 1), max_splits // 2): ceil(total / S)
    / 2 is about total / compute_units.  Returns the work list (entries
    tile * 2 + part, longest item first, then tile, then part), the split slot
    of every tile (its rank among the split tiles by tile id, -1 if whole) and
    the number of split tiles.
    """
    kept = np.asarray(kept, dtype=np.int64)
    S = min(max(int(compute_units) // 2, 1), max_splits // 2)
    avg = -(-int(kept.sum()) // S)
    split = (kept >= 2) & (2 * kept > avg)
    slot = np.full(len(kept), -1, dtype=np.int64)
    slot[split] = np.arange(int(split.sum()))
    items = []
    for t, k in enumerate(kept.tolist()):
        if split[t]:
            items.append(((k + 1) // 2, t, 0))
            items.append((k // 2, t, 1))
        else:
            items.append((k, t, 0))
    items.sort(key=lambda x: (-x[0], x[1], x[2]))
    order = np.array([2 * t + part for _, t, part in items], dtype=np.int64)
    return order, slot, int(split.sum())


def head_workload(head_count: np.ndarray, nb: int) -> np.ndarray:
    """Eq 1: L_h = mean over query blocks of the kept key-block count."""
    return np.asarray(head_count, dtype=np.float64) / nb


def imbalance(loads: Sequence[float]) -> float:
    """Eq 2: rho = max load / mean load."""
    x = np.asarray(loads, dtype=np.float64)
    return float(x.max() / x.mean())


# --------------------------------------------------------------------------
# Attention  ([GSRS] S3.1, S3.2, A.1): exact softmax over the kept keys
# --------------------------------------------------------------------------

def _tile_tokens(order: np.ndarray, block: int, b: int) -> np.ndarray:
    return order[b * block: min(len(order), (b + 1) * block)]


def masked_attention(q, k, v, order, block, row_ptr, col_idx, sm_scale,
                     tiles: Optional[Sequence[int]] = None):
    """Softmax attention of every query over the keys of its row's kept blocks.

    q, k, v: float64 [H][N][d] in natural token order.  Returns O [H][N][d] and
    LSE [H][N] (natural log), NaN outside the requested tiles.
    """
    H, N, d = q.shape
    nb = num_blocks(N, block)
    o = np.full((H, N, d), np.nan)
    lse = np.full((H, N), np.nan)
    todo = range(H * nb) if tiles is None else tiles
    for t in todo:
        h, i = divmod(int(t), nb)
        qt = _tile_tokens(order, block, i)
        cols = col_idx[row_ptr[t]: row_ptr[t + 1]]
        kt = np.concatenate([_tile_tokens(order, block, int(j)) for j in cols])
        logits = sm_scale * (q[h, qt] @ k[h, kt].T)
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        l = p.sum(axis=1, keepdims=True)
        o[h, qt] = (p @ v[h, kt]) / l
        lse[h, qt] = (m + np.log(l))[:, 0]
    return o, lse


def precise_block_importance(q, k, order, block, row_ptr, col_idx, sm_scale,
                             tiles: Optional[Sequence[int]] = None):
    """[GSRS] S5.3, A.2: the importance of key block j for query block i is the
    attention weight the block's queries give to j's keys, averaged over those
    queries, with the softmax taken over the keys actually evaluated (the row's
    kept blocks); it sums to 1 over the kept blocks of each row.

    Written out from that definition: per tile the full probability matrix of
    its queries over its kept keys, summed over each kept block's keys,
    averaged over the queries.  Returns fp64 [H][nb][nb] (0 for blocks not
    kept; NaN rows outside the requested tiles).
    """
    H, N, d = q.shape
    nb = num_blocks(N, block)
    out = np.zeros((H, nb, nb))
    todo = range(H * nb) if tiles is None else tiles
    if tiles is not None:
        out[:] = np.nan
    for t in todo:
        h, i = divmod(int(t), nb)
        qt = _tile_tokens(order, block, i)
        cols = [int(j) for j in col_idx[row_ptr[t]: row_ptr[t + 1]]]
        toks = [_tile_tokens(order, block, j) for j in cols]
        kt = np.concatenate(toks)
        logits = sm_scale * (q[h, qt] @ k[h, kt].T)
        prob = np.exp(logits - logits.max(axis=1, keepdims=True))
        prob /= prob.sum(axis=1, keepdims=True)
        out[h, i] = 0.0
        start = 0
        for j, tk in zip(cols, toks):
            out[h, i, j] = prob[:, start: start + len(tk)].sum(axis=1).mean()
            start += len(tk)
    return out


def dense_attention(q, k, v, sm_scale, rows: Optional[np.ndarray] = None, chunk: int = 2048):
    """Plain softmax attention over all N keys, float64; optionally a row subset."""
    H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    o = np.zeros((H, len(rows), d))
    lse = np.zeros((H, len(rows)))
    for h in range(H):
        for s in range(0, len(rows), chunk):
            r = rows[s: s + chunk]
            logits = sm_scale * (q[h, r] @ k[h].T)
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            l = p.sum(axis=1, keepdims=True)
            o[h, s: s + len(r)] = (p @ v[h]) / l
            lse[h, s: s + len(r)] = (m + np.log(l))[:, 0]
    return o, lse


def attention_recall(lse_kept: np.ndarray, lse_dense: np.ndarray) -> np.ndarray:
    """Fraction of each query's full attention weight that falls on kept keys."""
    return np.exp(lse_kept - lse_dense)


def kept_flops(row_ptr, col_idx, n_tokens: int, block: int, head_dim: int) -> int:
    """4 * d * sum over kept (i, j) of r_i * c_j (QK^T and PV multiply-adds)."""
    r = block_sizes(n_tokens, block)
    nb = len(r)
    total = 0
    for t in range(len(row_ptr) - 1):
        i = t % nb
        total += int(r[i]) * int(r[col_idx[row_ptr[t]: row_ptr[t + 1]]].sum())
    return 4 * head_dim * total


# --------------------------------------------------------------------------
# The whole routing frontend on one GPU's heads
# --------------------------------------------------------------------------

def route(q, k, grid, tile, block, top_p, k_min, sm_scale=None):
    """Order -> pool -> scores -> Top-p + floor.  q, k float64 [H][N][d]."""
    H, N, d = q.shape
    if sm_scale is None or sm_scale == 0:
        sm_scale = 1.0 / math.sqrt(d)
    order = token_order(grid, tile)
    qbar = pool(q, order, block)
    kbar = pool(k, order, block)
    s64 = block_scores(qbar, kbar, sm_scale)
    s32 = s64.astype(np.float32)
    rc, hc = select_counts(s32, top_p, k_min)
    return {"order": order, "qbar": qbar, "kbar": kbar, "scores64": s64, "scores32": s32,
            "row_count": rc, "head_count": hc, "sm_scale": sm_scale}
