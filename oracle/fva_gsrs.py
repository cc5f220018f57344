"""Oracle: growing sparsity and reduced search across denoising steps.

TEST INFRASTRUCTURE ONLY -- imported by tests/, the smoke check and the bench's
CPU-baseline leg, never by the product path.  Plain NumPy written from the
definitions; it shares no code with the HIP library.

Source: "Sparse Attention for Video Generation Acceleration via Growing
Sparsity and Reduced Search" (GSRS):
  S5.1, A.5  pipeline: full attention for the warm-up steps, a first search
             over the full key space, later searches only over the early
             candidate set (the first search's mask), the latest mask reused
             between searches; the Top-p threshold decreases from search to
             search (growing sparsity).
  S5.2, A.4  Top-p keeps the shortest prefix of the blocks ranked by
             importance whose cumulative importance reaches p.
  A.2        the importance recovered at a search is normalised over the
             evaluated key blocks (all blocks at the first search, the
             candidate set later), so it sums to one over them.
  S6.1       default schedule: 50 steps, warm-up 20% (10 steps), searches at
             steps 10, 20, 30, 40 with p = 0.95, 0.9, 0.85, 0.8.

Readings where the pages leave a step open:
  * a search step's attention output is the attention over the evaluated set
    (its block LSEs give the importance); the new mask serves the steps after;
  * re-selection ranks only the evaluated blocks (importance descending,
    equal importance by lower id) and the other blocks follow by ascending id;
    the cutoff uses the weights w = rint(max(importance, 0) * 2^40) of the evaluated
    blocks, W their sum, k_p = min{k : sum_{r<k} w_(r) >= fl(p * W)}; p >= 1
    keeps every evaluated block, p <= 0 none before the floor; the Top-k
    floor is min(k_min, number of evaluated blocks);
  * "without reduced search" every search is a full-space search.
"""

from __future__ import annotations

from typing import Dict, Sequence, Tuple

import numpy as np

ACT_DENSE, ACT_FULL_SEARCH, ACT_CANDIDATE_SEARCH, ACT_REUSE = 0, 1, 2, 3
FIXED_POINT_BITS = 40


def select_from_importance(imp32: np.ndarray, row_ptr: np.ndarray, col_idx: np.ndarray,
                           top_p: float, k_min: int):
    """Re-selection inside the evaluated set of every row ([H][nb][nb] float32
    importance, CSR of the evaluated mask).  Returns (ranked [H*nb][nb],
    row_count [H*nb], head_count [H])."""
    H, nb, _ = imp32.shape
    rows = H * nb
    ranked = np.zeros((rows, nb), dtype=np.int64)
    count = np.zeros(rows, dtype=np.int64)
    p = float(np.float32(top_p))
    for r in range(rows):
        h, i = divmod(r, nb)
        cand = np.asarray(col_idx[row_ptr[r]: row_ptr[r + 1]], dtype=np.int64)
        vals = imp32[h, i, cand].astype(np.float32)
        # importance descending, equal values by lower block id (-0.0 == +0.0)
        order = sorted(range(len(cand)), key=lambda t: (-float(vals[t]) + 0.0, int(cand[t])))
        ranked_c = cand[order]
        others = np.setdiff1d(np.arange(nb), cand)
        ranked[r] = np.concatenate([ranked_c, others])
        c = len(cand)
        if p >= 1.0:
            kp = c
        elif not p > 0.0:
            kp = 0
        else:
            w = [max(0, int(np.rint(float(vals[t]) * 2.0 ** FIXED_POINT_BITS))) for t in order]
            W = sum(w)
            target = p * float(W)          # one fp64 product, as fl(p * W)
            run, kp = 0, 0
            while kp < c and run < target:
                run += w[kp]
                kp += 1
            kp = max(kp, 1) if c else 0
        count[r] = max(kp, min(int(k_min), c))
    head = count.reshape(H, nb).sum(axis=1)
    return ranked, count, head


def gsrs_action(step: int, num_steps: int, warmup: int, search_steps: Sequence[int],
                top_ps: Sequence[float], reduced: bool = True) -> Tuple[int, float]:
    """What step `step` does under the schedule (S5.1, A.5, S6.1): dense during
    the warm-up, a full-space search at the first search step, candidate-set
    searches at later ones (full-space ones without reduced search), reuse of
    the latest mask otherwise.  Returns (action, p of that search or 1.0)."""
    if step < 0 or step >= num_steps:
        raise ValueError("step out of range")
    if step < warmup:
        return ACT_DENSE, 1.0
    searches = [s for s in search_steps if s >= warmup]
    if step in searches:
        j = list(search_steps).index(step)
        first = step == min(searches)
        if first or not reduced:
            return ACT_FULL_SEARCH, float(top_ps[j])
        return ACT_CANDIDATE_SEARCH, float(top_ps[j])
    if not searches or step < min(searches):
        return ACT_DENSE, 1.0
    return ACT_REUSE, 1.0
