"""Oracle: runtime load balancing (RLB) and slack-aware sparse augmentation (SASA).

TEST INFRASTRUCTURE ONLY -- imported by tests/, the smoke check and the bench's
CPU-baseline leg, never by the product path.  Exhaustive enumeration written
from the definitions; it shares no code with the library's native search.

Source: "FVAttn: Adaptive Sparse Attention with Runtime Load Balancing for
Video Generation" (full paper text, translated):
  S2.2 Eq 2   rho = max_r L_r / mean_r L_r over the ranks' workloads.
  S3.2 Eq 5   a migration plan is a permutation sigma of the ranks; rank r
              sends one local head h_r to sigma(r) and receives one from
              sigma^-1(r); L_new_r = L_r - L_{h_r} + L_{h_{sigma^-1(r)}}.
  S3.2 Eq 6   sigma* minimises (max_r L_new_r, Var_r L_new_r) in
              lexicographic order over the one-send-one-receive plans that
              move at most about 20% of the local heads; the paper searches a
              pairing topology for 8 ranks and a one-way ring for other sizes,
              and every rank runs the same deterministic search.
  S3.3 Eq 7   slack dL_r = L_new_max - L_new_r.
  S3.3 Eq 8-9 budget B_r = n1 * dL_r, augmented load L_new_r + B_r, only
              where dL_r > n2 * L_new_max; extra blocks follow the routing's
              ranking on the heads that were not migrated out.
  S3.3 Eq 10  visible cost max(0, max_r L_aug_r - L_new_max) (+ fixed S).
  S3.3        gating: rho < k1 no mechanism, k1 <= rho < k2 SASA only,
              rho >= k2 RLB then SASA.
  S4.1        k1 = 1.05, k2 = 1.10, n1 = 0.8, n2 = 0.07, one head per rank.

Readings where the pages leave a step open:
  * workloads are integers: L_h = kept (query block, key block) tiles of head
    h, L_r = sum over the rank's heads; rank r holds heads r*Hl .. r*Hl+Hl-1;
  * "at most ~20% of the local heads" = at most one head sent and one head
    received per rank, so every rank keeps Hl heads;
  * topology "pairs": sigma is any involution (disjoint pairs of ranks, each
    pair swaps one head each way); topology "ring": sigma is the identity or
    the cycle r -> r+1 mod R with every rank sending one head;
  * Eq 6 is compared exactly: the total load is invariant under migration, so
    Var_r L_new_r orders like sum_r L_new_r^2; remaining ties go to fewer moved
    heads, then the lexicographically smallest sigma, then the smallest vector
    of sent heads (-1 for a rank that sends none);
  * rho thresholds and n1, n2 are per-mille integers (1050, 1100, 800, 70);
    rho >= k2 is R * max * 1000 >= k2 * sum; all-zero loads gate to "none";
    B_r = floor(n1 * dL_r / 1000), triggered when 1000 * dL_r > n2 * L_new_max;
  * on one GPU the budget becomes a refill per mille f_r shared by the heads
    of rank r that did not move (per-row refill e_i = min(nb - k_i,
    floor(k_i f / 1000)) in the routing's ranking): the smallest f that adds
    as many blocks over those heads as any f in [0, 1000 (nb - 1)] can without
    exceeding B_r; moved heads get f = 0.
"""

from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

MODE_NONE, MODE_SASA, MODE_RLB_SASA = 0, 1, 2
K1_PM, K2_PM, N1_PM, N2_PM = 1050, 1100, 800, 70


def rank_loads(head_load: np.ndarray) -> np.ndarray:
    """L_r = sum of the workloads of the heads rank r holds ([R][Hl] input)."""
    return np.asarray(head_load, dtype=np.int64).sum(axis=1)


def gate(loads: Sequence[int], k1_pm: int = K1_PM, k2_pm: int = K2_PM) -> int:
    """S3.3 gating on Eq 2's rho = max / mean, compared in integers."""
    L = [int(x) for x in loads]
    R, tot, mx = len(L), sum(L), max(L)
    if tot == 0:
        return MODE_NONE
    if 1000 * R * mx >= k2_pm * tot:
        return MODE_RLB_SASA
    if 1000 * R * mx >= k1_pm * tot:
        return MODE_SASA
    return MODE_NONE


def involutions(R: int) -> List[Tuple[int, ...]]:
    """Every permutation of range(R) that is its own inverse (pairings)."""
    out: List[Tuple[int, ...]] = []

    def rec(sig: List[int], free: List[int]):
        if not free:
            out.append(tuple(sig))
            return
        r, rest = free[0], free[1:]
        rec(sig, rest)
        for i, s in enumerate(rest):
            nxt = list(sig)
            nxt[r], nxt[s] = s, r
            rec(nxt, rest[:i] + rest[i + 1:])

    rec(list(range(R)), list(range(R)))
    return out


def candidate_sigmas(R: int, topology: str) -> List[Tuple[int, ...]]:
    if topology == "pairs":
        return involutions(R)
    if topology == "ring":
        ident = tuple(range(R))
        ring = tuple((r + 1) % R for r in range(R))
        return [ident] if ring == ident else [ident, ring]
    raise ValueError(topology)


def migrate(head_load: np.ndarray, sigma: Sequence[int], send: Sequence[int]) -> np.ndarray:
    """Eq 5 for one plan: rank r loses head send[r], sigma(r) gains it."""
    w = np.asarray(head_load, dtype=np.int64)
    L = w.sum(axis=1)
    out = L.copy()
    for r, s in enumerate(sigma):
        if s != r:
            out[r] -= w[r, send[r]]
            out[s] += w[r, send[r]]
    return out


def plan_key(loads_new: np.ndarray, sigma, send):
    L = [int(x) for x in loads_new]
    moves = sum(1 for r, s in enumerate(sigma) if s != r)
    return (max(L), sum(x * x for x in L), moves, tuple(sigma), tuple(send))


def rlb_search(head_load: np.ndarray, topology: str = "pairs") -> Dict[str, object]:
    """Eq 6 by exhaustive enumeration of every candidate sigma and every
    choice of sent heads (Eq 5 evaluated for each, vectorised over the head
    choices of one sigma)."""
    w = np.asarray(head_load, dtype=np.int64)
    R, Hl = w.shape
    L = w.sum(axis=1)
    best = None
    for sigma in candidate_sigmas(R, topology):
        movers = [r for r in range(R) if sigma[r] != r]
        # every choice of sent heads, in lexicographic order (mixed radix Hl)
        m = len(movers)
        code = np.arange(Hl ** m, dtype=np.int64)[:, None]
        combos = (code // (Hl ** np.arange(m - 1, -1, -1, dtype=np.int64))) % Hl
        new = np.broadcast_to(L, (len(combos), R)).copy()
        for j, r in enumerate(movers):
            moved = w[r, combos[:, j]]
            new[:, r] -= moved
            new[:, sigma[r]] += moved
        # lexicographic minimum over (max, sum of squares, sent heads in rank
        # order): keep the rows attaining the minimum of each key in turn
        keys = [new.max(axis=1), (new * new).sum(axis=1)] + [combos[:, j] for j in range(m)]
        idx = np.arange(len(combos))
        for key in keys:
            kk = key[idx]
            idx = idx[kk == kk.min()]
        i = int(idx[0])
        send = [-1] * R
        for j, r in enumerate(movers):
            send[r] = int(combos[i, j])
        key = plan_key(new[i], sigma, send)
        if best is None or key < best[0]:
            best = (key, list(sigma), send, new[i].copy())
    key, sigma, send, new = best
    return {"sigma": np.array(sigma, dtype=np.int64), "send": np.array(send, dtype=np.int64),
            "loads_new": new, "moves": key[2]}


def sasa_budgets(loads_new: Sequence[int], n1_pm: int = N1_PM, n2_pm: int = N2_PM):
    """Eq 7-9: slack to the critical rank, trigger, discounted budget."""
    L = np.asarray(loads_new, dtype=np.int64)
    lmax = int(L.max())
    slack = lmax - L
    trig = 1000 * slack > n2_pm * lmax
    budget = np.where(trig, (n1_pm * slack) // 1000, 0).astype(np.int64)
    return slack, budget


def balance(head_load: np.ndarray, topology: str = "pairs", k1_pm: int = K1_PM, k2_pm: int = K2_PM,
            n1_pm: int = N1_PM, n2_pm: int = N2_PM) -> Dict[str, object]:
    """Gating, then RLB (Eq 5-6) when rho >= k2, then SASA (Eq 7-9) when rho >= k1."""
    w = np.asarray(head_load, dtype=np.int64)
    R = w.shape[0]
    L = w.sum(axis=1)
    mode = gate(L, k1_pm, k2_pm)
    if mode == MODE_RLB_SASA:
        rlb = rlb_search(w, topology)
        sigma, send, new = rlb["sigma"], rlb["send"], rlb["loads_new"]
    else:
        sigma, send, new = np.arange(R), np.full(R, -1), L.copy()
    slack, budget = sasa_budgets(new, n1_pm, n2_pm)
    if mode == MODE_NONE:
        budget = np.zeros(R, np.int64)
    return {"mode": mode, "sigma": np.asarray(sigma, np.int64), "send": np.asarray(send, np.int64),
            "loads": L, "loads_new": np.asarray(new, np.int64), "slack": slack, "budget": budget,
            "moves": int(np.sum(np.asarray(sigma) != np.arange(R)))}


def refill_added(row_count: np.ndarray, nb: int, f: int) -> int:
    """Blocks one refill per mille f adds over the given rows."""
    k = np.asarray(row_count, dtype=np.int64)
    return int(np.minimum(nb - k, (k * int(f)) // 1000).sum())


def refill_from_budget(row_count: np.ndarray, nb: int, R: int, Hl: int, send: Sequence[int],
                       budget: Sequence[int]):
    """Per-head refill per mille from the rank budgets (one-GPU SASA).

    row_count is [R*Hl][nb].  For rank r the eligible heads are its own heads
    except the one it sent.  The refill added over them, A(f), never falls as
    f grows, so bisection finds the most blocks A* = A(f) reachable within
    budget[r] for f in [0, 1000 (nb - 1)] (the top of that range fills every
    row with k_i >= 1), then the smallest f with A(f) = A*; that f is the
    refill of every eligible head of r, and moved heads get 0.  Returns the
    per-head refill [R*Hl] and the blocks added per rank.
    """
    rc = np.asarray(row_count, dtype=np.int64).reshape(R * Hl, nb)
    refill = np.zeros(R * Hl, dtype=np.int64)
    added = np.zeros(R, dtype=np.int64)
    fmax = 1000 * (nb - 1)
    for r in range(R):
        heads = [r * Hl + j for j in range(Hl) if j != send[r]]
        rows = rc[heads].reshape(-1)
        B = int(budget[r])
        # largest f with A(f) <= B  (A(0) = 0 <= B)
        lo, hi = 0, fmax
        while lo < hi:
            mid = (lo + hi + 1) // 2
            if refill_added(rows, nb, mid) <= B:
                lo = mid
            else:
                hi = mid - 1
        best = refill_added(rows, nb, lo)
        # smallest f with A(f) >= best
        a, b = 0, lo
        while a < b:
            mid = (a + b) // 2
            if refill_added(rows, nb, mid) >= best:
                b = mid
            else:
                a = mid + 1
        for h in heads:
            refill[h] = a
        added[r] = best
    return refill, added
