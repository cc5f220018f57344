"""GPU test: non-finite values in one head's Q and K.

The mask of a head whose inputs hold NaN or infinity is unspecified, but the
call must still complete with a structurally valid plan: every row count in
[min(k_min, nb), nb], every ranking row a permutation of the block ids, every
CSR row ascending and in range, a work list that is a permutation of the
items.  Heads are independent through routing and attention (FVAttn S2.1
states the problem per head), so the other heads' outputs equal those of the
same call on clean inputs: bit for bit where their tiles are processed the
same way, and within one bf16 unit in the last place where a different split
decision (the split rule reads the total over all heads) changes the order in
which a tile's partial sums are combined.
"""

import numpy as np
import pytest
import torch

import adaptive_block_sparse_fva_amd as F
from gpu_helpers import device_inputs, host, problem_for, run_chain, say
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,bad_head", [("two_head", 1), ("rank480p", 2)])
def test_nonfinite_head_leaves_the_others_and_the_plan_valid(name, bad_head):
    wl = WORKLOADS[name]
    say(f"[gpu] non-finite inputs in head {bad_head} of {name}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    prob = problem_for(wl, wl.top_p[0])
    _, clean = run_chain(prob, q, k, v)
    clean_o, clean_lse = clean["o"], clean["lse"]

    rng = np.random.default_rng(5)
    toks = rng.choice(wl.seq_len, size=6, replace=False)
    qb, kb = q.clone(), k.clone()
    qb[bad_head, toks[:3], :] = float("nan")
    kb[bad_head, toks[3:5], :] = float("inf")
    kb[bad_head, toks[5], 0] = float("-inf")
    buf, res = run_chain(prob, qb, kb, v)

    H, nb = wl.num_heads, res["nb"]
    rows = H * nb
    lo = min(wl.k_min, nb)
    rc = res["row_count"]
    assert rc.min() >= lo and rc.max() <= nb
    ranked = res["ranked"].reshape(rows, nb)
    np.testing.assert_array_equal(np.sort(ranked, axis=1), np.tile(np.arange(nb), (rows, 1)))
    row_ptr, col_idx = res["row_ptr"], res["col_idx"]
    kept = np.diff(row_ptr)
    assert kept.min() >= lo and kept.max() <= nb
    for r in range(rows):
        c = col_idx[row_ptr[r]: row_ptr[r + 1]]
        assert c.min() >= 0 and c.max() < nb and np.all(np.diff(c) > 0), r
    items, nsplit = int(res["plan_meta"][0]), int(res["plan_meta"][1])
    wo = res["work_order"]
    assert items == rows + nsplit
    assert len(np.unique(wo)) == items

    # the clean heads: the same outputs as the clean call
    o, lse = res["o"], res["lse"]
    for h in range(H):
        if h == bad_head:
            continue
        a = o[h].astype(np.float64)
        b = clean_o[h].astype(np.float64)
        ulp = np.maximum(np.abs(b), 2.0 ** -126) * 2.0 ** -7
        assert np.all(np.abs(a - b) <= ulp), h
        assert np.max(np.abs(lse[h] - clean_lse[h])) <= 1e-5, h
        same = np.mean(a == b)
        say(f"[gpu]   head {h}: {same:.4f} of O bit-identical to the clean call")
