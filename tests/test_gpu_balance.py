"""GPU chain with the cross-rank balance step (FVAttn S3.2-S3.3 on simulated ranks).

R ranks of Hl heads are routed as one R*Hl-head problem; the per-head counts
go to the host search (fva_balance) and budget conversion (fva_sasa_refill),
and the resulting per-head refill feeds fva_plan.  Every integer output must
match the oracle exactly, and attention over the augmented mask must match
the fp64 masked softmax.
"""

import numpy as np
import pytest
import torch

import adaptive_block_sparse_fva_amd as F
import oracle as O
import oracle.fva_balance as B
from gpu_helpers import device_inputs, host, problem_for, say
from synth import Workload, make_inputs
from test_gpu_parity import check_attention

pytestmark = pytest.mark.gpu

WORLD = [
    # name, R, Hl, d, grid, block, p, k_min, topology, k1, k2
    ("ring_forced", 4, 3, 64, (3, 16, 32), 64, 0.9, 2, "ring", 0, 0),
    ("pairs_gated", 8, 2, 128, (4, 24, 32), 128, 0.95, 3, "pairs", 1050, 1100),
    ("sasa_only", 4, 3, 64, (3, 16, 32), 64, 0.9, 2, "pairs", 0, 1_000_000),
    ("balanced", 4, 3, 128, (3, 16, 32), 64, 0.9, 2, "pairs", 1050, 1100),
]


@pytest.mark.parametrize("case", WORLD, ids=[c[0] for c in WORLD])
def test_balanced_refill_chain(case):
    name, R, Hl, d, grid, block, p, kmin, topology, k1, k2 = case
    wl = Workload(name, R * Hl, d, grid, block, (p,), kmin, 0, seed=19, heads="lograndom")
    say(f"[gpu] balance {name} R={R} Hl={Hl} N={wl.seq_len} nb={wl.num_blocks} {topology}")
    inp = make_inputs(wl, cache=False)
    q, k, v = device_inputs(inp)
    prob = problem_for(wl, p, 0)
    buf = F.Buffers.allocate(prob)
    buf.route(q, k, v)
    torch.cuda.synchronize()
    nb = buf.nb
    hc = buf.head_count.cpu().numpy().astype(np.int64)
    rc = buf.row_count.cpu().numpy().astype(np.int64)

    prm = F.balance_params(R, Hl, topology, k1, k2)
    bal = F.balance(prm, hc.reshape(R, Hl))
    ref = B.balance(hc.reshape(R, Hl), topology, k1, k2)
    assert bal["mode"] == ref["mode"]
    for key in ("sigma", "send", "loads_new", "budget"):
        np.testing.assert_array_equal(bal[key], ref[key], err_msg=key)
    refill, added = F.sasa_refill(prm, nb, rc, bal["send"], bal["budget"])
    refill_ref, added_ref = B.refill_from_budget(rc.reshape(R * Hl, nb), nb, R, Hl, bal["send"],
                                                 bal["budget"])
    np.testing.assert_array_equal(refill, refill_ref)
    np.testing.assert_array_equal(added, added_ref)
    say(f"  mode {bal['mode']} moves {bal['moves']} loads {bal['loads_new'].tolist()} "
        f"budget {bal['budget'].tolist()} added {added.tolist()}")

    buf.plan(head_refill=torch.from_numpy(refill).cuda())
    buf.attn(q)
    torch.cuda.synchronize()
    res = host(buf)
    S32 = res["scores"]
    rc_o, hc_o = O.select_counts(S32, p, kmin)
    np.testing.assert_array_equal(rc, rc_o)
    pl = O.plan(S32, rc, 0, head_refill=refill)
    np.testing.assert_array_equal(res["row_ptr"], pl["row_ptr"])
    np.testing.assert_array_equal(res["col_idx"], pl["col_idx"])
    np.testing.assert_array_equal(res["head_count_final"], pl["head_count"])
    work, slot, nsplit = O.work_items(pl["kept"], F.compute_units())
    np.testing.assert_array_equal(res["work_order"], work)

    # SASA bookkeeping: the blocks added per rank are the budget's, on the
    # rank's heads that stayed; moved heads keep their routed counts; no rank
    # passes the post-migration critical load (Eq 10's first term is 0)
    extra = (res["head_count_final"] - hc).reshape(R, Hl)
    for r in range(R):
        s = int(bal["send"][r])
        assert extra[r].sum() == added[r] <= bal["budget"][r]
        if s >= 0:
            assert extra[r, s] == 0
    lmax = int(bal["loads_new"].max())
    assert int((bal["loads_new"] + added).max()) <= lmax
    # the refilled set is a prefix of each row's ranking (no re-sort)
    for row in range(R * Hl * nb):
        a, b = res["row_ptr"][row], res["row_ptr"][row + 1]
        np.testing.assert_array_equal(np.sort(res["ranked"][row][: b - a]), res["col_idx"][a:b])
    check_attention(wl, inp, res, label=name)


def test_head_refill_values_are_clamped():
    wl = Workload("clamp", 4, 64, (2, 16, 16), 64, (0.8,), 1, 0, seed=23, heads="lograndom")
    say("[gpu] head_refill clamping")
    inp = make_inputs(wl, cache=False)
    q, k, v = device_inputs(inp)
    buf = F.Buffers.allocate(problem_for(wl, 0.8, 0))
    buf.route(q, k, v)
    given = np.array([-5, 10 ** 9, 0, 500], np.int32)
    buf.plan(head_refill=torch.from_numpy(given).cuda())
    torch.cuda.synchronize()
    res = host(buf)
    pl = O.plan(res["scores"], res["row_count"], 0,
                head_refill=[0, F.fva.FVA_MAX_HEAD_REFILL, 0, 500])
    np.testing.assert_array_equal(res["row_ptr"], pl["row_ptr"])
    np.testing.assert_array_equal(res["col_idx"], pl["col_idx"])
    nb = res["nb"]
    assert np.all(np.diff(res["row_ptr"])[nb: 2 * nb] == nb)  # the huge refill fills every row
