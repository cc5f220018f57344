"""GPU: growing sparsity with reduced search (GSRS S5.1, S5.2, A.2, A.4, A.5).

fva_reselect against the oracle's re-selection from the same fp32 importance
(bit-exact ranking, counts and mask), and whole multi-step trajectories: the
mask every step evaluates, the selection at every search, the importance
against the fp64 oracle, and every step's attention output.
"""

import math

import numpy as np
import pytest
import torch

import adaptive_block_sparse_fva_amd as F
import oracle as O
import oracle.fva_gsrs as G
from adaptive_block_sparse_fva_amd.gsrs import GsrsRunner
from gpu_helpers import LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, device_inputs, f64_inputs, problem_for, say
from synth import WORKLOADS, Workload, make_inputs
from synth.workloads import trajectory_parts, trajectory_step

pytestmark = pytest.mark.gpu

IMPORTANCE_ABS = 1e-4


def _csr(row_ptr_t, col_idx_t):
    rp = row_ptr_t.cpu().numpy().astype(np.int64)
    return rp, col_idx_t[: int(rp[-1])].cpu().numpy().astype(np.int64)


def _expected_mask(ranked, count):
    rp = np.concatenate([[0], np.cumsum(count)])
    cols = np.concatenate([np.sort(ranked[r][: count[r]]) for r in range(len(count))])
    return rp, cols


def _check_selection(H, nb, imp, ev_rp, ev_cols, p, k_min, ranked_t, count_t, head_t, new_rp_t, new_cols_t):
    ranked, count, head = G.select_from_importance(imp, ev_rp, ev_cols, p, k_min)
    np.testing.assert_array_equal(ranked_t.cpu().numpy().astype(np.int64).reshape(H * nb, nb), ranked)
    np.testing.assert_array_equal(count_t.cpu().numpy(), count)
    np.testing.assert_array_equal(head_t.cpu().numpy(), head)
    rp, cols = _expected_mask(ranked, count)
    got_rp, got_cols = _csr(new_rp_t, new_cols_t)
    np.testing.assert_array_equal(got_rp, rp)
    np.testing.assert_array_equal(got_cols, cols)
    for r in range(H * nb):   # the new mask lies inside the evaluated one
        assert set(cols[rp[r]: rp[r + 1]].tolist()) <= set(ev_cols[ev_rp[r]: ev_rp[r + 1]].tolist())
    return count


RESELECT = [
    # name, workload or ad-hoc, evaluated p, new p, k_min
    ("two_head", 0.95, 0.8, 4),
    ("rank480p", 0.95, 0.85, 8),
    ("rank480p_p1", 0.95, 1.0, 8),
    ("two_head_p0_floor", 0.9, 0.0, 6),
    ("odd_kmin_over", 0.7, 0.9, 50),
]


@pytest.mark.parametrize("case", RESELECT, ids=[c[0] for c in RESELECT])
def test_reselect_matches_oracle(case):
    name, p_eval, p_new, k_min = case
    if name.startswith("two_head"):
        wl = WORKLOADS["two_head"]
    elif name.startswith("rank480p"):
        wl = WORKLOADS["rank480p"]
    else:
        wl = Workload(name, 2, 128, (3, 13, 29), 64, (p_eval,), 2, 0, seed=29, heads="lograndom",
                      tile=(5, 7))
    say(f"[gpu] reselect {name} eval p={p_eval} new p={p_new} k_min={k_min}")
    inp = make_inputs(wl, cache=wl.name in WORKLOADS)
    q, k, v = device_inputs(inp)
    prob = problem_for(wl, p_eval, 0)
    buf = F.Buffers.allocate(prob)
    buf.route(q, k, v)
    buf.plan()
    sz = F.sizes(prob)
    block_lse = torch.empty(sz.block_lse_capacity, dtype=torch.float32, device="cuda")
    buf.attn(q, block_lse=block_lse)
    imp = buf.importance(block_lse)
    sp = problem_for(wl, p_new, 0)
    sp.k_min = k_min
    H, nb = wl.num_heads, buf.nb
    ranked = torch.empty(sz.ranked_elems, dtype=torch.int16, device="cuda")
    count = torch.empty(sz.num_rows, dtype=torch.int32, device="cuda")
    head = torch.full((H,), 12345, dtype=torch.int32, device="cuda")  # must be overwritten
    F.reselect(sp, buf.row_ptr, buf.col_idx, imp, ranked, count, head)
    new = F.Buffers.allocate(prob)
    F.plan(prob, ranked, count, new.row_ptr, new.col_idx, new.head_count_final, new.work_order,
           new.plan_meta, new.tile_counter)
    torch.cuda.synchronize()
    ev_rp, ev_cols = _csr(buf.row_ptr, buf.col_idx)
    kept = _check_selection(H, nb, imp.cpu().numpy(), ev_rp, ev_cols, p_new, k_min, ranked, count,
                            head, new.row_ptr, new.col_idx)
    say(f"  evaluated {len(ev_cols)} blocks -> kept {int(kept.sum())}")


TRAJ = [
    # name, heads, d, grid, block, k_min, steps, warmup, searches, ps, reduced
    ("traj_reduced", 2, 128, (3, 16, 32), 64, 2, 8, 2, [2, 4, 6], [0.95, 0.85, 0.75], True),
    ("traj_full_search", 2, 128, (3, 16, 32), 64, 2, 8, 2, [2, 4, 6], [0.95, 0.85, 0.75], False),
    ("traj_b128_d64", 3, 64, (2, 24, 40), 128, 3, 6, 1, [1, 3, 5], [0.9, 0.8, 0.7], True),
]


@pytest.mark.parametrize("case", TRAJ, ids=[c[0] for c in TRAJ])
def test_trajectory_matches_oracle(case):
    name, H, d, grid, block, k_min, steps, warm, at, ps, reduced = case
    wl = Workload(name, H, d, grid, block, (1.0,), k_min, 0, seed=37, heads="lograndom")
    say(f"[gpu] gsrs trajectory {name} N={wl.seq_len} nb={wl.num_blocks} steps={steps}")
    parts = trajectory_parts(wl, steps)
    prob = problem_for(wl, 1.0, 0)
    runner = GsrsRunner(prob, F.gsrs_schedule(steps, warm, at, ps, reduced))
    nb = runner.nb
    order = O.token_order(wl.grid, wl.tile_hw)
    scale = 1.0 / math.sqrt(d)
    full_rp = np.arange(H * nb + 1) * nb
    full_cols = np.tile(np.arange(nb), H * nb)
    cand = None   # the first search's mask
    latest = None
    for t in range(steps):
        inp = trajectory_step(parts, t)
        q, k, v = device_inputs(inp)
        act, p = runner.step(t, q, k, v)
        torch.cuda.synchronize()
        exp_act, exp_p = G.gsrs_action(t, steps, warm, at, ps, reduced)
        assert act == exp_act and p == float(np.float32(exp_p))
        ev_rp, ev_cols = _csr(runner.evaluated.row_ptr, runner.evaluated.col_idx)
        if act in (G.ACT_DENSE, G.ACT_FULL_SEARCH):
            np.testing.assert_array_equal(ev_rp, full_rp)
            np.testing.assert_array_equal(ev_cols, full_cols)
        elif act == G.ACT_CANDIDATE_SEARCH:
            np.testing.assert_array_equal(ev_rp, cand[0])
            np.testing.assert_array_equal(ev_cols, cand[1])
        else:
            np.testing.assert_array_equal(ev_rp, latest[0])
            np.testing.assert_array_equal(ev_cols, latest[1])
        q64, k64, v64 = f64_inputs(inp)
        if act in (G.ACT_FULL_SEARCH, G.ACT_CANDIDATE_SEARCH):
            imp = runner.importance.cpu().numpy()
            ref_imp = O.precise_block_importance(q64, k64, order, block, ev_rp, ev_cols, scale)
            err = np.abs(imp.astype(np.float64) - ref_imp).max()
            assert err <= IMPORTANCE_ABS, err
            kept = _check_selection(H, nb, imp, ev_rp, ev_cols, p, k_min, runner.sel_ranked,
                                    runner.sel_count, runner.sel_head, runner.current.row_ptr,
                                    runner.current.col_idx)
            latest = _csr(runner.current.row_ptr, runner.current.col_idx)
            if act == G.ACT_FULL_SEARCH and cand is None:
                cand = latest
            say(f"  step {t}: search p={p:.2f} evaluated {len(ev_cols)} -> kept {int(kept.sum())} "
                f"(importance err {err:.1e})")
        o_ref, lse_ref = O.masked_attention(q64, k64, v64, order, block, ev_rp, ev_cols, scale)
        do = np.abs(runner.buf.o.float().cpu().numpy() - o_ref)
        dl = np.abs(runner.buf.lse.cpu().numpy() - lse_ref)
        assert do.max() <= O_MAX_ABS and do.mean() <= O_MEAN_ABS and dl.max() <= LSE_MAX_ABS, \
            (t, do.max(), do.mean(), dl.max())
