"""GPU: the problem options the workload tests leave at their defaults.

- an explicit softmax scale (the routing's block scores and the attention
  both use it) against the oracle at that scale;
- the attention call without its LSE output gives the same O bit for bit;
- token rows padded past d (stride_token > d, as a fused QKV projection
  leaves them) give the same outputs as contiguous tensors, and nothing is
  written into the padding;
- extreme values: very sharp logits and all-zero queries;
- the compute-unit count the plan's split rule reads is the device's own.
"""

import numpy as np
import pytest
import torch

import adaptive_block_sparse_fva_amd as F
import oracle as O
from gpu_helpers import (LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, S_REL, device_inputs, f64_inputs,
                         problem_for, run_chain, say)
from synth import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


SCALES = [("two_head", 0.05), ("two_head", 0.2), ("tiny", 0.3)]


@pytest.mark.parametrize("name,scale", SCALES, ids=[f"{n}-s{s}" for n, s in SCALES])
def test_explicit_softmax_scale(name, scale):
    wl = WORKLOADS[name]
    p = wl.top_p[0]
    say(f"[gpu] sm_scale {scale} on {name}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    _, res = run_chain(problem_for(wl, p, sm_scale=scale), q, k, v)
    H, nb = wl.num_heads, res["nb"]
    q64, k64, v64 = f64_inputs(inp)
    order = O.token_order(wl.grid, wl.tile_hw)
    s64 = O.block_scores(O.pool(q64, order, wl.block), O.pool(k64, order, wl.block), scale)
    err = np.abs(res["scores"].astype(np.float64) - s64).max()
    assert err <= S_REL * np.abs(s64).max(), f"score error {err}"
    S32 = res["scores"]
    for r in range(H * nb):
        h, i = divmod(r, nb)
        np.testing.assert_array_equal(res["ranked"][r], O.ranking(S32[h, i]), err_msg=f"row {r}")
    rc, hc = O.select_counts(S32, p, wl.k_min)
    np.testing.assert_array_equal(res["row_count"], rc)
    np.testing.assert_array_equal(res["head_count"], hc)
    pl = O.plan(S32, rc, wl.refill_per_mille)
    np.testing.assert_array_equal(res["row_ptr"], pl["row_ptr"])
    np.testing.assert_array_equal(res["col_idx"], pl["col_idx"])
    o_ref, lse_ref = O.masked_attention(q64, k64, v64, order, wl.block, pl["row_ptr"], pl["col_idx"], scale)
    do = np.abs(res["o"] - o_ref)
    dl = np.abs(res["lse"] - lse_ref)
    say(f"  O max-abs {do.max():.3e} mean-abs {do.mean():.3e}; LSE max-abs {dl.max():.3e}")
    assert do.max() <= O_MAX_ABS and do.mean() <= O_MEAN_ABS and dl.max() <= LSE_MAX_ABS


@pytest.mark.parametrize("name", ["two_head", "rank480p"])
def test_lse_output_is_optional(name):
    wl = WORKLOADS[name]
    say(f"[gpu] attention without LSE on {name}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    prob = problem_for(wl, wl.top_p[0])
    buf, with_lse = run_chain(prob, q, k, v)
    buf.o.zero_()
    buf.attn(q, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(buf.o.float().cpu(), torch.from_numpy(with_lse["o"]).float())


PADDED = [
    # name, heads, d, grid, block, p, k_min, pad
    ("two_head", None, None, None, None, None, None, 8),
    ("d64_ragged", 3, 64, (3, 9, 11), 64, 0.8, 2, 24),
]


@pytest.mark.parametrize("case", PADDED, ids=[c[0] for c in PADDED])
def test_padded_token_rows(case):
    name, H, d, grid, block, p, kmin, pad = case
    wl = WORKLOADS[name] if H is None else Workload(name, H, d, grid, block, (p,), kmin, 0, seed=53,
                                                    heads="lograndom")
    p = wl.top_p[0]
    say(f"[gpu] token rows padded by {pad} on {name}")
    inp = make_inputs(wl, cache=False) if H is not None else make_inputs(wl)
    q, k, v = device_inputs(inp)
    _, ref = run_chain(problem_for(wl, p), q, k, v)
    Hh, N, dd = q.shape
    width = dd + pad

    def padded(x):
        t = torch.full((Hh, N, width), float("nan"), dtype=torch.bfloat16, device="cuda")
        t[:, :, :dd] = x
        return t

    qp, kp, vp = padded(q), padded(k), padded(v)
    prob = problem_for(wl, p, stride_head=N * width, stride_token=width)
    buf = F.Buffers.allocate(prob)
    sentinel = torch.tensor(12345.0, dtype=torch.bfloat16)
    # the allocated o follows the problem's strides; the padding between its
    # rows (storage outside the view) is filled to see that nothing writes it
    assert buf.o.shape == (Hh, N, dd) and buf.o.stride() == (N * width, width, 1)
    n_storage = buf.o.untyped_storage().nbytes() // 2
    o_storage = buf.o.as_strided((n_storage,), (1,))
    o_storage.fill_(sentinel.item())
    buf.run(qp, kp, vp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(buf.o.float().cpu().numpy(), ref["o"])
    np.testing.assert_array_equal(buf.lse.cpu().numpy(), ref["lse"].astype(np.float32))
    np.testing.assert_array_equal(buf.row_ptr.cpu().numpy(), ref["row_ptr"])
    in_view = np.zeros(n_storage, bool)
    offs = (np.arange(Hh)[:, None, None] * N * width + np.arange(N)[None, :, None] * width
            + np.arange(dd)[None, None, :])
    in_view[offs.ravel()] = True
    outside = o_storage.float().cpu().numpy()[~in_view]
    assert outside.size > 0 and bool((outside == sentinel.item()).all()), "padding was written"


def _scaled_bits(bits: np.ndarray, pow2: int) -> np.ndarray:
    """bf16 bits times 2^pow2, exactly (only the exponent changes)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** pow2)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


VALUES = [("sharp_logits", 3), ("zero_queries", None)]


@pytest.mark.parametrize("name,pow2", VALUES, ids=[c[0] for c in VALUES])
def test_extreme_values(name, pow2):
    """Q and K times 8 (logits x 64: the running maximum moves by far more than
    the rescale threshold, most weights underflow), and all-zero queries
    (every block score ties at 0, so the ranking is by block id alone, and
    every kept key has the same weight)."""
    import dataclasses

    from test_gpu_parity import check_attention, check_routing_and_plan

    wl = WORKLOADS["two_head"]
    p = wl.top_p[0]
    say(f"[gpu] {name}")
    inp = make_inputs(wl)
    if pow2 is None:
        inp = dataclasses.replace(inp, q=np.zeros_like(inp.q))
    else:
        inp = dataclasses.replace(inp, q=_scaled_bits(inp.q, pow2), k=_scaled_bits(inp.k, pow2))
    q, k, v = device_inputs(inp)
    _, res = run_chain(problem_for(wl, p), q, k, v)
    check_routing_and_plan(wl, inp, res, p, wl.refill_per_mille)
    if pow2 is None:
        check_attention(wl, inp, res, label=name)
    else:
        # O to the usual bar; the LSE to a bar relative to its size: with
        # logits of magnitude 10^2 .. 10^4 the fp32 dot products themselves
        # carry errors of ~1e-6 relative (d = 128 terms of up to 10^5 each),
        # and a sharp softmax's LSE is its largest logit
        q64, k64, v64 = f64_inputs(inp)
        order = O.token_order(wl.grid, wl.tile_hw)
        o_ref, lse_ref = O.masked_attention(q64, k64, v64, order, wl.block, res["row_ptr"], res["col_idx"],
                                            1.0 / np.sqrt(wl.head_dim))
        do = np.abs(res["o"] - o_ref)
        dl = np.abs(res["lse"] - lse_ref)
        rel = dl / (1e-3 + 2.0 ** -16 * np.abs(lse_ref))
        say(f"  O max-abs {do.max():.3e} mean-abs {do.mean():.3e}; LSE max-abs {dl.max():.3e} "
            f"(|LSE| up to {np.abs(lse_ref).max():.3e}, worst error / bar {rel.max():.2f})")
        assert do.max() <= O_MAX_ABS and do.mean() <= O_MEAN_ABS
        assert rel.max() <= 1.0
    if pow2 is None:
        np.testing.assert_array_equal(res["ranked"], np.tile(np.arange(res["nb"]), (wl.num_heads * res["nb"], 1)))


def test_compute_units_is_the_device_count():
    """The plan's split rule uses this count; it is the device's own."""
    assert F.compute_units() == torch.cuda.get_device_properties(0).multi_processor_count
