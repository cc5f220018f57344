"""GPU test: one call of the whole hot path (routing, plan, attention)
captured in a HIP graph and replayed gives the eager call's outputs bit for
bit.

Every C-ABI call only enqueues kernels on the caller's stream (no allocation,
copy, fill or host synchronisation inside a call), so a caller that keeps its
buffers can capture a step once and replay it.  The replays run with eager
work and synchronisations between them (every output cleared), and each
replay is compared with the eager result.
"""

import time

import pytest
import torch

import adaptive_block_sparse_fva_amd as F
from gpu_helpers import device_inputs, problem_for, say
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> torch.Tensor:
    """Bit pattern of a tensor (bitwise comparison, NaN-safe)."""
    if t.dtype in (torch.bfloat16, torch.float16, torch.int16):
        return t.contiguous().view(torch.int16)
    if t.dtype in (torch.float32, torch.int32):
        return t.contiguous().view(torch.int32)
    return t


@pytest.mark.parametrize("name", ["two_head", "rank480p"])
def test_graph_replay_matches_eager(name):
    wl = WORKLOADS[name]
    say(f"[gpu] graph replay {name}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    prob = problem_for(wl, wl.top_p[0])
    buf = F.Buffers.allocate(prob)
    buf.run(q, k, v)
    torch.cuda.synchronize()
    rows = wl.num_heads * buf.nb
    nnz = int(buf.row_ptr[-1].item())
    items, nsplit = int(buf.plan_meta[0].item()), int(buf.plan_meta[1].item())
    # the written part of every output
    parts = {
        "o": lambda b: b.o,
        "lse": lambda b: b.lse,
        "scores": lambda b: b.scores,
        "ranked": lambda b: b.ranked,
        "row_count": lambda b: b.row_count,
        "head_count": lambda b: b.head_count,
        "order": lambda b: b.order,
        "kv": lambda b: b.kv,
        "row_ptr": lambda b: b.row_ptr,
        "col_idx": lambda b: b.col_idx[:nnz],
        "head_count_final": lambda b: b.head_count_final,
        "work_order": lambda b: b.work_order[:items],
        "plan_meta": lambda b: b.plan_meta[: 2 + rows + nsplit],
        "tile_counter": lambda b: b.tile_counter,
    }
    ref = {n: _bits(f(buf)).clone() for n, f in parts.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        buf.run(q, k, v)
    torch.cuda.synchronize()

    for rep in range(3):
        for n, f in parts.items():
            f(buf).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, f in parts.items():
            assert torch.equal(_bits(f(buf)), ref[n]), f"replay {rep}: {n} differs from the eager call"

    # informational: eager calls and replays back to back
    def per_call(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps * 1e3

    say(f"[gpu]   {name}: eager {per_call(lambda: buf.run(q, k, v)):.4f} ms, "
        f"graph replay {per_call(g.replay):.4f} ms per call (host clock)")
