"""fva_route_noalloc: the routing call for callers that cannot allocate, with
its workspace in the library's static device array, against fva_route with a
caller-allocated workspace.  Outputs must be bitwise the same; two calls in a
row, the second on a smaller problem (the array keeps the first call's
contents, which must not leak into the second's results)."""

import ctypes

import pytest
import torch

import adaptive_block_sparse_fva_amd as F
from adaptive_block_sparse_fva_amd import fva
from gpu_helpers import device_inputs, problem_for, say
from synth import WORKLOADS, make_inputs


def test_route_noalloc_argument_checks_without_a_device():
    lib = F.load_library()
    fake = ctypes.c_void_p(1 << 20)
    p = F.make_problem(5, 32760, 128, (21, 30, 52), 128, (8, 16), 0.95, 8)
    # q k v scores ranked row_count head_count order kv stream
    assert lib.fva_route_noalloc(ctypes.byref(p), None, fake, None, None, fake, fake, fake, fake,
                                 None, None) == fva.FVA_ERR_ARG
    assert lib.fva_route_noalloc(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake,
                                 None, None) == fva.FVA_ERR_ARG
    # 8 heads x 2048 blocks: pooled means 16 MiB + scores 128 MiB > the static array
    big = F.make_problem(8, 2048 * 128, 128, (1, 256, 1024), 128, (8, 16), 0.9, 8)
    assert F.sizes(big).workspace_bytes > fva.FVA_NOALLOC_SCRATCH_BYTES
    assert lib.fva_route_noalloc(ctypes.byref(big), fake, fake, None, None, fake, fake, fake, fake,
                                 None, None) == fva.FVA_ERR_WORKSPACE


@pytest.mark.gpu
def test_route_noalloc_matches_route_on_two_calls():
    for name in ("rank480p", "two_head"):
        wl = WORKLOADS[name]
        say(f"[gpu] route_noalloc vs route {name}")
        inp = make_inputs(wl)
        q, k, v = device_inputs(inp)
        prob = problem_for(wl, wl.top_p[0])
        assert F.sizes(prob).workspace_bytes <= fva.FVA_NOALLOC_SCRATCH_BYTES
        ref = F.Buffers.allocate(prob)
        ref.route(q, k, v)
        got = F.Buffers.allocate(prob)
        got.kv.zero_()
        F.route_noalloc(prob, q, k, v, got.scores, got.ranked, got.row_count, got.head_count,
                        got.order, got.kv)
        alone = F.Buffers.allocate(prob)
        F.route_noalloc(prob, q, k, None, None, alone.ranked, alone.row_count, alone.head_count,
                        alone.order, None)
        torch.cuda.synchronize()
        for key in ("ranked", "row_count", "head_count", "order"):
            assert torch.equal(getattr(got, key), getattr(ref, key)), (name, key)
            assert torch.equal(getattr(alone, key), getattr(ref, key)), (name, key)
        assert torch.equal(got.scores, ref.scores), name
        assert torch.equal(got.kv.view(torch.int16), ref.kv.view(torch.int16)), name
