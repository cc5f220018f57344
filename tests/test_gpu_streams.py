"""GPU test: the entry points keep no state between calls, so independent
calls may run at the same time.

Two problems of different shapes, each with its own buffers, go through
route -> plan -> attention on two streams with their launches interleaved,
and then from two host threads at once; every output equals the one of the
same call run alone, bit for bit.  (The persistent attention grid takes its
work from the call's own queue counter and never waits on another
workgroup, so two attention launches sharing the compute units only slow
each other down.)
"""

import threading

import pytest
import torch

import adaptive_block_sparse_fva_amd as F
from gpu_helpers import device_inputs, host, problem_for, say
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

NAMES = ("two_head", "rank480p")


def _setup():
    out = []
    for name in NAMES:
        wl = WORKLOADS[name]
        q, k, v = device_inputs(make_inputs(wl))
        out.append((name, problem_for(wl, wl.top_p[0]), q, k, v))
    torch.cuda.synchronize()
    return out


def _same(a: dict, b: dict, label: str):
    for key in ("order", "scores", "ranked", "row_count", "head_count", "row_ptr", "col_idx",
                "head_count_final", "plan_meta", "work_order", "tile_counter", "o", "lse"):
        x, y = a[key], b[key]
        if key == "plan_meta":
            n = 2 + len(a["row_count"]) + int(x[1])
            x, y = x[:n], y[:n]
        assert x.shape == y.shape and (x == y).all(), f"{label}: {key} differs from the call run alone"


def _alone(cases):
    refs = []
    for name, prob, q, k, v in cases:
        buf = F.Buffers.allocate(prob)
        buf.run(q, k, v)
        torch.cuda.synchronize()
        refs.append(host(buf))
    return refs


def test_two_streams_interleaved():
    cases = _setup()
    refs = _alone(cases)
    say("[gpu] two problems on two streams, launches interleaved")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [F.Buffers.allocate(c[1]) for c in cases]
    torch.cuda.synchronize()
    for rep in range(2):
        for (name, prob, q, k, v), buf, s in zip(cases, bufs, streams):
            buf.route(q, k, v, stream=s)
        for buf, s in zip(bufs, streams):
            buf.plan(stream=s)
        for (name, prob, q, k, v), buf, s in zip(cases, bufs, streams):
            buf.attn(q, stream=s)
        torch.cuda.synchronize()
        for (name, *_), buf, ref in zip(cases, bufs, refs):
            _same(host(buf), ref, f"{name} (round {rep})")


def test_two_host_threads():
    cases = _setup()
    refs = _alone(cases)
    say("[gpu] two problems from two host threads, each on its own stream")
    bufs = [F.Buffers.allocate(c[1]) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            name, prob, q, k, v = cases[i]
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    bufs[i].run(q, k, v)
            streams[i].synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a host thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for (name, *_), buf, ref in zip(cases, bufs, refs):
        _same(host(buf), ref, name)
