"""Benchmark of one adaptive block-sparse attention call on one MI355X.

A step is one whole call of the hot path on resident inputs: fva_route
(order, pooled scores, ranking, Top-p + floor) -> fva_plan (refill, CSR, LPT
order) -> fva_sparse_attn_fwd.  The default workload is one rank's share of a
480p-style video DiT layer: 5 heads x 32,760 tokens (21 x 30 x 52 latent grid),
head_dim 128, block 128, p = 0.95, k_min = 8.

Prints ONE JSON line (see the keys below).  `--gpus N` with N > 1 exits: this
build runs on one GPU.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("ms/attention call + dense-equiv TFLOPS; kept-block MFMA util at 5 heads×32K tokens")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
WARMUP_MIN_S = 0.1          # least GPU-busy time of the warm-up


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="rank480p")
    ap.add_argument("--top-p", type=float, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle's attention sample on workloads other "
                         "than rank480p (rank480p runs every tile)")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-dense", action="store_true")
    ap.add_argument("--skip-balance", action="store_true",
                    help="skip the eight-rank balance simulation (RLB + SASA)")
    ap.add_argument("--skip-gsrs", action="store_true",
                    help="skip the growing-sparsity / reduced-search trajectory")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device to device three times (a known byte count for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def kept_flops_and_pairs(row_ptr, col_idx, n_tokens, block, head_dim, num_heads, nb):
    import numpy as np
    sizes = np.minimum(block, n_tokens - np.arange(nb) * block).astype(np.int64)
    col_sizes = sizes[col_idx]
    per_row = np.add.reduceat(col_sizes, row_ptr[:-1]) if len(col_idx) else np.zeros(len(row_ptr) - 1)
    q_sizes = np.tile(sizes, num_heads)
    return int(4 * head_dim * int((q_sizes * per_row).sum())), int(len(col_idx))


def measured_traffic():
    """HBM traffic of the attention launch from the committed counter summary,
    or None when the kernel source differs from the one the counters were taken on."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "sparse_attn_fwd_rank480p_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["source_files"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return int(rec["fetch_kib_per_dispatch"] * rec["fetch_scale"] * 1024
               + rec["write_kib_per_dispatch"] * rec["write_scale"] * 1024)


def list_schedule_makespan(costs, workers):
    """Greedy list scheduling (each tile to the earliest-free worker)."""
    import heapq
    heap = [0.0] * workers
    heapq.heapify(heap)
    for c in costs:
        t = heapq.heappop(heap)
        heapq.heappush(heap, t + float(c))
    return max(heap)


def cpu_baseline(wl, inp, p, gpu_o, row_ptr_gpu, col_idx_gpu, budget_s, all_tiles):
    """The oracle as it stands, on the host cores: full routing + plan, and the
    fp64 masked attention on every tile (all_tiles) or on a seeded sample of
    tiles bounded by budget_s, extrapolated by kept FLOPs."""
    import numpy as np
    import oracle as O
    from synth import bf16_bits_to_f64

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    q64, k64, v64 = (bf16_bits_to_f64(x) for x in (inp.q, inp.k, inp.v))
    t0 = time.perf_counter()
    r = O.route(q64, k64, wl.grid, wl.tile_hw, wl.block, p, wl.k_min)
    t1 = time.perf_counter()
    pl = O.plan(r["scores32"], r["row_count"], wl.refill_per_mille)
    t2 = time.perf_counter()
    nb, H = wl.num_blocks, wl.num_heads
    total_flops, _ = kept_flops_and_pairs(pl["row_ptr"], pl["col_idx"], wl.seq_len, wl.block,
                                          wl.head_dim, H, nb)
    rng = np.random.default_rng(123)
    perm = rng.permutation(H * nb)
    scale = 1.0 / math.sqrt(wl.head_dim)
    done, flops, start = [], 0, time.perf_counter()
    sizes = np.minimum(wl.block, wl.seq_len - np.arange(nb) * wl.block)
    # attention on the GPU's own mask so that the sample doubles as a parity check
    for t in perm:
        o_ref, _ = O.masked_attention(q64, k64, v64, r["order"], wl.block, row_ptr_gpu, col_idx_gpu,
                                      scale, [int(t)])
        h, i = divmod(int(t), nb)
        toks = r["order"][i * wl.block: min(wl.seq_len, (i + 1) * wl.block)]
        err = np.abs(gpu_o[h, toks] - o_ref[h, toks])
        done.append((err.max(), err.mean()))
        cols = col_idx_gpu[row_ptr_gpu[t]: row_ptr_gpu[t + 1]]
        flops += 4 * wl.head_dim * int(sizes[i]) * int(sizes[cols].sum())
        if not all_tiles and time.perf_counter() - start > budget_s:
            break
    t_attn_sample = time.perf_counter() - start
    gpu_flops, _ = kept_flops_and_pairs(row_ptr_gpu, col_idx_gpu, wl.seq_len, wl.block,
                                        wl.head_dim, H, nb)
    complete = len(done) == H * nb
    t_attn_full = t_attn_sample if complete else t_attn_sample * gpu_flops / max(flops, 1)
    value_ms = (t1 - t0 + t2 - t1 + t_attn_full) * 1e3
    errs = np.array(done)
    if complete:
        what = (f"fp64 masked attention on all {H * nb} tiles ({gpu_flops / 1e9:.1f} GFLOP kept, "
                f"{t_attn_sample:.1f}s)")
    else:
        what = (f"fp64 masked attention on {len(done)} of {H * nb} seeded-random tiles "
                f"({flops / 1e9:.1f} of {gpu_flops / 1e9:.1f} GFLOP kept, {t_attn_sample:.1f}s), "
                f"extrapolated by kept FLOPs")
    return {
        "value": round(value_ms, 1),
        "unit": "ms",
        "cores": blas_threads if blas_threads else cores,
        "kind": "oracle",
        "sample": f"full routing+plan ({t1 - t0:.2f}s + {t2 - t1:.2f}s); {what}",
        "host_cores_visible": cores,
        "sample_parity": {"o_max_abs": float(errs[:, 0].max()), "o_mean_abs": float(errs[:, 1].mean()),
                          "o_mean_abs_per_tile_max": float(errs[:, 1].max()), "tiles": len(done)},
        "oracle_matches_gpu_mask": bool(np.array_equal(pl["row_ptr"], row_ptr_gpu)
                                        and np.array_equal(pl["col_idx"], col_idx_gpu)),
    }


def measured_cu_imbalance(trace, grid):
    """The one-GPU analog of FVAttn S2.2 Eq 2 from a traced attention launch:
    per-item start/end clocks grouped by workgroup and by compute unit.

    load = the summed durations of the items a unit (or workgroup) ran;
    finish = when its last item ended, from the launch's first item start.
    rho = max / mean of each, over the units that ran items."""
    import numpy as np
    rt0, rt1, c0, c1, place, wg = (trace[:, j] for j in range(6))
    start = rt0.min()
    xcc = (place >> 32) & 0xffff
    cu = (xcc << 8) | ((place >> 8) & 0xff)  # XCC, engine, array and CU fields
    dur = (rt1 - rt0).astype(np.float64)

    def rho(keys):
        uk, inv = np.unique(keys, return_inverse=True)
        load = np.bincount(inv, weights=dur)
        fin = np.zeros(len(uk))
        np.maximum.at(fin, inv, (rt1 - start).astype(np.float64))
        return len(uk), float(load.max() / load.mean()), float(fin.max() / fin.mean())

    n_cu, rho_cu_load, rho_cu_finish = rho(cu)
    n_wg, rho_wg_load, rho_wg_finish = rho(wg)
    span_us = float(rt1.max() - start) / 100.0  # 100 MHz constant clock
    return {"clock": "s_memrealtime (100 MHz) per work item, one traced launch",
            "compute_units_seen": int(n_cu), "workgroups_seen": int(n_wg),
            "per_compute_unit": {"load": round(rho_cu_load, 4), "finish": round(rho_cu_finish, 4)},
            "per_workgroup": {"load": round(rho_wg_load, 4), "finish": round(rho_wg_finish, 4)},
            "span_us": round(span_us, 1),
            "mean_item_us": round(float(dur.mean()) / 100.0, 2),
            "cycles_per_us": round(float((c1 - c0).sum()) / float(dur.sum()) * 100.0, 1)}


def balance_simulation(stream, cpu_reps=200, reps=3):
    """FVAttn S3.2-S3.3 on eight simulated ranks of five heads (the 480p-style
    layer split across 8 GPUs), run one rank after another on this GPU.

    The 40 heads are routed in one call; their kept-block counts go to the
    host search (fva_balance: gating, one-head-per-rank migration plan, slack
    budgets) and budget conversion (fva_sasa_refill).  Each rank's head set --
    before migration, after it, and after it with the slack refill -- is then
    gathered into its own buffers (one GPU's stand-in for the point-to-point
    head transfer) and its plan + attention timed.  Reports the search time
    and the imbalance of block counts and of measured attention times.
    """
    import numpy as np
    import torch

    import adaptive_block_sparse_fva_amd as F
    from synth import WORKLOADS, make_inputs

    wl = WORKLOADS["world480p"]
    R, Hl = 8, 5
    H, N, d, B, p = wl.num_heads, wl.seq_len, wl.head_dim, wl.block, wl.top_p[0]
    inp = make_inputs(wl, cache=False)
    dev = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    del inp
    wprob = F.make_problem(H, N, d, wl.grid, B, wl.tile_hw, p, wl.k_min, 0)
    wbuf = F.Buffers.allocate(wprob)
    wbuf.route(q, k, v)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    wbuf.route(q, k, v)
    e1.record(stream)
    torch.cuda.synchronize()
    world_route_ms = e0.elapsed_time(e1)
    nb = wbuf.nb
    hc = wbuf.head_count.cpu().numpy().astype(np.int64)
    rc = wbuf.row_count.cpu().numpy().astype(np.int64)
    del wbuf

    def host_us(fn):
        fn()
        t0 = time.perf_counter()
        for _ in range(cpu_reps):
            fn()
        return (time.perf_counter() - t0) / cpu_reps * 1e6

    prm = F.balance_params(R, Hl, "pairs")
    bal = F.balance(prm, hc.reshape(R, Hl))
    refill, added = F.sasa_refill(prm, nb, rc, bal["send"], bal["budget"])
    forced = F.balance_params(R, Hl, "pairs", 0, 0)
    ring = F.balance_params(R, Hl, "ring", 0, 0)
    timing_us = {
        "balance_pairs": round(host_us(lambda: F.balance(forced, hc.reshape(R, Hl))), 1),
        "balance_ring": round(host_us(lambda: F.balance(ring, hc.reshape(R, Hl))), 1),
        "sasa_refill": round(host_us(lambda: F.sasa_refill(prm, nb, rc, bal["send"], bal["budget"])), 1),
    }
    ring_plan = F.balance(ring, hc.reshape(R, Hl))

    sigma, send = bal["sigma"], bal["send"]
    src = np.empty(R, np.int64)
    src[sigma] = np.arange(R)

    def heads_of(r, migrated):
        own = [r * Hl + j for j in range(Hl)]
        if not migrated or sigma[r] == r:
            return own
        s = int(src[r])
        return [h for j, h in enumerate(own) if j != send[r]] + [s * Hl + int(send[s])]

    rprob = F.make_problem(Hl, N, d, wl.grid, B, wl.tile_hw, p, wl.k_min, 0)
    rbuf = F.Buffers.allocate(rprob)
    schedules = {"routed": (False, False), "rlb": (True, False), "rlb_sasa": (True, True)}
    attn_ms, plan_ms, kept = {}, {}, {}
    for name, (migrated, sasa) in schedules.items():
        attn_ms[name], plan_ms[name], kept[name] = [], [], []
        for r in range(R):
            idx = torch.tensor(heads_of(r, migrated), dtype=torch.long, device="cuda")
            qr, kr, vr = (torch.index_select(x, 0, idx).contiguous() for x in (q, k, v))
            f = refill[idx.cpu().numpy()] if sasa else np.zeros(Hl, np.int32)
            fr = torch.from_numpy(np.ascontiguousarray(f, dtype=np.int32)).cuda()
            rbuf.route(qr, kr, vr)
            rbuf.plan(head_refill=fr)
            rbuf.attn(qr)
            torch.cuda.synchronize()
            if not np.array_equal(rbuf.head_count.cpu().numpy(), hc[idx.cpu().numpy()]):
                raise RuntimeError("a rank's routed counts differ from the world routing")
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            tp, ta = [], []
            for _ in range(reps):
                ev[0].record(stream)
                rbuf.plan(head_refill=fr)
                ev[1].record(stream)
                rbuf.attn(qr)
                ev[2].record(stream)
                torch.cuda.synchronize()
                tp.append(ev[0].elapsed_time(ev[1]))
                ta.append(ev[1].elapsed_time(ev[2]))
            plan_ms[name].append(round(float(np.median(tp)), 4))
            attn_ms[name].append(round(float(np.median(ta)), 4))
            kept[name].append(int(rbuf.row_ptr[-1].item()))
    del rbuf

    def rho(x):
        x = np.asarray(x, dtype=np.float64)
        return round(float(x.max() / x.mean()), 4)

    return {
        "world": "world480p: 8 ranks x 5 heads of the 480p-style layer, routed as one 40-head call",
        "topology": "pairs", "k1_k2_n1_n2_per_mille": [1050, 1100, 800, 70],
        "mode": int(bal["mode"]), "moves": int(bal["moves"]),
        "sigma": sigma.tolist(), "send_head": send.tolist(),
        "rank_blocks": {"routed": hc.reshape(R, Hl).sum(axis=1).tolist(),
                        "rlb": bal["loads_new"].tolist(),
                        "rlb_sasa": (bal["loads_new"] + added).tolist()},
        "rho_blocks": {"routed": bal["rho_per_mille"] / 1000, "rlb": bal["rho_new_per_mille"] / 1000,
                       "rlb_sasa": rho(bal["loads_new"] + added),
                       "ring_rlb": ring_plan["rho_new_per_mille"] / 1000},
        "budget": bal["budget"].tolist(), "blocks_added": added.tolist(),
        "head_refill_per_mille": refill.tolist(),
        "rank_attn_ms": attn_ms, "rank_plan_ms": plan_ms, "rank_kept_blocks": kept,
        "rho_attn_time": {k2: rho(v2) for k2, v2 in attn_ms.items()},
        "critical_attn_ms": {k2: max(v2) for k2, v2 in attn_ms.items()},
        "host_us": timing_us,
        "world_route_ms": round(world_route_ms, 4),
    }


def gsrs_trajectory(stream, steps=10, warmup=2, at=(2, 4, 6, 8), ps=(0.95, 0.9, 0.85, 0.8)):
    """GSRS S5.1 / A.5 / A.7 on a synthetic denoising trajectory of the
    480p-style rank share (inputs of each step from synth.trajectory_step):
    dense warm-up, searches with decreasing p, mask reuse between them; once
    with reduced search (later searches over the first search's mask) and once
    without (every search over all blocks).  Per step: time (HIP events around
    the step's calls, route included), the evaluated density and the
    attention recall against dense attention on the same inputs.  A search's
    overhead is its step time minus the time of the reuse step after it."""
    import numpy as np
    import torch

    import adaptive_block_sparse_fva_amd as F
    from adaptive_block_sparse_fva_amd.gsrs import GsrsRunner
    from synth import WORKLOADS
    from synth.workloads import trajectory_parts, trajectory_step

    wl = WORKLOADS["rank480p"]
    H, N, d, B = wl.num_heads, wl.seq_len, wl.head_dim, wl.block
    parts = trajectory_parts(wl, steps)
    dev = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    inputs = []
    for t in range(steps):
        x = trajectory_step(parts, t)
        inputs.append((dev(x.q), dev(x.k), dev(x.v)))
    del parts
    prob = F.make_problem(H, N, d, wl.grid, B, wl.tile_hw, 1.0, wl.k_min, 0)
    dense = F.Buffers.allocate(prob)
    lse_dense = []
    for q, k, v in inputs:
        dense.run(q, k, v)
        lse_dense.append(dense.lse.clone())
    torch.cuda.synchronize()
    del dense

    out = {"workload": f"rank480p-shaped trajectory, {steps} steps (eta 0.5, kappa 0.5, beta 12)",
           "warmup": warmup, "search_steps": list(at), "top_p": list(ps)}
    for label, reduced in (("reduced_search", True), ("full_search", False)):
        sched = F.gsrs_schedule(steps, warmup, list(at), list(ps), reduced)
        for attempt in range(2):  # the first pass warms up, the second is timed
            runner = GsrsRunner(prob, sched)
            ms, acts, dens, rec = [], [], [], []
            nb = runner.nb
            for t, (q, k, v) in enumerate(inputs):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                act, _ = runner.step(t, q, k, v)
                e1.record(stream)
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
                acts.append(act)
                ev = int(runner.evaluated.row_ptr[-1].item())
                dens.append(ev / (H * nb * nb))
                rec.append(torch.exp(runner.buf.lse - lse_dense[t]).mean().item())
        names = {F.fva.FVA_GSRS_DENSE: "dense", F.fva.FVA_GSRS_FULL_SEARCH: "full_search",
                 F.fva.FVA_GSRS_CANDIDATE_SEARCH: "candidate_search", F.fva.FVA_GSRS_REUSE: "reuse"}
        overhead, later = 0.0, 0.0
        searches = [t for t, a in enumerate(acts)
                    if a in (F.fva.FVA_GSRS_FULL_SEARCH, F.fva.FVA_GSRS_CANDIDATE_SEARCH)]
        for t in searches:
            if t + 1 < steps and acts[t + 1] == F.fva.FVA_GSRS_REUSE:
                overhead += ms[t] - ms[t + 1]
                if t != searches[0]:
                    later += ms[t] - ms[t + 1]
        out[label] = {"total_ms": round(sum(ms), 4), "step_ms": [round(x, 4) for x in ms],
                      "actions": [names[a] for a in acts],
                      "evaluated_density": [round(x, 4) for x in dens],
                      "recall": [round(x, 4) for x in rec],
                      "search_overhead_ms": round(overhead, 4),
                      "later_search_overhead_ms": round(later, 4)}
        del runner
    r, f = out["reduced_search"]["search_overhead_ms"], out["full_search"]["search_overhead_ms"]
    out["overhead_ratio_full_over_reduced"] = round(f / r, 3) if r > 0 else None
    r2, f2 = (out["reduced_search"]["later_search_overhead_ms"],
              out["full_search"]["later_search_overhead_ms"])
    out["later_search_overhead_ratio"] = round(f2 / r2, 3) if r2 > 0 else None
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library covers one "
              "GPU's share of the heads, and the multi-GPU head migration is a host-side simulation "
              "(the balance step), not a multi-GPU run.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        n = 256 * 1024 * 1024  # float32: 1 GiB read and 1 GiB written per copy
        x = torch.ones(n, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print("copied 1 GiB x 3", flush=True)
        return

    import adaptive_block_sparse_fva_amd as F
    from synth import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    p = args.top_p if args.top_p is not None else wl.top_p[0]
    torch.cuda.set_device(0)
    inp = make_inputs(wl)
    dev = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    H, N, d, B = wl.num_heads, wl.seq_len, wl.head_dim, wl.block
    prob = F.make_problem(H, N, d, wl.grid, B, wl.tile_hw, p, wl.k_min, wl.refill_per_mille)
    buf = F.Buffers.allocate(prob)
    stream = torch.cuda.current_stream()

    # Warm-up: W steps, continued until the warm-up has kept the GPU busy for
    # WARMUP_MIN_S.  Coming out of idle the chip runs the step ~12% slower for
    # its first ~20 ms and reaches its steady rate after ~40 ms (measured on
    # this workload), so a handful of steps would leave that ramp inside the
    # timed region.  The JSON line reports the steps actually run.
    warm_run = 0
    warm_t0 = time.perf_counter()
    while warm_run < args.warmup or time.perf_counter() - warm_t0 < WARMUP_MIN_S:
        buf.run(q, k, v)
        torch.cuda.synchronize()
        warm_run += 1

    K = args.steps
    # Timed region: K whole steps between two events.  Inside it only the
    # attention call is bracketed (its duration feeds the roofline figure):
    # every timing event recorded between two launches leaves the GPU idle
    # for a few microseconds, so the route and plan phases are timed in a
    # separate pass below rather than here.
    ev_a = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    ev_run = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev_run[0].record(stream)
    for s in range(K):
        buf.route(q, k, v)
        buf.plan()
        ev_a[s][0].record(stream)
        buf.attn(q)
        ev_a[s][1].record(stream)
    ev_run[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev_run[0].elapsed_time(ev_run[1])
    ms_per_step = total_ms / K
    t_attn = np.array([e[0].elapsed_time(e[1]) for e in ev_a])

    # per-phase breakdown (diagnostic, untimed for the headline): the same
    # steps with an event between every two phases
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for s in range(K):
        e = ev[s]
        e[0].record(stream)
        buf.route(q, k, v)
        e[1].record(stream)
        buf.plan()
        e[2].record(stream)
        buf.attn(q)
        e[3].record(stream)
    torch.cuda.synchronize()
    t_route = np.array([e[0].elapsed_time(e[1]) for e in ev])
    t_plan = np.array([e[1].elapsed_time(e[2]) for e in ev])
    t_step = np.array([e[0].elapsed_time(e[3]) for e in ev])

    nb = buf.nb
    row_ptr = buf.row_ptr.cpu().numpy().astype(np.int64)
    col_idx = buf.col_idx[: int(row_ptr[-1])].cpu().numpy().astype(np.int64)
    head_final = buf.head_count_final.cpu().numpy()
    kept, pairs = kept_flops_and_pairs(row_ptr, col_idx, N, B, d, H, nb)
    dense_flops = 4.0 * N * N * d * H
    attn_avg_ms = float(t_attn.mean())
    achieved_tflops = kept / (attn_avg_ms * 1e-3) / 1e12
    # Routing (FVAttn S3.1: pooled Q/K scores, Top-p + floor, counts,
    # ranking) on its own algorithmic bytes: Q and K read once, the ranking,
    # the counts and the order table written (the scores stay in the
    # workspace).  The step itself runs the fused pass, which also writes K
    # and V in the attention's layout (V read once more, K and V written) and
    # exports the scores; that pass and the K/V re-layout on its own are
    # reported beside it.  Rates are over calls back to back (same inputs,
    # same outputs): inside a step, the event in front of the first routing
    # kernel leaves a few idle microseconds that are no part of routing.
    route_bytes = 2 * H * N * d * 2 + H * nb * nb * 2 + H * nb * 4 + H * 4 + nb * B * 4
    kv_bytes = 2 * H * N * d * 2 + 2 * H * nb * B * d * 2 + nb * B * 4
    fused_bytes = route_bytes + H * N * d * 2 + 2 * H * nb * B * d * 2 + H * nb * nb * 4

    def back_to_back_ms(fn, n=10):
        er = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(5):  # untimed: after the attention calls the caches hold their output
            fn()
        torch.cuda.synchronize()
        er[0].record(stream)
        for _ in range(n):
            fn()
        er[1].record(stream)
        torch.cuda.synchronize()
        return er[0].elapsed_time(er[1]) / n

    def hbm(nbytes, ms):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"bytes": nbytes, "ms_back_to_back": round(ms, 4), "GB/s": round(gbs, 1),
                "frac": round(gbs / PEAK_HBM_GBS, 4), "frac_of_copy": round(gbs / copy_gbs, 4)}

    rbuf = F.Buffers.allocate(prob)
    plan_b2b_ms = back_to_back_ms(lambda: buf.plan())
    route_b2b_ms = back_to_back_ms(lambda: rbuf.route(q, k, with_scores=False))
    if not (torch.equal(rbuf.ranked, buf.ranked) and torch.equal(rbuf.row_count, buf.row_count)):
        raise RuntimeError("routing alone decided differently from the fused pass")
    fused_ms = back_to_back_ms(lambda: buf.route(q, k, v))
    kv_ms = back_to_back_ms(lambda: rbuf.kv_layout(k, v))
    del rbuf
    route_gbs = route_bytes / (route_b2b_ms * 1e-3) / 1e9

    # one-GPU analog of the load-imbalance factor: work list-scheduled onto the
    # persistent workgroups -- the plan's work items (heavy tiles cut in two,
    # heaviest first), whole tiles heaviest first, whole tiles in natural order
    workers = F.attn_workgroups(prob)
    costs = np.diff(row_ptr)
    meta = buf.plan_meta.cpu().numpy()
    items = buf.work_order[: int(meta[0])].cpu().numpy()
    slot = meta[2: 2 + H * nb]
    it_tile, it_part = items // 2, items % 2
    it_cost = np.where(slot[it_tile] < 0, costs[it_tile],
                       np.where(it_part == 0, (costs[it_tile] + 1) // 2, costs[it_tile] // 2))
    planned = list_schedule_makespan(it_cost, workers)
    lpt = list_schedule_makespan(np.sort(costs)[::-1], workers)
    natural = list_schedule_makespan(costs, workers)
    ideal = costs.sum() / workers
    # the same per compute unit (its resident workgroups share its throughput,
    # so a unit behaves like one worker at the unit's rate)
    cus = F.compute_units()
    ideal_cu = costs.sum() / cus
    per_cu = {"planned": round(list_schedule_makespan(it_cost, cus) / ideal_cu, 4),
              "natural": round(list_schedule_makespan(costs, cus) / ideal_cu, 4)}

    # measured imbalance: one traced attention launch (bitwise the same call,
    # per-item clocks), next to the list-scheduling estimate above
    trace = torch.empty((int(meta[0]), F.fva.FVA_TRACE_FIELDS), dtype=torch.int64, device="cuda")
    buf.attn(q, item_trace=trace)
    torch.cuda.synchronize()
    measured = measured_cu_imbalance(trace.cpu().numpy(), workers)
    del trace

    # GSRS precise block importance (phase 1 inside the attention call, phase
    # 2 as its own kernel): cost over the plain attention call
    nnz = int(row_ptr[-1])
    block_lse = torch.empty(nnz * B, dtype=torch.float32, device="cuda")
    imp = torch.empty((H, nb, nb), dtype=torch.float32, device="cuda")
    buf.attn(q, block_lse=block_lse)
    buf.importance(block_lse, imp)
    torch.cuda.synchronize()
    # the chip's clock moves by several percent between bursts of work, so the
    # plain and the recording attention call are timed in alternating rounds
    plain_ms, lse_ms, imp_ms = [], [], []
    for _ in range(5):
        plain_ms.append(back_to_back_ms(lambda: buf.attn(q), n=4))
        lse_ms.append(back_to_back_ms(lambda: buf.attn(q, block_lse=block_lse), n=4))
        imp_ms.append(back_to_back_ms(lambda: buf.importance(block_lse, imp), n=4))
    attn_plain_ms, attn_lse_ms, imp_ms = (float(np.median(x)) for x in (plain_ms, lse_ms, imp_ms))
    precise = {"attn_ms": round(attn_plain_ms, 4), "attn_with_block_lse_ms": round(attn_lse_ms, 4),
               "importance_kernel_ms": round(imp_ms, 4),
               "overhead_vs_attn": round((attn_lse_ms + imp_ms) / attn_plain_ms - 1.0, 4),
               "block_lse_bytes": nnz * B * 4,
               "timed": "medians of 5 alternating rounds of 4 calls each"}

    # the bf16 MFMA rate this device sustains with no memory traffic (its
    # clock under MFMA load depends on the operand data): context for the
    # roofline fraction against the nominal peak
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(2 * cus * 256, dtype=torch.float32, device="cuda")
    ceiling = {}
    for label, rnd in (("random_operands", True), ("zero_operands", False)):
        F.mfma_probe(200, rnd, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        flops = F.mfma_probe(20000, rnd, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        ceiling[label] = round(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)

    # the HBM rate a plain device copy reaches on this machine (1 GiB read and
    # 1 GiB written per copy): the achievable counterpart of the 8 TB/s peak
    xa = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
    xb = torch.empty_like(xa)
    xb.copy_(xa)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        xb.copy_(xa)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * xa.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del xa, xb

    dense = None
    if not args.skip_dense:
        dprob = F.make_problem(H, N, d, wl.grid, B, wl.tile_hw, 1.0, wl.k_min, 0)
        dbuf = F.Buffers.allocate(dprob)
        dbuf.run(q, k, v)
        dbuf.run(q, k, v)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            dbuf.run(q, k, v)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / reps
        dense = {"ms_per_call": round(dense_ms, 4),
                 "tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 1),
                 "sparse_speedup": round(dense_ms / ms_per_step, 3)}
        lse_dense = dbuf.lse.clone()
        del dbuf

        # token order (FVAttn S3.1 / GSRS A.6): the frame/tile order against the
        # generalised Hilbert curve at the same p -- kept density, attention
        # recall (share of each query's dense softmax mass on its kept keys)
        # and time per call
        def order_stats(b, ms):
            rp = b.row_ptr.cpu().numpy().astype(np.int64)
            recall = torch.exp(b.lse - lse_dense).mean().item()
            return {"density": round(float(rp[-1]) / (H * nb * nb), 4), "recall": round(recall, 4),
                    "ms_per_call": round(ms, 4)}
        hprob = F.make_problem(H, N, d, wl.grid, B, wl.tile_hw, p, wl.k_min, wl.refill_per_mille,
                               order="hilbert")
        hbuf = F.Buffers.allocate(hprob)
        hbuf.run(q, k, v)
        hbuf.run(q, k, v)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            hbuf.run(q, k, v)
        e1.record(stream)
        torch.cuda.synchronize()
        order_cmp = {"tiles": order_stats(buf, ms_per_step),
                     "hilbert": order_stats(hbuf, e0.elapsed_time(e1) / reps)}
        dense["order_comparison"] = order_cmp
        del hbuf

    balance = None
    if not args.skip_balance:
        print("bench: eight-rank balance simulation", file=sys.stderr, flush=True)
        balance = balance_simulation(stream)

    gsrs = None
    if not args.skip_gsrs:
        print("bench: growing-sparsity trajectory", file=sys.stderr, flush=True)
        gsrs = gsrs_trajectory(stream)

    cpu = None
    if not args.skip_cpu_baseline:
        gpu_o = buf.o.float().cpu().numpy().astype(np.float64)
        cpu = cpu_baseline(wl, inp, p, gpu_o, row_ptr, col_idx, args.cpu_seconds,
                           all_tiles=wl.name == "rank480p")

    out = {
        "metric": METRIC,
        "value": round(ms_per_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": warm_run,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Q/K/V with a grid-locality term; no model weights)",
        "config": {"workload": wl.name, "heads": H, "seq_len": N, "grid": list(wl.grid),
                   "head_dim": d, "block": B, "tile": list(wl.tile_hw), "top_p": p,
                   "k_min": wl.k_min, "refill_per_mille": wl.refill_per_mille,
                   "parallelism": "1 GPU (one Ulysses rank's head share)"},
        "dense_equiv_tflops": round(dense_flops / (ms_per_step * 1e-3) / 1e12, 1),
        "kept_block_mfma_util": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
        "density": round(pairs / (H * nb * nb), 4),
        "head_density": [round(float(x) / (nb * nb), 4) for x in head_final],
        "ms": {"route": round(float(t_route.mean()), 4), "plan": round(float(t_plan.mean()), 4),
               "attn": round(attn_avg_ms, 4), "route_back_to_back": round(fused_ms, 4),
               "plan_back_to_back": round(plan_b2b_ms, 4), "step_median": round(float(np.median(t_step)), 4),
               "step_p10": round(float(np.percentile(t_step, 10)), 4),
               "step_p90": round(float(np.percentile(t_step, 90)), 4),
               "host_wall_per_step": round(wall / K * 1e3, 4),
               "note": "attn from the timed region; route, plan and step_* from a second pass of the "
                       "same steps with an event between every two phases (each event leaves the GPU idle "
                       "for a few us); *_back_to_back: calls of that phase alone, back to back"},
        "route_hbm": dict(hbm(route_bytes, route_b2b_ms),
                          what="routing alone: Q, K read; ranking, counts, order written"),
        "route_fused_hbm": dict(hbm(fused_bytes, fused_ms),
                                what="the step's routing pass: routing + scores exported + K/V "
                                     "re-laid out for the attention (V read, K and V written)"),
        "kv_layout_hbm": dict(hbm(kv_bytes, kv_ms),
                              what="K/V re-layout alone (fva_kv_layout): K, V read, written"),
        "roofline": {"bound": "mfma", "achieved": round(achieved_tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic() if wl.name == "rank480p" else None,
                     "kernel": "sparse_attn_fwd_kernel<128,128,64,2>",
                     "algorithmic_flops_per_launch": kept,
                     "timed": "attention call = attention kernel + merge of split tiles",
                     "sustained_mfma_tflops": ceiling,
                     "sustained_copy_gbs": round(copy_gbs, 1),
                     "frac_of_sustained": round(achieved_tflops / ceiling["random_operands"], 4)},
        "precise_importance": precise,
        "cu_imbalance": {"workgroups": workers, "split_tiles": int(meta[1]),
                         "planned": round(planned / ideal, 4), "lpt_whole_tiles": round(lpt / ideal, 4),
                         "natural": round(natural / ideal, 4), "compute_units": cus,
                         "per_compute_unit": per_cu, "measured": measured},
        "dense_reference": dense,
        "balance": balance,
        "gsrs": gsrs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
