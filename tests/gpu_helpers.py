"""Helpers for the GPU parity tests: run the HIP chain through the C ABI and
bring every output back as NumPy arrays for comparison with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import adaptive_block_sparse_fva_amd as F
from synth import bf16_bits_to_f64

# Acceptance bar for attention outputs against the fp64 masked softmax.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
# Block scores are fp32 on the GPU and fp64 in the oracle.
S_REL = 1e-4


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def problem_for(wl, top_p, refill=None, tile=None, **kw):
    return F.make_problem(wl.num_heads, wl.seq_len, wl.head_dim, wl.grid, wl.block,
                          wl.tile_hw if tile is None else tile, top_p, wl.k_min,
                          wl.refill_per_mille if refill is None else refill, **kw)


def to_device(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def device_inputs(inp):
    return to_device(inp.q), to_device(inp.k), to_device(inp.v)


def run_chain(prob, q, k, v, work_order=None, with_lse=True):
    """route -> plan -> attention on the current stream; returns (Buffers, host dict)."""
    buf = F.Buffers.allocate(prob)
    buf.route(q, k, v)
    buf.plan()
    if work_order is not None:
        buf.attn(q, work_order=work_order, with_lse=with_lse)
    else:
        buf.attn(q, with_lse=with_lse)
    torch.cuda.synchronize()
    return buf, host(buf)


def host(buf) -> dict:
    H, nb = buf.prob.num_heads, buf.nb
    rows = H * nb
    row_ptr = buf.row_ptr.cpu().numpy().astype(np.int64)
    meta = buf.plan_meta.cpu().numpy().astype(np.int64)
    return {
        "nb": nb,
        "order": buf.order.cpu().numpy().astype(np.int64),
        "scores": buf.scores.cpu().numpy().reshape(H, nb, nb),
        "ranked": buf.ranked.cpu().numpy().astype(np.int64).reshape(rows, nb),
        "row_count": buf.row_count.cpu().numpy().astype(np.int64),
        "head_count": buf.head_count.cpu().numpy().astype(np.int64),
        "row_ptr": row_ptr,
        "col_idx": buf.col_idx[: int(row_ptr[-1])].cpu().numpy().astype(np.int64),
        "head_count_final": buf.head_count_final.cpu().numpy().astype(np.int64),
        "plan_meta": meta,
        "work_order": buf.work_order[: int(meta[0])].cpu().numpy().astype(np.int64),
        "tile_counter": buf.tile_counter.cpu().numpy(),
        "o": buf.o.float().cpu().numpy().astype(np.float64),
        "lse": buf.lse.cpu().numpy().astype(np.float64),
    }


def f64_inputs(inp):
    return bf16_bits_to_f64(inp.q), bf16_bits_to_f64(inp.k), bf16_bits_to_f64(inp.v)


def sample_tiles(row_ptr, num_heads, nb, per_head, seed=0):
    """Seeded tile sample: per head the heaviest and lightest rows plus random ones."""
    rng = np.random.default_rng(seed)
    kept = np.diff(row_ptr)
    out = []
    for h in range(num_heads):
        rows = np.arange(h * nb, (h + 1) * nb)
        k = kept[rows]
        pick = {int(rows[np.argmax(k)]), int(rows[np.argmin(k)]), int(rows[-1])}
        extra = rng.choice(rows, size=min(per_head, nb), replace=False)
        pick.update(int(x) for x in extra)
        out.extend(sorted(pick))
    return np.array(out, dtype=np.int64)


def tile_rows(order, block, n_tokens, tiles, nb):
    """Natural token indices of the query rows of the given tiles, per head."""
    per_head = {}
    for t in tiles:
        h, i = divmod(int(t), nb)
        toks = order[i * block: min(n_tokens, (i + 1) * block)]
        per_head.setdefault(h, []).append(toks)
    return {h: np.concatenate(v) for h, v in per_head.items()}
