"""Multi-step runner for growing sparsity with reduced search.

"Sparse Attention for Video Generation Acceleration via Growing Sparsity and
Reduced Search", S5.1 and A.5: dense warm-up steps, a first search over every
key block, later searches over the first search's mask only (the candidate
set), the latest mask reused between searches, a lower Top-p at each search.

This module only sequences library calls and keeps device buffers between
steps: fva_gsrs_action decides what a step does; fva_kv_layout (order, K/V
re-layout of the step's inputs), fva_schedule (work list of the all-blocks
mask), fva_plan, fva_sparse_attn_fwd (with per-block LSEs at a search),
fva_block_importance and fva_reselect do the work on the GPU.  No step runs
the pooled-score routing: every mask here comes from the precise importance
of a search, or is the all-blocks mask.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from .fva import (FVA_GSRS_CANDIDATE_SEARCH, FVA_GSRS_DENSE, FVA_GSRS_FULL_SEARCH,
                  FVA_GSRS_REUSE, Buffers, GsrsSchedule, Problem, block_importance,
                  gsrs_action, plan, reselect, schedule, sizes, sparse_attn_fwd)


@dataclass
class MaskPlan:
    """A materialised mask and its work list (fva_plan's outputs)."""

    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    head_count: torch.Tensor
    work_order: torch.Tensor
    plan_meta: torch.Tensor
    tile_counter: torch.Tensor

    @classmethod
    def allocate(cls, prob: Problem, device="cuda") -> "MaskPlan":
        sz = sizes(prob)
        i32 = dict(dtype=torch.int32, device=device)
        return cls(torch.empty(sz.num_rows + 1, **i32), torch.empty(sz.col_idx_capacity, **i32),
                   torch.empty(prob.num_heads, **i32), torch.empty(sz.work_order_elems, **i32),
                   torch.empty(sz.plan_meta_elems, **i32), torch.zeros(sz.tile_counter_elems, **i32))

    def copy_from(self, other: "MaskPlan") -> None:
        for name in ("row_ptr", "col_idx", "head_count", "work_order", "plan_meta", "tile_counter"):
            getattr(self, name).copy_(getattr(other, name))


class GsrsRunner:
    """Runs one attention call per denoising step under a GSRS schedule.

    step(t, q, k, v) enqueues the step's calls on the current stream and
    returns (action, p); the output is in .buf.o / .buf.lse, the mask the
    step's attention used in .evaluated, and the latest selected mask in
    .current.
    """

    def __init__(self, prob: Problem, schedule: GsrsSchedule, device="cuda"):
        self.prob = prob
        self.schedule = schedule
        self.buf = Buffers.allocate(prob, device)
        sz = sizes(prob)
        self.nb = sz.num_blocks
        H, nb = prob.num_heads, self.nb
        self.full = MaskPlan.allocate(prob, device)
        self.candidates = MaskPlan.allocate(prob, device)
        self.current = MaskPlan.allocate(prob, device)
        # the all-blocks mask: every row keeps 0 .. nb-1
        rows = sz.num_rows
        self.full.row_ptr.copy_(torch.arange(rows + 1, dtype=torch.int32, device=device) * nb)
        self.full.col_idx[: rows * nb].copy_(
            torch.arange(nb, dtype=torch.int32, device=device).repeat(rows))
        self.full.head_count.fill_(nb * nb)
        self.sel_ranked = torch.empty(sz.ranked_elems, dtype=torch.int16, device=device)
        self.sel_count = torch.empty(sz.num_rows, dtype=torch.int32, device=device)
        self.sel_head = torch.empty(H, dtype=torch.int32, device=device)
        self.block_lse = torch.empty(sz.block_lse_capacity, dtype=torch.float32, device=device)
        self.importance = torch.empty((H, nb, nb), dtype=torch.float32, device=device)
        self.evaluated = None
        self._have_full = False
        self._have_candidates = False

    def _plan(self, ranked, count, mp: MaskPlan, stream=None):
        plan(self.prob, ranked, count, mp.row_ptr, mp.col_idx, mp.head_count, mp.work_order,
             mp.plan_meta, mp.tile_counter, stream)

    def _attn(self, q, mp: MaskPlan, block_lse=None, stream=None):
        sparse_attn_fwd(self.prob, q, self.buf.kv, self.buf.order, mp.row_ptr, mp.col_idx,
                        mp.work_order, mp.plan_meta, mp.tile_counter, self.buf.o,
                        self.buf.attn_workspace, self.buf.lse, block_lse, stream)

    def step(self, t: int, q, k, v, stream=None):
        action, p = gsrs_action(self.schedule, t)
        self.buf.kv_layout(k, v, stream)  # order and K/V re-layout of this step's inputs
        if not self._have_full:
            mp = self.full
            schedule(self.prob, mp.row_ptr, mp.work_order, mp.plan_meta, mp.tile_counter, stream)
            self._have_full = True
        if action == FVA_GSRS_DENSE:
            self._attn(q, self.full, stream=stream)
            self.evaluated = self.full
        elif action in (FVA_GSRS_FULL_SEARCH, FVA_GSRS_CANDIDATE_SEARCH):
            if action == FVA_GSRS_CANDIDATE_SEARCH and not self._have_candidates:
                raise RuntimeError("a candidate-set search needs an earlier full-space search")
            ev = self.full if action == FVA_GSRS_FULL_SEARCH else self.candidates
            self._attn(q, ev, self.block_lse, stream)
            block_importance(self.prob, self.buf.order, ev.row_ptr, ev.col_idx, self.buf.lse,
                             self.block_lse, self.importance, stream)
            sp = Problem.from_buffer_copy(self.prob)
            sp.top_p = ctypes.c_float(p).value
            reselect(sp, ev.row_ptr, ev.col_idx, self.importance, self.sel_ranked, self.sel_count,
                     self.sel_head, stream)
            self._plan(self.sel_ranked, self.sel_count, self.current, stream)
            if action == FVA_GSRS_FULL_SEARCH and not self._have_candidates:
                with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
                    self.candidates.copy_from(self.current)
                self._have_candidates = True
            self.evaluated = ev
        elif action == FVA_GSRS_REUSE:
            self._attn(q, self.current, stream=stream)
            self.evaluated = self.current
        else:
            raise RuntimeError(f"unknown action {action}")
        return action, p
