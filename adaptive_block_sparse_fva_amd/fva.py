"""ctypes binding of libfva.so: the C ABI in include/fva.h, argument marshalling only.

Every step of the routing, plan and attention runs in the library's HIP
kernels; this module only turns torch tensors into device pointers and the
current HIP stream into a handle, and raises on a non-zero status.  It refuses
to run (FvaError) when the library has not been built.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libfva.so")

FVA_OK = 0
FVA_ERR_ARG = 1
FVA_ERR_UNSUPPORTED = 2
FVA_ERR_HIP = 3
FVA_ERR_WORKSPACE = 4
FVA_MAX_BLOCKS = 2048
FVA_MAX_TILES = 16384
FVA_MAX_SPLITS = 1024
FVA_ORDER_TILES = 0
FVA_ORDER_HILBERT = 1
FVA_MAX_HEAD_REFILL = 1000 * (FVA_MAX_BLOCKS - 1)
FVA_RLB_PAIRS = 0
FVA_RLB_RING = 1
FVA_BALANCE_NONE = 0
FVA_BALANCE_SASA = 1
FVA_BALANCE_RLB_SASA = 2
FVA_RLB_MAX_PAIR_RANKS = 12
FVA_RLB_MAX_RANKS = 64
FVA_RLB_MAX_HEADS = 64
FVA_RLB_MAX_HEAD_LOAD = 1 << 22
FVA_GSRS_MAX_SEARCHES = 16
FVA_GSRS_DENSE = 0
FVA_GSRS_FULL_SEARCH = 1
FVA_GSRS_CANDIDATE_SEARCH = 2
FVA_GSRS_REUSE = 3
FVA_TRACE_FIELDS = 6
FVA_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTED = (
    "fva_sizes",
    "fva_attn_workgroups",
    "fva_compute_units",
    "fva_route",
    "fva_route_noalloc",
    "fva_kv_layout",
    "fva_plan",
    "fva_schedule",
    "fva_sparse_attn_fwd",
    "fva_sparse_attn_fwd_traced",
    "fva_block_importance",
    "fva_mfma_probe",
    "fva_balance",
    "fva_sasa_refill",
    "fva_reselect",
    "fva_gsrs_action",
    "fva_status_string",
    "fva_last_error",
    "fva_version",
)


class FvaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: status {status}" + (f" ({detail})" if detail else ""))


class Problem(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("grid_t", ctypes.c_int32),
        ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("tile_h", ctypes.c_int32),
        ("tile_w", ctypes.c_int32),
        ("top_p", ctypes.c_float),
        ("k_min", ctypes.c_int32),
        ("refill_per_mille", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("stride_head", ctypes.c_int64),
        ("stride_token", ctypes.c_int64),
        ("order_kind", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class Sizes(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("num_rows", ctypes.c_int32),
        ("order_elems", ctypes.c_int64),
        ("scores_elems", ctypes.c_int64),
        ("ranked_elems", ctypes.c_int64),
        ("col_idx_capacity", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("tile_counter_elems", ctypes.c_int32),
        ("kv_elems", ctypes.c_int64),
        ("work_order_elems", ctypes.c_int64),
        ("plan_meta_elems", ctypes.c_int64),
        ("attn_workspace_bytes", ctypes.c_int64),
        ("block_lse_capacity", ctypes.c_int64),
    ]


class BalanceParams(ctypes.Structure):
    _fields_ = [
        ("num_ranks", ctypes.c_int32),
        ("heads_per_rank", ctypes.c_int32),
        ("topology", ctypes.c_int32),
        ("k1_per_mille", ctypes.c_int32),
        ("k2_per_mille", ctypes.c_int32),
        ("n1_per_mille", ctypes.c_int32),
        ("n2_per_mille", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class BalanceInfo(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("moves", ctypes.c_int32),
        ("rho_per_mille", ctypes.c_int32),
        ("rho_new_per_mille", ctypes.c_int32),
        ("load_total", ctypes.c_int64),
        ("load_max", ctypes.c_int64),
        ("load_new_max", ctypes.c_int64),
        ("load_aug_max", ctypes.c_int64),
    ]


class GsrsSchedule(ctypes.Structure):
    _fields_ = [
        ("num_steps", ctypes.c_int32),
        ("warmup_steps", ctypes.c_int32),
        ("num_searches", ctypes.c_int32),
        ("reduced", ctypes.c_int32),
        ("search_step", ctypes.c_int32 * FVA_GSRS_MAX_SEARCHES),
        ("top_p", ctypes.c_float * FVA_GSRS_MAX_SEARCHES),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfva.so (once).  Raises FvaError if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FvaError(-1, "load_library",
                       f"{path} not built; run `python -m adaptive_block_sparse_fva_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Problem)
    vp = ctypes.c_void_p
    lib.fva_sizes.argtypes = [P, ctypes.POINTER(Sizes)]
    lib.fva_attn_workgroups.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    lib.fva_compute_units.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    lib.fva_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fva_route_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fva_kv_layout.argtypes = [P, vp, vp, vp, vp, vp]
    lib.fva_plan.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fva_schedule.argtypes = [P, vp, vp, vp, vp, vp]
    lib.fva_sparse_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        ctypes.c_size_t, vp]
    lib.fva_sparse_attn_fwd_traced.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               ctypes.c_size_t, vp, vp]
    lib.fva_block_importance.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.fva_mfma_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_int64,
                                   ctypes.POINTER(ctypes.c_double), vp]
    BP = ctypes.POINTER(BalanceParams)
    lib.fva_balance.argtypes = [BP, vp, vp, vp, vp, vp, vp, ctypes.POINTER(BalanceInfo)]
    lib.fva_sasa_refill.argtypes = [BP, ctypes.c_int32, vp, vp, vp, vp, vp]
    lib.fva_reselect.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.fva_gsrs_action.argtypes = [ctypes.POINTER(GsrsSchedule), ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float)]
    lib.fva_status_string.argtypes = [ctypes.c_int]
    lib.fva_status_string.restype = ctypes.c_char_p
    lib.fva_last_error.argtypes = []
    lib.fva_last_error.restype = ctypes.c_char_p
    lib.fva_version.argtypes = []
    for name in ("fva_sizes", "fva_attn_workgroups", "fva_compute_units", "fva_route",
                 "fva_route_noalloc", "fva_kv_layout", "fva_plan", "fva_schedule", "fva_sparse_attn_fwd",
                 "fva_sparse_attn_fwd_traced", "fva_block_importance", "fva_mfma_probe",
                 "fva_balance", "fva_sasa_refill", "fva_reselect", "fva_gsrs_action", "fva_version"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != FVA_OK:
        lib = load_library()
        detail = lib.fva_status_string(status).decode()
        if status == FVA_ERR_HIP:
            detail += ": " + lib.fva_last_error().decode()
        raise FvaError(status, where, detail)


def make_problem(num_heads: int, seq_len: int, head_dim: int, grid: Sequence[int], block: int,
                 tile: Sequence[int], top_p: float, k_min: int, refill_per_mille: int = 0,
                 sm_scale: float = 0.0, stride_head: Optional[int] = None,
                 stride_token: Optional[int] = None, order: str = "tiles") -> Problem:
    """Problem struct; default strides describe contiguous [H][N][d] tensors;
    order is "tiles" (frame-major spatial tiles) or "hilbert"."""
    if stride_token is None:
        stride_token = head_dim
    if stride_head is None:
        stride_head = seq_len * stride_token
    kinds = {"tiles": FVA_ORDER_TILES, "hilbert": FVA_ORDER_HILBERT}
    if order not in kinds:
        raise FvaError(FVA_ERR_ARG, "make_problem", f"unknown order {order!r}")
    return Problem(num_heads, seq_len, head_dim, grid[0], grid[1], grid[2], block, tile[0],
                   tile[1], float(top_p), k_min, refill_per_mille, float(sm_scale), stride_head,
                   stride_token, kinds[order], 0)


def sizes(prob: Problem) -> Sizes:
    out = Sizes()
    _check(load_library().fva_sizes(ctypes.byref(prob), ctypes.byref(out)), "fva_sizes")
    return out


def attn_workgroups(prob: Problem) -> int:
    out = ctypes.c_int32(0)
    _check(load_library().fva_attn_workgroups(ctypes.byref(prob), ctypes.byref(out)),
           "fva_attn_workgroups")
    return int(out.value)


def compute_units() -> int:
    """Compute units of the current device (the count the plan's split rule uses)."""
    out = ctypes.c_int32(0)
    _check(load_library().fva_compute_units(ctypes.byref(out)), "fva_compute_units")
    return int(out.value)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise FvaError(FVA_ERR_ARG, "binding", "tensors must live on the GPU")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def route(prob, q, k, v, scores, ranked, row_count, head_count, order, kv, workspace,
          stream=None):
    """fva_route; v and kv may both be None (routing only), scores may be None."""
    st = load_library().fva_route(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(scores),
                                  _ptr(ranked), _ptr(row_count), _ptr(head_count), _ptr(order),
                                  _ptr(kv), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "fva_route")


def route_noalloc(prob, q, k, v, scores, ranked, row_count, head_count, order, kv, stream=None):
    """fva_route_noalloc: fva_route with the workspace in the library's own static
    device array (no allocation); v and kv may both be None, scores may be None."""
    st = load_library().fva_route_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(scores), _ptr(ranked), _ptr(row_count),
                                          _ptr(head_count), _ptr(order), _ptr(kv), _stream(stream))
    _check(st, "fva_route_noalloc")


def kv_layout(prob, k, v, order, kv, stream=None):
    """fva_kv_layout: the caller's K and V in the attention's layout (and the order table)."""
    st = load_library().fva_kv_layout(ctypes.byref(prob), _ptr(k), _ptr(v), _ptr(order), _ptr(kv),
                                      _stream(stream))
    _check(st, "fva_kv_layout")


def schedule(prob, row_ptr, work_order, plan_meta, tile_counter, stream=None):
    """fva_schedule: the heaviest-first work list of a given CSR mask."""
    st = load_library().fva_schedule(ctypes.byref(prob), _ptr(row_ptr), _ptr(work_order),
                                     _ptr(plan_meta), _ptr(tile_counter), _stream(stream))
    _check(st, "fva_schedule")


def plan(prob, ranked, row_count, row_ptr, col_idx, head_count_final, work_order, plan_meta,
         tile_counter, stream=None, head_refill=None):
    """head_refill: optional device int32 [H], a refill per mille per head."""
    st = load_library().fva_plan(ctypes.byref(prob), _ptr(ranked), _ptr(row_count),
                                 _ptr(head_refill), _ptr(row_ptr), _ptr(col_idx),
                                 _ptr(head_count_final), _ptr(work_order), _ptr(plan_meta),
                                 _ptr(tile_counter), _stream(stream))
    _check(st, "fva_plan")


def sparse_attn_fwd(prob, q, kv, order, row_ptr, col_idx, work_order, plan_meta, tile_counter, o,
                    workspace, lse=None, block_lse=None, stream=None, item_trace=None):
    """fva_sparse_attn_fwd, or fva_sparse_attn_fwd_traced when item_trace (device int64
    [work items][FVA_TRACE_FIELDS]) is given."""
    lib = load_library()
    args = [ctypes.byref(prob), _ptr(q), _ptr(kv), _ptr(order), _ptr(row_ptr), _ptr(col_idx),
            _ptr(work_order), _ptr(plan_meta), _ptr(tile_counter), _ptr(o), _ptr(lse),
            _ptr(block_lse), _ptr(workspace), workspace.numel() * workspace.element_size()]
    if item_trace is None:
        _check(lib.fva_sparse_attn_fwd(*args, _stream(stream)), "fva_sparse_attn_fwd")
    else:
        _check(lib.fva_sparse_attn_fwd_traced(*args, _ptr(item_trace), _stream(stream)),
               "fva_sparse_attn_fwd_traced")


def block_importance(prob, order, row_ptr, col_idx, lse, block_lse, importance, stream=None):
    st = load_library().fva_block_importance(ctypes.byref(prob), _ptr(order), _ptr(row_ptr),
                                             _ptr(col_idx), _ptr(lse), _ptr(block_lse),
                                             _ptr(importance), _stream(stream))
    _check(st, "fva_block_importance")


def mfma_probe(iters: int, random_operands: bool, sink: torch.Tensor, stream=None) -> float:
    """Enqueue the MFMA-rate diagnostic kernel; returns the FLOPs it performs."""
    flops = ctypes.c_double(0.0)
    st = load_library().fva_mfma_probe(int(iters), 1 if random_operands else 0, _ptr(sink),
                                       sink.numel(), ctypes.byref(flops), _stream(stream))
    _check(st, "fva_mfma_probe")
    return float(flops.value)


def balance_params(num_ranks: int, heads_per_rank: int, topology: str = "pairs",
                   k1_per_mille: int = 1050, k2_per_mille: int = 1100, n1_per_mille: int = 800,
                   n2_per_mille: int = 70) -> BalanceParams:
    """Parameters of the cross-rank balance step; defaults are the paper's."""
    kinds = {"pairs": FVA_RLB_PAIRS, "ring": FVA_RLB_RING}
    if topology not in kinds:
        raise FvaError(FVA_ERR_ARG, "balance_params", f"unknown topology {topology!r}")
    return BalanceParams(num_ranks, heads_per_rank, kinds[topology], k1_per_mille, k2_per_mille,
                         n1_per_mille, n2_per_mille, 0)


def _host(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _hp(a: np.ndarray) -> int:
    return a.ctypes.data


def balance(prm: BalanceParams, head_load) -> Dict[str, object]:
    """fva_balance on host arrays: head_load [R][Hl] -> the plan and budgets."""
    R = prm.num_ranks
    w = _host(head_load, np.int32)
    if w.size != R * prm.heads_per_rank:
        raise FvaError(FVA_ERR_ARG, "balance", "head_load must hold num_ranks * heads_per_rank values")
    sigma = np.empty(R, np.int32)
    send = np.empty(R, np.int32)
    load_new = np.empty(R, np.int64)
    slack = np.empty(R, np.int64)
    budget = np.empty(R, np.int64)
    info = BalanceInfo()
    st = load_library().fva_balance(ctypes.byref(prm), _hp(w), _hp(sigma), _hp(send), _hp(load_new),
                                    _hp(slack), _hp(budget), ctypes.byref(info))
    _check(st, "fva_balance")
    out = {name: getattr(info, name) for name, _ in BalanceInfo._fields_}
    out.update(sigma=sigma, send=send, loads_new=load_new, slack=slack, budget=budget)
    return out


def sasa_refill(prm: BalanceParams, nb: int, row_count, send_head, budget):
    """fva_sasa_refill on host arrays -> (head_refill int32 [R*Hl], added int64 [R])."""
    R, Hl = prm.num_ranks, prm.heads_per_rank
    rc = _host(row_count, np.int32)
    send = _host(send_head, np.int32)
    bud = _host(budget, np.int64)
    if rc.size != R * Hl * nb or send.size != R or bud.size != R:
        raise FvaError(FVA_ERR_ARG, "sasa_refill", "array sizes do not match the parameters")
    refill = np.empty(R * Hl, np.int32)
    added = np.empty(R, np.int64)
    st = load_library().fva_sasa_refill(ctypes.byref(prm), int(nb), _hp(rc), _hp(send), _hp(bud),
                                        _hp(refill), _hp(added))
    _check(st, "fva_sasa_refill")
    return refill, added


def reselect(prob, row_ptr, col_idx, importance, ranked, row_count, head_count, stream=None):
    """fva_reselect: re-selection with prob.top_p / prob.k_min inside the
    evaluated mask (row_ptr, col_idx) from its precise importance."""
    st = load_library().fva_reselect(ctypes.byref(prob), _ptr(row_ptr), _ptr(col_idx),
                                     _ptr(importance), _ptr(ranked), _ptr(row_count),
                                     _ptr(head_count), _stream(stream))
    _check(st, "fva_reselect")


def gsrs_schedule(num_steps: int, warmup_steps: int, search_steps: Sequence[int],
                  top_ps: Sequence[float], reduced: bool = True) -> GsrsSchedule:
    if len(search_steps) != len(top_ps) or len(search_steps) > FVA_GSRS_MAX_SEARCHES:
        raise FvaError(FVA_ERR_ARG, "gsrs_schedule", "one p per search, at most 16 searches")
    s = GsrsSchedule()
    s.num_steps, s.warmup_steps = num_steps, warmup_steps
    s.num_searches, s.reduced = len(search_steps), 1 if reduced else 0
    for j, (t, p) in enumerate(zip(search_steps, top_ps)):
        s.search_step[j] = int(t)
        s.top_p[j] = float(p)
    return s


def gsrs_action(schedule: GsrsSchedule, step: int):
    """fva_gsrs_action -> (action, p)."""
    act = ctypes.c_int32(0)
    p = ctypes.c_float(0.0)
    st = load_library().fva_gsrs_action(ctypes.byref(schedule), int(step), ctypes.byref(act),
                                        ctypes.byref(p))
    _check(st, "fva_gsrs_action")
    return int(act.value), float(p.value)


@dataclass
class Buffers:
    """Every device buffer one call of the hot path needs, allocated with torch."""

    prob: Problem
    nb: int
    scores: torch.Tensor
    ranked: torch.Tensor
    row_count: torch.Tensor
    head_count: torch.Tensor
    order: torch.Tensor
    workspace: torch.Tensor
    kv: torch.Tensor
    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    head_count_final: torch.Tensor
    work_order: torch.Tensor
    plan_meta: torch.Tensor
    tile_counter: torch.Tensor
    attn_workspace: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor

    @classmethod
    def allocate(cls, prob: Problem, device="cuda") -> "Buffers":
        sz = sizes(prob)
        H, N, d = prob.num_heads, prob.seq_len, prob.head_dim
        i32 = dict(dtype=torch.int32, device=device)
        return cls(
            prob=prob,
            nb=sz.num_blocks,
            scores=torch.empty(sz.scores_elems, dtype=torch.float32, device=device),
            ranked=torch.empty(sz.ranked_elems, dtype=torch.int16, device=device),
            row_count=torch.empty(sz.num_rows, **i32),
            head_count=torch.empty(H, **i32),
            order=torch.empty(sz.order_elems, **i32),
            workspace=torch.empty(max(16, sz.workspace_bytes) // 4, dtype=torch.float32,
                                  device=device),
            kv=torch.empty(sz.kv_elems, dtype=torch.bfloat16, device=device),
            row_ptr=torch.empty(sz.num_rows + 1, **i32),
            col_idx=torch.empty(sz.col_idx_capacity, **i32),
            head_count_final=torch.empty(H, **i32),
            work_order=torch.empty(sz.work_order_elems, **i32),
            plan_meta=torch.empty(sz.plan_meta_elems, **i32),
            tile_counter=torch.zeros(sz.tile_counter_elems, **i32),
            attn_workspace=torch.empty(max(16, sz.attn_workspace_bytes) // 4, dtype=torch.float32,
                                       device=device),
            # o follows the problem's strides, as q does (the kernels write it so)
            o=torch.empty_strided((H, N, d), (prob.stride_head, prob.stride_token, 1),
                                  dtype=torch.bfloat16, device=device),
            lse=torch.empty((H, N), dtype=torch.float32, device=device),
        )

    def route(self, q, k, v=None, stream=None, with_scores=True):
        """Routing; with v also the K/V re-layout into .kv (in the same pass).
        with_scores=False leaves the scores inside the workspace."""
        route(self.prob, q, k, v, self.scores if with_scores else None, self.ranked,
              self.row_count, self.head_count, self.order, None if v is None else self.kv,
              self.workspace, stream)

    def kv_layout(self, k, v, stream=None):
        """K and V into .kv (and the order table into .order) without routing."""
        kv_layout(self.prob, k, v, self.order, self.kv, stream)

    def schedule(self, stream=None):
        """Work list of the mask currently in .row_ptr (e.g. one written by the caller)."""
        schedule(self.prob, self.row_ptr, self.work_order, self.plan_meta, self.tile_counter,
                 stream)

    def plan(self, stream=None, head_refill=None):
        plan(self.prob, self.ranked, self.row_count, self.row_ptr, self.col_idx,
             self.head_count_final, self.work_order, self.plan_meta, self.tile_counter, stream,
             head_refill)

    def attn(self, q, work_order=None, with_lse=True, block_lse=None, stream=None,
             item_trace=None):
        """Attention over the K/V in .kv (from route(q, k, v) or kv_layout()),
        the work items taken in the plan's order (or in work_order's);
        block_lse (float, >= row_ptr[-1] * B elements) also records per-block
        LSEs; item_trace (int64 [items][FVA_TRACE_FIELDS]) records per-item
        clocks."""
        sparse_attn_fwd(self.prob, q, self.kv, self.order, self.row_ptr, self.col_idx,
                        self.work_order if work_order is None else work_order, self.plan_meta,
                        self.tile_counter, self.o, self.attn_workspace,
                        self.lse if with_lse else None, block_lse, stream, item_trace)

    def importance(self, block_lse, out=None, stream=None):
        """Precise block importance [H][nb][nb] from the last attn(block_lse=...)."""
        H = self.prob.num_heads
        if out is None:
            out = torch.empty((H, self.nb, self.nb), dtype=torch.float32, device=self.lse.device)
        block_importance(self.prob, self.order, self.row_ptr, self.col_idx, self.lse, block_lse, out,
                         stream)
        return out

    def run(self, q, k, v, stream=None):
        """One full call of the hot path: route -> plan -> attention."""
        self.route(q, k, v, stream)
        self.plan(stream)
        self.attn(q, stream=stream)
        return self.o


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
