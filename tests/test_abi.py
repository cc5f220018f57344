"""CPU-only checks of the C ABI: the library loads, exports every declared
symbol, reports sizes and rejects bad arguments before touching a device."""

import ctypes
import os
import re

import pytest

import adaptive_block_sparse_fva_amd as F
from adaptive_block_sparse_fva_amd import fva

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fva.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fva_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_surface():
    assert _declared_functions() == sorted(fva.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = F.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.fva_version() >= 100


def test_struct_layout_matches_header(tmp_path):
    """ctypes mirrors of fva_problem / fva_sizes_t agree with the C compiler."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields_p = [f[0] for f in fva.Problem._fields_]
    fields_s = [f[0] for f in fva.Sizes._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "fva.h"', "int main(void){",
            'printf("%zu %zu\\n", sizeof(fva_problem), sizeof(fva_sizes_t));']
    prog += [f'printf("%zu\\n", offsetof(fva_problem, {f}));' for f in fields_p]
    prog += [f'printf("%zu\\n", offsetof(fva_sizes_t, {f}));' for f in fields_s]
    prog += ["return 0;}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    vals = [int(x) for x in out]
    assert vals[0] == ctypes.sizeof(fva.Problem) and vals[1] == ctypes.sizeof(fva.Sizes)
    assert vals[2:2 + len(fields_p)] == [getattr(fva.Problem, f).offset for f in fields_p]
    assert vals[2 + len(fields_p):] == [getattr(fva.Sizes, f).offset for f in fields_s]


def _ok_problem(**kw):
    args = dict(num_heads=5, seq_len=32760, head_dim=128, grid=(21, 30, 52), block=128,
                tile=(8, 16), top_p=0.95, k_min=8)
    args.update(kw)
    return F.make_problem(**args)


def test_sizes_of_the_480p_share():
    s = F.sizes(_ok_problem())
    assert s.num_blocks == 256 and s.num_rows == 1280
    assert s.order_elems == 256 * 128
    assert s.scores_elems == 5 * 256 * 256 == s.ranked_elems == s.col_idx_capacity
    # pooled means, then room for the scores when the caller passes none
    assert s.workspace_bytes == 2 * 5 * 256 * 128 * 4 + 5 * 256 * 256 * 4
    assert s.tile_counter_elems == 2


@pytest.mark.parametrize("bad,status", [
    (dict(seq_len=32761), fva.FVA_ERR_ARG),             # N != T*H*W
    (dict(num_heads=0), fva.FVA_ERR_ARG),
    (dict(top_p=float("nan")), fva.FVA_ERR_ARG),
    (dict(k_min=0), fva.FVA_ERR_ARG),
    (dict(refill_per_mille=1001), fva.FVA_ERR_ARG),
    (dict(refill_per_mille=-1), fva.FVA_ERR_ARG),
    (dict(tile=(8, 0)), fva.FVA_ERR_ARG),
    (dict(tile=(-8, 16)), fva.FVA_ERR_ARG),
    (dict(sm_scale=-1.0), fva.FVA_ERR_ARG),
    (dict(sm_scale=float("inf")), fva.FVA_ERR_ARG),
    (dict(stride_token=100), fva.FVA_ERR_ARG),          # < d
    (dict(stride_token=132), fva.FVA_ERR_ARG),          # not a multiple of 8
    (dict(head_dim=96), fva.FVA_ERR_UNSUPPORTED),
    (dict(block=32), fva.FVA_ERR_UNSUPPORTED),
    (dict(grid=(1, 1, 300000), seq_len=300000), fva.FVA_ERR_UNSUPPORTED),  # nb > 2048
    (dict(num_heads=70), fva.FVA_ERR_UNSUPPORTED),      # H*nb > 16384
])
def test_sizes_rejects_bad_problems(bad, status):
    with pytest.raises(F.FvaError) as ei:
        F.sizes(_ok_problem(**bad))
    assert ei.value.status == status


def test_edge_problems_are_accepted():
    # a single short block, raster order, p outside (0, 1), the largest k_min
    for kw in (dict(seq_len=35, grid=(1, 5, 7), block=64, tile=(8, 8)),
               dict(tile=(0, 0)),
               dict(top_p=1.5), dict(top_p=-3.0), dict(k_min=100000), dict(refill_per_mille=1000),
               dict(head_dim=64, block=64, stride_token=64)):
        F.sizes(_ok_problem(**kw))


def test_entry_points_reject_null_pointers_without_a_device():
    lib = F.load_library()
    p = _ok_problem()
    null = None
    st = lib.fva_route(ctypes.byref(p), *([null] * 10), 0, null)
    assert st == fva.FVA_ERR_ARG
    st = lib.fva_plan(ctypes.byref(p), *([null] * 10))
    assert st == fva.FVA_ERR_ARG
    st = lib.fva_sparse_attn_fwd(ctypes.byref(p), *([null] * 12), 0, null)
    assert st == fva.FVA_ERR_ARG
    st = lib.fva_sparse_attn_fwd_traced(ctypes.byref(p), *([null] * 12), 0, null, null)
    assert st == fva.FVA_ERR_ARG
    st = lib.fva_kv_layout(ctypes.byref(p), *([null] * 5))
    assert st == fva.FVA_ERR_ARG
    st = lib.fva_schedule(ctypes.byref(p), *([null] * 5))
    assert st == fva.FVA_ERR_ARG
    st = lib.fva_block_importance(ctypes.byref(p), *([null] * 7))
    assert st == fva.FVA_ERR_ARG
    assert lib.fva_sizes(None, None) == fva.FVA_ERR_ARG
    assert lib.fva_status_string(fva.FVA_ERR_WORKSPACE) == b"workspace too small"


def test_compute_units_checks_its_argument_and_needs_a_device():
    import torch
    lib = F.load_library()
    assert lib.fva_compute_units(None) == fva.FVA_ERR_ARG
    out = ctypes.c_int32(-1)
    st = lib.fva_compute_units(ctypes.byref(out))
    if torch.cuda.is_available():
        assert st == fva.FVA_OK and out.value > 0
    else:
        assert st == fva.FVA_ERR_HIP and out.value == -1


def test_route_rejects_small_workspace_before_launch():
    lib = F.load_library()
    p = _ok_problem()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: the check fails first
    st = lib.fva_route(ctypes.byref(p), *([fake] * 10), 16, None)
    assert st == fva.FVA_ERR_WORKSPACE
    mis = ctypes.c_void_p((1 << 20) + 2)
    st = lib.fva_route(ctypes.byref(p), mis, *([fake] * 9), 1 << 30, None)
    assert st == fva.FVA_ERR_ARG
    # the re-laid-out K/V buffer must be 16-byte aligned too
    st = lib.fva_route(ctypes.byref(p), *([fake] * 8), ctypes.c_void_p((1 << 20) + 8), fake,
                       1 << 30, None)
    assert st == fva.FVA_ERR_ARG


def test_route_optional_outputs():
    """v and kv come together (routing only without them); scores may be NULL.
    Checked on the host: each call below fails on the workspace size, which
    is tested after the pointers."""
    lib = F.load_library()
    p = _ok_problem()
    fake = ctypes.c_void_p(1 << 20)

    def call(v=fake, scores=fake, kv=fake):
        # q k v scores ranked row_count head_count order kv workspace bytes stream
        return lib.fva_route(ctypes.byref(p), fake, fake, v, scores, fake, fake, fake, fake, kv, fake,
                             16, None)

    assert call() == fva.FVA_ERR_WORKSPACE
    assert call(v=None, kv=None) == fva.FVA_ERR_WORKSPACE
    assert call(scores=None) == fva.FVA_ERR_WORKSPACE
    assert call(v=None, kv=None, scores=None) == fva.FVA_ERR_WORKSPACE
    assert call(v=None) == fva.FVA_ERR_ARG
    assert call(kv=None) == fva.FVA_ERR_ARG


def test_kv_layout_and_schedule_argument_checks():
    lib = F.load_library()
    p = _ok_problem()
    fake = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 8)
    assert lib.fva_kv_layout(ctypes.byref(p), mis, fake, fake, fake, None) == fva.FVA_ERR_ARG
    assert lib.fva_kv_layout(ctypes.byref(p), fake, fake, fake, mis, None) == fva.FVA_ERR_ARG
    assert lib.fva_kv_layout(ctypes.byref(p), fake, fake, None, fake, None) == fva.FVA_ERR_ARG
    bad = _ok_problem(k_min=0)
    assert lib.fva_kv_layout(ctypes.byref(bad), fake, fake, fake, fake, None) == fva.FVA_ERR_ARG
    assert lib.fva_schedule(ctypes.byref(bad), fake, fake, fake, fake, None) == fva.FVA_ERR_ARG
    assert lib.fva_schedule(ctypes.byref(p), fake, None, fake, fake, None) == fva.FVA_ERR_ARG


def test_sizes_of_kv_plan_and_attention_buffers():
    p = _ok_problem()
    sz = F.sizes(p)
    rows = p.num_heads * sz.num_blocks
    assert sz.kv_elems == 2 * p.num_heads * sz.num_blocks * p.block * p.head_dim
    splits = min(rows, fva.FVA_MAX_SPLITS)
    assert sz.work_order_elems == rows + splits
    assert sz.plan_meta_elems == 2 + rows + fva.FVA_MAX_SPLITS
    assert sz.attn_workspace_bytes == splits * 2 * (p.block * p.head_dim + 2 * p.block) * 4
    small = F.sizes(_ok_problem(num_heads=1, seq_len=1024, head_dim=64, grid=(4, 16, 16), block=64,
                                tile=(8, 8)))
    assert small.work_order_elems == 32 and small.attn_workspace_bytes == 16 * 2 * (64 * 64 + 128) * 4


def test_attention_argument_checks_before_launch():
    lib = F.load_library()
    p = _ok_problem()
    need = F.sizes(p).attn_workspace_bytes
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: the checks fail first
    mis = ctypes.c_void_p((1 << 20) + 8)

    def call(kv=fake, ws=fake, nbytes=need):
        # q kv order row_ptr col_idx work_order plan_meta tile_counter o lse block_lse workspace
        # bytes stream
        return lib.fva_sparse_attn_fwd(ctypes.byref(p), fake, kv, *([fake] * 6), fake, None, None, ws,
                                       nbytes, None)

    assert call(kv=mis) == fva.FVA_ERR_ARG
    assert call(kv=None) == fva.FVA_ERR_ARG
    assert call(ws=mis) == fva.FVA_ERR_ARG
    assert call(ws=None) == fva.FVA_ERR_ARG
    assert call(nbytes=need - 1) == fva.FVA_ERR_WORKSPACE
    # block LSEs need the row LSEs they are normalised by
    st = lib.fva_sparse_attn_fwd(ctypes.byref(p), fake, fake, *([fake] * 6), fake, None, fake, fake,
                                 need, None)
    assert st == fva.FVA_ERR_ARG
    # the traced call needs an 8-byte aligned trace buffer
    for trace in (None, ctypes.c_void_p((1 << 20) + 4)):
        st = lib.fva_sparse_attn_fwd_traced(ctypes.byref(p), fake, fake, *([fake] * 6), fake, None,
                                            None, fake, need, trace, None)
        assert st == fva.FVA_ERR_ARG


def test_order_kind_and_reserved_are_checked():
    lib = F.load_library()
    out = fva.Sizes()
    for kind, want in ((fva.FVA_ORDER_TILES, fva.FVA_OK), (fva.FVA_ORDER_HILBERT, fva.FVA_OK),
                       (2, fva.FVA_ERR_ARG), (-1, fva.FVA_ERR_ARG)):
        p = _ok_problem()
        p.order_kind = kind
        assert lib.fva_sizes(ctypes.byref(p), ctypes.byref(out)) == want
    p = _ok_problem()
    p.reserved = 1
    assert lib.fva_sizes(ctypes.byref(p), ctypes.byref(out)) == fva.FVA_ERR_ARG
    with pytest.raises(F.FvaError):
        F.make_problem(1, 1024, 64, (4, 16, 16), 64, (8, 8), 0.9, 1, order="zigzag")


def test_binding_refuses_cpu_tensors():
    import torch
    p = _ok_problem(num_heads=1, seq_len=1024, head_dim=64, grid=(4, 16, 16), block=64, tile=(8, 8))
    t = torch.zeros(16)
    with pytest.raises(F.FvaError):
        fva.route(p, t, t, t, t, t, t, t, t, t, t)
