"""The C ABI without a GPU: the library loads, exports every function that
include/mq.h declares, and rejects invalid arguments on the host before any
HIP call.  Every call below fails validation, so nothing is launched."""
import ctypes
import os
import re

import pytest

from nested_integer_weight_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mq.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in _lib.STATUS.items():
        assert L.mq_status_str(code).decode().startswith(name)
    assert L.mq_status_str(123).decode() == "MQ_UNKNOWN"


@pytest.mark.parametrize("n,k", [(1, 64), (512, 512), (14336, 4096), (4096, 14336), (3, 192)])
def test_plane_bytes(L, n, k):
    bits = [2, 1, 1, 2, 2]
    got = [L.mq_plane_bytes(n, k, p) for p in range(5)]
    assert got == [n * k * b // 8 for b in bits]
    assert sum(got) == n * k
    assert L.mq_plane_bytes(n, k, 5) == 0 and L.mq_plane_bytes(n, k, -1) == 0


def test_plane_bytes_bad_shape(L):
    assert L.mq_plane_bytes(0, 64, 0) == 0
    assert L.mq_plane_bytes(4, 96, 0) == 0  # k % 64


def test_planes_needed_table(L):
    # PREFIX reads r bits -> planes covering bits 2,3,4,6,8; ROUND reads r+1.
    assert [L.mq_planes_needed(r, 0) for r in (2, 3, 4, 6, 8)] == [1, 2, 3, 4, 5]
    assert [L.mq_planes_needed(r, 1) for r in (2, 3, 4, 6, 8)] == [2, 3, 4, 5, 5]
    assert [L.mq_planes_needed(r, 2) for r in (2, 3, 4, 6, 8)] == [2, 3, 4, 5, 5]
    assert L.mq_planes_needed(5, 0) == -1 and L.mq_planes_needed(2, 7) == -1 and L.mq_planes_needed(2, 3) == -1


def _packed(n=64, k=128, planes=(16, 32, 48, 64, 80)):
    c = _lib.MqPacked()
    c.n, c.k = n, k
    for i, p in enumerate(planes):
        c.plane[i] = p
    return c


def _linear(L, x=4096, dt=1, m=1, w=None, r=4, rule=0, group=64, s=4096, z=8192, y=12288):
    w = _packed() if w is None else w
    return L.mq_linear(x, dt, m, None if w is False else ctypes.byref(w), r, rule, group, s, z, y, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(r=5), 2), (dict(r=1), 2), (dict(r=9), 2),
    (dict(rule=3), 8), (dict(rule=-1), 8),
    (dict(group=32), 3), (dict(group=96), 3), (dict(group=0), 3),
    (dict(w=_packed(k=100)), 3), (dict(w=_packed(n=0)), 1), (dict(w=False), 1),
    (dict(m=-1), 1),
    (dict(x=0), 1), (dict(y=0), 1), (dict(s=0), 1),
    (dict(x=4100), 4), (dict(y=12289), 4), (dict(z=8200), 4),
    (dict(w=_packed(planes=(16, 0, 48, 64, 80)), r=3), 5),
    (dict(w=_packed(planes=(16, 32, 48, 0, 80)), r=4, rule=1), 5),
    (dict(w=_packed(planes=(18, 32, 48, 64, 80))), 4),
    (dict(dt=0), 6), (dict(dt=7), 6),
    (dict(w=_packed(k=(1 << 22) + 64)), 9),
])
def test_linear_validation(L, kw, status):
    assert _linear(L, **kw) == status


def test_m_zero_with_bad_width_still_rejected(L):
    assert _linear(L, m=0, r=5) == 2


def test_pack_validation(L):
    w = _packed()
    assert L.mq_pack_parent(None, 64, 128, ctypes.byref(w), None) == 1
    assert L.mq_pack_parent(4096, 64, 128, None, None) == 1
    assert L.mq_pack_parent(4096, 64, 100, ctypes.byref(w), None) == 3
    assert L.mq_pack_parent(4096, 32, 128, ctypes.byref(w), None) == 3  # n mismatch
    assert L.mq_pack_parent(4097, 64, 128, ctypes.byref(w), None) == 4
    assert L.mq_pack_parent(4096, 64, 128, ctypes.byref(_packed(planes=(16, 32, 0, 64, 80))), None) == 5


def test_slice_and_dequant_validation(L):
    w = _packed()
    assert L.mq_slice_codes(ctypes.byref(w), 7, 0, 4096, None) == 2
    assert L.mq_slice_codes(ctypes.byref(w), 4, 0, None, None) == 1
    assert L.mq_slice_codes(ctypes.byref(w), 4, 0, 4099, None) == 4
    assert L.mq_dequant(ctypes.byref(w), 4, 0, 64, 4096, 8192, 5, 12288, None) == 6
    assert L.mq_dequant(ctypes.byref(w), 4, 0, 48, 4096, 8192, 0, 12288, None) == 3
    assert L.mq_dequant(ctypes.byref(w), 4, 0, 64, None, 8192, 0, 12288, None) == 1


def test_mixed_reports_first_invalid_call(L):
    good = _packed()
    calls = (_lib.MqCall * 3)()
    for i in range(3):
        c = calls[i]
        c.x, c.x_dtype, c.m, c.w = 4096, 1, 1, ctypes.pointer(good)
        c.r, c.rule, c.group, c.scales, c.zeros, c.y = 4, 0, 64, 4096, 8192, 12288
    calls[2].r = 5
    calls[1].group = 32  # the first invalid one
    failed = ctypes.c_int32(99)
    assert L.mq_linear_mixed(calls, 3, None, 0, ctypes.byref(failed), None) == 3
    assert failed.value == 1
    assert L.mq_linear_mixed(None, 2, None, 0, None, None) == 1


def test_workspace_query_is_pure(L):
    assert L.mq_linear_workspace_bytes(1, 14336, 4096) == 0
    assert L.mq_linear_workspace_bytes(0, 14336, 4096) == 0
    ws = L.mq_linear_workspace_bytes(64, 4096, 14336)
    assert ws % (64 * 4096 * 4) == 0


def test_noalloc_validation_before_any_hip_call(L):
    w = _packed(n=6144, k=14336)
    args = dict(x=4096, dt=2, s=4096, z=8192, y=12288)
    # invalid arguments are rejected exactly as by mq_linear
    assert L.mq_linear_noalloc(args["x"], 2, 1, ctypes.byref(w), 5, 0, 128, args["s"], args["z"], args["y"],
                               None) == 2
    assert L.mq_linear_noalloc(args["x"], 2, 1, ctypes.byref(w), 4, 0, 96, args["s"], args["z"], args["y"],
                               None) == 3
    # m = 0 is a no-op
    assert L.mq_linear_noalloc(args["x"], 2, 0, ctypes.byref(w), 4, 0, 128, args["s"], args["z"], args["y"],
                               None) == 0
    # a shape whose split-k workspace exceeds the static scratch is refused
    assert L.mq_linear_workspace_bytes(2048, 6144, 14336) > _lib.NOALLOC_SCRATCH_BYTES
    assert L.mq_linear_noalloc(args["x"], 2, 2048, ctypes.byref(w), 4, 0, 128, args["s"], args["z"], args["y"],
                               None) == 9


def _produce(L, w=4096, n=64, k=256, group=64, widths=(3, 4, 8), lams=(1.0, 1.0, 1.0), nw=None, rule=0,
             n_grid=80, grid_den=100, codes=8192, s=12288, z=16384):
    wa = (ctypes.c_int32 * max(len(widths), 1))(*widths)
    la = (ctypes.c_float * max(len(lams), 1))(*lams)
    nw = len(widths) if nw is None else nw
    return L.mq_produce_parent(w, n, k, group, wa, la, nw, rule, n_grid, grid_den, codes, s, z, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=0), 1), (dict(codes=0), 1), (dict(s=0), 1), (dict(z=0), 1),
    (dict(n=0), 1), (dict(k=96), 3), (dict(group=96), 3), (dict(group=2048, k=4096), 3),
    (dict(rule=3), 8),
    (dict(widths=(3, 5, 8)), 2), (dict(widths=(3, 3, 8)), 2), (dict(widths=(1,), lams=(1.0,)), 2),
    (dict(nw=0), 1), (dict(widths=(2, 3, 4, 6, 8, 8), lams=(1.0,) * 6), 1),
    (dict(lams=(1.0, -1.0, 1.0)), 1), (dict(lams=(1.0, float("nan"), 1.0)), 1),
    (dict(lams=(1.0, float("inf"), 1.0)), 1),
    (dict(n_grid=0), 1), (dict(n_grid=101), 1), (dict(grid_den=0), 1), (dict(n_grid=300, grid_den=400), 1),
    (dict(w=4100), 4), (dict(codes=8200), 4), (dict(s=12290), 4), (dict(n=1 << 20, k=1 << 21), 9),
])
def test_produce_validation(L, kw, status):
    assert _produce(L, **kw) == status


def test_mixed_workspace_query_is_pure(L):
    w1 = _packed(n=14336, k=4096)
    w2 = _packed(n=4096, k=14336)
    arr = (_lib.MqCall * 3)()
    for i, w in enumerate((w1, w1, w2)):
        arr[i].x, arr[i].x_dtype, arr[i].m, arr[i].w = 4096, 1, 8, ctypes.pointer(w)
        arr[i].r, arr[i].rule, arr[i].group = 2, 0, 128
        arr[i].scales, arr[i].zeros, arr[i].y = 8192, 12288, 16384 + 4096 * i
    single = max(L.mq_linear_workspace_bytes(8, w.n, w.k) for w in (w1, w1, w2))
    got = L.mq_linear_mixed_workspace_bytes(arr, 3)
    assert got >= single and got % 4 == 0
    assert L.mq_linear_mixed_workspace_bytes(arr, 3) == got           # pure: same answer again
    assert L.mq_linear_mixed_workspace_bytes(None, 3) == 0
    assert L.mq_linear_mixed_workspace_bytes(arr, 0) == 0
    for i in range(3):
        arr[i].m = 1                                                     # GEMV calls: no workspace
    assert L.mq_linear_mixed_workspace_bytes(arr, 3) == 0
