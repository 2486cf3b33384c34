"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/af.h declares, and rejects bad arguments with the
documented status before any device work."""
import ctypes
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
from autoregressive_normalizing_flow_amd import binding as B  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    try:
        return B.load_library()
    except ImportError as e:  # the library is built by __graft_entry__.build()
        pytest.skip(str(e))


def test_exports_every_header_function(lib):
    names = B.header_functions()
    assert "af_forward" in names and "af_inverse_jacobi" in names and "af_prefill" in names
    for n in names:
        assert hasattr(lib, n), n
    import re
    ver = int(re.search(r"#define AF_ABI_VERSION (\d+)", open(B.HEADER).read()).group(1))
    assert lib.af_abi_version() == ver
    assert lib.af_status_str(0) == b"AF_OK"
    assert lib.af_status_str(4) == b"AF_ERR_NONFINITE"


# A plan over fake (never dereferenced) device pointers: af_plan_create only
# records them.
_FAKE = np.zeros(64, dtype=np.float32)


def fake_weights(n_layers, n_blocks=1):
    addr = ctypes.c_void_p(_FAKE.ctypes.data)
    keep = []
    ws = (B.af_block_weights * n_blocks)()
    for w in ws:
        for n in ("w_in", "b_in", "pos", "ln_f_g", "ln_f_b", "w_head", "b_head"):
            setattr(w, n, addr)
        for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g",
                  "ln2_b", "w_1", "b_1", "w_2", "b_2"):
            arr = (ctypes.c_void_p * n_layers)(*([addr] * n_layers))
            keep.append(arr)
            setattr(w, n, ctypes.cast(arr, B._PP))
    return ws, keep


def make_plan(lib, C=16, d=64, H=2, layers=1, max_len=64, dtype=B.AF_F32, T=1):
    ws, keep = fake_weights(layers, T)
    cfg = B.af_block_cfg(C, d, H, layers, max_len, dtype)
    h = ctypes.c_void_p()
    st = lib.af_plan_create(ctypes.byref(cfg), T, ws, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,expect", [
    (dict(C=0), B.AF_ERR_ARG),
    (dict(C=300), B.AF_ERR_ARG),
    (dict(d=96, H=3), B.AF_ERR_UNSUPPORTED),     # d/64 not a power of two
    (dict(d=64, H=3), B.AF_ERR_ARG),             # d % H
    (dict(d=256, H=16), B.AF_ERR_UNSUPPORTED),   # dh = 16
    (dict(d=64, H=1, dtype=B.AF_BF16), B.AF_ERR_UNSUPPORTED),  # bf16 needs d % 256
    (dict(layers=0), B.AF_ERR_ARG),
    (dict(max_len=0), B.AF_ERR_ARG),
    (dict(dtype=7), B.AF_ERR_ARG),
    (dict(T=0), B.AF_ERR_ARG),
    (dict(), B.AF_OK),
    (dict(d=512, H=8, dtype=B.AF_BF16, T=4), B.AF_OK),
])
def test_plan_create_validation(lib, kw, expect):
    st, h = make_plan(lib, **kw)
    assert st == expect, lib.af_last_error()
    if st == B.AF_OK:
        lib.af_plan_destroy(h)
    else:
        assert lib.af_last_error()


@pytest.mark.parametrize("field", ["pos", "b_head", "ln1_g", "w_2"])
def test_plan_create_rejects_misaligned_weights(lib, field):
    ws, keep = fake_weights(2)
    odd = ctypes.c_void_p(_FAKE.ctypes.data + 4)
    if field in ("pos", "b_head"):
        setattr(ws[0], field, odd)
    else:
        arr = (ctypes.c_void_p * 2)(ctypes.c_void_p(_FAKE.ctypes.data), odd)
        keep.append(arr)
        setattr(ws[0], field, ctypes.cast(arr, B._PP))
    cfg = B.af_block_cfg(16, 64, 2, 2, 64, B.AF_F32)
    h = ctypes.c_void_p()
    assert lib.af_plan_create(ctypes.byref(cfg), 1, ws, ctypes.byref(h)) == B.AF_ERR_ARG
    assert b"16-byte" in lib.af_last_error()


def test_workspace_bytes_monotone_and_cache_first(lib):
    st, h = make_plan(lib, C=48, d=1024, H=16, layers=8, max_len=1560, dtype=B.AF_BF16)
    assert st == B.AF_OK
    a = lib.af_workspace_bytes(h, 1, 16)
    b = lib.af_workspace_bytes(h, 1, 1560)
    c = lib.af_workspace_bytes(h, 2, 1560)
    assert 0 < a < b < c
    cache = lib.af_cache_bytes(h, 1)
    # 8 layers x (K + V) x 16 heads x 1600 padded positions x 64 x bf16
    assert cache == 8 * 2 * 16 * 1600 * 64 * 2
    assert lib.af_workspace_bytes(h, 0, 16) == 0
    lib.af_plan_destroy(h)


def test_entry_points_reject_bad_arguments_before_device_work(lib):
    st, h = make_plan(lib)
    assert st == B.AF_OK
    buf = ctypes.c_void_p(_FAKE.ctypes.data)
    iters = (ctypes.c_int32 * 16)()
    big = lib.af_workspace_bytes(h, 1, 64)
    # NULL inputs
    assert lib.af_forward(h, None, buf, buf, 1, 64, 1, 0, buf, big, None) == B.AF_ERR_ARG
    # L beyond max_len
    assert lib.af_forward(h, buf, ctypes.c_void_p(_FAKE.ctypes.data + 64), buf, 1, 65,
                          1, 0, buf, 1 << 40, None) == B.AF_ERR_ARG
    # workspace too small (checked before any launch)
    aligned = ctypes.c_void_p(1 << 20)
    assert lib.af_forward(h, buf, ctypes.c_void_p(_FAKE.ctypes.data + 64), buf, 1, 64,
                          1, 0, aligned, 16, None) == B.AF_ERR_WORKSPACE
    # log-det entries must group whole samples; unknown flags
    assert lib.af_forward(h, buf, ctypes.c_void_p(_FAKE.ctypes.data + 64), buf, 3, 64,
                          2, 0, aligned, 1 << 40, None) == B.AF_ERR_ARG
    assert lib.af_forward(h, buf, ctypes.c_void_p(_FAKE.ctypes.data + 64), buf, 1, 64,
                          0, 0, aligned, 1 << 40, None) == B.AF_ERR_ARG
    assert lib.af_forward(h, buf, ctypes.c_void_p(_FAKE.ctypes.data + 64), buf, 1, 64,
                          1, 4, aligned, 1 << 40, None) == B.AF_ERR_ARG
    # misaligned workspace
    assert lib.af_forward(h, buf, ctypes.c_void_p(_FAKE.ctypes.data + 64), buf, 1, 64,
                          1, 0, ctypes.c_void_p((1 << 20) + 4), big, None) == B.AF_ERR_ARG

    def inv(**kw):
        a = dict(z=buf, N=1, L=64, B=16, tau=1e-3, max_iters=0, init=0, x_init=None,
                 F=0, P=0, x_last=None, x=ctypes.c_void_p(_FAKE.ctypes.data + 128),
                 ws=aligned, wsb=big)
        a.update(kw)
        return lib.af_inverse_jacobi(h, a["z"], a["N"], a["L"], a["B"],
                                     ctypes.c_float(a["tau"]), a["max_iters"], a["init"],
                                     a["x_init"], a["F"], a["P"], a["x_last"], a["x"],
                                     iters, a["ws"], a["wsb"], None)

    assert inv(tau=math.nan) == B.AF_ERR_ARG
    assert inv(B=0) == B.AF_ERR_ARG
    assert inv(init=9) == B.AF_ERR_ARG
    assert inv(init=1) == B.AF_ERR_ARG                 # GIVEN without x_init
    assert inv(init=2, F=8) == B.AF_ERR_ARG            # frame shorter than block
    assert inv(P=1) == B.AF_ERR_ARG                    # prefix needs x_last
    assert inv(P=10, x_last=buf) == B.AF_ERR_ARG       # P + L > max_len
    assert inv(x=buf) == B.AF_ERR_ARG                  # x aliases z
    assert inv(wsb=8) == B.AF_ERR_WORKSPACE
    # token buffers are read as 16-byte vectors
    odd = ctypes.c_void_p(_FAKE.ctypes.data + 132)
    assert inv(x=odd) == B.AF_ERR_ARG
    assert inv(init=1, x_init=odd) == B.AF_ERR_ARG
    assert lib.af_forward(h, odd, ctypes.c_void_p(_FAKE.ctypes.data + 64), buf, 1, 64,
                          1, 0, aligned, big, None) == B.AF_ERR_ARG
    assert lib.af_prefill(h, None, 1, 8, aligned, big, None) == B.AF_ERR_ARG
    lib.af_plan_destroy(h)


def test_attention_validation(lib):
    a = ctypes.c_void_p(1 << 20)
    ws = lib.afk_attention_workspace_bytes(1, 100, 4, 64, 300)
    assert ws > 0 and lib.afk_attention_workspace_bytes(1, 100, 4, 48, 300) == 0
    ok = dict(N=1, R=100, H=4, dh=64, Lcap=448, P=300, ws=ws)

    def call(**kw):
        c = dict(ok)
        c.update(kw)
        return lib.afk_attention(a, a, a, a, c["N"], c["R"], c["H"], c["dh"], c["Lcap"],
                                 c["P"], a, c["ws"], None)
    assert call(dh=48) == B.AF_ERR_UNSUPPORTED
    assert call(Lcap=400) == B.AF_ERR_ARG            # not a multiple of 64
    assert call(P=400) == B.AF_ERR_ARG               # pos_base + R beyond Lcap
    assert call(R=0) == B.AF_ERR_ARG
    assert call(ws=ws - 1) == B.AF_ERR_WORKSPACE
    assert lib.afk_attention(None, a, a, a, 1, 100, 4, 64, 448, 300, a, ws, None) == B.AF_ERR_ARG
    assert lib.afk_attention(ctypes.c_void_p((1 << 20) + 2), a, a, a, 1, 100, 4, 64, 448, 300,
                             a, ws, None) == B.AF_ERR_ARG


def test_stream_copy_validation(lib):
    a, b = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 24)
    assert lib.afk_stream_copy(a, b, 0, None) == B.AF_OK          # nothing to do
    assert lib.afk_stream_copy(None, b, 16, None) == B.AF_ERR_ARG
    assert lib.afk_stream_copy(a, b, 24, None) == B.AF_ERR_ARG     # not whole 16-byte words
    assert lib.afk_stream_copy(ctypes.c_void_p((1 << 20) + 8), b, 16, None) == B.AF_ERR_ARG
    # overlapping ranges, either order
    assert lib.afk_stream_copy(a, ctypes.c_void_p((1 << 20) + 64), 128, None) == B.AF_ERR_ARG
    assert lib.afk_stream_copy(ctypes.c_void_p((1 << 20) + 64), a, 128, None) == B.AF_ERR_ARG


def test_stack_restrictions(lib):
    st, h = make_plan(lib, T=2)
    assert st == B.AF_OK
    buf = ctypes.c_void_p(_FAKE.ctypes.data)
    iters = (ctypes.c_int32 * 16)()
    big = lib.af_workspace_bytes(h, 1, 16)
    x = ctypes.c_void_p(_FAKE.ctypes.data + 128)
    assert lib.af_inverse_jacobi(h, buf, 1, 64, 16, ctypes.c_float(1e-3), 0, 2, None, 16,
                                 0, None, x, iters, ctypes.c_void_p(1 << 20), big,
                                 None) == B.AF_ERR_UNSUPPORTED
    assert lib.af_prefill(h, buf, 1, 8, ctypes.c_void_p(1 << 20), big, None) == B.AF_ERR_UNSUPPORTED
    assert lib.af_refresh_kv(h, buf, 1, 8, 0, None, ctypes.c_void_p(1 << 20), big,
                             None) == B.AF_ERR_UNSUPPORTED
    lib.af_plan_destroy(h)


def test_refresh_kv_validation(lib):
    st, h = make_plan(lib)          # max_len 64
    assert st == B.AF_OK
    buf = ctypes.c_void_p(_FAKE.ctypes.data)
    ws = ctypes.c_void_p(1 << 20)
    big = lib.af_workspace_bytes(h, 1, 64)
    assert lib.af_refresh_kv(h, None, 1, 8, 0, None, ws, big, None) == B.AF_ERR_ARG
    assert lib.af_refresh_kv(h, buf, 1, 8, 8, None, ws, big, None) == B.AF_ERR_ARG   # no x_last
    assert lib.af_refresh_kv(h, buf, 1, 60, 8, buf, ws, big, None) == B.AF_ERR_ARG   # past max_len
    assert lib.af_refresh_kv(h, buf, 1, 0, 0, None, ws, big, None) == B.AF_ERR_ARG
    assert lib.af_refresh_kv(h, buf, 1, 8, 0, None, ws, 16, None) == B.AF_ERR_WORKSPACE
    lib.af_plan_destroy(h)


def test_last_residual_needs_a_finished_call(lib):
    st, h = make_plan(lib)
    assert st == B.AF_OK
    out = (ctypes.c_float * 4)()
    assert lib.af_plan_last_residual(h, 2, out) == B.AF_ERR_ARG
    assert lib.af_plan_last_residual(h, 2, None) == B.AF_ERR_ARG
    assert lib.af_plan_last_residual(None, 2, out) == B.AF_ERR_ARG
    lib.af_plan_destroy(h)


def test_profile_class_names(lib):
    st, h = make_plan(lib)
    assert lib.af_profile_enable(h, b"nope") == B.AF_ERR_ARG
    assert lib.af_profile_disable(h) == B.AF_OK
    lib.af_plan_destroy(h)


def test_graph_controls(lib):
    st, h = make_plan(lib)
    assert st == B.AF_OK
    c = ctypes.c_longlong(-1)
    r = ctypes.c_longlong(-1)
    assert lib.af_plan_graph_stats(h, ctypes.byref(c), ctypes.byref(r)) == B.AF_OK
    assert (c.value, r.value) == (0, 0)
    assert lib.af_plan_graph_stats(h, None, ctypes.byref(r)) == B.AF_ERR_ARG
    assert lib.af_plan_set_graphs(h, 0) == B.AF_OK
    assert lib.af_plan_set_graphs(h, 1) == B.AF_OK
    assert lib.af_plan_set_graphs(None, 1) == B.AF_ERR_ARG
    assert lib.af_plan_set_fused_refresh(h, 0) == B.AF_OK
    assert lib.af_plan_set_fused_refresh(None, 1) == B.AF_ERR_ARG
    assert lib.af_plan_set_row_split(h, 0) == B.AF_OK
    assert lib.af_plan_set_row_split(h, 1) == B.AF_OK
    assert lib.af_plan_set_row_split(None, 1) == B.AF_ERR_ARG
    assert lib.af_plan_set_overlap_refresh(h, 0) == B.AF_OK
    assert lib.af_plan_set_overlap_refresh(h, 1) == B.AF_OK
    assert lib.af_plan_set_overlap_refresh(None, 1) == B.AF_ERR_ARG
    calls = []
    cb = B._BLOCK_DONE_FN(lambda user, t, b: calls.append((t, b)))
    assert lib.af_plan_set_block_done(h, cb, None) == B.AF_OK
    assert lib.af_plan_set_block_done(h, B._BLOCK_DONE_FN(), None) == B.AF_OK   # NULL
    assert lib.af_plan_set_block_done(None, cb, None) == B.AF_ERR_ARG
    assert calls == []
    lib.af_plan_destroy(h)


def test_workspace_has_room_for_the_row_split(lib):
    # blocks of 1024 to 4096 rows of one sample may be split over two
    # streams: from 1024 rows the workspace holds a second half's scratch
    # (tens of MB at d = 1024, against about 0.2 MB per extra row), and past
    # N * R = 4096 it no longer does (one layer: no refresh runs beside the
    # next block, whose scratch would cover the half's)
    st, h = make_plan(lib, C=48, d=1024, H=16, layers=1, max_len=4680, dtype=B.AF_BF16)
    assert st == B.AF_OK
    ws = lambda n, r: lib.af_workspace_bytes(h, n, r)
    assert ws(1, 1024) - ws(1, 1023) > 20e6
    assert ws(1, 4097) < ws(1, 4096)
    assert ws(2, 2049) < ws(2, 2048)
    # from two layers a block's cache refresh may run beside the next block:
    # the workspace holds a second full set of the per-pass scratch (which does
    # not depend on the layer count) at every block size; beside the cache the
    # one-layer workspace holds one set plus the higher-precision forward's lo
    # halves (a second cache among them), which are not doubled
    st, h2 = make_plan(lib, C=48, d=1024, H=16, layers=2, max_len=4680, dtype=B.AF_BF16)
    assert st == B.AF_OK
    c1, c2 = lib.af_cache_bytes(h, 1), lib.af_cache_bytes(h2, 1)
    for r in (100, 1023, 4097):
        one = ws(1, r) - 2 * c1
        two = lib.af_workspace_bytes(h2, 1, r) - 2 * c2
        assert 1.6 < two / one < 2.0, (r, one, two)
    lib.af_plan_destroy(h2)
    st, h32 = make_plan(lib, C=16, d=64, H=2, layers=1, max_len=2048)   # fp32: never split
    assert lib.af_workspace_bytes(h32, 1, 1024) - lib.af_workspace_bytes(h32, 1, 1023) < 1e6
    lib.af_plan_destroy(h32)
    lib.af_plan_destroy(h)
