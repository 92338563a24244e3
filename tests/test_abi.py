"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments before touching the GPU.  Runs without a GPU: every call here fails
validation on the host and launches nothing."""

import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "littlebit.h")
INIT_HEADER = os.path.join(ROOT, "include", "littlebit_init.h")

lb = pytest.importorskip("binary_rank_gemv_amd.littlebit",
                         reason="liblittlebit.so not built (run python -m binary_rank_gemv_amd.build)")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(littlebit_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(lb.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(lb.EXPORTED)


def test_init_library_is_separate():
    """The offline initialization lives in its own library; the layer library
    neither exports it nor links rocBLAS / rocSOLVER."""
    import subprocess
    names = declared_functions(INIT_HEADER)
    assert set(names) == set(lb.INIT_EXPORTED)
    init = ctypes.CDLL(lb.INIT_LIB_PATH)
    for name in names:
        assert hasattr(init, name), name
    layer = ctypes.CDLL(lb.LIB_PATH)
    assert not hasattr(layer, "littlebit_dual_svid_init")
    deps = subprocess.run(["readelf", "-d", lb.LIB_PATH], capture_output=True, text=True).stdout
    needed = re.findall(r"\(NEEDED\).*\[(.*)\]", deps)
    assert needed and not any("rocblas" in d or "rocsolver" in d for d in needed), needed


def test_workspace_error_rejects_bad_arguments():
    f = lb.LIB.littlebit_workspace_error
    assert f(None, 4096, FAKE, None) == lb.LB_ERR_INVALID_ARG
    assert f(FAKE, 4096, None, None) == lb.LB_ERR_INVALID_ARG
    assert f(FAKE + 16, 4096, FAKE, None) == lb.LB_ERR_WORKSPACE
    assert f(FAKE, 4095, FAKE, None) == lb.LB_ERR_WORKSPACE
    assert f(FAKE, 4096, FAKE + 2, None) == lb.LB_ERR_INVALID_ARG


@pytest.mark.parametrize("R,K", [(16, 64), (20, 600), (1472, 4096), (11008, 1472), (168, 13824), (1, 1)])
def test_packed_bytes_matches_format(R, K):
    assert lb.littlebit_packed_bytes(R, K) == oracle.packed_factor_bytes(R, K)


def test_packed_bytes_rejects_nonpositive():
    assert lb.littlebit_packed_bytes(0, 64) == 0
    assert lb.littlebit_packed_bytes(16, -1) == 0


def test_status_strings():
    for s in (lb.LB_OK, lb.LB_ERR_INVALID_ARG, lb.LB_ERR_UNSUPPORTED, lb.LB_ERR_WORKSPACE, lb.LB_ERR_HIP):
        assert lb.littlebit_status_string(s).startswith("LB_")


FAKE = 1 << 20   # a non-null, 256-byte aligned address that is never dereferenced


def _layer(m=64, n=64, r=16, nb=2, **over):
    s = lb._Layer()
    s.m, s.n, s.nbranches = m, n, nb
    for i in range(2):
        s.br[i] = lb._Branch(FAKE, FAKE, FAKE, FAKE, FAKE, r)
    for k, v in over.items():
        setattr(s, k, v)
    return s


def _fwd(layer, mask=3, x=FAKE, batch=1, ldx=64, y=FAKE, ldy=64, ws=FAKE, ws_bytes=1 << 30, flags=0):
    return lb.LIB.littlebit_linear_fwd(ctypes.byref(layer), mask, x, batch, ldx, y, ldy, ws, ws_bytes, flags, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), lb.LB_ERR_INVALID_ARG),
    (dict(y=None), lb.LB_ERR_INVALID_ARG),
    (dict(batch=0), lb.LB_ERR_INVALID_ARG),
    (dict(mask=0), lb.LB_ERR_INVALID_ARG),
    (dict(mask=4), lb.LB_ERR_INVALID_ARG),
    (dict(ldx=32), lb.LB_ERR_INVALID_ARG),
    (dict(ldy=60), lb.LB_ERR_INVALID_ARG),
    (dict(x=FAKE + 1), lb.LB_ERR_INVALID_ARG),
    (dict(flags=3), lb.LB_ERR_INVALID_ARG),
    (dict(flags=8), lb.LB_ERR_INVALID_ARG),
    (dict(flags=1, batch=17), lb.LB_ERR_INVALID_ARG),
    (dict(ws=None), lb.LB_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), lb.LB_ERR_WORKSPACE),
    (dict(ws_bytes=64), lb.LB_ERR_WORKSPACE),
])
def test_linear_fwd_rejects_bad_arguments(kwargs, status):
    assert _fwd(_layer(), **kwargs) == status
    assert lb.littlebit_last_error()


def test_linear_fwd_rejects_bad_layers():
    assert lb.LIB.littlebit_linear_fwd(None, 3, FAKE, 1, 64, FAKE, 64, FAKE, 1 << 30, 0, None) == lb.LB_ERR_INVALID_ARG
    assert _fwd(_layer(m=0)) == lb.LB_ERR_INVALID_ARG
    assert _fwd(_layer(nb=3)) == lb.LB_ERR_INVALID_ARG
    assert _fwd(_layer(nb=1), mask=2) == lb.LB_ERR_INVALID_ARG
    assert _fwd(_layer(r=0)) == lb.LB_ERR_INVALID_ARG
    assert _fwd(_layer(r=5000)) == lb.LB_ERR_UNSUPPORTED
    assert _fwd(_layer(n=40000), ldx=40000) == lb.LB_ERR_UNSUPPORTED
    bad = _layer()
    bad.br[1].g = None
    assert _fwd(bad) == lb.LB_ERR_INVALID_ARG
    mis = _layer()
    mis.br[0].h = FAKE + 2
    assert _fwd(mis) == lb.LB_ERR_INVALID_ARG


def test_workspace_bytes_queries():
    L = _layer(m=11008, n=4096, r=1472)
    w1 = lb.LIB.littlebit_linear_workspace_bytes(ctypes.byref(L), 1)
    w16 = lb.LIB.littlebit_linear_workspace_bytes(ctypes.byref(L), 16)
    assert 0 < w1 < w16
    assert lb.LIB.littlebit_linear_workspace_bytes(ctypes.byref(L), 0) == 0
    assert lb.LIB.littlebit_linear_workspace_bytes(None, 1) == 0
    arr = (lb._Layer * 7)(*[_layer(m=5120, n=5120, r=688) for _ in range(7)])
    assert lb.LIB.littlebit_block_workspace_bytes(arr, 1) > 0


def test_pack_rejects_bad_arguments():
    P = lb.LIB.littlebit_pack
    assert P(None, 0, 4, 4, 4, 0, FAKE, None) == lb.LB_ERR_INVALID_ARG
    assert P(FAKE, 0, 4, 4, 4, 0, None, None) == lb.LB_ERR_INVALID_ARG
    assert P(FAKE, 0, 0, 4, 4, 0, FAKE, None) == lb.LB_ERR_INVALID_ARG
    assert P(FAKE, 0, 4, 4, 3, 0, FAKE, None) == lb.LB_ERR_INVALID_ARG
    assert P(FAKE, 5, 4, 4, 4, 0, FAKE, None) == lb.LB_ERR_INVALID_ARG
    assert P(FAKE, 0, 4, 4, 4, 2, FAKE, None) == lb.LB_ERR_INVALID_ARG
    assert P(FAKE, 0, 4, 4, 4, 0, FAKE + 1, None) == lb.LB_ERR_INVALID_ARG


def test_block_fwd_rejects_bad_arguments():
    arr = (lb._Layer * 7)(*[_layer() for _ in range(7)])
    ys = (ctypes.c_void_p * 7)(*([FAKE] * 7))
    B = lb.LIB.littlebit_block_fwd
    assert B(None, FAKE, FAKE, FAKE, FAKE, ys, 1, FAKE, 1 << 30, None) == lb.LB_ERR_INVALID_ARG
    assert B(arr, None, FAKE, FAKE, FAKE, ys, 1, FAKE, 1 << 30, None) == lb.LB_ERR_INVALID_ARG
    assert B(arr, FAKE, FAKE, FAKE, FAKE, ys, 0, FAKE, 1 << 30, None) == lb.LB_ERR_INVALID_ARG
    assert B(arr, FAKE, FAKE, FAKE, FAKE, ys, 1, FAKE, 16, None) == lb.LB_ERR_WORKSPACE
    ys2 = (ctypes.c_void_p * 7)(*([FAKE] * 6 + [None]))
    assert B(arr, FAKE, FAKE, FAKE, FAKE, ys2, 1, FAKE, 1 << 30, None) == lb.LB_ERR_INVALID_ARG


def test_dual_svid_init_rejects_bad_arguments():
    arr = (lb._InitBranch * 2)()
    for b in range(2):
        arr[b] = lb._InitBranch(FAKE, FAKE, FAKE, FAKE, FAKE)
    init = lb._init_lib()
    f = init.littlebit_dual_svid_init
    assert f(None, 64, 32, 32, 8, 2, 0, arr, None) == lb.LB_ERR_INVALID_ARG
    assert f(FAKE, 64, 32, 16, 8, 2, 0, arr, None) == lb.LB_ERR_INVALID_ARG       # ldw < n
    assert f(FAKE, 64, 32, 32, 33, 2, 0, arr, None) == lb.LB_ERR_INVALID_ARG      # r > min(m, n)
    assert f(FAKE, 64, 32, 32, 0, 2, 0, arr, None) == lb.LB_ERR_INVALID_ARG
    assert f(FAKE, 64, 32, 32, 8, 3, 0, arr, None) == lb.LB_ERR_INVALID_ARG      # nbranches
    assert f(FAKE, 40000, 32, 32, 8, 1, 0, arr, None) == lb.LB_ERR_UNSUPPORTED
    assert f(FAKE, 64, 32, 32, 8, 2, -1, arr, None) == lb.LB_ERR_INVALID_ARG   # itq_iters
    arr[1] = lb._InitBranch(FAKE, None, FAKE, FAKE, FAKE)
    assert f(FAKE, 64, 32, 32, 8, 2, 0, arr, None) == lb.LB_ERR_INVALID_ARG
    assert "NULL output" in init.littlebit_init_last_error().decode()


def _noalloc(layer, mask=3, x=FAKE, batch=1, ldx=64, y=FAKE, ldy=64, flags=0):
    return lb.LIB.littlebit_linear_fwd_noalloc(ctypes.byref(layer), mask, x, batch, ldx, y, ldy, flags, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), lb.LB_ERR_INVALID_ARG),
    (dict(y=None), lb.LB_ERR_INVALID_ARG),
    (dict(batch=0), lb.LB_ERR_INVALID_ARG),
    (dict(mask=4), lb.LB_ERR_INVALID_ARG),
    (dict(ldx=32), lb.LB_ERR_INVALID_ARG),
    (dict(x=FAKE + 1), lb.LB_ERR_INVALID_ARG),
    (dict(flags=3), lb.LB_ERR_INVALID_ARG),
    (dict(flags=1, batch=17), lb.LB_ERR_INVALID_ARG),
])
def test_noalloc_rejects_bad_arguments(kwargs, status):
    """The no-alloc variant validates like littlebit_linear_fwd, before it
    looks up its scratch or launches anything."""
    assert _noalloc(_layer(), **kwargs) == status
    assert "littlebit_linear_fwd_noalloc" in lb.littlebit_last_error()
