"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

Every entry point validates its arguments before touching the HIP runtime, so
these calls return synchronously with a status code.
"""

import ctypes
import os
import re

import pytest

import linear_attention_tree_amd as lat
from linear_attention_tree_amd import bole

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bole.h")

E_NULL, E_SHAPE, E_DTYPE, E_UNSUPPORTED = 1, 2, 3, 4
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"BOLE_API\s+[\w\s\*]+?\b(bole_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    return bole.lib()


def test_exports_every_declared_symbol(L):
    names = declared_symbols()
    assert set(names) == {"bole_tree_prep", "bole_gc_workspace_bytes", "bole_factor_gc",
                          "bole_verify", "bole_factor_verify", "bole_tree_verify",
                          "bole_commit_tree_verify",
                          "bole_verify_neumann", "bole_factor_inverse", "bole_verify_inverse",
                          "bole_commit_path", "bole_tree_conv", "bole_conv_commit",
                          "bole_forest_build", "bole_forest_workspace_bytes",
                          "bole_forest_build_noalloc",
                          "bole_status_string"}
    for n in names:
        assert hasattr(L, n), n
        assert hasattr(lat, n), n   # same names in the Python binding


def test_internal_launchers_are_hidden(L):
    for n in ("bole_verify_launch", "bole_factor_gc_launch", "bole_commit_launch",
              "bole_verify_neumann_launch", "bole_verify_inverse_launch",
              "bole_factor_inverse_launch", "bole_forest_build_launch",
              "bole_tree_verify_launch", "bole_commit_tree_verify_launch",
              "bole_tree_conv_launch", "bole_conv_commit_launch", "bole_forest_scratch"):
        with pytest.raises(AttributeError):
            getattr(L, n)


def test_status_strings_and_workspace(L):
    assert lat.bole_status_string(0) == "ok"
    assert "NULL" in lat.bole_status_string(1)
    assert lat.bole_status_string(77) == "unknown status"
    assert lat.bole_gc_workspace_bytes(16, 32) == 2 * 16 * 32 * 64 * 64 * 4
    assert lat.bole_gc_workspace_bytes(0, 32) == 0


def test_tree_prep_argument_errors(L):
    f = L.bole_tree_prep
    assert f(None, FAKE, 1, 1, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, None, None) == E_NULL
    assert f(FAKE, FAKE, 0, 1, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, None, None) == E_SHAPE
    assert f(FAKE, FAKE, 1, 0, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, None, None) == E_SHAPE
    # gates without a logP output
    assert f(FAKE, FAKE, 1, 1, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, None, None, None) == E_NULL
    assert f(FAKE, FAKE, 1, 1, FAKE, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == E_SHAPE


@pytest.mark.parametrize("fn", ["bole_factor_gc", "bole_factor_inverse"])
def test_factor_gc_argument_errors(L, fn):
    f = getattr(L, fn)
    args = [FAKE] * 7
    assert f(7, *args, 1, 1, 1, 128, FAKE, FAKE, None, None) == E_DTYPE
    assert f(1, None, *args[1:], 1, 1, 1, 128, FAKE, FAKE, None, None) == E_NULL
    assert f(1, *args, 1, 1, 0, 128, FAKE, FAKE, None, None) == E_SHAPE
    for dk in (0, 8, 24, 272):
        assert f(1, *args, 1, 1, 1, dk, FAKE, FAKE, None, None) == E_UNSUPPORTED


def _verify(L, dtype=1, B=1, N=1, H=1, dk=128, dv=128, n_slots=1, O=FAKE, fn="bole_verify"):
    p = [FAKE] * 6
    return getattr(L, fn)(dtype, *p, n_slots, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         B, N, H, dk, dv, O, FAKE, None, None)


@pytest.mark.parametrize("fn", ["bole_verify", "bole_verify_neumann", "bole_verify_inverse"])
def test_verify_argument_errors(L, fn):
    assert _verify(L, dtype=2, fn=fn) == E_DTYPE
    assert _verify(L, O=None, fn=fn) == E_NULL
    assert _verify(L, B=0, fn=fn) == E_SHAPE
    assert _verify(L, n_slots=0, fn=fn) == E_SHAPE
    assert _verify(L, dv=100, fn=fn) == E_UNSUPPORTED
    assert _verify(L, dk=512, fn=fn) == E_UNSUPPORTED


def test_factor_verify_argument_errors(L):
    f = L.bole_factor_verify

    def call(dtype=1, dk=128, dv=128, O=FAKE, B=1):
        return f(dtype, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 B, 1, 1, dk, dv, O, FAKE, None, None)

    assert call(dtype=9) == E_DTYPE
    assert call(O=None) == E_NULL
    assert call(B=0) == E_SHAPE
    assert call(dk=256) == E_UNSUPPORTED          # one staged chunk only
    assert call(dtype=0, dk=128) == E_UNSUPPORTED
    assert call(dtype=0, dk=64, dv=24) == E_UNSUPPORTED


def test_tree_verify_argument_errors(L):
    f = L.bole_tree_verify

    def call(dtype=1, dk=128, dv=128, parent=FAKE, logP=FAKE, B=1, H=1):
        return f(dtype, FAKE, FAKE, FAKE, parent, FAKE, FAKE, FAKE, 1, FAKE, FAKE, B, 1, H, dk, dv,
                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, logP, None, None)

    assert call(dtype=3) == E_DTYPE
    assert call(parent=None) == E_NULL
    assert call(logP=None) == E_NULL
    assert call(B=0) == E_SHAPE
    assert call(H=0) == E_SHAPE
    assert call(dk=256) == E_UNSUPPORTED
    assert call(dtype=0, dk=128) == E_UNSUPPORTED
    assert call(dv=40) == E_UNSUPPORTED


def test_commit_tree_verify_argument_errors(L):
    f = L.bole_commit_tree_verify
    A = ctypes.c_void_p(0x1000)          # 8-byte aligned, never dereferenced
    U = ctypes.c_void_p(0x1004)          # not 8-byte aligned

    def call(dtype=1, dk=128, dv=128, pool=A, prev_k=A, accept=A, B=1, H=1, N0=1):
        return f(dtype, A, A, A, A, A, A, pool, 1, A, A, B, 1, H, dk, dv,
                 A, A, A, A, A, A, A, prev_k, A, A, A, A, accept, N0, None, None)

    assert call(dtype=3) == E_DTYPE
    assert call(pool=None) == E_NULL
    assert call(prev_k=None) == E_NULL
    assert call(accept=None) == E_NULL
    assert call(B=0) == E_SHAPE
    assert call(N0=0) == E_SHAPE
    assert call(dk=256) == E_UNSUPPORTED
    assert call(dtype=0, dk=128) == E_UNSUPPORTED
    assert call(prev_k=U) == E_UNSUPPORTED


def test_tree_conv_argument_errors(L):
    f = L.bole_tree_conv
    A = ctypes.c_void_p(0x1000)          # 16-byte aligned, never dereferenced
    U = ctypes.c_void_p(0x1002)          # not 16-byte aligned

    def call(dtype=1, x=A, st=A, B=1, N=1, C=64, W=4, y=A, slot=A):
        return f(dtype, x, A, None, st, 1, slot, A, A, B, N, C, W, y, None, None)

    assert call(dtype=4) == E_DTYPE
    assert call(x=None) == E_NULL
    assert call(st=None) == E_NULL            # a state is needed for W > 1
    # no state is needed for W == 1: validation gets past the pointers and stops
    # at the channel count (nothing is launched)
    assert call(st=None, slot=None, W=1, C=12) == E_UNSUPPORTED
    assert call(B=0) == E_SHAPE
    assert call(W=9) == E_UNSUPPORTED
    assert call(W=0) == E_UNSUPPORTED
    assert call(C=12) == E_UNSUPPORTED        # not a multiple of 8
    assert call(y=U) == E_UNSUPPORTED


def test_conv_commit_argument_errors(L):
    f = L.bole_conv_commit

    def call(dtype=1, st=FAKE, acc=FAKE, B=1, W=4):
        return f(dtype, st, 1, FAKE, FAKE, FAKE, FAKE, acc, B, 1, 64, W, None, None)

    assert call(dtype=2) == E_DTYPE
    assert call(st=None) == E_NULL
    assert call(acc=None) == E_NULL
    assert call(B=0) == E_SHAPE
    assert call(W=9) == E_UNSUPPORTED


def test_commit_argument_errors(L):
    f = L.bole_commit_path

    def call(Lyr=1, dtype=1, stride=0, B=1, dk=128, acc=FAKE):
        return f(Lyr, FAKE, stride, 1, FAKE, dtype, FAKE, 0, FAKE, 0, FAKE, 0, FAKE, FAKE, acc,
                 B, 1, 1, dk, 128, None, None)

    assert call(dtype=5) == E_DTYPE
    assert call(acc=None) == E_NULL
    assert call(Lyr=0) == E_SHAPE
    assert call(stride=-1) == E_SHAPE
    assert call(B=0) == E_SHAPE
    assert call(dk=20) == E_UNSUPPORTED


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        lat.bole_tree_prep(t, t, None, t, t.long(), t, t, None)


def test_forest_build_argument_errors(L):
    f = L.bole_forest_build
    ws = ctypes.c_void_p(0x1000)

    def call(B=2, M=10, cap=8, mt=64, ws=ws, rho=FAKE):
        return f(FAKE, FAKE, FAKE, B, M, cap, mt, rho, FAKE, FAKE, FAKE, ws, None, None)

    assert call(rho=None) == E_NULL
    assert call(ws=None) == E_NULL
    assert call(B=0) == E_SHAPE
    assert call(B=4096) == E_SHAPE
    assert call(M=0) == E_SHAPE
    assert call(cap=0) == E_SHAPE
    assert call(mt=0) == E_SHAPE
    assert call(mt=65) == E_SHAPE
    assert call(B=257, mt=64) == E_SHAPE                     # more than 16384 listed keys
    assert call(ws=ctypes.c_void_p(0x1004)) == E_UNSUPPORTED  # workspace not 8-byte aligned
    assert lat.bole_forest_workspace_bytes(16, 64) == 12 * 16 * 64
    assert lat.bole_forest_workspace_bytes(0, 64) == 0
    assert lat.bole_forest_workspace_bytes(300, 64) == 0
