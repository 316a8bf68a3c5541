"""CPU oracle for closed-form tree verification of Gated DeltaNet layers.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does, and
this package never imports the product library.  Everything here is float64
unless a step is defined in float32 (the log-space gate products, see
``tree_prep``).

Two independent formulations live here:

* ``bole_oracle.c`` (plain C, via ctypes): the definition.  Each node's output
  is ordinary sequential GDN decoding (Eq. 1 of the pages) along its
  root-to-node path from the shared pre-tree state; the accepted path's new
  state is the walked state after the accepted node.
* ``closed_form`` (numpy): Theorem 1 written out with explicit G, C, R, B0 and
  the finite Neumann series of Lemma 3, plus Eq. 10 for the commit.  It is used
  as a pin for the walk (the two must agree to rounding) and as the reference
  for the G/C factors.
* ``tree_conv`` (numpy): the tree-parallel short causal convolution of the
  pipeline's first stage and its conv-state commit, one node at a time.
* ``forest`` (Python/numpy): budget selection by cumulative draft probability
  and the packed-forest builder, one candidate at a time.

Pins of the oracle itself are in tests/test_oracle.py, tests/test_oracle_conv.py and
tests/test_oracle_forest.py.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

from .closed_form import (closed_form_tree, commit_closed_form, inverse_factors,  # noqa: F401
                          tree_factors)
from .tree_conv import conv_commit, tree_conv  # noqa: F401
from .forest import build_forest  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bole_oracle.c")
_LIB = os.path.join(_HERE, "libbole_oracle.so")
_lib = None

ERR_BAD_PARENT = 1
ERR_CYCLE = 2
ERR_TREE_SIZE = 4
ERR_BAD_ACCEPT = 8
ERR_BAD_SLOT = 16


def build(force: bool = True) -> str:
    """Compile the C oracle (gcc, -O2 -ffp-contract=off)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.bole_ref_tree_prep.restype = ctypes.c_uint32
        L.bole_ref_tree_prep.argtypes = [P, P, i32, i32, P, i32, i32, P, P, P, P, P]
        L.bole_ref_sequential.restype = None
        L.bole_ref_sequential.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P]
        L.bole_ref_prefix_batch.restype = None
        L.bole_ref_prefix_batch.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, i32]
        L.bole_ref_verify.restype = None
        L.bole_ref_verify.argtypes = [P] * 10 + [i32] * 5 + [P, P, P, P, i64, i32]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def tree_prep(parent, tree_off, log_gamma=None):
    """Topology and log-space gate products.

    parent [N] int32 (local, -1 = root), tree_off [B+1] int32,
    log_gamma [L, N, H] float32 or None.
    Returns dict(depth, anc (uint64), order, tree_depth, logP, err).
    Entries of invalid trees are left at their fill values (depth/order -1,
    anc 0, tree_depth -1, logP NaN)."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    tree_off = np.ascontiguousarray(tree_off, dtype=np.int32)
    B, N = len(tree_off) - 1, len(parent)
    depth = np.full(N, -1, np.int32)
    anc = np.zeros(N, np.uint64)
    order = np.full(N, -1, np.int32)
    tdep = np.full(B, -1, np.int32)
    logP = None
    L = H = 0
    if log_gamma is not None:
        log_gamma = np.ascontiguousarray(log_gamma, dtype=np.float32)
        L, _, H = log_gamma.shape
        logP = np.full(log_gamma.shape, np.nan, np.float32)
    err = _load().bole_ref_tree_prep(_p(parent), _p(tree_off), B, N, _p(log_gamma), L, H,
                                     _p(depth), _p(anc), _p(order), _p(tdep), _p(logP))
    return dict(depth=depth, anc=anc, order=order, tree_depth=tdep, logP=logP, err=int(err))


def sequential(S, q, k, v, g, beta):
    """Token-order decoding of n tokens from state S ([dv, dk], float64).
    Returns (S_final, o [n, dv], u [n, dv])."""
    S = np.array(S, dtype=np.float64, order="C")
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v))
    g, beta = (np.ascontiguousarray(a, dtype=np.float64) for a in (g, beta))
    n, dk = k.shape
    dv = v.shape[1]
    o = np.zeros((n, dv))
    u = np.zeros((n, dv))
    _load().bole_ref_sequential(n, dk, dv, _p(S), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                _p(o), _p(u))
    return S, o, u


def prefix_states(k, v, g, beta, nthreads: Optional[int] = None):
    """Committed states after running the recurrence from zero over each unit's
    prefix tokens.  k [U, n, dk], v [U, n, dv], g/beta [U, n] -> S [U, dv, dk]."""
    k, v, g, beta = (np.ascontiguousarray(a, dtype=np.float64) for a in (k, v, g, beta))
    U, n, dk = k.shape
    dv = v.shape[2]
    S = np.zeros((U, dv, dk))
    _load().bole_ref_prefix_batch(U, n, dk, dv, None, _p(k), _p(v), _p(g), _p(beta), _p(S),
                                  nthreads or default_threads())
    return S


def verify(parent, tree_off, q, k, v, g, beta, S_pre, slot, accept=None, units=None,
           nthreads: Optional[int] = None):
    """Walk oracle for one layer.

    q, k [N, H, dk]; v [N, H, dv]; g, beta [N, H]; S_pre [n_slots, H, dv, dk];
    slot [B]; accept [B] or None.  All floats are widened to float64.
    units: optional iterable of (b, h) pairs to compute (others stay NaN).
    Returns (O [N,H,dv], U [N,H,dv], S_new [B,H,dv,dk] or None)."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    tree_off = np.ascontiguousarray(tree_off, dtype=np.int32)
    slot = np.ascontiguousarray(slot, dtype=np.int32)
    q, k, v, g, beta, S_pre = (np.ascontiguousarray(a, dtype=np.float64)
                               for a in (q, k, v, g, beta, S_pre))
    N, H, dk = q.shape
    dv = v.shape[2]
    B = len(tree_off) - 1
    O = np.full((N, H, dv), np.nan)
    U = np.full((N, H, dv), np.nan)
    S_new = None
    acc = None
    if accept is not None:
        acc = np.ascontiguousarray(accept, dtype=np.int32)
        S_new = np.full((B, H, dv, dk), np.nan)
    ul = None
    n_units = 0
    if units is not None:
        ul = np.ascontiguousarray([b * H + h for (b, h) in units], dtype=np.int64)
        n_units = len(ul)
    _load().bole_ref_verify(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(S_pre), _p(slot),
                            _p(parent), _p(tree_off), _p(acc), B, N, H, dk, dv, _p(O), _p(U),
                            _p(S_new), _p(ul), n_units, nthreads or default_threads())
    return O, U, S_new
