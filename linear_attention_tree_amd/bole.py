"""Thin ctypes binding of libbole.so (the C ABI declared in include/bole.h).

Argument marshalling only: every function checks tensor placement, dtype,
contiguity and shapes, then passes raw device pointers, sizes and the current
HIP stream to the library.  All arithmetic runs in the library's HIP kernels;
there is no CPU or PyTorch fallback, and a missing library is an error.

Tensor conventions (see bole.h for the full contract):
  parent [N] int32, tree_off [B+1] int32, accept [B] int32, slot [B] int32
  anc [N] int64 (the uint64 ancestor bit sets, stored bit for bit)
  err [1] int32 (the device uint32 error word), or None
  q, k [N, H, d_k], v [N, H, d_v] in float32 or bfloat16
  logP, beta [N, H] float32; state_pool [n_slots, H, d_v, d_k] float32
  G, C [B, H, 64, 64] float32 (level-order positions); O [N, H, d_v] like v;
  U [N, H, d_v] float32
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbole.so")

BOLE_F32, BOLE_BF16 = 0, 1
ERR_BAD_PARENT, ERR_CYCLE, ERR_TREE_SIZE, ERR_BAD_ACCEPT, ERR_BAD_SLOT = 1, 2, 4, 8, 16
ERR_BAD_PROB, ERR_DISCONNECTED = 32, 64
MAX_TREE = 64

_lib = None


class BoleError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({status_string(code)})")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libbole.so (built in-tree by linear_attention_tree_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m linear_attention_tree_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.bole_tree_prep.restype = ctypes.c_int
        L.bole_tree_prep.argtypes = [P, P, i32, i32, P, i32, i32, P, P, P, P, P, P, P]
        L.bole_gc_workspace_bytes.restype = ctypes.c_size_t
        L.bole_gc_workspace_bytes.argtypes = [i32, i32]
        for fn in ("bole_factor_gc", "bole_factor_inverse"):
            getattr(L, fn).restype = ctypes.c_int
            getattr(L, fn).argtypes = [i32, P, P, P, P, P, P, P, i32, i32, i32, i32, P, P, P, P]
        for fn in ("bole_verify", "bole_verify_neumann", "bole_verify_inverse"):
            getattr(L, fn).restype = ctypes.c_int
            getattr(L, fn).argtypes = ([i32, P, P, P, P, P, P, i32, P, P, P, P, P, P, P]
                                       + [i32] * 5 + [P, P, P, P])
        L.bole_factor_verify.restype = ctypes.c_int
        L.bole_factor_verify.argtypes = ([i32, P, P, P, P, P, P, i32, P, P, P, P, P, P]
                                         + [i32] * 5 + [P, P, P, P])
        L.bole_tree_verify.restype = ctypes.c_int
        L.bole_tree_verify.argtypes = ([i32, P, P, P, P, P, P, P, i32, P, P]
                                       + [i32] * 5 + [P] * 9)
        L.bole_commit_tree_verify.restype = ctypes.c_int
        L.bole_commit_tree_verify.argtypes = ([i32, P, P, P, P, P, P, P, i32, P, P]
                                              + [i32] * 5 + [P] * 13 + [i32, P, P])
        L.bole_tree_conv.restype = ctypes.c_int
        L.bole_tree_conv.argtypes = [i32, P, P, P, P, i32, P, P, P, i32, i32, i32, i32, P, P, P]
        L.bole_conv_commit.restype = ctypes.c_int
        L.bole_conv_commit.argtypes = [i32, P, i32, P, P, P, P, P, i32, i32, i32, i32, P, P]
        L.bole_commit_path.restype = ctypes.c_int
        L.bole_commit_path.argtypes = [i32, P, i64, i32, P, i32, P, i64, P, i64, P, i64, P, P,
                                       P, i32, i32, i32, i32, i32, P, P]
        L.bole_forest_workspace_bytes.restype = ctypes.c_size_t
        L.bole_forest_workspace_bytes.argtypes = [i32, i32]
        L.bole_forest_build.restype = ctypes.c_int
        L.bole_forest_build.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.bole_forest_build_noalloc.restype = ctypes.c_int
        L.bole_forest_build_noalloc.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P, P, P, P]
        L.bole_status_string.restype = ctypes.c_char_p
        L.bole_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().bole_status_string(int(code)).decode()


def bole_status_string(code: int) -> str:
    return status_string(code)


def bole_gc_workspace_bytes(B: int, H: int) -> int:
    return int(lib().bole_gc_workspace_bytes(int(B), int(H)))


# ---------------------------------------------------------------------------
# marshalling helpers

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: Optional[torch.Tensor], name: str, dtype=None, ndim=None, allow_none=False,
          contiguous=True):
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, has {t.dim()}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return BOLE_BF16
    if dt == torch.float32:
        return BOLE_F32
    raise ValueError(f"unsupported token dtype {dt}")


def _check(fn: str, code: int):
    if code != 0:
        raise BoleError(fn, code)


# ---------------------------------------------------------------------------
# the four calls

def bole_tree_prep(parent, tree_off, log_gamma, depth, anc, order, tree_depth, logP,
                   err=None, stream=None):
    _need(parent, "parent", torch.int32, 1)
    _need(tree_off, "tree_off", torch.int32, 1)
    N, B = parent.shape[0], tree_off.shape[0] - 1
    L = H = 0
    _need(log_gamma, "log_gamma", torch.float32, 3, allow_none=True)
    if log_gamma is not None:
        L, Ng, H = log_gamma.shape
        if Ng != N:
            raise ValueError("log_gamma must be [L, N, H]")
        _need(logP, "logP", torch.float32, 3)
        if tuple(logP.shape) != tuple(log_gamma.shape):
            raise ValueError("logP must match log_gamma")
    for t, nm, dt, n in ((depth, "depth", torch.int32, N), (anc, "anc", torch.int64, N),
                         (order, "order", torch.int32, N),
                         (tree_depth, "tree_depth", torch.int32, B)):
        _need(t, nm, dt, 1)
        if t.shape[0] != n:
            raise ValueError(f"{nm} must have {n} entries")
    _need(err, "err", torch.int32, 1, allow_none=True)
    _check("bole_tree_prep", lib().bole_tree_prep(
        _ptr(parent), _ptr(tree_off), B, N, _ptr(log_gamma), L, H, _ptr(depth), _ptr(anc),
        _ptr(order), _ptr(tree_depth), _ptr(logP if log_gamma is not None else None),
        _ptr(err), _stream(stream)))


def bole_factor_gc(q, k, logP, beta, anc, order, tree_off, G, C, err=None, stream=None):
    _factor("bole_factor_gc", q, k, logP, beta, anc, order, tree_off, G, C, err, stream)


def bole_factor_inverse(q, k, logP, beta, anc, order, tree_off, W, M, err=None, stream=None):
    """Factor producer of the explicit-inverse solve: W = (I+G)^-1 and M = C W
    in place of G and C (same shapes and layout)."""
    _factor("bole_factor_inverse", q, k, logP, beta, anc, order, tree_off, W, M, err, stream)


def _factor(fn, q, k, logP, beta, anc, order, tree_off, G, C, err, stream):
    _need(q, "q", (torch.float32, torch.bfloat16), 3)
    _need(k, "k", q.dtype, 3)
    N, H, d_k = q.shape
    B = tree_off.shape[0] - 1
    if tuple(k.shape) != (N, H, d_k):
        raise ValueError("k must match q")
    for t, nm in ((logP, "logP"), (beta, "beta")):
        _need(t, nm, torch.float32, 2)
        if tuple(t.shape) != (N, H):
            raise ValueError(f"{nm} must be [N, H]")
    _need(anc, "anc", torch.int64, 1)
    _need(order, "order", torch.int32, 1)
    _need(tree_off, "tree_off", torch.int32, 1)
    if anc.shape[0] != N or order.shape[0] != N:
        raise ValueError("anc and order need N entries")
    for t, nm in ((G, "G"), (C, "C")):
        _need(t, nm, torch.float32, 4)
        if tuple(t.shape) != (B, H, MAX_TREE, MAX_TREE):
            raise ValueError(f"{nm} must be [B, H, 64, 64]")
    _need(err, "err", torch.int32, 1, allow_none=True)
    _check(fn, getattr(lib(), fn)(
        _code(q.dtype), _ptr(q), _ptr(k), _ptr(logP), _ptr(beta), _ptr(anc), _ptr(order),
        _ptr(tree_off), B, N, H, d_k, _ptr(G), _ptr(C), _ptr(err), _stream(stream)))


def bole_verify(q, k, v, logP, beta, state_pool, slot, G, C, order, depth, tree_off, tree_depth,
                O, U, err=None, stream=None):
    _verify("bole_verify", q, k, v, logP, beta, state_pool, slot, G, C, order, depth, tree_off,
            tree_depth, O, U, err, stream)


def bole_verify_neumann(q, k, v, logP, beta, state_pool, slot, G, C, order, depth, tree_off,
                        tree_depth, O, U, err=None, stream=None):
    """bole_verify solving by the d-step Neumann propagation."""
    _verify("bole_verify_neumann", q, k, v, logP, beta, state_pool, slot, G, C, order, depth,
            tree_off, tree_depth, O, U, err, stream)


def bole_verify_inverse(q, k, v, logP, beta, state_pool, slot, W, M, order, depth, tree_off,
                        tree_depth, O, U, err=None, stream=None):
    """bole_verify with W and M from bole_factor_inverse in place of G and C."""
    _verify("bole_verify_inverse", q, k, v, logP, beta, state_pool, slot, W, M, order, depth,
            tree_off, tree_depth, O, U, err, stream)


def _verify(fn, q, k, v, logP, beta, state_pool, slot, G, C, order, depth, tree_off, tree_depth,
            O, U, err, stream):
    _need(q, "q", (torch.float32, torch.bfloat16), 3)
    _need(k, "k", q.dtype, 3)
    _need(v, "v", q.dtype, 3)
    N, H, d_k = q.shape
    d_v = v.shape[2]
    B = tree_off.shape[0] - 1
    if tuple(k.shape) != (N, H, d_k) or tuple(v.shape[:2]) != (N, H):
        raise ValueError("q, k, v shapes disagree")
    for t, nm in ((logP, "logP"), (beta, "beta")):
        _need(t, nm, torch.float32, 2)
        if tuple(t.shape) != (N, H):
            raise ValueError(f"{nm} must be [N, H]")
    _need(state_pool, "state_pool", torch.float32, 4)
    if tuple(state_pool.shape[1:]) != (H, d_v, d_k):
        raise ValueError("state_pool must be [n_slots, H, d_v, d_k]")
    _need(slot, "slot", torch.int32, 1)
    for t, nm in ((G, "G"), (C, "C")):
        _need(t, nm, torch.float32, 4)
        if tuple(t.shape) != (B, H, MAX_TREE, MAX_TREE):
            raise ValueError(f"{nm} must be [B, H, 64, 64]")
    _need(order, "order", torch.int32, 1)
    _need(depth, "depth", torch.int32, 1)
    _need(tree_off, "tree_off", torch.int32, 1)
    _need(tree_depth, "tree_depth", torch.int32, 1)
    if order.shape[0] != N or depth.shape[0] != N:
        raise ValueError("order and depth need N entries")
    _need(O, "O", v.dtype, 3)
    _need(U, "U", torch.float32, 3)
    if tuple(O.shape) != (N, H, d_v) or tuple(U.shape) != (N, H, d_v):
        raise ValueError("O and U must be [N, H, d_v]")
    if slot.shape[0] != B or tree_depth.shape[0] != B:
        raise ValueError("slot and tree_depth need B entries")
    _need(err, "err", torch.int32, 1, allow_none=True)
    _check(fn, getattr(lib(), fn)(
        _code(q.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(logP), _ptr(beta), _ptr(state_pool),
        state_pool.shape[0], _ptr(slot), _ptr(G), _ptr(C), _ptr(order), _ptr(depth),
        _ptr(tree_off), _ptr(tree_depth), B, N, H, d_k, d_v, _ptr(O), _ptr(U), _ptr(err),
        _stream(stream)))


def bole_factor_verify(q, k, v, logP, beta, state_pool, slot, anc, order, depth, tree_off,
                       tree_depth, O, U, err=None, stream=None):
    """bole_factor_gc + bole_verify in one launch (G/C stay on chip)."""
    _need(q, "q", (torch.float32, torch.bfloat16), 3)
    _need(k, "k", q.dtype, 3)
    _need(v, "v", q.dtype, 3)
    N, H, d_k = q.shape
    d_v = v.shape[2]
    B = tree_off.shape[0] - 1
    if tuple(k.shape) != (N, H, d_k) or tuple(v.shape[:2]) != (N, H):
        raise ValueError("q, k, v shapes disagree")
    for t, nm in ((logP, "logP"), (beta, "beta")):
        _need(t, nm, torch.float32, 2)
        if tuple(t.shape) != (N, H):
            raise ValueError(f"{nm} must be [N, H]")
    _need(state_pool, "state_pool", torch.float32, 4)
    if tuple(state_pool.shape[1:]) != (H, d_v, d_k):
        raise ValueError("state_pool must be [n_slots, H, d_v, d_k]")
    _need(slot, "slot", torch.int32, 1)
    _need(anc, "anc", torch.int64, 1)
    _need(order, "order", torch.int32, 1)
    _need(depth, "depth", torch.int32, 1)
    _need(tree_off, "tree_off", torch.int32, 1)
    _need(tree_depth, "tree_depth", torch.int32, 1)
    if anc.shape[0] != N or order.shape[0] != N or depth.shape[0] != N:
        raise ValueError("anc, order and depth need N entries")
    _need(O, "O", v.dtype, 3)
    _need(U, "U", torch.float32, 3)
    if tuple(O.shape) != (N, H, d_v) or tuple(U.shape) != (N, H, d_v):
        raise ValueError("O and U must be [N, H, d_v]")
    if slot.shape[0] != B or tree_depth.shape[0] != B:
        raise ValueError("slot and tree_depth need B entries")
    _need(err, "err", torch.int32, 1, allow_none=True)
    _check("bole_factor_verify", lib().bole_factor_verify(
        _code(q.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(logP), _ptr(beta), _ptr(state_pool),
        state_pool.shape[0], _ptr(slot), _ptr(anc), _ptr(order), _ptr(depth), _ptr(tree_off),
        _ptr(tree_depth), B, N, H, d_k, d_v, _ptr(O), _ptr(U), _ptr(err), _stream(stream)))


def bole_tree_verify(q, k, v, parent, log_gamma, beta, state_pool, slot, tree_off, O, U,
                     depth, anc, order, tree_depth, logP, err=None, stream=None):
    """bole_tree_prep (one layer) + bole_factor_verify in one launch; writes the
    prep outputs (depth, anc, order, tree_depth, this layer's logP) as well."""
    _need(q, "q", (torch.float32, torch.bfloat16), 3)
    _need(k, "k", q.dtype, 3)
    _need(v, "v", q.dtype, 3)
    N, H, d_k = q.shape
    d_v = v.shape[2]
    B = tree_off.shape[0] - 1
    if tuple(k.shape) != (N, H, d_k) or tuple(v.shape[:2]) != (N, H):
        raise ValueError("q, k, v shapes disagree")
    _need(parent, "parent", torch.int32, 1)
    _need(tree_off, "tree_off", torch.int32, 1)
    for t, nm in ((log_gamma, "log_gamma"), (beta, "beta"), (logP, "logP")):
        _need(t, nm, torch.float32, 2)
        if tuple(t.shape) != (N, H):
            raise ValueError(f"{nm} must be [N, H]")
    _need(state_pool, "state_pool", torch.float32, 4)
    if tuple(state_pool.shape[1:]) != (H, d_v, d_k):
        raise ValueError("state_pool must be [n_slots, H, d_v, d_k]")
    _need(slot, "slot", torch.int32, 1)
    _need(anc, "anc", torch.int64, 1)
    _need(order, "order", torch.int32, 1)
    _need(depth, "depth", torch.int32, 1)
    _need(tree_depth, "tree_depth", torch.int32, 1)
    if parent.shape[0] != N or anc.shape[0] != N or order.shape[0] != N or depth.shape[0] != N:
        raise ValueError("parent, anc, order and depth need N entries")
    _need(O, "O", v.dtype, 3)
    _need(U, "U", torch.float32, 3)
    if tuple(O.shape) != (N, H, d_v) or tuple(U.shape) != (N, H, d_v):
        raise ValueError("O and U must be [N, H, d_v]")
    if slot.shape[0] != B or tree_depth.shape[0] != B:
        raise ValueError("slot and tree_depth need B entries")
    _need(err, "err", torch.int32, 1, allow_none=True)
    _check("bole_tree_verify", lib().bole_tree_verify(
        _code(q.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(parent), _ptr(log_gamma), _ptr(beta),
        _ptr(state_pool), state_pool.shape[0], _ptr(slot), _ptr(tree_off), B, N, H, d_k, d_v,
        _ptr(O), _ptr(U), _ptr(depth), _ptr(anc), _ptr(order), _ptr(tree_depth), _ptr(logP),
        _ptr(err), _stream(stream)))


def bole_commit_tree_verify(q, k, v, parent, log_gamma, beta, state_pool, slot, tree_off, O, U,
                            depth, anc, order, tree_depth, logP, prev_k, prev_U, prev_logP,
                            prev_anc, prev_tree_off, prev_accept, err=None, stream=None):
    """The previous round's path commit (prev_*) into the slots, then
    bole_tree_verify of this round, in one launch; state_pool is updated in
    place."""
    _need(q, "q", (torch.float32, torch.bfloat16), 3)
    _need(k, "k", q.dtype, 3)
    _need(v, "v", q.dtype, 3)
    N, H, d_k = q.shape
    d_v = v.shape[2]
    B = tree_off.shape[0] - 1
    if tuple(k.shape) != (N, H, d_k) or tuple(v.shape[:2]) != (N, H):
        raise ValueError("q, k, v shapes disagree")
    _need(parent, "parent", torch.int32, 1)
    _need(tree_off, "tree_off", torch.int32, 1)
    for t, nm in ((log_gamma, "log_gamma"), (beta, "beta"), (logP, "logP")):
        _need(t, nm, torch.float32, 2)
        if tuple(t.shape) != (N, H):
            raise ValueError(f"{nm} must be [N, H]")
    _need(state_pool, "state_pool", torch.float32, 4)
    if tuple(state_pool.shape[1:]) != (H, d_v, d_k):
        raise ValueError("state_pool must be [n_slots, H, d_v, d_k]")
    _need(slot, "slot", torch.int32, 1)
    _need(anc, "anc", torch.int64, 1)
    _need(order, "order", torch.int32, 1)
    _need(depth, "depth", torch.int32, 1)
    _need(tree_depth, "tree_depth", torch.int32, 1)
    if parent.shape[0] != N or anc.shape[0] != N or order.shape[0] != N or depth.shape[0] != N:
        raise ValueError("parent, anc, order and depth need N entries")
    _need(O, "O", v.dtype, 3)
    _need(U, "U", torch.float32, 3)
    if tuple(O.shape) != (N, H, d_v) or tuple(U.shape) != (N, H, d_v):
        raise ValueError("O and U must be [N, H, d_v]")
    if slot.shape[0] != B or tree_depth.shape[0] != B:
        raise ValueError("slot and tree_depth need B entries")
    _need(prev_k, "prev_k", q.dtype, 3)
    N0 = prev_k.shape[0]
    if tuple(prev_k.shape) != (N0, H, d_k):
        raise ValueError("prev_k must be [N0, H, d_k]")
    _need(prev_U, "prev_U", torch.float32, 3)
    if tuple(prev_U.shape) != (N0, H, d_v):
        raise ValueError("prev_U must be [N0, H, d_v]")
    _need(prev_logP, "prev_logP", torch.float32, 2)
    if tuple(prev_logP.shape) != (N0, H):
        raise ValueError("prev_logP must be [N0, H]")
    _need(prev_anc, "prev_anc", torch.int64, 1)
    _need(prev_tree_off, "prev_tree_off", torch.int32, 1)
    _need(prev_accept, "prev_accept", torch.int32, 1)
    if prev_anc.shape[0] != N0 or prev_tree_off.shape[0] != B + 1 or prev_accept.shape[0] != B:
        raise ValueError("prev_anc needs N0 entries, prev_tree_off B+1, prev_accept B")
    _need(err, "err", torch.int32, 1, allow_none=True)
    _check("bole_commit_tree_verify", lib().bole_commit_tree_verify(
        _code(q.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(parent), _ptr(log_gamma), _ptr(beta),
        _ptr(state_pool), state_pool.shape[0], _ptr(slot), _ptr(tree_off), B, N, H, d_k, d_v,
        _ptr(O), _ptr(U), _ptr(depth), _ptr(anc), _ptr(order), _ptr(tree_depth), _ptr(logP),
        _ptr(prev_k), _ptr(prev_U), _ptr(prev_logP), _ptr(prev_anc), _ptr(prev_tree_off),
        _ptr(prev_accept), N0, _ptr(err), _stream(stream)))


def bole_tree_conv(x, weight, bias, conv_state, slot, parent, tree_off, y, err=None,
                   stream=None):
    """Tree-parallel short causal convolution (+ bias, SiLU) of x [N, C]."""
    _need(x, "x", (torch.float32, torch.bfloat16), 2)
    N, C = x.shape
    _need(weight, "weight", torch.float32, 2)
    W = weight.shape[1]
    if weight.shape[0] != C:
        raise ValueError("weight must be [C, W]")
    _need(bias, "bias", torch.float32, 1, allow_none=True)
    if bias is not None and bias.shape[0] != C:
        raise ValueError("bias must be [C]")
    _need(parent, "parent", torch.int32, 1)
    _need(tree_off, "tree_off", torch.int32, 1)
    B = tree_off.shape[0] - 1
    n_slots = 0
    if W > 1:
        _need(conv_state, "conv_state", x.dtype, 3)
        _need(slot, "slot", torch.int32, 1)
        if tuple(conv_state.shape[1:]) != (W - 1, C):
            raise ValueError("conv_state must be [n_slots, W-1, C]")
        if slot.shape[0] != B:
            raise ValueError("slot needs B entries")
        n_slots = conv_state.shape[0]
    _need(y, "y", x.dtype, 2)
    if tuple(y.shape) != (N, C) or parent.shape[0] != N:
        raise ValueError("y must be [N, C] and parent [N]")
    _need(err, "err", torch.int32, 1, allow_none=True)
    _check("bole_tree_conv", lib().bole_tree_conv(
        _code(x.dtype), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state if W > 1 else None),
        n_slots, _ptr(slot if W > 1 else None), _ptr(parent), _ptr(tree_off), B, N, C, W, _ptr(y),
        _ptr(err), _stream(stream)))


def bole_conv_commit(conv_state, slot, x, parent, tree_off, accept, err=None, stream=None):
    """The accepted paths' conv states, in place."""
    _need(x, "x", (torch.float32, torch.bfloat16), 2)
    N, C = x.shape
    _need(conv_state, "conv_state", x.dtype, 3)
    W = conv_state.shape[1] + 1
    if conv_state.shape[2] != C:
        raise ValueError("conv_state must be [n_slots, W-1, C]")
    for t, nm in ((slot, "slot"), (parent, "parent"), (tree_off, "tree_off"), (accept, "accept")):
        _need(t, nm, torch.int32, 1)
    B = tree_off.shape[0] - 1
    if slot.shape[0] != B or accept.shape[0] != B or parent.shape[0] != N:
        raise ValueError("slot and accept need B entries, parent N")
    _need(err, "err", torch.int32, 1, allow_none=True)
    _check("bole_conv_commit", lib().bole_conv_commit(
        _code(x.dtype), _ptr(conv_state), conv_state.shape[0], _ptr(slot), _ptr(x), _ptr(parent),
        _ptr(tree_off), _ptr(accept), B, N, C, W, _ptr(err), _stream(stream)))


def _layer_view(t, name, inner_ndim):
    """Accept [L, *inner] or [*inner] (L = 1); inner dims must be contiguous."""
    if t.dim() == inner_ndim:
        t = t.unsqueeze(0)
    if t.dim() != inner_ndim + 1:
        raise ValueError(f"{name} must have {inner_ndim} or {inner_ndim + 1} dims")
    if not t[0].is_contiguous() and t.shape[0] > 0:
        raise ValueError(f"{name} must be contiguous within a layer")
    return t


def bole_commit_path(state_pool, slot, k, U, logP, anc, tree_off, accept, err=None,
                     stream=None):
    """state_pool [L, n_slots, H, d_v, d_k] (or without L), k [L, N, H, d_k],
    U [L, N, H, d_v], logP [L, N, H]; layer strides are taken from the tensors."""
    sp = _layer_view(state_pool, "state_pool", 4)
    kk = _layer_view(k, "k", 3)
    uu = _layer_view(U, "U", 3)
    lp = _layer_view(logP, "logP", 2)
    _need(sp, "state_pool", torch.float32, contiguous=False)
    _need(kk, "k", (torch.float32, torch.bfloat16), contiguous=False)
    _need(uu, "U", torch.float32, contiguous=False)
    _need(lp, "logP", torch.float32, contiguous=False)
    L, n_slots, H, d_v, d_k = sp.shape
    N = kk.shape[1]
    B = tree_off.shape[0] - 1
    if tuple(kk.shape) != (L, N, H, d_k) or tuple(uu.shape) != (L, N, H, d_v) \
            or tuple(lp.shape) != (L, N, H):
        raise ValueError("k, U, logP must be [L, N, H, ...] matching the state pool")
    for t, nm, dt, n in ((slot, "slot", torch.int32, B), (anc, "anc", torch.int64, N),
                         (tree_off, "tree_off", torch.int32, B + 1),
                         (accept, "accept", torch.int32, B)):
        _need(t, nm, dt, 1)
        if t.shape[0] != n:
            raise ValueError(f"{nm} must have {n} entries")
    _need(err, "err", torch.int32, 1, allow_none=True)
    _check("bole_commit_path", lib().bole_commit_path(
        L, _ptr(sp), sp.stride(0), n_slots, _ptr(slot), _code(kk.dtype), _ptr(kk), kk.stride(0),
        _ptr(uu), uu.stride(0), _ptr(lp), lp.stride(0), _ptr(anc), _ptr(tree_off), _ptr(accept),
        B, N, H, d_k, d_v, _ptr(err), _stream(stream)))


def bole_forest_workspace_bytes(B: int, max_tree: int) -> int:
    return int(lib().bole_forest_workspace_bytes(B, max_tree))


def _forest_args(cand_parent, p_draft, cand_off, capacity, rho, parent, cand_of, tree_off, err):
    _need(cand_parent, "cand_parent", torch.int32, 1)
    _need(p_draft, "p_draft", torch.float32, 1)
    _need(cand_off, "cand_off", torch.int32, 1)
    M_total = cand_parent.shape[0]
    B = cand_off.shape[0] - 1
    if p_draft.shape[0] != M_total:
        raise ValueError("p_draft must match cand_parent")
    _need(rho, "rho", torch.float32, 1)
    if rho.shape[0] != M_total:
        raise ValueError("rho needs M_total entries")
    for t, nm in ((parent, "parent"), (cand_of, "cand_of")):
        _need(t, nm, torch.int32, 1)
        if t.shape[0] != capacity:
            raise ValueError(f"{nm} needs capacity entries")
    _need(tree_off, "tree_off", torch.int32, 1)
    if tree_off.shape[0] != B + 1:
        raise ValueError("tree_off needs B + 1 entries")
    _need(err, "err", torch.int32, 1, allow_none=True)
    return B, M_total


def bole_forest_build(cand_parent, p_draft, cand_off, capacity, max_tree, rho, parent, cand_of,
                      tree_off, workspace, err=None, stream=None):
    """Budget selection by cumulative draft probability and the packed forest
    (see bole.h).  cand_parent [M_total] int32, p_draft [M_total] float32,
    cand_off [B+1] int32; outputs rho [M_total] float32, parent and cand_of
    [capacity] int32, tree_off [B+1] int32; workspace uint8 of at least
    bole_forest_workspace_bytes(B, max_tree) bytes."""
    B, M_total = _forest_args(cand_parent, p_draft, cand_off, capacity, rho, parent, cand_of,
                              tree_off, err)
    _need(workspace, "workspace", torch.uint8, 1)
    if workspace.numel() < bole_forest_workspace_bytes(B, max_tree):
        raise ValueError("workspace too small")
    _check("bole_forest_build", lib().bole_forest_build(
        _ptr(cand_parent), _ptr(p_draft), _ptr(cand_off), B, M_total, int(capacity),
        int(max_tree), _ptr(rho), _ptr(parent), _ptr(cand_of), _ptr(tree_off), _ptr(workspace),
        _ptr(err), _stream(stream)))


def bole_forest_build_noalloc(cand_parent, p_draft, cand_off, capacity, max_tree, rho, parent,
                              cand_of, tree_off, err=None, stream=None):
    """bole_forest_build with the library's own fixed device scratch in place of
    the workspace argument (see bole.h): the same outputs, no allocation."""
    B, M_total = _forest_args(cand_parent, p_draft, cand_off, capacity, rho, parent, cand_of,
                              tree_off, err)
    _check("bole_forest_build_noalloc", lib().bole_forest_build_noalloc(
        _ptr(cand_parent), _ptr(p_draft), _ptr(cand_off), B, M_total, int(capacity),
        int(max_tree), _ptr(rho), _ptr(parent), _ptr(cand_of), _ptr(tree_off), _ptr(err),
        _stream(stream)))
