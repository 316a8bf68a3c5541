"""Measurement baselines: the per-node full-state-snapshot tree verifier the
pages compare Bole against (arXiv page, section V's verification-core
comparison with SGLang-Tree's serial delta-rule verifier).  Not part of
libbole's interface: the benchmark runs it in the same harness as the
closed-form path, and the tests check it against the oracle.

Its kernels are in snapshot.hip, built into libbole_baselines.so beside it,
with stream.hip's plain streaming kernel, the bandwidth ceiling the verify
kernels are set against.
The per-round level lists (nodes grouped by depth, with global parent
indices) are the baseline's own host-side preparation, done once per round.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbole_baselines.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m linear_attention_tree_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        P, i32 = ctypes.c_void_p, ctypes.c_int32
        L.snapshot_level.restype = ctypes.c_int
        L.snapshot_level.argtypes = [i32, P, P, P, P, P, P, P, P, P, P, i32, P, P, P, i32, i32,
                                     i32, P]
        L.snapshot_commit.restype = ctypes.c_int
        L.snapshot_commit.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P]
        L.stream_mix.restype = ctypes.c_int
        L.stream_mix.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, i32, i32, P]
        _lib = L
    return _lib


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    return ctypes.c_void_p((stream or torch.cuda.current_stream()).cuda_stream)


def stream_mix(src, dst, n_read, n_write, grid=2048, block=256, stream=None):
    """One launch of the streaming kernel: n_read 16-byte vectors read from the
    device tensor src, n_write written to dst (grid-stride, non-temporal
    writes)."""
    if n_read * 16 > src.numel() * src.element_size() or \
            n_write * 16 > dst.numel() * dst.element_size():
        raise ValueError("stream_mix: counts exceed the buffers")
    code = lib().stream_mix(_ptr(src), _ptr(dst), n_read, n_write, grid, block, _stream(stream))
    if code != 0:
        raise RuntimeError(f"stream_mix failed: {code}")


def level_lists(parent, tree_off):
    """(levels, parent_node, node_tree) of a packed forest: levels[d] holds the
    global indices of the nodes at depth d; parent_node the global parent of
    each node (-1 for a root); node_tree the tree of each node.  Raises on a
    parent out of range or a cycle."""
    parent = np.asarray(parent, np.int64)
    tree_off = np.asarray(tree_off, np.int64)
    N, B = len(parent), len(tree_off) - 1
    node_tree = np.repeat(np.arange(B), np.diff(tree_off))
    if len(node_tree) != N:
        raise ValueError("tree_off does not cover the nodes")
    size = np.diff(tree_off)[node_tree]
    if np.any(parent < -1) or np.any(parent >= size):
        raise ValueError("parent out of range")
    gpar = np.where(parent < 0, -1, tree_off[node_tree] + parent)
    depth = np.full(N, -1, np.int64)
    depth[gpar < 0] = 0
    for d in range(1, 65):
        todo = (depth < 0) & (gpar >= 0)
        if not todo.any():
            break
        ready = todo & (depth[np.maximum(gpar, 0)] == d - 1)
        depth[ready] = d
    if np.any(depth < 0):
        raise ValueError("cycle in the parent links")
    levels = [np.nonzero(depth == d)[0].astype(np.int32) for d in range(int(depth.max()) + 1)]
    return levels, gpar.astype(np.int32), node_tree.astype(np.int32)


class SnapshotVerifier:
    """Per-node snapshot verification of one packed forest: each layer is one
    launch per tree depth, each node's full float32 state kept in `snap`
    [N, H, d_v, d_k]; commit copies the accepted nodes' states into the slots."""

    def __init__(self, parent, tree_off, H, device="cuda"):
        levels, gpar, ntree = level_lists(parent, tree_off)
        dev = torch.device(device)
        self.H = H
        self.n_levels = len(levels)
        self.level_sizes = [len(x) for x in levels]
        self.levels = [torch.from_numpy(x).to(dev) for x in levels]
        self.parent_node = torch.from_numpy(gpar).to(dev)
        self.node_tree = torch.from_numpy(ntree).to(dev)
        self.tree_off = torch.as_tensor(np.asarray(tree_off, np.int32)).to(dev)

    def layer(self, q, k, v, g, beta, state_pool, slot, snap, O, U, stream=None):
        """One layer: O, U and every node's state from the slots' states."""
        N, H, d_k = q.shape
        d_v = v.shape[2]
        for t in (q, k, v, g, beta, state_pool, snap, O, U):
            if not t.is_contiguous():
                raise ValueError("contiguous tensors expected")
        if snap.shape != (N, H, d_v, d_k) or snap.dtype != torch.float32:
            raise ValueError("snap must be float32 [N, H, d_v, d_k]")
        bf16 = 1 if q.dtype == torch.bfloat16 else 0
        L, st = lib(), _stream(stream)
        for lv, n in zip(self.levels, self.level_sizes):
            code = L.snapshot_level(bf16, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(state_pool), _ptr(slot), _ptr(self.node_tree),
                                    _ptr(self.parent_node), _ptr(lv), n, _ptr(snap), _ptr(O),
                                    _ptr(U), H, d_k, d_v, st)
            if code:
                raise RuntimeError(f"snapshot_level failed: {code}")

    def commit(self, snap, state_pool, slot, accept, stream=None):
        B = self.tree_off.shape[0] - 1
        _, H, d_v, d_k = snap.shape
        code = lib().snapshot_commit(_ptr(snap), _ptr(state_pool), _ptr(slot), _ptr(self.tree_off),
                                     _ptr(accept), B, H, d_k, d_v, _stream(stream))
        if code:
            raise RuntimeError(f"snapshot_commit failed: {code}")
