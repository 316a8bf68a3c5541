"""Tree-parallel short causal convolution: the oracle.

TEST INFRASTRUCTURE ONLY (the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the product library never does).  Plain float64
numpy, one node at a time.

A GDN layer passes its mixed projections through a short causal depthwise
convolution before the recurrence (arXiv page of Bole, section II-A).  The
fused tree pipeline runs it as its first per-layer stage, tree-parallel, with
the bias and SiLU in the same pass; a node's inputs come from its ancestors
(review page, fused-pipeline paragraph; arXiv page, section IV-C).  The pages
give no kernel width, so it is a parameter W.

Reading (stated, since the pages leave it open): node i's window is the last W
entries of the sequence formed by the request's committed conv state (the
W - 1 inputs that preceded the tree, oldest first) followed by the inputs along
i's root-to-node path.  A node therefore sees exactly what ordinary causal
decoding of that path would see.  Every root of a tree starts from the same
committed state.  After acceptance the request's conv state becomes the last
W - 1 entries of the committed state followed by the accepted path's inputs.
"""

from __future__ import annotations

import numpy as np


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def root_path(parent: np.ndarray, off: int, i: int) -> list:
    """Local ids from the root of node i's tree down to i (parents followed up)."""
    path = [i]
    while parent[off + path[-1]] >= 0:
        path.append(int(parent[off + path[-1]]))
        if len(path) > 64:
            raise ValueError("cycle in parent links")
    return path[::-1]


def window(state: np.ndarray, x_path: np.ndarray, W: int) -> np.ndarray:
    """The last W rows of state (W-1 rows) followed by x_path (rows root first)."""
    seq = np.concatenate([state, x_path], axis=0)
    return seq[-W:]


def tree_conv(parent, tree_off, x, weight, bias, conv_state, slot):
    """y[N, C] = silu(bias + sum_j weight[:, j] * window_i[j]) for every node i.

    x [N, C], weight [C, W] (tap j multiplies the j-th oldest entry of the
    window, so tap W-1 multiplies node i's own input), bias [C] or None,
    conv_state [n_slots, W-1, C] (oldest first), slot [B]."""
    x = np.asarray(x, np.float64)
    weight = np.asarray(weight, np.float64)
    C, W = weight.shape
    b_vec = np.zeros(C) if bias is None else np.asarray(bias, np.float64)
    state = np.asarray(conv_state, np.float64)
    assert state.ndim == 3 and state.shape[1:] == (W - 1, C)
    y = np.zeros_like(x)
    for b in range(len(tree_off) - 1):
        off, end = int(tree_off[b]), int(tree_off[b + 1])
        for i in range(end - off):
            path = root_path(parent, off, i)
            win = window(state[slot[b]], x[[off + j for j in path]], W)  # [W, C]
            y[off + i] = silu(b_vec + np.sum(weight.T * win, axis=0))
    return y


def conv_commit(parent, tree_off, x, conv_state, slot, accept):
    """The conv states after acceptance (a copy): slot[b]'s state becomes the
    last W-1 rows of itself followed by the accepted path's inputs; accept[b]
    == -1 leaves it unchanged."""
    x = np.asarray(x, np.float64)
    out = np.array(conv_state, np.float64, copy=True)
    Wm1 = out.shape[1]
    for b in range(len(tree_off) - 1):
        a = int(accept[b])
        if a < 0 or Wm1 == 0:
            continue
        off = int(tree_off[b])
        path = root_path(parent, off, a)
        seq = np.concatenate([out[slot[b]], x[[off + j for j in path]]], axis=0)
        out[slot[b]] = seq[-Wm1:]
    return out
