"""Pins of the tree-convolution oracle (CPU only).

Each pin checks the oracle against something it does not compute itself:
numpy's own convolution routine over explicit token sequences (a chain tree is
ordinary causal decoding; every tree node is the chain of its own root-to-node
path), the pointwise closed form at W = 1, and the commit's definition on
chains and short paths.  Planted mistakes (reversed taps, a window one entry
short, the state ignored, a root that skips the state) must each be caught.
"""

import numpy as np
import pytest

from oracle.tree_conv import conv_commit, silu, tree_conv
import workloads as W


def rand_conv(rng, N, C, Wd, n_slots=3):
    x = rng.standard_normal((N, C))
    w = rng.standard_normal((C, Wd))
    b = rng.standard_normal(C)
    st = rng.standard_normal((n_slots, Wd - 1, C))
    return x, w, b, st


def causal_conv_np(seq, w, b):
    """y[t] for the last len(seq) - (W-1) positions of seq [L, C], per channel
    with numpy's convolve: tap W-1 on the newest entry."""
    Wd = w.shape[1]
    out = np.stack([np.convolve(seq[:, c], w[c, ::-1], mode="valid")
                    for c in range(seq.shape[1])], axis=1)
    assert out.shape[0] == seq.shape[0] - (Wd - 1)
    return silu(out + b)


@pytest.mark.parametrize("Wd", [2, 3, 4, 6])
def test_chain_is_causal_decoding(Wd):
    rng = np.random.default_rng(Wd)
    T, C = 9, 5
    f = W.chain_forest(1, T)
    x, w, b, st = rand_conv(rng, T, C, Wd)
    slot = np.array([2], np.int32)
    y = tree_conv(f.parent, f.tree_off, x, w, b, st, slot)
    ref = causal_conv_np(np.concatenate([st[2], x]), w, b)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_every_node_is_its_path_chain(seed):
    """Several trees (and several roots) in one forest; every node's output is
    numpy's causal convolution of its own explicit token sequence."""
    rng = np.random.default_rng(100 + seed)
    Wd, C = 4, 6
    trees = [W.random_tree(rng, 12, 5), np.array([-1, 0, -1, 2, 1], np.int32),
             np.array([-1], np.int32)]
    f = W.forest_from_trees(trees)
    x, w, b, st = rand_conv(rng, f.N, C, Wd, n_slots=4)
    slot = np.array([3, 0, 1], np.int32)
    y = tree_conv(f.parent, f.tree_off, x, w, b, st, slot)
    for bi in range(f.B):
        off = f.tree_off[bi]
        for i in range(f.tree_off[bi + 1] - off):
            seq, j = [], i
            while j >= 0:                       # explicit sequence: node, parent, ... root
                seq.append(x[off + j])
                j = f.parent[off + j]
            tokens = np.concatenate([st[slot[bi]], np.array(seq[::-1])])
            ref = causal_conv_np(tokens, w, b)[-1]
            assert np.allclose(y[off + i], ref, rtol=1e-13, atol=1e-13)


def test_width_one_is_pointwise():
    rng = np.random.default_rng(3)
    f = W.forest_from_trees([W.random_tree(rng, 10, 4)])
    x, w, b, st = rand_conv(rng, f.N, 7, 1)
    y = tree_conv(f.parent, f.tree_off, x, w, b, st, np.array([0], np.int32))
    z = x * w[:, 0] + b
    assert np.allclose(y, z / (1 + np.exp(-z)), rtol=1e-14)


def test_commit_chain_and_short_paths():
    rng = np.random.default_rng(4)
    Wd, C = 4, 3
    # tree 0: chain of 6, accept the leaf: state = last 3 inputs
    # tree 1: accept a root: state shifts by one entry
    # tree 2: accept -1: unchanged
    trees = [np.arange(-1, 5, dtype=np.int32), np.array([-1, 0, 0], np.int32),
             np.array([-1, 0], np.int32)]
    f = W.forest_from_trees(trees, [5, 0, -1])
    x, w, b, st = rand_conv(rng, f.N, C, Wd, n_slots=3)
    slot = np.array([2, 0, 1], np.int32)
    out = conv_commit(f.parent, f.tree_off, x, st, slot, f.accept)
    assert np.array_equal(out[2], x[3:6])
    assert np.array_equal(out[0], np.concatenate([st[0][1:], x[6:7]]))
    assert np.array_equal(out[1], st[1])


def test_commit_then_conv_is_decoding_the_path():
    """Committing the accepted path and then convolving the next token equals
    decoding the whole sequence at once."""
    rng = np.random.default_rng(5)
    Wd, C, T = 3, 4, 7
    f = W.chain_forest(1, T)
    x, w, b, st = rand_conv(rng, T + 1, C, Wd, n_slots=1)
    f.accept[:] = 3                                   # accept the first four nodes
    new = conv_commit(f.parent, f.tree_off, x[:T], st, np.array([0], np.int32), f.accept)
    nxt = tree_conv(np.array([-1], np.int32), np.array([0, 1], np.int32), x[T:T + 1], w, b, new,
                    np.array([0], np.int32))
    ref = causal_conv_np(np.concatenate([st[0], x[:4], x[T:T + 1]]), w, b)[-1]
    assert np.allclose(nxt[0], ref, rtol=1e-13)


@pytest.mark.parametrize("mutation", ["taps_reversed", "short_window", "no_state", "root_zeros"])
def test_pins_catch_planted_mistakes(mutation):
    rng = np.random.default_rng(6)
    Wd, C, T = 4, 5, 8
    f = W.chain_forest(1, T)
    x, w, b, st = rand_conv(rng, T, C, Wd, n_slots=1)
    slot = np.array([0], np.int32)
    ref = causal_conv_np(np.concatenate([st[0], x]), w, b)
    ww, ss = w.copy(), st.copy()
    if mutation == "taps_reversed":
        ww = w[:, ::-1].copy()
    if mutation == "short_window":
        ww[:, 0] = 0.0
    if mutation in ("no_state", "root_zeros"):
        ss = np.zeros_like(st)
    y = tree_conv(f.parent, f.tree_off, x, ww, b, ss, slot)
    assert np.max(np.abs(y - ref)) > 1e-6
