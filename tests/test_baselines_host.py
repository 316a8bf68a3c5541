"""Host-side preparation of the snapshot baseline (CPU): its level lists
group every node by the depth the oracle's tree preparation gives, with
global parent indices, and it refuses bad parents and cycles."""

import numpy as np
import pytest

import oracle
import workloads as W


def test_level_lists_match_oracle_depths():
    from linear_attention_tree_amd.baselines import level_lists
    for name, seed in (("ragged", 0), ("batched", 1), ("multilayer", 2), ("tiny", 0)):
        f = W.make_forest(W.CONFIGS[name], seed)
        levels, gpar, ntree = level_lists(f.parent, f.tree_off)
        ref = oracle.tree_prep(f.parent, f.tree_off)
        assert ref["err"] == 0
        depth = np.full(f.N, -1)
        for d, nodes in enumerate(levels):
            assert np.all(depth[nodes] == -1)
            depth[nodes] = d
        assert np.array_equal(depth, ref["depth"])
        for b in range(f.B):
            o, e = f.tree_off[b], f.tree_off[b + 1]
            assert np.all(ntree[o:e] == b)
            loc = f.parent[o:e]
            assert np.array_equal(gpar[o:e], np.where(loc < 0, -1, o + loc))


@pytest.mark.parametrize("parent", [[-1, 0, 5], [-1, 2, 1], [-1, -2, 0]])
def test_level_lists_refuse_bad_topology(parent):
    from linear_attention_tree_amd.baselines import level_lists
    with pytest.raises(ValueError):
        level_lists(np.array(parent), np.array([0, 3]))


def test_stream_mix_refuses_bad_arguments():
    """The streaming kernel's argument checks run before any launch (no GPU
    needed): negative counts, launch shapes outside 1..65536 workgroups of a
    multiple of 64 threads up to 1024, and null or misaligned buffers."""
    from linear_attention_tree_amd.baselines import lib
    L = lib()
    buf = (np.zeros(64, np.float32).ctypes.data + 15) // 16 * 16  # 16-byte aligned host address
    ok = dict(src=buf, dst=buf, n_read=1, n_write=1, grid=1, block=64)
    bad = [dict(n_read=-1), dict(n_write=-1), dict(grid=0), dict(grid=65537), dict(block=32),
           dict(block=96), dict(block=2048), dict(src=None), dict(dst=None), dict(src=buf + 4),
           dict(dst=buf + 8)]
    for change in bad:
        a = {**ok, **change}
        assert L.stream_mix(a["src"], a["dst"], a["n_read"], a["n_write"], a["grid"],
                            a["block"], None) == 2, change
    # zero counts need no buffers; they are refused only for a bad launch shape
    assert L.stream_mix(None, None, 0, 0, 0, 64, None) == 2
