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
