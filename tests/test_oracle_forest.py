"""Pins of the budget-selection / forest-builder oracle (CPU only).

Each pin checks the oracle against something it does not compute itself: a
hand-worked example with exact binary-fraction probabilities
(tests/golden/forest_small.json), numpy's lexsort as the global ranking when
no per-request limit binds, float64 path products within float32's rounding
bound, the prefix-closure and counting properties the pages state, and the
error cases.  Planted mistakes in a copy of the selection must each fail one
of them.
"""

import json
import os

import numpy as np
import pytest

from oracle import forest as F
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    return json.load(open(os.path.join(HERE, "golden", "forest_small.json")))


def test_golden_hand_worked_example():
    g = golden()
    for case in g["cases"]:
        out = F.build_forest(np.array(g["cand_parent"], np.int32),
                             np.array(g["p_draft"], np.float32), np.array(g["cand_off"]),
                             case["capacity"], case["max_tree"])
        assert out["err"] == 0
        assert np.array_equal(out["rho"], np.array(g["rho"], np.float32))
        assert out["tree_off"].tolist() == case["tree_off"]
        assert out["parent"].tolist() == case["parent"]
        assert out["cand_of"].tolist() == case["cand_of"]


def float64_paths(parent, p):
    """rho in float64 and depth by an explicit parent walk."""
    M = len(parent)
    rho = np.ones(M)
    depth = np.zeros(M, np.int64)
    for i in range(M):
        j = i
        rho[i] = float(p[i])
        while parent[j] >= 0:
            j = parent[j]
            rho[i] *= float(p[j])
            depth[i] += 1
    return rho, depth


@pytest.mark.parametrize("seed", range(3))
def test_rho_is_the_path_product(seed):
    """rho equals the float64 product of the path's probabilities within
    float32's rounding bound (one rounding per factor), and a child never
    exceeds its parent, exactly."""
    c = W.make_candidates(4, seed)
    for b in range(c.B):
        o, e = c.cand_off[b], c.cand_off[b + 1]
        par, p = c.cand_parent[o:e], c.p_draft[o:e]
        rho, depth, err = F.score_tree(par, p)
        assert err == 0
        ref, dref = float64_paths(par, p)
        assert np.array_equal(depth, dref)
        assert np.all(np.abs(rho - ref) <= (depth + 1) * 2.0 ** -24 * ref + 1e-45)
        for i in range(len(par)):
            if par[i] >= 0:
                assert rho[i] <= rho[par[i]]


def test_without_a_tree_limit_selection_is_the_global_top():
    """No per-request limit binding: the selected set is the first `capacity`
    candidates of numpy's lexsort of (rho desc, depth, request, index)."""
    c = W.make_candidates(6, 11)
    rho_all, keys = [], []
    for b in range(c.B):
        o, e = c.cand_off[b], c.cand_off[b + 1]
        rho, depth, _ = F.score_tree(c.cand_parent[o:e], c.p_draft[o:e])
        for i in range(e - o):
            keys.append((-float(rho[i]), depth[i], b, i, o + i))
    k = np.array(keys)
    order = np.lexsort((k[:, 3], k[:, 2], k[:, 1], k[:, 0]))
    for capacity in (6, 50, 200, len(keys)):
        out = F.build_forest(c.cand_parent, c.p_draft, c.cand_off, capacity, 10 ** 6)
        want = set(k[order[:capacity], 4].astype(int).tolist())
        got = set(out["cand_of"][:out["n_nodes"]].tolist())
        assert got == want and out["n_nodes"] == capacity


@pytest.mark.parametrize("capacity,max_tree", [(40, 8), (100, 64), (700, 64), (2000, 64),
                                               (16, 1)])
def test_selection_is_prefix_closed_and_counts_add_up(capacity, max_tree):
    c = W.make_candidates(16, 5)
    out = F.build_forest(c.cand_parent, c.p_draft, c.cand_off, capacity, max_tree)
    sizes = np.diff(out["tree_off"])
    M = np.diff(c.cand_off)
    assert out["n_nodes"] == min(capacity, int(np.sum(np.minimum(M, max_tree))))
    assert np.all(sizes <= max_tree)
    for b in range(c.B):
        o, n = out["tree_off"][b], sizes[b]
        par = out["parent"][o:o + n]
        cand = out["cand_of"][o:o + n]
        if n:
            assert par[0] == -1 and cand[0] == c.cand_off[b]          # the root is node 0
        for j in range(n):
            if j:
                assert 0 <= par[j] < j                                 # parents come first
                assert c.cand_parent[cand[j]] + c.cand_off[b] == cand[par[j]]
    assert np.all(out["parent"][out["n_nodes"]:] == -1)
    assert np.all(out["cand_of"][out["n_nodes"]:] == -1)


def test_equal_scores_fall_to_depth():
    """A child with p = 1 ties its parent's rho; the parent still comes first,
    and a capacity that stops between them takes the parent."""
    par = np.array([-1, 0, 1, 0], np.int32)
    p = np.array([1.0, 1.0, 1.0, 0.5], np.float32)
    for capacity, want in ((1, [0]), (2, [0, 1]), (3, [0, 1, 2])):
        out = F.build_forest(par, p, np.array([0, 4]), capacity, 64)
        assert out["cand_of"][:capacity].tolist() == want


def test_negative_zero_is_a_zero_score():
    """p = -0.0 is a probability of zero: it scores like +0.0, so it ranks below
    every positive score, ties with other zeros fall to depth, and the selection
    stays prefix-closed (the -0.0 child never precedes its root).  The reported
    rho keeps the float32 product's sign."""
    nz = np.float32(-0.0)
    par = np.array([-1, 0, 0], np.int32)
    out = F.build_forest(par, np.array([1.0, nz, 0.5], np.float32), np.array([0, 3]), 2, 64)
    assert out["cand_of"].tolist() == [0, 2] and out["parent"].tolist() == [-1, 0]
    assert np.signbit(out["rho"][1]) and out["rho"][1] == 0.0
    # a -0.0 root: every score is zero, taken level by level (depth, then index)
    par = np.array([-1, 0, 1, 0], np.int32)
    p = np.array([nz, 1.0, 0.5, nz], np.float32)
    out = F.build_forest(par, p, np.array([0, 4]), 3, 64)
    assert out["cand_of"].tolist() == [0, 1, 3] and out["parent"].tolist() == [-1, 0, 0]
    assert out["rho"].view(np.uint32).tolist() == [0x80000000, 0x80000000, 0x80000000, 0]


@pytest.mark.parametrize("bad,bits", [
    (([-1, 0, 7], [1.0, 0.5, 0.5]), F.ERR_BAD_PARENT),
    (([-1, 1, 1], [1.0, 0.5, 0.5]), F.ERR_BAD_PARENT),
    (([-1, 2, 1], [1.0, 0.5, 0.5]), F.ERR_CYCLE),
    (([-1, 0, 1], [1.0, 1.5, 0.5]), F.ERR_BAD_PROB),
    (([-1, 0, 1], [1.0, float("nan"), 0.5]), F.ERR_BAD_PROB),
    (([-1, 0, 1], [1.0, -0.25, 0.5]), F.ERR_BAD_PROB)])
def test_bad_candidate_trees_are_reported_and_skipped(bad, bits):
    good = ([-1, 0, 0], [1.0, 0.5, 0.25])
    par = np.array(good[0] + bad[0] + good[0], np.int32)
    p = np.array(good[1] + bad[1] + good[1], np.float32)
    out = F.build_forest(par, p, np.array([0, 3, 6, 9]), 9, 64)
    assert out["err"] == bits
    assert out["tree_off"].tolist() == [0, 3, 3, 6]
    assert out["cand_of"][:6].tolist() == [0, 1, 2, 6, 7, 8]


def mutated_build(mutation, cand_parent, p_draft, cand_off, capacity, max_tree):
    """A copy of the selection with one planted mistake."""
    B = len(cand_off) - 1
    entries = []
    for b in range(B):
        o, e = cand_off[b], cand_off[b + 1]
        rho, depth, _ = F.score_tree(cand_parent[o:e], p_draft[o:e])
        if mutation == "own_p_only":
            rho = p_draft[o:e].astype(np.float32)
        for i in range(e - o):
            r = float(rho[i])
            key = (r if mutation == "ascending" else -r,
                   -depth[i] if mutation == "deep_first" else depth[i], b, i)
            entries.append((key, b, i))
    entries.sort()
    taken = [[] for _ in range(B)]
    total = 0
    for _, b, i in entries:
        cap_ok = True if mutation == "no_tree_limit" else len(taken[b]) < max_tree
        if total < capacity and cap_ok:
            taken[b].append(cand_off[b] + i)
            total += 1
    return taken


@pytest.mark.parametrize("mutation", ["ascending", "own_p_only", "no_tree_limit", "deep_first"])
def test_pins_catch_planted_mistakes(mutation):
    g = golden()
    par = np.array(g["cand_parent"], np.int32)
    p = np.array(g["p_draft"], np.float32)
    off = np.array(g["cand_off"])
    caught = False
    for case in g["cases"]:
        taken = mutated_build(mutation, par, p, off, case["capacity"], case["max_tree"])
        got = [c for t in taken for c in t]
        want = [c for c in case["cand_of"] if c >= 0]
        caught |= sorted(got) != sorted(want) or got != want
    # equal-score case for the depth tie-break
    par2 = np.array([-1, 0, 1, 0], np.int32)
    p2 = np.array([1.0, 1.0, 1.0, 0.5], np.float32)
    taken = mutated_build(mutation, par2, p2, np.array([0, 4]), 2, 64)
    caught |= taken[0] != [0, 1]
    assert caught
