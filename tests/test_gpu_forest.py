"""GPU parity of bole_forest_build (budget selection and the packed forest)
against the oracle: bit-exact rho, parent, cand_of and tree_off, and the same
error bits.  Drafted candidate trees (depth 8, top-k 4) over budgets from
the pages' 128 up to every candidate, per-request limits from 1 to 64, many
requests, 1024-candidate trees and deep chains, tied scores and zero
probabilities, rejected requests, and the packed forest fed straight into
bole_tree_verify.
"""

import json
import os
import sys

import numpy as np
import pytest

import workloads as W
from oracle import forest as OF

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)

HERE = os.path.dirname(os.path.abspath(__file__))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_build(cand_parent, p_draft, cand_off, capacity, max_tree):
    from linear_attention_tree_amd import ForestBuilder
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    fb = ForestBuilder(len(cand_off) - 1, len(cand_parent), capacity, max_tree)
    fb.build(d(np.asarray(cand_parent, np.int32)), d(np.asarray(p_draft, np.float32)),
             d(np.asarray(cand_off, np.int32)))
    torch.cuda.synchronize()
    return dict(rho=fb.rho.cpu().numpy(), parent=fb.parent.cpu().numpy(),
                cand_of=fb.cand_of.cpu().numpy(), tree_off=fb.tree_off.cpu().numpy(),
                err=int(fb.err.item()))


def assert_same(out, ref):
    assert out["err"] == ref["err"]
    assert np.array_equal(out["rho"].view(np.uint32), ref["rho"].view(np.uint32))
    assert np.array_equal(out["tree_off"], ref["tree_off"])
    assert np.array_equal(out["parent"], ref["parent"])
    assert np.array_equal(out["cand_of"], ref["cand_of"])


def test_forest_golden():
    g = json.load(open(os.path.join(HERE, "golden", "forest_small.json")))
    for case in g["cases"]:
        say(f"forest golden capacity={case['capacity']} max_tree={case['max_tree']}")
        out = gpu_build(g["cand_parent"], g["p_draft"], g["cand_off"], case["capacity"],
                        case["max_tree"])
        assert out["err"] == 0
        assert out["rho"].tolist() == g["rho"]
        assert out["tree_off"].tolist() == case["tree_off"]
        assert out["parent"].tolist() == case["parent"]
        assert out["cand_of"].tolist() == case["cand_of"]


@pytest.mark.parametrize("B,capacity,max_tree", [
    (16, 1024, 64), (16, 768, 64), (16, 128, 64), (16, 256, 64), (16, 5000, 64),
    (64, 2048, 32), (1, 64, 64), (300, 600, 8), (40, 40, 1), (256, 4096, 64),
    (4095, 3000, 4)])
def test_forest_matches_oracle(B, capacity, max_tree):
    c = W.make_candidates(B, seed=B + capacity)
    say(f"forest B={B} M_total={c.cand_off[-1]} capacity={capacity} max_tree={max_tree}")
    out = gpu_build(c.cand_parent, c.p_draft, c.cand_off, capacity, max_tree)
    ref = OF.build_forest(c.cand_parent, c.p_draft, c.cand_off, capacity, max_tree)
    assert_same(out, ref)
    say(f"  {int(out['tree_off'][-1])} nodes packed")


def test_forest_large_trees_ties_and_zeros():
    """1024-candidate trees (a random recursive tree and a 1024-deep chain),
    probabilities of exactly 1 (tied scores) and 0, and several roots."""
    rng = np.random.default_rng(21)
    rt = W.random_tree(rng, 1024, 40)
    chain = np.arange(-1, 1023, dtype=np.int32)
    multi = np.array([-1, 0, -1, 2, 2, -1, 5, 6], np.int32)
    trees = [rt, chain, multi]
    probs = [rng.uniform(0.0, 1.0, 1024).astype(np.float32),
             np.where(rng.uniform(size=1024) < 0.5, 1.0,
                      rng.uniform(0.9, 1.0, 1024)).astype(np.float32),
             np.array([1, 1, 0.5, 0, 1, 1, 0.25, 1], np.float32)]
    probs[0][rng.integers(0, 1024, 30)] = 0.0
    probs[0][0] = 1.0
    off = np.zeros(4, np.int32)
    off[1:] = np.cumsum([len(t) for t in trees])
    par, p = np.concatenate(trees), np.concatenate(probs)
    for capacity, max_tree in ((100, 64), (140, 64), (2056, 64), (30, 10)):
        say(f"forest large trees capacity={capacity} max_tree={max_tree}")
        assert_same(gpu_build(par, p, off, capacity, max_tree),
                    OF.build_forest(par, p, off, capacity, max_tree))


def test_forest_negative_zero_probabilities():
    """A draft probability of -0.0 is a valid zero: its score ranks as +0.0 (then
    by depth), below every positive score, while the reported rho keeps the
    product's sign bit.  At a root (so the whole tree scores -0.0, and a -0.0
    child of it +0.0), at inner nodes, and beside ordinary requests; bit-exact
    against the oracle, at capacities that cut through the zero scores."""
    nz = np.float32(-0.0)
    trees = [
        (np.array([-1, 0, 0], np.int32), np.array([1.0, nz, 0.5], np.float32)),
        (np.array([-1, 0, 1, 0, 3], np.int32), np.array([nz, 1.0, 0.5, nz, 0.25], np.float32)),
        (np.array([-1, 0, 0, 1, 2, 2], np.int32),
         np.array([1.0, 0.75, nz, nz, 0.0, 0.5], np.float32)),
    ]
    good = W.make_candidates(2, seed=11)
    par = np.concatenate([t[0] for t in trees] + [good.cand_parent]).astype(np.int32)
    p = np.concatenate([t[1] for t in trees] + [good.p_draft]).astype(np.float32)
    off = np.concatenate([[0], np.cumsum([len(t[0]) for t in trees]),
                          sum(len(t[0]) for t in trees) + good.cand_off[1:]]).astype(np.int32)
    for capacity in (2, 4, 8, 12, 40, len(par)):
        for max_tree in (2, 64):
            say(f"forest -0.0: capacity={capacity} max_tree={max_tree}")
            out = gpu_build(par, p, off, capacity, max_tree)
            ref = OF.build_forest(par, p, off, capacity, max_tree)
            assert ref["err"] == 0
            assert_same(out, ref)
    # the smallest case on its own: the -0.0 child does not outrank its root
    out = gpu_build(trees[0][0], trees[0][1], np.array([0, 3], np.int32), 2, 64)
    assert out["err"] == 0
    assert out["cand_of"].tolist() == [0, 2] and out["parent"].tolist() == [-1, 0]


@pytest.mark.parametrize("bad,bits", [
    (([-1, 0, 7], [1.0, 0.5, 0.5]), OF.ERR_BAD_PARENT),
    (([-1, 1, 1], [1.0, 0.5, 0.5]), OF.ERR_BAD_PARENT),
    (([-1, 2, 1], [1.0, 0.5, 0.5]), OF.ERR_CYCLE),
    (([-1, 0, 1], [1.0, 1.5, 0.5]), OF.ERR_BAD_PROB),
    (([-1, 0, 1], [1.0, float("nan"), 0.5]), OF.ERR_BAD_PROB),
    (([-1, 0, 1], [1.0, -0.25, 0.5]), OF.ERR_BAD_PROB)])
def test_forest_rejected_request(bad, bits):
    good = W.make_candidates(2, seed=3)
    g0 = good.cand_parent[:good.cand_off[1]], good.p_draft[:good.cand_off[1]]
    g1 = good.cand_parent[good.cand_off[1]:], good.p_draft[good.cand_off[1]:]
    par = np.concatenate([g0[0], np.array(bad[0], np.int32), g1[0]]).astype(np.int32)
    p = np.concatenate([g0[1], np.array(bad[1], np.float32), g1[1]]).astype(np.float32)
    off = np.array([0, len(g0[0]), len(g0[0]) + 3, len(par)], np.int32)
    say(f"forest rejected request: bits {bits}")
    out = gpu_build(par, p, off, 100, 64)
    ref = OF.build_forest(par, p, off, 100, 64)
    assert out["err"] == ref["err"] == bits
    assert out["tree_off"][2] == out["tree_off"][1]
    assert_same(out, ref)


def test_forest_oversized_request_is_rejected():
    """More than 1024 candidates in one request: TREE_SIZE, no node from it; the
    other requests are packed as if it had none."""
    c = W.make_candidates(3, seed=4)
    big = np.concatenate([np.array([-1], np.int32), np.zeros(1100, np.int32)])
    pb = np.full(1101, 0.5, np.float32)
    pb[0] = 1.0
    o1 = c.cand_off[1]
    par = np.concatenate([c.cand_parent[:o1], big, c.cand_parent[o1:]]).astype(np.int32)
    p = np.concatenate([c.p_draft[:o1], pb, c.p_draft[o1:]]).astype(np.float32)
    off = np.concatenate([[0, o1, o1 + 1101], 1101 + c.cand_off[2:]]).astype(np.int32)
    out = gpu_build(par, p, off, 200, 64)
    assert out["err"] == 4
    # the oracle on the same requests with the oversized one emptied
    par2 = np.concatenate([c.cand_parent[:o1], c.cand_parent[o1:]])
    p2 = np.concatenate([c.p_draft[:o1], c.p_draft[o1:]])
    off2 = np.concatenate([[0, o1, o1], c.cand_off[2:]]).astype(np.int32)
    ref = OF.build_forest(par2, p2, off2, 200, 64)
    assert np.array_equal(out["tree_off"], ref["tree_off"])
    assert np.array_equal(out["parent"], ref["parent"])
    shift = np.where(ref["cand_of"] >= o1, ref["cand_of"] + 1101, ref["cand_of"])
    assert np.array_equal(out["cand_of"], np.where(ref["cand_of"] < 0, -1, shift))


def test_forest_feeds_tree_verify():
    """The packed forest (capacity-sized buffers, unused slots -1) goes straight
    into bole_tree_verify and the commit; the round matches the oracle run on
    the same packed trees."""
    from helpers import block_rel_err, make_case, oracle_layer, state_rel_err, tolerance
    cfg = W.Config("forest_round", 48, B=8, H=4, d_k=128, d_v=128, dtype="bf16", tree="fixed",
                   T=64, D=12, prefix=64)
    c = W.make_candidates(cfg.B, seed=8)
    capacity = 300
    out = gpu_build(c.cand_parent, c.p_draft, c.cand_off, capacity, 64)
    assert out["err"] == 0
    n = int(out["tree_off"][-1])
    assert n == capacity
    rng = np.random.default_rng(5)
    sizes = np.diff(out["tree_off"])
    accept = np.array([int(rng.integers(s)) for s in sizes], np.int32)
    forest = W.Forest(parent=out["parent"][:n].copy(), tree_off=out["tree_off"].copy(),
                      accept=accept)
    case = make_case(cfg, forest=forest, n_layers=1)
    from helpers import gpu_round
    res = gpu_round(case, tree=True)
    assert res["err"] == 0
    O, U, S_new = oracle_layer(case, 0)
    tol = tolerance(cfg)
    units = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    eo = block_rel_err(res["O"][0], O, forest.tree_off)
    eu = block_rel_err(res["U"][0], U, forest.tree_off)
    es = state_rel_err(res["S"][0], S_new, case.slot, units)
    say(f"  forest round: O {eo:.2e}  U {eu:.2e}  S_new {es:.2e}")
    assert eo <= tol and eu <= tol and es <= tol
