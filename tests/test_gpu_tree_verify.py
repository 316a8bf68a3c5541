"""GPU parity of bole_tree_verify: tree preparation inside the verify launch.

Its preparation outputs must be bit-identical to bole_tree_prep (and so to the
oracle's), its O and U bit-identical to bole_tree_prep + bole_factor_verify
(same arithmetic on the same values), and the whole round (with the commit
fed from its outputs) within the usual bars of the fp64 oracle.  Rejected
trees (bad parent, cycle) set the same error bits and tree_depth -1 while the
other trees of the forest are unaffected.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as W

from helpers import (block_rel_err, gpu_round, make_case, oracle_layer, state_rel_err,
                     to_dev, tolerance)

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _prep_of(rnd, logP):
    t = rnd.topo
    return dict(depth=t.depth.cpu().numpy(), anc=t.anc.cpu().numpy().view(np.uint64),
                order=t.order.cpu().numpy(), tree_depth=t.tree_depth.cpu().numpy(),
                logP=logP.cpu().numpy())


def _two_paths(case):
    """(prep + factor_verify) and tree_verify on the same inputs, fresh buffers."""
    from linear_attention_tree_amd import TreeRound
    f = case.forest
    d = to_dev(case, 0)
    pool = torch.from_numpy(case.S_pre[0]).cuda()
    slot = torch.from_numpy(case.slot).cuda()
    ra = TreeRound(f.parent, f.tree_off, case.cfg.H)
    logPa = ra.prep(d["g"][None])[0]
    Oa, Ua = ra.layer(d["q"], d["k"], d["v"], logPa, d["beta"], pool, slot, fused=True)
    rb = TreeRound(f.parent, f.tree_off, case.cfg.H)
    Ob, Ub, logPb = rb.tree_layer(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, slot)
    torch.cuda.synchronize()
    return (ra, logPa, Oa, Ua), (rb, logPb, Ob, Ub)


@pytest.mark.parametrize("name", ["tiny", "decode", "batched", "ragged", "target"])
def test_tree_verify_bit_identical_to_prep_then_fused(name):
    case = make_case(name, n_layers=1)
    f = case.forest
    say(f"tree_verify vs prep + factor_verify {name} B={f.B} N={f.N}")
    (ra, logPa, Oa, Ua), (rb, logPb, Ob, Ub) = _two_paths(case)
    assert ra.error_bits() == 0 and rb.error_bits() == 0
    pa, pb = _prep_of(ra, logPa), _prep_of(rb, logPb)
    for key in ("depth", "anc", "order", "tree_depth"):
        assert np.array_equal(pa[key], pb[key]), key
    assert np.array_equal(pa["logP"].view(np.uint32), pb["logP"].view(np.uint32))
    assert torch.equal(Oa, Ob) and torch.equal(Ua, Ub)
    # and the preparation outputs are the oracle's, bit for bit
    ref = oracle.tree_prep(f.parent, f.tree_off, case.layers[0].g[None])
    for key in ("depth", "anc", "order", "tree_depth"):
        assert np.array_equal(pb[key], ref[key]), key
    assert np.array_equal(pb["logP"].view(np.uint32), ref["logP"][0].view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "batched", "ragged", "target"])
def test_tree_verify_round_parity(name):
    """tree_verify then the commit (fed its anc and logP) against the oracle."""
    case = make_case(name, n_layers=1)
    tol = tolerance(case.cfg)
    say(f"tree_verify + commit {name}")
    out = gpu_round(case, tree=True)
    assert out["err"] == 0
    O, U, S_new = oracle_layer(case, 0)
    f = case.forest
    units = [(b, h) for b in range(f.B) for h in range(case.cfg.H)]
    eo = block_rel_err(out["O"][0], O, f.tree_off)
    eu = block_rel_err(out["U"][0], U, f.tree_off)
    es = state_rel_err(out["S"][0], S_new, case.slot, units)
    say(f"  O {eo:.2e}  U {eu:.2e}  S_new {es:.2e}  (bar {tol:g})")
    assert eo <= tol and eu <= tol and es <= tol


@pytest.mark.parametrize("bad,bits", [("bad_parent", oracle.ERR_BAD_PARENT),
                                      ("cycle", oracle.ERR_CYCLE)])
def test_tree_verify_rejected_tree(bad, bits):
    """A rejected tree is reported and skipped; its neighbours are computed as by
    the two-launch path."""
    rng = np.random.default_rng(11)
    badt = {"bad_parent": np.array([-1, 0, 9, 1], np.int32),
            "cycle": np.array([-1, 2, 3, 1], np.int32)}[bad]
    trees = [W.random_tree(rng, 20, 6), badt, W.random_tree(rng, 31, 8)]
    forest = W.forest_from_trees(trees, [5, 0, 30])
    cfg = W.Config(f"rej_{bad}", 46, B=3, H=2, d_k=64, d_v=64, dtype="bf16", tree="fixed",
                   T=64, D=12, prefix=16)
    case = make_case(cfg, forest=forest, n_layers=1)
    say(f"tree_verify rejected tree: {bad}")
    (ra, logPa, Oa, Ua), (rb, logPb, Ob, Ub) = _two_paths(case)
    assert ra.error_bits() == bits and rb.error_bits() == bits
    assert rb.topo.tree_depth.cpu().numpy()[1] == -1
    f = forest
    for b in (0, 2):
        sl = slice(f.tree_off[b], f.tree_off[b + 1])
        assert torch.equal(Oa[sl], Ob[sl]) and torch.equal(Ua[sl], Ub[sl])
        assert torch.equal(logPa[sl], logPb[sl])
        for key in ("depth", "anc", "order"):
            assert torch.equal(getattr(ra.topo, key)[sl], getattr(rb.topo, key)[sl]), key
