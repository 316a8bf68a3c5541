"""GPU parity of the tree convolution (bole_tree_conv) and its conv-state
commit (bole_conv_commit) against the fp64 oracle.

The convolution is compared per tree (max|y - ref| / max|ref| over the tree's
rows): 1e-4 for float32 inputs, 2e-2 for bf16 (whose output is rounded to
bf16).  The commit only moves stored values, so it must match bit for bit.
Widths 1 to 8, ragged channel blocks, deep chains, several roots, single-node
trees, a missing bias, and rejected trees.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tok(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def run(cfg, forest, C, Wd, with_bias=True, n_extra=2):
    from linear_attention_tree_amd import bole
    n_slots = forest.B + n_extra
    ci = W.make_conv(cfg, forest.N, n_slots, C=C, W=Wd)
    slot = np.random.default_rng(C + Wd).permutation(n_slots)[:forest.B].astype(np.int32)
    x = dev_tok(ci.x, cfg.dtype)
    st = dev_tok(ci.state, cfg.dtype)
    y = torch.empty_like(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    bias = d(ci.bias) if with_bias else None
    bole.bole_tree_conv(x, d(ci.weight), bias, st, d(slot), d(forest.parent), d(forest.tree_off),
                        y, err)
    bole.bole_conv_commit(st, d(slot), x, d(forest.parent), d(forest.tree_off),
                          d(forest.accept), err)
    torch.cuda.synchronize()
    ref = oracle.tree_conv(forest.parent, forest.tree_off, ci.x64, ci.weight,
                           ci.bias if with_bias else None, ci.state64, slot)
    ref_st = oracle.conv_commit(forest.parent, forest.tree_off, ci.x64, ci.state64, slot,
                                forest.accept)
    return dict(y=y.float().cpu().numpy().astype(np.float64), ref=ref,
                st=st.float().cpu().numpy().astype(np.float64), ref_st=ref_st,
                err=int(err.item()))


def tree_err(y, ref, tree_off, trees=None):
    worst = 0.0
    for b in (range(len(tree_off) - 1) if trees is None else trees):
        sl = slice(tree_off[b], tree_off[b + 1])
        scale = np.max(np.abs(ref[sl]))
        worst = max(worst, np.max(np.abs(y[sl] - ref[sl])) / scale)
    return worst


def conv_cfg(dtype):
    return W.Config(f"conv_{dtype}", 50, B=16, H=4, d_k=32, d_v=32, dtype=dtype, tree="fixed",
                    T=64, D=12, prefix=0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Wd", [1, 2, 3, 4, 5, 6, 7, 8])  # each width is its own instantiation
def test_tree_conv_parity(dtype, Wd):
    cfg = conv_cfg(dtype)
    forest = W.make_forest(W.CONFIGS["target"], seed=Wd)
    C = 392  # not a multiple of the channel block: a ragged last block
    say(f"tree conv {dtype} W={Wd} N={forest.N} C={C}")
    out = run(cfg, forest, C, Wd)
    tol = 1e-4 if dtype == "f32" else 2e-2
    e = tree_err(out["y"], out["ref"], forest.tree_off)
    say(f"  y {e:.2e} (bar {tol:g})")
    assert out["err"] == 0
    assert e <= tol
    assert np.array_equal(out["st"], out["ref_st"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tree_conv_shapes(dtype):
    """Chains of 64, several roots, single-node trees, no bias, accept -1."""
    cfg = conv_cfg(dtype)
    rng = np.random.default_rng(9)
    trees = [np.arange(-1, 63, dtype=np.int32), np.array([-1, 0, -1, 2, 1, -1], np.int32),
             np.array([-1], np.int32), W.random_tree(rng, 40, 12)]
    forest = W.forest_from_trees(trees, [63, 4, -1, 17])
    for Wd in (3, 8):
        say(f"tree conv shapes {dtype} W={Wd}")
        out = run(cfg, forest, 64, Wd, with_bias=False)
        tol = 1e-4 if dtype == "f32" else 2e-2
        e = tree_err(out["y"], out["ref"], forest.tree_off)
        say(f"  y {e:.2e}")
        assert out["err"] == 0 and e <= tol
        assert np.array_equal(out["st"], out["ref_st"])


@pytest.mark.parametrize("bad,bits", [("bad_parent", oracle.ERR_BAD_PARENT),
                                      ("cycle", oracle.ERR_CYCLE)])
def test_tree_conv_rejected_tree(bad, bits):
    cfg = conv_cfg("bf16")
    badt = {"bad_parent": np.array([-1, 0, 9, 1], np.int32),
            "cycle": np.array([-1, 2, 3, 1], np.int32)}[bad]
    rng = np.random.default_rng(10)
    good = [W.random_tree(rng, 20, 6), W.random_tree(rng, 31, 8)]
    forest = W.forest_from_trees([good[0], badt, good[1]], [5, 0, 30])
    from linear_attention_tree_amd import bole
    ci = W.make_conv(cfg, forest.N, 3, C=64, W=4)
    say(f"tree conv rejected: {bad}")
    x = dev_tok(ci.x, "bf16")
    st = dev_tok(ci.state, "bf16")
    st0 = st.clone()
    y = torch.zeros_like(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    slot = np.array([0, 1, 2], np.int32)
    bole.bole_tree_conv(x, d(ci.weight), d(ci.bias), st, d(slot), d(forest.parent),
                        d(forest.tree_off), y, err)
    bole.bole_conv_commit(st, d(slot), x, d(forest.parent), d(forest.tree_off),
                          d(forest.accept), err)
    torch.cuda.synchronize()
    assert int(err.item()) == bits
    assert torch.equal(st[1], st0[1])  # the rejected tree's slot is untouched
    # good trees: against the oracle on a forest without the bad tree
    fg = W.forest_from_trees(good, [5, 30])
    keep = np.r_[forest.tree_off[0]:forest.tree_off[1], forest.tree_off[2]:forest.tree_off[3]]
    ref = oracle.tree_conv(fg.parent, fg.tree_off, ci.x64[keep], ci.weight, ci.bias,
                           ci.state64, np.array([0, 2], np.int32))
    yk = y.float().cpu().numpy().astype(np.float64)[keep]
    assert tree_err(yk, ref, fg.tree_off) <= 2e-2


def test_tree_conv_target_shape():
    """The benchmarked launch: the target forest (16 trees x 64 nodes), the mixed
    q/k/v projection's 12288 channels, width 4, bf16; every output against the
    oracle, and the commit bit for bit."""
    cfg = W.CONFIGS["target"]
    forest = W.make_forest(cfg, seed=0)
    C = W.conv_channels(cfg)
    say(f"tree conv target shape: N={forest.N} C={C} W={W.CONV_WIDTH}")
    out = run(cfg, forest, C, W.CONV_WIDTH)
    e = tree_err(out["y"], out["ref"], forest.tree_off)
    say(f"  y {e:.2e} (bar 0.02)")
    assert out["err"] == 0 and e <= 2e-2
    assert np.array_equal(out["st"], out["ref_st"])
