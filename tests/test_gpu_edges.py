"""GPU parity on edge shapes and degenerate inputs, against the fp64 oracle.

Head dimensions from 16 to 256 (two value tiles, several staged key chunks,
partial 64-wide commit blocks), single-node trees, a 64-node chain (the deepest
path a tree can hold), trees with several roots, beta = 0 and gates whose
products underflow float32.  Both the two-call path (bole_factor_gc +
bole_verify) and the fused bole_factor_verify run where the latter supports
the shape, and so does bole_tree_verify (preparation inside the launch).  Same
bars as the main parity tests.
"""

import sys

import numpy as np
import pytest

import workloads as W
from helpers import (block_rel_err, gpu_round, make_case, oracle_layer, state_rel_err,
                     tolerance)

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def edge_cfg(name, cid, dtype, d_k, d_v, H=2, D=12, gate_mu=0.0):
    return W.Config(name, cid, B=3, H=H, d_k=d_k, d_v=d_v, dtype=dtype, tree="fixed",
                    T=64, D=D, prefix=32, gate_mu=gate_mu)


def mixed_forest(seed):
    """A single-node tree, a full 64-node tree and a mid-size one."""
    rng = np.random.default_rng([seed, 5])
    trees = [np.array([-1], np.int32), W.random_tree(rng, 64, 12), W.random_tree(rng, 23, 6)]
    accept = [0, int(rng.integers(64)), 22]
    return W.forest_from_trees(trees, accept)


def fused_ok(cfg):
    return cfg.d_k <= (128 if cfg.dtype == "bf16" else 64)


def check(case, fused, label, misalign=False, tree=False):
    tol = tolerance(case.cfg)
    out = gpu_round(case, fused=fused, misalign=misalign, tree=tree)
    assert out["err"] == 0
    O, U, S_new = oracle_layer(case, 0)
    f = case.forest
    units = [(b, h) for b in range(f.B) for h in range(case.cfg.H)]
    eo = block_rel_err(out["O"][0], O, f.tree_off)
    eu = block_rel_err(out["U"][0], U, f.tree_off)
    es = state_rel_err(out["S"][0], S_new, case.slot, units)
    say(f"  {label}{' tree' if tree else ' fused' if fused else ''}: O {eo:.2e}  U {eu:.2e}  "
        f"S_new {es:.2e}")
    assert np.all(np.isfinite(out["O"][0])) and np.all(np.isfinite(out["U"][0]))
    assert eo <= tol and eu <= tol and es <= tol
    return out


SHAPES = [("bf16", 16, 16), ("bf16", 48, 80), ("bf16", 64, 192), ("bf16", 256, 256),
          ("f32", 32, 48), ("f32", 128, 128)]


@pytest.mark.parametrize("dtype,d_k,d_v", SHAPES)
def test_head_dims(dtype, d_k, d_v):
    cfg = edge_cfg(f"dims_{dtype}_{d_k}_{d_v}", 40, dtype, d_k, d_v)
    case = make_case(cfg, forest=mixed_forest(1), n_layers=1)
    say(f"head dims {dtype} d_k={d_k} d_v={d_v}")
    check(case, False, "split")
    if fused_ok(cfg):
        check(case, True, "split")
        check(case, True, "split", tree=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chain_of_64(dtype):
    """Depth 63: the diagonal blocks need every squaring round, and the accepted
    path is 64 long (four K steps in the commit)."""
    cfg = edge_cfg(f"chain_{dtype}", 41, dtype, 64, 64)
    f = W.chain_forest(2, 64)
    f = W.Forest(parent=f.parent, tree_off=f.tree_off, accept=np.array([63, 17], np.int32))
    case = make_case(cfg, forest=f, n_layers=1)
    say(f"chain of 64 {dtype}")
    check(case, False, "split")
    check(case, True, "split")
    check(case, True, "split", tree=True)


def test_several_roots():
    """A tree whose nodes hang from three roots (each root is its own path start)."""
    cfg = edge_cfg("roots", 42, "bf16", 128, 128)
    parent = np.array([-1, 0, -1, 2, 1, -1, 5, 3, 3, 6, 0, 9], np.int32)
    f = W.forest_from_trees([parent, W.random_tree(np.random.default_rng(8), 30, 5)], [9, 29])
    case = make_case(cfg, forest=f, n_layers=1)
    say("several roots")
    check(case, False, "split")
    check(case, True, "split")
    check(case, True, "split", tree=True)


def test_beta_zero():
    """beta = 0: no node writes its state, so U = 0 exactly and O = P q^T S_pre."""
    cfg = edge_cfg("beta0", 43, "bf16", 128, 128)
    case = make_case(cfg, forest=mixed_forest(2), n_layers=1)
    case.layers[0].beta[:] = 0.0
    say("beta = 0")
    out = check(case, True, "fused path")
    assert np.all(out["U"][0] == 0.0)


def test_gate_products_underflow():
    """Gates of -20 per node: P underflows float32 within a few levels (the
    oracle keeps it in float64); ratios along short paths stay representable."""
    cfg = edge_cfg("decay", 44, "bf16", 128, 128)
    case = make_case(cfg, forest=mixed_forest(3), n_layers=1)
    case.layers[0].g[:] = np.float32(-20.0)
    say("gate products underflow")
    check(case, False, "split")
    check(case, True, "split")
    check(case, True, "split", tree=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unaligned_token_buffers(dtype):
    """v, O and U one element past an aligned address: V and the outputs move
    element by element instead of in 16-byte row pieces."""
    cfg = edge_cfg(f"unaligned_{dtype}", 45, dtype, 64, 48)
    case = make_case(cfg, forest=mixed_forest(4), n_layers=1)
    say(f"unaligned token buffers {dtype}")
    check(case, False, "split", misalign=True)
    check(case, True, "split", misalign=True)
    check(case, True, "split", misalign=True, tree=True)
