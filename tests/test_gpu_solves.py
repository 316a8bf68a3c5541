"""GPU parity of the alternative exact solves of (I + G) U = R against the fp64
oracle: bole_verify_neumann (the d-step propagation of Eq. 8) and
bole_factor_inverse + bole_verify_inverse (W = (I+G)^-1 by repeated squaring,
M = C W).  Same bars as the main parity tests; the producer's W and M are
checked against the oracle's Neumann polynomial entry by entry, with their
triangular structure and zero padding exact.  Deep chains (63 propagation
steps, six squaring factors), single-node trees, several roots, head
dimensions that take several staged key chunks, float32 and bf16 tokens.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import (block_rel_err, gpu_round, make_case, oracle_layer, state_rel_err,
                     tolerance)

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)

SOLVES = ["neumann", "inverse"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_round(case, solve, label):
    tol = tolerance(case.cfg)
    out = gpu_round(case, solve=solve)
    assert out["err"] == 0
    O, U, S_new = oracle_layer(case, 0)
    f = case.forest
    units = [(b, h) for b in range(f.B) for h in range(case.cfg.H)]
    eo = block_rel_err(out["O"][0], O, f.tree_off)
    eu = block_rel_err(out["U"][0], U, f.tree_off)
    es = state_rel_err(out["S"][0], S_new, case.slot, units)
    say(f"  {label} {solve}: O {eo:.2e}  U {eu:.2e}  S_new {es:.2e}  (bar {tol:g})")
    assert np.all(np.isfinite(out["O"][0])) and np.all(np.isfinite(out["U"][0]))
    assert eo <= tol and eu <= tol and es <= tol
    return out


@pytest.mark.parametrize("solve", SOLVES)
@pytest.mark.parametrize("name", ["tiny", "decode", "batched", "ragged", "target"])
def test_solve_round_parity(name, solve):
    case = make_case(name, n_layers=1)
    say(f"{solve} round {name} B={case.B} N={case.N} H={case.cfg.H}")
    check_round(case, solve, name)


def edge_cfg(name, cid, dtype, d_k, d_v, H=2):
    return W.Config(name, cid, B=4, H=H, d_k=d_k, d_v=d_v, dtype=dtype, tree="fixed",
                    T=64, D=12, prefix=32)


def deep_forest(seed):
    """A 64-node chain (depth 63), a single node, a tree with several roots and a
    full random tree."""
    rng = np.random.default_rng([seed, 8])
    trees = [np.arange(-1, 63, dtype=np.int32), np.array([-1], np.int32),
             np.array([-1, 0, -1, 2, 1, -1, 5], np.int32), W.random_tree(rng, 64, 12)]
    return W.forest_from_trees(trees, [63, 0, 4, int(rng.integers(64))])


@pytest.mark.parametrize("solve", SOLVES)
@pytest.mark.parametrize("dtype,d_k,d_v", [("bf16", 128, 128), ("f32", 64, 64),
                                           ("f32", 256, 128), ("bf16", 48, 80)])
def test_solve_deep_and_degenerate_trees(dtype, d_k, d_v, solve):
    cfg = edge_cfg(f"solve_{dtype}_{d_k}_{d_v}", 47, dtype, d_k, d_v)
    case = make_case(cfg, forest=deep_forest(3), n_layers=1)
    say(f"{solve} deep trees {dtype} d_k={d_k} d_v={d_v}")
    check_round(case, solve, "deep")


@pytest.mark.parametrize("name", ["tiny", "decode", "ragged"])
def test_factor_inverse_against_oracle(name):
    """W and M per (tree, head) against the oracle's Neumann polynomial of its own
    float64 G and C, in level-order positions."""
    case = make_case(name, n_layers=1)
    say(f"factor_inverse {name}")
    out = gpu_round(case, commit=False, solve="inverse")
    assert out["err"] == 0
    x = case.layers[0]
    f = case.forest
    worst_w = worst_m = 0.0
    for b in range(f.B):
        o, T = f.tree_off[b], f.sizes()[b]
        par = f.parent[o:o + T]
        for h in range(case.cfg.H):
            _, G, C, d = oracle.tree_factors(par, x.q64[o:o + T, h], x.k64[o:o + T, h],
                                             x.g64[o:o + T, h], x.beta64[o:o + T, h])
            Wr, Mr = oracle.inverse_factors(G, C, d)
            lev = np.ix_(out["order"][o:o + T], out["order"][o:o + T])
            Wr, Mr = Wr[lev], Mr[lev]
            Wg, Mg = out["G"][b, h], out["C"][b, h]
            # lower triangular in level order, unit diagonal, zero padding
            assert np.all(np.triu(Wg[:T, :T], 1) == 0) and np.all(np.triu(Mg[:T, :T], 1) == 0)
            assert np.all(np.diag(Wg[:T, :T]) == 1.0)
            assert np.all(Wg[T:] == 0) and np.all(Wg[:, T:] == 0)
            assert np.all(Mg[T:] == 0) and np.all(Mg[:, T:] == 0)
            worst_w = max(worst_w, np.max(np.abs(Wg[:T, :T] - Wr)) / np.max(np.abs(Wr)))
            worst_m = max(worst_m, np.max(np.abs(Mg[:T, :T] - Mr)) / np.max(np.abs(Mr)))
    say(f"  W rel {worst_w:.2e}  M rel {worst_m:.2e}")
    assert worst_w < 1e-4 and worst_m < 1e-4


def test_solves_agree_on_the_target():
    """The three solves of one layer at the target shape agree with each other
    within the bar (each is also checked against the oracle above)."""
    case = make_case("target", n_layers=1)
    tol = tolerance(case.cfg)
    outs = {s: gpu_round(case, commit=False, solve=s) for s in ("blocked", "neumann", "inverse")}
    f = case.forest
    for s in SOLVES:
        du = block_rel_err(outs[s]["U"][0], outs["blocked"]["U"][0], f.tree_off)
        do = block_rel_err(outs[s]["O"][0], outs["blocked"]["O"][0], f.tree_off)
        say(f"  {s} vs blocked: U {du:.2e}  O {do:.2e}")
        assert du <= tol and do <= tol
