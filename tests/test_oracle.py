"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each check names what it pins.  Sources: Bole, arXiv 2608.01651 (Lemmas 1-3,
Theorem 1, Eq. 10) and the xllm-io review of it (Eqs. 1, 2, 4-6, 10 in LaTeX).
"""

import itertools
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle.closed_form import closed_form_tree, commit_closed_form, inverse_factors, tree_factors
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def rand_inputs(rng, T, dk, dv, gate_mu=0.0):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    x = rng.standard_normal(T) + gate_mu
    g = -np.logaddexp(0.0, x)
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S = rng.standard_normal((dv, dk)) * 0.3
    return q, k, v, g, beta, S


def walk_one(parent, q, k, v, g, beta, S, accept=None):
    """Oracle walk for a single tree / head via the C library."""
    T = len(parent)
    acc = None if accept is None else np.array([accept], np.int32)
    O, U, Sn = oracle.verify(np.asarray(parent, np.int32), np.array([0, T], np.int32),
                             q[:, None, :], k[:, None, :], v[:, None, :], g[:, None],
                             beta[:, None], S[None, None], np.zeros(1, np.int32), accept=acc)
    return O[:, 0], U[:, 0], (None if Sn is None else Sn[0, 0])


def parent_first_trees(T):
    """Every labelled tree on T nodes whose parents precede children."""
    for choice in itertools.product(*[range(i) for i in range(1, T)]):
        yield np.array([-1, *choice], dtype=np.int32)


# ---------------------------------------------------------------------------
# Eq. 1 itself

def test_sequential_matches_textbook_gated_delta_rule():
    """Pins Eq. 1 (sign of the delta term, transposition of S, where gamma and
    beta enter) against the gated delta rule in product form,
    S_t = gamma_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T  (slot layout),
    o_t = S_t q_t: a different algebraic arrangement of the same update."""
    rng = np.random.default_rng(1)
    n, dk, dv = 20, 8, 6
    q, k, v, g, beta, S0 = rand_inputs(rng, n, dk, dv)
    S_fin, o, u = oracle.sequential(S0, q, k, v, g, beta)
    S = S0.copy()
    for t in range(n):
        S = np.exp(g[t]) * S @ (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) \
            + beta[t] * np.outer(v[t], k[t])
        assert rel(o[t], S @ q[t]) < 1e-12
    assert rel(S_fin, S) < 1e-12


def test_hand_worked_scalar_tree():
    """Pins the walk, the closed form and Eq. 10 to a hand-derived example."""
    gd = json.load(open(os.path.join(GOLD, "scalar_tree.json")))
    parent = np.array(gd["parent"], np.int32)
    g = np.log(np.array(gd["gamma"]))
    beta = np.array(gd["beta"])
    k = np.array(gd["k"])[:, None]
    v = np.array(gd["v"])[:, None]
    q = np.array(gd["q"])[:, None]
    S = np.array([[gd["S_pre"]]])
    O, U, _ = walk_one(parent, q, k, v, g, beta, S)
    np.testing.assert_allclose(O[:, 0], gd["O"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(U[:, 0], gd["U"], rtol=1e-14, atol=1e-14)
    cf = closed_form_tree(parent, q, k, v, g, beta, S)
    np.testing.assert_allclose(cf["O"][:, 0], gd["O"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(cf["P"], gd["P"], rtol=1e-14)
    np.testing.assert_allclose(cf["G"], gd["G"], rtol=1e-14, atol=1e-15)
    for a, s in gd["S_new"].items():
        _, _, Sn = walk_one(parent, q, k, v, g, beta, S, accept=int(a))
        assert abs(Sn[0, 0] - s) < 1e-14
        Sc = commit_closed_form(parent, int(a), k, cf["U"], cf["P"], S)
        assert abs(Sc[0, 0] - s) < 1e-14


# ---------------------------------------------------------------------------
# the five checks

def test_chain_tree_is_token_order_decoding():
    """Check 1: a chain tree reproduces ordinary token-order decoding, bit for bit
    (same float64 operation sequence; the oracle is built with -ffp-contract=off)."""
    rng = np.random.default_rng(2)
    T, dk, dv = 12, 16, 16
    q, k, v, g, beta, S = rand_inputs(rng, T, dk, dv)
    parent = np.arange(-1, T - 1, dtype=np.int32)
    O, U, Sn = walk_one(parent, q, k, v, g, beta, S, accept=T - 1)
    S_fin, o, u = oracle.sequential(S, q, k, v, g, beta)
    assert np.array_equal(O, o)
    assert np.array_equal(U, u)
    assert np.array_equal(Sn, S_fin)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6])
def test_closed_form_equals_walk_all_small_trees(T):
    """Check 2a: Theorem 1 (explicit G, C, R, B0, Neumann series) equals sequential
    tree execution on every parent-first labelled tree with T <= 6 nodes."""
    rng = np.random.default_rng(10 + T)
    dk, dv = 5, 4
    for parent in parent_first_trees(T):
        q, k, v, g, beta, S = rand_inputs(rng, T, dk, dv)
        O, U, _ = walk_one(parent, q, k, v, g, beta, S)
        cf = closed_form_tree(parent, q, k, v, g, beta, S)
        assert rel(cf["U"], U) < 1e-12, parent
        assert rel(cf["O"], O) < 1e-12, parent


def test_closed_form_equals_walk_random_trees_and_library_solve():
    """Check 2b: 200 random trees with T <= 16, depth up to 15.  U from the
    Neumann series is also compared with scipy's unit-lower-triangular solve of
    (I + G) U = R in level order (Lemma 2 against a library routine)."""
    rng = np.random.default_rng(3)
    for it in range(200):
        T = int(rng.integers(1, 17))
        D = int(rng.integers(1, 16))
        parent = W.random_tree(rng, T, D)
        if it % 3 == 0:           # shuffle labels: parents need not precede children
            perm = rng.permutation(T)
            inv = np.argsort(perm)
            parent = np.array([-1 if parent[perm[i]] < 0 else inv[parent[perm[i]]]
                               for i in range(T)], np.int32)
        q, k, v, g, beta, S = rand_inputs(rng, T, 6, 5, gate_mu=float(rng.normal()))
        O, U, _ = walk_one(parent, q, k, v, g, beta, S)
        cf = closed_form_tree(parent, q, k, v, g, beta, S)
        assert rel(cf["U"], U) < 1e-12
        assert rel(cf["O"], O) < 1e-12
        prep = oracle.tree_prep(parent, np.array([0, T], np.int32))
        order = prep["order"]
        Gl = cf["G"][np.ix_(order, order)]
        Rl = cf["R"][order]
        Ul = scipy.linalg.solve_triangular(np.eye(T) + Gl, Rl, lower=True, unit_diagonal=True)
        assert rel(Ul, U[order]) < 1e-12


def test_nilpotency_depth_bound():
    """Check 3 (Lemma 3): G^(d+1) = 0 exactly, while G^d is nonzero on the row of
    the deepest node (generic data), with d the maximum strict-ancestor count."""
    rng = np.random.default_rng(4)
    for _ in range(50):
        T = int(rng.integers(2, 33))
        parent = W.random_tree(rng, T, int(rng.integers(1, 12)))
        q, k, v, g, beta, S = rand_inputs(rng, T, 8, 4)
        P, G, C, d = tree_factors(parent, q, k, g, beta)
        prep = oracle.tree_prep(parent, np.array([0, T], np.int32))
        assert d == prep["tree_depth"][0]
        Gd = np.linalg.matrix_power(G, d)
        Gd1 = Gd @ G
        assert np.all(Gd1 == 0.0)
        deepest = int(np.argmax(prep["depth"]))
        assert np.any(Gd[deepest] != 0.0)


def test_unit_determinant():
    """Check 4 (arXiv page, Theorem 1 discussion: I+G is unit lower triangular, det = 1):
    in level order the strict upper part is exactly 0 and the diagonal exactly 1."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        T = int(rng.integers(1, 40))
        parent = W.random_tree(rng, T, int(rng.integers(1, 16)))
        q, k, v, g, beta, S = rand_inputs(rng, T, 8, 4)
        _, G, _, _ = tree_factors(parent, q, k, g, beta)
        order = oracle.tree_prep(parent, np.array([0, T], np.int32))["order"]
        M = np.eye(T) + G[np.ix_(order, order)]
        assert np.all(np.triu(M, 1) == 0.0)
        assert np.all(np.diag(M) == 1.0)
        assert abs(np.linalg.det(M) - 1.0) < 1e-12


def test_inverse_factors_against_library_inverse():
    """The explicit-inverse factors: W from the finite Neumann polynomial equals
    scipy's unit-lower-triangular solve of (I + G) W = I in level order (a
    library routine), W (I + G) = I, and W R, B0 + M R reproduce U and O of
    the walk (Lemma 3 and Eq. 2 with the inverse formed first)."""
    rng = np.random.default_rng(12)
    for _ in range(60):
        T = int(rng.integers(1, 33))
        parent = W.random_tree(rng, T, int(rng.integers(1, 16)))
        q, k, v, g, beta, S = rand_inputs(rng, T, 8, 5, gate_mu=float(rng.normal()))
        cf = closed_form_tree(parent, q, k, v, g, beta, S)
        Wm, M = inverse_factors(cf["G"], cf["C"], cf["d"])
        order = oracle.tree_prep(parent, np.array([0, T], np.int32))["order"]
        lev = np.ix_(order, order)
        Wl = scipy.linalg.solve_triangular(np.eye(T) + cf["G"][lev], np.eye(T), lower=True,
                                           unit_diagonal=True)
        assert rel(Wm[lev], Wl) < 1e-12
        assert rel(Wm @ (np.eye(T) + cf["G"]), np.eye(T)) < 1e-12
        O, U, _ = walk_one(parent, q, k, v, g, beta, S)
        assert rel(Wm @ cf["R"], U) < 1e-12
        assert rel(cf["B0"] + M @ cf["R"], O) < 1e-12


def test_inverse_factors_catch_a_short_polynomial():
    """One Neumann term short (sum to d - 1) misses W on a chain of depth d.
    Nearly parallel keys, beta near 1 and gates near 1 make every G entry of
    order 1, so the dropped term (-G)^d is of order 1 too."""
    rng = np.random.default_rng(13)
    T = 9
    parent = np.arange(-1, T - 1, dtype=np.int32)
    q, k, v, g, beta, S = rand_inputs(rng, T, 8, 5)
    k = np.ones((T, 8)) + 0.1 * rng.standard_normal((T, 8))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    g = np.full(T, -0.01)
    beta = np.full(T, 0.9)
    cf = closed_form_tree(parent, q, k, v, g, beta, S)
    assert cf["d"] == T - 1
    W_full, _ = inverse_factors(cf["G"], cf["C"], cf["d"])
    W_short, _ = inverse_factors(cf["G"], cf["C"], cf["d"] - 1)
    ref = scipy.linalg.solve_triangular(np.eye(T) + cf["G"], np.eye(T), lower=True,
                                        unit_diagonal=True)
    assert rel(W_full, ref) < 1e-12
    assert rel(W_short, ref) > 1e-3


def test_reconstructed_state_every_node():
    """Check 5 (Lemma 1 / Eq. 10): P_a S_pre + (D_a K_a)^T U_a equals the walked
    state after node a, for every node a of random trees."""
    rng = np.random.default_rng(6)
    for _ in range(15):
        T = int(rng.integers(1, 20))
        parent = W.random_tree(rng, T, int(rng.integers(1, 10)))
        q, k, v, g, beta, S = rand_inputs(rng, T, 7, 5)
        cf = closed_form_tree(parent, q, k, v, g, beta, S)
        for a in range(T):
            _, _, Sa = walk_one(parent, q, k, v, g, beta, S, accept=a)
            Sc = commit_closed_form(parent, a, k, cf["U"], cf["P"], S)
            assert rel(Sc, Sa) < 1e-12


# ---------------------------------------------------------------------------
# special cases with closed forms

def test_zero_beta_is_pure_decay():
    """beta = 0: no writes, u = 0 and o_i = P_i S_pre^T q_i."""
    rng = np.random.default_rng(7)
    T = 9
    parent = W.random_tree(rng, T, 4)
    q, k, v, g, beta, S = rand_inputs(rng, T, 6, 5)
    beta[:] = 0.0
    O, U, _ = walk_one(parent, q, k, v, g, beta, S)
    assert np.all(U == 0.0)
    logp = np.zeros(T)
    for i in range(T):
        x = i
        while x >= 0:
            logp[i] += g[x]
            x = parent[x]
    assert rel(O, np.exp(logp)[:, None] * (q @ S.T)) < 1e-13


def test_single_node_is_one_step():
    """T = 1: one recurrence step, u = beta (v - gamma S^T k), o = (gamma S + u k^T) q."""
    rng = np.random.default_rng(8)
    q, k, v, g, beta, S = rand_inputs(rng, 1, 6, 4)
    O, U, Sn = walk_one(np.array([-1], np.int32), q, k, v, g, beta, S, accept=0)
    gam = np.exp(g[0])
    u = beta[0] * (v[0] - gam * S @ k[0])
    assert rel(U[0], u) < 1e-13
    assert rel(Sn, gam * S + np.outer(u, k[0])) < 1e-13
    assert rel(O[0], (gam * S + np.outer(u, k[0])) @ q[0]) < 1e-13


def test_orthogonal_keys_give_zero_G():
    """Mutually orthogonal keys: G = 0, so U = R (no propagation)."""
    rng = np.random.default_rng(9)
    T, dk = 8, 8
    parent = W.random_tree(rng, T, 5)
    q, k, v, g, beta, S = rand_inputs(rng, T, dk, 3)
    k = np.linalg.qr(rng.standard_normal((dk, dk)))[0][:T]
    cf = closed_form_tree(parent, q, k, v, g, beta, S)
    assert np.max(np.abs(cf["G"])) < 1e-15
    O, U, _ = walk_one(parent, q, k, v, g, beta, S)
    assert rel(U, cf["R"]) < 1e-12


def test_ungated_chain_is_deltanet():
    """All gates 1 (g = 0) on a chain: ungated DeltaNet, S_t = S_{t-1}(I - b k k^T) + b v k^T."""
    rng = np.random.default_rng(11)
    T = 10
    q, k, v, g, beta, S = rand_inputs(rng, T, 6, 6)
    g[:] = 0.0
    O, U, Sn = walk_one(np.arange(-1, T - 1, dtype=np.int32), q, k, v, g, beta, S, accept=T - 1)
    St = S.copy()
    for t in range(T):
        St = St @ (np.eye(6) - beta[t] * np.outer(k[t], k[t])) + beta[t] * np.outer(v[t], k[t])
    assert rel(Sn, St) < 1e-12


# ---------------------------------------------------------------------------
# mutations planted in (a copy of) the closed form must be caught by the walk

@pytest.mark.parametrize("mutation", ["g_sign", "c_no_diag", "g_transpose", "drop_last_term",
                                      "p_excludes_self"])
def test_pins_catch_planted_mistakes(mutation):
    rng = np.random.default_rng(12)
    T = 10
    parent = W.random_tree(rng, T, 5)
    q, k, v, g, beta, S = rand_inputs(rng, T, 6, 5)
    O, U, _ = walk_one(parent, q, k, v, g, beta, S)
    P, G, C, d = tree_factors(parent, q, k, g, beta)
    St = S.T
    if mutation == "p_excludes_self":
        P = P / np.exp(g)
    B0 = P[:, None] * (q @ St)
    R = beta[:, None] * (v - P[:, None] * (k @ St))
    if mutation == "g_sign":
        G = -G
    if mutation == "g_transpose":
        G = G.T
    if mutation == "c_no_diag":
        C = C - np.diag(np.diag(C))
    steps = d - 1 if mutation == "drop_last_term" else d
    Uc, Z = R.copy(), R.copy()
    for _ in range(steps):
        Z = -G @ Z
        Uc += Z
    Oc = B0 + C @ Uc
    assert max(rel(Uc, U), rel(Oc, O)) > 1e-6


# ---------------------------------------------------------------------------
# tree preparation

def test_tree_prep_golden():
    gd = json.load(open(os.path.join(GOLD, "tree_prep.json")))
    r = oracle.tree_prep(np.array(gd["parent"]), np.array(gd["tree_off"]))
    assert r["err"] == 0
    assert r["depth"].tolist() == gd["depth"]
    assert r["anc"].tolist() == gd["anc"]
    assert r["order"].tolist() == gd["order"]
    assert r["tree_depth"].tolist() == gd["tree_depth"]


def test_logp_chain_is_float32_running_sum():
    """logP on a chain equals numpy's sequential float32 accumulation of g
    (root first), and logP(root) == g(root) bit for bit."""
    rng = np.random.default_rng(13)
    T, H, L = 64, 3, 2
    g = (-np.logaddexp(0, rng.standard_normal((L, T, H)))).astype(np.float32)
    r = oracle.tree_prep(np.arange(-1, T - 1, dtype=np.int32), np.array([0, T], np.int32), g)
    ref = np.add.accumulate(g, axis=1, dtype=np.float32)
    assert np.array_equal(r["logP"].view(np.uint32), ref.view(np.uint32))


def test_logp_tree_paths():
    """logP of every node equals the float32 sum of g over its path, root first."""
    rng = np.random.default_rng(14)
    f = W.make_forest(W.CONFIGS["ragged"], seed=3)
    g = (-np.logaddexp(0, rng.standard_normal((1, f.N, 2)) - 3)).astype(np.float32)
    r = oracle.tree_prep(f.parent, f.tree_off, g)
    assert r["err"] == 0
    for b in range(f.B):
        o = f.tree_off[b]
        for i in range(f.sizes()[b]):
            path, x = [], i
            while x >= 0:
                path.append(x)
                x = f.parent[o + x]
            for h in range(2):
                acc = np.float32(0.0)
                for nd in path[::-1]:
                    acc = np.float32(acc + g[0, o + nd, h])
                assert r["logP"][0, o + i, h].view(np.uint32) == acc.view(np.uint32)


@pytest.mark.parametrize("case,bits", [
    ("bad_parent_range", oracle.ERR_BAD_PARENT),
    ("self_parent", oracle.ERR_BAD_PARENT),
    ("cycle", oracle.ERR_CYCLE),
    ("too_big", oracle.ERR_TREE_SIZE),
    ("empty", oracle.ERR_TREE_SIZE),
])
def test_tree_prep_errors(case, bits):
    good = np.array([-1, 0, 0], np.int32)
    if case == "bad_parent_range":
        trees, off = [good, np.array([-1, 5], np.int32)], [0, 3, 5]
    elif case == "self_parent":
        trees, off = [good, np.array([-1, 1], np.int32)], [0, 3, 5]
    elif case == "cycle":
        trees, off = [good, np.array([-1, 2, 1], np.int32)], [0, 3, 6]
    elif case == "too_big":
        trees, off = [good, np.arange(-1, 64, dtype=np.int32)], [0, 3, 68]
    else:
        trees, off = [good, np.zeros(0, np.int32)], [0, 3, 3]
    r = oracle.tree_prep(np.concatenate(trees), np.array(off, np.int32))
    assert r["err"] == bits
    assert r["depth"][:3].tolist() == [0, 1, 1]   # the valid tree is still prepared


def test_prefix_state_is_sequential():
    """Committed prefix states are token-order decoding from a zero state."""
    cfg = W.CONFIGS["tiny"]
    pt = W.make_prefix(cfg, 0, 0, 0)
    S = oracle.prefix_states(pt.k64[None], pt.v64[None], pt.g64[None], pt.beta64[None])[0]
    S2, _, _ = oracle.sequential(np.zeros((cfg.d_v, cfg.d_k)), pt.q64, pt.k64, pt.v64,
                                 pt.g64, pt.beta64)
    assert np.array_equal(S, S2)
