"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Bars: tree preparation bit-exact; O, U and the committed state within a max
block-relative error of 1e-4 for float32 token inputs and 2e-2 for bf16 q/k/v
with float32 state (block = one tree x one head; error = max|x - ref| /
max|ref| over the block).
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.closed_form import tree_factors

from helpers import (block_rel_err, gpu_round, make_case, oracle_layer, state_rel_err,
                     tolerance)

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


PARITY_CONFIGS = ["tiny", "decode", "batched", "ragged", "target"]


def all_units(case):
    return [(b, h) for b in range(case.B) for h in range(case.cfg.H)]


@pytest.fixture(scope="module")
def cases():
    return {}


def get_case(cases, name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in cases:
        cases[key] = make_case(name, **kw)
    return cases[key]


# ---------------------------------------------------------------------------
# tree preparation

def _check_prep(out, ref, forest, valid):
    for b in np.nonzero(valid)[0]:
        sl = slice(forest.tree_off[b], forest.tree_off[b + 1])
        assert np.array_equal(out["depth"][sl], ref["depth"][sl])
        assert np.array_equal(out["anc"][sl], ref["anc"][sl])
        assert np.array_equal(out["order"][sl], ref["order"][sl])
        assert out["tree_depth"][b] == ref["tree_depth"][b]
        if ref["logP"] is not None:
            assert np.array_equal(out["logP"][:, sl].view(np.uint32),
                                  ref["logP"][:, sl].view(np.uint32))


def _gpu_prep(parent, tree_off, g):
    from linear_attention_tree_amd import TreeRound
    rnd = TreeRound(parent, tree_off, g.shape[2])
    logP = rnd.prep(torch.from_numpy(g).cuda())
    torch.cuda.synchronize()
    return dict(depth=rnd.topo.depth.cpu().numpy(),
                anc=rnd.topo.anc.cpu().numpy().view(np.uint64),
                order=rnd.topo.order.cpu().numpy(), tree_depth=rnd.topo.tree_depth.cpu().numpy(),
                logP=logP.cpu().numpy(), err=rnd.error_bits())


@pytest.mark.parametrize("name", PARITY_CONFIGS + ["multilayer"])
def test_tree_prep_bit_exact(name):
    cfg = W.CONFIGS[name]
    f = W.make_forest(cfg, seed=1)
    L = min(cfg.L, 4)
    g = np.stack([W.make_layer(cfg, f.N, l, seed=1).g for l in range(L)])
    say(f"tree_prep {name} N={f.N} L={L}")
    out = _gpu_prep(f.parent, f.tree_off, g)
    ref = oracle.tree_prep(f.parent, f.tree_off, g)
    assert out["err"] == ref["err"] == 0
    _check_prep(out, ref, f, np.ones(f.B, bool))


def test_tree_prep_adversarial_topologies():
    rng = np.random.default_rng(5)
    trees = [
        np.arange(-1, 63, dtype=np.int32),                    # chain of 64
        np.array([-1] + [0] * 63, dtype=np.int32),            # star of 64
        np.array([-1], dtype=np.int32),                       # singleton
        np.array([3, 0, 3, -1, 1], dtype=np.int32),           # child before parent
        np.array([-1, 0, -1, 2], dtype=np.int32),             # two roots in one tree
    ]
    for T in (2, 17, 33, 64):                                 # shuffled random trees
        p = W.random_tree(rng, T, 63)
        perm = rng.permutation(T)
        inv = np.argsort(perm)
        trees.append(np.array([-1 if p[perm[i]] < 0 else inv[p[perm[i]]] for i in range(T)],
                              np.int32))
    f = W.forest_from_trees(trees)
    g = (-np.logaddexp(0, rng.standard_normal((2, f.N, 3)))).astype(np.float32)
    say(f"tree_prep adversarial N={f.N}")
    out = _gpu_prep(f.parent, f.tree_off, g)
    ref = oracle.tree_prep(f.parent, f.tree_off, g)
    assert out["err"] == ref["err"] == 0
    _check_prep(out, ref, f, np.ones(f.B, bool))


@pytest.mark.parametrize("bad,bits", [
    ("bad_parent", oracle.ERR_BAD_PARENT), ("self_parent", oracle.ERR_BAD_PARENT),
    ("cycle", oracle.ERR_CYCLE), ("too_big", oracle.ERR_TREE_SIZE),
    ("empty", oracle.ERR_TREE_SIZE)])
def test_tree_prep_error_bits(bad, bits):
    good = [np.array([-1, 0, 0, 1], np.int32), np.array([-1, 0], np.int32)]
    badt = {"bad_parent": np.array([-1, 7], np.int32), "self_parent": np.array([-1, 1], np.int32),
            "cycle": np.array([-1, 2, 3, 1], np.int32),
            "too_big": np.arange(-1, 64, dtype=np.int32),
            "empty": np.zeros(0, np.int32)}[bad]
    trees = [good[0], badt, good[1]]
    f = W.forest_from_trees(trees)
    g = np.full((1, f.N, 2), -0.5, np.float32)
    say(f"tree_prep error {bad}")
    out = _gpu_prep(f.parent, f.tree_off, g)
    ref = oracle.tree_prep(f.parent, f.tree_off, g)
    assert out["err"] == ref["err"] == bits
    assert out["tree_depth"][1] == -1
    _check_prep(out, ref, f, np.array([True, False, True]))


# ---------------------------------------------------------------------------
# factor producer

@pytest.mark.parametrize("name", ["tiny", "decode", "ragged"])
def test_factor_gc_against_definition(cases, name):
    case = get_case(cases, name, n_layers=1)
    say(f"factor_gc {name}")
    out = gpu_round(case, commit=False)
    x = case.layers[0]
    f = case.forest
    worst_g = worst_c = 0.0
    for b in range(f.B):
        o, T = f.tree_off[b], f.sizes()[b]
        par = f.parent[o:o + T]
        for h in range(case.cfg.H):
            P, G, C, d = tree_factors(par, x.q64[o:o + T, h], x.k64[o:o + T, h],
                                      x.g64[o:o + T, h], x.beta64[o:o + T, h])
            lev = out["order"][o:o + T]          # level position -> local node
            Gg = out["G"][b, h]
            Cg = out["C"][b, h]
            G = G[np.ix_(lev, lev)]
            C = C[np.ix_(lev, lev)]
            # level order is parent-before-child: G strictly lower, C lower triangular
            assert np.all(np.triu(Gg[:T, :T]) == 0) and np.all(np.triu(Cg[:T, :T], 1) == 0)
            # exact zeros outside the ancestor mask and the padding
            assert np.all(Gg[T:] == 0) and np.all(Gg[:, T:] == 0)
            assert np.all(Cg[T:] == 0) and np.all(Cg[:, T:] == 0)
            assert np.all(Gg[:T, :T][G == 0] == 0)
            assert np.all(Cg[:T, :T][C == 0] == 0)
            worst_g = max(worst_g, np.max(np.abs(Gg[:T, :T] - G)) / max(np.max(np.abs(G)), 1e-30))
            worst_c = max(worst_c, np.max(np.abs(Cg[:T, :T] - C)) / np.max(np.abs(C)))
    say(f"  G rel {worst_g:.2e}  C rel {worst_c:.2e}")
    assert worst_g < 1e-5 and worst_c < 1e-5


# ---------------------------------------------------------------------------
# verify + commit

@pytest.mark.parametrize("name", PARITY_CONFIGS)
def test_verify_commit_parity(cases, name):
    case = get_case(cases, name, n_layers=1)
    tol = tolerance(case.cfg)
    say(f"verify+commit {name} B={case.B} N={case.N} H={case.cfg.H}")
    out = gpu_round(case)
    assert out["err"] == 0
    O, U, S_new = oracle_layer(case, 0)
    eo = block_rel_err(out["O"][0], O, case.forest.tree_off)
    eu = block_rel_err(out["U"][0], U, case.forest.tree_off)
    es = state_rel_err(out["S"][0], S_new, case.slot, all_units(case))
    say(f"  O {eo:.2e}  U {eu:.2e}  S_new {es:.2e}  (bar {tol:g})")
    assert eo <= tol and eu <= tol and es <= tol
    # slots not owned by any request are untouched
    free = sorted(set(range(case.n_slots)) - set(case.slot.tolist()))
    for s in free:
        assert np.array_equal(out["S"][0][s], case.S_pre[0][s])


# ---------------------------------------------------------------------------
# invariants (bit-exact on the GPU)

def test_verify_idempotent_and_state_immutable(cases):
    from linear_attention_tree_amd import TreeRound
    from helpers import to_dev
    case = get_case(cases, "ragged", n_layers=1)
    f = case.forest
    say("invariants: idempotence / immutability")
    d = to_dev(case, 0)
    rnd = TreeRound(f.parent, f.tree_off, case.cfg.H)
    logP = rnd.prep(d["g"][None])[0]
    pool = torch.from_numpy(case.S_pre[0]).cuda()
    slot = torch.from_numpy(case.slot).cuda()
    before = pool.clone()
    O1, U1 = rnd.layer(d["q"], d["k"], d["v"], logP, d["beta"], pool, slot)
    O2, U2 = rnd.layer(d["q"], d["k"], d["v"], logP, d["beta"], pool, slot)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)
    assert torch.equal(O1, O2) and torch.equal(U1, U2)
    # a dropped round (no commit) leaves the state as it was; accept = -1 too
    rnd.commit(pool.unsqueeze(0), slot, d["k"][None], U1[None], logP[None],
               np.full(f.B, -1, np.int32))
    torch.cuda.synchronize()
    assert torch.equal(pool, before)
    assert rnd.error_bits() == 0


def test_sibling_independence():
    """Perturbing a node's inputs leaves every non-descendant's O and U bit-unchanged."""
    from linear_attention_tree_amd import TreeRound
    from helpers import to_dev
    case = make_case("batched", n_layers=1, seed=4)
    f = case.forest
    b = 3
    o, T = int(f.tree_off[b]), int(f.sizes()[b])
    ref = oracle.tree_prep(f.parent, f.tree_off)
    victim = T - 1
    desc = [i for i in range(T) if (int(ref["anc"][o + i]) >> victim) & 1]
    say("invariants: sibling independence")
    res = []
    for pert in (False, True):
        d = to_dev(case, 0)
        if pert:
            for key in ("q", "k", "v"):
                d[key][o + victim] = -d[key][o + victim] * 0.5
            d["g"][o + victim] -= 0.3
            d["beta"][o + victim] *= 0.5
        rnd = TreeRound(f.parent, f.tree_off, case.cfg.H)
        logP = rnd.prep(d["g"][None])[0]
        pool = torch.from_numpy(case.S_pre[0]).cuda()
        O, U = rnd.layer(d["q"], d["k"], d["v"], logP, d["beta"], pool,
                         torch.from_numpy(case.slot).cuda())
        torch.cuda.synchronize()
        res.append((O.float().cpu().numpy(), U.cpu().numpy()))
    keep = np.ones(f.N, bool)
    for i in desc:
        keep[o + i] = False
    assert np.array_equal(res[0][0][keep], res[1][0][keep])
    assert np.array_equal(res[0][1][keep], res[1][1][keep])
    assert not np.array_equal(res[0][1][o + victim], res[1][1][o + victim])


@pytest.mark.parametrize("dtype,d_k", [("bf16", 128), ("f32", 64)])
def test_value_tiles_are_independent(dtype, d_k):
    """Value tiling changes only the schedule (arXiv page, section IV-B: each
    value tile's B0, R, U and O need no other tile).  At d_v = 256 every head
    runs as two 128-column tiles in separate workgroups; each tile's O and U
    columns must equal, bit for bit, a d_v = 128 call on just those V columns
    and state rows.  Through bole_tree_verify and through the two-call path
    (bole_factor_gc + bole_verify)."""
    from linear_attention_tree_amd import TreeRound
    from helpers import to_dev
    cfg = W.Config(f"tiles_{dtype}", 41, B=3, H=2, d_k=d_k, d_v=256, dtype=dtype, tree="fixed",
                   T=64, D=12, prefix=32)
    case = make_case(cfg, n_layers=1, seed=6)
    f = case.forest
    say(f"invariants: value tiles {dtype} d_k={d_k}")
    d = to_dev(case, 0)
    slot = torch.from_numpy(case.slot).cuda()
    pool = torch.from_numpy(case.S_pre[0]).cuda()  # [slots, H, d_v, d_k]: row v holds S[:, v]

    def run(v, pl):
        rnd = TreeRound(f.parent, f.tree_off, cfg.H)
        O_t, U_t, _ = rnd.tree_layer(d["q"], d["k"], v, d["g"], d["beta"], pl, slot)
        logP = rnd.prep(d["g"][None])[0]
        O_s, U_s = rnd.layer(d["q"], d["k"], v, logP, d["beta"], pl, slot)
        torch.cuda.synchronize()
        assert rnd.error_bits() == 0
        return [x.clone() for x in (O_t, U_t, O_s, U_s)]

    whole = run(d["v"], pool)
    for r in range(2):
        cols = slice(128 * r, 128 * (r + 1))
        part = run(d["v"][..., cols].contiguous(), pool[:, :, cols, :].contiguous())
        for w_, p_ in zip(whole, part):
            assert torch.equal(w_[..., cols], p_)


def test_bad_slot_and_accept_bits():
    from linear_attention_tree_amd import TreeRound
    from helpers import to_dev
    case = make_case("decode", n_layers=1, seed=2)
    f = case.forest
    say("error bits: slot / accept")
    d = to_dev(case, 0)
    rnd = TreeRound(f.parent, f.tree_off, case.cfg.H)
    logP = rnd.prep(d["g"][None])[0]
    pool = torch.from_numpy(case.S_pre[0]).cuda()
    bad_slot = torch.tensor([case.n_slots], dtype=torch.int32).cuda()
    rnd.layer(d["q"], d["k"], d["v"], logP, d["beta"], pool, bad_slot)
    torch.cuda.synchronize()
    assert rnd.error_bits() == oracle.ERR_BAD_SLOT
    rnd.err.zero_()
    before = pool.clone()
    rnd.commit(pool.unsqueeze(0), torch.from_numpy(case.slot).cuda(), d["k"][None],
               torch.zeros(f.N, case.cfg.H, case.cfg.d_v, device="cuda")[None], logP[None],
               np.array([f.sizes()[0]], np.int32))
    torch.cuda.synchronize()
    assert rnd.error_bits() == oracle.ERR_BAD_ACCEPT
    assert torch.equal(pool, before)


# ---------------------------------------------------------------------------
# fused factor + verify

@pytest.mark.parametrize("name", ["tiny", "decode", "batched", "ragged", "target"])
def test_factor_verify_bit_identical_to_two_calls(cases, name):
    """One-launch factor+verify gives exactly the bits of factor_gc then verify."""
    from linear_attention_tree_amd import TreeRound
    from helpers import to_dev
    case = get_case(cases, name, n_layers=1)
    f = case.forest
    say(f"factor_verify vs two calls {name}")
    d = to_dev(case, 0)
    rnd = TreeRound(f.parent, f.tree_off, case.cfg.H)
    logP = rnd.prep(d["g"][None])[0]
    pool = torch.from_numpy(case.S_pre[0]).cuda()
    slot = torch.from_numpy(case.slot).cuda()
    O1, U1 = rnd.layer(d["q"], d["k"], d["v"], logP, d["beta"], pool, slot)
    O2, U2 = rnd.layer(d["q"], d["k"], d["v"], logP, d["beta"], pool, slot, fused=True)
    torch.cuda.synchronize()
    assert rnd.error_bits() == 0
    assert torch.equal(O1, O2) and torch.equal(U1, U2)
    O, U, _ = oracle_layer(case, 0, accept=False)
    eo = block_rel_err(O2.float().cpu().numpy(), O, f.tree_off)
    eu = block_rel_err(U2.cpu().numpy(), U, f.tree_off)
    say(f"  fused O {eo:.2e}  U {eu:.2e}")
    assert eo <= tolerance(case.cfg) and eu <= tolerance(case.cfg)


# ---------------------------------------------------------------------------
# HIP graph capture

@pytest.mark.parametrize("path", ["fused", "tree"])
@pytest.mark.parametrize("name", ["decode", "target"])
def test_graph_replay_matches_eager(cases, name, path):
    """The whole step (prep, fused factor + verify, commit; or tree_verify then
    the commit) captured in a HIP graph reproduces the eager launches bit for
    bit, replay after replay, with eager work and synchronizations between the
    replays."""
    from linear_attention_tree_amd import TreeRound, bole
    from helpers import to_dev
    case = get_case(cases, name, n_layers=1)
    f = case.forest
    say(f"graph replay {name} {path}")
    d = to_dev(case, 0)
    rnd = TreeRound(f.parent, f.tree_off, case.cfg.H)
    t = rnd.topo
    g = d["g"][None].contiguous()
    logP = torch.empty_like(g)
    pool0 = torch.from_numpy(case.S_pre[0]).cuda()
    pool = pool0.clone()
    slot = torch.from_numpy(case.slot).cuda()
    accept = torch.from_numpy(f.accept).cuda()
    O = torch.empty(f.N, case.cfg.H, case.cfg.d_v, dtype=d["v"].dtype, device="cuda")
    U = torch.empty(f.N, case.cfg.H, case.cfg.d_v, dtype=torch.float32, device="cuda")

    def step():
        if path == "tree":
            bole.bole_tree_verify(d["q"], d["k"], d["v"], t.parent, g[0], d["beta"], pool, slot,
                                  t.tree_off, O, U, t.depth, t.anc, t.order, t.tree_depth,
                                  logP[0], rnd.err)
        else:
            bole.bole_tree_prep(t.parent, t.tree_off, g, t.depth, t.anc, t.order, t.tree_depth,
                                logP, rnd.err)
            bole.bole_factor_verify(d["q"], d["k"], d["v"], logP[0], d["beta"], pool, slot,
                                    t.anc, t.order, t.depth, t.tree_off, t.tree_depth, O, U,
                                    rnd.err)
        bole.bole_commit_path(pool, slot, d["k"], U, logP[0], t.anc, t.tree_off, accept,
                              rnd.err)

    step()
    torch.cuda.synchronize()
    ref = (O.clone(), U.clone(), pool.clone(), logP.clone())
    assert rnd.error_bits() == 0
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pool.copy_(pool0)
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        pool.copy_(pool0)
        O.zero_()
        U.zero_()
        logP.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (O, U, pool, logP)):
            assert torch.equal(a, b), f"replay {rep} differs"
        _ = (pool0 * 2.0).sum().item()  # eager work between replays
    assert rnd.error_bits() == 0
