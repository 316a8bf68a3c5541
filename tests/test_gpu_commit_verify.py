"""bole_commit_tree_verify: the previous round's accepted-path commit done
inside the next round's tree verify.

Against bole_commit_path followed by bole_tree_verify on the same inputs, bit
for bit (committed states, O, U, the preparation outputs and the error bits).
The cases cover:
- paths longer than 16 nodes (two 64-node chains);
- requests with nothing to commit;
- a rejected new tree, and an empty new tree range;
- a bad previous accepted node;
- float32 tokens, partial head dimensions and two value tiles.
Then two rounds against the fp64 oracle: round one's commit, and round two's
walk from the committed state.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import block_rel_err, prefix_slots, state_rel_err, tolerance

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def cfg_of(name, cid, dtype="bf16", d_k=128, d_v=128, B=4, H=3, T=64, D=12):
    return W.Config(name, cid, B=B, H=H, d_k=d_k, d_v=d_v, dtype=dtype, tree="fixed", T=T, D=D,
                    prefix=32)


def device_round(cfg, forest, x):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731

    def tok(a):
        a = np.ascontiguousarray(a)
        if cfg.dtype == "bf16":
            return d(a.view(np.int16)).view(torch.bfloat16)
        return d(a)

    N, B = len(forest.parent), len(forest.tree_off) - 1
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    return dict(q=tok(x.q), k=tok(x.k), v=tok(x.v), g=d(x.g), beta=d(x.beta),
                parent=d(forest.parent.astype(np.int32)),
                tree_off=d(forest.tree_off.astype(np.int32)),
                O=torch.zeros(N, cfg.H, cfg.d_v, dtype=tdt, device="cuda"),
                U=torch.zeros(N, cfg.H, cfg.d_v, dtype=torch.float32, device="cuda"),
                depth=torch.zeros(N, dtype=torch.int32, device="cuda"),
                anc=torch.zeros(N, dtype=torch.int64, device="cuda"),
                order=torch.zeros(N, dtype=torch.int32, device="cuda"),
                tree_depth=torch.zeros(B, dtype=torch.int32, device="cuda"),
                logP=torch.zeros(N, cfg.H, dtype=torch.float32, device="cuda"),
                err=torch.zeros(1, dtype=torch.int32, device="cuda"))


def tree_verify(r, pool, slot):
    from linear_attention_tree_amd import bole
    bole.bole_tree_verify(r["q"], r["k"], r["v"], r["parent"], r["g"], r["beta"], pool, slot,
                          r["tree_off"], r["O"], r["U"], r["depth"], r["anc"], r["order"],
                          r["tree_depth"], r["logP"], r["err"])


def outputs(r, pool):
    torch.cuda.synchronize()
    return dict(pool=pool.clone(), O=r["O"].clone(), U=r["U"].clone(), depth=r["depth"].clone(),
                anc=r["anc"].clone(), order=r["order"].clone(),
                tree_depth=r["tree_depth"].clone(), logP=r["logP"].clone(),
                err=int(r["err"].item()))


def run_pair(cfg, f1, x1, f2, x2, pool0, slot_np, accept1, prev_off=None):
    """Round one by bole_tree_verify; then round two both ways: the reference
    (bole_commit_path of round one, then bole_tree_verify) and the fused call.
    prev_off replaces round one's offsets in both commits (bad ranges)."""
    from linear_attention_tree_amd import bole
    slot = torch.from_numpy(slot_np).cuda()
    acc = torch.from_numpy(np.asarray(accept1, np.int32)).cuda()
    r1 = device_round(cfg, f1, x1)
    tree_verify(r1, torch.from_numpy(pool0).cuda(), slot)
    torch.cuda.synchronize()
    assert int(r1["err"].item()) == 0

    p_off = r1["tree_off"] if prev_off is None else torch.from_numpy(prev_off).cuda()
    ref2 = device_round(cfg, f2, x2)
    pool_a = torch.from_numpy(pool0).cuda()
    bole.bole_commit_path(pool_a, slot, r1["k"], r1["U"], r1["logP"], r1["anc"], p_off,
                          acc, ref2["err"])
    tree_verify(ref2, pool_a, slot)
    want = outputs(ref2, pool_a)

    fus2 = device_round(cfg, f2, x2)
    pool_b = torch.from_numpy(pool0).cuda()
    bole.bole_commit_tree_verify(
        fus2["q"], fus2["k"], fus2["v"], fus2["parent"], fus2["g"], fus2["beta"], pool_b, slot,
        fus2["tree_off"], fus2["O"], fus2["U"], fus2["depth"], fus2["anc"], fus2["order"],
        fus2["tree_depth"], fus2["logP"], r1["k"], r1["U"], r1["logP"], r1["anc"],
        p_off, acc, fus2["err"])
    got = outputs(fus2, pool_b)
    return got, want


def assert_same(got, want):
    assert got["err"] == want["err"]
    for key in ("pool", "O", "U", "depth", "anc", "order", "tree_depth", "logP"):
        a, b = got[key], want[key]
        if a.dtype in (torch.float32, torch.bfloat16):
            a, b = a.view(torch.int32 if a.dtype == torch.float32 else torch.int16), \
                b.view(torch.int32 if b.dtype == torch.float32 else torch.int16)
        assert torch.equal(a, b), key


def two_rounds(cfg, seed, f1=None, f2=None, accept1=None):
    f1 = f1 if f1 is not None else W.make_forest(cfg, seed)
    f2 = f2 if f2 is not None else W.make_forest(cfg, seed + 1)
    accept1 = f1.accept if accept1 is None else accept1
    x1 = W.make_layer(cfg, len(f1.parent), 0, seed)
    x2 = W.make_layer(cfg, len(f2.parent), 0, seed + 1)
    n_slots = cfg.B + 2
    slot = np.random.default_rng([seed, 3]).permutation(n_slots)[: cfg.B].astype(np.int32)
    pool0 = prefix_slots(cfg, 0, n_slots, slot, seed)
    return f1, x1, f2, x2, pool0, slot, np.asarray(accept1, np.int32)


@pytest.mark.parametrize("dtype,d_k,d_v", [("bf16", 128, 128), ("bf16", 64, 192),
                                           ("bf16", 48, 80), ("f32", 64, 64), ("f32", 32, 48)])
def test_matches_commit_then_tree_verify(dtype, d_k, d_v):
    cfg = cfg_of(f"cv_{dtype}_{d_k}_{d_v}", 60, dtype, d_k, d_v)
    f1, x1, f2, x2, pool0, slot, acc = two_rounds(cfg, 11)
    acc[1] = -1  # nothing to commit for request 1
    say(f"commit+verify {dtype} d_k={d_k} d_v={d_v} accept {acc.tolist()}")
    got, want = run_pair(cfg, f1, x1, f2, x2, pool0, slot, acc)
    assert got["err"] == 0
    assert_same(got, want)
    # request 1's slot is untouched
    s1 = slot[1]
    assert np.array_equal(got["pool"][s1].cpu().numpy().view(np.uint32), pool0[s1].view(np.uint32))


def test_long_paths():
    """Accepted paths of 64 and 18 nodes (chains): the steps past the first 16
    positions, each with its own staged key tile."""
    cfg = cfg_of("cv_chain", 61, B=2, H=2)
    f1 = W.chain_forest(2, 64)
    f1 = W.Forest(parent=f1.parent, tree_off=f1.tree_off, accept=np.array([63, 17], np.int32))
    f1, x1, f2, x2, pool0, slot, acc = two_rounds(cfg, 12, f1=f1)
    say(f"commit+verify long paths, accept {acc.tolist()}")
    got, want = run_pair(cfg, f1, x1, f2, x2, pool0, slot, acc)
    assert got["err"] == 0
    assert_same(got, want)


def test_rejected_trees_and_bad_accept():
    """Round two's request 1 has a cycle and request 2 an empty range: both
    still commit.  Request 3's previous accepted node is out of range: no
    commit, and the verify reads the old state."""
    cfg = cfg_of("cv_bad", 62, B=4, H=2)
    f1, x1, f2, x2, pool0, slot, acc = two_rounds(cfg, 13)
    sizes1 = np.diff(f1.tree_off)
    acc[3] = sizes1[3]  # one past the last node
    trees = [f2.parent[f2.tree_off[b]:f2.tree_off[b + 1]].copy() for b in range(cfg.B)]
    trees[1][5] = 7
    trees[1][7] = 5          # 5 -> 7 -> 5
    trees[2] = trees[2][:0]  # empty range
    par = np.concatenate(trees).astype(np.int32)
    off = np.zeros(cfg.B + 1, np.int32)
    off[1:] = np.cumsum([len(t) for t in trees])
    f2 = W.Forest(parent=par, tree_off=off, accept=np.zeros(cfg.B, np.int32))
    x2 = W.make_layer(cfg, len(par), 0, 14)
    say(f"commit+verify rejected trees, accept {acc.tolist()}")
    got, want = run_pair(cfg, f1, x1, f2, x2, pool0, slot, acc)
    from linear_attention_tree_amd import bole
    bits = bole.ERR_CYCLE | bole.ERR_TREE_SIZE | bole.ERR_BAD_ACCEPT
    assert got["err"] == want["err"] == bits, (got["err"], want["err"])
    assert_same(got, want)
    td = got["tree_depth"].cpu().numpy()
    assert td[1] == -1
    # the committed slots of requests 1 and 2 differ from the old ones; request 3's does not
    for b, changed in ((1, True), (2, True), (3, False)):
        same = np.array_equal(got["pool"][slot[b]].cpu().numpy().view(np.uint32),
                              pool0[slot[b]].view(np.uint32))
        assert same != changed, b


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_rounds_against_oracle(dtype):
    d = 128 if dtype == "bf16" else 64
    cfg = cfg_of(f"cv_oracle_{dtype}", 63, dtype, d, d, B=3, H=2)
    f1, x1, f2, x2, pool0, slot, acc = two_rounds(cfg, 15)
    say(f"commit+verify vs oracle {dtype}, accept {acc.tolist()}")
    got, _ = run_pair(cfg, f1, x1, f2, x2, pool0, slot, acc)
    assert got["err"] == 0
    # round one's commit, then round two's walk from the committed states
    _, _, S1 = oracle.verify(f1.parent, f1.tree_off, x1.q64, x1.k64, x1.v64, x1.g64, x1.beta64,
                             pool0, slot, acc)
    pool1 = pool0.astype(np.float64)
    for b in range(cfg.B):
        pool1[slot[b]] = S1[b]
    O2, U2, _ = oracle.verify(f2.parent, f2.tree_off, x2.q64, x2.k64, x2.v64, x2.g64, x2.beta64,
                              pool1, slot, None)
    units = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    tol = tolerance(cfg)
    es = state_rel_err(got["pool"].cpu().numpy(), S1, slot, units)
    eo = block_rel_err(got["O"].float().cpu().numpy(), O2, f2.tree_off)
    eu = block_rel_err(got["U"].cpu().numpy(), U2, f2.tree_off)
    say(f"  committed state {es:.2e}  O {eo:.2e}  U {eu:.2e} (bar {tol:g})")
    assert es <= tol and eo <= tol and eu <= tol


def test_runner_commit_tree_layer():
    """TreeRound.commit_tree_layer (the runner's form of the fused call) over
    three rounds equals TreeRound.commit followed by tree_layer, bit for bit."""
    from linear_attention_tree_amd import TreeRound
    cfg = cfg_of("cv_runner", 64, B=3, H=2)
    forests = [W.make_forest(cfg, 20 + r) for r in range(3)]
    xs = [W.make_layer(cfg, len(f.parent), 0, 20 + r) for r, f in enumerate(forests)]
    n_slots = cfg.B + 1
    slot_np = np.array([2, 0, 3], np.int32)
    pool0 = prefix_slots(cfg, 0, n_slots, slot_np, 20)
    slot = torch.from_numpy(slot_np).cuda()
    outs = {}
    for mode in ("fused", "two_calls"):
        pool = torch.from_numpy(pool0).cuda()
        prev = None
        res = []
        for f, x in zip(forests, xs):
            r = device_round(cfg, f, x)
            rnd = TreeRound(f.parent, f.tree_off, cfg.H)
            if prev is None:
                O, U, lp = rnd.tree_layer(r["q"], r["k"], r["v"], r["g"], r["beta"], pool, slot)
            elif mode == "fused":
                p_rnd, p_r, p_U, p_lp, p_acc = prev
                O, U, lp = rnd.commit_tree_layer(p_rnd, p_r["k"], p_U, p_lp, p_acc, r["q"], r["k"],
                                                 r["v"], r["g"], r["beta"], pool, slot)
            else:
                p_rnd, p_r, p_U, p_lp, p_acc = prev
                p_rnd.commit(pool, slot, p_r["k"], p_U, p_lp, p_acc)
                O, U, lp = rnd.tree_layer(r["q"], r["k"], r["v"], r["g"], r["beta"], pool, slot)
            prev = (rnd, r, U, lp, f.accept)
            torch.cuda.synchronize()
            assert rnd.error_bits() == 0
            res.append((O.view(torch.int16).clone(), U.view(torch.int32).clone()))
        res.append(pool.view(torch.int32).clone())
        outs[mode] = res
    say("runner commit_tree_layer: three rounds")
    for a, b in zip(outs["fused"][:-1], outs["two_calls"][:-1]):
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(outs["fused"][-1], outs["two_calls"][-1])


def test_target_shape():
    """The headline shape (16 trees x 64 nodes, 32 heads, d = 128, bf16) in
    the launch configuration the bench times: against the two calls bit for
    bit, and eight sampled (request, head) units against the fp64 oracle over
    both rounds."""
    cfg = W.CONFIGS["target"]
    f1, x1, f2, x2, pool0, slot, acc = two_rounds(cfg, 30)
    say(f"commit+verify target shape, N1={len(f1.parent)} N2={len(f2.parent)}")
    got, want = run_pair(cfg, f1, x1, f2, x2, pool0, slot, acc)
    assert got["err"] == 0
    assert_same(got, want)
    rng = np.random.default_rng(31)
    units = [(int(b), int(h)) for b, h in zip(rng.integers(0, cfg.B, 8), rng.integers(0, cfg.H, 8))]
    _, _, S1 = oracle.verify(f1.parent, f1.tree_off, x1.q64, x1.k64, x1.v64, x1.g64, x1.beta64,
                             pool0, slot, acc, units)
    pool1 = pool0.astype(np.float64)
    for b, h in units:
        pool1[slot[b], h] = S1[b, h]
    O2, U2, _ = oracle.verify(f2.parent, f2.tree_off, x2.q64, x2.k64, x2.v64, x2.g64, x2.beta64,
                              pool1, slot, None, units)
    tol = tolerance(cfg)
    es = state_rel_err(got["pool"].cpu().numpy(), S1, slot, units)
    eo = block_rel_err(got["O"].float().cpu().numpy(), O2, f2.tree_off, units)
    eu = block_rel_err(got["U"].cpu().numpy(), U2, f2.tree_off, units)
    say(f"  sampled units {units}: committed state {es:.2e}  O {eo:.2e}  U {eu:.2e}")
    assert es <= tol and eo <= tol and eu <= tol


def test_bad_previous_ranges():
    """Previous ranges that are empty, longer than 64 nodes or past the previous
    forest: TREE_SIZE, no commit for those requests, the others committed."""
    cfg = cfg_of("cv_badprev", 65, B=4, H=2)
    f1, x1, f2, x2, pool0, slot, acc = two_rounds(cfg, 16)
    n1 = len(f1.parent)
    off = f1.tree_off.astype(np.int32).copy()
    off[1] = off[0]            # request 0: empty
    off[2] = off[1] + 65       # request 1: 65 nodes
    off[3] = off[2] + 10       # request 2: 10 nodes (committed)
    off[4] = n1 + 5            # request 3: past the end of the previous forest
    acc = np.zeros(cfg.B, np.int32)
    say(f"commit+verify bad previous ranges {off.tolist()}")
    got, want = run_pair(cfg, f1, x1, f2, x2, pool0, slot, acc, prev_off=off)
    from linear_attention_tree_amd import bole
    assert got["err"] == want["err"] == bole.ERR_TREE_SIZE, (got["err"], want["err"])
    assert_same(got, want)
    for b, changed in ((0, False), (1, False), (2, True), (3, False)):
        same = np.array_equal(got["pool"][slot[b]].cpu().numpy().view(np.uint32),
                              pool0[slot[b]].view(np.uint32))
        assert same != changed, b
