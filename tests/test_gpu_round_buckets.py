"""Capacity-bucketed round graphs (BucketedRound): budget selection and forest
packing, every layer's bole_tree_verify and one commit over all layers,
captured once per capacity bucket and replayed for rounds with other drafted
candidates, tokens and accepted nodes copied into the same buffers.

Each replay must equal the same round launched call by call, bit for bit
(outputs, committed states, packed forest); the packed forest must equal the
oracle's; and the round's O, U and committed states must match the fp64
oracle run on that packed forest.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import block_rel_err, state_rel_err
from oracle import forest as OF

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_bucketed_round_replays():
    B, L, H, d = 4, 2, 4, 64
    buckets = [64, 128, 256]
    sets = [W.make_candidates(B, seed=40 + s) for s in range(3)]
    M_total = int(sets[0].cand_off[-1])
    from linear_attention_tree_amd import BucketedRound
    rnd = BucketedRound(B, L, H, d, d, torch.bfloat16, M_total, buckets)
    cmax = buckets[-1]
    rng = np.random.default_rng(3)
    q = rng.standard_normal((L, cmax, H, d)).astype(np.float32)
    k = rng.standard_normal((L, cmax, H, d)).astype(np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((L, cmax, H, d)).astype(np.float32)
    g = (-np.logaddexp(0.0, rng.standard_normal((L, cmax, H)))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((L, cmax, H))))).astype(np.float32)
    toks = {}
    for nm, a in (("q", q), ("k", k), ("v", v)):
        bits, vals = W.round_storage(a, "bf16")
        toks[nm] = vals
        getattr(rnd, nm).copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())
    rnd.g.copy_(torch.from_numpy(g).cuda())
    rnd.beta.copy_(torch.from_numpy(beta).cuda())
    n_slots = B + 2
    pool0 = (0.2 * rng.standard_normal((L, n_slots, H, d, d))).astype(np.float32)
    slot_np = np.array([3, 0, 5, 1], np.int32)
    slot = torch.from_numpy(slot_np).cuda()
    pool = torch.from_numpy(pool0).cuda()

    def load(c):
        rnd.cand_parent.copy_(torch.from_numpy(c.cand_parent).cuda())
        rnd.p_draft.copy_(torch.from_numpy(c.p_draft).cuda())
        rnd.cand_off.copy_(torch.from_numpy(c.cand_off).cuda())

    load(sets[0])  # the pass before each capture runs a real round
    rnd.capture(pool, slot)
    torch.cuda.synchronize()
    assert int(rnd.err.item()) == 0

    def snapshot(cap):
        f = rnd.forest[cap]
        return dict(O=rnd.O[:, :cap].clone(), U=rnd.U[:, :cap].clone(), pool=pool.clone(),
                    parent=f.parent.clone(), tree_off=f.tree_off.clone(),
                    cand_of=f.cand_of.clone())

    for si, budget in ((1, 60), (2, 128), (0, 200), (1, 256), (2, 64)):
        c = sets[si]
        cap = rnd.bucket(budget)
        ref = OF.build_forest(c.cand_parent, c.p_draft, c.cand_off, cap, 64)
        sizes = np.diff(ref["tree_off"])
        accept = (sizes - 1).astype(np.int32)        # each request's last packed node
        say(f"bucketed round: set {si}, budget {budget} -> bucket {cap}, sizes {sizes.tolist()}")
        load(c)
        rnd.accept.copy_(torch.from_numpy(accept).cuda())
        pool.copy_(torch.from_numpy(pool0).cuda())
        assert rnd.replay(budget) == cap
        torch.cuda.synchronize()
        got = snapshot(cap)
        pool.copy_(torch.from_numpy(pool0).cuda())
        rnd.run_eager(cap, pool, slot)
        torch.cuda.synchronize()
        want = snapshot(cap)
        assert int(rnd.err.item()) == 0
        for key in got:
            assert torch.equal(got[key], want[key]), key
        # the packed forest is the oracle's
        assert np.array_equal(got["tree_off"].cpu().numpy(), ref["tree_off"])
        assert np.array_equal(got["parent"].cpu().numpy(), ref["parent"])
        assert np.array_equal(got["cand_of"].cpu().numpy(), ref["cand_of"])
        # and the round is the oracle's walk over it (every layer)
        n = int(ref["tree_off"][-1])
        for l in range(L):
            O, U, S_new = oracle.verify(ref["parent"][:n], ref["tree_off"], toks["q"][l, :n],
                                        toks["k"][l, :n], toks["v"][l, :n],
                                        g[l, :n].astype(np.float64), beta[l, :n].astype(np.float64),
                                        pool0[l], slot_np, accept)
            units = [(b, h) for b in range(B) for h in range(H)]
            eo = block_rel_err(got["O"][l, :n].float().cpu().numpy(), O, ref["tree_off"])
            eu = block_rel_err(got["U"][l, :n].cpu().numpy(), U, ref["tree_off"])
            es = state_rel_err(got["pool"][l].cpu().numpy(), S_new, slot_np, units)
            say(f"  layer {l}: O {eo:.2e}  U {eu:.2e}  S_new {es:.2e}")
            assert eo <= 2e-2 and eu <= 2e-2 and es <= 2e-2


def test_bucketed_round_deferred_matches_two_launch_rounds():
    """deferred=True (each layer's launch carries its commit of the previous
    round): over five rounds with changing candidates, tokens and buckets,
    every round's O and U equal the two-launch rounds' bit for bit, and the
    pool after deferred round r equals the two-launch pool before round r's
    commit."""
    from linear_attention_tree_amd import BucketedRound
    B, L, H, d = 4, 2, 4, 64
    buckets = [64, 128, 256]
    sets = [W.make_candidates(B, seed=50 + s) for s in range(3)]
    M_total = int(sets[0].cand_off[-1])
    ref = BucketedRound(B, L, H, d, d, torch.bfloat16, M_total, buckets)
    dfr = BucketedRound(B, L, H, d, d, torch.bfloat16, M_total, buckets, deferred=True)
    cmax = buckets[-1]
    rng = np.random.default_rng(9)
    n_slots = B + 2
    pool0 = torch.from_numpy((0.2 * rng.standard_normal((L, n_slots, H, d, d))).astype(np.float32))
    slot = torch.from_numpy(np.array([3, 0, 5, 1], np.int32)).cuda()
    pool_r, pool_d = pool0.clone().cuda(), pool0.clone().cuda()

    def load(rnd, c, toks):
        rnd.cand_parent.copy_(torch.from_numpy(c.cand_parent).cuda())
        rnd.p_draft.copy_(torch.from_numpy(c.p_draft).cuda())
        rnd.cand_off.copy_(torch.from_numpy(c.cand_off).cuda())
        for nm, a in toks.items():
            rnd.tokens()[nm].copy_(a)

    def draw_tokens():
        q = rng.standard_normal((L, cmax, H, d)).astype(np.float32)
        k = rng.standard_normal((L, cmax, H, d)).astype(np.float32)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((L, cmax, H, d)).astype(np.float32)
        g = (-np.logaddexp(0.0, rng.standard_normal((L, cmax, H)))).astype(np.float32)
        beta = (1 / (1 + np.exp(-rng.standard_normal((L, cmax, H))))).astype(np.float32)
        out = {}
        for nm, a in (("q", q), ("k", k), ("v", v)):
            bits, _ = W.round_storage(a, "bf16")
            out[nm] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        out["g"] = torch.from_numpy(g).cuda()
        out["beta"] = torch.from_numpy(beta).cuda()
        return out

    toks = draw_tokens()
    load(ref, sets[0], toks)
    load(dfr, sets[0], toks)
    dfr.tokens(1 - dfr.parity)["k"].copy_(toks["k"])
    ref.accept.fill_(-1)
    dfr.accept.fill_(-1)
    ref.capture(pool_r, slot)
    dfr.capture(pool_d, slot)
    torch.cuda.synchronize()
    assert int(ref.err.item()) == 0 and int(dfr.err.item()) == 0
    pool_r.copy_(pool0)
    pool_d.copy_(pool0)
    prev_accept = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    for r, (si, budget) in enumerate(((0, 100), (1, 60), (2, 256), (1, 128), (0, 200))):
        c = sets[si]
        cap = ref.bucket(budget)
        f = OF.build_forest(c.cand_parent, c.p_draft, c.cand_off, cap, 64)
        accept = torch.from_numpy((np.diff(f["tree_off"]) - 1).astype(np.int32)).cuda()
        toks = draw_tokens()
        load(ref, c, toks)
        load(dfr, c, toks)
        ref.accept.copy_(accept)        # committed at the end of its round
        dfr.accept.copy_(prev_accept)   # the previous round's, committed first
        before = pool_r.clone()
        par = dfr.parity
        assert ref.replay(budget) == cap and dfr.replay(budget) == cap
        torch.cuda.synchronize()
        say(f"deferred bucketed round {r}: set {si}, bucket {cap}")
        assert int(ref.err.item()) == 0 and int(dfr.err.item()) == 0
        assert torch.equal(ref.O[:, :cap].view(torch.int16), dfr.O[:, :cap].view(torch.int16))
        assert torch.equal(ref.U[:, :cap].view(torch.int32),
                           dfr.tokens(par)["U"][:, :cap].view(torch.int32))
        assert torch.equal(pool_d.view(torch.int32), before.view(torch.int32))
        prev_accept = accept
