"""GPU parity of the multi-layer round at full shape: 36 GDN layers, 32 trees of
64 nodes (depth <= 12), 32 heads, d_k = d_v = 128, bf16 q/k/v, two rounds,
every (layer, request, head) unit checked against the float64 oracle.

Round 1 runs 36 x bole_tree_verify on the first forest (and, on the same
states, the two-call bole_factor_gc + bole_verify path).  Round 2 runs 36 x
bole_commit_tree_verify on a second forest: each launch commits round 1's
accepted path of its layer into the slot and verifies round 2's tree against
the committed state.  One bole_commit_path over all layers then commits round
2.  Checked per layer: round 1's O and U (both paths), the state round 2's
launches committed, round 2's O and U (the oracle run from its own round-1
state), the final committed state, untouched free slots, and the preparation
outputs of both forests bit for bit.

The committed states are drawn directly (workloads.make_states, at the spread
the prefix recipe produces) instead of from 256 prefix tokens per unit, so the
oracle can check every unit; the token operands of each layer serve both
rounds (the rounds' trees differ).
"""

import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import workloads as W

from helpers import block_rel_err, state_rel_err, tolerance

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tok(a, dev):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)


@pytest.mark.timeout(900)
def test_multilayer_full_shape_two_rounds():
    from linear_attention_tree_amd import TreeRound
    cfg = W.CONFIGS["multilayer"]
    L, H, dk, dv = cfg.L, cfg.H, cfg.d_k, cfg.d_v
    f1, f2 = W.make_forest(cfg, 0), W.make_forest(cfg, 1)
    B, N = f1.B, f1.N
    assert f2.N == N
    n_slots = B + 2
    slot = np.random.default_rng(3).permutation(n_slots)[:B].astype(np.int32)
    free = sorted(set(range(n_slots)) - set(slot.tolist()))
    dev = torch.device("cuda:0")
    t0 = time.time()
    say(f"multilayer full shape: L={L} B={B} T={cfg.T} H={H} d={dk}; generating tokens")
    with ThreadPoolExecutor(8) as ex:
        layers = list(ex.map(lambda l: W.make_layer(cfg, N, l, 0), range(L)))
    say(f"  tokens generated ({time.time() - t0:.1f} s)")

    q = torch.stack([_tok(x.q, dev) for x in layers])
    k = torch.stack([_tok(x.k, dev) for x in layers])
    v = torch.stack([_tok(x.v, dev) for x in layers])
    g = torch.stack([torch.from_numpy(x.g) for x in layers]).to(dev)
    beta = torch.stack([torch.from_numpy(x.beta) for x in layers]).to(dev)
    pool = torch.empty(L, n_slots, H, dv, dk, dtype=torch.float32, device=dev)
    for l in range(L):
        pool[l].copy_(torch.from_numpy(W.make_states(cfg, n_slots, l, 0)))
    slot_d = torch.from_numpy(slot).to(dev)
    r1 = TreeRound(f1.parent, f1.tree_off, H, device=dev)
    r2 = TreeRound(f2.parent, f2.tree_off, H, device=dev)
    O1 = torch.empty(L, N, H, dv, dtype=torch.bfloat16, device=dev)
    U1 = torch.empty(L, N, H, dv, dtype=torch.float32, device=dev)
    O1s, U1s = torch.empty_like(O1), torch.empty_like(U1)
    O2, U2 = torch.empty_like(O1), torch.empty_like(U1)
    logP1 = torch.empty(L, N, H, dtype=torch.float32, device=dev)
    logP2 = torch.empty_like(logP1)

    say("  round 1: 36 x bole_tree_verify, then the two-call path on the same states")
    for l in range(L):
        r1.tree_layer(q[l], k[l], v[l], g[l], beta[l], pool[l], slot_d, O=O1[l], U=U1[l],
                      logP=logP1[l])
    for l in range(L):
        r1.layer(q[l], k[l], v[l], logP1[l], beta[l], pool[l], slot_d, O=O1s[l], U=U1s[l])
    say("  round 2: 36 x bole_commit_tree_verify (round 1's commit inside)")
    for l in range(L):
        r2.commit_tree_layer(r1, k[l], U1[l], logP1[l], f1.accept, q[l], k[l], v[l], g[l],
                             beta[l], pool[l], slot_d, O=O2[l], U=U2[l], logP=logP2[l])
    torch.cuda.synchronize()
    S1_gpu = pool.cpu().numpy()
    say("  commit of round 2 over all layers (bole_commit_path)")
    r2.commit(pool, slot_d, k, U2, logP2, f2.accept)
    torch.cuda.synchronize()
    S2_gpu = pool.cpu().numpy()
    del pool
    assert r1.error_bits() == 0 and r2.error_bits() == 0

    # preparation outputs of both forests, bit for bit (logP of every layer)
    g_host = np.stack([x.g for x in layers])
    for rnd, f, lp in ((r1, f1, logP1), (r2, f2, logP2)):
        ref = oracle.tree_prep(f.parent, f.tree_off, g_host)
        assert ref["err"] == 0
        assert np.array_equal(rnd.topo.depth.cpu().numpy(), ref["depth"])
        assert np.array_equal(rnd.topo.anc.cpu().numpy().view(np.uint64), ref["anc"])
        assert np.array_equal(rnd.topo.order.cpu().numpy(), ref["order"])
        assert np.array_equal(rnd.topo.tree_depth.cpu().numpy(), ref["tree_depth"])
        assert np.array_equal(lp.cpu().numpy().view(np.uint32), ref["logP"].view(np.uint32))
    say(f"  preparation bit-exact for both forests ({time.time() - t0:.1f} s)")

    tol = tolerance(cfg)
    units = [(b, h) for b in range(B) for h in range(H)]
    worst = dict(O1=0.0, U1=0.0, O1s=0.0, U1s=0.0, S1=0.0, O2=0.0, U2=0.0, S2=0.0)
    for l in range(L):
        x = layers[l]
        q64, k64, v64, g64, b64 = x.q64, x.k64, x.v64, x.g64, x.beta64
        S0 = W.make_states(cfg, n_slots, l, 0)
        O1r, U1r, S1r = oracle.verify(f1.parent, f1.tree_off, q64, k64, v64, g64, b64, S0, slot,
                                      f1.accept)
        S1p = S0.copy()
        S1p[slot] = S1r.astype(np.float32)
        O2r, U2r, S2r = oracle.verify(f2.parent, f2.tree_off, q64, k64, v64, g64, b64, S1p, slot,
                                      f2.accept)
        e = dict(
            O1=block_rel_err(O1[l].float().cpu().numpy(), O1r, f1.tree_off),
            U1=block_rel_err(U1[l].cpu().numpy(), U1r, f1.tree_off),
            O1s=block_rel_err(O1s[l].float().cpu().numpy(), O1r, f1.tree_off),
            U1s=block_rel_err(U1s[l].cpu().numpy(), U1r, f1.tree_off),
            S1=state_rel_err(S1_gpu[l], S1r, slot, units),
            O2=block_rel_err(O2[l].float().cpu().numpy(), O2r, f2.tree_off),
            U2=block_rel_err(U2[l].cpu().numpy(), U2r, f2.tree_off),
            S2=state_rel_err(S2_gpu[l], S2r, slot, units))
        for key, val in e.items():
            worst[key] = max(worst[key], val)
        if l % 6 == 5 or any(not (val <= tol) for val in e.values()):
            say(f"  layer {l}: " + " ".join(f"{key} {val:.2e}" for key, val in e.items())
                + f" ({time.time() - t0:.1f} s)")
        assert all(val <= tol for val in e.values()), (l, e)
        for s in free:  # slots no request owns are never written
            assert np.array_equal(S1_gpu[l][s], S0[s]) and np.array_equal(S2_gpu[l][s], S0[s])
    say("  worst over 36 layers: " + " ".join(f"{key} {val:.2e}" for key, val in worst.items())
        + f" (bar {tol:g})")
