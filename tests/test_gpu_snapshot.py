"""The per-node snapshot verifier (the measurement baseline the bench runs
beside the closed-form path) against the float64 oracle: O, U, the committed
state, and the stored snapshots of chosen nodes (each equals the oracle's
walked state after that node), on the float32 exactness case, the bf16
workloads and one layer of the multi-layer round's shape (32 trees x 64 nodes,
32 heads).  Bars as for the library: 1e-4 for float32 tokens, 2e-2 for bf16.
Also the streaming kernel the bench sets the verify kernels against: it reads
and writes every vector it is given."""

import sys

import numpy as np
import pytest

import oracle
import workloads as W

from helpers import block_rel_err, make_case, state_rel_err, to_dev, tolerance

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_snapshot(case):
    from linear_attention_tree_amd.baselines import SnapshotVerifier
    f, cfg = case.forest, case.cfg
    d = to_dev(case, 0)
    sv = SnapshotVerifier(f.parent, f.tree_off, cfg.H)
    pool = torch.from_numpy(case.S_pre[0]).cuda()
    slot = torch.from_numpy(case.slot).cuda()
    snap = torch.empty(f.N, cfg.H, cfg.d_v, cfg.d_k, dtype=torch.float32, device="cuda")
    O = torch.empty(f.N, cfg.H, cfg.d_v, dtype=d["v"].dtype, device="cuda")
    U = torch.empty(f.N, cfg.H, cfg.d_v, dtype=torch.float32, device="cuda")
    sv.layer(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, slot, snap, O, U)
    sv.commit(snap, pool, slot, torch.from_numpy(f.accept).cuda())
    torch.cuda.synchronize()
    return (O.float().cpu().numpy(), U.cpu().numpy(), pool.cpu().numpy(), snap.cpu().numpy())


def check(case, label):
    f, cfg = case.forest, case.cfg
    tol = tolerance(cfg)
    O, U, pool, snap = run_snapshot(case)
    x = case.layers[0]
    args = (f.parent, f.tree_off, x.q64, x.k64, x.v64, x.g64, x.beta64, case.S_pre[0], case.slot)
    O_ref, U_ref, S_ref = oracle.verify(*args, f.accept)
    units = [(b, h) for b in range(f.B) for h in range(cfg.H)]
    eo = block_rel_err(O, O_ref, f.tree_off)
    eu = block_rel_err(U, U_ref, f.tree_off)
    es = state_rel_err(pool, S_ref, case.slot, units)
    # another node of every tree (its last): its stored snapshot is the
    # oracle's state after it
    last = (np.diff(f.tree_off) - 1).astype(np.int32)
    _, _, S_last = oracle.verify(*args, last)
    snap_last = snap[f.tree_off[:-1] + last]
    en = max(float(np.max(np.abs(snap_last[b, h] - S_last[b, h])) / np.max(np.abs(S_last[b, h])))
             for b, h in units)
    say(f"  {label}: O {eo:.2e}  U {eu:.2e}  committed {es:.2e}  snapshots {en:.2e}  (bar {tol:g})")
    assert max(eo, eu, es, en) <= tol
    free = sorted(set(range(case.n_slots)) - set(case.slot.tolist()))
    for s in free:
        assert np.array_equal(pool[s], case.S_pre[0][s])


@pytest.mark.parametrize("name", ["tiny", "decode", "batched", "ragged"])
def test_snapshot_verifier_matches_oracle(name):
    say(f"snapshot verifier: {name}")
    check(make_case(name, n_layers=1), name)


@pytest.mark.timeout(600)
def test_snapshot_verifier_at_multilayer_shape():
    """One layer at the multi-layer round's shape (states drawn directly)."""
    from helpers import Case
    cfg = W.CONFIGS["multilayer"]
    f = W.make_forest(cfg, 0)
    n_slots = f.B + 2
    slot = np.random.default_rng(4).permutation(n_slots)[:f.B].astype(np.int32)
    case = Case(cfg=cfg, forest=f, layers=[W.make_layer(cfg, f.N, 0, 0)],
                S_pre=[W.make_states(cfg, n_slots, 0, 0)], slot=slot, n_slots=n_slots)
    say("snapshot verifier: one layer of 32 trees x 64 nodes, 32 heads")
    check(case, "multilayer shape")


@pytest.mark.parametrize("n_read,n_write,grid,block", [(1000, 777, 3, 64), (4096, 4096, 8, 256),
                                                        (0, 100, 2, 128), (50, 0, 1, 64)])
def test_stream_mix_moves_every_vector(n_read, n_write, grid, block):
    """Written vector i holds, in components 1..3, the number of source vectors
    its thread read (a source of ones; thread i mod threads reads the indices
    congruent to it), and in component 0 that count plus i; nothing past
    n_write is touched."""
    from linear_attention_tree_amd.baselines import stream_mix
    say(f"stream_mix read {n_read} write {n_write} grid {grid} block {block}")
    src = torch.ones(max(n_read, 1) * 4, dtype=torch.float32, device="cuda")
    dst = torch.full(((n_write + 8) * 4,), -7.0, dtype=torch.float32, device="cuda")
    stream_mix(src, dst, n_read, n_write, grid, block)
    torch.cuda.synchronize()
    out = dst.view(-1, 4).cpu().numpy()
    nt = grid * block
    i = np.arange(n_write)
    tid = i % nt
    count = np.where(tid < n_read, (n_read - 1 - tid) // nt + 1, 0).astype(np.float32)
    assert np.array_equal(out[:n_write, 1], count)
    assert np.array_equal(out[:n_write, 3], count)
    assert np.array_equal(out[:n_write, 0], count + i.astype(np.float32))
    assert np.all(out[n_write:] == -7.0)
