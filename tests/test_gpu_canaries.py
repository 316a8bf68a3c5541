"""Guard canaries: no kernel writes outside its outputs, and a rejected tree's
rows stay untouched.

Every output buffer of every call sits inside an allocation with 256 poisoned
bytes (two 128-byte lines) before and after it, and its own bytes start
poisoned too.  After each call the guards must be bit-unchanged; the rows of a
tree that preparation rejects (a cycle) must still hold the poison where the
header promises no output for it; and every other value must equal, bit for
bit, the same call on ordinary buffers.  Cases: a ragged forest, head
dimensions that leave value tiles, key chunks and channel blocks partly empty
(bf16 and float32), and a forest with a rejected tree between two valid ones.
"""

import sys

import numpy as np
import pytest

import workloads as W

from helpers import make_case, to_dev

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)

PAD = 256
POISON = 0xA5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Guarded:
    """A tensor whose bytes, and PAD bytes on each side of them, start as POISON."""

    def __init__(self, shape, dtype, dev="cuda", init=None):
        elem = torch.empty((), dtype=dtype).element_size()
        self.n = int(np.prod(shape)) * elem
        self.raw = torch.full((self.n + 2 * PAD,), POISON, dtype=torch.uint8, device=dev)
        self.t = self.raw[PAD:PAD + self.n].view(dtype).view(shape)
        if init is not None:
            self.t.copy_(init)

    def guards_intact(self):
        return bool((self.raw[:PAD] == POISON).all().item()
                    and (self.raw[PAD + self.n:] == POISON).all().item())

    def rows_poisoned(self, lo, hi):
        """Rows [lo, hi) along the first dimension still hold the poison."""
        per = self.n // self.t.shape[0]
        return bool((self.raw[PAD + lo * per:PAD + hi * per] == POISON).all().item())


def like(t):
    return torch.empty_like(t)


def rejected_forest():
    bad = np.array([-1, 2, 3, 1, 0], np.int32)  # nodes 1 -> 2 -> 3 -> 1: a cycle
    rng = np.random.default_rng(12)
    return W.forest_from_trees([W.random_tree(rng, 20, 6), bad, W.random_tree(rng, 64, 12)],
                               [7, 0, 40])


CASES = {
    "ragged": (W.CONFIGS["ragged"], None, 4),
    "dims_bf16": (W.Config("canary_bf16", 60, B=3, H=3, d_k=48, d_v=80, dtype="bf16",
                           tree="fixed", T=64, D=12, prefix=16), None, 3),
    "dims_f32": (W.Config("canary_f32", 61, B=3, H=3, d_k=32, d_v=48, dtype="f32",
                          tree="fixed", T=64, D=12, prefix=16), None, 3),
    "rejected": (W.Config("canary_bad", 62, B=3, H=2, d_k=64, d_v=64, dtype="bf16",
                          tree="fixed", T=64, D=12, prefix=16), rejected_forest, 2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_outputs_stay_inside_their_buffers(name):
    from linear_attention_tree_amd import bole
    cfg0, forest_fn, H = CASES[name]
    from dataclasses import replace
    cfg = replace(cfg0, H=H)
    forest = forest_fn() if forest_fn else W.make_forest(cfg, 0)
    bad = [] if forest_fn is None else [1]
    accept = forest.accept.copy()
    accept[bad] = -1
    case = make_case(cfg, forest=forest, n_layers=1, prefix_units=[])
    case.S_pre[0][:] = W.make_states(cfg, case.n_slots, 0, 0)
    f = case.forest
    N, B, dk, dv = f.N, f.B, cfg.d_k, cfg.d_v
    d = to_dev(case, 0)
    tdt = d["dtype"]
    dev = "cuda"
    say(f"canaries: {name} (N={N}, B={B}, H={H}, d_k={dk}, d_v={dv}, {cfg.dtype})")
    parent = torch.from_numpy(f.parent).to(dev)
    tree_off = torch.from_numpy(f.tree_off).to(dev)
    slot = torch.from_numpy(case.slot).to(dev)
    acc_t = torch.from_numpy(accept).to(dev)
    pool0 = torch.from_numpy(case.S_pre[0]).to(dev)
    fused = dk <= (128 if cfg.dtype == "bf16" else 64)
    bad_rows = [(int(f.tree_off[b]), int(f.tree_off[b + 1])) for b in bad]

    def topo_set(guard):
        mk = (lambda s, t: Guarded(s, t)) if guard else (lambda s, t: type(
            "Plain", (), {"t": torch.empty(s, dtype=t, device=dev)})())
        return dict(depth=mk((N,), torch.int32), anc=mk((N,), torch.int64),
                    order=mk((N,), torch.int32), tree_depth=mk((B,), torch.int32),
                    logP=mk((N, H), torch.float32))

    def outs(guard):
        mk = (lambda s, t: Guarded(s, t)) if guard else (lambda s, t: type(
            "Plain", (), {"t": torch.empty(s, dtype=t, device=dev)})())
        return dict(O=mk((N, H, dv), tdt), U=mk((N, H, dv), torch.float32))

    def run(guard):
        res, err = {}, torch.zeros(1, dtype=torch.int32, device=dev)
        tp = topo_set(guard)
        bole.bole_tree_prep(parent, tree_off, d["g"][None], tp["depth"].t, tp["anc"].t,
                            tp["order"].t, tp["tree_depth"].t, tp["logP"].t[None], err)
        res["prep"] = tp
        mkgc = (lambda: Guarded((B, H, 64, 64), torch.float32)) if guard else (lambda: type(
            "Plain", (), {"t": torch.empty(B, H, 64, 64, device=dev)})())
        G, C = mkgc(), mkgc()
        bole.bole_factor_gc(d["q"], d["k"], tp["logP"].t, d["beta"], tp["anc"].t, tp["order"].t,
                            tree_off, G.t, C.t, err)
        res["G"], res["C"] = G, C
        o = outs(guard)
        bole.bole_verify(d["q"], d["k"], d["v"], tp["logP"].t, d["beta"], pool0, slot, G.t, C.t,
                         tp["order"].t, tp["depth"].t, tree_off, tp["tree_depth"].t, o["O"].t,
                         o["U"].t, err)
        res["verify"] = o
        mkpool = (lambda: Guarded(pool0.shape, torch.float32, init=pool0)) if guard else (
            lambda: type("Plain", (), {"t": pool0.clone()})())
        pool_c = mkpool()
        kst, ust, lst = d["k"][None], o["U"].t[None], tp["logP"].t[None]
        bole.bole_commit_path(pool_c.t[None], slot, kst, ust, lst, tp["anc"].t, tree_off, acc_t,
                              err)
        res["commit_pool"] = pool_c
        if fused:
            o2 = outs(guard)
            bole.bole_factor_verify(d["q"], d["k"], d["v"], tp["logP"].t, d["beta"], pool0, slot,
                                    tp["anc"].t, tp["order"].t, tp["depth"].t, tree_off,
                                    tp["tree_depth"].t, o2["O"].t, o2["U"].t, err)
            res["factor_verify"] = o2
            o3, tp3 = outs(guard), topo_set(guard)
            bole.bole_tree_verify(d["q"], d["k"], d["v"], parent, d["g"], d["beta"], pool0, slot,
                                  tree_off, o3["O"].t, o3["U"].t, tp3["depth"].t, tp3["anc"].t,
                                  tp3["order"].t, tp3["tree_depth"].t, tp3["logP"].t, err)
            res["tree_verify"], res["tree_prep"] = o3, tp3
            o4, tp4 = outs(guard), topo_set(guard)
            pool_d = mkpool()
            bole.bole_commit_tree_verify(d["q"], d["k"], d["v"], parent, d["g"], d["beta"],
                                         pool_d.t, slot, tree_off, o4["O"].t, o4["U"].t,
                                         tp4["depth"].t, tp4["anc"].t, tp4["order"].t,
                                         tp4["tree_depth"].t, tp4["logP"].t, d["k"], o3["U"].t,
                                         tp3["logP"].t, tp3["anc"].t, tree_off, acc_t, err)
            res["commit_tree_verify"], res["ctv_prep"], res["ctv_pool"] = o4, tp4, pool_d
        # the tree convolution over a channel count that leaves the last block
        # partly empty, and its conv-state commit
        Cc, Wd = 8 * (H * (dk + dv) // 8 + 9), 4
        gen = torch.Generator(device=dev)
        gen.manual_seed(5)
        x = torch.randn(N, Cc, generator=gen, device=dev).to(tdt)
        st0 = torch.randn(case.n_slots, Wd - 1, Cc, generator=gen, device=dev).to(tdt)
        wgt = torch.randn(Cc, Wd, generator=gen, device=dev)
        bias = torch.randn(Cc, generator=gen, device=dev)
        y = Guarded((N, Cc), tdt) if guard else type("Plain", (), {"t": torch.empty(N, Cc, dtype=tdt, device=dev)})()
        bole.bole_tree_conv(x, wgt, bias, st0, slot, parent, tree_off, y.t, err)
        res["conv_y"] = y
        st = Guarded(st0.shape, tdt, init=st0) if guard else type("Plain", (), {"t": st0.clone()})()
        bole.bole_conv_commit(st.t, slot, x, parent, tree_off, acc_t, err)
        res["conv_state"] = st
        torch.cuda.synchronize()
        res["err"] = int(err.item())
        return res

    ref = run(False)
    got = run(True)
    assert got["err"] == ref["err"]
    assert bool(got["err"] & 2) == bool(bad)  # CYCLE reported exactly when a tree is rejected

    def flat(v):
        return {k: x for k, x in v.items()} if isinstance(v, dict) else {"": v}

    n_checked = 0
    for key, val in got.items():
        if key == "err":
            continue
        for sub, g in flat(val).items():
            label = f"{key}{'.' + sub if sub else ''}"
            assert g.guards_intact(), f"{label}: a guard line was written"
            r = flat(ref[key])[sub].t
            gt = g.t
            if key in ("G", "C"):  # the rejected tree's tiles are unspecified
                keep = [b for b in range(B) if b not in bad]
                gt, r = gt[keep], r[keep]
            elif key in ("verify", "factor_verify", "tree_verify", "commit_tree_verify", "conv_y"):
                for lo, hi in bad_rows:  # no output for a rejected tree
                    assert g.rows_poisoned(lo, hi), f"{label}: rows of the rejected tree written"
                rows = np.ones(N, bool)
                for lo, hi in bad_rows:
                    rows[lo:hi] = False
                gt, r = gt[torch.from_numpy(rows).to(dev)], r[torch.from_numpy(rows).to(dev)]
            elif key in ("prep", "tree_prep", "ctv_prep") and bad_rows:
                rows = np.ones(gt.shape[0], bool)
                if sub == "tree_depth":
                    assert int(gt[1].item()) == -1
                    rows[1] = False
                else:
                    for lo, hi in bad_rows:
                        rows[lo:hi] = False
                gt, r = gt[torch.from_numpy(rows).to(dev)], r[torch.from_numpy(rows).to(dev)]
            a = gt.contiguous().view(torch.uint8)
            b = r.contiguous().view(torch.uint8)
            assert torch.equal(a, b), f"{label}: differs from the call on ordinary buffers"
            n_checked += 1
    say(f"  {n_checked} guarded outputs intact and bit-identical")
