"""Shared test plumbing: build seeded cases, run the oracle, run the HIP library.

The oracle and the library see exactly the same stored values (workloads
rounds them); committed prefix states for the cases come from the oracle's
token-order decoding of seeded prefix tokens, never from the library.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

import oracle
import workloads as W


@dataclass
class Case:
    cfg: W.Config
    forest: W.Forest
    layers: List[W.LayerInputs]
    S_pre: List[np.ndarray]     # per layer [n_slots, H, d_v, d_k] float32
    slot: np.ndarray            # [B] int32
    n_slots: int

    @property
    def B(self):
        return self.forest.B

    @property
    def N(self):
        return self.forest.N


def prefix_slots(cfg: W.Config, layer: int, n_slots: int, slot: np.ndarray, seed: int,
                 units: Optional[Sequence[Tuple[int, int]]] = None) -> np.ndarray:
    """State pool for one layer; slot[b] of head h holds the oracle's prefix state
    for (b, h).  Units not listed (when `units` is given) stay zero."""
    S = np.zeros((n_slots, cfg.H, cfg.d_v, cfg.d_k), np.float32)
    todo = [(b, h) for b in range(len(slot)) for h in range(cfg.H)] if units is None else list(units)
    if not todo or cfg.prefix == 0:
        return S
    toks = [W.make_prefix(cfg, layer, b, h, seed) for (b, h) in todo]
    st = oracle.prefix_states(np.stack([t.k64 for t in toks]), np.stack([t.v64 for t in toks]),
                              np.stack([t.g64 for t in toks]), np.stack([t.beta64 for t in toks]))
    for (b, h), s in zip(todo, st):
        S[slot[b], h] = s.astype(np.float32)
    return S


def make_case(name, seed: int = 0, n_layers: Optional[int] = None, forest=None,
              prefix_units=None, extra_slots: int = 3) -> Case:
    """`name` is a workload name or a Config."""
    cfg = W.CONFIGS[name] if isinstance(name, str) else name
    forest = forest if forest is not None else W.make_forest(cfg, seed)
    L = cfg.L if n_layers is None else n_layers
    layers = [W.make_layer(cfg, forest.N, l, seed) for l in range(L)]
    n_slots = forest.B + extra_slots
    rng = np.random.default_rng([seed, 99])
    slot = rng.permutation(n_slots)[: forest.B].astype(np.int32)
    S_pre = [prefix_slots(cfg, l, n_slots, slot, seed, prefix_units) for l in range(L)]
    return Case(cfg=cfg, forest=forest, layers=layers, S_pre=S_pre, slot=slot, n_slots=n_slots)


def oracle_layer(case: Case, l: int, units=None, accept=True):
    """fp64 walk oracle for layer l: (O, U, S_new or None)."""
    x = case.layers[l]
    f = case.forest
    return oracle.verify(f.parent, f.tree_off, x.q64, x.k64, x.v64, x.g64, x.beta64,
                         case.S_pre[l], case.slot, f.accept if accept else None, units)


def block_rel_err(x: np.ndarray, ref: np.ndarray, tree_off: np.ndarray, units=None) -> float:
    """max over (tree, head) blocks of max|x - ref| / max|ref| (rows = tree nodes)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    B = len(tree_off) - 1
    H = ref.shape[1]
    starts = np.asarray(tree_off[:-1], np.int64)
    if units is None and B > 0 and np.all(np.diff(tree_off) > 0) and tree_off[-1] == len(ref):
        # every block at once: per-row maxima over d, then per-tree maxima
        d = np.maximum.reduceat(np.max(np.abs(x - ref), axis=2), starts, axis=0)
        den = np.maximum.reduceat(np.max(np.abs(ref), axis=2), starts, axis=0)
        rel = np.where(den > 0, d / np.where(den > 0, den, 1.0), d)
        if np.isnan(rel).any():
            return float("nan")
        return float(np.max(rel))
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(H)]
    worst = 0.0
    for b, h in todo:
        sl = slice(tree_off[b], tree_off[b + 1])
        d = np.max(np.abs(x[sl, h] - ref[sl, h]))
        den = np.max(np.abs(ref[sl, h]))
        worst = max(worst, float(d / den) if den > 0 else float(d))
    return worst


def state_rel_err(S_gpu: np.ndarray, S_ref: np.ndarray, slot, units) -> float:
    """max over the listed (request, head) units of max|S - ref| / max|ref| over
    the unit's d_v x d_k state; S_gpu is a slot pool, S_ref per request."""
    if len(set(units)) == len(slot) * S_ref.shape[1]:  # every unit at once
        a = np.asarray(S_gpu[np.asarray(slot)], np.float64)
        r = np.asarray(S_ref, np.float64)
        d = np.max(np.abs(a - r), axis=(2, 3))
        den = np.maximum(np.max(np.abs(r), axis=(2, 3)), 1e-300)
        out = d / den
        return float("nan") if np.isnan(out).any() else float(np.max(out))
    worst = 0.0
    for b, h in units:
        a = np.asarray(S_gpu[slot[b], h], np.float64)
        r = S_ref[b, h]
        worst = max(worst, float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-300)))
    return worst


def tolerance(cfg: W.Config) -> float:
    """Bar from the benchmark spec: 1e-4 for float32 inputs, 2e-2 for bf16 q/k/v."""
    return 1e-4 if cfg.dtype == "f32" else 2e-2


# ---------------------------------------------------------------------------
# device side (imports torch lazily so CPU-only tests never touch it)

def to_dev(case: Case, l: int, device="cuda"):
    import torch
    x = case.layers[l]
    tdt = torch.float32 if x.dtype == "f32" else torch.bfloat16

    def tok(a):
        a = np.ascontiguousarray(a)
        if x.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).to(device)

    return dict(q=tok(x.q), k=tok(x.k), v=tok(x.v),
                g=torch.from_numpy(x.g).to(device), beta=torch.from_numpy(x.beta).to(device),
                dtype=tdt)


def offset_copy(t, dtype=None):
    """t's values in a contiguous buffer that starts one element past the
    allocation, so it is not 16-byte aligned."""
    import torch
    flat = torch.zeros(t.numel() + 1, dtype=dtype or t.dtype, device=t.device)
    view = flat[1:].view(t.shape)
    view.copy_(t)
    return view


def gpu_round(case: Case, layers=None, commit=True, device="cuda", fused=False, misalign=False,
              tree=False, solve="blocked"):
    """Run prep, factor, verify (and commit) on the GPU through the C ABI.

    fused: bole_factor_verify after bole_tree_prep; tree: bole_tree_verify per
    layer (preparation inside the verify launch).  misalign: v, O and U live one
    element past an aligned address (the kernels' element-wise fallbacks).
    solve: the two-call path's solve ("blocked", "neumann" or "inverse"; G and
    C in the result then hold W and M).  Returns dict with per-layer O, U (numpy float64), the state pools after
    commit, the prep outputs and the error word."""
    import torch
    from linear_attention_tree_amd import TreeRound
    f = case.forest
    layers = list(range(len(case.layers))) if layers is None else list(layers)
    rnd = TreeRound(f.parent, f.tree_off, case.cfg.H, device=device)
    dev = [to_dev(case, l, device) for l in layers]
    g_all = torch.stack([d["g"] for d in dev])
    logP = torch.empty_like(g_all) if tree else rnd.prep(g_all)
    slot = torch.from_numpy(case.slot).to(device)
    pools = torch.stack([torch.from_numpy(case.S_pre[l]) for l in layers]).to(device)
    Os, Us = [], []
    for li, d in enumerate(dev):
        v, O, U = d["v"], None, None
        if misalign:
            v = offset_copy(v)
            O = offset_copy(torch.empty_like(v))
            U = offset_copy(torch.empty(v.shape, dtype=torch.float32, device=v.device))
        if tree:
            O, U, _ = rnd.tree_layer(d["q"], d["k"], v, d["g"], d["beta"], pools[li], slot, O=O,
                                     U=U, logP=logP[li])
        else:
            O, U = rnd.layer(d["q"], d["k"], v, logP[li], d["beta"], pools[li], slot, O=O, U=U,
                             fused=fused, solve=solve)
        Os.append(O)
        Us.append(U)
    out = dict(logP=logP.cpu().numpy(), depth=rnd.topo.depth.cpu().numpy(),
               anc=rnd.topo.anc.cpu().numpy().view(np.uint64),
               order=rnd.topo.order.cpu().numpy(), tree_depth=rnd.topo.tree_depth.cpu().numpy(),
               G=rnd.G.cpu().numpy(), C=rnd.C.cpu().numpy())
    out["O"] = [o.float().cpu().numpy().astype(np.float64) for o in Os]
    out["U"] = [u.cpu().numpy().astype(np.float64) for u in Us]
    if commit:
        kst = torch.stack([d["k"] for d in dev])
        ust = torch.stack(Us)
        rnd.commit(pools, slot, kst, ust, logP, f.accept)
    torch.cuda.synchronize()
    out["S"] = pools.cpu().numpy()
    out["err"] = rnd.error_bits()
    return out
