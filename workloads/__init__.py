"""Seeded synthetic workloads for closed-form tree verification of Gated DeltaNet layers.

This module only draws random numbers and rounds them to the storage types the
library consumes.  It holds none of the method's arithmetic: no recurrence, no
gate products, no factors.  Both the CPU oracle (``oracle/``) and the HIP
library read their inputs from here, so the two see exactly the same bits.

Workload shapes follow the five verification settings studied on the pages
(Bole, arXiv 2608.01651: single-request decode, batched verify, ragged forests,
a multi-layer round) plus the B=16/T=64 headline shape.  Trees are random
recursive trees with a depth cap, which stand in for the drafter-built proposal
trees of the paper's evaluation (no drafter or dataset is used).

Value distributions (per node and head):
  q, k ~ N(0, 1), then L2-normalised over the key dimension,
  v ~ N(0, 1),
  g = log(gamma) = -softplus(x) with x ~ N(mu_x, 1)  (mu_x = 0, or -3 for the
      deep-chain stress setting so that gamma sits near 1),
  beta = sigmoid(N(0, 1)).
q, k, v are drawn and normalised in float32; gates are computed in float64 and
rounded to float32.  For bf16 workloads q/k/v are then rounded to bfloat16
(round to nearest even).  Both sides receive exactly these stored values.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

# RNG stream ids (part of the SeedSequence entropy).
STREAM_TOPOLOGY = 0
STREAM_TOKENS = 1
STREAM_PREFIX = 2
STREAM_ACCEPT = 3

MAX_TREE = 64  # one 64-bit ancestor mask per node


@dataclass(frozen=True)
class Config:
    name: str
    cid: int            # entropy id for the seed sequence
    B: int              # requests (trees)
    H: int              # state heads
    d_k: int
    d_v: int
    dtype: str          # "f32" or "bf16" for q/k/v (gates and state are always f32)
    tree: str           # "heap7" | "fixed" | "ragged"
    T: int              # nodes per tree (fixed) or max size (ragged)
    D: int              # depth cap: a new node's parent has depth < D
    prefix: int         # prefix tokens used to build the committed state
    L: int = 1          # GDN layers in the round
    gate_mu: float = 0.0
    T_min: int = 0      # ragged: smallest tree
    N_cap: int = 0      # ragged: total node cap


CONFIGS: Dict[str, Config] = {
    # Exactness case: full binary tree of 7 nodes, float32 everything.
    "tiny": Config("tiny", 1, B=1, H=1, d_k=16, d_v=16, dtype="f32", tree="heap7",
                   T=7, D=2, prefix=32),
    # Single-request decode shape.
    "decode": Config("decode", 2, B=1, H=16, d_k=128, d_v=128, dtype="bf16",
                     tree="fixed", T=8, D=4, prefix=256),
    # Batched verify, 16 trees of 32 nodes.
    "batched": Config("batched", 3, B=16, H=32, d_k=128, d_v=128, dtype="bf16",
                      tree="fixed", T=32, D=8, prefix=256),
    # Ragged forest, sizes 8..64, deep chains with gates near one.
    "ragged": Config("ragged", 4, B=16, H=32, d_k=128, d_v=128, dtype="bf16",
                     tree="ragged", T=64, D=16, prefix=256, gate_mu=-3.0,
                     T_min=8, N_cap=768),
    # Multi-layer round: 36 layers, 32 trees of 64 nodes.
    "multilayer": Config("multilayer", 5, B=32, H=32, d_k=128, d_v=128, dtype="bf16",
                         tree="fixed", T=64, D=12, prefix=256, L=36),
    # Headline throughput shape: the multi-layer tree rule at 16 requests, one layer.
    "target": Config("target", 6, B=16, H=32, d_k=128, d_v=128, dtype="bf16",
                     tree="fixed", T=64, D=12, prefix=256),
}


def _rng(seed: int, cfg: Config, stream: int, *more: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg.cid, stream, *more]))


# ----------------------------------------------------------------------------
# rounding helpers (storage formats only)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even); returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in workload")
    u = x.view(np.uint32)
    # finite inputs cannot carry past bit 31
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float -> storage array (float32, or uint16 bfloat16 bit patterns)."""
    x32 = np.asarray(x).astype(np.float32, copy=False)
    if dtype == "f32":
        return np.ascontiguousarray(x32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def widen(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 copy of exactly the stored values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    return np.asarray(stored, dtype=np.float64)


def round_storage(x: np.ndarray, dtype: str):
    """float -> (storage array, float64 view of exactly the stored values)."""
    st = to_storage(x, dtype)
    return st, widen(st, dtype)


# ----------------------------------------------------------------------------
# topology

def random_tree(rng: np.random.Generator, T: int, D: int) -> np.ndarray:
    """Random recursive tree: node 0 is the root; node i picks its parent uniformly
    among earlier nodes whose depth is below D.  Parents precede children."""
    parent = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int32)
    for i in range(1, T):
        cand = np.nonzero(depth[:i] < D)[0]
        p = int(cand[rng.integers(len(cand))])
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


@dataclass
class Forest:
    parent: np.ndarray      # [N] int32, local parent index, -1 for the root
    tree_off: np.ndarray    # [B+1] int32
    accept: np.ndarray      # [B] int32, last accepted local node (-1 = none)

    @property
    def B(self) -> int:
        return len(self.tree_off) - 1

    @property
    def N(self) -> int:
        return int(self.tree_off[-1])

    def sizes(self) -> np.ndarray:
        return np.diff(self.tree_off)


def make_forest(cfg: Config, seed: int = 0) -> Forest:
    rng = _rng(seed, cfg, STREAM_TOPOLOGY)
    if cfg.tree == "heap7":
        trees = [np.array([-1, 0, 0, 1, 1, 2, 2], dtype=np.int32)] * cfg.B
    elif cfg.tree == "fixed":
        trees = [random_tree(rng, cfg.T, cfg.D) for _ in range(cfg.B)]
    elif cfg.tree == "ragged":
        while True:
            sizes = rng.integers(cfg.T_min, cfg.T + 1, size=cfg.B)
            if sizes.sum() <= cfg.N_cap:
                break
        trees = [random_tree(rng, int(t), cfg.D) for t in sizes]
    else:
        raise ValueError(cfg.tree)
    off = np.zeros(cfg.B + 1, dtype=np.int32)
    off[1:] = np.cumsum([len(t) for t in trees])
    parent = np.concatenate(trees).astype(np.int32)
    if cfg.tree == "heap7":
        accept = np.full(cfg.B, 3, dtype=np.int32)  # root -> leftmost leaf
    else:
        arng = _rng(seed, cfg, STREAM_ACCEPT)
        accept = np.array([arng.integers(len(t)) for t in trees], dtype=np.int32)
    return Forest(parent=parent, tree_off=off, accept=accept)


# ----------------------------------------------------------------------------
# per-layer token operands

def _unit_rows(rng, n, d):
    x = rng.standard_normal((n, d), dtype=np.float32)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x


def _gates(rng, shape, mu):
    x = rng.standard_normal(shape) + mu
    g = -(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))   # -softplus(x)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(shape)))
    return g, beta


@dataclass
class LayerInputs:
    """Token operands of one GDN layer, token-major [N, H, d]."""
    q: np.ndarray           # storage (float32 or uint16 bf16 bits)
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray           # [N, H] float32, log of the decay gate
    beta: np.ndarray        # [N, H] float32
    dtype: str

    @property
    def q64(self):          # float64 copies of exactly the stored values
        return widen(self.q, self.dtype)

    @property
    def k64(self):
        return widen(self.k, self.dtype)

    @property
    def v64(self):
        return widen(self.v, self.dtype)

    @property
    def g64(self):
        return self.g.astype(np.float64)

    @property
    def beta64(self):
        return self.beta.astype(np.float64)


def make_layer(cfg: Config, N: int, layer: int = 0, seed: int = 0) -> LayerInputs:
    rng = _rng(seed, cfg, STREAM_TOKENS, layer)
    H = cfg.H
    q = _unit_rows(rng, N * H, cfg.d_k).reshape(N, H, cfg.d_k)
    k = _unit_rows(rng, N * H, cfg.d_k).reshape(N, H, cfg.d_k)
    v = rng.standard_normal((N, H, cfg.d_v), dtype=np.float32)
    g, beta = _gates(rng, (N, H), cfg.gate_mu)
    return LayerInputs(q=to_storage(q, cfg.dtype), k=to_storage(k, cfg.dtype),
                       v=to_storage(v, cfg.dtype), g=g.astype(np.float32),
                       beta=beta.astype(np.float32), dtype=cfg.dtype)


@dataclass
class PrefixTokens:
    """Committed-prefix tokens of one (layer, request, head) state, [P, d]."""
    q64: np.ndarray
    k64: np.ndarray
    v64: np.ndarray
    g64: np.ndarray
    beta64: np.ndarray


def make_prefix(cfg: Config, layer: int, b: int, h: int, seed: int = 0) -> PrefixTokens:
    """Tokens that precede the tree for one state head.  The committed state the
    tree starts from is the result of running the sequential recurrence over
    them from a zero state (done by the caller)."""
    rng = _rng(seed, cfg, STREAM_PREFIX, layer, b, h)
    P = cfg.prefix
    q = _unit_rows(rng, P, cfg.d_k)
    k = _unit_rows(rng, P, cfg.d_k)
    v = rng.standard_normal((P, cfg.d_v), dtype=np.float32)
    g, beta = _gates(rng, (P,), cfg.gate_mu)
    return PrefixTokens(q64=round_storage(q, cfg.dtype)[1], k64=round_storage(k, cfg.dtype)[1],
                        v64=round_storage(v, cfg.dtype)[1],
                        g64=g.astype(np.float32).astype(np.float64),
                        beta64=beta.astype(np.float32).astype(np.float64))


# Spread of the committed states the prefix recipe produces (256 prefix tokens
# of the default gates from a zero state: entries with standard deviation
# about 0.06, largest magnitudes about 0.6).
STATE_STD = 0.06


def make_states(cfg: Config, n_slots: int, layer: int = 0, seed: int = 0,
                std: float = STATE_STD) -> np.ndarray:
    """Committed states drawn directly, [n_slots, H, d_v, d_k] float32 with
    N(0, std^2) entries: a stand-in for prefix-built states where running the
    recurrence over every prefix would dominate a large case."""
    rng = _rng(seed, cfg, STREAM_PREFIX, layer, 1 << 22)
    return (rng.standard_normal((n_slots, cfg.H, cfg.d_v, cfg.d_k), dtype=np.float32)
            * np.float32(std))


def chain_forest(B: int, T: int) -> Forest:
    """B chains of T nodes each (node i's parent is i-1)."""
    one = np.arange(-1, T - 1, dtype=np.int32)
    off = np.arange(0, (B + 1) * T, T, dtype=np.int32)
    return Forest(parent=np.tile(one, B), tree_off=off,
                  accept=np.full(B, T - 1, dtype=np.int32))


def forest_from_trees(trees: List[np.ndarray], accept: Optional[List[int]] = None) -> Forest:
    off = np.zeros(len(trees) + 1, dtype=np.int32)
    off[1:] = np.cumsum([len(t) for t in trees])
    acc = np.array(accept if accept is not None else [len(t) - 1 for t in trees], dtype=np.int32)
    return Forest(parent=np.concatenate(trees).astype(np.int32), tree_off=off, accept=acc)


@dataclass
class PrefixBulk:
    """Committed-prefix tokens of all B x H state heads of one layer, [P, B, H, d]
    (storage arrays as for LayerInputs).  Drawn from one stream per layer; the
    per-head generator ``make_prefix`` serves the oracle-checked tests."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray       # [P, B, H] float32
    beta: np.ndarray    # [P, B, H] float32


def make_prefix_bulk(cfg: Config, B: int, layer: int = 0, seed: int = 0) -> PrefixBulk:
    rng = _rng(seed, cfg, STREAM_PREFIX, layer, 1 << 20)
    P, H = cfg.prefix, cfg.H
    q = _unit_rows(rng, P * B * H, cfg.d_k).reshape(P, B, H, cfg.d_k)
    k = _unit_rows(rng, P * B * H, cfg.d_k).reshape(P, B, H, cfg.d_k)
    v = rng.standard_normal((P, B, H, cfg.d_v), dtype=np.float32)
    g, beta = _gates(rng, (P, B, H), cfg.gate_mu)
    return PrefixBulk(q=to_storage(q, cfg.dtype), k=to_storage(k, cfg.dtype),
                      v=to_storage(v, cfg.dtype), g=g.astype(np.float32),
                      beta=beta.astype(np.float32))


# ----------------------------------------------------------------------------
# device-side generation for large timing runs
#
# The multi-layer round moves gigabytes of token operands and states; drawing
# them with numpy would dominate the run.  These draw the same distributions
# (the recipe in the module docstring) with a seeded torch generator on the
# device.  They serve timing only: the oracle-checked tests use the numpy
# streams above.

@dataclass
class DeviceLayer:
    q: "object"      # [N, H, d_k] token dtype
    k: "object"
    v: "object"      # [N, H, d_v]
    g: "object"      # [N, H] float32
    beta: "object"   # [N, H] float32


def _device_gen(torch, dev, cfg: Config, stream: int, *parts: int):
    seq = np.random.SeedSequence([cfg.cid, stream, *parts])
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seq.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
    return gen


def device_layer(cfg: Config, N: int, layer: int, seed: int, torch, dev, lead=()) -> DeviceLayer:
    """One layer's token operands (or a [*lead, N, H, ...] batch of them)."""
    gen = _device_gen(torch, dev, cfg, STREAM_TOKENS, seed, layer, 1 << 21)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    H = cfg.H

    def unit(d):
        x = torch.randn(*lead, N, H, d, generator=gen, device=dev, dtype=torch.float32)
        return (x / x.norm(dim=-1, keepdim=True)).to(tdt)

    q, k = unit(cfg.d_k), unit(cfg.d_k)
    v = torch.randn(*lead, N, H, cfg.d_v, generator=gen, device=dev, dtype=torch.float32).to(tdt)
    x = torch.randn(*lead, N, H, generator=gen, device=dev, dtype=torch.float64) + cfg.gate_mu
    g = (-torch.nn.functional.softplus(x)).to(torch.float32)
    beta = torch.sigmoid(torch.randn(*lead, N, H, generator=gen, device=dev,
                                      dtype=torch.float64)).to(torch.float32)
    return DeviceLayer(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), g=g.contiguous(),
                       beta=beta.contiguous())


def device_states(cfg: Config, n_slots: int, seed: int, torch, dev, lead=()):
    """Committed states drawn directly on the device, [*lead, n_slots, H, d_v,
    d_k] float32 with N(0, STATE_STD^2) entries (the spread of prefix-built
    states; see make_states)."""
    gen = _device_gen(torch, dev, cfg, STREAM_PREFIX, seed, 1 << 22)
    return torch.randn(*lead, n_slots, cfg.H, cfg.d_v, cfg.d_k, generator=gen, device=dev,
                       dtype=torch.float32) * STATE_STD


def device_prefix(cfg: Config, B: int, layer: int, seed: int, torch, dev) -> DeviceLayer:
    """The committed-prefix tokens of all B x H state heads of one layer,
    [P, B, H, ...] (P = cfg.prefix)."""
    return device_layer(cfg, B, layer, seed + (1 << 20), torch, dev, lead=(cfg.prefix,))


# ----------------------------------------------------------------------------
# short causal convolution inputs

STREAM_CONV = 4
CONV_WIDTH = 4  # GDN's usual kernel width; the pages do not fix one


@dataclass
class ConvInputs:
    """Inputs of the tree convolution for one layer: x [N, C] and the committed
    conv states [n_slots, W-1, C] (storage arrays, as for LayerInputs), float32
    weights [C, W] and bias [C]."""
    x: np.ndarray
    weight: np.ndarray
    bias: np.ndarray
    state: np.ndarray
    dtype: str

    @property
    def x64(self):
        return widen(self.x, self.dtype)

    @property
    def state64(self):
        return widen(self.state, self.dtype)


def conv_channels(cfg: Config) -> int:
    """The mixed q, k, v projection a GDN layer convolves: 2 H d_k + H d_v."""
    return cfg.H * (2 * cfg.d_k + cfg.d_v)


def make_conv(cfg: Config, N: int, n_slots: int, C: Optional[int] = None, W: int = CONV_WIDTH,
              layer: int = 0, seed: int = 0) -> ConvInputs:
    """x, states ~ N(0, 1); weight ~ N(0, 1/W); bias ~ N(0, 0.01)."""
    rng = _rng(seed, cfg, STREAM_CONV, layer, W)
    C = conv_channels(cfg) if C is None else C
    x = rng.standard_normal((N, C), dtype=np.float32)
    st = rng.standard_normal((n_slots, W - 1, C), dtype=np.float32)
    w = (rng.standard_normal((C, W)) / np.sqrt(W)).astype(np.float32)
    b = (0.1 * rng.standard_normal(C)).astype(np.float32)
    return ConvInputs(x=to_storage(x, cfg.dtype), weight=w, bias=b,
                      state=to_storage(st, cfg.dtype), dtype=cfg.dtype)


# ----------------------------------------------------------------------------
# drafted candidate trees for budget selection

STREAM_DRAFT = 5
DRAFT_DEPTH = 8   # the pages' maximum draft depth
DRAFT_TOPK = 4    # and their top-k


@dataclass
class Candidates:
    """Drafted candidate trees of B requests, packed CSR-style: cand_parent
    [M_total] (local parent, -1 for the root), p_draft [M_total] float32 (the
    drafter's conditional probability of each candidate given its parent; 1 for
    the root, the token the request already holds), cand_off [B+1]."""
    cand_parent: np.ndarray
    p_draft: np.ndarray
    cand_off: np.ndarray

    @property
    def B(self) -> int:
        return len(self.cand_off) - 1


def draft_tree(rng: np.random.Generator, depth: int = DRAFT_DEPTH, topk: int = DRAFT_TOPK,
               vocab: int = 32, sigma: float = 2.0):
    """One drafted candidate tree: the root gets topk children; at every further
    level the first topk nodes of the level before (earlier parents first,
    siblings in descending p) get topk children each.  A node's children carry
    the topk largest probabilities of a softmax over vocab N(0, sigma^2) logits,
    in descending order.  Nodes are numbered level by level."""
    parent, p = [-1], [1.0]
    level = [0]
    for _ in range(depth):
        nxt = []
        for u in level[:topk]:
            z = rng.standard_normal(vocab) * sigma
            e = np.exp(z - z.max())
            probs = np.sort(e / e.sum())[::-1][:topk]
            for q in probs:
                parent.append(u)
                p.append(float(q))
                nxt.append(len(parent) - 1)
        level = nxt
    return np.array(parent, np.int32), np.array(p, np.float32)


def make_candidates(B: int, seed: int = 0, depth: int = DRAFT_DEPTH,
                    topk: int = DRAFT_TOPK) -> Candidates:
    rng = np.random.default_rng(np.random.SeedSequence([seed, B, STREAM_DRAFT, depth, topk]))
    trees = [draft_tree(rng, depth, topk) for _ in range(B)]
    off = np.zeros(B + 1, np.int32)
    off[1:] = np.cumsum([len(t[0]) for t in trees])
    return Candidates(cand_parent=np.concatenate([t[0] for t in trees]),
                      p_draft=np.concatenate([t[1] for t in trees]), cand_off=off)
