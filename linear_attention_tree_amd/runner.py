"""Device-buffer plumbing around the calls of libbole.

``TreeRound`` owns the per-round topology buffers of one packed forest and the
per-layer G/C workspace, allocates outputs with PyTorch and issues the calls in
stream order.  It performs no arithmetic of its own.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import bole


@dataclass
class Topology:
    parent: torch.Tensor      # [N] int32
    tree_off: torch.Tensor    # [B+1] int32
    depth: torch.Tensor       # [N] int32
    anc: torch.Tensor         # [N] int64 (uint64 bits)
    order: torch.Tensor       # [N] int32
    tree_depth: torch.Tensor  # [B] int32

    @property
    def B(self) -> int:
        return self.tree_off.shape[0] - 1

    @property
    def N(self) -> int:
        return self.parent.shape[0]


class TreeRound:
    """One verification round over a packed forest on one device."""

    def __init__(self, parent, tree_off, H: int, device="cuda", err: Optional[torch.Tensor] = None):
        dev = torch.device(device)
        parent = torch.as_tensor(parent, dtype=torch.int32).to(dev)
        tree_off = torch.as_tensor(tree_off, dtype=torch.int32).to(dev)
        N, B = parent.shape[0], tree_off.shape[0] - 1
        self.H = H
        self.device = dev
        self.topo = Topology(parent=parent, tree_off=tree_off,
                             depth=torch.empty(N, dtype=torch.int32, device=dev),
                             anc=torch.empty(N, dtype=torch.int64, device=dev),
                             order=torch.empty(N, dtype=torch.int32, device=dev),
                             tree_depth=torch.empty(B, dtype=torch.int32, device=dev))
        self.err = err if err is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        self.G = torch.empty(B, H, bole.MAX_TREE, bole.MAX_TREE, dtype=torch.float32, device=dev)
        self.C = torch.empty_like(self.G)

    def prep(self, log_gamma: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
        """Topology plus logP for all layers of log_gamma [L, N, H]; returns logP."""
        t = self.topo
        logP = None if log_gamma is None else torch.empty_like(log_gamma)
        bole.bole_tree_prep(t.parent, t.tree_off, log_gamma, t.depth, t.anc, t.order,
                            t.tree_depth, logP, self.err, stream)
        return logP

    # the two-call path's exact solves: (producer, verify) of each
    SOLVES = {"blocked": ("bole_factor_gc", "bole_verify"),
              "neumann": ("bole_factor_gc", "bole_verify_neumann"),
              "inverse": ("bole_factor_inverse", "bole_verify_inverse")}

    def factor(self, q, k, logP, beta, stream=None, solve="blocked"):
        """G and C into the workspace (W and M for solve="inverse")."""
        t = self.topo
        getattr(bole, self.SOLVES[solve][0])(q, k, logP, beta, t.anc, t.order, t.tree_off, self.G,
                                             self.C, self.err, stream)

    def verify(self, q, k, v, logP, beta, state_pool, slot, O=None, U=None, stream=None,
               solve="blocked"):
        t = self.topo
        N, H, _ = q.shape
        d_v = v.shape[2]
        if O is None:
            O = torch.empty(N, H, d_v, dtype=v.dtype, device=v.device)
        if U is None:
            U = torch.empty(N, H, d_v, dtype=torch.float32, device=v.device)
        getattr(bole, self.SOLVES[solve][1])(q, k, v, logP, beta, state_pool, slot, self.G,
                                             self.C, t.order, t.depth, t.tree_off, t.tree_depth,
                                             O, U, self.err, stream)
        return O, U

    def layer(self, q, k, v, logP, beta, state_pool, slot, O=None, U=None, stream=None,
              fused=False, solve="blocked"):
        """Factor producer then value-tiled verify for one layer (or both in one
        launch with fused=True).  solve picks the two-call path's solve of
        (I+G) U = R: "blocked" substitution, the d-step "neumann" propagation,
        or the explicit "inverse"."""
        if not fused:
            self.factor(q, k, logP, beta, stream, solve)
            return self.verify(q, k, v, logP, beta, state_pool, slot, O, U, stream, solve)
        if solve != "blocked":
            raise ValueError("the fused verify solves by blocked substitution only")
        t = self.topo
        N, H, _ = q.shape
        d_v = v.shape[2]
        if O is None:
            O = torch.empty(N, H, d_v, dtype=v.dtype, device=v.device)
        if U is None:
            U = torch.empty(N, H, d_v, dtype=torch.float32, device=v.device)
        bole.bole_factor_verify(q, k, v, logP, beta, state_pool, slot, t.anc, t.order, t.depth,
                                t.tree_off, t.tree_depth, O, U, self.err, stream)
        return O, U

    def tree_layer(self, q, k, v, log_gamma, beta, state_pool, slot, O=None, U=None,
                   logP=None, stream=None):
        """Tree preparation for this layer and the fused verify in one launch
        (bole_tree_verify).  Fills the topology buffers; returns O, U and the
        layer's logP [N, H]."""
        t = self.topo
        N, H, _ = q.shape
        d_v = v.shape[2]
        if O is None:
            O = torch.empty(N, H, d_v, dtype=v.dtype, device=v.device)
        if U is None:
            U = torch.empty(N, H, d_v, dtype=torch.float32, device=v.device)
        if logP is None:
            logP = torch.empty(N, H, dtype=torch.float32, device=v.device)
        bole.bole_tree_verify(q, k, v, t.parent, log_gamma, beta, state_pool, slot, t.tree_off, O,
                              U, t.depth, t.anc, t.order, t.tree_depth, logP, self.err, stream)
        return O, U, logP

    def commit_tree_layer(self, prev, prev_k, prev_U, prev_logP, prev_accept, q, k, v, log_gamma,
                          beta, state_pool, slot, O=None, U=None, logP=None, stream=None):
        """The previous round's commit of this layer, then this round's
        tree_layer, in one launch (bole_commit_tree_verify).  prev is the
        previous round's TreeRound (its topology), prev_k / prev_U / prev_logP
        that round's keys, U and logP of this layer, prev_accept its accepted
        nodes (-1: nothing to commit).  Request b must keep its slot between
        the rounds.  Returns O, U and the layer's logP [N, H]."""
        t, pt = self.topo, prev.topo
        N, H, _ = q.shape
        d_v = v.shape[2]
        if O is None:
            O = torch.empty(N, H, d_v, dtype=v.dtype, device=v.device)
        if U is None:
            U = torch.empty(N, H, d_v, dtype=torch.float32, device=v.device)
        if logP is None:
            logP = torch.empty(N, H, dtype=torch.float32, device=v.device)
        prev_accept = torch.as_tensor(prev_accept, dtype=torch.int32).to(self.device)
        bole.bole_commit_tree_verify(q, k, v, t.parent, log_gamma, beta, state_pool, slot,
                                     t.tree_off, O, U, t.depth, t.anc, t.order, t.tree_depth, logP,
                                     prev_k, prev_U, prev_logP, pt.anc, pt.tree_off, prev_accept,
                                     self.err, stream)
        return O, U, logP

    def commit(self, state_pool, slot, k, U, logP, accept, stream=None):
        t = self.topo
        accept = torch.as_tensor(accept, dtype=torch.int32).to(self.device)
        bole.bole_commit_path(state_pool, slot, k, U, logP, t.anc, t.tree_off, accept,
                              self.err, stream)

    def error_bits(self) -> int:
        return int(self.err.item()) & 0xFFFFFFFF


class ForestBuilder:
    """Budget selection and forest packing into fixed-capacity buffers (their
    addresses do not change from round to round, so a captured graph can reuse
    them)."""

    def __init__(self, B: int, M_total: int, capacity: int, max_tree: int = bole.MAX_TREE,
                 device="cuda", err: Optional[torch.Tensor] = None):
        dev = torch.device(device)
        self.capacity, self.max_tree = capacity, max_tree
        self.rho = torch.empty(M_total, dtype=torch.float32, device=dev)
        self.parent = torch.empty(capacity, dtype=torch.int32, device=dev)
        self.cand_of = torch.empty(capacity, dtype=torch.int32, device=dev)
        self.tree_off = torch.empty(B + 1, dtype=torch.int32, device=dev)
        nbytes = bole.bole_forest_workspace_bytes(B, max_tree)
        if nbytes == 0:
            raise ValueError("forest shape out of range")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.err = err if err is not None else torch.zeros(1, dtype=torch.int32, device=dev)

    def build(self, cand_parent, p_draft, cand_off, stream=None):
        bole.bole_forest_build(cand_parent, p_draft, cand_off, self.capacity, self.max_tree,
                               self.rho, self.parent, self.cand_of, self.tree_off,
                               self.workspace, self.err, stream)
        return self.parent, self.tree_off, self.cand_of


def capture_graph(fn):
    """A HIP graph of the launches fn() makes on the current stream (one
    uncaptured pass first, on the side stream torch captures on)."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


class BucketedRound:
    """A whole verification round as one captured HIP graph per capacity
    bucket: budget selection and forest packing (bole_forest_build), each
    layer's bole_tree_verify, then one bole_commit_path over all layers.

    Every buffer the graphs touch keeps its address: a round copies its
    drafted candidates, its token operands (packed-forest order, the first
    `capacity` rows of each layer) and its accepted nodes into the input
    buffers and replays the graph of the smallest bucket whose capacity holds
    its budget.  The verify grid does not depend on the node count, so one
    bucket's graph serves every forest up to its capacity.

    deferred=True: each layer's launch carries that layer's commit of the
    previous round (bole_commit_tree_verify) and there is no commit launch.
    Rounds alternate between two sets of token, U and logP buffers (`parity`,
    flipped by every replay; the caller fills the token buffers of the parity
    about to run, `tokens()`), and each round keeps its forest offsets and
    ancestor sets for the next.  `accept` holds the previous round's accepted
    nodes when a round runs (-1 for nothing to commit: set it so before the
    first round and before capture)."""

    def __init__(self, B: int, L: int, H: int, d_k: int, d_v: int, dtype: torch.dtype,
                 M_total: int, buckets, max_tree: int = bole.MAX_TREE, device="cuda",
                 deferred: bool = False):
        dev = torch.device(device)
        i32, f32 = torch.int32, torch.float32
        self.B, self.L, self.H = B, L, H
        self.deferred = deferred
        self.buckets = sorted(int(c) for c in buckets)
        cmax = self.buckets[-1]
        self.cand_parent = torch.zeros(M_total, dtype=i32, device=dev)
        self.p_draft = torch.zeros(M_total, dtype=f32, device=dev)
        self.cand_off = torch.zeros(B + 1, dtype=i32, device=dev)

        def token_set():
            return dict(q=torch.zeros(L, cmax, H, d_k, dtype=dtype, device=dev),
                        k=torch.zeros(L, cmax, H, d_k, dtype=dtype, device=dev),
                        v=torch.zeros(L, cmax, H, d_v, dtype=dtype, device=dev),
                        g=torch.zeros(L, cmax, H, dtype=f32, device=dev),
                        beta=torch.zeros(L, cmax, H, dtype=f32, device=dev),
                        U=torch.zeros(L, cmax, H, d_v, dtype=f32, device=dev),
                        logP=torch.zeros(L, cmax, H, dtype=f32, device=dev),
                        anc=torch.zeros(cmax, dtype=torch.int64, device=dev),
                        tree_off=torch.zeros(B + 1, dtype=i32, device=dev))

        self.sets = [token_set()] + ([token_set()] if deferred else [])
        self.parity = 0
        self.accept = torch.zeros(B, dtype=i32, device=dev)
        self.O = torch.zeros(L, cmax, H, d_v, dtype=dtype, device=dev)
        self.err = torch.zeros(1, dtype=i32, device=dev)
        self.forest = {c: ForestBuilder(B, M_total, c, max_tree, dev, self.err)
                       for c in self.buckets}
        self.topo = {c: Topology(parent=self.forest[c].parent, tree_off=self.forest[c].tree_off,
                                 depth=torch.zeros(c, dtype=i32, device=dev),
                                 anc=torch.zeros(c, dtype=torch.int64, device=dev),
                                 order=torch.zeros(c, dtype=i32, device=dev),
                                 tree_depth=torch.zeros(B, dtype=i32, device=dev))
                     for c in self.buckets}
        self.graphs = {}

    # the current parity's buffers (the only set without deferred)
    def tokens(self, parity: Optional[int] = None) -> dict:
        return self.sets[self.parity if parity is None else parity]

    q = property(lambda self: self.tokens()["q"])
    k = property(lambda self: self.tokens()["k"])
    v = property(lambda self: self.tokens()["v"])
    g = property(lambda self: self.tokens()["g"])
    beta = property(lambda self: self.tokens()["beta"])
    U = property(lambda self: self.tokens()["U"])
    logP = property(lambda self: self.tokens()["logP"])

    def bucket(self, budget: int) -> int:
        for c in self.buckets:
            if budget <= c:
                return c
        raise ValueError(f"budget {budget} exceeds the largest bucket {self.buckets[-1]}")

    def run_eager(self, capacity: int, state_pool, slot, commit=True, parity=None):
        """One round launched call by call (what the graph of `capacity` holds)."""
        fb, t, c = self.forest[capacity], self.topo[capacity], capacity
        par = self.parity if parity is None else parity
        cur = self.sets[par]
        fb.build(self.cand_parent, self.p_draft, self.cand_off)
        if self.deferred:
            prev = self.sets[1 - par]
            for l in range(self.L):
                bole.bole_commit_tree_verify(
                    cur["q"][l, :c], cur["k"][l, :c], cur["v"][l, :c], fb.parent,
                    cur["g"][l, :c], cur["beta"][l, :c], state_pool[l], slot, fb.tree_off,
                    self.O[l, :c], cur["U"][l, :c], t.depth, t.anc, t.order, t.tree_depth,
                    cur["logP"][l, :c], prev["k"][l], prev["U"][l], prev["logP"][l], prev["anc"],
                    prev["tree_off"], self.accept, self.err)
            # this round's forest, kept for the next round's commits
            cur["anc"][:c].copy_(t.anc)
            cur["tree_off"].copy_(fb.tree_off)
            return
        for l in range(self.L):
            bole.bole_tree_verify(cur["q"][l, :c], cur["k"][l, :c], cur["v"][l, :c], fb.parent,
                                  cur["g"][l, :c], cur["beta"][l, :c], state_pool[l], slot,
                                  fb.tree_off, self.O[l, :c], cur["U"][l, :c], t.depth, t.anc,
                                  t.order, t.tree_depth, cur["logP"][l, :c], self.err)
        if commit:
            bole.bole_commit_path(state_pool, slot, cur["k"][:, :c], cur["U"][:, :c],
                                  cur["logP"][:, :c], t.anc, fb.tree_off, self.accept, self.err)

    def capture(self, state_pool, slot, commit=True):
        """Capture every bucket's round (and with deferred, both parities)
        against these state-pool and slot buffers (they too must keep their
        addresses).  The uncaptured pass that precedes each capture runs the
        round once, commits included, on the inputs loaded now: load a valid
        round first (empty candidate sets give empty trees, which the verify
        calls report), and with deferred set `accept` to -1."""
        for c in self.buckets:
            for par in range(len(self.sets)):
                self.graphs[(c, par)] = capture_graph(
                    lambda c_=c, p_=par: self.run_eager(c_, state_pool, slot, commit, p_))

    def replay(self, budget: int) -> int:
        c = self.bucket(budget)
        self.graphs[(c, self.parity)].replay()
        if self.deferred:
            self.parity ^= 1
        return c
