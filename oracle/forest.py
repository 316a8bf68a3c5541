"""Budget selection and the packed-forest builder: the oracle.

TEST INFRASTRUCTURE ONLY (the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the product library never does).  Plain Python
and numpy, one candidate at a time.

What the pages fix (review page, section 三, the hardware-aware budget and the
SGLang integration paragraphs): each drafted node is scored with its path's
cumulative draft probability, rho(v) = the product of p_draft(u | parent(u))
over the nodes u on v's root-to-node path; the highest-scoring nodes across
all requests fill the calibrated capacity; since a child's cumulative
probability never exceeds its parent's, every request's selection is
prefix-connected; the device packs the selection into one flat ragged forest.

Readings (the pages leave these open):
  * rho is a float32 running product taken root first, rho(root) = p(root),
    rho(v) = fl32(rho(parent(v)) * p(v)).  With 0 <= p <= 1 each factor can
    only lower it, in float32 too.  The root of a candidate tree is the token
    the request already holds; its p is normally 1.
  * Candidates are ranked by the key (rho descending, depth ascending, request
    ascending, candidate index ascending).  The key is a total order in which a
    parent always precedes its children (equal rho falls to depth).
  * Besides the global capacity, each request takes at most max_tree nodes (the
    verify kernels' tree limit).  Selection is greedy in key order: a candidate
    is taken while its request holds fewer than max_tree and the forest fewer
    than capacity nodes.
  * A request's selected nodes are numbered 0, 1, ... in key order, so the root
    is node 0 and parents precede children; parent[] holds local numbers.
    Requests are packed in order; capacity slots past the last node hold -1.
  * A candidate tree with a bad parent link, a cycle, or a probability outside
    [0, 1] (NaN included) is reported and contributes no node.
"""

from __future__ import annotations

import numpy as np

ERR_BAD_PARENT = 1
ERR_CYCLE = 2
ERR_BAD_PROB = 32


def score_tree(parent, p):
    """(rho float32 [M], depth int [M], err) for one candidate tree.  Parents are
    followed up to the root; rho multiplies along the path root first."""
    parent = np.asarray(parent)
    p = np.asarray(p, dtype=np.float32)
    M = len(parent)
    rho = np.zeros(M, dtype=np.float32)
    depth = np.zeros(M, dtype=np.int64)
    for i in range(M):
        if not (-1 <= parent[i] < M) or parent[i] == i:
            return rho, depth, ERR_BAD_PARENT
    for i in range(M):
        if not (0.0 <= p[i] <= 1.0):  # False for NaN as well
            return rho, depth, ERR_BAD_PROB
    for i in range(M):
        path, j = [i], i
        while parent[j] >= 0:
            j = int(parent[j])
            path.append(j)
            if len(path) > M:
                return rho, depth, ERR_CYCLE
        x = p[path[-1]]                   # the root's own factor
        for u in reversed(path[:-1]):     # then down the path, root first
            x = np.float32(x * p[u])
        rho[i] = x
        depth[i] = len(path) - 1
    return rho, depth, 0


def build_forest(cand_parent, p_draft, cand_off, capacity, max_tree):
    """Select and pack.  cand_parent [M_total] (local parent within its request's
    candidate tree, -1 for the root), p_draft [M_total], cand_off [B+1].

    Returns dict: rho [M_total] float32, parent [capacity] int32 (local parent of
    each packed node, -1 for a root or an unused slot), cand_of [capacity] int32
    (global candidate index of each packed node, -1 for an unused slot),
    tree_off [B+1] int32, n_nodes, err (OR of the error bits)."""
    cand_off = np.asarray(cand_off)
    B = len(cand_off) - 1
    M_total = int(cand_off[-1])
    rho = np.zeros(M_total, dtype=np.float32)
    entries = []                      # (key tuple, request, local index)
    err = 0
    for b in range(B):
        o, e = int(cand_off[b]), int(cand_off[b + 1])
        r, d, eb = score_tree(np.asarray(cand_parent)[o:e], np.asarray(p_draft)[o:e])
        err |= eb
        if eb:
            continue
        rho[o:e] = r
        for i in range(e - o):
            entries.append(((-float(r[i]), int(d[i]), b, i), b, i))
    entries.sort(key=lambda t: t[0])
    taken = [[] for _ in range(B)]    # local candidate indices, in key order
    total = 0
    for _, b, i in entries:
        if total < capacity and len(taken[b]) < max_tree:
            taken[b].append(i)
            total += 1
    tree_off = np.zeros(B + 1, dtype=np.int32)
    parent = np.full(capacity, -1, dtype=np.int32)
    cand_of = np.full(capacity, -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        o = int(cand_off[b])
        local = {i: n for n, i in enumerate(taken[b])}
        for n, i in enumerate(taken[b]):
            pi = int(cand_parent[o + i])
            parent[pos + n] = -1 if pi < 0 else local[pi]   # KeyError: not prefix-closed
            cand_of[pos + n] = o + i
        pos += len(taken[b])
        tree_off[b + 1] = pos
    return dict(rho=rho, parent=parent, cand_of=cand_of, tree_off=tree_off, n_nodes=pos,
                err=err)
