"""Theorem 1 of Bole (arXiv 2608.01651) written out in numpy, float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Notation follows the pages (arXiv page, section IV-A; the xllm-io review,
section 三, Eqs. 2, 4, 5, 6, 10), for one tree and one head:

  A(i)      strict proposal ancestors of node i,
  P_i       = prod over r in A(i) and i itself of gamma_r            (Lemma 1 / Eq. 4)
  C_ij      = (P_i / P_j) q_i . k_j   for j in A(i) or j = i, else 0  (Eq. 4)
  G_ij      = beta_i (P_i / P_j) k_i . k_j  for j in A(i), else 0    (Lemma 2 / Eq. 5)
  R         = D_beta (V - D_P K S_pre)                               (Eq. 2)
  B0        = D_P Q S_pre                                            (Eq. 2 / Eq. 7)
  U         = (I + G)^{-1} R = sum_{m=0}^{d} (-G)^m R                (Eq. 5, Eq. 6)
  O         = B0 + C U                                               (Eq. 2)
  W         = (I + G)^{-1} = sum_{m=0}^{d} (-G)^m, M = C W            (Lemma 3; an explicit
                                                                      inverse, one exact solve)
  S_new     = P_a S_pre + (D_a K_a)^T U_a  for the path a            (Eq. 10)

Here S_pre is the paper's d_k x d_v state.  The serving slot stores its
transpose ([d_v, d_k]); the functions below take and return slot layout and
transpose internally.  gamma = exp(g) with g the log-gate input; P is the plain
float64 product of the path's gammas (not the library's float32 log sums).
"""

from __future__ import annotations

import numpy as np


def _paths(parent):
    """Root-to-node path of every local node (parent < 0 marks a root)."""
    T = len(parent)
    paths = []
    for i in range(T):
        p, x = [i], i
        while parent[x] >= 0:
            x = int(parent[x])
            p.append(x)
            if len(p) > T:
                raise ValueError("cycle in parent array")
        paths.append(p[::-1])
    return paths


def tree_factors(parent, q, k, g, beta):
    """P, G, C and d for one tree/head.  q, k: [T, dk]; g, beta: [T]."""
    parent = np.asarray(parent)
    T = len(parent)
    paths = _paths(parent)
    gamma = np.exp(np.asarray(g, dtype=np.float64))
    P = np.array([np.prod(gamma[p]) for p in paths])
    G = np.zeros((T, T))
    C = np.zeros((T, T))
    for i, p in enumerate(paths):
        for j in p:               # ancestors-or-self of i
            ratio = P[i] / P[j]
            C[i, j] = ratio * float(q[i] @ k[j])
            if j != i:
                G[i, j] = beta[i] * ratio * float(k[i] @ k[j])
    d = max(len(p) - 1 for p in paths)
    return P, G, C, d


def closed_form_tree(parent, q, k, v, g, beta, S_slot):
    """Theorem 1 for one tree/head.  q, k [T, dk]; v [T, dv]; g, beta [T];
    S_slot [dv, dk] (slot layout).  Returns dict with O, U, G, C, R, B0, P, d."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    beta = np.asarray(beta, dtype=np.float64)
    S = np.asarray(S_slot, dtype=np.float64).T          # paper's S_pre: [dk, dv]
    P, G, C, d = tree_factors(parent, q, k, g, beta)
    B0 = P[:, None] * (q @ S)
    R = beta[:, None] * (v - P[:, None] * (k @ S))
    U = R.copy()
    Z = R.copy()
    for _ in range(d):            # finite Neumann series, Lemma 3
        Z = -G @ Z
        U = U + Z
    O = B0 + C @ U
    return dict(O=O, U=U, G=G, C=C, R=R, B0=B0, P=P, d=d)


def inverse_factors(G, C, d):
    """W = (I + G)^{-1} as the finite Neumann polynomial sum_{m=0}^{d} (-G)^m
    (Lemma 3: G^{d+1} = 0), and M = C W, so that U = W R and O = B0 + M R."""
    G = np.asarray(G, dtype=np.float64)
    T = G.shape[0]
    W = np.eye(T)
    term = np.eye(T)
    for _ in range(d):
        term = -G @ term
        W = W + term
    return W, np.asarray(C, dtype=np.float64) @ W


def commit_closed_form(parent, a, k, U, P, S_slot):
    """Eq. 10 for one tree/head: state after accepted node a, slot layout."""
    path = _paths(np.asarray(parent))[a]
    Ka = np.asarray(k, dtype=np.float64)[path]                  # [La, dk]
    Ua = np.asarray(U, dtype=np.float64)[path]                  # [La, dv]
    Da = P[a] / np.asarray(P)[path]                             # diag of D_a
    S = np.asarray(S_slot, dtype=np.float64).T
    S_new = P[a] * S + (Da[:, None] * Ka).T @ Ua                # [dk, dv]
    return S_new.T
