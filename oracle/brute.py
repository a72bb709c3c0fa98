"""Brute-force transfer products in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

Each step of the gated delta rule is an affine map of the state,
    S_t = S_{t-1} M_t + beta_t v_t k_t^T,     M_t = Diag(a_t) (I - beta_t k_t k_t^T),
with a_t = exp(g_t) (SFDA summary, "Kernarchitektur", transposed, zero phase:
decay first, then the rank-one erase).  Here every M_t is built as an explicit
d_k x d_k matrix and the state is assembled from products of them:
    S_t = h0 M_1 ... M_t + sum_{j<=t} beta_j v_j k_j^T M_{j+1} ... M_t,   o_t = S_t q_t.
This is the brute-force ground truth the SFDA summary ("Ergebnisse") checks its
chunk recursion and affine transfer against.  O(T^2 d_k^3): tiny inputs only.
"""
from __future__ import annotations

import numpy as np


def transition(k_t, beta_t, a_t):
    """M_t = Diag(a_t) (I - beta_t k_t k_t^T) as an explicit matrix."""
    dk = k_t.shape[0]
    return np.diag(a_t) @ (np.eye(dk) - beta_t * np.outer(k_t, k_t))


def _decays(g, T, dk):
    if g is None:
        return np.ones((T, dk))
    g = np.asarray(g, np.float64)
    if g.ndim == 1:
        return np.repeat(np.exp(g)[:, None], dk, axis=1)
    return np.exp(g)


def product(Ms):
    """Left-to-right product M_1 M_2 ... M_n (identity when empty)."""
    out = None
    for M in Ms:
        out = M.copy() if out is None else out @ M
    return out


def forward(q, k, v, beta, g=None, h0=None):
    """One head.  Returns (o [T, dv], hT [dv, dk])."""
    q, k, v, beta = (np.asarray(a, np.float64) for a in (q, k, v, beta))
    T, dk = q.shape
    dv = v.shape[1]
    a = _decays(g, T, dk)
    Ms = [transition(k[t], beta[t], a[t]) for t in range(T)]
    S0 = np.zeros((dv, dk)) if h0 is None else np.asarray(h0, np.float64)
    o = np.zeros((T, dv))
    S = S0
    for t in range(T):
        P = product(Ms[: t + 1])
        S = S0 @ P
        for j in range(t + 1):
            W = np.outer(beta[j] * v[j], k[j])
            tail = product(Ms[j + 1: t + 1])
            S = S + (W if tail is None else W @ tail)
        o[t] = S @ q[t]
    if T == 0:
        S = S0.copy()
    return o, S


def chunk_product(k, beta, g=None):
    """Transition product M_1 ... M_L of one chunk, explicitly."""
    k, beta = np.asarray(k, np.float64), np.asarray(beta, np.float64)
    L, dk = k.shape
    a = _decays(g, L, dk)
    P = product([transition(k[t], beta[t], a[t]) for t in range(L)])
    return np.eye(dk) if P is None else P
