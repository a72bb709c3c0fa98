"""Chunkwise (WY / affine chunk-transfer) evaluation in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

This is a second, independent evaluation of the operator that the C oracle
computes step by step.  It follows the chunkwise form the pages describe:

* ReWY abstract: the chunked evaluation turns the recurrence into dense matrix
  work per chunk; its backward treats the per-chunk correction as a single
  triangular system, solved once transposed, with no explicit inverse to
  differentiate.
* SFDA summary, "Der konstruktive Chunk-WY-Theorem": within a chunk the product
  of transitions is the decay product minus a rank <= C correction with a
  triangular core; "Zentrale Beitraege": the chunk's write summary B_chunk is the
  zero-initial-state recursion, so S_end = S_start P_chunk + B_chunk exactly.

Gates are handled in one way for all three operators: the log-decay is a
per-channel matrix G (L x d_k) per chunk -- zeros for no gate, the scalar
broadcast across channels for a scalar gate.  Pairwise decays are formed
explicitly as E[t, s, c] = exp(gamma[t, c] - gamma[s, c]) with gamma the
in-chunk cumulative sum; no centring, no factorisation -- this keeps it plainly
checkable and independent of how the GPU path factors the decays.

Per chunk, with S0 the entering state (d_v x d_k):
    A[t,s]  = beta_t sum_c K[t,c] K[s,c] E[t,s,c]   (s < t)     strictly lower
    Pm[t,s] = sum_c Q[t,c] K[s,c] E[t,s,c]          (s <= t)    lower
    R = diag(beta) (V - (K*Gam) S0^T),   (I + A) U = R
    O = (Q*Gam) S0^T + Pm U
    S1 = S0 Diag(Gam_L) + U^T (K * Gam_L / Gam)
with Gam = exp(gamma).  The reverse pass below differentiates exactly these
lines; the triangular system is differentiated as a residual: lambda solves
(I + A)^T lambda = dU and dA = -lambda U^T on the strict lower triangle.
"""
from __future__ import annotations

import numpy as np


def _as_channel_gate(g, T, dk):
    """Log-decay as [T, dk] per head: zeros (none), broadcast scalar, or vector."""
    if g is None:
        return np.zeros((T, dk))
    g = np.asarray(g, dtype=np.float64)
    if g.ndim == 1:
        return np.repeat(g[:, None], dk, axis=1)
    return g


def _chunk_forward(Q, K, V, beta, G, S0):
    L = Q.shape[0]
    gam = np.cumsum(G, axis=0)
    Gam = np.exp(gam)
    E = np.exp(gam[:, None, :] - gam[None, :, :])               # [t, s, c]
    strict = np.tril(np.ones((L, L)), -1)
    lower = np.tril(np.ones((L, L)))
    A = beta[:, None] * np.einsum("tc,sc,tsc->ts", K, K, E) * strict
    Pm = np.einsum("tc,sc,tsc->ts", Q, K, E) * lower
    X = V - (K * Gam) @ S0.T
    R = beta[:, None] * X
    U = np.linalg.solve(np.eye(L) + A, R)
    O = (Q * Gam) @ S0.T + Pm @ U
    Kd = K * np.exp(gam[-1][None, :] - gam)
    S1 = S0 * Gam[-1][None, :] + U.T @ Kd
    cache = dict(gam=gam, Gam=Gam, E=E, A=A, Pm=Pm, X=X, U=U, Kd=Kd, strict=strict, lower=lower)
    return O, S1, cache


def _chunk_backward(Q, K, V, beta, G, S0, dO, dS1, c):
    gam, Gam, E, A, Pm, X, U, Kd = (c[n] for n in ("gam", "Gam", "E", "A", "Pm", "X", "U", "Kd"))
    L = Q.shape[0]
    # O = (Q*Gam) S0^T + Pm U ;  S1 = S0 Diag(Gam_L) + U^T Kd
    dU = Pm.T @ dO + Kd @ dS1.T
    dPm = (dO @ U.T) * c["lower"]
    dQG = dO @ S0
    dKd = U @ dS1
    dS0 = dS1 * Gam[-1][None, :] + dO.T @ (Q * Gam)
    # (I + A) U = R: one transposed triangular solve
    lam = np.linalg.solve((np.eye(L) + A).T, dU)
    dA = -(lam @ U.T) * c["strict"]
    # R = diag(beta) X,  X = V - (K*Gam) S0^T
    dbeta = np.sum(lam * X, axis=1)
    dX = beta[:, None] * lam
    dV = dX.copy()
    dKG = -dX @ S0
    dS0 -= dX.T @ (K * Gam)
    dQ = dQG * Gam
    dK = dKG * Gam + dKd * np.exp(gam[-1][None, :] - gam)
    dgam = dQG * Q * Gam + dKG * K * Gam - dKd * Kd
    dgam[-1] += np.sum(dKd * Kd, axis=0) + np.sum(S0 * dS1, axis=0) * Gam[-1]
    # A[t,s] = beta_t sum_c K[t,c] K[s,c] E[t,s,c]
    WA = (beta[:, None] * dA)[:, :, None] * K[:, None, :] * K[None, :, :] * E
    dK += np.einsum("ts,sc,tsc->tc", beta[:, None] * dA, K, E)
    dK += np.einsum("ts,tc,tsc->sc", beta[:, None] * dA, K, E)
    dbeta += np.einsum("ts,tc,sc,tsc->t", dA, K, K, E)
    dgam += WA.sum(axis=1) - WA.sum(axis=0)
    # Pm[t,s] = sum_c Q[t,c] K[s,c] E[t,s,c]
    WP = dPm[:, :, None] * Q[:, None, :] * K[None, :, :] * E
    dQ += np.einsum("ts,sc,tsc->tc", dPm, K, E)
    dK += np.einsum("ts,tc,tsc->sc", dPm, Q, E)
    dgam += WP.sum(axis=1) - WP.sum(axis=0)
    # gamma = cumsum(G): dG is the reverse cumulative sum of dgam
    dG = np.cumsum(dgam[::-1], axis=0)[::-1]
    return dQ, dK, dV, dbeta, dG, dS0, lam


def _split(T, C):
    return [(t0, min(t0 + C, T)) for t0 in range(0, T, C)]


def forward(q, k, v, beta, g=None, h0=None, C=16, trace=None):
    """Chunked forward of one head or of [B,H,...] batches.  Returns (o, hT, states)
    where states[n] is the state entering chunk n.  For one head, ``trace`` (a
    list) receives per chunk a dict with gam, T = (I + A)^{-1}, Pm and U."""
    q = np.asarray(q, np.float64)
    if q.ndim == 4:
        B, H = q.shape[:2]
        outs = [forward(q[b, h], k[b, h], v[b, h], beta[b, h],
                        None if g is None else g[b, h], None if h0 is None else h0[b, h], C, trace)
                for b in range(B) for h in range(H)]
        o = np.stack([x[0] for x in outs]).reshape(B, H, *outs[0][0].shape)
        hT = np.stack([x[1] for x in outs]).reshape(B, H, *outs[0][1].shape)
        st = np.stack([x[2] for x in outs]).reshape(B, H, *outs[0][2].shape)
        return o, hT, st
    k, v, beta = (np.asarray(a, np.float64) for a in (k, v, beta))
    T, dk = q.shape
    dv = v.shape[1]
    G = _as_channel_gate(g, T, dk)
    S = np.zeros((dv, dk)) if h0 is None else np.array(h0, np.float64)
    o = np.zeros((T, dv))
    states = []
    for t0, t1 in _split(T, C):
        states.append(S.copy())
        O, S, cache = _chunk_forward(q[t0:t1], k[t0:t1], v[t0:t1], beta[t0:t1], G[t0:t1], S)
        o[t0:t1] = O
        if trace is not None:
            L = t1 - t0
            trace.append(dict(gam=cache["gam"], T=np.linalg.inv(np.eye(L) + cache["A"]),
                              Pm=cache["Pm"], U=cache["U"]))
    return o, S, np.array(states).reshape(len(states), dv, dk)


def backward(q, k, v, beta, g, h0, do, dhT=None, C=16, trace=None):
    """Chunked reverse mode (ReWY form) of one head or of [B,H,...] batches.
    Returns dict dq, dk, dv, dbeta, dg (None without a gate, [T] for a scalar
    gate, [T, dk] for a vector gate), dh0.  For one head, ``trace`` (a dict)
    receives per chunk, in chunk order, "dS1" (the state cotangent leaving the
    chunk) and "lam" (the solution of (I + A)^T lam = dU)."""
    q = np.asarray(q, np.float64)
    if q.ndim == 4:
        B, H = q.shape[:2]
        res = [backward(q[b, h], k[b, h], v[b, h], beta[b, h], None if g is None else g[b, h],
                        None if h0 is None else h0[b, h], do[b, h],
                        None if dhT is None else dhT[b, h], C, trace)
               for b in range(B) for h in range(H)]
        out = {}
        for name in res[0]:
            if res[0][name] is None:
                out[name] = None
            else:
                out[name] = np.stack([r[name] for r in res]).reshape(B, H, *res[0][name].shape)
        return out
    k, v, beta, do = (np.asarray(a, np.float64) for a in (k, v, beta, do))
    T, dk = q.shape
    dv = v.shape[1]
    G = _as_channel_gate(g, T, dk)
    S = np.zeros((dv, dk)) if h0 is None else np.array(h0, np.float64)
    spans = _split(T, C)
    saved = []
    for t0, t1 in spans:
        S0 = S
        _, S, cache = _chunk_forward(q[t0:t1], k[t0:t1], v[t0:t1], beta[t0:t1], G[t0:t1], S0)
        saved.append((S0, cache))
    dS = np.zeros((dv, dk)) if dhT is None else np.array(dhT, np.float64)
    dq = np.zeros_like(q)
    dkk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    db = np.zeros_like(beta)
    dG = np.zeros((T, dk))
    dS1s, lams = [], []
    for (t0, t1), (S0, cache) in reversed(list(zip(spans, saved))):
        dS1s.append(dS)
        r = _chunk_backward(q[t0:t1], k[t0:t1], v[t0:t1], beta[t0:t1], G[t0:t1], S0,
                            do[t0:t1], dS, cache)
        dq[t0:t1], dkk[t0:t1], dvv[t0:t1], db[t0:t1], dG[t0:t1], dS = r[:6]
        lams.append(r[6])
    if trace is not None:
        trace["dS1"] = dS1s[::-1]
        trace["lam"] = lams[::-1]
    if g is None:
        dg = None
    elif np.asarray(g).ndim == 1:
        dg = dG.sum(axis=1)
    else:
        dg = dG
    return {"dq": dq, "dk": dkk, "dv": dvv, "dbeta": db, "dg": dg, "dh0": dS}


def chunk_transfer(k, v, beta, g=None):
    """Affine summary of one chunk (one head): S_end = S_start @ P + Bw.

    P (d_k x d_k) is the chunk's transition product written in WY form,
    Diag(Gam_L) - W^T Kd with W = (I + A)^{-1} diag(beta) (K*Gam); Bw (d_v x d_k)
    is the state the chunk writes from a zero initial state."""
    k, v, beta = (np.asarray(a, np.float64) for a in (k, v, beta))
    L, dk = k.shape
    G = _as_channel_gate(g, L, dk)
    gam = np.cumsum(G, axis=0)
    Gam = np.exp(gam)
    E = np.exp(gam[:, None, :] - gam[None, :, :])
    A = beta[:, None] * np.einsum("tc,sc,tsc->ts", k, k, E) * np.tril(np.ones((L, L)), -1)
    W = np.linalg.solve(np.eye(L) + A, beta[:, None] * (k * Gam))
    Kd = k * np.exp(gam[-1][None, :] - gam)
    P = np.diag(Gam[-1]) - W.T @ Kd
    _, Bw, _ = _chunk_forward(np.zeros_like(k), k, v, beta, G, np.zeros((v.shape[1], dk)))
    return P, Bw
