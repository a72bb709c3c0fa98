"""Phase-controlled gate (SFDA), recurrent form, fp64 -- TEST INFRASTRUCTURE ONLY.

Reading of the SFDA technical summary (gist.science), "Kernarchitektur" and
"Reelle Implementierung", transposed to the d_v x d_k orientation of this
operator, with real inputs:
  * the state is complex, S = A + i B (d_v x d_k);
  * step t applies the complex diagonal gate Lambda_t = diag(exp(g_t) exp(i theta_t))
    (one log-decay and one phase per key channel; a scalar g is shared by all
    channels, no g means no decay), then the rank-one erase with the real key,
    then the write of the real value:
        S_t = S_{t-1} Lambda_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T;
  * the output is the real part, o_t = Re(S_t q_t).
With theta = 0 and a real initial state B stays zero and this is KDA ("KDA als
Spezialfall", "Zentrale Beitraege").  In real arithmetic each key channel's pair
(A_c, B_c) is turned by a 2 x 2 rotation-decay block and the erase and write act
on A and B separately.

Three evaluations, pinned against each other and against closed forms in
tests/test_oracle_sfda.py:
  forward           the recurrence in complex numpy, vectorised over heads;
  forward_products  explicit complex transition matrices and their products
                    (brute force, O(T^2 d_k^3));
  forward_blocks    the real 2 x 2 rotation-decay form (A, B real);
and the reverse mode of the recurrence, ``backward``, pinned by central
differences and, at zero phase, by the C oracle's reverse mode.
"""
from __future__ import annotations

import numpy as np

from . import brute


def _f64(x):
    return None if x is None else np.asarray(x, np.float64)


def _gate(g, theta, T, dk, lead):
    """Complex per-channel gates [..., T, dk]: exp(g) exp(i theta)."""
    theta = _f64(theta)
    if g is None:
        mag = np.ones(lead + (T, dk))
    else:
        g = _f64(g)
        mag = np.exp(g)[..., None] * np.ones(dk) if g.ndim == len(lead) + 1 else np.exp(g)
    return mag * np.exp(1j * theta)


def _beta(beta, k, eps):
    beta = _f64(beta)
    if eps is None:
        return beta
    return beta / (np.sum(_f64(k) ** 2, axis=-1) + eps)   # Kaczmarz step (KLA abstract)


def forward(q, k, v, beta, g, theta, h0_re=None, h0_im=None, eps=None):
    """Inputs [B, H, T, .]: q, k [dk]; v [dv]; beta [B,H,T]; g None, [B,H,T] or
    [B,H,T,dk]; theta [B,H,T,dk]; h0_re / h0_im [B,H,dv,dk] or None (zero).
    ``eps`` not None: beta is eta of the Kaczmarz step.
    Returns o [B,H,T,dv] (real) and the final state [B,H,dv,dk] (complex)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Bn, H, T, dk = q.shape
    dv = v.shape[-1]
    lam = _gate(g, theta, T, dk, (Bn, H))
    b = _beta(beta, k, eps)
    S = np.zeros((Bn, H, dv, dk), np.complex128)
    if h0_re is not None:
        S += _f64(h0_re)
    if h0_im is not None:
        S += 1j * _f64(h0_im)
    o = np.zeros((Bn, H, T, dv))
    for t in range(T):
        S = S * lam[:, :, t, None, :]                        # gate the key channels
        p = np.einsum("bhvc,bhc->bhv", S, k[:, :, t])        # S k
        u = b[:, :, t, None] * (v[:, :, t] - p)              # beta (v - S k)
        S = S + u[..., :, None] * k[:, :, t, None, :]        # + u k^T
        o[:, :, t] = np.einsum("bhvc,bhc->bhv", S, q[:, :, t]).real
    return o, S


def forward_products(q, k, v, beta, g, theta, h0=None, eps=None):
    """One head, brute force: complex M_t = Lambda_t (I - beta_t k_t k_t^T) as
    explicit matrices, S_t = h0 M_1..M_t + sum_j beta_j v_j k_j^T M_{j+1}..M_t.
    q, k [T, dk]; v [T, dv]; beta [T]; g None, [T] or [T, dk]; theta [T, dk];
    h0 complex [dv, dk] or None.  Returns (o [T, dv] real, S_T complex)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, dk = q.shape
    dv = v.shape[1]
    lam = _gate(g, theta, T, dk, ())
    b = _beta(beta, k, eps)
    Ms = [brute.transition(k[t], b[t], lam[t]) for t in range(T)]
    S0 = np.zeros((dv, dk), np.complex128) if h0 is None else np.asarray(h0, np.complex128)
    o = np.zeros((T, dv))
    S = S0
    for t in range(T):
        P = brute.product(Ms[: t + 1])
        S = S0 @ P
        for j in range(t + 1):
            W = np.outer(b[j] * v[j], k[j]).astype(np.complex128)
            tail = brute.product(Ms[j + 1: t + 1])
            S = S + (W if tail is None else W @ tail)
        o[t] = (S @ q[t]).real
    return o, S


def forward_blocks(q, k, v, beta, g, theta, h0_re=None, h0_im=None, eps=None):
    """The real form: A, B [.., dv, dk] real; per key channel c the pair
    (A[:, c], B[:, c]) is turned by exp(g) [[cos, -sin], [sin, cos]](theta); then
    the erase with k acts on A and B, the write of v on A; o = A q."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Bn, H, T, dk = q.shape
    dv = v.shape[-1]
    b = _beta(beta, k, eps)
    theta = _f64(theta)
    if g is None:
        mag = np.ones((Bn, H, T, dk))
    else:
        g = _f64(g)
        mag = np.exp(g)[..., None] * np.ones(dk) if g.ndim == 3 else np.exp(g)
    A = np.zeros((Bn, H, dv, dk)) if h0_re is None else _f64(h0_re).copy()
    Bm = np.zeros((Bn, H, dv, dk)) if h0_im is None else _f64(h0_im).copy()
    o = np.zeros((Bn, H, T, dv))
    for t in range(T):
        c, s, m = np.cos(theta[:, :, t]), np.sin(theta[:, :, t]), mag[:, :, t]
        A, Bm = (m * c)[:, :, None, :] * A - (m * s)[:, :, None, :] * Bm, \
                (m * s)[:, :, None, :] * A + (m * c)[:, :, None, :] * Bm
        kt = k[:, :, t]
        pa = np.einsum("bhvc,bhc->bhv", A, kt)
        pb = np.einsum("bhvc,bhc->bhv", Bm, kt)
        A = A + (b[:, :, t, None] * (v[:, :, t] - pa))[..., None] * kt[:, :, None, :]
        Bm = Bm - (b[:, :, t, None] * pb)[..., None] * kt[:, :, None, :]
        o[:, :, t] = np.einsum("bhvc,bhc->bhv", A, q[:, :, t])
    return o, A + 1j * Bm


def backward(q, k, v, beta, g, theta, h0_re=None, h0_im=None, dout=None, dhT_re=None, dhT_im=None, eps=None):
    """Reverse mode of ``forward``: the vector-Jacobian products of
        L = <o, dout> + <Re S_T, dhT_re> + <Im S_T, dhT_im>
    with respect to every input.  Shapes as for ``forward``; dout [B,H,T,dv] or
    None (zero), dhT_re / dhT_im [B,H,dv,dk] or None.  With ``eps`` the beta
    argument is eta of the Kaczmarz step and "dbeta" holds d eta (dk then
    includes the path through the step size).

    Each step is taken back in the order it was taken forward.  A complex
    quantity Z carries the cotangent Zb = dL/dRe Z + i dL/dIm Z; a real input x
    that enters as x w gets Re(conj(w) Zb); through the holomorphic exp of the
    gate, lb = conj(lam) lamb; g and theta are the real and imaginary parts of
    the gate's logarithm, so dg = Re lb (summed over the channels for a scalar
    g) and dtheta = Im lb.

    Returns a dict: dq, dk, dv [B,H,T,.], dbeta [B,H,T], dg (None / like g),
    dtheta [B,H,T,dk], dh0_re, dh0_im [B,H,dv,dk]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Bn, H, T, dk = q.shape
    dv = v.shape[-1]
    lam = _gate(g, theta, T, dk, (Bn, H))
    b = _beta(beta, k, eps)
    S = np.zeros((Bn, H, dv, dk), np.complex128)
    if h0_re is not None:
        S += _f64(h0_re)
    if h0_im is not None:
        S += 1j * _f64(h0_im)
    prev = np.empty((T, Bn, H, dv, dk), np.complex128)   # the state entering each step
    for t in range(T):
        prev[t] = S
        St = S * lam[:, :, t, None, :]
        u = b[:, :, t, None] * (v[:, :, t] - np.einsum("bhvc,bhc->bhv", St, k[:, :, t]))
        S = St + u[..., :, None] * k[:, :, t, None, :]
    do = np.zeros((Bn, H, T, dv)) if dout is None else _f64(dout)
    Sb = np.zeros((Bn, H, dv, dk), np.complex128)
    if dhT_re is not None:
        Sb += _f64(dhT_re)
    if dhT_im is not None:
        Sb += 1j * _f64(dhT_im)
    dq = np.zeros_like(q)
    dkk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    db = np.zeros((Bn, H, T))
    lb = np.zeros((Bn, H, T, dk), np.complex128)
    for t in range(T - 1, -1, -1):
        kt, qt, lt = k[:, :, t], q[:, :, t], lam[:, :, t]
        Sp = prev[t]
        St = Sp * lt[:, :, None, :]                          # gated state
        p = np.einsum("bhvc,bhc->bhv", St, kt)
        u = b[:, :, t, None] * (v[:, :, t] - p)
        Sn = St + u[..., :, None] * kt[:, :, None, :]        # state after the step
        # o_t = Re(Sn q_t)
        Sb = Sb + do[:, :, t, :, None] * qt[:, :, None, :]
        dq[:, :, t] = np.einsum("bhvc,bhv->bhc", Sn.real, do[:, :, t])
        # Sn = St + u k^T
        ub = np.einsum("bhvc,bhc->bhv", Sb, kt)
        dkk[:, :, t] = np.einsum("bhv,bhvc->bhc", np.conj(u), Sb).real
        # u = b (v - p)
        dvv[:, :, t] = b[:, :, t, None] * ub.real
        db[:, :, t] = np.einsum("bhv,bhv->bh", np.conj(ub), v[:, :, t] - p).real
        pb = -b[:, :, t, None] * ub
        # p = St k
        Stb = Sb + pb[..., :, None] * kt[:, :, None, :]
        dkk[:, :, t] += np.einsum("bhvc,bhv->bhc", np.conj(St), pb).real
        # St = Sp diag(lam_t)
        lamb = np.einsum("bhvc,bhvc->bhc", Stb, np.conj(Sp))
        lb[:, :, t] = np.conj(lt) * lamb
        Sb = Stb * np.conj(lt)[:, :, None, :]
    out = {"dq": dq, "dk": dkk, "dv": dvv, "dtheta": lb.imag.copy(), "dh0_re": Sb.real.copy(),
           "dh0_im": Sb.imag.copy(), "dg": None}
    if g is not None:
        out["dg"] = lb.real.sum(axis=-1) if _f64(g).ndim == 3 else lb.real.copy()
    if eps is None:
        out["dbeta"] = db
    else:   # beta = eta / n, n = ||k||^2 + eps
        n = np.sum(k ** 2, axis=-1) + eps
        out["dbeta"] = db / n
        out["dk"] = dkk - 2.0 * (db * b / n)[..., None] * k
    return out
