"""fp64 CPU oracle for the chunkwise gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and the
two share no code.

Contents
--------
* ``forward`` / ``backward``: the plain sequential recurrence and its
  hand-derived reverse mode, in C (``dn_oracle.c``), fp64, threads over heads.
  This is the definition every other result is compared with.
* ``chunked``: the same operator evaluated chunk by chunk in the WY / affine
  chunk-transfer form, in numpy fp64 (pinned to the sequential form for every
  chunk size).
* ``brute``: the explicit product of d_k x d_k transition matrices.
* ``sfda``: the phase-controlled gate of the SFDA summary (complex state,
  per-channel rotation-decay, real inputs, real-part readout), recurrent form,
  in three evaluations pinned against each other and the above.
* ``kaczmarz_*``: the Kaczmarz step size of the KLA abstract on top of
  ``forward`` / ``backward``.

Operator (per head, state S in R^{d_v x d_k}):
    S_t = S_{t-1} Diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
Sources: ReWY abstract (DeltaNet / GDN / KDA operators, exact chunkwise
reformulation); SFDA technical summary, "Kernarchitektur" (decay-then-erase
recurrence, read in transposed form with zero phase); KLA abstract (Kaczmarz
step); Fast Weight Attention abstract (read-after-write readout).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdn_oracle.so")
_lib = None

GATE_NONE, GATE_SCALAR, GATE_VECTOR = 0, 1, 2


def build_oracle() -> str:
    """Compile ``dn_oracle.c`` into ``libdn_oracle.so`` (always recompiles)."""
    src = os.path.join(_HERE, "dn_oracle.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O3", "-march=x86-64-v2", "-std=c99", "-D_POSIX_C_SOURCE=200809L",
           "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build_oracle()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.dn_oracle_fwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, i]
    lib.dn_oracle_fwd.restype = i
    lib.dn_oracle_bwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp,
                                  dp, dp, dp, dp, dp, dp, i]
    lib.dn_oracle_bwd.restype = i
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _gate_of(g, dk):
    """None -> no gate; [B,H,T] -> scalar gate; [B,H,T,dk] -> vector gate."""
    if g is None:
        return GATE_NONE
    if g.ndim == 4:
        if g.shape[-1] != dk:
            raise ValueError("vector gate must be [B,H,T,dk]")
        return GATE_VECTOR
    return GATE_SCALAR


def _shapes(q, v):
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    return B, H, T, dk, dv


def forward(q, k, v, beta, g=None, h0=None, gate=None, nthreads=0):
    """Sequential forward.  Shapes: q,k [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T];
    g None, [B,H,T] (scalar gate) or [B,H,T,dk] (vector gate); h0 None or [B,H,dv,dk].
    Returns (o [B,H,T,dv], hT [B,H,dv,dk]) in fp64."""
    q, k, v, beta, g, h0 = map(_f64, (q, k, v, beta, g, h0))
    B, H, T, dk, dv = _shapes(q, v)
    if gate is None:
        gate = _gate_of(g, dk)
    o = np.zeros((B, H, T, dv))
    hT = np.zeros((B, H, dv, dk))
    rc = _load().dn_oracle_fwd(B * H, T, dk, dv, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                               _ptr(g), _ptr(h0), _ptr(o), _ptr(hT), int(nthreads))
    if rc != 0:
        raise RuntimeError("dn_oracle_fwd failed")
    return o, hT


def backward(q, k, v, beta, g, h0, do, dhT=None, gate=None, nthreads=0):
    """Reverse mode of ``forward`` for L = <O, dO> + <hT, dhT>.
    Returns a dict with dq, dk, dv, dbeta, dg (None without a gate), dh0."""
    q, k, v, beta, g, h0, do, dhT = map(_f64, (q, k, v, beta, g, h0, do, dhT))
    B, H, T, dk, dv = _shapes(q, v)
    if gate is None:
        gate = _gate_of(g, dk)
    dq = np.zeros_like(q)
    dkk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    db = np.zeros_like(beta)
    dg = None if gate == GATE_NONE else np.zeros_like(g)
    dh0 = np.zeros((B, H, dv, dk))
    rc = _load().dn_oracle_bwd(B * H, T, dk, dv, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                               _ptr(g), _ptr(h0), _ptr(do), _ptr(dhT), _ptr(dq), _ptr(dkk),
                               _ptr(dvv), _ptr(db), _ptr(dg), _ptr(dh0), int(nthreads))
    if rc != 0:
        raise RuntimeError("dn_oracle_bwd failed")
    return {"dq": dq, "dk": dkk, "dv": dvv, "dbeta": db, "dg": dg, "dh0": dh0}


# --------------------------------------------------------------------------- Kaczmarz step
# KLA abstract: the Kaczmarz (normalised least-squares) step of the delta rule sets
# beta_t = eta_t / (||k_t||^2 + eps); nothing else in the recurrence changes.


def kaczmarz_beta(eta, k, eps):
    """beta_t = eta_t / (||k_t||^2 + eps), fp64."""
    eta, k = _f64(eta), _f64(k)
    return eta / (np.sum(k * k, axis=-1) + eps)


def kaczmarz_forward(q, k, v, eta, g=None, h0=None, eps=1e-6, gate=None, nthreads=0):
    """``forward`` with beta = kaczmarz_beta(eta, k, eps)."""
    return forward(q, k, v, kaczmarz_beta(eta, k, eps), g, h0, gate=gate, nthreads=nthreads)


def kaczmarz_backward(q, k, v, eta, g, h0, do, dhT=None, eps=1e-6, gate=None, nthreads=0):
    """Reverse mode through beta = eta / n, n = ||k||^2 + eps (chain rule on top of
    ``backward``): d eta = d beta / n and dk gains -2 (d beta) beta k / n.
    Returns the dict of ``backward`` with "deta" in place of "dbeta"."""
    k64 = _f64(k)
    n = np.sum(k64 * k64, axis=-1) + eps
    beta = _f64(eta) / n
    gr = backward(q, k, v, beta, g, h0, do, dhT, gate=gate, nthreads=nthreads)
    db = gr.pop("dbeta")
    gr["deta"] = db / n
    gr["dk"] = gr["dk"] - (2.0 * db * beta / n)[..., None] * k64
    return gr
