"""Pins for the fp64 oracle (CPU only).

The oracle is trusted only because it agrees with things other than itself:
  * a worked example computed by hand (tests/golden/hand_example.json),
  * central finite differences of its own forward for every gradient,
  * the explicit d_k x d_k transition-matrix products (brute force),
  * the chunkwise WY form for every chunk size, including non-divisors
    (C = 1 is the recurrent form, C = T the fully parallel masked form),
  * the affine chunk transfer S_end = S_start P + B_chunk,
  * closed forms: beta = 0 (pure decay), alpha = 1 (GDN with g = 0 is DeltaNet),
    the Kaczmarz projection, orthonormal keys,
  * a vector gate with equal channels is the scalar gate.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute, chunked

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_case(seed, B=1, H=2, T=9, dk=3, dv=4, gate=1, h0=True, beta_scale=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, dv))
    beta = beta_scale / (1 + np.exp(-r.standard_normal((B, H, T))))
    if gate == 0:
        g = None
    elif gate == 1:
        g = -np.logaddexp(0, r.standard_normal((B, H, T))) / 4
    else:
        g = -np.logaddexp(0, r.standard_normal((B, H, T, dk))) / 4
    hh = 0.5 * r.standard_normal((B, H, dv, dk)) if h0 else None
    do = r.standard_normal((B, H, T, dv))
    dhT = r.standard_normal((B, H, dv, dk))
    return dict(q=q, k=k, v=v, beta=beta, g=g, h0=hh, do=do, dhT=dhT)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return np.max(np.abs(a - b)) / (den if den > 0 else 1.0)


# --------------------------------------------------------------------------- golden


def test_hand_example():
    gd = json.load(open(os.path.join(HERE, "golden", "hand_example.json")))
    x = gd["inputs"]
    q = np.array(x["q"])[None, None]
    k = np.array(x["k"])[None, None]
    v = np.array(x["v"])[None, None]
    beta = np.array(x["beta"])[None, None]
    g = np.log(np.array(x["g_exp"]))[None, None]
    do = np.array(x["do"])[None, None]
    o, hT = oracle.forward(q, k, v, beta, g, None)
    gr = oracle.backward(q, k, v, beta, g, None, do, None)
    ex = gd["expected"]
    np.testing.assert_allclose(o[0, 0], ex["o"], atol=1e-14)
    np.testing.assert_allclose(hT[0, 0], ex["hT"], atol=1e-14)
    for name in ("dq", "dk", "dv", "dbeta", "dg", "dh0"):
        np.testing.assert_allclose(gr[name][0, 0], ex[name], atol=1e-14, err_msg=name)


# --------------------------------------------------------------------------- finite differences


def _loss(c, **over):
    d = dict(c)
    d.update(over)
    o, hT = oracle.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    return np.sum(o * d["do"]) + np.sum(hT * d["dhT"])


@pytest.mark.parametrize("gate", [0, 1, 2])
def test_finite_differences(gate):
    c = rand_case(11 + gate, T=7, gate=gate)
    gr = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"], c["do"], c["dhT"])
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("h0", "dh0")]
    if gate:
        names.append(("g", "dg"))
    h = 1e-6
    for inp, gname in names:
        x = c[inp]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xp[idx] += h
            xm = x.copy()
            xm[idx] -= h
            fd[idx] = (_loss(c, **{inp: xp}) - _loss(c, **{inp: xm})) / (2 * h)
        assert rel(gr[gname], fd) < 1e-7, (gate, gname, rel(gr[gname], fd))



def _loss_kacz(c, eps, **over):
    d = dict(c)
    d.update(over)
    o, hT = oracle.kaczmarz_forward(d["q"], d["k"], d["v"], d["eta"], d["g"], d["h0"], eps=eps)
    return np.sum(o * d["do"]) + np.sum(hT * d["dhT"])


@pytest.mark.parametrize("gate", [1, 2])
def test_finite_differences_kaczmarz(gate):
    """The Kaczmarz chain rule (d eta and the extra dk term) against central
    differences of the Kaczmarz forward, with unnormalised keys so ||k|| matters."""
    c = rand_case(41 + gate, T=6, gate=gate)
    r = np.random.default_rng(5 + gate)
    c["k"] = r.standard_normal(c["k"].shape) * 1.3
    c["eta"] = 1 / (1 + np.exp(-r.standard_normal(c["beta"].shape)))
    eps = 1e-3
    gr = oracle.kaczmarz_backward(c["q"], c["k"], c["v"], c["eta"], c["g"], c["h0"], c["do"], c["dhT"], eps=eps)
    h = 1e-6
    for inp, gname in [("eta", "deta"), ("k", "dk"), ("q", "dq")]:
        x = c[inp]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xp[idx] += h
            xm = x.copy()
            xm[idx] -= h
            fd[idx] = (_loss_kacz(c, eps, **{inp: xp}) - _loss_kacz(c, eps, **{inp: xm})) / (2 * h)
        assert rel(gr[gname], fd) < 1e-7, (gate, gname, rel(gr[gname], fd))


def test_kaczmarz_step_projects_onto_the_key():
    """With g = 0 and eta = 1 one Kaczmarz step solves S k = v exactly (the KLA
    abstract's normalised least-squares step): o for q = k is v up to eps."""
    r = np.random.default_rng(8)
    dk, dv = 5, 3
    k = r.standard_normal((1, 1, 1, dk)) * 2.0
    v = r.standard_normal((1, 1, 1, dv))
    h0 = r.standard_normal((1, 1, dv, dk))
    eps = 1e-12
    o, hT = oracle.kaczmarz_forward(k, k, v, np.ones((1, 1, 1)), None, h0, eps=eps)
    assert np.max(np.abs(o[0, 0, 0] - v[0, 0, 0])) < 1e-9

# --------------------------------------------------------------------------- brute force


@pytest.mark.parametrize("gate", [0, 1, 2])
def test_brute_force_transfer_product(gate):
    c = rand_case(21 + gate, H=2, T=10, gate=gate)
    o, hT = oracle.forward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"])
    for h in range(2):
        ob, hb = brute.forward(c["q"][0, h], c["k"][0, h], c["v"][0, h], c["beta"][0, h],
                               None if c["g"] is None else c["g"][0, h], c["h0"][0, h])
        assert rel(o[0, h], ob) < 1e-12
        assert rel(hT[0, h], hb) < 1e-12


# --------------------------------------------------------------------------- chunk invariance


@pytest.mark.parametrize("gate", [0, 1, 2])
@pytest.mark.parametrize("C", [1, 2, 3, 5, 8, 16, 37])
def test_chunked_equals_sequential(gate, C):
    T = 37
    c = rand_case(31 + gate, H=2, T=T, dk=5, dv=4, gate=gate)
    o, hT = oracle.forward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"])
    oc, hc, _ = chunked.forward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"], C=C)
    assert rel(oc, o) < 1e-11
    assert rel(hc, hT) < 1e-11
    gs = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"], c["do"], c["dhT"])
    gc = chunked.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"], c["do"], c["dhT"], C=C)
    for n in ("dq", "dk", "dv", "dbeta", "dg", "dh0"):
        if gs[n] is None:
            assert gc[n] is None
            continue
        assert rel(gc[n], gs[n]) < 1e-10, (n, rel(gc[n], gs[n]))


@pytest.mark.parametrize("gate", [0, 1, 2])
def test_affine_chunk_transfer(gate):
    c = rand_case(41 + gate, H=1, T=12, dk=4, dv=3, gate=gate)
    q, k, v, beta = (c[n][0, 0] for n in ("q", "k", "v", "beta"))
    g = None if c["g"] is None else c["g"][0, 0]
    S = c["h0"][0, 0]
    for t0 in range(0, 12, 4):
        sl = slice(t0, t0 + 4)
        P, Bw = chunked.chunk_transfer(k[sl], v[sl], beta[sl], None if g is None else g[sl])
        assert rel(P, brute.chunk_product(k[sl], beta[sl], None if g is None else g[sl])) < 1e-12
        _, S_seq = oracle.forward(q[sl][None, None], k[sl][None, None], v[sl][None, None],
                                  beta[sl][None, None], None if g is None else g[sl][None, None],
                                  S[None, None])
        S = S @ P + Bw
        assert rel(S, S_seq[0, 0]) < 1e-12
    _, hT = oracle.forward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"])
    assert rel(S, hT[0, 0]) < 1e-12


# --------------------------------------------------------------------------- closed forms


@pytest.mark.parametrize("gate", [1, 2])
def test_beta_zero_is_pure_decay(gate):
    c = rand_case(51 + gate, H=2, T=11, gate=gate)
    beta = np.zeros_like(c["beta"])
    q, k, v, h0, do, dhT = (c[n] for n in ("q", "k", "v", "h0", "do", "dhT"))
    gch = c["g"] if gate == 2 else np.repeat(c["g"][..., None], q.shape[-1], axis=-1)
    G = np.cumsum(gch, axis=2)                                   # [B,H,T,dk]
    S = h0[:, :, None] * np.exp(G)[:, :, :, None, :]             # [B,H,T,dv,dk]
    o_ref = np.einsum("bhtic,bhtc->bhti", S, q)
    o, hT = oracle.forward(q, k, v, beta, c["g"], h0)
    assert rel(o, o_ref) < 1e-13
    assert rel(hT, S[:, :, -1]) < 1e-13
    gr = oracle.backward(q, k, v, beta, c["g"], h0, do, dhT)
    assert np.max(np.abs(gr["dk"])) == 0 and np.max(np.abs(gr["dv"])) == 0
    assert rel(gr["dq"], np.einsum("bhtic,bhti->bhtc", S, do)) < 1e-13
    T = q.shape[2]
    outer = np.einsum("bhti,bhtc->bhtic", do, q)                 # do_s q_s^T
    dh0 = dhT * np.exp(G[:, :, -1])[:, :, None, :] + np.sum(outer * np.exp(G)[:, :, :, None, :], axis=2)
    assert rel(gr["dh0"], dh0) < 1e-13
    # dL/dG_s[c] = sum_i (do_s q_s^T)[i,c] S_s[i,c] (+ dhT term at the last step); dg = reverse cumsum
    dG = np.sum(outer * S, axis=3)
    dG[:, :, -1] += np.sum(dhT * S[:, :, -1], axis=2)
    dg = np.cumsum(dG[:, :, ::-1], axis=2)[:, :, ::-1]
    if gate == 1:
        dg = dg.sum(-1)
    assert rel(gr["dg"], dg) < 1e-12
    # dbeta_t = (dS_t k_t) . (v_t - S_t k_t) with dS_t the total cotangent of S_t
    db = np.zeros_like(beta)
    for t in range(T):
        dS = dhT * np.exp(G[:, :, -1] - G[:, :, t])[:, :, None, :]
        for s in range(t, T):
            dS = dS + outer[:, :, s] * np.exp(G[:, :, s] - G[:, :, t])[:, :, None, :]
        du = np.einsum("bhic,bhc->bhi", dS, k[:, :, t])
        p = np.einsum("bhic,bhc->bhi", S[:, :, t], k[:, :, t])
        db[:, :, t] = np.sum(du * (v[:, :, t] - p), axis=-1)
    assert rel(gr["dbeta"], db) < 1e-12
    assert np.max(np.abs(db)) > 1e-3  # dbeta does not vanish at beta = 0


def test_alpha_one_gdn_is_deltanet():
    c = rand_case(61, H=2, T=13, gate=1)
    g0 = np.zeros_like(c["g"])
    args = (c["q"], c["k"], c["v"], c["beta"])
    o1, h1 = oracle.forward(*args, g0, c["h0"])
    o0, h0 = oracle.forward(*args, None, c["h0"])
    assert np.array_equal(o1, o0) and np.array_equal(h1, h0)
    g1 = oracle.backward(*args, g0, c["h0"], c["do"], c["dhT"])
    g0_ = oracle.backward(*args, None, c["h0"], c["do"], c["dhT"])
    for n in ("dq", "dk", "dv", "dbeta", "dh0"):
        assert np.array_equal(g1[n], g0_[n]), n


def test_kaczmarz_projection():
    """beta_t = eta_t / ||k_t||^2 gives S_t k_t = (1 - eta_t) Sbar_t k_t + eta_t v_t; eta = 1 is an
    exact projection S_t k_t = v_t (KLA abstract: Kaczmarz-derived step)."""
    r = np.random.default_rng(71)
    T, dk, dv = 10, 4, 3
    k = r.standard_normal((1, 1, T, dk)) * 2.0
    v = r.standard_normal((1, 1, T, dv))
    g = -np.abs(r.standard_normal((1, 1, T))) / 5
    h0 = r.standard_normal((1, 1, dv, dk))
    for eta in (np.ones(T), r.uniform(0.1, 0.9, T)):
        beta = (eta / np.sum(k[0, 0] ** 2, axis=-1))[None, None]
        o, _ = oracle.forward(k, k, v, beta, g, h0)                 # q_t = k_t reads S_t k_t
        for t in range(T):
            _, Sprev = oracle.forward(k[:, :, :t], k[:, :, :t], v[:, :, :t], beta[:, :, :t],
                                      g[:, :, :t], h0)
            pbar = np.exp(g[0, 0, t]) * Sprev[0, 0] @ k[0, 0, t]
            ref = (1 - eta[t]) * pbar + eta[t] * v[0, 0, t]
            assert rel(o[0, 0, t], ref) < 1e-12


@pytest.mark.parametrize("gate", [0, 1])
def test_orthonormal_keys(gate):
    r = np.random.default_rng(81 + gate)
    T = dk = 6
    dv = 3
    k = np.eye(dk)[None, None, :T]
    q = r.standard_normal((1, 1, T, dk))
    v = r.standard_normal((1, 1, T, dv))
    beta = np.ones((1, 1, T))
    g = None if gate == 0 else -np.abs(r.standard_normal((1, 1, T)))
    G = np.zeros(T) if g is None else np.cumsum(g[0, 0])
    o, hT = oracle.forward(q, k, v, beta, g, None)
    for t in range(T):
        ref = sum(np.exp(G[t] - G[s]) * q[0, 0, t, s] * v[0, 0, s] for s in range(t + 1))
        assert rel(o[0, 0, t], ref) < 1e-13
    Sref = np.stack([np.exp(G[-1] - G[s]) * v[0, 0, s] for s in range(T)], axis=1)
    assert rel(hT[0, 0], Sref) < 1e-13


def test_vector_gate_with_equal_channels_is_scalar():
    c = rand_case(91, H=2, T=15, gate=1)
    gv = np.repeat(c["g"][..., None], c["q"].shape[-1], axis=-1)
    args = (c["q"], c["k"], c["v"], c["beta"])
    os_, hs = oracle.forward(*args, c["g"], c["h0"])
    ov, hv = oracle.forward(*args, gv, c["h0"])
    assert rel(ov, os_) < 1e-14 and rel(hv, hs) < 1e-14
    gs = oracle.backward(*args, c["g"], c["h0"], c["do"], c["dhT"])
    gvv = oracle.backward(*args, gv, c["h0"], c["do"], c["dhT"])
    for n in ("dq", "dk", "dv", "dbeta", "dh0"):
        assert rel(gvv[n], gs[n]) < 1e-13
    assert rel(gvv["dg"].sum(-1), gs["dg"]) < 1e-13


def test_empty_and_null_paths():
    c = rand_case(101, H=2, T=0, gate=1)
    o, hT = oracle.forward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"])
    assert o.shape[2] == 0 and np.array_equal(hT, c["h0"])
    gr = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"], c["do"], c["dhT"])
    assert np.array_equal(gr["dh0"], c["dhT"])
    # no dO and no dhT: every gradient is zero
    c = rand_case(102, H=1, T=5, gate=2)
    gr = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0"], None, None)
    assert all(np.max(np.abs(gr[n])) == 0 for n in ("dq", "dk", "dv", "dbeta", "dg", "dh0"))
