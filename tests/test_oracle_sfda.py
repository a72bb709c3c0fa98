"""Pins of the phase-controlled gate's oracle (oracle/sfda.py, SFDA technical
summary, "Kernarchitektur", real inputs, transposed orientation): against the
independent C oracle at zero phase (KDA), against explicit products of complex
transition matrices, between the complex and the real 2 x 2 rotation-decay
forms, and against closed forms (pure rotation, decay of the magnitudes, the
Kaczmarz projection); its reverse mode against central differences of the
forward for every input and against the C oracle's reverse mode at zero
phase."""
import numpy as np
import pytest

import oracle
from oracle import sfda


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    den = np.max(np.abs(b))
    return np.max(np.abs(a - b)) / (den if den > 0 else 1.0)


def case(seed, Bn=2, H=2, T=7, dk=6, dv=5, gate="vector", phase=0.7, complex_h0=True):
    r = np.random.default_rng(seed)
    c = dict(q=r.standard_normal((Bn, H, T, dk)), k=r.standard_normal((Bn, H, T, dk)) * 0.5,
             v=r.standard_normal((Bn, H, T, dv)), beta=1 / (1 + np.exp(-r.standard_normal((Bn, H, T)))),
             theta=phase * r.standard_normal((Bn, H, T, dk)),
             h0_re=r.standard_normal((Bn, H, dv, dk)),
             h0_im=r.standard_normal((Bn, H, dv, dk)) if complex_h0 else None)
    c["g"] = {"none": None, "scalar": -np.abs(r.standard_normal((Bn, H, T))) / 4,
              "vector": -np.abs(r.standard_normal((Bn, H, T, dk))) / 4}[gate]
    return c


def run(c, **over):
    d = dict(c)
    d.update(over)
    return sfda.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], d["h0_re"], d["h0_im"])


@pytest.mark.parametrize("gate", ["none", "scalar", "vector"])
def test_zero_phase_is_the_c_oracle(gate):
    """theta = 0, real h0: the complex recurrence is the KDA / GDN / DeltaNet one."""
    c = case(1, gate=gate, complex_h0=False)
    o, S = run(c, theta=np.zeros_like(c["theta"]))
    o_ref, h_ref = oracle.forward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0_re"])
    assert rel(o, o_ref) < 1e-12 and rel(S.real, h_ref) < 1e-12
    assert np.max(np.abs(S.imag)) == 0.0


@pytest.mark.parametrize("gate", ["none", "scalar", "vector"])
def test_recurrence_equals_transition_products(gate):
    c = case(2, Bn=1, H=2, T=5, dk=4, dv=3, gate=gate)
    o, S = run(c)
    for h in range(2):
        g = None if c["g"] is None else c["g"][0, h]
        h0 = c["h0_re"][0, h] + 1j * c["h0_im"][0, h]
        ob, Sb = sfda.forward_products(c["q"][0, h], c["k"][0, h], c["v"][0, h], c["beta"][0, h], g,
                                       c["theta"][0, h], h0)
        assert rel(o[0, h], ob) < 1e-12 and rel(S[0, h], Sb) < 1e-12


@pytest.mark.parametrize("gate", ["none", "scalar", "vector"])
def test_complex_form_equals_real_rotation_blocks(gate):
    c = case(3, gate=gate)
    o, S = run(c)
    ob, Sb = sfda.forward_blocks(c["q"], c["k"], c["v"], c["beta"], c["g"], c["theta"], c["h0_re"], c["h0_im"])
    assert rel(o, ob) < 1e-12 and rel(S, Sb) < 1e-12


def test_pure_rotation_closed_form():
    """beta = 0, g = 0: every key channel of the state turns by the summed phase."""
    c = case(4, gate="none")
    o, S = run(c, beta=np.zeros_like(c["beta"]))
    S0 = c["h0_re"] + 1j * c["h0_im"]
    expect = S0 * np.exp(1j * np.sum(c["theta"], axis=2))[:, :, None, :]
    assert rel(S, expect) < 1e-13
    # and the readout of the last step is the real part of S_T q_T
    assert rel(o[:, :, -1], np.einsum("bhvc,bhc->bhv", expect, c["q"][:, :, -1]).real) < 1e-13


def test_decay_of_magnitudes():
    """beta = 0: |S_T| = |S_0| exp(sum_t g_t) element by element, whatever the phases."""
    c = case(5, gate="vector")
    _, S = run(c, beta=np.zeros_like(c["beta"]))
    S0 = c["h0_re"] + 1j * c["h0_im"]
    assert rel(np.abs(S), np.abs(S0) * np.exp(np.sum(c["g"], axis=2))[:, :, None, :]) < 1e-13


def test_kaczmarz_projection_with_phases():
    """With the Kaczmarz step and eta = 1 the last step solves S_T k_T = v_T exactly:
    the erase removes the gated state's whole component along k_T, real and
    imaginary, and the write puts v_T there (KLA abstract's projection)."""
    c = case(6, gate="vector")
    eta = np.ones_like(c["beta"])
    _, S = sfda.forward(c["q"], c["k"], c["v"], eta, c["g"], c["theta"], c["h0_re"], c["h0_im"], eps=0.0)
    Sk = np.einsum("bhvc,bhc->bhv", S, c["k"][:, :, -1])
    assert rel(Sk, c["v"][:, :, -1]) < 1e-12


def test_a_plausible_mistake_is_caught():
    """A planted mistake -- the phase applied with the opposite sign -- fails the
    pins above (the transition-product comparison catches it)."""
    c = case(7, Bn=1, H=1, T=4, dk=4, dv=3)
    o_wrong, _ = run(c, theta=-c["theta"])
    h0 = c["h0_re"][0, 0] + 1j * c["h0_im"][0, 0]
    ob, _ = sfda.forward_products(c["q"][0, 0], c["k"][0, 0], c["v"][0, 0], c["beta"][0, 0], c["g"][0, 0],
                                  c["theta"][0, 0], h0)
    assert rel(o_wrong[0, 0], ob) > 1e-3


def _loss(c, do, dr, di, eps=None, **over):
    d = dict(c)
    d.update(over)
    o, S = sfda.forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], d["h0_re"], d["h0_im"], eps=eps)
    return np.sum(o * do) + np.sum(S.real * dr) + np.sum(S.imag * di)


def _central_differences(c, do, dr, di, name, eps=None, h=1e-6):
    x = c[name]
    fd = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        a = x.copy()
        a[i] += h
        lp = _loss(c, do, dr, di, eps, **{name: a})
        a[i] -= 2 * h
        lm = _loss(c, do, dr, di, eps, **{name: a})
        fd[i] = (lp - lm) / (2 * h)
    return fd


@pytest.mark.parametrize("gate", ["none", "scalar", "vector"])
@pytest.mark.parametrize("kz", [None, 1e-3])
def test_backward_central_differences(gate, kz):
    c = case(11, Bn=1, H=2, T=6, dk=4, dv=3, gate=gate)
    r = np.random.default_rng(12)
    do, dr, di = r.standard_normal((1, 2, 6, 3)), r.standard_normal((1, 2, 3, 4)), r.standard_normal((1, 2, 3, 4))
    gr = sfda.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["theta"], c["h0_re"], c["h0_im"], do, dr, di,
                       eps=kz)
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "theta": "dtheta", "h0_re": "dh0_re",
             "h0_im": "dh0_im"}
    if gate != "none":
        names["g"] = "dg"
    for name, key in names.items():
        fd = _central_differences(c, do, dr, di, name, kz)
        assert rel(gr[key], fd) < 1e-7, (name, rel(gr[key], fd))
    if gate == "none":
        assert gr["dg"] is None


@pytest.mark.parametrize("gate", ["none", "scalar", "vector"])
def test_backward_zero_phase_is_the_c_oracle(gate):
    """theta = 0, real h0 and dhT: the reverse mode is the C oracle's (KDA / GDN /
    DeltaNet), and dh0 has no imaginary part."""
    c = case(13, gate=gate, complex_h0=False)
    r = np.random.default_rng(14)
    do, dr = r.standard_normal(c["v"].shape), r.standard_normal(c["h0_re"].shape)
    gr = sfda.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], np.zeros_like(c["theta"]), c["h0_re"], None, do, dr)
    ref = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["h0_re"], do, dr)
    for key in ("dq", "dk", "dv", "dbeta", "dg"):
        if ref[key] is None:
            assert gr[key] is None
            continue
        assert rel(gr[key], ref[key]) < 1e-12, key
    assert rel(gr["dh0_re"], ref["dh0"]) < 1e-12
    assert np.max(np.abs(gr["dh0_im"])) == 0.0


def test_a_plausible_reverse_mode_mistake_is_caught():
    """The phase gradient taken through the gate without its conjugate (the
    reverse mode run at the opposite phases) disagrees with central differences."""
    c = case(15, Bn=1, H=1, T=4, dk=3, dv=2)
    r = np.random.default_rng(16)
    do, dr, di = r.standard_normal((1, 1, 4, 2)), r.standard_normal((1, 1, 2, 3)), r.standard_normal((1, 1, 2, 3))
    wrong = sfda.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], -c["theta"], c["h0_re"], c["h0_im"], do, dr, di)
    assert rel(wrong["dtheta"], _central_differences(c, do, dr, di, "theta")) > 1e-3
