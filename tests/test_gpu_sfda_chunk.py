"""Parity of the chunkwise phase-controlled gate (dn_chunk_phase_fwd /
dn_chunk_phase_bwd; SFDA summary, chunk-WY form of the complex recurrence with
real inputs) with the fp64 oracle (oracle/sfda.py, the recurrence and its
reverse mode): o, the complex final state and every gradient (q, k, v, beta,
g, theta, the complex initial state) at nonzero phase, for every gate type, both
I/O types, d in {16, 32, 64, 128} and ragged sequences; strong decay; at zero phase
the chunkwise real path (KDA / GDN / DeltaNet); the recurrent phase entry point;
zero steps; the backward recomputing the states equals the one from the saved
buffer bitwise; sampled heads at the benchmark's full shape."""
import numpy as np
import pytest
import torch

from oracle import sfda
from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W
from helpers import TOL, rel_err, rel_err_heads, say

pytestmark = pytest.mark.gpu

CASES = [
    # gate, dtype, B, H, T, d
    ("vector", "fp32", 1, 2, 16 * 3 + 5, 64),
    ("vector", "bf16", 2, 2, 16 * 4 + 9, 64),
    ("scalar", "fp32", 2, 3, 16 * 2 + 1, 32),
    ("scalar", "bf16", 1, 2, 16 * 5, 64),
    ("none", "fp32", 1, 2, 37, 16),
    ("none", "bf16", 2, 1, 16 * 3 + 15, 32),
    ("vector", "fp32", 3, 1, 7, 32),
    ("vector", "bf16", 1, 1, 1, 16),
    ("vector", "fp32", 1, 2, 16 * 3 + 5, 128),
    ("scalar", "bf16", 2, 1, 16 * 2 + 11, 128),
    ("none", "fp32", 1, 1, 16 * 4, 128),
]


def _case(gate, dtype, Bn, H, T, d, seed):
    w = W.custom(Bn, H, T, d, d, 16, gate, dtype, h0_std=0.5, seed=seed, phase=True)
    return w, W.make_inputs(w)


def _gpu(inp):
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    o, hr, hi, st = B.chunk_phase_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], d["h0"], d["h0_im"])
    gr = B.chunk_phase_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], d["do"], d["dhT"], d["dhT_im"], st)
    torch.cuda.synchronize()
    out = {"o": o, "hT_re": hr, "hT_im": hi, **gr}
    return {n: (None if t is None else t.cpu().double().numpy()) for n, t in out.items()}


def _oracle(inp):
    f = {n: W.to_f64(t) for n, t in inp.items()}
    o, S = sfda.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["theta"], f["h0"], f["h0_im"])
    gr = sfda.backward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["theta"], f["h0"], f["h0_im"], f["do"],
                       f["dhT"], f["dhT_im"])
    return {"o": o, "hT_re": S.real, "hT_im": S.imag, **gr}


NAMES = ("o", "hT_re", "hT_im", "dq", "dk", "dv", "dbeta", "dg", "dtheta", "dh0_re", "dh0_im")


def _compare(gpu, ref, tol, label):
    errs = {}
    for n in NAMES:
        if ref.get(n) is None:
            assert gpu.get(n) is None, n
            continue
        assert np.isfinite(gpu[n]).all(), f"{label} {n} not finite"
        errs[n] = rel_err(gpu[n], ref[n])
        errs[n + " (per head)"] = rel_err_heads(gpu[n], ref[n])
    say(f"{label} errors: " + ", ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{label} over tolerance {tol}: {bad}"


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_chunk_phase_against_oracle(case):
    gate, dtype, Bn, H, T, d = case
    w, inp = _case(gate, dtype, Bn, H, T, d, seed=61 + T)
    _compare(_gpu(inp), _oracle(inp), TOL[dtype], f"phase {case}")


def test_chunk_phase_strong_decay():
    """g = -4 per step and channel with phases: the pairwise complex decays stay bounded."""
    w, inp = _case("vector", "fp32", 1, 2, 16 * 3 + 3, 32, seed=71)
    inp["g"].fill_(-4.0)
    _compare(_gpu(inp), _oracle(inp), TOL["fp32"], "phase g=-4")


@pytest.mark.parametrize("gate", ["none", "scalar", "vector"])
def test_zero_phase_is_the_real_chunkwise_path(gate):
    """theta = 0 and a real state: o, hT and the gradients of the real path (dh0_im
    and hT_im zero)."""
    w, inp = _case(gate, "fp32", 1, 2, 16 * 2 + 5, 32, seed=73)
    inp["theta"].zero_()
    inp["h0_im"] = None
    inp["dhT_im"] = None
    gpu = _gpu(inp)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    o, hT, st = B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], C=16)
    gr = B.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["do"], d["dhT"], st, C=16)
    real = {"o": o, "hT_re": hT, "dq": gr["dq"], "dk": gr["dk"], "dv": gr["dv"], "dbeta": gr["dbeta"],
            "dg": gr["dg"], "dh0_re": gr["dh0"]}
    for n, t in real.items():
        if t is None:
            assert gpu[n] is None
            continue
        e = rel_err(gpu[n], t.cpu().double().numpy())
        assert e <= 1e-5, (n, e)
    assert np.max(np.abs(gpu["hT_im"])) == 0.0 and np.max(np.abs(gpu["dh0_im"])) == 0.0


def test_chunkwise_equals_recurrent_phase_forward():
    w, inp = _case("vector", "fp32", 2, 2, 16 * 3 + 2, 64, seed=75)
    gpu = _gpu(inp)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    sr, si = d["h0"].clone(), d["h0_im"].clone()
    o = B.recurrent_phase_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], sr, si)
    torch.cuda.synchronize()
    assert rel_err(gpu["o"], o.cpu().double().numpy()) <= 1e-5
    assert rel_err(gpu["hT_re"], sr.cpu().double().numpy()) <= 1e-5
    assert rel_err(gpu["hT_im"], si.cpu().double().numpy()) <= 1e-5


def test_zero_steps_pass_the_state_through():
    w, inp = _case("scalar", "fp32", 1, 2, 0, 16, seed=77)
    gpu = _gpu(inp)
    assert np.array_equal(gpu["hT_re"], inp["h0"].double().numpy())
    assert np.array_equal(gpu["hT_im"], inp["h0_im"].double().numpy())
    assert np.array_equal(gpu["dh0_re"], inp["dhT"].double().numpy())
    assert np.array_equal(gpu["dh0_im"], inp["dhT_im"].double().numpy())


def test_forward_without_states_matches():
    """Without a saved buffer the per-chunk matrices go to the workspace: o and the
    final state are bitwise those of the saving forward."""
    w, inp = _case("vector", "bf16", 2, 2, 16 * 4 + 3, 64, seed=79)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    a = B.chunk_phase_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], d["h0"], d["h0_im"])
    b = B.chunk_phase_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], d["h0"], d["h0_im"],
                          save_states=False)
    torch.cuda.synchronize()
    assert b[3] is None
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


def _phase_sweep(n=16, seed=2027):
    import random
    rng = random.Random(seed)
    out = []
    for case in range(n):
        gate = rng.choice(["none", "scalar", "vector"])
        dtype = rng.choice(["bf16", "fp32"])
        d = rng.choice([16, 32, 64, 128])
        T = rng.choice([1, 15, 16, 17, 16 * 3 + 5, 16 * 9, rng.randint(1, 200)])
        Bn, H = rng.choice([(1, 1), (1, 3), (2, 2), (3, 1)])
        h0 = rng.choice([0.0, 0.5])
        out.append((gate, dtype, Bn, H, T, d, h0, 3000 + case))
    return out


@pytest.mark.parametrize("case", _phase_sweep(), ids=lambda c: "-".join(map(str, c[:6])))
def test_chunk_phase_random_shapes(case):
    """Seeded random shapes: gate, I/O type, d, length (one step, around one chunk,
    ragged, whole multiples, arbitrary), batch and heads, zero or random initial state."""
    gate, dtype, Bn, H, T, d, h0, seed = case
    w = W.custom(Bn, H, T, d, d, 16, gate, dtype, h0_std=h0, seed=seed, phase=True)
    inp = W.make_inputs(w)
    _compare(_gpu(inp), _oracle(inp), TOL[dtype], f"phase sweep {case}")


@pytest.mark.parametrize("gate,dtype,T,d", [("vector", "bf16", 16 * 5 + 3, 64), ("scalar", "fp32", 16 * 2 + 9, 128),
                                             ("none", "bf16", 16 * 3, 32), ("vector", "fp32", 1, 16)])
def test_backward_recomputing_the_states_matches(gate, dtype, T, d):
    """Without the saved buffer the backward reruns the forward's per-chunk products and
    state pass from h0 into its workspace: every gradient is bitwise the one from the
    saved states."""
    w, inp = _case(gate, dtype, 2, 2, T, d, seed=83 + T)
    x = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    o, hr, hi, st = B.chunk_phase_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["theta"], x["h0"], x["h0_im"])
    a = B.chunk_phase_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["theta"], x["do"], x["dhT"], x["dhT_im"], st)
    b = B.chunk_phase_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["theta"], x["do"], x["dhT"], x["dhT_im"], None,
                          h0_re=x["h0"], h0_im=x["h0_im"])
    torch.cuda.synchronize()
    for n in a:
        if a[n] is None:
            assert b[n] is None
            continue
        assert torch.equal(a[n], b[n]), n
    say(f"phase recompute {gate} {dtype} T={T} d={d}: bitwise equal")


def test_chunk_phase_full_size_sampled_heads():
    """The benchmark's shape and launch configuration (bench.py --phase-chunk on the KDA
    workload: B=4, H=16, T=8192, d=128, per-channel gate, bf16, saved states): o, the
    final state and every gradient of two sampled heads (the first and the last) against
    the oracle run on those heads alone (heads are independent)."""
    w0 = W.CONFIGS["kda_bf16"]
    w = W.custom(w0.B, w0.H, w0.T, w0.dk, w0.dk, 16, w0.gate, w0.dtype, h0_std=0.5, seed=w0.seed, phase=True)
    say(f"[phase full size] {w.describe()}")
    inp = W.make_inputs(w)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    o, hr, hi, st = B.chunk_phase_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], d["h0"], d["h0_im"])
    gr = B.chunk_phase_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], d["do"], d["dhT"], d["dhT_im"], st)
    torch.cuda.synchronize()
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    out = {"o": o, "hT_re": hr, "hT_im": hi, **gr}
    gpu = {n: W.to_f64(t, heads) for n, t in out.items()}
    del d, st, out, gr
    f = {n: W.to_f64(t, heads) for n, t in inp.items()}
    ob, S = sfda.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["theta"], f["h0"], f["h0_im"])
    ref = {"o": ob, "hT_re": S.real, "hT_im": S.imag,
           **sfda.backward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["theta"], f["h0"], f["h0_im"], f["do"],
                           f["dhT"], f["dhT_im"])}
    _compare(gpu, ref, TOL[w.dtype], f"phase full size, heads {heads}")
