"""Shared helpers of the parity tests: run the HIP path through the C ABI and the
fp64 oracle on the same rounded inputs, and compare them."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W

# Tolerances of the parity bar: max |gpu - oracle| / max |oracle| per tensor.
TOL = {"fp32": 1e-4, "bf16": 2e-2}
OUTPUTS = ("o", "hT", "dq", "dk", "dv", "dbeta", "dg", "dh0")


def nthreads():
    return max(1, min(16, os.cpu_count() or 1))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def rel_err_heads(x, ref, floor_frac=1e-2):
    """Worst over the (b, h) heads of max |x - ref| / max |ref| within the head, so a
    local error in a low-magnitude head is not hidden under another head's maximum
    (a head's maximum is floored at floor_frac of the largest head's, so a head that
    is zero up to rounding does not divide by its own noise)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.ndim < 3 or ref.size == 0:
        return rel_err(x, ref)
    nh = ref.shape[0] * ref.shape[1]
    d = np.abs(x - ref).reshape(nh, -1).max(axis=1)
    m = np.abs(ref).reshape(nh, -1).max(axis=1)
    if m.max() == 0:
        return float(d.max())
    return float((d / np.maximum(m, floor_frac * m.max())).max())


def gpu_run(w: W.Workload, inp: dict, policy: str | None = None, dhT=True):
    """fwd + bwd on the GPU through the C ABI (with the Kaczmarz flag when the
    workload has one: inp["beta"] is then eta).  Returns a dict of CPU tensors."""
    policy = policy or w.policy
    kz = w.kaczmarz_eps
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    o, hT, states = B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], C=w.C,
                                save_states=(policy == "save"), kaczmarz_eps=kz)
    gr = B.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["do"],
                     d["dhT"] if dhT else None, states, C=w.C, kaczmarz_eps=kz)
    torch.cuda.synchronize()
    out = {"o": o, "hT": hT, **gr}
    if states is not None:   # the saved buffer's regions (not its alignment gaps)
        sv = B.saved_regions(states, B.shape_of(d["q"], d["v"], d["g"], w.C, kz))
        out.update({"states": sv["states"], "saved_T": sv["T"], "saved_P": sv["P"], "saved_gam": sv["gam"],
                    "saved_kz_beta": sv["kz_beta"], "saved_kz_rn": sv["kz_rn"]})
    return {n: (None if t is None else t.cpu()) for n, t in out.items()}


def oracle_run(inp: dict, heads=None, dhT=True, kaczmarz_eps=None, backward=True):
    """fp64 oracle on the same rounded inputs (optionally only some (b, h) heads).
    With ``kaczmarz_eps``, inp["beta"] is eta and "dbeta" holds d eta;
    ``backward=False`` returns o and hT only."""
    f = {n: W.to_f64(t, heads) for n, t in inp.items()}
    args = (f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"])
    dh = f.get("dhT") if dhT else None
    gr = {}
    if kaczmarz_eps is None:
        o, hT = oracle.forward(*args, nthreads=nthreads())
        if backward:
            gr = oracle.backward(*args, f["do"], dh, nthreads=nthreads())
    else:
        o, hT = oracle.kaczmarz_forward(*args, eps=kaczmarz_eps, nthreads=nthreads())
        if backward:
            gr = oracle.kaczmarz_backward(*args, f["do"], dh, eps=kaczmarz_eps, nthreads=nthreads())
            gr["dbeta"] = gr.pop("deta")
    return {"o": o, "hT": hT, **gr}


def select(t, heads):
    if t is None or heads is None:
        return t
    return torch.stack([t[b, h] for b, h in heads])[None]


def compare(gpu: dict, ref: dict, tol: float, heads=None, label=""):
    """Every output within ``tol`` of the oracle, normalised over the whole tensor and
    per head (rel_err_heads)."""
    errs, herrs = {}, {}
    for n in OUTPUTS:
        if ref.get(n) is None:
            assert gpu.get(n) is None, n
            continue
        x = select(gpu[n], heads)
        assert torch.isfinite(x.float()).all(), f"{label} {n} has non-finite values"
        xn = x.to(torch.float64).numpy()
        errs[n] = rel_err(xn, ref[n])
        herrs[n] = rel_err_heads(xn, ref[n])
    say(f"{label} errors: " + ", ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    say(f"{label} worst head: " + ", ".join(f"{n}={e:.2e}" for n, e in herrs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    bad.update({f"{n} (per head)": e for n, e in herrs.items() if not e <= tol})
    assert not bad, f"{label} over tolerance {tol}: {bad}"
    return errs
