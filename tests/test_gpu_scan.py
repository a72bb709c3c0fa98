"""The chunk-parallel scan of the state passes (exact affine chunk transfer,
SFDA summary): shapes with few heads and at least 16 chunks take it (the plan is
pinned in test_abi.py).  Parity with the fp64 oracle for every gate, both I/O
types, ragged last segments and chunks, both state policies, nonzero h0 / dhT
and the Kaczmarz step; agreement with the sequential pass (DN_FLAG_NO_SCAN) on
the same inputs, outputs and saved chunk states; and a full-size few-head
workload."""
import pytest
import torch

from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W
from helpers import TOL, compare, gpu_run, oracle_run, rel_err, say

pytestmark = pytest.mark.gpu

CASES = [
    # gate, dtype, B, H, T, d, C, kla       segments (test_abi's rule)
    ("scalar", "bf16", 1, 2, 40 * 64 + 37, 128, 64, False),   # 41 chunks -> 9 segments of 5, ragged
    ("vector", "bf16", 1, 1, 40 * 32, 64, 32, False),         # 40 chunks -> 10 segments of 4
    ("none", "bf16", 1, 2, 48 * 64 + 1, 128, 64, False),      # 49 chunks -> 10 segments of 5
    ("scalar", "fp32", 2, 2, 2048 + 77, 64, 64, False),       # 34 chunks -> 7 segments of 5
    ("vector", "fp32", 1, 1, 36 * 16 + 9, 32, 16, False),     # 37 chunks -> 8 segments of 5
    ("none", "fp32", 1, 2, 40 * 16 + 3, 32, 16, False),       # 41 chunks -> 9 segments of 5
    ("scalar", "bf16", 1, 2, 2000, 128, 64, True),            # Kaczmarz step, 32 chunks -> 8 of 4
]


def _uses_scan(w, no_scan=False):
    sh = B.make_shape(w.B, w.H, w.T, w.dk, w.dv, w.C, w.dtype, w.gate, w.kaczmarz_eps, no_scan)
    lay = B.dn_workspace_layout(sh, B.DN_PASS_FWD)
    return lay["total"] > lay["seg_end"]


def _w(case, seed):
    gate, dtype, Bn, H, T, d, C, kla = case
    return W.custom(Bn, H, T, d, d, C, gate, dtype, h0_std=0.5, kla=kla, seed=seed)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("policy", ["save", "recompute"])
def test_scan_matches_oracle(case, policy):
    w = _w(case, 70 + case[4] % 97)
    say(f"[scan] {w.describe()} policy={policy}")
    assert _uses_scan(w)
    inp = W.make_inputs(w)
    compare(gpu_run(w, inp, policy), oracle_run(inp, kaczmarz_eps=w.kaczmarz_eps), TOL[w.dtype],
            label=f"{case} {policy}")


@pytest.mark.parametrize("gate,dtype", [("scalar", "bf16"), ("vector", "bf16"), ("scalar", "fp32")])
def test_scan_agrees_with_the_sequential_pass(gate, dtype):
    d = 128 if dtype == "bf16" else 64
    w = W.custom(1, 2, 40 * 64 + 17, d, d, 64, gate, dtype, h0_std=0.5, seed=5)
    assert _uses_scan(w) and not _uses_scan(w, no_scan=True)
    inp = W.make_inputs(w)
    dev = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    out = {}
    for no_scan in (False, True):
        o, hT, st = B.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["h0"], C=64,
                                no_scan=no_scan)
        gr = B.chunk_bwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["h0"], dev["do"], dev["dhT"],
                         st, C=64, no_scan=no_scan)
        sv = B.saved_regions(st, B.shape_of(dev["q"], dev["v"], dev["g"], 64, no_scan=no_scan))
        out[no_scan] = {"o": o, "hT": hT, "states": sv["states"], **gr}
    torch.cuda.synchronize()
    tol = TOL[dtype]
    for n, x in out[False].items():
        if x is None:
            continue
        e = rel_err(x.double().cpu().numpy(), out[True][n].double().cpu().numpy())
        say(f"  scan vs sequential {n}: {e:.2e}")
        assert e <= tol, n


def test_scan_full_size_few_heads():
    w = W.CONFIGS["gdn_bf16_4h_32k"]
    say(f"[scan] {w.describe()}")
    assert _uses_scan(w)
    inp = W.make_inputs(w)
    compare(gpu_run(w, inp), oracle_run(inp), TOL[w.dtype], label=w.name)
