"""fp32 working matrices at d = 128: the fp32 path (every tile and matrix-core
operand in fp32) at the widths the bf16 path covers, against the fp64 oracle at
the fp32 tolerance; and the two precision options side by side on the full
Gated DeltaNet workloads -- the bf16 path and the fp32 path fed the exact fp32
copy of the same bf16 data (so both see identical inputs) -- with the fp32
option held to the fp32 tolerance on o, hT and every gradient."""
import pytest
import torch

from delta_rule_linear_gated_amd import workloads as W
from helpers import TOL, compare, gpu_run, oracle_run, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gate", ["none", "scalar"])
@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("policy", ["save", "recompute"])
def test_fp32_d128(gate, C, policy):
    w = W.custom(2, 3, 3 * C + 5, 128, 128, C, gate, "fp32", h0_std=0.5, seed=91)
    inp = W.make_inputs(w)
    compare(gpu_run(w, inp, policy), oracle_run(inp), TOL["fp32"], label=f"fp32 d=128 {gate} C={C} {policy}")


def test_fp32_d128_kaczmarz():
    w = W.custom(1, 4, 200, 128, 128, 64, "scalar", "fp32", h0_std=0.5, kla=True, seed=92)
    inp = W.make_inputs(w)
    compare(gpu_run(w, inp, "recompute"), oracle_run(inp, kaczmarz_eps=w.kaczmarz_eps), TOL["fp32"],
            label="fp32 d=128 Kaczmarz")


def _upcast(inp):
    return {n: (t.float() if t is not None and t.dtype == torch.bfloat16 else t) for n, t in inp.items()}


@pytest.mark.parametrize("name", ["gdn_bf16", "kla_gdn_bf16_32k"])
def test_working_precision_options_full_size(name):
    """Both precision options on the full workload, every head."""
    w = W.CONFIGS[name]
    say(f"[fp32-work] {w.describe()}")
    inp = W.make_inputs(w)
    ref = oracle_run(inp, kaczmarz_eps=w.kaczmarz_eps)
    e16 = compare(gpu_run(w, inp), ref, TOL["bf16"], label=f"{name} bf16 operands")
    e32 = compare(gpu_run(w, _upcast(inp)), ref, TOL["fp32"], label=f"{name} fp32 working matrices")
    say(f"[fp32-work] {name}: hT {e16['hT']:.2e} -> {e32['hT']:.2e}, dh0 {e16['dh0']:.2e} -> {e32['dh0']:.2e}, "
        f"dg {e16['dg']:.2e} -> {e32['dg']:.2e}")
