"""Edge and degenerate cases of the chunkwise path against the fp64 oracle:
beta = 0 (pure decay; dbeta is still non-zero), keys that are exactly zero,
a single token, the largest head count (B * H = 65535), strong per-channel
decay (up to -5 per step and channel, the C x C products' factors reaching
e^{+80} on a 16-row block), and a NaN confined to the head it was put in."""
import numpy as np
import pytest
import torch

from delta_rule_linear_gated_amd import workloads as W
from helpers import TOL, compare, gpu_run, oracle_run, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_zero_beta(gate):
    w = W.custom(1, 2, 150, 128, 128, 64, gate, "bf16", h0_std=0.5, seed=81)
    inp = W.make_inputs(w)
    inp["beta"].zero_()
    compare(gpu_run(w, inp), oracle_run(inp), TOL["bf16"], label=f"beta=0 {gate}")


def test_zero_keys():
    w = W.custom(1, 2, 150, 64, 64, 32, "vector", "fp32", h0_std=0.5, seed=82)
    inp = W.make_inputs(w)
    inp["k"][:, :, 10:40] = 0   # a run of tokens that neither erase nor write
    inp["k"][:, :, 97] = 0
    compare(gpu_run(w, inp), oracle_run(inp), TOL["fp32"], label="zero keys")


@pytest.mark.parametrize("gate", ["none", "scalar", "vector"])
@pytest.mark.parametrize("policy", ["save", "recompute"])
def test_single_token(gate, policy):
    w = W.custom(2, 3, 1, 128, 128, 64, gate, "bf16", h0_std=0.5, seed=83)
    inp = W.make_inputs(w)
    compare(gpu_run(w, inp, policy), oracle_run(inp), TOL["bf16"], label=f"T=1 {gate} {policy}")


def test_largest_head_count():
    """B * H = 65535, the ABI's limit (grid dimension); the oracle on sampled heads."""
    w = W.custom(5, 13107, 40, 16, 16, 16, "scalar", "fp32", h0_std=0.5, seed=84)
    say(f"[edges] {w.describe()}")
    inp = W.make_inputs(w)
    gpu = gpu_run(w, inp)
    r = np.random.default_rng(3)
    heads = [(0, 0), (4, 13106)] + [(int(b), int(h)) for b, h in zip(r.integers(0, 5, 30), r.integers(0, 13107, 30))]
    compare(gpu, oracle_run(inp, heads=heads), TOL["fp32"], heads=heads, label="B*H=65535")


def test_strong_vector_decay():
    """g = -2 per step and channel: gam_C = -128 over a chunk of 64."""
    w = W.custom(1, 2, 130, 128, 128, 64, "vector", "bf16", h0_std=0.5, seed=85)
    inp = W.make_inputs(w)
    inp["g"].fill_(-2.0)
    gpu = gpu_run(w, inp)
    for n in ("o", "hT", "dq", "dk", "dv", "dbeta", "dg", "dh0"):
        assert torch.isfinite(gpu[n].float()).all(), n
    compare(gpu, oracle_run(inp), TOL["bf16"], label="g=-2 vector")


def test_nan_stays_in_its_head():
    w = W.custom(1, 4, 100, 64, 64, 32, "scalar", "bf16", h0_std=0.5, seed=86)
    inp = W.make_inputs(w)
    clean = gpu_run(w, inp)
    inp["q"][0, 1, 37, 5] = float("nan")
    dirty = gpu_run(w, inp)
    assert torch.isnan(dirty["o"][0, 1].float()).any()
    for n in ("o", "hT", "dq", "dk", "dv", "dbeta", "dg", "dh0"):
        for h in (0, 2, 3):
            assert torch.equal(dirty[n][0, h], clean[n][0, h]), (n, h)


@pytest.mark.parametrize("dtype,d,C", [("bf16", 128, 64), ("bf16", 64, 32), ("fp32", 64, 32)])
@pytest.mark.parametrize("policy", ["save", "recompute"])
def test_vector_decay_four_per_step(dtype, d, C, policy):
    """g = -4 per step and channel: gam_C = -256 over a chunk of 64 (a factor
    e^{128} if the chunk's pairs were split at its centre); split at 16-row block
    boundaries no factor exceeds e^{64}."""
    w = W.custom(1, 2, 3 * C + 7, d, d, C, "vector", dtype, h0_std=0.5, seed=87)
    inp = W.make_inputs(w)
    inp["g"].fill_(-4.0)
    gpu = gpu_run(w, inp, policy)
    for n in ("o", "hT", "dq", "dk", "dv", "dbeta", "dg", "dh0"):
        assert torch.isfinite(gpu[n].float()).all(), n
    compare(gpu, oracle_run(inp), TOL[dtype], label=f"g=-4 vector {dtype} d={d} C={C} {policy}")


def test_vector_decay_mixed_strengths():
    """Per-step, per-channel decays drawn from -U(0, 5): channels that forget within
    a few steps beside ones that keep their state, in every chunk."""
    w = W.custom(2, 2, 300, 128, 128, 64, "vector", "bf16", h0_std=0.5, seed=88)
    inp = W.make_inputs(w)
    r = np.random.default_rng(88)
    inp["g"].copy_(torch.from_numpy(-5.0 * r.random(tuple(inp["g"].shape))).float())
    gpu = gpu_run(w, inp)
    for n in ("o", "hT", "dq", "dk", "dv", "dbeta", "dg", "dh0"):
        assert torch.isfinite(gpu[n].float()).all(), n
    compare(gpu, oracle_run(inp), TOL["bf16"], label="g ~ -U(0,5) vector")
