"""Parity of the HIP path with the fp64 oracle over seeded random shapes: gate,
I/O type, d, chunk size, sequence length (1, 2, around one chunk, ragged and
whole multiples, arbitrary), batch and heads, state policy, the Kaczmarz step
and h0, drawn from a fixed seed so that every run checks the same cases."""
import random

import pytest
import torch

from delta_rule_linear_gated_amd import workloads as W
from helpers import OUTPUTS, TOL, gpu_run, oracle_run, rel_err, say

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2026):
    rng = random.Random(seed)
    out = []
    for case in range(n):
        gate = rng.choice(["none", "scalar", "vector"])
        dtype = rng.choice(["bf16", "bf16", "fp32"])
        d = rng.choice([16, 32, 64, 128] if dtype == "bf16" else [16, 32, 64])
        C = rng.choice([16, 32, 64])
        if dtype == "fp32" and d == 64 and gate == "vector" and C == 64:
            C = 32   # the one fp32 shape whose backward tiles do not fit at C = 64
        T = rng.choice([1, 2, C - 1, C, C + 1, 3 * C + 5, 7 * C, rng.randint(1, 400)])
        B, H = rng.choice([(1, 1), (1, 3), (2, 2), (3, 1)])
        policy = rng.choice(["save", "recompute"])
        kla = gate == "scalar" and dtype == "bf16" and rng.random() < 0.3
        h0 = rng.choice([0.0, 0.1])
        out.append(W.custom(B, H, T, d, d, C, gate, dtype, h0_std=h0, kla=kla, policy=policy,
                            seed=1000 + case, name=f"sweep{case}"))
    return out


@pytest.mark.parametrize("w", _cases(), ids=lambda w: w.name)
def test_random_shape(w):
    say(f"[sweep] {w.describe()} kaczmarz={w.kaczmarz_eps is not None}")
    inp = W.make_inputs(w, cotangents=True)
    gpu = gpu_run(w, inp)
    ref = oracle_run(inp, kaczmarz_eps=w.kaczmarz_eps)
    errs = {n: rel_err(gpu[n].to(torch.float64).numpy(), ref[n]) for n in OUTPUTS if ref.get(n) is not None}
    say(f"[sweep] {w.name} errors: " + ", ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL[w.dtype]}
    assert not bad, f"{w.name} over tolerance {TOL[w.dtype]}: {bad}"
