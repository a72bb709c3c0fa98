"""Seeded synthetic workloads for the chunkwise gated delta rule.

This module only draws and rounds inputs; it holds none of the operator's
arithmetic.  Both the HIP path and the fp64 oracle are fed from it: the oracle
receives the already-rounded values (exactly upcast to fp64), so a parity gap
measures kernel error, not input quantisation.

Distributions (per head, per step):
  q, k  ~ N(0, 1), then L2-normalised per token (fp64), then rounded
  v     ~ N(0, 1)
  beta  = sigmoid(N(0, 1))                           fp32
  g     = -softplus(N(0, 1)) / 16                    fp32 log-decay, scalar [B,H,T]
                                                     or per channel [B,H,T,dk]
  h0    = h0_std * N(0, 1)  (None when h0_std == 0)  fp32 [B,H,dv,dk]
  dO    ~ N(0, 1) in the I/O dtype; dhT ~ N(0, 1) fp32
  theta = 0.5 N(0, 1) fp32 [B,H,T,dk], h0_im like h0 and dhT_im like dhT
                                                     (phase-controlled gate only)
The long-context workload uses the Kaczmarz step of the KLA abstract: keys are
left unnormalised and the step input is eta = sigmoid(N(0, 1)) (fp32, returned
under "beta"), which the operator turns into beta_t = eta_t / (||k_t||^2 + eps)
with eps = ``Workload.kaczmarz_eps`` (1e-6 unless a custom workload sets it).

Rounding: fp64 -> fp32 (round to nearest), then fp32 -> bf16 (round to nearest
even) for bf16 workloads.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

GATES = ("none", "scalar", "vector")
DTYPES = ("fp32", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    C: int
    gate: str = "scalar"
    dtype: str = "bf16"
    h0_std: float = 0.0
    kla: bool = False
    policy: str = "save"          # "save": forward keeps per-chunk states; "recompute"
    seed: int = 1
    kz_eps: float = 1e-6          # eps of the Kaczmarz step (kla workloads)
    phase: bool = False           # phase-controlled gate: draw theta (and an imaginary h0)

    @property
    def kaczmarz_eps(self):
        """eps of the Kaczmarz step (its "beta" input is then eta), else None."""
        return self.kz_eps if self.kla else None

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.T

    def describe(self) -> str:
        return (f"{self.name}: gate={self.gate} dtype={self.dtype} B={self.B} H={self.H} "
                f"T={self.T} dk={self.dk} dv={self.dv} C={self.C} policy={self.policy}")


# The five workloads of the operator: DeltaNet, GDN fp32, GDN bf16 (headline),
# KDA (per-channel gate), and long-context KLA-GDN with state recomputation.
CONFIGS = {
    "deltanet_fp32": Workload("deltanet_fp32", 1, 1, 64, 16, 16, 16, "none", "fp32", 0.0, False,
                              "save", 1),
    "gdn_fp32": Workload("gdn_fp32", 2, 4, 1024, 64, 64, 64, "scalar", "fp32", 0.1, False,
                         "save", 2),
    "gdn_bf16": Workload("gdn_bf16", 8, 16, 4096, 128, 128, 64, "scalar", "bf16", 0.0, False,
                         "save", 3),
    "kda_bf16": Workload("kda_bf16", 4, 16, 8192, 128, 128, 64, "vector", "bf16", 0.0, False,
                         "save", 4),
    "kla_gdn_bf16_32k": Workload("kla_gdn_bf16_32k", 1, 32, 32768, 128, 128, 64, "scalar",
                                 "bf16", 0.0, True, "recompute", 5),
}
CONFIG_ORDER = ["deltanet_fp32", "gdn_fp32", "gdn_bf16", "kda_bf16", "kla_gdn_bf16_32k"]
# Few heads, long sequence (one sequence of a 4-head layer): the sequential state
# passes alone would occupy 32 compute units, so the chunk-parallel scan runs.
EXTRA = {
    "gdn_bf16_4h_32k": Workload("gdn_bf16_4h_32k", 1, 4, 32768, 128, 128, 64, "scalar", "bf16", 0.5, False,
                                "save", 6),
}
CONFIGS.update(EXTRA)
HEADLINE = "gdn_bf16"


def torch_dtype(dtype: str):
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _rng(seed: int, stream: int):
    return np.random.default_rng([int(seed), int(stream)])


def _l2norm(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-30)


def _round(x64: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x64.astype(np.float32)))
    return t.to(torch_dtype(dtype)).contiguous()


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def make_inputs(w: Workload, seed: int | None = None, cotangents: bool = True,
                device: str | torch.device = "cpu") -> dict:
    """Draw one batch of inputs for workload ``w``.

    Returns a dict of torch tensors (on ``device``): q, k, v (I/O dtype), beta
    (eta when ``w.kaczmarz_eps`` is set),
    g (None / [B,H,T] / [B,H,T,dk]), h0 (None or [B,H,dv,dk]) in fp32, and, when
    ``cotangents``, do (I/O dtype) and dhT (fp32).  Every tensor has its own
    random stream, so a workload is reproducible tensor by tensor."""
    s = w.seed if seed is None else seed
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    out = {}
    q = _l2norm(_rng(s, 0).standard_normal((B, H, T, dk)))
    out["q"] = _round(q, w.dtype)
    del q
    k = _rng(s, 1).standard_normal((B, H, T, dk))
    if not w.kla:
        k = _l2norm(k)
    out["k"] = _round(k, w.dtype)
    del k
    out["v"] = _round(_rng(s, 2).standard_normal((B, H, T, dv)), w.dtype)
    # beta, or eta for the Kaczmarz step (same distribution)
    out["beta"] = _round(_sigmoid(_rng(s, 3).standard_normal((B, H, T))), "fp32")
    if w.gate == "none":
        out["g"] = None
    elif w.gate == "scalar":
        out["g"] = _round(-_softplus(_rng(s, 4).standard_normal((B, H, T))) / 16.0, "fp32")
    elif w.gate == "vector":
        out["g"] = _round(-_softplus(_rng(s, 4).standard_normal((B, H, T, dk))) / 16.0, "fp32")
    else:
        raise ValueError(w.gate)
    if w.h0_std > 0:
        out["h0"] = _round(w.h0_std * _rng(s, 5).standard_normal((B, H, dv, dk)), "fp32")
    else:
        out["h0"] = None
    if w.phase:   # phases in radians, per step and key channel; the state's imaginary part
        out["theta"] = _round(0.5 * _rng(s, 8).standard_normal((B, H, T, dk)), "fp32")
        out["h0_im"] = _round(w.h0_std * _rng(s, 9).standard_normal((B, H, dv, dk)), "fp32") \
            if w.h0_std > 0 else None
    if cotangents:
        out["do"] = _round(_rng(s + 100, 6).standard_normal((B, H, T, dv)), w.dtype)
        out["dhT"] = _round(_rng(s + 100, 7).standard_normal((B, H, dv, dk)), "fp32")
        if w.phase:   # cotangent of the final state's imaginary part
            out["dhT_im"] = _round(_rng(s + 100, 10).standard_normal((B, H, dv, dk)), "fp32")
    if str(device) != "cpu":
        out = {n: (None if t is None else t.to(device)) for n, t in out.items()}
    return out


def custom(B, H, T, dk, dv, C, gate="scalar", dtype="bf16", h0_std=0.0, kla=False,
           policy="save", seed=7, name="custom", kz_eps=1e-6, phase=False) -> Workload:
    """A workload of any shape, with the same distributions."""
    return Workload(name, B, H, T, dk, dv, C, gate, dtype, h0_std, kla, policy, seed, kz_eps, phase)


def to_f64(t, heads=None) -> np.ndarray | None:
    """Exact fp64 copy of a (rounded) tensor; ``heads`` selects [(b, h), ...]."""
    if t is None:
        return None
    t = t.detach()
    if heads is not None:
        t = torch.stack([t[b, h] for b, h in heads])[None]
    return t.to("cpu", torch.float64).numpy()
