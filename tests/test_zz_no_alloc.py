"""dn_chunk_fwd_noalloc: the forward without saved states whose scratch is the
library's per-device array instead of a caller workspace.  Checked against
dn_chunk_fwd (states NULL, caller workspace) on the same inputs -- the same
kernels, so bitwise equal -- on two calls in a row, the second smaller, and
against the fp64 oracle within the parity tolerance."""
from __future__ import annotations

import pytest
import torch

from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W

from helpers import TOL, oracle_run, rel_err, say


def test_noalloc_rejects_shapes_beyond_its_scratch():
    # rejected on the host before any HIP call (the pointers are never touched)
    sh = B.make_shape(8, 16, 4096, 128, 128, 64, "bf16", "scalar")
    need = B.dn_workspace_bytes(sh, B.DN_PASS_FWD)
    assert need > B.DN_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    st = B.dn_chunk_fwd_noalloc(sh, fake, fake, fake, fake, fake, None, fake, None, 0)
    assert st == B.DN_ERR_WORKSPACE
    assert "scratch" in B.dn_last_error()
    # a bad shape is reported as such
    bad = B.make_shape(1, 1, 64, 48, 48, 64, "bf16", "scalar")
    assert B.dn_chunk_fwd_noalloc(bad, fake, fake, fake, fake, fake, None, fake, None, 0) == B.DN_ERR_UNSUPPORTED


def _run_both(w, kz=None):
    inp = W.make_inputs(w, cotangents=False)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    sh = B.shape_of(d["q"], d["v"], d["g"], w.C, kz)
    need = B.dn_workspace_bytes(sh, B.DN_PASS_FWD)
    assert 0 < need <= B.DN_NOALLOC_SCRATCH_BYTES
    o1, hT1 = torch.empty_like(d["v"]), torch.empty(w.B, w.H, w.dv, w.dk, device="cuda")
    o2, hT2 = torch.full_like(d["v"], float("nan")), torch.full_like(hT1, float("nan"))
    ws = B.workspace(sh, B.DN_PASS_FWD, "cuda")
    say(f"noalloc case {w.describe()} scratch {need} bytes")
    B._check(B.dn_chunk_fwd(sh, d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], o1, hT1, None, ws,
                            ws.numel()))
    B._check(B.dn_chunk_fwd_noalloc(sh, d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], o2, hT2))
    torch.cuda.synchronize()
    return inp, (o1, hT1), (o2, hT2)


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_forward_on_consecutive_calls():
    cases = [
        # few heads and a long sequence: the scan's segment buffers live in the scratch too
        (W.custom(1, 2, 4100, 64, 64, 64, "vector", "bf16", h0_std=0.5, seed=71), None),
        # then a smaller call, scalar gate with the Kaczmarz step, reusing the array
        (W.custom(2, 3, 300, 128, 128, 64, "scalar", "bf16", h0_std=0.5, kla=True, seed=72), 1e-6),
        # and a smaller one still, fp32, no gate
        (W.custom(1, 2, 70, 32, 32, 16, "none", "fp32", h0_std=0.5, seed=73), None),
    ]
    for w, kz in cases:
        if kz is not None:
            w = W.custom(w.B, w.H, w.T, w.dk, w.dv, w.C, w.gate, w.dtype, h0_std=w.h0_std, kla=True,
                         seed=w.seed, kz_eps=kz)
        inp, (o1, hT1), (o2, hT2) = _run_both(w, w.kaczmarz_eps)
        assert torch.equal(o1, o2), "o differs from dn_chunk_fwd"
        assert torch.equal(hT1, hT2), "hT differs from dn_chunk_fwd"
        ref = oracle_run(inp, dhT=False, kaczmarz_eps=w.kaczmarz_eps, backward=False)
        eo = rel_err(o2.cpu().double().numpy(), ref["o"])
        eh = rel_err(hT2.cpu().double().numpy(), ref["hT"])
        say(f"  o {eo:.2e} hT {eh:.2e}")
        assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]
