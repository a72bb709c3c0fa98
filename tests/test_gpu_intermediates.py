"""Parity of the per-chunk intermediates the HIP path leaves in the forward's
saved buffer (cumulative log-decay, (I + A)^{-1}, intra-chunk scores, U, chunk-entry
states) and in the backward's workspace (the triangular-residual adjoint lambda
and the state cotangent per chunk) with the fp64 chunked evaluation of the
oracle.  A mismatch here names the stage that
is wrong when an end-to-end parity test fails."""
import numpy as np
import pytest
import torch

from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W
from helpers import rel_err, say
from oracle import chunked

pytestmark = pytest.mark.gpu

CASES = [
    ("scalar", "fp32", 70, 32, 32, 1e-4),
    ("vector", "fp32", 70, 32, 32, 1e-4),
    ("scalar", "bf16", 150, 128, 64, 2e-2),
    ("vector", "bf16", 150, 128, 64, 2e-2),
    ("none", "bf16", 100, 64, 64, 2e-2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:5])))
def test_workspace_intermediates(case):
    gate, dtype, T, d, C, tol = case
    w = W.custom(1, 2, T, d, d, C, gate, dtype, h0_std=0.5, seed=23)
    say(f"[intermediates] {w.describe()}")
    inp = W.make_inputs(w)
    dev = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    sh = B.shape_of(dev["q"], dev["v"], dev["g"], C)
    o, hT, states = B.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["h0"], C=C)
    ws = B.workspace(sh, B.DN_PASS_BWD, "cuda")
    B.chunk_bwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["h0"], dev["do"], dev["dhT"],
                states, C=C, ws=ws)
    torch.cuda.synchronize()
    lay = B.dn_workspace_layout(sh, B.DN_PASS_BWD)
    wsb = ws.cpu()
    NT = -(-T // C)
    et = torch.float32 if dtype == "fp32" else torch.bfloat16

    def region(off, count, dt):
        nbytes = count * torch.tensor([], dtype=dt).element_size()
        return wsb[off:off + nbytes].view(dt).to(torch.float64).numpy()

    gw = d if gate == "vector" else 1
    for h in range(2):
        f = {n: W.to_f64(t)[0, h] if t is not None else None for n, t in inp.items()}
        tr = []
        chunked.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"], C=C, trace=tr)
        trb = {}
        chunked.backward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"], f["do"], f["dhT"], C=C,
                         trace=trb)
        _, _, st_ref = chunked.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"], C=C)
        sv = B.saved_regions(states, sh)
        if gate != "none":
            gam = sv["gam"][0, h].cpu().to(torch.float64).numpy().reshape(T, gw)
            ref = np.concatenate([c["gam"] if gate == "vector" else c["gam"][:, :1] for c in tr])
            say(f"  head {h} gam err {rel_err(gam, ref):.2e}")
            assert rel_err(gam, ref) < 1e-5
        # T and P as the forward saved them (row-major), lambda and dS1 from the backward's workspace
        Tm = sv["T"][0, h].cpu().to(torch.float64).numpy()
        Pm = sv["P"][0, h].cpu().to(torch.float64).numpy()
        Um = sv["U"][0, h].cpu().to(torch.float64).numpy()
        lam = region(lay["lam"], 2 * NT * C * d, et).reshape(2, NT, C, d)[h]
        dS1 = region(lay["dS1"], 2 * NT * d * d, et).reshape(2, NT, d, d)[h]
        st = sv["states"][0, h].cpu().to(torch.float64).numpy()
        for n in range(NT):
            L = tr[n]["T"].shape[0]
            errs = dict(T=rel_err(Tm[n, :L, :L], tr[n]["T"]), P=rel_err(Pm[n, :L, :L], tr[n]["Pm"]),
                        U=rel_err(Um[n, :L], tr[n]["U"]), S0=rel_err(st[n], st_ref[n]), lam=rel_err(lam[n, :L], trb["lam"][n]),
                        dS1=rel_err(dS1[n], trb["dS1"][n]))
            say(f"  head {h} chunk {n}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
            bad = {k: v for k, v in errs.items() if not v <= tol}
            assert not bad, (h, n, bad)
            assert not Um[n, L:].any(), (h, n, "U rows past the sequence")
