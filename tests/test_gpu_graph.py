"""The entry points under HIP graph capture: they allocate, free, synchronise
and memset nothing, so a captured forward + backward and a captured run of
decode calls replay exactly.  Every replay (with new inputs copied into the
captured buffers and eager work in between) is compared with eager calls."""
import pytest
import torch

from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W

pytestmark = pytest.mark.gpu


def _inputs(w, seed):
    return {n: (None if t is None else t.cuda()) for n, t in W.make_inputs(w, seed=seed).items()}


@pytest.mark.parametrize("policy", ["save", "recompute"])
def test_graph_fwd_bwd(policy):
    w = W.custom(2, 4, 300, 128, 128, 64, "scalar", "bf16", h0_std=0.5, seed=1)
    static = _inputs(w, 100)
    sh = B.shape_of(static["q"], static["v"], static["g"], 64)
    save = policy == "save"
    ws_f = B.workspace(sh, B.DN_PASS_FWD, "cuda")
    ws_b = B.workspace(sh, B.DN_PASS_BWD if save else B.DN_PASS_BWD_RECOMPUTE, "cuda")

    def step(d):
        o, hT, st = B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], C=64, save_states=save,
                                ws=ws_f)
        gr = B.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["do"], d["dhT"], st, C=64,
                         ws=ws_b)
        return {"o": o, "hT": hT, **gr}

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm up on a side stream before capture
        step(static)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step(static)
    for seed in (7, 8, 9):
        fresh = _inputs(w, seed)
        for n, t in fresh.items():
            if t is not None:
                static[n].copy_(t)
        g.replay()
        torch.cuda.synchronize()
        ref = step(fresh)        # eager, between replays
        torch.cuda.synchronize()
        for n, t in ref.items():
            if t is not None:
                assert torch.equal(out[n], t), (policy, seed, n)


def test_graph_decode_steps():
    """Eight decode calls (one token each, state in place) captured once."""
    w = W.custom(8, 16, 8, 128, 128, 64, "vector", "bf16", h0_std=0.5, seed=2)
    static = _inputs(w, 200)
    state = static["h0"].clone()

    def run(d, st):
        outs = []
        for t in range(8):
            sl = lambda x: None if x is None else x[:, :, t:t + 1].contiguous()
            outs.append(B.recurrent_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["beta"]), sl(d["g"]), st))
        return outs

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(static, state.clone())
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run(static, state)
    for seed in (3, 4):
        fresh = _inputs(w, seed)
        for n, t in fresh.items():
            if t is not None:
                static[n].copy_(t)
        state.copy_(fresh["h0"])
        g.replay()
        torch.cuda.synchronize()
        ref_state = fresh["h0"].clone()
        ref = run(fresh, ref_state)
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), seed
        assert torch.equal(state, ref_state), seed
