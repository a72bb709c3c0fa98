#!/usr/bin/env python3
"""Throughput of the chunkwise gated delta rule on one MI355X.

One step = one forward (dn_chunk_fwd) + one ReWY backward (dn_chunk_bwd) over
one batch of synthetic input already resident in HBM, through the C ABI.
Default workload: Gated DeltaNet, bf16 q/k/v/dO with fp32 gate / beta / state,
B=8, H=16, T=4096, d_k=d_v=128, chunk 64, states saved by the forward.

Prints ONE JSON line: tokens/s (B*T per second, all heads), algorithmic
TFLOP/s and its fraction of the bf16 dense MFMA peak, the roofline of the
dominant kernel (algorithmic bytes per launch / average launch time from HIP
events recorded around each launch on the launch stream), the recomputation
policy's step time, and the fp64 CPU oracle timed on the host.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--policy save|recompute]
                    [--no-cpu-baseline] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd tokens/s and TFLOP/s (% MFMA peak), GDN bf16 T=4096 d=128, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def algorithmic_flops_per_token_head(C: int, dk: int, dv: int) -> float:
    """Flops the method must do per token and head, causal C x C products counted
    as triangles, recomputation excluded: forward 2C(dk+dv) + 6 dk dv + C^2/3,
    backward 4C(dk+dv) + 12 dk dv."""
    return (2 * C * (dk + dv) + 6 * dk * dv + C * C / 3) + (4 * C * (dk + dv) + 12 * dk * dv)


def kernel_budget(name: str, C: int, d: int, E: int, gw: int, saved: bool, kz: bool = False):
    """Algorithmic (flops, HBM bytes) of one kernel per chunk and head: the
    contractions it performs (triangles halved) and the tensors it must read and
    write once.  E = bytes per I/O element, gw = gate values per step, kz = the
    Kaczmarz step (prep writes beta and 1 / (||k||^2 + eps), bwd_chunk reads the latter)."""
    sc = C * 4 * (1 + gw)                     # beta + gate (or d gam) per chunk, fp32
    if name in ("prep", "prep_recompute"):
        fl = 2 * (C * (C - 1) / 2 * d + C * (C + 1) / 2 * d) + C ** 3 / 3 + (2 * C * d if kz else 0)
        by = 2 * C * d * E + sc + C * gw * 4 + 2 * C * C * E + (2 * C * 4 if kz else 0)
    elif name in ("fwd_state", "fwd_state_recompute"):
        fl = 2 * (3 * C * d * d + C * C * d)
        by = (3 if name == "fwd_state" else 2) * C * d * E + 2 * C * C * E + sc
        by += (C * d * E if name == "fwd_state" else 0) + (d * d * E if (saved or name != "fwd_state") else 0)
    elif name == "bwd_state":
        fl = 2 * (3 * C * d * d + C * C * d)
        by = 3 * C * d * E + 2 * C * C * E + sc + d * d * E + 2 * C * d * E
    elif name == "bwd_chunk":
        fl = 2 * (4 * C * d * d + 3.5 * C * C * d)
        by = 4 * C * d * E + 2 * d * d * E + C * d * E + C * C * E + sc + 2 * C * d * E + sc
        by += C * 4 if kz else 0
    elif name in ("fwd_summary", "fwd_summary_recompute"):
        # scan segment summaries: the state recurrence (no output) over d_v + d_k rows
        fl = 2 * (2 * C * d * 2 * d + C * C * 2 * d)
        by = 2 * C * d * E + C * C * E + sc
    elif name == "bwd_summary":
        fl = 2 * (3 * C * d * 2 * d + 2 * C * C * 2 * d)
        by = 3 * C * d * E + 2 * C * C * E + sc
    else:
        return None
    return fl, by


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gdn_bf16")
    ap.add_argument("--policy", default=None, choices=[None, "save", "recompute"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-recompute-leg", action="store_true")
    ap.add_argument("--no-scan", action="store_true",
                    help="force one sequential state pass (DN_FLAG_NO_SCAN) where the chunk-parallel scan "
                         "would run")
    ap.add_argument("--decode", action="store_true",
                    help="instead of fwd+bwd, time the recurrent (decode) entry point: --decode-batch "
                         "sequences with the workload's heads and dims, --decode-tokens tokens per "
                         "sequence and call, the fp32 state updated in place")
    ap.add_argument("--phase", action="store_true",
                    help="with --decode: the phase-controlled gate (dn_recurrent_phase_fwd, complex state, "
                         "per-channel decay and phase)")
    ap.add_argument("--graph", action="store_true",
                    help="with --decode: also time the calls captured in a HIP graph and replayed")
    ap.add_argument("--decode-batch", type=int, default=64)
    ap.add_argument("--decode-tokens", type=int, default=1)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run --steps device-to-device copies of MIB MiB "
                         "(a known-size reference for the HBM byte counters) and exit")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this operator build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from delta_rule_linear_gated_amd import binding as B
    from delta_rule_linear_gated_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "launches": max(1, args.steps)}), flush=True)
        return
    B.lib()  # fail loudly if the HIP library is missing
    w = W.CONFIGS[args.workload]
    if args.decode:
        decode_bench(args, w)
        return
    policy = args.policy or w.policy
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.describe()}", file=sys.stderr, flush=True)
    inp_cpu = W.make_inputs(w)
    inp = {n: (None if t is None else t.to(dev)) for n, t in inp_cpu.items()}
    q, k, v, beta, g, h0, do, dhT = (inp[n] for n in ("q", "k", "v", "beta", "g", "h0", "do", "dhT"))
    sh = B.shape_of(q, v, g, w.C, w.kaczmarz_eps, args.no_scan)   # Kaczmarz workloads: beta carries eta
    E = 2 if w.dtype == "bf16" else 4
    NT = -(-w.T // w.C)
    lay = B.dn_workspace_layout(sh, B.DN_PASS_FWD)
    uses_scan = lay["total"] > lay["seg_end"]

    def buffers(pol):
        bufs = dict(
            o=torch.empty_like(v),
            hT=torch.empty(w.B, w.H, w.dv, w.dk, device=dev),
            states=(B.saved_buffer(sh, dev) if pol == "save" else None),
            wsf=B.workspace(sh, B.DN_PASS_FWD, dev),
            wsb=B.workspace(sh, B.DN_PASS_BWD if pol == "save" else B.DN_PASS_BWD_RECOMPUTE, dev),
            dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
            dbeta=torch.empty_like(beta), dg=(None if g is None else torch.empty_like(g)),
            dh0=torch.empty(w.B, w.H, w.dv, w.dk, device=dev))
        return bufs

    stream = torch.cuda.current_stream(dev)

    def step(b):
        st = B.dn_chunk_fwd(sh, q, k, v, beta, g, h0, b["o"], b["hT"], b["states"], b["wsf"],
                            b["wsf"].numel(), stream)
        if st != B.DN_OK:
            raise B.DnError(st, B.dn_last_error())
        st = B.dn_chunk_bwd(sh, q, k, v, beta, g, h0, do, dhT, b["states"], b["dq"], b["dk"], b["dv"],
                            b["dbeta"], b["dg"], b["dh0"], b["wsb"], b["wsb"].numel(), stream)
        if st != B.DN_OK:
            raise B.DnError(st, B.dn_last_error())

    def timed(pol, steps, warmup, events):
        b = buffers(pol)
        for _ in range(warmup):
            step(b)
        torch.cuda.synchronize()
        if events:
            B.dn_profile_collect()
            B.dn_profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(steps):
            step(b)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kern = {}
        if events:
            B.dn_profile_enable(False)
            kern = B.dn_profile_collect()
        del b
        return (t1 - t0) * 1e3 / steps, kern

    print(f"[bench] warmup {args.warmup}, timing {args.steps} steps ({policy})", file=sys.stderr, flush=True)
    ms, kern = timed(policy, args.steps, args.warmup, events=True)
    tokens = w.B * w.T
    value = tokens / (ms / 1e3)
    fl_th = algorithmic_flops_per_token_head(w.C, w.dk, w.dv)
    tflops = fl_th * w.token_heads / (ms / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS

    # roofline of the dominant kernel
    gw = w.dk if w.gate == "vector" else (0 if w.gate == "none" else 1)
    per_kernel = {}
    for name, (tot, n) in kern.items():
        avg_ms = tot / max(n, 1)
        per_kernel[name] = {"avg_ms": round(avg_ms, 4), "launches": n, "share": None}
    total_k = sum(t for t, _ in kern.values()) or 1.0
    for name, (tot, n) in kern.items():
        per_kernel[name]["share"] = round(tot / total_k, 3)
    roofline = None
    budgeted = [n for n in kern if kernel_budget(n, w.C, w.dk, E, gw, policy == "save", w.kla)]
    if budgeted:   # the costliest kernel with an algorithmic budget (not the scan's small combine)
        dom = max(budgeted, key=lambda n: kern[n][0])
        fl, by = kernel_budget(dom, w.C, w.dk, E, gw, policy == "save", w.kla)
        units = w.B * w.H * NT                      # chunk-heads per launch
        avg_s = kern[dom][0] / kern[dom][1] / 1e3
        ach_gbs = by * units / avg_s / 1e9
        ach_tf = fl * units / avg_s / 1e12
        intensity = fl / by
        ridge = peak * 1e3 / PEAK_HBM_GBS
        if intensity < ridge:
            roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach_gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(ach_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": int(by * units),
                        "algorithmic_flops_per_launch": int(fl * units),
                        "achieved_tflops": round(ach_tf, 2), "avg_launch_ms": round(avg_s * 1e3, 4)}
        else:
            roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach_tf, 2), "peak": peak,
                        "unit": "TFLOP/s", "frac": round(ach_tf / peak, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": int(by * units),
                        "algorithmic_flops_per_launch": int(fl * units),
                        "achieved_gbs": round(ach_gbs, 1), "avg_launch_ms": round(avg_s * 1e3, 4)}

    # measured HBM traffic of the dominant kernel, from the committed rocprofv3
    # summary of this workload -- only while the kernel sources are unchanged
    if roofline is not None:
        from delta_rule_linear_gated_amd import profiling
        summ = profiling.load_summary(os.path.join(ROOT, "profiles", f"{w.name}_all_kernels_rocprof.md"))
        if summ and summ.get("source_sha256") == profiling.source_digest():
            rec = summ["kernels"].get(roofline["kernel"], {})
            if "bytes" in rec:
                roofline["traffic"] = rec["bytes"]
                roofline["traffic_source"] = f"profiles/{w.name}_all_kernels_rocprof.md"

    other = None
    if not args.no_recompute_leg and w.B * w.H * w.T > 0:
        pol2 = "recompute" if policy == "save" else "save"
        ms2, _ = timed(pol2, max(1, args.steps // 2), 2, events=False)
        other = {"policy": pol2, "ms_per_step": round(ms2, 4), "tokens_per_s": round(tokens / (ms2 / 1e3), 1)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp_cpu)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: gate={w.gate} B={w.B} H={w.H} T={w.T} dk={w.dk} dv={w.dv} "
                               f"C={w.C} policy={policy}, fwd+bwd"
                               + (", state passes by the chunk-parallel scan" if uses_scan else "")
                               + (f", Kaczmarz step in-kernel (eps={w.kaczmarz_eps:g})" if w.kla else ""),
                   "global_batch": w.B, "seq_len": w.T, "heads": w.H, "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / peak, 4),
        "algorithmic_gflop_per_step": round(fl_th * w.token_heads / 1e9, 2),
        "roofline": roofline, "kernels": per_kernel, "other_policy": other, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def decode_bench(args, w0):
    """Decode throughput of dn_recurrent_fwd: one call advances every sequence of a
    serving batch by --decode-tokens tokens.  HBM-bound: each call reads and writes
    the fp32 state once (2 dv dk 4 bytes per head) plus the tokens' q, k, v, beta, g
    and o."""
    import torch

    from delta_rule_linear_gated_amd import binding as B
    from delta_rule_linear_gated_amd import workloads as W

    gate = "vector" if args.phase else w0.gate   # the phase-controlled gate decays per channel
    w = W.custom(args.decode_batch, w0.H, args.decode_tokens, w0.dk, w0.dv, w0.C, gate, w0.dtype,
                 h0_std=0.5, kla=w0.kla, seed=w0.seed, name=f"decode_{w0.name}", kz_eps=w0.kz_eps,
                 phase=args.phase)
    dev = torch.device("cuda:0")
    print(f"[bench] decode: generating {w.describe()}", file=sys.stderr, flush=True)
    inp_cpu = W.make_inputs(w, cotangents=False)
    inp = {n: (None if t is None else t.to(dev)) for n, t in inp_cpu.items()}
    q, k, v, beta, g = (inp[n] for n in ("q", "k", "v", "beta", "g"))
    state = inp["h0"].clone()
    state_im = inp["h0_im"].clone() if args.phase else None
    o = torch.empty_like(v)
    sh = B.make_shape(w.B, w.H, w.T, w.dk, w.dv, w.C, w.dtype, w.gate, w.kaczmarz_eps)
    stream = torch.cuda.current_stream(dev)

    def call():
        stream = torch.cuda.current_stream(dev)   # (the capture stream while a graph is captured)
        if args.phase:
            st = B.dn_recurrent_phase_fwd(sh, q, k, v, beta, g, inp["theta"], state, state_im, o, stream)
        else:
            st = B.dn_recurrent_fwd(sh, q, k, v, beta, g, state, o, stream)
        if st != B.DN_OK:
            raise B.DnError(st, B.dn_last_error())

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()           # the timed calls, without timing events
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    B.dn_profile_collect()              # then the kernel's own duration, from HIP events
    B.dn_profile_enable(True)
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    B.dn_profile_enable(False)
    kern = B.dn_profile_collect()
    graph = None
    if args.graph:   # calls captured once in a HIP graph and replayed (no per-call launch cost)
        per = 16
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(per):
                call()
        gr.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // per)
        t0 = time.perf_counter()
        for _ in range(reps):
            gr.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) * 1e3 / (reps * per)
        graph = {"calls_per_replay": per, "replays": reps, "ms_per_call": round(gms, 5),
                 "tokens_per_s": round(w.B * w.T / (gms / 1e3), 1)}
    E = 2 if w.dtype == "bf16" else 4
    gw = w.dk if w.gate == "vector" else (0 if w.gate == "none" else 1)
    heads = w.B * w.H
    nst = 2 if args.phase else 1           # real (and imaginary) state, read and written once
    by = heads * (nst * 2 * w.dv * w.dk * 4 + w.T * ((2 * w.dk + 2 * w.dv) * E + 4 * (1 + gw)
                                                  + (4 * w.dk if args.phase else 0)))
    fl = heads * w.T * (8 if not args.phase else 16) * w.dv * w.dk   # decay, S k, rank-one update, S q
    kname = "recurrent_phase" if args.phase else "recurrent"
    tot, n = kern.get(kname, (0.0, 0))
    roofline = None
    if n:
        avg_s = tot / n / 1e3
        ach = by / avg_s / 1e9
        roofline = {"kernel": kname, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                    "algorithmic_bytes_per_launch": int(by), "algorithmic_flops_per_launch": int(fl),
                    "avg_launch_ms": round(avg_s * 1e3, 4)}
    tokens = w.B * w.T
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build_oracle()
        f = {nm: W.to_f64(t) for nm, t in inp_cpu.items()}
        threads = min(16, os.cpu_count() or 1)
        t0 = time.perf_counter()
        reps = 0
        while True:
            if args.phase:
                from oracle import sfda
                sfda.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["theta"], f["h0"], f["h0_im"],
                             eps=w.kaczmarz_eps)
            elif w.kla:
                oracle.kaczmarz_forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"], eps=w.kaczmarz_eps,
                                        nthreads=threads)
            else:
                oracle.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"], nthreads=threads)
            reps += 1
            if time.perf_counter() - t0 > 2.0:
                break
        dt = (time.perf_counter() - t0) / reps
        if args.phase:
            threads = 1   # the phase-controlled gate's oracle is numpy, one thread
        cpu = {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"the whole batch ({w.B * w.H} heads x {w.T} token(s)), fp64, {reps} repetitions"}
    line = {
        "metric": "decode tokens/s (recurrent form, state in place" + (", phase-controlled gate)" if args.phase
                                                                         else ")"),
        "value": round(tokens / (ms / 1e3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"decode{' (phase-controlled gate)' if args.phase else ''}: gate={w.gate} "
                               f"B={w.B} H={w.H} dk={w.dk} dv={w.dv}, {w.T} token(s) "
                               f"per sequence and call", "global_batch": w.B, "seq_len": w.T, "heads": w.H,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline, "graph_replay": graph, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, inp_cpu):
    """The fp64 oracle (sequential recurrence + reverse mode, C, threads over
    heads) on the same workload, timed on the host.  Sample: every head of the
    batch at full length when that fits the time budget, else the first heads."""
    import oracle
    from delta_rule_linear_gated_amd import workloads as W

    threads = max(1, min(16, os.cpu_count() or 1))
    nheads_all = w.B * w.H
    # ~0.65 core-seconds per head of 4096 steps at d = 128 (fwd + bwd); keep it to ~20 s wall
    est = 0.65 * (w.T / 4096) * (w.dk * w.dv / 16384) * nheads_all / threads
    nheads = nheads_all if est <= 20 else max(1, int(nheads_all * 20 / est))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:nheads]
    f = {n: W.to_f64(t, heads) for n, t in inp_cpu.items()}
    print(f"[bench] cpu baseline: oracle on {nheads} heads x T={w.T}, {threads} threads", file=sys.stderr,
          flush=True)
    args = (f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"])
    t0 = time.perf_counter()
    if w.kla:   # Kaczmarz step: beta carries eta
        oracle.kaczmarz_forward(*args, eps=w.kaczmarz_eps, nthreads=threads)
        oracle.kaczmarz_backward(*args, f["do"], f["dhT"], eps=w.kaczmarz_eps, nthreads=threads)
    else:
        oracle.forward(*args, nthreads=threads)
        oracle.backward(*args, f["do"], f["dhT"], nthreads=threads)
    dt = time.perf_counter() - t0
    tok = nheads * w.T / w.H  # tokens of all heads: the sample covers nheads/H batch rows
    return {"value": round(tok / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{nheads} of {nheads_all} heads, full length T={w.T}, fwd+bwd, fp64 "
                      f"({dt:.1f} s wall)"}


if __name__ == "__main__":
    main()
