#!/usr/bin/env python3
"""Throughput of the chunkwise gated delta rule on one MI355X.

One step = one forward (dn_chunk_fwd) + one ReWY backward (dn_chunk_bwd) over
one batch of synthetic input already resident in HBM, through the C ABI.
Default workload: Gated DeltaNet, bf16 q/k/v/dO with fp32 gate / beta / state,
B=8, H=16, T=4096, d_k=d_v=128, chunk 64, states saved by the forward.

Timing: W untimed warmup steps, then K steps bracketed by synchronisations,
each step bracketed by HIP events on the launch stream (three per step:
before the forward, between forward and backward, after the backward; no
events inside the library).  ms_per_step and value use the median step; the
fwd and bwd medians and the wall-clock mean are reported beside it.  A second
pass of K steps records events around every kernel launch inside the library
(dn_profile_enable) for the per-kernel durations behind the roofline.

Prints ONE JSON line: tokens/s (B*T per second, all heads), algorithmic
TFLOP/s and its fraction of the dense MFMA peak, the whole step against the
HBM roof (minimum bytes of the operator), the roofline of the dominant kernel
(the minimum bytes of the pass it belongs to / its average launch time; its
own tensor budget beside it), the recomputation policy's step time, and the
fp64 CPU oracle timed on the host (threaded, and one thread on a smaller sample).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--policy save|recompute]
                    [--no-cpu-baseline] [--gpus 1]
"""
from __future__ import annotations

import argparse
import dataclasses
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


def algorithmic_bytes_per_token_head(dk: int, dv: int, E: int, gw: int):
    """Minimum HBM bytes per token and head of (forward, backward): every input
    read once and every output written once, nothing else (no saved states, no
    per-chunk intermediates).  E = bytes per I/O element, gw = gate values per
    step (0 none, 1 scalar, dk per-channel), 4 bytes each.
      forward : q, k, v read, o written, beta, g read
      backward: q, k, v, dO read, dq, dk, dv written, beta read, dbeta written,
                g read, dg written"""
    fwd = (2 * dk + dv) * E + dv * E + 4 + 4 * gw
    bwd = (2 * dk + dv) * E + dv * E + (2 * dk + dv) * E + 8 + 8 * gw
    return fwd, bwd


FWD_KERNELS = ("prep", "fwd_state", "fwd_summary")
PEAK_FP32_VALU_TFLOPS = 157.3   # MI355X fp32 vector ALUs (256 CUs x 128 lanes x 2 flops x 2.4 GHz)


def phase_flops_per_chunk(name: str, C: int, D: int) -> int:
    """Algorithmic fp32 flops of one chunk-head of the phase-controlled gate's
    kernels: a complex multiply-add counts 8, a real-by-complex one 4, a complex
    exponential 10 (turn reduction, exp, sin, cos, scaling); pairs (t, u <= t)
    number C (C + 1) / 2.  Recomputation counts as work here: these kernels are
    bound by the vector ALUs, not by HBM."""
    pairs = C * (C + 1) // 2
    if name == "phase_prep":        # pairwise G, H per channel; T by forward substitution
        return pairs * D * 20 + 4 * C * C * (C - 1)
    if name == "phase_fwd_state":   # X, Y; U, O; S1; the gated tiles
        return 24 * C * D * D + 8 * pairs * D * 2 + 6 * D * D + 29 * C * D
    if name == "phase_bwd_state":   # Ub; P^H dO; lambda; dS0; the gated tiles
        return 20 * C * D * D + 6 * pairs * D * 2 + 6 * D * D + 27 * C * D
    if name == "phase_bwd_chunk":   # X, U; Ab, Pb; dS1.S0; the three row sums; pair terms per element
        # (each pair factor formed by both of its elements, one complex product each)
        return 28 * C * D * D + 8 * pairs * D * 2 + 32 * C * C * D + 8 * D * D + 60 * C * D
    return 0


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
        by += C * d * E if (saved and name == "fwd_state") else 0   # U beside the saved states
    elif name == "bwd_state":
        fl = 2 * (3 * C * d * d + C * C * d)
        by = 3 * C * d * E + 2 * C * C * E + sc + d * d * E + 2 * C * d * E
    elif name == "bwd_chunk":
        # with saved states U is read (not X, R, U = T R formed again, which needs T)
        fl = 2 * (3 * C * d * d + 2.5 * C * C * d) if saved else 2 * (4 * C * d * d + 3.5 * C * C * d)
        by = 4 * C * d * E + 2 * d * d * E + C * d * E + (C * d * E if saved else C * C * E) + sc + 2 * C * d * E + sc
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gdn_bf16")
    ap.add_argument("--policy", default=None, choices=[None, "save", "recompute"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-recompute-leg", action="store_true")
    ap.add_argument("--no-scan", action="store_true",
                    help="force one sequential state pass (DN_FLAG_NO_SCAN) where the chunk-parallel scan "
                         "would run")
    ap.add_argument("--fp32-work", action="store_true",
                    help="the precision option with fp32 working matrices: the workload's bf16 data, upcast "
                         "exactly to fp32, through the fp32 path (fp32 tiles and fp32 matrix-core operands)")
    ap.add_argument("--phase-chunk", action="store_true",
                    help="instead of the real gates, time the chunkwise phase-controlled gate "
                         "(dn_chunk_phase_fwd + dn_chunk_phase_bwd, chunks of 16) on the workload's batch, heads, "
                         "length and gate at d = --phase-d (default: the workload's dk), with phases "
                         "theta = 0.5 N(0, 1)")
    ap.add_argument("--phase-d", type=int, default=None, choices=[16, 32, 64, 128],
                    help="with --phase-chunk: the head size (dk = dv)")
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
    if args.phase_chunk:
        phase_chunk_bench(args, w)
        return
    policy = args.policy or w.policy
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.describe()}", file=sys.stderr, flush=True)
    inp_cpu = W.make_inputs(w)
    if args.fp32_work:   # the same bf16 values, held and computed in fp32
        if w.dtype != "bf16":
            print("--fp32-work takes a bf16 workload", file=sys.stderr)
            sys.exit(2)
        inp_cpu = {n: (t.float() if t is not None and t.dtype == torch.bfloat16 else t) for n, t in inp_cpu.items()}
        w = dataclasses.replace(w, dtype="fp32")
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

    def fwd(b):
        st = B.dn_chunk_fwd(sh, q, k, v, beta, g, h0, b["o"], b["hT"], b["states"], b["wsf"],
                            b["wsf"].numel(), stream)
        if st != B.DN_OK:
            raise B.DnError(st, B.dn_last_error())

    def bwd(b):
        st = B.dn_chunk_bwd(sh, q, k, v, beta, g, h0, do, dhT, b["states"], b["dq"], b["dk"], b["dv"],
                            b["dbeta"], b["dg"], b["dh0"], b["wsb"], b["wsb"].numel(), stream)
        if st != B.DN_OK:
            raise B.DnError(st, B.dn_last_error())

    def median(xs):
        s = sorted(xs)
        m = len(s) // 2
        return s[m] if len(s) % 2 else 0.5 * (s[m - 1] + s[m])

    def timed(pol, steps, warmup, kernels):
        """Median step / fwd / bwd ms from per-step HIP events, the wall-clock mean,
        and (kernels=True) a second pass with per-launch events inside the library."""
        b = buffers(pol)
        for _ in range(warmup):
            fwd(b)
            bwd(b)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(stream)
            fwd(b)
            ev[i][1].record(stream)
            bwd(b)
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        res = {"median_ms": median([e[0].elapsed_time(e[2]) for e in ev]),
               "fwd_ms": median([e[0].elapsed_time(e[1]) for e in ev]),
               "bwd_ms": median([e[1].elapsed_time(e[2]) for e in ev]),
               "wall_mean_ms": (t1 - t0) * 1e3 / steps}
        kern = {}
        if kernels:
            B.dn_profile_collect()
            B.dn_profile_enable(True)
            for _ in range(steps):
                fwd(b)
                bwd(b)
            torch.cuda.synchronize()
            B.dn_profile_enable(False)
            kern = B.dn_profile_collect()
        del b
        return res, kern

    print(f"[bench] warmup {args.warmup}, timing {args.steps} steps ({policy})", file=sys.stderr, flush=True)
    res, kern = timed(policy, args.steps, args.warmup, kernels=True)
    ms = res["median_ms"]
    tokens = w.B * w.T
    value = tokens / (ms / 1e3)
    fl_th = algorithmic_flops_per_token_head(w.C, w.dk, w.dv)
    tflops = fl_th * w.token_heads / (ms / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    gw = w.dk if w.gate == "vector" else (0 if w.gate == "none" else 1)
    by_fwd, by_bwd = algorithmic_bytes_per_token_head(w.dk, w.dv, E, gw)
    step_bytes = (by_fwd + by_bwd) * w.token_heads
    step_roof = {"algorithmic_bytes": int(step_bytes), "achieved_gbs": round(step_bytes / (ms / 1e3) / 1e9, 1),
                 "hbm_frac": round(step_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                 "fwd_bytes_per_token_head": by_fwd, "bwd_bytes_per_token_head": by_bwd}

    per_kernel = {}
    for name, (tot, n) in kern.items():
        per_kernel[name] = {"avg_ms": round(tot / max(n, 1), 4), "launches": n, "share": None}
    total_k = sum(t for t, _ in kern.values()) or 1.0
    for name, (tot, n) in kern.items():
        per_kernel[name]["share"] = round(tot / total_k, 3)

    # roofline of the dominant kernel: the minimum bytes of the pass it belongs to
    # (per token-head, times the token-heads one launch covers) over its average
    # launch time; the kernel's own tensor budget (which counts the saved states
    # and per-chunk intermediates it reads and writes) is reported beside it
    roofline = None
    budgeted = [n for n in kern if kernel_budget(n, w.C, w.dk, E, gw, policy == "save", w.kla)]
    if budgeted:   # the costliest kernel with a budget (not the scan's small combine)
        dom = max(budgeted, key=lambda n: kern[n][0])
        fl, by = kernel_budget(dom, w.C, w.dk, E, gw, policy == "save", w.kla)
        chunks = w.B * w.H * NT                      # chunk-heads per launch
        units = w.token_heads                        # token-heads per launch
        avg_s = kern[dom][0] / kern[dom][1] / 1e3
        alg_per_unit = by_fwd if dom in FWD_KERNELS else by_bwd
        alg = alg_per_unit * units
        ach_gbs = alg / avg_s / 1e9
        kb_gbs = by * chunks / avg_s / 1e9
        ach_tf = fl * chunks / avg_s / 1e12
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach_gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                    "algorithmic_bytes_per_launch": int(alg),
                    "algorithmic_bytes_per_token_head": alg_per_unit, "token_heads_per_launch": units,
                    "avg_launch_ms": round(avg_s * 1e3, 4),
                    "kernel_budget": {"bytes_per_launch": int(by * chunks), "achieved_gbs": round(kb_gbs, 1),
                                      "frac": round(kb_gbs / PEAK_HBM_GBS, 4)},
                    "kernel_flops_per_launch": int(fl * chunks), "achieved_tflops": round(ach_tf, 2),
                    "mfma_frac": round(ach_tf / peak, 4)}

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
        r2, _ = timed(pol2, max(10, args.steps // 2), 3, kernels=False)
        ms2 = r2["median_ms"]
        other = {"policy": pol2, "ms_per_step": round(ms2, 4), "fwd_ms": round(r2["fwd_ms"], 4),
                 "bwd_ms": round(r2["bwd_ms"], 4), "tokens_per_s": round(tokens / (ms2 / 1e3), 1)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp_cpu)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "fwd_ms": round(res["fwd_ms"], 4), "bwd_ms": round(res["bwd_ms"], 4),
        "wall_mean_ms": round(res["wall_mean_ms"], 4), "timing": "median of per-step HIP events",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic" + (" (bf16 values, held in fp32)" if args.fp32_work else ""),
        "config": {"workload": f"{w.name}: gate={w.gate} B={w.B} H={w.H} T={w.T} dk={w.dk} dv={w.dv} "
                               f"C={w.C} policy={policy}, fwd+bwd"
                               + (", state passes by the chunk-parallel scan" if uses_scan else "")
                               + (f", Kaczmarz step in-kernel (eps={w.kaczmarz_eps:g})" if w.kla else "")
                               + (", fp32 working matrices" if args.fp32_work else ", bf16 matrix-core operands, "
                                  "fp32 accumulation" if w.dtype == "bf16" else ""),
                   "global_batch": w.B, "seq_len": w.T, "heads": w.H, "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / peak, 4),
        "algorithmic_gflop_per_step": round(fl_th * w.token_heads / 1e9, 2), "step_hbm": step_roof,
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


def phase_chunk_bench(args, w0):
    """fwd + bwd of the chunkwise phase-controlled gate: median of per-step HIP
    events, like the main bench; the per-kernel durations from a second pass."""
    import torch

    from delta_rule_linear_gated_amd import binding as B
    from delta_rule_linear_gated_amd import workloads as W

    d = args.phase_d or w0.dk
    w = W.custom(w0.B, w0.H, w0.T, d, d, 16, w0.gate, w0.dtype, h0_std=0.5, seed=w0.seed, name=f"phase_{w0.name}",
                 phase=True)
    dev = torch.device("cuda:0")
    print(f"[bench] phase: generating {w.describe()}", file=sys.stderr, flush=True)
    inp_cpu = W.make_inputs(w)
    x = {n: (None if t is None else t.to(dev)) for n, t in inp_cpu.items()}
    sh = B.make_shape(w.B, w.H, w.T, d, d, 16, w.dtype, w.gate)
    stream = torch.cuda.current_stream(dev)
    o = torch.empty_like(x["v"])
    hr = torch.empty(w.B, w.H, d, d, device=dev)
    hi = torch.empty_like(hr)
    recompute = args.policy == "recompute"   # the backward reruns the state pass instead of reading saved states
    st = None if recompute else torch.empty(max(B.dn_phase_states_bytes(sh) // 4, 1), device=dev)
    nwf = B.dn_phase_workspace_bytes(sh, B.DN_PASS_FWD) if recompute else 0
    wsf = torch.empty(max(nwf, 1), dtype=torch.uint8, device=dev)
    nws = B.dn_phase_workspace_bytes(sh, B.DN_PASS_BWD_RECOMPUTE if recompute else B.DN_PASS_BWD)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    gr = {n: torch.empty_like(x[m]) for n, m in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dbeta", "beta"),
                                                  ("dtheta", "theta"))}
    gr["dg"] = None if x["g"] is None else torch.empty_like(x["g"])
    gr["dh0_re"], gr["dh0_im"] = torch.empty_like(hr), torch.empty_like(hr)

    def fwd():
        st_ = B.dn_chunk_phase_fwd(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], x["theta"], x["h0"], x["h0_im"], o,
                                   hr, hi, st, wsf if recompute else None, nwf, stream)
        if st_ != B.DN_OK:
            raise B.DnError(st_, B.dn_last_error())

    def bwd():
        st_ = B.dn_chunk_phase_bwd(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], x["theta"], x["h0"], x["h0_im"],
                                   x["do"], x["dhT"], x["dhT_im"], st, gr["dq"], gr["dk"], gr["dv"], gr["dbeta"],
                                   gr["dg"], gr["dtheta"], gr["dh0_re"], gr["dh0_im"], ws, nws, stream)
        if st_ != B.DN_OK:
            raise B.DnError(st_, B.dn_last_error())

    steps = max(5, args.steps // 5)   # a step takes milliseconds here
    for _ in range(max(1, args.warmup // 5)):
        fwd()
        bwd()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    med = lambda xs: sorted(xs)[len(xs) // 2]
    ms = med([e[0].elapsed_time(e[2]) for e in ev])
    fms = med([e[0].elapsed_time(e[1]) for e in ev])
    bms = med([e[1].elapsed_time(e[2]) for e in ev])
    B.dn_profile_collect()              # per-kernel durations from HIP events, a pass of their own
    B.dn_profile_enable(True)
    for _ in range(steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    B.dn_profile_enable(False)
    kern = B.dn_profile_collect()
    chunks = w.B * w.H * ((w.T + 15) // 16)
    per_kernel = {n: {"avg_ms": round(t / max(c, 1), 4), "launches": c,
                      "tflops": round(phase_flops_per_chunk(n, 16, d) * chunks / (t / max(c, 1) / 1e3) / 1e12, 2)}
                  for n, (t, c) in kern.items()}
    roofline = None
    if kern:
        dom = max(kern, key=lambda n: kern[n][0])
        avg_s = kern[dom][0] / kern[dom][1] / 1e3
        fl = phase_flops_per_chunk(dom, 16, d) * chunks
        roofline = {"kernel": dom, "bound": "alu", "achieved": round(fl / avg_s / 1e12, 2),
                    "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(fl / avg_s / 1e12 / PEAK_FP32_VALU_TFLOPS, 4), "traffic": None,
                    "algorithmic_flops_per_launch": int(fl), "chunk_heads_per_launch": chunks,
                    "avg_launch_ms": round(avg_s * 1e3, 4)}
    E = 2 if w.dtype == "bf16" else 4
    gw = d if w.gate == "vector" else (0 if w.gate == "none" else 1)
    by_f, by_b = algorithmic_bytes_per_token_head(d, d, E, gw)
    by = (by_f + by_b + 3 * 4 * d) * w.token_heads   # + theta read, dtheta written (fp32 per channel)
    cpu = None if args.no_cpu_baseline else phase_cpu_baseline(w, inp_cpu)
    line = {
        "metric": "chunkwise phase-controlled gate fwd+bwd tokens/s", "value": round(w.B * w.T / (ms / 1e3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": steps, "ms_per_step": round(ms, 4), "fwd_ms": round(fms, 4),
        "bwd_ms": round(bms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"phase-controlled gate, chunks of 16: gate={w.gate} B={w.B} H={w.H} T={w.T} d={d}, "
                               f"fp32 arithmetic (fp32 matrix cores and vector ALUs), "
                               f"{'recomputed' if recompute else 'saved'} states", "global_batch": w.B,
                   "seq_len": w.T, "heads": w.H, "parallelism": "none (1 GPU)"},
        "roofline": roofline, "kernels": per_kernel,
        "step_hbm": {"algorithmic_bytes": int(by), "achieved_gbs": round(by / (ms / 1e3) / 1e9, 1),
                     "hbm_frac": round(by / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 5)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def phase_cpu_baseline(w, inp_cpu):
    """The phase-controlled gate's fp64 oracle (oracle/sfda.py: the complex
    recurrence and its reverse mode, numpy) on a bounded sample of the workload:
    the first heads of the first sequence over the first steps."""
    from oracle import sfda
    from delta_rule_linear_gated_amd import workloads as W

    nh, Ts = min(w.H, 8 if w.dk <= 64 else 4), min(w.T, 8192)   # about 5-10 s of one core
    heads = [(0, h) for h in range(nh)]
    f = {}
    for n, t in inp_cpu.items():
        x = W.to_f64(t, heads)
        if x is not None and n not in ("h0", "h0_im", "dhT", "dhT_im"):
            x = x[:, :, :Ts]
        f[n] = x
    print(f"[bench] cpu baseline: phase oracle on {nh} heads x T={Ts}", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    sfda.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["theta"], f["h0"], f["h0_im"])
    sfda.backward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["theta"], f["h0"], f["h0_im"], f["do"], f["dhT"],
                  f["dhT_im"])
    dt = time.perf_counter() - t0
    tok = nh * Ts / w.H   # tokens of whole sequences: the sample covers nh / H of a sequence's heads
    return {"value": round(tok / dt, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{nh} heads of sequence 0, steps 0..{Ts - 1}, fwd+bwd, fp64 numpy ({dt:.1f} s wall)"}


def host_info() -> dict:
    """The host the CPU baseline ran on: CPU model and the logical CPUs this
    process may use (the oracle's thread count is capped at 16 beside it)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


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
    def run(f, nthreads):
        args = (f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"])
        t0 = time.perf_counter()
        if w.kla:   # Kaczmarz step: beta carries eta
            oracle.kaczmarz_forward(*args, eps=w.kaczmarz_eps, nthreads=nthreads)
            oracle.kaczmarz_backward(*args, f["do"], f["dhT"], eps=w.kaczmarz_eps, nthreads=nthreads)
        else:
            oracle.forward(*args, nthreads=nthreads)
            oracle.backward(*args, f["do"], f["dhT"], nthreads=nthreads)
        return time.perf_counter() - t0

    dt = run(f, threads)
    tok = nheads * w.T / w.H  # tokens of all heads: the sample covers nheads/H batch rows
    # one thread on the first head alone
    f1 = {n: W.to_f64(t, heads[:1]) for n, t in inp_cpu.items()}
    dt1 = run(f1, 1)
    return {"value": round(tok / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{nheads} of {nheads_all} heads, full length T={w.T}, fwd+bwd, fp64 "
                      f"({dt:.1f} s wall)",
            "single_thread": {"value": round(w.T / w.H / dt1, 1), "unit": "tokens/s", "cores": 1,
                              "sample": f"1 head, full length T={w.T}, fwd+bwd, fp64 ({dt1:.1f} s wall)"},
            "host": host_info()}


if __name__ == "__main__":
    main()
