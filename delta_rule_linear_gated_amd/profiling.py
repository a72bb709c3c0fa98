"""Summaries of rocprofv3 output for the operator's kernels.

``python -m delta_rule_linear_gated_amd.profiling summarize ...`` turns the CSV
output of a ``--kernel-trace --stats`` run and of ``--pmc FETCH_SIZE`` /
``--pmc WRITE_SIZE`` runs (plus the same counters over a device copy of known
size) into a short markdown summary with an embedded JSON block.  bench.py
reads that block to report the measured HBM traffic of its dominant kernel,
and only while the kernel sources still hash to the digest recorded in it.

Counter scaling: each counter is divided by what it reads for the reference
copy (bytes moved / counter value), so a kernel's traffic is
``FETCH_SIZE * fetch_scale + WRITE_SIZE * write_scale`` (KiB -> bytes).

``python -m delta_rule_linear_gated_amd.profiling counters ...`` summarises
``--pmc`` runs of the matrix-core and LDS counters per kernel:
  MFMA busy      SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * CUs * 4 SIMDs)
  executed MFMA  SQ_INSTS_VALU_MFMA_MOPS_{BF16,F32} * 512 flops per dispatch,
                 and those flops over the dispatch's duration against the peak
  LDS conflicts  SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles)
GRBM_GUI_ACTIVE counts GPU-busy cycles once per XCD on this part; the busy
fraction divides by the per-XCD value (the counter divided by --xcds).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


# The sources the chunkwise kernels are built from (the measured path): the
# device headers, the launch code and the per-variant units.  Other files under
# csrc/ (the C ABI, the recurrent and phase-gate kernels, the scratch array) do
# not change these kernels.
KERNEL_SOURCES = ("dn_device.h", "dn_fwd_kernels.h", "dn_bwd_kernels.h", "dn_internal.h", "dn_launch.h",
                  "dn_launch.hip")


def source_digest() -> str:
    """sha256 over the sources of the chunkwise kernels, in name order."""
    h = hashlib.sha256()
    names = set(KERNEL_SOURCES) | {os.path.basename(x) for x in glob.glob(os.path.join(CSRC, "dn_[fb]wd_*_g*.hip"))}
    for path in sorted(os.path.join(CSRC, n) for n in names):
        if os.path.isfile(path):
            h.update(os.path.basename(path).encode())
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def _trailing_bools(name: str) -> list:
    """The bool template arguments at the end of a kernel name, demangled
    ("..., true, false>(") or mangled ("...Lb1ELb0EEEv")."""
    m = re.search(r"((?:(?:true|false), )*(?:true|false))>\(", name)
    if m:
        return [x == "true" for x in m.group(1).split(", ")]
    m = re.search(r"((?:Lb[01]E)+)EEv", name)
    if m:
        return [x == "1" for x in re.findall(r"Lb([01])E", m.group(1))]
    return []


def kernel_key(name: str) -> str:
    """Map a rocprofv3 kernel name (demangled or mangled) to the names
    dn_profile_collect uses."""
    for k in ("phase_prep", "phase_fwd_state", "phase_bwd_state", "phase_bwd_chunk"):
        if k + "_kernel" in name:
            return k
    if "recompute_bwd_state_kernel" in name:   # the recomputed forward chains and bwd_state, one launch
        return "fwd_state_recompute+bwd_state"
    if "prep_kernel" in name:
        return "prep"
    if "fwd_state_kernel" in name:   # <..., SAVE, OUTPUT>
        b = _trailing_bools(name)[-2:]
        if b == [False, False]:
            return "fwd_summary"
        return "fwd_state" if b[-1:] == [True] else "fwd_state_recompute"
    if "bwd_state_kernel" in name:   # <..., SUMMARY>
        return "bwd_summary" if _trailing_bools(name)[-1:] == [True] else "bwd_state"
    if "scan_combine_kernel" in name:
        return "scan_combine"
    if "bwd_chunk_kernel" in name:
        return "bwd_chunk"
    if "copyBuffer" in name or "elementwise" in name:
        return "copy"
    return name


def _csv(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def counter_means(d):
    """{kernel key: mean counter value per dispatch} of one --pmc run."""
    acc = collections.defaultdict(list)
    for r in _csv(_find(d, "counter_collection.csv")):
        acc[kernel_key(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def copy_value(d):
    """Counter value of the copy kernel dispatches (the largest-valued copy kernel)."""
    best = 0.0
    for r in _csv(_find(d, "counter_collection.csv")):
        if kernel_key(r["Kernel_Name"]) == "copy":
            best = max(best, float(r["Counter_Value"]))
    return best


def timed_means(d, steps, warmup):
    """{kernel key: mean duration (us) of its launches in the timed steps} from the
    kernel trace: a kernel launched n times over warmup + steps steps has its last
    n * steps / (warmup + steps) launches in the timed region (the warmup launches
    also see the clock ramp up, so the all-launch average runs high)."""
    acc = collections.defaultdict(list)
    rows = sorted(_csv(_find(d, "kernel_trace.csv")), key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        acc[kernel_key(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = {}
    for k, v in acc.items():
        n = max(1, round(len(v) * steps / (steps + warmup)))
        out[k] = sum(v[-n:]) / n
    return out


def summarize(args) -> str:
    stats = _csv(_find(args.trace, "kernel_stats.csv"))
    timed = timed_means(args.trace, args.steps, args.warmup) if args.steps else {}
    fetch = counter_means(args.fetch)
    write = counter_means(args.write)
    copy_kib = args.copy_mib * 1024.0
    fetch_scale = copy_kib / copy_value(args.copy_fetch)
    write_scale = copy_kib / copy_value(args.copy_write)
    kern = {}
    for r in stats:
        k = kernel_key(r["Name"])
        if k == "copy":
            continue
        f = fetch.get(k)
        w = write.get(k)
        rec = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
               "share": float(r["Percentage"]) / 100.0}
        if k in timed:
            rec["timed_avg_us"] = timed[k]
        if f is not None and w is not None:
            rec.update(fetch_kib=f, write_kib=w,
                       bytes=int((f * fetch_scale + w * write_scale) * 1024))
        kern[k] = rec
    data = {"workload": args.workload, "source_sha256": source_digest(),
            "fetch_scale": fetch_scale, "write_scale": write_scale, "copy_mib": args.copy_mib,
            "kernels": kern}
    lines = [f"# {args.title}", "", "Commands (from /tmp, TMPDIR=/tmp):", ""]
    for c in args.command:
        lines.append(f"    {c}")
    lines += ["", "| kernel | calls | avg us (all) | avg us (timed steps) | share | FETCH_SIZE KiB | WRITE_SIZE KiB "
              "| HBM bytes (scaled) |", "|---|---|---|---|---|---|---|---|"]
    for k, r in kern.items():
        lines.append(f"| {k} | {r['calls']} | {r['avg_us']:.1f} | {r.get('timed_avg_us', float('nan')):.1f} | "
                     f"{r['share']:.3f} | "
                     f"{r.get('fetch_kib', float('nan')):.0f} | {r.get('write_kib', float('nan')):.0f} | "
                     f"{r.get('bytes', 0):,} |")
    lines += ["", f"Copy calibration ({args.copy_mib} MiB read + written per copy): FETCH_SIZE scale "
              f"{fetch_scale:.4f}, WRITE_SIZE scale {write_scale:.4f} (true KiB per counted KiB).", "",
              "```json", json.dumps(data, indent=1), "```", ""]
    return "\n".join(lines)


def counter_table(d):
    """{kernel key: {counter: mean value per dispatch}} plus the dispatch fields
    (duration ns, VGPRs, AGPRs, LDS bytes) of one --pmc run."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _csv(_find(d, "counter_collection.csv")):
        k = kernel_key(r["Kernel_Name"])
        acc[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for f, name in (("Start_Timestamp", None), ("VGPR_Count", "vgpr"), ("Accum_VGPR_Count", "agpr"),
                        ("LDS_Block_Size", "lds_bytes")):
            if name and f in r and r[f] not in ("", None):
                acc[k]["_" + name].append(float(r[f]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def counters(args) -> str:
    tab = collections.defaultdict(dict)
    for d in args.run:
        for k, cs in counter_table(d).items():
            tab[k].update(cs)
    timed = {}
    if args.summary:
        s = load_summary(args.summary)
        if s:
            timed = {k: r.get("timed_avg_us", r.get("avg_us")) for k, r in s["kernels"].items()}
    rows = []
    data = {"workload": args.workload, "source_sha256": source_digest(), "cus": args.cus, "xcds": args.xcds,
            "clock_ghz": args.clock_ghz, "kernels": {}}
    for k in sorted(tab, key=lambda x: -(timed.get(x) or 0)):
        if k == "copy":
            continue
        c = tab[k]
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        grbm = c.get("GRBM_GUI_ACTIVE")
        mfma_busy = busy / (grbm / args.xcds * args.cus * 4) if busy is not None and grbm else None
        fl_bf16 = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        fl_f32 = c.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) * 512
        us = timed.get(k)
        tf_bf16 = fl_bf16 / (us * 1e-6) / 1e12 if us else None
        tf_f32 = fl_f32 / (us * 1e-6) / 1e12 if us else None
        conf = c.get("SQ_LDS_BANK_CONFLICT")
        act = c.get("SQ_LDS_IDX_ACTIVE")
        rec = {"avg_us": us, "mfma_busy": mfma_busy, "mfma_flops_bf16": fl_bf16, "mfma_flops_f32": fl_f32,
               "mfma_tflops_bf16": tf_bf16, "mfma_tflops_f32": tf_f32,
               "mfma_peak_frac_bf16": tf_bf16 / args.peak_bf16 if tf_bf16 is not None else None,
               "mfma_peak_frac_f32": tf_f32 / args.peak_f32 if tf_f32 is not None else None,
               "lds_conflict_frac": conf / act if conf is not None and act else None,
               "raw": {n: v for n, v in c.items()}}
        data["kernels"][k] = rec

        def f(x, fmt):
            return "-" if x is None else format(x, fmt)
        rows.append(f"| {k} | {f(us, '.1f')} | {f(mfma_busy, '.1%')} | {fl_bf16 / 1e9:.2f} | {f(tf_bf16, '.1f')} | "
                    f"{f(rec['mfma_peak_frac_bf16'], '.2%')} | {fl_f32 / 1e9:.3f} | {f(rec['lds_conflict_frac'], '.1%')} | "
                    f"{f(c.get('_vgpr'), '.0f')} / {f(c.get('_agpr'), '.0f')} | {f(c.get('_lds_bytes'), '.0f')} |")
    lines = [f"# {args.title}", "", "Commands (from /tmp, TMPDIR=/tmp):", ""]
    for cmd in args.command:
        lines.append(f"    {cmd}")
    lines += ["", "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x CUs x 4); executed flops = "
              "SQ_INSTS_VALU_MFMA_MOPS_* x 512 per dispatch; TFLOP/s = executed flops / the kernel's average "
              "duration in the timed steps (kernel-trace summary); LDS conflicts = SQ_LDS_BANK_CONFLICT / "
              "SQ_LDS_IDX_ACTIVE.", "",
              "| kernel | avg us | MFMA busy | bf16 MFMA GFLOP / launch | bf16 TFLOP/s | of bf16 peak | "
              "fp32 MFMA GFLOP / launch | LDS conflict cycles | VGPR_Count / Accum_VGPR_Count fields | LDS bytes |",
              "|---|---|---|---|---|---|---|---|---|---|", *rows, "",
              "```json", json.dumps(data, indent=1), "```", ""]
    return "\n".join(lines)


def load_summary(path):
    """The JSON block of a summary written by ``summarize`` (None if absent)."""
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", txt, re.S)
    return json.loads(m.group(1)) if m else None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--trace", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-fetch", required=True)
    s.add_argument("--copy-write", required=True)
    s.add_argument("--copy-mib", type=float, required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", action="append", default=[])
    s.add_argument("--steps", type=int, default=0, help="timed steps of the traced bench run")
    s.add_argument("--warmup", type=int, default=0, help="warmup steps of the traced bench run")
    s.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--run", action="append", required=True, help="a --pmc output directory (repeatable)")
    c.add_argument("--summary", help="the kernel-trace summary of the same workload (for durations)")
    c.add_argument("--workload", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--clock-ghz", type=float, default=2.4)
    c.add_argument("--peak-bf16", type=float, default=2516.6)
    c.add_argument("--peak-f32", type=float, default=157.3)
    c.add_argument("--out", required=True)
    sub.add_parser("digest")
    a = ap.parse_args()
    if a.cmd == "digest":
        print(source_digest())
        return
    txt = summarize(a) if a.cmd == "summarize" else counters(a)
    with open(a.out, "w") as f:
        f.write(txt)
    print(txt)


if __name__ == "__main__":
    main()
