#!/usr/bin/env python3
"""Benchmark of the packed shared-prefix attention path on one MI355X.

One step = the whole hot path over one batch already resident in HBM:
  pg_build_layout (host builder + upload) -> pg_position_ids -> pg_rope (Q, K)
  -> pg_attn_fwd (O, lse). The layout upload runs on a copy stream that the
  compute stream waits for, so it overlaps the previous step's kernels.
Default workload: GRPO-style bf16, 16 prompts x 8 responses, 32/8 heads,
d = 128 (the configuration the useful-TFLOP/s target is quoted on).

Prints ONE JSON line. `value` = useful attention FLOP per step / step time
(useful FLOP = 4 * d * Hq * allowed query-key pairs of the packed layout).
`roofline` is for pg_attn_fwd alone, timed with HIP events on its stream.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")
KERNEL_SOURCES = ["shared_prefix_packed_amd/csrc/pg_attn_mfma.hip",
                  "shared_prefix_packed_amd/csrc/pg_internal.h",
                  "shared_prefix_packed_amd/csrc/pg_layout.cpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per attention launch from committed rocprofv3 counters, or
    None when they were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(workload)
    if not r or r.get("kernel_hash") != kernel_source_hash():
        return None
    return r.get("hbm_bytes_per_launch")


# ------------------------------------------------------ rocprofv3 summaries --
# `--profile-recipe` prints the rocprofv3 runs of this script behind each
# summary under profiles/ (run from the repository root after
# `export TMPDIR=/tmp`); `--profile-summary` turns their CSV output into the
# markdown, and with --record-traffic stores the attention kernel's calibrated
# HBM bytes per launch in profiles/attn_traffic.json under the current kernel
# source hash. Both take the same --workload and --profile-dir.

COPY_BYTES = 1 << 30
SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_LDS_IDX_ACTIVE",
               "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES",
               "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU_TRANS_F32", "GRBM_GUI_ACTIVE"]
TCC_COUNTERS = ["TCC_HIT_sum", "TCC_MISS_sum", "GRBM_GUI_ACTIVE"]
TRACE_STEPS, TRACE_WARMUP = 10, 3


def profile_recipe(workload: int, root: str):
    """(name, output directory, command) of every run behind one summary."""
    tag = f"wl{workload}"
    run = f"python3 bench.py --no-cpu-baseline --no-unpacked --workload {workload}"
    fwd_only = run + " --no-backward --no-gathers --no-decode --steps 2 --warmup 1"
    d = lambda name: os.path.join(root, name)
    pmc = lambda counters, out, prog, limit=150: (
        f"timeout -s KILL {limit} rocprofv3 --pmc {' '.join(counters)} -d {out} -o pmc "
        f"--output-format csv -- {prog}")
    copy = f"python3 bench.py --copy-bytes {COPY_BYTES}"
    return [
        ("trace", d(f"{tag}_trace"),
         f"timeout -s KILL 300 rocprofv3 --kernel-trace --stats -d {d(f'{tag}_trace')} -o trace "
         "--output-format csv -- "
         f"{run} --steps {TRACE_STEPS} --warmup {TRACE_WARMUP}"),
        ("fetch", d(f"{tag}_fetch"), pmc(["FETCH_SIZE"], d(f"{tag}_fetch"), run + " --steps 3 --warmup 1")),
        ("write", d(f"{tag}_write"), pmc(["WRITE_SIZE"], d(f"{tag}_write"), run + " --steps 3 --warmup 1")),
        ("cal_fetch", d("copy_fetch"), pmc(["FETCH_SIZE"], d("copy_fetch"), copy, 60)),
        ("cal_write", d("copy_write"), pmc(["WRITE_SIZE"], d("copy_write"), copy, 60)),
        ("sq", d(f"{tag}_sq"), pmc(SQ_COUNTERS, d(f"{tag}_sq"), fwd_only)),
        ("tcc", d(f"{tag}_tcc"), pmc(TCC_COUNTERS, d(f"{tag}_tcc"), fwd_only)),
    ]


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob
    paths = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not paths:
        raise SystemExit(f"bench.py: no *{suffix} under {directory}")
    for path in paths:
        with open(path, newline="") as f:
            yield from csv.DictReader(f)


def _short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    depth, cut = 0, len(name)
    for i in range(len(name) - 1, -1, -1):   # drop the trailing argument list
        if name[i] == ")":
            depth += 1
        elif name[i] == "(":
            depth -= 1
            if depth == 0:
                cut = i
                break
    return name[:cut].strip()[:60]


def _kernel_durations(trace_dir: str):
    """Kernel name -> dispatch durations in us, in launch order."""
    rows = [r for r in _csv_rows(trace_dir, "kernel_trace.csv")]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = {}
    for r in rows:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        out.setdefault(_short_name(r["Kernel_Name"]), []).append(dur)
    return out


def _counter_medians(pmc_dir: str):
    """Kernel name -> counter name -> median over dispatches of the per-dispatch sum."""
    import statistics
    per = {}
    for r in _csv_rows(pmc_dir, "counter_collection.csv"):
        key = (_short_name(r["Kernel_Name"]), r["Counter_Name"])
        d = per.setdefault(key, {})
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    out = {}
    for (k, c), vals in per.items():
        out.setdefault(k, {})[c] = statistics.median(vals.values())
    return out


def _algorithmic_bytes(kernel: str, T: int, Hq: int, Hkv: int, d: int, elem: int):
    """Compulsory HBM bytes of one launch: every tensor the kernel must touch, once."""
    q = T * Hq * d * elem         # one [T, Hq, d] tensor
    kv = T * Hkv * d * elem       # one [T, Hkv, d] tensor
    row = T * Hq * 4              # one fp32 value per (token, query head)
    table = {
        "positions_kernel": T * 3 * 4 + T * 8,                # g0, pe, ss per token in; int64 out
        "rope_kernel": 2 * (q + kv) + T * 8,                   # Q, K, positions in; Q, K out
        "attn_fwd_bf16_d128": 2 * q + 2 * kv + row,            # Q, K, V in; O, lse out
        "bwd_dq_kernel": 4 * q + 2 * kv + 2 * row,             # Q, dO, O, K, V, lse in; dQ, D out
        "bwd_dkv_kernel": 2 * q + 4 * kv + 2 * row,            # Q, dO, K, V, lse, D in; dK, dV out
    }
    base = kernel[5:] if kernel.startswith("void ") else kernel
    return table.get(base.split("<")[0])


def profile_summary(args) -> int:
    """Markdown summary of the runs `profile_recipe` lists (see the comment above)."""
    import numpy as np
    from workloads import make_workload
    import shared_prefix_packed_amd as pg
    recipe = {name: (out, cmd) for name, out, cmd in profile_recipe(args.workload, args.profile_dir)}
    w = make_workload(args.workload)
    L = pg.pg_build_layout_host(w.prefix_lens, w.suffix_counts, w.suffix_lens, w.num_q_heads,
                                w.num_kv_heads, w.head_dim, w.rope_theta)
    pairs = int(L.summary().useful_pairs)
    L.close()
    T, Hq, Hkv, d = w.total_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim
    fwd_flop = 4 * d * Hq * pairs
    attn = "attn_fwd_bf16_d128"
    lines = [f"# rocprofv3 summary: {w.name} (T={T}, {w.num_groups} groups, Hq={Hq}, Hkv={Hkv}, d={d})", "",
             "Every command runs from the repository root after `export TMPDIR=/tmp`; "
             f"`python3 bench.py --profile-summary --workload {args.workload} --record-traffic` "
             "then writes this file from their output (and the attention entry of "
             "profiles/attn_traffic.json).", "",
             "Kernel trace:", "", "    " + recipe["trace"][1], "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    durs = _kernel_durations(recipe["trace"][0])
    total = sum(sum(v) for v in durs.values())
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {len(v)} | {np.mean(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                     f"{100 * sum(v) / total:.1f} |")
    a = durs.get(attn, [])
    timed = a[TRACE_WARMUP:TRACE_WARMUP + TRACE_STEPS]
    if timed:
        t_us = float(np.mean(timed))
        tf = fwd_flop / (t_us * 1e-6) / 1e12
        lines += ["", f"{attn}: {len(a)} launches = {TRACE_WARMUP} warm-up + {len(timed)} timed steps. "
                  f"Over the timed steps: mean {t_us:.1f} us, median {float(np.median(timed)):.1f} us; "
                  f"{fwd_flop} useful FLOP per launch (4 d Hq x {pairs} allowed pairs) / {t_us:.1f} us = "
                  f"{tf:.1f} TFLOP/s = {100 * tf / PEAK_BF16_TFLOPS:.1f} % of the "
                  f"{PEAK_BF16_TFLOPS} TFLOP/s dense bf16 peak (bench.py's `roofline.achieved` is the "
                  f"HIP-event mean of the same timed launches)."]
    bwd_q, bwd_kv = durs.get("bwd_dq_kernel"), durs.get("bwd_dkv_kernel")
    if bwd_q and bwd_kv:
        bq, bk = float(np.mean(bwd_q[2:] or bwd_q)), float(np.mean(bwd_kv[2:] or bwd_kv))
        bflop = 10 * d * Hq * pairs
        lines += ["", f"Backward (pg_attn_bwd after the forward steps, its 2 warm-up calls left out): dQ "
                  f"{bq:.1f} us + dK/dV {bk:.1f} us = {bq + bk:.1f} us for {bflop} useful FLOP "
                  f"(10 d Hq per allowed pair) = {bflop / ((bq + bk) * 1e-6) / 1e12:.1f} TFLOP/s = "
                  f"{100 * bflop / ((bq + bk) * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.1f} % of peak; dQ kernel "
                  f"alone {0.6 * bflop / (bq * 1e-6) / 1e12:.1f} TFLOP/s (S, dP, dQ), dK/dV kernel alone "
                  f"{0.8 * bflop / (bk * 1e-6) / 1e12:.1f} TFLOP/s (S, dP, dV, dK)."]

    fetch, write = _counter_medians(recipe["fetch"][0]), _counter_medians(recipe["write"][0])
    cf, cw = _counter_medians(recipe["cal_fetch"][0]), _counter_medians(recipe["cal_write"][0])
    copy_kib = COPY_BYTES / 1024.0

    def cal(meds, counter):
        vals = [c[counter] for c in meds.values() if counter in c]
        v = max(vals) if vals else 0.0   # the copy is the largest dispatch of its run
        return copy_kib / v if v else float("nan")
    ff, fw = cal(cf, "FETCH_SIZE"), cal(cw, "WRITE_SIZE")
    lines += ["", "HBM traffic, one counter per run, then the same two passes over a plain device copy:", ""]
    lines += ["    " + recipe[n][1] for n in ("fetch", "write", "cal_fetch", "cal_write")]
    lines += ["", f"Calibration: the {COPY_BYTES}-byte copy reads FETCH_SIZE "
              f"{copy_kib / ff:.0f} KiB and WRITE_SIZE {copy_kib / fw:.0f} KiB, so bytes = FETCH_SIZE x 1024 x "
              f"{ff:.3f} and WRITE_SIZE x 1024 x {fw:.3f}.", "",
              "| kernel | FETCH KiB (median) | WRITE KiB (median) | HBM MB/launch (calibrated) | algorithmic MB | ratio |",
              "|---|---|---|---|---|---|"]
    attn_bytes = None
    for k in sorted(set(fetch) | set(write), key=lambda k: -(fetch.get(k, {}).get("FETCH_SIZE", 0))):
        fk, wk = fetch.get(k, {}).get("FETCH_SIZE", 0.0), write.get(k, {}).get("WRITE_SIZE", 0.0)
        hbm = (fk * ff + wk * fw) * 1024
        alg = _algorithmic_bytes(k, T, Hq, Hkv, d, 2 if w.dtype == "bf16" else 4)
        if k == attn:
            attn_bytes = int(round(hbm))
        lines.append(f"| {k} | {fk:.0f} | {wk:.0f} | {hbm / 1e6:.1f} | "
                     f"{'' if alg is None else f'{alg / 1e6:.1f}'} | {'' if alg is None else f'{hbm / alg:.2f}'} |")
    lines += ["", "Algorithmic bytes: each tensor a kernel must read or write, once (positions: three "
              "per-token tables in, int64 positions out; RoPE: Q, K, positions in, Q, K out; attention: "
              "Q, K, V in, O and lse out; dQ launch: Q, dO, O, K, V, lse in, dQ and D out; dK/dV launch: "
              "Q, dO, K, V, lse, D in, dK and dV out). The excess is K/V (forward, dQ) or Q/dO (dK/dV) "
              "re-read by the work items of a group, which L2 serves only in part."]

    meds = {}
    for n in ("sq", "tcc"):
        if os.path.isdir(recipe[n][0]):
            meds.update(_counter_medians(recipe[n][0]).get(attn, {}))
    if meds:
        lines += ["", f"Counters of {attn} (medians over its dispatches, one run per pass):", "",
                  "    " + recipe["sq"][1], "    " + recipe["tcc"][1], "",
                  "| counter | value |", "|---|---|"]
        for c, v in sorted(meds.items()):
            lines.append(f"| {c} | {v:.0f} |")
        gui = meds.get("GRBM_GUI_ACTIVE")
        if gui:
            simd_cycles = gui / 8 * 1024   # GRBM_GUI_ACTIVE sums the 8 XCDs; 1024 SIMDs
            derived = []
            if "SQ_VALU_MFMA_BUSY_CYCLES" in meds:
                derived.append(f"MFMA busy {100 * meds['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.1f} %")
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in meds:
                derived.append("MFMA and VALU issuing together "
                               f"{100 * meds['SQ_VALU_MFMA_COEXEC_CYCLES'] / simd_cycles:.1f} %")
            if meds.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in meds:
                derived.append("LDS bank conflicts "
                               f"{100 * meds['SQ_LDS_BANK_CONFLICT'] / meds['SQ_LDS_IDX_ACTIVE']:.1f} % of LDS cycles")
            if "TCC_HIT_sum" in meds and meds.get("TCC_HIT_sum", 0) + meds.get("TCC_MISS_sum", 0) > 0:
                derived.append("L2 hit rate "
                               f"{100 * meds['TCC_HIT_sum'] / (meds['TCC_HIT_sum'] + meds['TCC_MISS_sum']):.1f} %")
            if timed:
                derived.append(f"clock {gui / 8 / (float(np.median(timed)) * 1e-6) / 1e9:.2f} GHz "
                               "(GRBM_GUI_ACTIVE per XCD over the median timed launch)")
            lines += ["", "Derived (SIMD cycles = GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs): " +
                      "; ".join(derived) + "."]
    print("\n".join(lines))

    if args.record_traffic and attn_bytes:
        try:
            with open(TRAFFIC_FILE) as f:
                rec = json.load(f)
        except (OSError, ValueError):
            rec = {}
        rec[w.name] = {"kernel_hash": kernel_source_hash(), "hbm_bytes_per_launch": attn_bytes,
                       "fetch_kib": fetch.get(attn, {}).get("FETCH_SIZE"),
                       "write_kib": write.get(attn, {}).get("WRITE_SIZE"),
                       "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    return 0


def cpu_baseline(w, qkv, budget_s: float):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload:
    whole groups, one query head at a time (group-major), until the time
    budget is spent. Reports useful FLOP/s of the sample."""
    import numpy as np
    from oracle import pg_oracle as O
    from workloads import bf16_bits_to_f32
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    r = w.num_q_heads // w.num_kv_heads
    lay = O.layout(w.prefix_lens, w.suffix_counts, w.suffix_lens)
    conv = (lambda x: bf16_bits_to_f32(x)) if w.dtype == "bf16" else (lambda x: x)
    t0 = time.perf_counter()
    units = 0
    flop = 0
    groups = set()
    soff = 0
    for g in range(w.num_groups):
        n = int(w.suffix_counts[g])
        sub = O.layout(w.prefix_lens[g:g + 1], w.suffix_counts[g:g + 1],
                       w.suffix_lens[soff:soff + n])
        soff += n
        a, b = int(lay["group_off"][g]), int(lay["group_off"][g + 1])
        if b == a:
            continue
        for h in range(w.num_q_heads):
            hk = h // r
            q = conv(qkv["q"][a:b, h:h + 1])
            k = conv(qkv["k"][a:b, hk:hk + 1])
            v = conv(qkv["v"][a:b, hk:hk + 1])
            O.attention(q, k, v, sub, w.softmax_scale, 1, 1)
            units += 1
            groups.add(g)
            flop += 4 * w.head_dim * O.useful_pairs(sub)
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle on {units} (group, query head) units from groups "
                   f"{sorted(groups)} of {w.name}: {flop / 1e9:.1f} useful GFLOP in {dt:.1f} s; "
                   f"BLAS threads={threads}, host cpus={os.cpu_count()}"),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, help="workload index 0..4 (default 2: GRPO)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-unpacked", action="store_true", help="skip the unpacked-layout baseline")
    ap.add_argument("--no-backward", action="store_true", help="skip timing pg_attn_bwd")
    ap.add_argument("--no-gathers", action="store_true", help="skip timing pg_pack_rows / pg_unpack_rows")
    ap.add_argument("--no-decode", action="store_true", help="skip timing pg_attn_decode")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes 5 times (calibrates "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE against a known byte count)")
    ap.add_argument("--profile-recipe", action="store_true",
                    help="no GPU work: print the rocprofv3 runs behind the --workload's profile summary")
    ap.add_argument("--profile-summary", action="store_true",
                    help="no GPU work: write the --workload's profile summary (markdown, stdout) from "
                         "the output of the --profile-recipe runs")
    ap.add_argument("--profile-dir", default="rocprof_out",
                    help="where the --profile-recipe runs write (default rocprof_out)")
    ap.add_argument("--record-traffic", action="store_true",
                    help="with --profile-summary: store the attention launch's calibrated HBM bytes in "
                         "profiles/attn_traffic.json under the current kernel source hash")
    args = ap.parse_args(argv)
    if args.profile_recipe:
        for _, _, cmd in profile_recipe(args.workload, args.profile_dir):
            print(cmd)
        return 0
    if args.profile_summary:
        return profile_summary(args)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(groups would shard across GPUs with no exchange between them)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 4 * n, "launches": 5}), flush=True)
        return 0
    import shared_prefix_packed_amd as pg
    from shared_prefix_packed_amd.baseline import unpacked_decode_workload, unpacked_workload
    from workloads import draw_decode, draw_qkv, draw_tensor, make_workload, sha256

    pg.load()   # fails loudly without the built library
    w = make_workload(args.workload)
    print(f"[bench] workload {w.name}: T={w.total_tokens} G={w.num_groups}", file=sys.stderr, flush=True)
    qkv = draw_qkv(w)
    dt_torch = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    q, k, v = dev(qkv["q"]), dev(qkv["k"]), dev(qkv["v"])
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    stream = torch.cuda.current_stream()
    qr = torch.empty_like(q)
    kr = torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    pos = torch.empty(T, dtype=torch.int64, device="cuda")

    def build():
        return pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, Hq, Hkv, d,
                                  w.rope_theta, stream=stream)

    info = build()
    summ = info.summary()
    useful_flop = 4 * d * Hq * int(summ.useful_pairs)
    info.close()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    attn_ms, rope_ms, pos_ms, layout_ms = [], [], [], []

    # Each step's layout is built on the host and uploaded on a copy stream;
    # the compute stream waits for that upload before its first kernel. The
    # host runs ahead of the GPU, so the upload of step i+1 overlaps the
    # kernels of step i instead of queueing behind them, as a training loop
    # that prepares its next batch would do.
    upload = torch.cuda.Stream()

    def step(record):
        t_host = time.perf_counter()
        L = pg.pg_build_layout(w.prefix_lens, w.suffix_counts, w.suffix_lens, Hq, Hkv, d,
                               w.rope_theta, stream=upload)
        t_host = time.perf_counter() - t_host
        stream.wait_stream(upload)
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record(stream)
        pg.pg_position_ids(L, pos=pos, stream=stream)
        e1.record(stream)
        pg.pg_rope(L, pos, q, k, q_out=qr, k_out=kr, stream=stream)
        e2.record(stream)
        pg.pg_attn_fwd(L, qr, kr, v, w.softmax_scale, o=o, lse=lse, stream=stream)
        e3.record(stream)
        L.close()
        if record:
            layout_ms.append(t_host * 1e3)
            return (e0, e1, e2, e3)
        return None

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        events.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for e0, e1, e2, e3 in events:
        pos_ms.append(e0.elapsed_time(e1))
        rope_ms.append(e1.elapsed_time(e2))
        attn_ms.append(e2.elapsed_time(e3))
    ms_per_step = wall * 1e3 / args.steps
    attn_avg = float(np.mean(attn_ms))
    attn_tflops = useful_flop / (attn_avg * 1e-3) / 1e12
    value = useful_flop / (ms_per_step * 1e-3) / 1e12

    # unpacked baseline (same kernel, prefix duplicated per response)
    speedup = None
    unpacked_ms = None
    if not args.no_unpacked:
        un = unpacked_workload(w.prefix_lens, w.suffix_counts, w.suffix_lens)
        idx = torch.from_numpy(un.gather).cuda()
        qu, ku, vu = qr[idx].contiguous(), kr[idx].contiguous(), v[idx].contiguous()
        Lu = pg.pg_build_layout(un.prefix_lens, un.suffix_counts, un.suffix_lens, Hq, Hkv, d,
                                w.rope_theta, stream=stream)
        ou = torch.empty_like(qu)
        lu = torch.empty((Hq, qu.shape[0]), dtype=torch.float32, device="cuda")
        for _ in range(2):
            pg.pg_attn_fwd(Lu, qu, ku, vu, w.softmax_scale, o=ou, lse=lu, stream=stream)
        ts = []
        for _ in range(max(3, args.steps // 2)):
            a_, b_ = ev(), ev()
            a_.record(stream)
            pg.pg_attn_fwd(Lu, qu, ku, vu, w.softmax_scale, o=ou, lse=lu, stream=stream)
            b_.record(stream)
            ts.append((a_, b_))
        torch.cuda.synchronize()
        unpacked_ms = float(np.mean([a_.elapsed_time(b_) for a_, b_ in ts]))
        speedup = unpacked_ms / attn_avg
        Lu.close()
        del qu, ku, vu, ou, lu

    # backward on the same batch: dQ, dK, dV for a seeded upstream gradient dO
    bwd = None
    if not args.no_backward and w.dtype == "bf16" and d == 128:
        do = dev(draw_tensor(w, "do"))
        L = build()
        dq, dk, dv = torch.empty_like(qr), torch.empty_like(kr), torch.empty_like(v)
        delta = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
        run_bwd = lambda: pg.pg_attn_bwd(L, qr, kr, v, o, lse, do, w.softmax_scale, dq=dq, dk=dk,
                                         dv=dv, delta=delta, stream=stream)
        for _ in range(2):
            run_bwd()
        ts = []
        for _ in range(max(3, args.steps // 2)):
            a_, b_ = ev(), ev()
            a_.record(stream)
            run_bwd()
            b_.record(stream)
            ts.append((a_, b_))
        torch.cuda.synchronize()
        bwd_ms = float(np.mean([a_.elapsed_time(b_) for a_, b_ in ts]))
        bwd_flop = 10 * d * Hq * int(summ.useful_pairs)
        bwd_tflops = bwd_flop / (bwd_ms * 1e-3) / 1e12
        bwd = {"ms": round(bwd_ms, 4), "useful_flop": bwd_flop,
               "useful_tflops": round(bwd_tflops, 2),
               "pct_of_bf16_peak": round(100 * bwd_tflops / PEAK_BF16_TFLOPS, 2),
               "flop_definition": "10 * d * Hq per allowed (query, key) pair: S, dP, dV, dQ, dK products",
               "kernels": "bwd_dq_kernel (which also forms D) + bwd_dkv_kernel, one pg_attn_bwd call"}
        L.close()
        del do, dq, dk, dv, delta

    # pack / unpack gathers either side of the path, on hidden-state rows
    gathers = None
    if not args.no_gathers:
        hidden = 2048
        Gn, Nn = len(w.prefix_lens), len(w.suffix_lens)
        ppad, spad = int(w.prefix_lens.max()), int(w.suffix_lens.max())
        L = build()
        pre = torch.randn((Gn, ppad, hidden), device="cuda").to(torch.bfloat16)
        suf = torch.randn((Nn, spad, hidden), device="cuda").to(torch.bfloat16)
        packed = torch.empty((T, hidden), dtype=torch.bfloat16, device="cuda")
        for _ in range(2):
            pg.pg_pack_rows(L, pre, suf, packed=packed, stream=stream)
            pg.pg_unpack_rows(L, packed, ppad, spad, stream=stream)
        tp, tu = [], []
        for _ in range(20):
            a_, b_, c_ = ev(), ev(), ev()
            a_.record(stream)
            pg.pg_pack_rows(L, pre, suf, packed=packed, stream=stream)
            b_.record(stream)
            outs = pg.pg_unpack_rows(L, packed, ppad, spad, stream=stream)
            c_.record(stream)
            tp.append((a_, b_))
            tu.append((b_, c_))
        # a plain device copy of the packed bytes: the practical ceiling
        cpy = torch.empty_like(packed)
        tc = []
        for _ in range(20):
            a_, b_ = ev(), ev()
            a_.record(stream)
            with torch.cuda.stream(stream):
                cpy.copy_(packed)
            b_.record(stream)
            tc.append((a_, b_))
        torch.cuda.synchronize()
        cms = float(np.mean([x.elapsed_time(y) for x, y in tc]))
        # the right-padded form [G, max_len] of the same rows, and back
        Lp = build()
        width = Lp.summary().max_group_len
        padded = torch.empty((Gn, width, hidden), dtype=torch.bfloat16, device="cuda")
        back = torch.empty_like(packed)
        for _ in range(2):
            pg.pg_pad_rows(Lp, packed, padded=padded, stream=stream)
            pg.pg_unpad_rows(Lp, padded, packed=back, stream=stream)
        tpa, tun = [], []
        for _ in range(20):
            a_, b_, c_ = ev(), ev(), ev()
            a_.record(stream)
            pg.pg_pad_rows(Lp, packed, padded=padded, stream=stream)
            b_.record(stream)
            pg.pg_unpad_rows(Lp, padded, packed=back, stream=stream)
            c_.record(stream)
            tpa.append((a_, b_))
            tun.append((b_, c_))
        torch.cuda.synchronize()
        pad_ms = float(np.mean([x.elapsed_time(y) for x, y in tpa]))
        unpad_ms = float(np.mean([x.elapsed_time(y) for x, y in tun]))
        Lp.close()
        pms = float(np.mean([x.elapsed_time(y) for x, y in tp]))
        ums = float(np.mean([x.elapsed_time(y) for x, y in tu]))
        rb = hidden * 2
        pack_bytes = 2 * T * rb                                         # read + write each packed row
        unpack_bytes = (T + Nn) * rb + (Gn * ppad + Nn * (spad + 1)) * rb   # rows read, padded outputs written
        gathers = {"row_bytes": rb,
                   "pack_ms": round(pms, 4), "pack_gbs": round(pack_bytes / (pms * 1e-3) / 1e9, 1),
                   "unpack_ms": round(ums, 4), "unpack_gbs": round(unpack_bytes / (ums * 1e-3) / 1e9, 1),
                   "device_copy_gbs": round(pack_bytes / (cms * 1e-3) / 1e9, 1),
                   "padded_width": int(width),
                   "pad_ms": round(pad_ms, 4),
                   "pad_gbs": round((T + Gn * width) * rb / (pad_ms * 1e-3) / 1e9, 1),
                   "unpad_ms": round(unpad_ms, 4),
                   "unpad_gbs": round(2 * T * rb / (unpad_ms * 1e-3) / 1e9, 1),
                   "hbm_peak_gbs": PEAK_HBM_GBS}
        L.close()
        del pre, suf, packed, outs, cpy, padded, back

    # one decode step with this batch's layout taken as the KV cache (response
    # segments at capacity, current lengths drawn in [1, capacity])
    decode = None
    if not args.no_decode and w.dtype == "bf16" and d == 128 and len(w.suffix_lens) > 0:
        dx = draw_decode(w)
        L = build()
        qd = dev(dx["q"])
        cur_np = dx["cur_lens"].astype(np.int64)
        cur = torch.from_numpy(dx["cur_lens"]).cuda()
        Nr = qd.shape[0]
        od = torch.empty_like(qd)
        ld = torch.empty((Hq, Nr), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, L.decode_workspace_size()), dtype=torch.uint8, device="cuda")

        def time_decode(layout, kc, vc, work):
            # steps back to back, as a decode loop issues them (the host's
            # enqueue of step i+1 overlaps step i on the GPU), between one
            # pair of events; the mean per step of three such runs
            for _ in range(3):
                pg.pg_attn_decode(layout, qd, kc, vc, cur, w.softmax_scale, o=od, lse=ld,
                                  workspace=work, stream=stream)
            ts = []
            for _ in range(3):
                a_, b_ = ev(), ev()
                a_.record(stream)
                for _ in range(20):
                    pg.pg_attn_decode(layout, qd, kc, vc, cur, w.softmax_scale, o=od, lse=ld,
                                      workspace=work, stream=stream)
                b_.record(stream)
                ts.append((a_, b_))
            torch.cuda.synchronize()
            return float(np.mean([a_.elapsed_time(b_) / 20 for a_, b_ in ts]))

        dec_ms = time_decode(L, kr, v, ws)
        # algorithmic bytes: each group's prompt K/V once (groups with
        # responses), each response's valid K/V rows once, Q read, O and lse written
        row_kv = Hkv * d * 2 * 2
        has_resp = np.asarray(w.suffix_counts) > 0
        prompt_rows = int(np.asarray(w.prefix_lens, dtype=np.int64)[has_resp].sum())
        valid_rows = int(np.clip(cur_np, 0, np.asarray(w.suffix_lens, dtype=np.int64)).sum())
        qo_bytes = 2 * Nr * Hq * d * 2 + Hq * Nr * 4
        dec_bytes = (prompt_rows + valid_rows) * row_kv + qo_bytes
        resp_prompt = np.repeat(np.asarray(w.prefix_lens, dtype=np.int64), w.suffix_counts)
        unpacked_bytes = int(resp_prompt.sum() + valid_rows) * row_kv + qo_bytes
        decode = {"ms": round(dec_ms, 4), "bytes": dec_bytes,
                  "gbs": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
                  "pct_of_hbm_peak": round(100 * dec_bytes / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                  "responses": Nr, "work_items": L.summary().num_dec_items,
                  "bytes_unpacked": unpacked_bytes,
                  "bytes_definition": "K and V rows read once (each group's prompt once, each "
                                      "response's valid rows once), Q read, O and lse written"}
        L.close()
        if not args.no_unpacked:
            un = unpacked_decode_workload(w.prefix_lens, w.suffix_counts, w.suffix_lens)
            idx = torch.from_numpy(un.gather).cuda()
            ku, vu = kr[idx].contiguous(), v[idx].contiguous()
            Lu = pg.pg_build_layout(un.prefix_lens, un.suffix_counts, un.suffix_lens, Hq, Hkv, d,
                                    w.rope_theta, stream=stream)
            wsu = torch.empty(max(1, Lu.decode_workspace_size()), dtype=torch.uint8, device="cuda")
            un_ms = time_decode(Lu, ku, vu, wsu)
            decode["unpacked_ms"] = round(un_ms, 4)
            decode["speedup_vs_unpacked"] = round(un_ms / dec_ms, 3)
            Lu.close()
            del ku, vu, wsu
        del qd, od, ld, ws

    traffic = load_traffic(w.name)
    roof = {
        "bound": "mfma",
        "achieved": round(attn_tflops, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
    }
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a CPU sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, qkv, args.cpu_budget)

    out = {
        "metric": "packed shared-prefix attn fwd: useful TFLOP/s, % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "groups": w.num_groups,
            "tokens": int(T),
            "num_q_heads": int(Hq),
            "num_kv_heads": int(Hkv),
            "head_dim": int(d),
            "useful_flop_per_step": useful_flop,
            "useful_pairs": int(summ.useful_pairs),
            "unpacked_pairs": int(summ.unpacked_pairs),
            "work_items": int(summ.num_items),
            "parallelism": "none (1 GPU)",
            "input_sha256": {n: sha256(qkv[n])[:16] for n in ("q", "k", "v")},
        },
        "attn_only_tflops": round(attn_tflops, 2),
        "pct_of_bf16_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "stage_ms": {
            "layout_host": round(float(np.mean(layout_ms)), 4),
            "position_ids": round(float(np.mean(pos_ms)), 4),
            "rope": round(float(np.mean(rope_ms)), 4),
            "attn_fwd": round(attn_avg, 4),
        },
        "attn_fwd_ms_stats": {"mean": round(attn_avg, 4), "median": round(float(np.median(attn_ms)), 4),
                              "min": round(float(np.min(attn_ms)), 4), "reps": len(attn_ms)},
        "rope_gbs": round(2 * T * (Hq + Hkv) * d * q.element_size() / (np.mean(rope_ms) * 1e-3) / 1e9, 1),
        "unpacked_attn_ms": None if unpacked_ms is None else round(unpacked_ms, 4),
        "speedup_vs_unpacked": None if speedup is None else round(speedup, 3),
        "roofline": roof,
        "backward": bwd,
        "gathers": gathers,
        "decode": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
