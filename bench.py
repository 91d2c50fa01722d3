#!/usr/bin/env python3
"""Benchmark of MLA paged-KV decode on one MI355X.

One step = one mla_decode call over one batch of synthetic input (the split-KV
partial kernel and the LSE merge kernel, back to back on one stream), with all
inputs resident in HBM.  The default workload is B=4, q_len=4, H=32, FP8 E4M3,
81,920-token cache per sequence (page_size 64).  The KV pool is replicated into
enough rotating copies that consecutive steps never find their cache in the
256 MB Infinity Cache.

Before the timed steps come the W warm-up steps and then as many more as it
takes to keep the GPU busy for --warmup-ms (default 250 ms): from idle, its
clocks take some 40 ms of sustained load to settle, and a serving GPU runs at
the settled clocks.

Prints one JSON line: metric / value (effective KV-read TB/s) / ms_per_step,
the roofline of the dominant kernel measured live with HIP events on the
launch stream, and the fp64 CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/step + effective KV-read TB/s (q_len=4, 80K-token cache)"
HBM_PEAK_GBS = 8000.0
# dense MFMA peak of the path's contraction type: bf16, fp8, fp16, and bf16 for bf16 q over an
# E4M3 cache (its operands are widened to bf16)
MFMA_PEAK_TFLOPS = {1: 2500.0, 2: 5000.0, 3: 2500.0, 4: 2500.0}
DTYPE_NAMES = {1: "bf16", 2: "fp8_e4m3", 3: "fp16", 4: "bf16_q.fp8_e4m3_kv"}
MALL_BYTES = 256 << 20
# published per-step latency for exactly this workload on the pages (another machine: context only)
PAGES_US = {"agentic_b4_q4_h32_fp8_80k": 49.5, "agentic_b16_q4_h32_fp8_80k": 148.1}
KERNEL_SOURCE = os.path.join(ROOT, "mla_paged_kv_decode_amd", "csrc", "mla_kernels.hip")


def code_hash(text: str) -> str:
    """sha256/16 of HIP source with comments and whitespace removed: edits to comments
    do not make a profile of the same code stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def kernel_hash() -> str:
    with open(KERNEL_SOURCE) as f:
        return code_hash(f.read())


def algorithmic(x) -> dict:
    """Algorithmic bytes / flops of one step (each KV row read once, no partials)."""
    import numpy as np

    import mla_inputs as mi

    e = 1 if mi.kv_format(x.dtype) == mi.FP8_E4M3 else 2
    eq = 1 if mi.q_format(x.dtype) == mi.FP8_E4M3 else 2
    L = x.seq_lens.astype(np.int64)
    B, q_len, H = x.B, x.q_len, x.H
    kv = int(L.sum()) * 576 * e
    q = B * q_len * H * 576 * eq
    o = B * q_len * H * 512 * 2
    lse = B * q_len * H * 4
    bt = int(((L + x.page_size - 1) // x.page_size).sum()) * 4
    sl = B * 4
    vis = 0
    for b in range(B):
        for t in range(q_len):
            vis += max(0, min(int(L[b]) - q_len + t + 1, int(L[b])))
    flops = 2 * (576 + 512) * H * vis
    return dict(kv_bytes=kv, bytes=kv + q + o + lse + bt + sl, flops=flops)


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they match this kernel source."""
    path = os.path.join(ROOT, "profiles", f"mla_split_kv_partial_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_code_sha256_16") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20


def warm_up(run_one, min_steps: int, min_ms: float) -> tuple[int, float]:
    """Untimed steps: at least min_steps, and more until min_ms of wall time has passed with the GPU
    kept busy (the host waits for the GPU every 16 steps).  Returns (steps run, ms)."""
    import torch

    t0 = time.perf_counter()
    n = 0
    for _ in range(min_steps):
        run_one(n)
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(16):
            run_one(n)
            n += 1
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def copy_calibration():
    """A plain device copy of known size, for scaling the rocprofv3 byte counters.

    Run under `rocprofv3 --pmc FETCH_SIZE` (and separately WRITE_SIZE): each of
    the three launches reads COPY_BYTES and writes COPY_BYTES.
    """
    import torch

    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.add(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(f"copy calibration: {COPY_BYTES} bytes read and {COPY_BYTES} bytes written per launch", flush=True)


def _csv_rows(path):
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)) or \
        sorted(glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no rocprofv3 csv under {path}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counter_avg(path, counter, name_part):
    """Mean per-dispatch value (KiB, as rocprofv3 reports it) of `counter` for kernels matching name_part."""
    vals = [float(r["Counter_Value"]) for r in _csv_rows(path)
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"{counter} for {name_part!r} not found under {path}")
    return sum(vals) / len(vals), len(vals)


COUNTER_PASSES = {
    "cnt_a": ["GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F8",
              "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS",
              "SQ_WAVE_CYCLES"],
    "cnt_b": ["SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_INSTS_SALU",
              "SQ_INSTS_MFMA", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16"],
}
N_XCD, N_SIMD = 8, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def _counters(path, name_part):
    """Per-dispatch means of every counter in a rocprofv3 --pmc run for kernels matching name_part, with the
    dispatch's own duration (ns) from the same run."""
    per = {}
    dur = {}
    for r in _csv_rows(path):
        if name_part not in r["Kernel_Name"]:
            continue
        per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = {k: sum(v) / len(v) for k, v in per.items()}
    out["_duration_ns"] = sum(dur.values()) / len(dur) if dur else None
    out["_dispatches"] = len(dur)
    return out


def derived_counters(c: dict) -> dict:
    """Clock, MFMA busy fraction, achieved MFMA rate and LDS figures from one dispatch's counters.
    GRBM_GUI_ACTIVE counts GPU-busy cycles on each XCD (summed over the 8); SQ_VALU_MFMA_BUSY_CYCLES sums
    matrix-core busy cycles over all 1024 SIMDs; one MOPS unit is 512 flops."""
    d = {}
    ns = c.get("_duration_ns")
    gui = c.get("GRBM_GUI_ACTIVE")
    if gui and ns:
        cyc = gui / N_XCD
        d["cycles_per_xcd"] = round(cyc)
        d["clock_ghz"] = round(cyc / ns, 3)
        if c.get("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            d["mfma_busy_frac"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD), 4)
    mops = sum(c.get(k, 0.0) for k in ("SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                       "SQ_INSTS_VALU_MFMA_MOPS_F16"))
    if mops and ns:
        d["mfma_tflops"] = round(mops * 512 / (ns * 1e-9) / 1e12, 1)
    for k in ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
              "SQ_INSTS_SALU", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_BUSY_CYCLES",
              "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU"):
        if k in c:
            d[k] = c[k]
    if c.get("SQ_ACTIVE_INST_LDS"):
        d["lds_bank_conflict_share"] = round(c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_ACTIVE_INST_LDS"], 4)
    if c.get("SQ_WAVE_CYCLES"):
        if "SQ_WAIT_ANY" in c:
            d["wait_any_share"] = round(c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"], 4)
        if "SQ_WAIT_INST_ANY" in c:
            d["wait_inst_share"] = round(c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"], 4)
    return d


def _trace_regions(path, steps=50):
    """Per-region kernel timings from the dispatch trace of one bench.py run, in the order bench.py runs
    them: steps (split-KV then merge), split-KV alone back to back, merge alone back to back.  Each
    region is averaged over its last `steps` launches, the timed ones: the warm-up steps run just
    before the timed steps, in the same pattern."""
    import csv
    import glob
    import re

    files = sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        return {}
    with open(files[0]) as f:
        ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                     "P" if "mla_split_kv" in r["Kernel_Name"] else "M" if "combine" in r["Kernel_Name"] else "o")
                    for r in csv.DictReader(f))
    seq = "".join(e[2] for e in ev)
    out = {}

    def stats(idx, stride):
        dur = [(ev[i][1] - ev[i][0]) / 1e3 for i in idx]
        per = [(ev[j][0] - ev[i][0]) / 1e3 for i, j in zip(idx[:-1], idx[1:])]
        return round(sum(dur) / len(dur), 2), round(sum(per) / len(per), 2) if per else None

    m = re.search(r"(?:PM){5,}", seq)  # the warm-up and timed steps (the first run of them)
    if m:
        ps = list(range(m.start(), m.end(), 2))[-steps:]
        d_p, period = stats(ps, 2)
        d_m, _ = stats([i + 1 for i in ps], 2)
        out["steps"] = {"split_kv_us": d_p, "merge_us": d_m, "step_period_us": period}
    m = re.search(r"P{5,}", seq)
    if m:
        d_p, period = stats(list(range(m.start(), m.end()))[-steps:], 1)
        out["split_kv_alone"] = {"duration_us": d_p, "period_us": period}
    m = re.search(r"M{5,}", seq)
    if m:
        d_m, period = stats(list(range(m.start(), m.end()))[-steps:], 1)
        out["merge_alone"] = {"duration_us": d_m, "period_us": period}
    return out


def summarize_profile(d: str, workload: str):
    """Turn the rocprofv3 runs under d/ (trace, fetch, write, cal_fetch, cal_write) into
    profiles/<kernel>_<workload>.md and the traffic JSON bench.py reports."""
    stats = _csv_rows(os.path.join(d, "trace"))
    cal_f, _ = _counter_avg(os.path.join(d, "cal_fetch"), "FETCH_SIZE", "CUDAFunctorOnSelf_add")
    cal_w, _ = _counter_avg(os.path.join(d, "cal_write"), "WRITE_SIZE", "CUDAFunctorOnSelf_add")
    f_scale = COPY_BYTES / (cal_f * 1024.0)
    w_scale = COPY_BYTES / (cal_w * 1024.0)
    out = {"workload": workload, "kernel_code_sha256_16": kernel_hash(),
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": cal_f, "write_kib": cal_w,
                           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
           "kernels": {}}
    for short, part in (("mla_split_kv_partial", "mla_split_kv"), ("mla_combine", "mla_combine")):
        fk, nf = _counter_avg(os.path.join(d, "fetch"), "FETCH_SIZE", part)
        wk, nw = _counter_avg(os.path.join(d, "write"), "WRITE_SIZE", part)
        st = [r for r in stats if part in r["Name"]]
        avg_ns = float(st[0]["AverageNs"]) if st else None
        out["kernels"][short] = {"fetch_bytes": round(fk * 1024 * f_scale), "write_bytes": round(wk * 1024 * w_scale),
                                 "dispatches_counted": [nf, nw], "avg_duration_ns": avg_ns,
                                 "calls": int(st[0]["Calls"]) if st else None}
    kp = out["kernels"]["mla_split_kv_partial"]
    out["hbm_bytes_per_launch"] = kp["fetch_bytes"] + kp["write_bytes"]
    cnt = {}
    for short, part in (("mla_split_kv_partial", "mla_split_kv"), ("mla_combine", "mla_combine")):
        raw = {}
        for pas in COUNTER_PASSES:
            if os.path.isdir(os.path.join(d, pas)):
                c = _counters(os.path.join(d, pas), part)
                dur = c.pop("_duration_ns")
                c.pop("_dispatches")
                raw.update(c)
                raw.setdefault("_duration_ns", dur)
        if raw:
            cnt[short] = {"raw": {k: v for k, v in raw.items() if not k.startswith("_")},
                          "duration_ns_under_counters": raw.get("_duration_ns"), "derived": derived_counters(raw)}
    if cnt:
        out["counters"] = cnt
    out["regions"] = _trace_regions(os.path.join(d, "trace"))
    base = os.path.join(ROOT, "profiles")
    with open(os.path.join(base, f"mla_split_kv_partial_{workload}_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    ran = ("the warm-up and timed steps of `mla_decode_varlen`, then the split-KV kernel alone"
           if workload.startswith("ragged_prefill") else
           "the warm-up, the timed steps, each kernel alone, and two replays of the captured graph")
    lines = [f"# rocprofv3 summary: {workload}", "",
             f"Kernel trace (`--kernel-trace --stats`) of one `bench.py --steps 50 --warmup 50` run: {ran}:", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name'][:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    reg = out["regions"]
    if reg:
        lines += ["", "The same trace by region of the bench run (durations are kernel execution; periods are "
                  "start-to-start, so they include the dispatch gaps bench.py's events also see):", ""]
        if "steps" in reg:
            r = reg["steps"]
            lines.append(f"- timed steps: split-KV {r['split_kv_us']} us, merge {r['merge_us']} us, one step every "
                         f"{r['step_period_us']} us")
        if "split_kv_alone" in reg:
            r = reg["split_kv_alone"]
            lines.append(f"- split-KV alone, back to back: {r['duration_us']} us each, one every {r['period_us']} us "
                         "(what `kernels_ms.split_kv_partial` and `roofline.avg_launch_ms` measure)")
        if "merge_alone" in reg:
            r = reg["merge_alone"]
            lines.append(f"- merge alone, back to back: {r['duration_us']} us each, one every {r['period_us']} us")
    lines += ["", "HBM traffic per launch (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`), scaled by a copy of "
              f"{COPY_BYTES} bytes (fetch x{f_scale:.3f}, write x{w_scale:.3f}):", "",
              "| kernel | read MB | written MB |", "|---|---|---|"]
    for k, v in out["kernels"].items():
        lines.append(f"| {k} | {v['fetch_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} |")
    if cnt:
        lines += ["", "Counters (`--pmc`, two passes of one `bench.py --steps 5 --warmup 2` run each), per dispatch, "
                  "with the dispatch's own duration in the same run:", "",
                  "- clock = GRBM_GUI_ACTIVE / 8 XCDs / duration",
                  "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs)",
                  "- MFMA rate = SQ_INSTS_VALU_MFMA_MOPS_{F8,BF16,F16} x 512 flops / duration",
                  "- LDS bank-conflict share = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS (cycles)",
                  "- wait shares = SQ_WAIT_ANY, SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES", "",
                  "| kernel | us | clock GHz | MFMA busy | MFMA TFLOP/s | LDS insts | LDS conflict share | "
                  "VALU insts | wait share |", "|---|---|---|---|---|---|---|---|---|"]
        for k, v in cnt.items():
            dv = v["derived"]
            us = (v["duration_ns_under_counters"] or 0) / 1e3
            lines.append(f"| {k} | {us:.1f} | {dv.get('clock_ghz', '')} | {dv.get('mfma_busy_frac', '')} | "
                         f"{dv.get('mfma_tflops', '')} | {dv.get('SQ_INSTS_LDS', 0):.4g} | "
                         f"{dv.get('lds_bank_conflict_share', '')} | {dv.get('SQ_INSTS_VALU', 0):.4g} | "
                         f"{dv.get('wait_any_share', '')} |")
    lines += ["", f"Kernel code sha256/16 (comments and whitespace removed): `{out['kernel_code_sha256_16']}`", "", "Commands (repository root):", "",
              "```",
              f"rocprofv3 --kernel-trace --stats -d {d}/trace -o run --output-format csv -- "
              f"python3 bench.py --workload {workload} --steps 50 --warmup 50 --no-cpu-baseline --no-configs --no-achievable",
              f"rocprofv3 --pmc FETCH_SIZE -d {d}/fetch -o run --output-format csv -- "
              f"python3 bench.py --workload {workload} --steps 5 --warmup 2 --warmup-ms 0 --no-cpu-baseline --no-configs --no-achievable",
              f"rocprofv3 --pmc WRITE_SIZE -d {d}/write -o run --output-format csv -- "
              f"python3 bench.py --workload {workload} --steps 5 --warmup 2 --warmup-ms 0 --no-cpu-baseline --no-configs --no-achievable",
              f"rocprofv3 --pmc FETCH_SIZE -d {d}/cal_fetch -o run --output-format csv -- python3 bench.py --copy-calibration",
              f"rocprofv3 --pmc WRITE_SIZE -d {d}/cal_write -o run --output-format csv -- python3 bench.py --copy-calibration",
              *[f"rocprofv3 --pmc {' '.join(cs)} -d {d}/{pas} -o run --output-format csv -- python3 bench.py "
                f"--workload {workload} --steps 5 --warmup 2 --warmup-ms 0 --no-cpu-baseline --no-configs --no-achievable"
                for pas, cs in COUNTER_PASSES.items() if os.path.isdir(os.path.join(d, pas))],
              f"python3 bench.py --summarize-profile {d} --workload {workload}",
              "```", ""]
    with open(os.path.join(base, f"mla_split_kv_partial_{workload}.md"), "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(out))


def cpu_baseline(x, max_threads: int):
    """Time the fp64 oracle on all (sequence, token) rows over a prefix of every sequence's keys."""
    import numpy as np

    import oracle

    nproc = os.cpu_count() or 1
    threads = max(1, min(max_threads, nproc, x.B * x.q_len))
    frac = 1.0 if x.name.startswith("agentic") else 0.05
    e = 1 if x.kv_cache.dtype == np.uint8 else 2

    def timed(f, nthreads):
        lens = np.maximum(1, (x.seq_lens.astype(np.int64) * f).astype(np.int64)).astype(np.int32)
        t0 = time.perf_counter()
        oracle.mla_decode(x.q, x.kv_cache, x.block_table, lens, dtype=x.dtype, softmax_scale=x.softmax_scale,
                          q_scale=x.q_scale, kv_scale=x.kv_scale, num_threads=nthreads)
        dt = time.perf_counter() - t0
        return float(lens.astype(np.int64).sum()) * 576 * e / dt / 1e12, int(lens.sum()), dt

    oracle.mla_decode(x.q[:1, :1, :1], x.kv_cache, x.block_table[:1], np.minimum(x.seq_lens[:1], 64), dtype=x.dtype,
                      softmax_scale=x.softmax_scale, q_scale=x.q_scale, kv_scale=x.kv_scale, num_threads=1)
    v, keys, dt = timed(frac, threads)
    # the same rows on one thread, over a quarter of that prefix (the rate is per key)
    v1, keys1, dt1 = timed(frac / 4, 1)
    return {"value": v, "unit": "TB/s", "cores": threads, "nproc": nproc, "kind": "oracle",
            "sample": f"all {x.B * x.q_len} (sequence, query token) rows of the workload, the first {frac:.0%} of "
                      f"each sequence's keys ({keys} keys; a prefix, so the rate is per KV byte read), fp64, "
                      f"{dt:.2f} s wall on {threads} threads of the {nproc} the host reports",
            "value_1core": v1,
            "sample_1core": f"the same rows over the first {frac / 4:.2%} of each sequence's keys ({keys1} keys), "
                            f"one thread, {dt1:.2f} s wall"}


def bench_pack(args):
    """The fused K/V pack + FP8 quantise kernel: T tokens of bf16 latent [512] and rope [64] scattered as
    E4M3 rows into a shuffled cache of T rows (a paged-cache append), K launches back to back."""
    import torch

    import mla_paged_kv_decode_amd as mla

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    T = args.pack_tokens
    g = torch.Generator(device="cpu").manual_seed(7)
    latent = torch.randn(T, 512, generator=g).to(torch.bfloat16).to(dev)
    rope = torch.randn(T, 64, generator=g).to(torch.bfloat16).to(dev)
    slots = torch.randperm(T, generator=g).to(torch.int64).to(dev)
    out = torch.empty(T, 576, dtype=torch.uint8, device=dev)
    kv_scale = float(latent.float().abs().max().item()) / 448.0

    def run():
        mla.kv_pack_quantize_fp8(latent, rope, kv_scale, slot_mapping=slots, out=out)

    warm_up(lambda i: run(), args.warmup, args.warmup_ms)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = T * (512 * 2 + 64 * 2 + 8 + 576)  # read latent, rope, slot; write the row
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "fused K/V pack + FP8 quantise (paged-cache append)", "value": round(gbs, 1),
                      "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": round(ms, 5), "higher_is_better": True, "dtype": "bf16->fp8_e4m3",
                      "data": "synthetic", "config": {"workload": f"kv_pack_{T}_tokens", "tokens": T},
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                                   "algorithmic_bytes_per_launch": nbytes}}), flush=True)


def bench_ragged(args):
    """mla_decode_varlen on a ragged prefill: every sequence's new tokens attend causally to its
    cached keys and to each other.  MFMA-bound: each key row serves many query rows."""
    import numpy as np
    import torch

    import mla_inputs as mi
    import mla_paged_kv_decode_amd as mla

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    x, new = mi.ragged_prefill_inputs(args.workload)
    ctx = mi.RAGGED_PREFILL[args.workload]["ctx"]
    H, dtype = x.H, x.dtype
    lens = [int(v) for v in x.seq_lens]
    B, max_new = len(new), max(new)
    q_pack = np.ascontiguousarray(np.concatenate([x.q[b, :n] for b, n in enumerate(new)], axis=0))
    tdt = torch.float8_e4m3fn if dtype == mi.FP8_E4M3 else torch.bfloat16
    raw = (lambda a: a if a.dtype == np.uint8 else a.view(np.int16))
    q = torch.from_numpy(raw(q_pack)).to(dev).view(tdt)
    kv = torch.from_numpy(raw(x.kv_cache)).to(dev).view(tdt)
    bt = torch.from_numpy(x.block_table).to(dev)
    sl = torch.from_numpy(x.seq_lens).to(dev)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(new)]).astype(np.int32), device=dev)
    total_q = int(sum(new))
    out = torch.empty(total_q, H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(total_q, H, dtype=torch.float32, device=dev)
    G, ws_bytes = mla.plan(B, max_new, H, x.max_seq_len)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    warm = {}

    def timed(stages):
        opts = mla.options(stages=stages)
        run = lambda: mla.decode_varlen(q, cu, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_q_len=max_new,
                                        max_seq_len=x.max_seq_len, out=out, lse=lse, workspace=ws, opts=opts)
        warm[stages] = warm_up(lambda i: run(), args.warmup, args.warmup_ms)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = timed(0)
    part = timed(1)
    vis = sum(max(0, min(L - n + t + 1, L)) for L, n in zip(lens, new) for t in range(n))
    flops = 2 * (576 + 512) * H * vis
    e = 1 if dtype == mi.FP8_E4M3 else 2
    nbytes = sum(lens) * 576 * e + total_q * H * (576 * e + 512 * 2 + 4)
    peak = MFMA_PEAK_TFLOPS[dtype]
    tfs = flops / (part * 1e-3) / 1e12
    print(json.dumps({"metric": "ragged prefill over the paged latent cache (mla_decode_varlen)",
                      "value": round(flops / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warm[0][0],
                      "warmup_ms": round(warm[0][1], 1), "ms_per_step": round(ms, 5),
                      "us_per_step": round(ms * 1e3, 2), "higher_is_better": True, "dtype": DTYPE_NAMES[dtype],
                      "data": "synthetic",
                      "config": {"workload": args.workload, "new_tokens": new, "cached_keys": ctx, "num_heads": H,
                                 "num_splits": G, "page_size": 64},
                      "roofline": {"bound": "mfma", "kernel": "mla_split_kv_partial", "achieved": round(tfs, 1),
                                   "peak": peak, "unit": "TFLOP/s", "frac": round(tfs / peak, 4),
                                   "traffic": load_traffic(args.workload),
                                   "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
                                   "avg_launch_ms": round(part, 5)},
                      "kernels_ms": {"split_kv_partial": round(part, 5)}}), flush=True)


# the five benchmark configurations, in order (the headline is the second: q_len 4, 80K keys, B 4)
CONFIG_WORKLOADS = ["tiny_b1_h16_bf16", "agentic_b4_q4_h32_fp8_80k", "agentic_b16_q4_h32_fp8_80k",
                    "dsv3_b64_q1_h128_bf16_ragged", "spec_b128_q4_h64_fp8_ragged"]
ACHIEVABLE_NOTE = ("rate the split-KV kernel's own load path reaches with no compute on this GPU: the streaming "
                   "probe (global_load_lds_dwordx4 into a 4-tile LDS ring, one 256-thread workgroup per compute "
                   "unit, two 36,864-byte tiles in flight per wave) over a 4 GiB buffer, best of 5 timed passes")
SUM_NOTE = "a plain reduction over the same 4 GiB (torch sum), best of 5: HBM to registers through torch's kernel"
PROBE_PATH = os.path.join(ROOT, "mla_paged_kv_decode_amd", "libmla_stream_probe.so")
PROBE_TILE = 36864


def achievable_read_gbs() -> dict:
    """Streaming read bandwidth with no compute, over a buffer far larger than the 256 MB cache: the
    HBM -> LDS probe built beside the library (the split-KV kernel's load path alone), and a plain
    torch reduction for comparison.  GB/s, best of 5 timed passes after an untimed one."""
    import ctypes

    import torch

    if not os.path.exists(PROBE_PATH):
        raise RuntimeError(f"{PROBE_PATH} is missing: build it with `python -m mla_paged_kv_decode_amd.build`")
    lib = ctypes.CDLL(PROBE_PATH)
    lib.mla_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p]
    lib.mla_stream_probe.restype = ctypes.c_int
    nbytes = ((4 << 30) // PROBE_TILE) * PROBE_TILE
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def best_of(run, nb):
        best = 0.0
        for i in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            if i > 0:
                best = max(best, nb / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        return round(best, 1)

    def probe():
        rc = lib.mla_stream_probe(buf.data_ptr(), nbytes, 0, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"mla_stream_probe failed ({rc})")

    out = {"probe_gbs": best_of(probe, nbytes), "sum_gbs": best_of(lambda: buf.sum(), nbytes)}
    del buf
    torch.cuda.empty_cache()
    return out


def measure_decode(workload: str, args, *, steps: int, warmup: int, warmup_ms: float, with_graph: bool) -> dict:
    """Time one decode workload: K steps back to back (both kernels), then each kernel alone, and with
    with_graph the same steps replayed from one captured HIP graph.  Returns the headline line and a
    compact record for the configs object."""
    import numpy as np
    import torch

    import mla_inputs as mi
    import mla_paged_kv_decode_amd as mla

    dev = torch.device("cuda:0")
    print(f"[bench] generating {workload}", file=sys.stderr, flush=True)
    x = mi.workload_inputs(workload)
    alg = algorithmic(x)
    tdt_of = {mi.BF16: torch.bfloat16, mi.FP16: torch.float16, mi.FP8_E4M3: torch.float8_e4m3fn}
    tq, tdt = tdt_of[mi.q_format(x.dtype)], tdt_of[mi.kv_format(x.dtype)]
    raw_q = x.q if x.q.dtype == np.uint8 else x.q.view(np.int16)
    raw_kv = x.kv_cache if x.kv_cache.dtype == np.uint8 else x.kv_cache.view(np.int16)
    kv0 = torch.from_numpy(raw_kv).to(dev).view(tdt)
    pool_bytes = kv0.numel() * kv0.element_size()
    # enough pool copies that a step never finds its KV in the 256 MB cache, capped for tiny pools
    copies = min(64, max(1, math.ceil(3 * MALL_BYTES / pool_bytes)))
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    q = torch.from_numpy(raw_q).to(dev).view(tq)
    bt = torch.from_numpy(x.block_table).to(dev)
    sl = torch.from_numpy(x.seq_lens).to(dev)
    B, q_len, H = x.B, x.q_len, x.H
    out = torch.empty(B, q_len, H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, q_len, H, dtype=torch.float32, device=dev)
    base_opts = mla.options(num_splits=args.num_splits, partial_fp32=args.partial_fp32, kernel=args.kernel,
                            merge=args.merge)
    num_splits, ws_bytes = mla.plan(B, q_len, H, x.max_seq_len, base_opts)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    del x.kv_cache  # host copy no longer needed (the CPU baseline regenerates if asked)

    calls = {}

    def step(i, stages=0, st=None):
        """Call i of a timed loop (KV copy i % copies); the arguments are marshalled once per (copy, stages,
        stream) so the loop measures the kernels, not the Python binding."""
        key = (i % copies, stages, (st or stream).cuda_stream)
        if key not in calls:
            opts = mla.options(num_splits=args.num_splits, partial_fp32=args.partial_fp32, stages=stages,
                               kernel=args.kernel, merge=args.merge)
            calls[key] = mla.PreparedDecode(q, kvs[i % copies], bt, sl, x.softmax_scale, x.q_scale, x.kv_scale,
                                            max_seq_len=x.max_seq_len, out=out, lse=lse, workspace=ws, opts=opts,
                                            stream=(st or stream).cuda_stream)
        else:
            calls[key]()

    def prepare(stages):
        """Marshal the calls of every pool copy (one untimed launch each) so no timed loop pays for it."""
        for i in range(copies):
            step(i, stages)
        torch.cuda.synchronize()

    def timed_eager(stages, first):
        """K back-to-back calls between two events on the launch stream; ms per call."""
        prepare(stages)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(K):
            step(first + i, stages)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    def timed_graph(stages, first):
        """K calls captured into one HIP graph, replayed between two events on the replay stream: the
        kernels back to back without host launch overhead.  Returns (ms per call, wall seconds)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for i in range(K):
                step(first + i, stages, st=cap)
        torch.cuda.synchronize()
        for _ in range(5):  # untimed replays: the first few of a new graph run slower
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K, time.perf_counter() - t0

    prepare(0)
    n_warm, warm_ms = warm_up(step, warmup, warmup_ms)

    K = steps
    # the step: both kernels, K times back to back (the headline figure)
    t0 = time.perf_counter()
    ms_per_step = timed_eager(0, n_warm)
    wall = time.perf_counter() - t0
    # each kernel alone, back to back, for its roofline (the merge re-merges the partials just written)
    part_avg = timed_eager(1, n_warm + K)
    merge_avg = timed_eager(2, n_warm + 2 * K) if num_splits > 1 else 0.0
    # the same K steps captured into one HIP graph and replayed (reported beside the headline)
    graph_ms = timed_graph(0, n_warm)[0] if with_graph else None

    value = alg["kv_bytes"] / (ms_per_step * 1e-3) / 1e12
    # the split-KV kernel against the roofline that binds it: HBM bytes at 8 TB/s or MFMA flops at
    # the dense peak of its operand type, whichever takes longer; the same for the whole step
    kern_gbs = alg["bytes"] / (part_avg * 1e-3) / 1e9
    kern_tfs = alg["flops"] / (part_avg * 1e-3) / 1e12
    step_gbs = alg["bytes"] / (ms_per_step * 1e-3) / 1e9
    mfma_peak = MFMA_PEAK_TFLOPS[x.dtype]
    mfma_bound = alg["flops"] / (mfma_peak * 1e12) > alg["bytes"] / (HBM_PEAK_GBS * 1e9)
    traffic = load_traffic(workload)
    tflops = alg["flops"] / (ms_per_step * 1e-3) / 1e12
    frac_step = tflops / mfma_peak if mfma_bound else step_gbs / HBM_PEAK_GBS
    pages_us = PAGES_US.get(workload)
    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "warmup_steps_run": n_warm,
        "warmup_ms": round(warm_ms, 1),
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "graph_us_per_step": round(graph_ms * 1e3, 2) if graph_ms is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(pages_us / (ms_per_step * 1e3), 4) if pages_us else None,
        "dtype": DTYPE_NAMES[x.dtype],
        "data": "synthetic",
        "config": {"workload": workload, "batch": B, "q_len": q_len, "num_heads": H, "d_qk": 576, "d_v": 512,
                   "page_size": x.page_size, "max_seq_len": x.max_seq_len,
                   "total_kv_tokens": int(x.seq_lens.astype(np.int64).sum()), "num_splits": num_splits,
                   "kv_pool_copies": copies, "parallelism": "single GPU"},
        # frac: the split-KV kernel alone (its own launches back to back); frac_step: the whole step
        # (both kernels and the gaps between them), the figure the 70 % target is judged on
        "roofline": ({"bound": "mfma", "kernel": "mla_split_kv_partial", "achieved": round(kern_tfs, 1),
                      "peak": mfma_peak, "unit": "TFLOP/s", "frac": round(kern_tfs / mfma_peak, 4)}
                     if mfma_bound else
                     {"bound": "hbm", "kernel": "mla_split_kv_partial", "achieved": round(kern_gbs, 1),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kern_gbs / HBM_PEAK_GBS, 4)})
        | {"traffic": traffic, "frac_step": round(frac_step, 4), "algorithmic_bytes_per_launch": alg["bytes"],
           "algorithmic_flops_per_launch": alg["flops"], "avg_launch_ms": round(part_avg, 5),
           "hbm_frac": round(kern_gbs / HBM_PEAK_GBS, 4), "mfma_frac": round(kern_tfs / mfma_peak, 4)},
        "kernels_ms": {"split_kv_partial": round(part_avg, 5), "merge": round(merge_avg, 5)},
        "tflops": round(tflops, 1),
        "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS[x.dtype], 4),
        "wall_s_timed": round(wall, 4),
    }
    compact = {"us_per_step": round(ms_per_step * 1e3, 2), "kv_tb_s": round(value, 4),
               "bytes_tb_s": round(step_gbs / 1e3, 4), "tflop_s": round(tflops, 1), "dtype": DTYPE_NAMES[x.dtype],
               "bound": "mfma" if mfma_bound else "hbm", "frac_step": round(frac_step, 4),
               "frac_split_kv": line["roofline"]["frac"],
               "kernels_us": {"split_kv": round(part_avg * 1e3, 2), "merge": round(merge_avg * 1e3, 2)},
               "num_splits": num_splits, "steps": K,
               "shape": {"batch": B, "q_len": q_len, "num_heads": H,
                         "total_kv_tokens": int(x.seq_lens.astype(np.int64).sum())}}
    del kvs, kv0, q, bt, sl, out, lse, ws, calls
    return {"line": line, "compact": compact}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warmup-ms", type=float, default=250.0,
                    help="keep warming up until this much wall time has passed (the GPU's clocks settle)")
    ap.add_argument("--workload", default="agentic_b4_q4_h32_fp8_80k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="time only --workload, not every configuration")
    ap.add_argument("--no-achievable", action="store_true", help="skip the streaming-read reference figure")
    ap.add_argument("--cpu-threads", type=int, default=16)
    ap.add_argument("--num-splits", type=int, default=0, help="override the planned KV slice count")
    ap.add_argument("--partial-fp32", action="store_true", help="keep split partials in fp32 (default bf16)")
    ap.add_argument("--kernel", type=int, default=0,
                    help="E4M3 split-KV kernel: 0 default, 1 four-wave, 2 twelve-wave role-specialised")
    ap.add_argument("--merge", type=int, default=0, help="merge kernel: 0 wide (default), 1 workgroup per row")
    ap.add_argument("--copy-calibration", action="store_true", help="run the counter-calibration copy and exit")
    ap.add_argument("--stream-probe", action="store_true",
                    help="print the achievable streaming read rates (HBM -> LDS probe, torch sum) and exit")
    ap.add_argument("--summarize-profile", metavar="DIR", help="summarise rocprofv3 runs under DIR into profiles/")
    ap.add_argument("--pack-tokens", type=int, default=0,
                    help="time the fused K/V pack + FP8 quantise kernel on this many tokens instead of the decode")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.stream_probe:
        print(json.dumps(achievable_read_gbs() | {"probe_note": ACHIEVABLE_NOTE, "sum_note": SUM_NOTE}))
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "sequences are independent, so the decode would shard by batch, each GPU with its own sequences and cache", file=sys.stderr)
        sys.exit(2)
    if args.pack_tokens > 0:
        bench_pack(args)
        return
    if args.workload.startswith("ragged_prefill"):
        bench_ragged(args)
        return

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    head = measure_decode(args.workload, args, steps=args.steps, warmup=args.warmup, warmup_ms=args.warmup_ms,
                          with_graph=True)
    line = head["line"]
    if not args.no_configs:
        # every benchmark configuration, timed the same way (fewer steps; no graph replay)
        line["configs"] = {}
        for name in CONFIG_WORKLOADS:
            if name == args.workload:
                line["configs"][name] = head["compact"]
                continue
            r = measure_decode(name, args, steps=min(args.steps, 20), warmup=min(args.warmup, 10),
                               warmup_ms=min(args.warmup_ms, 100.0), with_graph=False)
            line["configs"][name] = r["compact"]
            torch.cuda.empty_cache()
    if not args.no_achievable:
        ach = achievable_read_gbs()
        rf = line["roofline"]
        rf["achievable_gbs"] = ach["probe_gbs"]
        rf["achievable_note"] = ACHIEVABLE_NOTE
        if rf["unit"] == "GB/s" and ach["probe_gbs"] > 0:
            rf["frac_achievable"] = round(rf["achieved"] / ach["probe_gbs"], 4)
        rf["sum_read_gbs"] = ach["sum_gbs"]
        rf["sum_read_note"] = SUM_NOTE
    if not args.no_cpu_baseline:
        import mla_inputs as mi

        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        xb = mi.workload_inputs(args.workload)
        line["cpu_baseline"] = cpu_baseline(xb, args.cpu_threads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
