#!/usr/bin/env python3
"""Benchmark of blockwise exact causal attention, forward + backward, on one
MI355X.

One step is one pass of the whole path over one batch: attn_fwd (RoPE of q and
k, tile schedule, forward kernel) then attn_bwd (RoPE, tile schedule, dQ and
Delta kernel, dK/dV kernel with the RoPE backward).  Inputs are synthetic and
already resident in HBM when the timed region starts.

Throughput counts algorithmic FLOPs only: 4*D per visible (query, key) pair
for the forward and 10*D for the backward (QK^T recomputed, dP, dV, dK, dQ),
summed over heads; masked pairs are not credited.

Prints one JSON line.  --gpus N with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attention TFLOP/s fwd+bwd (32h×d128, S=32K–1M) and % of bf16 peak"
METRIC_F32 = "causal attention TFLOP/s fwd+bwd, fp32 tensors and fp32 MFMA (32h×d128) and % of fp32 matrix peak"
# MI355X dense bf16 MFMA peak: 256 CUs x 4 SIMDs x 1024 FLOP/clk x 2.4 GHz (the 2.5 PFLOP/s figure)
BF16_PEAK_TFLOPS = 2516.6
# dense fp32 MFMA peak: 256 CUs x 4 SIMDs x 64 FLOP/clk x 2.4 GHz (the 157.3 TFLOP/s figure)
FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
KERNELS = {"rope": 0, "fwd": 1, "bwd_dq": 2, "bwd_dkdv": 3, "decode": 4, "decode_merge": 5,
           "fwd_f32": 6, "bwd_dq_f32": 7, "bwd_dkdv_f32": 8, "packed_ce": 9}
CE_METRIC = "packed cross-entropy loss+gradient HBM GB/s (32768 tokens x 40192 vocab) and % of HBM peak"
DECODE_METRIC = "decode attention HBM GB/s (1M-token KV cache, 32h×d128, one new row) and % of HBM peak"


def visible_pairs(lengths, causal=True):
    """Number of visible (query, key) pairs of one batch row."""
    L = np.asarray(lengths, dtype=np.int64)
    return int(np.sum(L * (L + 1) // 2)) if causal else int(np.sum(L * L))


def row_visible_counts(lengths):
    return np.concatenate([np.arange(1, L + 1, dtype=np.int64) for L in lengths])


def cpu_baseline(w, q, k, v, do, seg, pos, budget_s):
    """Time the oracle (as it stands) on a sample of query rows of head 0:
    forward and backward contributions of those rows.  Returns the dict for
    the JSON line, in TFLOP/s with the same FLOP accounting as the GPU."""
    import oracle

    oracle.build(force=False)
    S, D = w.seqlen, w.head_dim
    lengths = w.extra["lengths"]
    counts = row_visible_counts(lengths)
    q0, k0, v0, d0 = (t[:1, :1].float().cpu().numpy().astype(np.float64) for t in (q, k, v, do))
    seg0 = None if seg is None else seg[:1]
    pos0 = pos[:1]

    def run(n_rows):
        rows = np.unique(np.linspace(0, S - 1, n_rows).astype(np.int64))
        t0 = time.perf_counter()
        oracle.attn_fwd(q0, k0, v0, seg0, pos0, theta=w.theta, causal=w.causal, rows=rows)
        oracle.attn_bwd(q0, k0, v0, d0, seg0, pos0, theta=w.theta, causal=w.causal, rows=rows)
        dt = time.perf_counter() - t0
        flops = 14.0 * D * float(np.sum(counts[rows]))
        return rows, dt, flops

    # grow the sample until one run takes about budget_s / 2 .. budget_s
    n = 16
    rows, dt, flops = run(n)
    while dt < 0.5 * budget_s and n < S:
        n = int(min(S, max(2 * n, n * 0.75 * budget_s / max(dt, 1e-3))))
        rows, dt, flops = run(n)
    model, avail = host_cpu()
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "cpu_model": model,
        "host_cores_available": avail,
        "kind": "oracle",
        "extrapolated": True,  # a rate measured on the sample, taken for the whole workload
        "sample": "fwd+bwd of %d evenly spaced query rows of head 0 (of %d rows x %d heads), %.1f s; "
                  "credited 14*D FLOPs per visible pair of those rows" % (len(rows), S, w.heads, dt),
        "seconds": dt,
    }


# rocprofv3 kernel-name fragments of the timed kernels
KERNEL_SYMBOLS = {"fwd": "attn_fwd_kernel", "bwd_dq": "attn_bwd_dq_kernel", "bwd_dkdv": "attn_bwd_dkdv_kernel",
                  "decode": "attn_decode_partial_kernel", "fwd_f32": "attn_fwd_f32_kernel",
                  "bwd_dq_f32": "attn_bwd_dq_f32_kernel", "bwd_dkdv_f32": "attn_bwd_dkdv_f32_kernel",
                  "packed_ce": "ce_row_kernel"}


# the sources each measured kernel family is built from: its own file, the
# headers it includes, the pre-pass whose tables it reads, and the build
# flags.  A stored record applies while these hash the same.
_HEADERS = ["common.hpp", "kernels.hpp"]
KERNEL_SOURCES = {
    "attention": ["attn_fwd.hip", "attn_bwd.hip", "prep.hip", "tile.hpp"] + _HEADERS + ["../build.py"],
    "f32": ["attn_f32.hip", "prep.hip", "tile.hpp"] + _HEADERS + ["../build.py"],
    "decode": ["attn_decode.hip", "prep.hip", "tile.hpp"] + _HEADERS + ["../build.py"],
    "packed_ce": ["packed_ce.hip"] + _HEADERS + ["../build.py"],
}


def kernel_family(kernel):
    if kernel.endswith("_f32"):
        return "f32"
    if kernel.startswith("decode"):
        return "decode"
    if kernel == "packed_ce":
        return "packed_ce"
    return "attention"


def kernel_source_hash(family):
    """sha256 over the sources of one kernel family: a traffic or counter
    record is only used while the kernels are the ones it was measured on."""
    import hashlib

    d = os.path.join(ROOT, "long_context_blockwise_attn_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        h.update(name.encode())
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)


def counter_rows(path, counter):
    """(kernel name, dispatch id, value) of one counter from a rocprofv3
    counter_collection CSV, in dispatch order."""
    import csv

    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    out.sort(key=lambda x: x[1])
    return out


def write_traffic_record(workload, fetch_csv, write_csv, copy_mib, command):
    """HBM bytes per launch of each timed kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by the
    factor that makes the last plain copy of the run (copy_mib MiB read and
    written) read exactly its size."""
    rec = {"workload": workload, "command": command, "kernels": {}}
    copy_bytes = float(copy_mib) * (1 << 20)
    for counter, path, key in (("FETCH_SIZE", fetch_csv, "read"), ("WRITE_SIZE", write_csv, "write")):
        rows = counter_rows(path, counter)
        copies = [r for r in rows if "copy" in r[0].lower()]
        if not copies:
            raise SystemExit("no copy kernel in %s" % path)
        cal_kib = copies[-1][2]
        factor = copy_bytes / (cal_kib * 1024.0)
        rec["%s_calibration" % key] = {"copy_bytes": copy_bytes, "counter_kib": cal_kib, "factor": factor}
        for name, sym in KERNEL_SYMBOLS.items():
            vals = [r[2] for r in rows if sym in r[0]]
            if vals:
                k = rec["kernels"].setdefault(name, {})
                k["%s_counter_kib" % key] = float(np.mean(vals))
                k["%s_bytes" % key] = float(np.mean(vals)) * 1024.0 * factor
                k["dispatches"] = len(vals)
    for name, k in rec["kernels"].items():
        k["traffic_bytes"] = k.get("read_bytes", 0.0) + k.get("write_bytes", 0.0)
        k["source_sha256"] = kernel_source_hash(kernel_family(name))
    with open(traffic_path(workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def load_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the stored record, or None when
    there is none or the kernels changed since it was measured."""
    try:
        with open(traffic_path(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if k is None or k.get("source_sha256") != kernel_source_hash(kernel_family(kernel)):
        return None
    return k.get("traffic_bytes")


def counters_path(workload):
    return os.path.join(ROOT, "profiles", "counters_%s.json" % workload)


# MFMA instruction counters: the hardware counts matrix work in units of 512
# FLOPs ("MOPS"); one counter per data type
MOPS_COUNTER = {"bf16": "SQ_INSTS_VALU_MFMA_MOPS_BF16", "f32": "SQ_INSTS_VALU_MFMA_MOPS_F32"}


def write_counter_record(workload, csvs, command, simds=1024, xcds=8):
    """Per-dispatch averages of every counter in the rocprofv3 --pmc CSVs
    (one pass each) for the timed kernels, with the kernel sources' hash, the
    dispatches' own durations (from the CSV timestamps) and what follows from
    them:
      - GRBM_GUI_ACTIVE counts the busy cycles of each of the `xcds`
        dies, so GRBM_GUI_ACTIVE / xcds / duration is the clock the kernel
        ran at;
      - SQ_VALU_MFMA_BUSY_CYCLES sums the matrix units' busy cycles over the
        `simds` SIMDs, so its share of simds x those cycles is the MFMA
        utilisation at that clock;
      - SQ_INSTS_VALU_MFMA_MOPS_BF16 (_F32) counts MFMA work in units of 512
        FLOPs."""
    import csv

    rec = {"workload": workload, "command": command, "simds": simds, "xcds": xcds, "kernels": {}}
    for path in csvs:
        rows, durs = {}, {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                rows.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
                durs.setdefault(r["Kernel_Name"], {})[r["Dispatch_Id"]] = (
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        for (kname, counter), vals in rows.items():
            for name, sym in KERNEL_SYMBOLS.items():
                if sym in kname:
                    k = rec["kernels"].setdefault(name, {})
                    k[counter] = float(np.mean(vals))
                    k.setdefault("dispatches", {})[counter] = len(vals)
                    k.setdefault("pmc_run_ms", {})[os.path.basename(path)] = 1e3 * float(
                        np.mean(list(durs[kname].values())))
    for name, k in rec["kernels"].items():
        k["source_sha256"] = kernel_source_hash(kernel_family(name))
        ms = float(np.mean(list(k["pmc_run_ms"].values())))
        if "GRBM_GUI_ACTIVE" in k:
            cycles = k["GRBM_GUI_ACTIVE"] / xcds
            k["clock_ghz"] = cycles / (ms * 1e-3) / 1e9
            if "SQ_VALU_MFMA_BUSY_CYCLES" in k:
                k["mfma_util_at_clock"] = k["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cycles)
    with open(counters_path(workload), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def load_counters(workload, kernel, avg_ms, peak):
    """Matrix-unit figures of `kernel` from the stored counter record (None
    when there is none or the kernels changed since it was taken): the MFMA
    FLOPs the hardware counted per launch and their rate over the live
    average launch time, against the dtype's peak; the clock the kernel ran
    at in the counter run and the MFMA utilisation at that clock; the raw
    counters per launch (VALU activity, LDS bank conflicts)."""
    try:
        with open(counters_path(workload)) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_sha256") != kernel_source_hash(kernel_family(kernel)):
        return None
    dtype = "f32" if kernel.endswith("_f32") else "bf16"
    out = {"source": os.path.relpath(counters_path(workload), ROOT)}
    mops = k.get(MOPS_COUNTER[dtype])
    if mops is not None:
        flops = 512.0 * mops
        out["mfma_flops_per_launch"] = flops
        out["mfma_tflops"] = flops / (avg_ms * 1e-3) / 1e12
        out["mfma_frac"] = out["mfma_tflops"] / peak
    for c in ("clock_ghz", "mfma_util_at_clock", "GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
              "SQ_ACTIVE_INST_VALU", "SQ_LDS_BANK_CONFLICT"):
        if c in k:
            out[c] = k[c]
    return out


def host_cpu():
    """CPU model of this host and the number of cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def event_arrays(lib, torch, names, n_each):
    """Ask the library to bracket the next n_each[name] launches of each
    kernel with HIP events on the launch stream."""
    ev, keep = {}, []
    for name in names:
        n = n_each[name]
        st = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        sp = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in st + sp:
            e.record()  # torch creates the underlying HIP event on first record
        torch.cuda.synchronize()
        arr_t = (ctypes.c_void_p * n)(*[e.cuda_event for e in st])
        arr_p = (ctypes.c_void_p * n)(*[e.cuda_event for e in sp])
        keep += [arr_t, arr_p]
        assert lib.attn_profile_events(KERNELS[name], arr_t, arr_p, n) == 0
        ev[name] = (st, sp)
    return ev, keep


def decode_bench(args, w):
    """One step = one attn_decode call: the n_q new rows of every (b,h)
    against the whole cache (keys already rotated, as a cache holds them).
    Throughput = algorithmic bytes (the K and V cache read once, q and o) per
    second; the path is bound by HBM."""
    import torch

    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import randn_bf16

    dev = torch.device("cuda:0")
    B, H, S, D, nq = w.batch, w.heads, w.seqlen, w.head_dim, w.extra["n_q"]
    q = randn_bf16((B, H, nq, D), w.seed * 16, dev)
    k = randn_bf16((B, H, S, D), w.seed * 16 + 1, dev)
    v = randn_bf16((B, H, S, D), w.seed * 16 + 2, dev)
    kc = bw.rope_apply(k, None, theta=w.theta)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
    p = bw.make_params(B, H, S, D, theta=w.theta, causal=w.causal)
    ws = torch.empty(bw.decode_workspace_bytes(p, nq), dtype=torch.uint8, device=dev)

    def step():
        bw.attn_decode(q, kc, v, None, theta=w.theta, causal=w.causal, out=o, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    lib = bw.load()
    ev, keep = event_arrays(lib, torch, ["decode", "decode_merge"], {"decode": args.steps, "decode_merge": args.steps})
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    kernel_ms = {}
    for name, (st, sp) in ev.items():
        cnt = lib.attn_profile_count(KERNELS[name])
        kernel_ms[name] = float(np.mean([a.elapsed_time(b) for a, b in zip(st[:cnt], sp[:cnt])]))
        lib.attn_profile_events(KERNELS[name], None, None, 0)

    cache_bytes = 2.0 * B * H * S * D * 2
    step_bytes = cache_bytes + 2.0 * B * H * nq * D * 2 + B * H * nq * 4
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    part_bytes = cache_bytes + B * H * nq * D * 2  # the partial kernel reads the cache and the rotated rows
    part_gbs = part_bytes / (kernel_ms["decode"] * 1e-3) / 1e9
    roofline = {"kernel": "decode", "bound": "hbm", "achieved": part_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": part_gbs / HBM_PEAK_GBS, "traffic": load_traffic(w.name, "decode"),
                "traffic_unit": "HBM bytes per launch", "bytes_per_launch": part_bytes}

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        rows = np.arange(S - nq, S, dtype=np.int64)
        qh = np.zeros((1, 1, S, D))
        qh[0, 0, S - nq:] = q[:1, :1].float().cpu().numpy()[0, 0]
        kh = k[:1, :1].float().cpu().numpy().astype(np.float64)
        vh = v[:1, :1].float().cpu().numpy().astype(np.float64)
        reps, dt = 0, 0.0
        t_start = time.perf_counter()
        while dt < 0.5 * args.cpu_seconds or reps == 0:
            oracle.attn_fwd(qh, kh, vh, None, None, theta=w.theta, causal=w.causal, rows=rows)
            reps += 1
            dt = time.perf_counter() - t_start
        head_bytes = 2.0 * S * D * 2 + 2.0 * nq * D * 2 + nq * 4
        model, avail = host_cpu()
        cpu = {"value": reps * head_bytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
               "cpu_model": model, "host_cores_available": avail, "kind": "oracle", "extrapolated": True,
               "sample": "%d oracle calls on head 0 of %d (the n_q rows against its whole cache, K rotated inside), "
                         "%.1f s; credited that head's bf16 cache bytes per call" % (reps, H, dt),
               "seconds": dt}

    out = {
        "metric": DECODE_METRIC,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "head_dim": D, "cache_len": S, "n_q": nq,
                   "rope_theta": w.theta, "mask": "causal" if w.causal else "none", "parallelism": "single GPU"},
        "pct_of_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
        "kernels_ms": {n: round(t, 4) for n, t in kernel_ms.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    del keep


def packed_ce_bench(args, w):
    """One step = one packed_ce_loss call over the packed rows: loss, per-row
    weights and the bf16 gradient of every row.  Algorithmic bytes: the
    logits of loss rows read once, the gradient of every row written once,
    targets and example ids read once; the path is bound by HBM."""
    import torch

    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import packed_ce_case

    dev = torch.device("cuda:0")
    logits, targets, seg, ne = packed_ce_case(w, device=dev)
    B, S, V = logits.shape
    N = B * S
    dl = torch.empty_like(logits)
    ws = torch.empty(bw.packed_ce_workspace_bytes(bw.make_ce_params(B, S, V, ne)), dtype=torch.uint8, device=dev)
    n_loss = int(((targets >= 0) & (targets < V)).sum().item())

    def step():
        bw.packed_ce_loss(logits, targets, seg, ne, dlogits=dl, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    lib = bw.load()
    ev, keep = event_arrays(lib, torch, ["packed_ce"], {"packed_ce": args.steps})
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    st, sp = ev["packed_ce"]
    cnt = lib.attn_profile_count(KERNELS["packed_ce"])
    row_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(st[:cnt], sp[:cnt])]))
    lib.attn_profile_events(KERNELS["packed_ce"], None, None, 0)

    row_bytes = 2.0 * n_loss * V + 2.0 * N * V + 8.0 * N  # loss-row logits, every gradient row, targets + ids
    step_bytes = row_bytes + 8.0 * N  # + counting pass (targets, ids)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    row_gbs = row_bytes / (row_ms * 1e-3) / 1e9
    roofline = {"kernel": "packed_ce", "bound": "hbm", "achieved": row_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": row_gbs / HBM_PEAK_GBS, "traffic": load_traffic(w.name, "packed_ce"),
                "traffic_unit": "HBM bytes per launch", "bytes_per_launch": row_bytes}

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        # the oracle on the first n rows (their examples as they stand), n
        # doubled until one call takes about half the budget
        tg = targets.cpu().numpy().reshape(-1)
        sg = seg.cpu().numpy()
        n, dt = 64, 0.0
        while True:
            x = logits[0, :n].float().cpu().numpy()
            t_start = time.perf_counter()
            oracle.packed_ce(x, tg[:n], sg[:, :n], ne)
            dt = time.perf_counter() - t_start
            if dt >= 0.5 * args.cpu_seconds or n >= S:
                break
            n = min(S, 2 * n)
        nl = int(((tg[:n] >= 0) & (tg[:n] < V)).sum())
        sample_bytes = 2.0 * nl * V + 2.0 * n * V + 8.0 * n
        model, avail = host_cpu()
        cpu = {"value": sample_bytes / dt / 1e9, "unit": "GB/s", "cores": 1, "cpu_model": model,
               "host_cores_available": avail, "kind": "oracle", "extrapolated": True,
               "sample": "the first %d rows (%d loss rows) of the packed row, loss and full gradient, %.1f s; "
                         "credited the same bytes per row as the GPU" % (n, nl, dt),
               "seconds": dt}

    out = {
        "metric": CE_METRIC,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": S, "vocab": V, "examples": ne, "loss_rows": n_loss,
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
        "kernels_ms": {"packed_ce": round(row_ms, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    del keep


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="packing_128k",
                    help="packing_128k (default: 128K of packed documents, causal + segment mask), llama7b_32k, "
                         "video_text_256k, full_1m, tiny, decode_1m (attn_decode; HBM GB/s), packed_ce_32k "
                         "(packed_ce_loss; HBM GB/s)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f32"],
                    help="bf16 (default: attn_fwd/attn_bwd) or f32 (attn_fwd_f32/attn_bwd_f32 on fp32 tensors)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=24.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic record of --workload from two rocprofv3 --pmc counter CSVs "
                         "(FETCH_SIZE, WRITE_SIZE) of runs made with --copy-calibration-mib, then exit")
    ap.add_argument("--traffic-command", default="", help="command line recorded with --traffic-from")
    ap.add_argument("--counters-from", nargs="+", metavar="PMC_CSV",
                    help="write the counter record of --workload (profiles/counters_<workload>.json) from rocprofv3 "
                         "--pmc counter CSVs, then exit")
    args = ap.parse_args()

    if args.counters_from:
        write_counter_record(args.workload + ("_f32" if args.dtype == "f32" else ""), args.counters_from,
                             args.traffic_command)
        return

    if args.traffic_from:
        # one record per workload and dtype (profiles/traffic_<workload>[_f32].json)
        write_traffic_record(args.workload + ("_f32" if args.dtype == "f32" else ""), args.traffic_from[0],
                             args.traffic_from[1], args.copy_calibration_mib or 1024, args.traffic_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (asked for %d GPUs)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import WORKLOADS, make_qkv, packing

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    if "n_q" in w.extra:
        decode_bench(args, w)
        return
    if "vocab" in w.extra:
        packed_ce_bench(args, w)
        return
    B, H, S, D = w.batch, w.heads, w.seqlen, w.head_dim
    f32 = args.dtype == "f32"
    seg_np, pos_np, lengths = packing(w)
    w.extra["lengths"] = lengths
    q, k, v, do = make_qkv(w, device=dev, with_grad_out=True, dtype="fp32" if f32 else "bf16")
    seg = None if seg_np is None else torch.from_numpy(seg_np).to(dev)
    pos = torch.from_numpy(pos_np).to(dev)
    do_bwd = w.backward

    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    pf = bw.make_params(B, H, S, D, theta=w.theta, causal=w.causal, kv_chunk=w.kv_chunk)
    ws_f = torch.empty(bw.workspace_bytes(pf, 2 if f32 else 0), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bw.workspace_bytes(pf, 3 if f32 else 1), dtype=torch.uint8, device=dev)
    fwd_fn, bwd_fn = (bw.attn_fwd_f32, bw.attn_bwd_f32) if f32 else (bw.attn_fwd, bw.attn_bwd)
    sfx = "_f32" if f32 else ""  # measurement-hook names of the kernels of this dtype

    def step():
        fwd_fn(q, k, v, seg, pos, theta=w.theta, causal=w.causal, kv_chunk=w.kv_chunk, out=o, lse=lse,
               workspace=ws_f)
        if do_bwd:
            bwd_fn(q, k, v, o, lse, do, seg, pos, theta=w.theta, causal=w.causal, kv_chunk=w.kv_chunk, dq=dq,
                   dk=dk, dv=dv, workspace=ws_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # live per-kernel timing: HIP events recorded by the library around each
    # launch, on the launch stream, over the timed region
    lib = bw.load()
    # RoPE pre-pass launches per step: the bf16 forward rotates k (its query
    # rows are rotated in the kernel's load), the bf16 backward writes q''
    # (rotated and scaled, also without RoPE) and k'; the fp32 path rotates q
    # and k in both passes, and nothing without RoPE
    if f32:
        rope_launches = (4 if do_bwd else 2) if w.theta > 0 else 0
    else:
        rope_launches = (1 if w.theta > 0 else 0) + ((2 if w.theta > 0 else 1) if do_bwd else 0)
    launches = {"rope": rope_launches, "fwd": 1, "bwd_dq": 1 if do_bwd else 0, "bwd_dkdv": 1 if do_bwd else 0}
    ev = {}
    keep = []
    for name, per in launches.items():
        n = per * args.steps
        if n == 0:
            continue
        st = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        sp = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in st + sp:
            e.record()  # torch creates the underlying HIP event on first record
        torch.cuda.synchronize()
        arr_t = (ctypes.c_void_p * n)(*[e.cuda_event for e in st])
        arr_p = (ctypes.c_void_p * n)(*[e.cuda_event for e in sp])
        keep += [arr_t, arr_p]
        rc = lib.attn_profile_events(KERNELS[name if name == "rope" else name + sfx], arr_t, arr_p, n)
        assert rc == 0
        ev[name] = (st, sp)

    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    kernel_ms = {}
    for name, (st, sp) in ev.items():
        kid = KERNELS[name if name == "rope" else name + sfx]
        cnt = lib.attn_profile_count(kid)
        times = [a.elapsed_time(b) for a, b in zip(st[:cnt], sp[:cnt])]
        kernel_ms[name] = {"avg_ms": float(np.mean(times)), "median_ms": float(np.median(times)),
                           "min_ms": float(np.min(times)), "launches_per_step": launches[name],
                           "launches_timed": cnt}
        lib.attn_profile_events(kid, None, None, 0)

    pairs = B * visible_pairs(lengths, w.causal)
    fwd_flops = 4.0 * D * H * pairs
    bwd_flops = 10.0 * D * H * pairs if do_bwd else 0.0
    tflops = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12

    # dominant kernel and its roofline (MFMA bound).  Each kernel is credited
    # the method's contractions it performs, 2*D FLOPs per visible pair each:
    # fwd 2 (QK^T, PV), dK/dV 4 (QK^T recomputed, dP, dV, dK), dQ 1 (dQ); the
    # dQ kernel also executes QK^T and dP again (3 in all), which the method's
    # 10*D backward does not count, so its executed fraction is given apart
    credited = {"fwd": 2, "bwd_dq": 1, "bwd_dkdv": 4}
    executed = {"fwd": 2, "bwd_dq": 3, "bwd_dkdv": 4}
    peak = FP32_PEAK_TFLOPS if f32 else BF16_PEAK_TFLOPS
    per_kernel = {}
    for n in credited:
        if n in kernel_ms:
            t = kernel_ms[n]["avg_ms"] * 1e-3
            per_kernel[n] = {"ms": round(kernel_ms[n]["avg_ms"], 4),
                             "ms_median": round(kernel_ms[n]["median_ms"], 4),
                             "ms_min": round(kernel_ms[n]["min_ms"], 4),
                             "frac": credited[n] * 2.0 * D * H * pairs / t / 1e12 / peak,
                             "executed_frac": executed[n] * 2.0 * D * H * pairs / t / 1e12 / peak}
    dom = max((n for n in credited if n in kernel_ms),
              key=lambda n: kernel_ms[n]["avg_ms"] * kernel_ms[n]["launches_per_step"])
    dom_flops = credited[dom] * 2.0 * D * H * pairs
    dom_tflops = dom_flops / (kernel_ms[dom]["avg_ms"] * 1e-3) / 1e12
    roofline = {"kernel": dom + sfx, "bound": "mfma", "achieved": dom_tflops, "peak": peak, "unit": "TFLOP/s",
                "frac": dom_tflops / peak, "traffic": load_traffic(w.name + sfx, dom + sfx),
                "traffic_unit": "HBM bytes per launch", "flops_per_launch": dom_flops,
                "executed_flops_per_launch": executed[dom] * 2.0 * D * H * pairs,
                "counters": load_counters(w.name + sfx, dom + sfx, kernel_ms[dom]["avg_ms"], peak),
                "kernels": per_kernel}

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v, do, seg_np, pos_np, args.cpu_seconds)

    mask = "causal" + ("+segment" if seg_np is not None else "")
    out = {
        "metric": METRIC_F32 if f32 else METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if f32 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "head_dim": D, "seq_len": S, "rope_theta": w.theta,
                   "mask": mask, "kv_chunk": w.kv_chunk, "pass": "fwd+bwd" if do_bwd else "fwd",
                   "visible_pairs": pairs, "parallelism": "single GPU"},
        ("pct_of_fp32_peak" if f32 else "pct_of_bf16_peak"): 100.0 * tflops / peak,
        # the method's forward and backward FLOPs over their kernels' average
        # times (the RoPE pre-passes not included)
        "fwd_tflops": fwd_flops / (kernel_ms["fwd"]["avg_ms"] * 1e-3) / 1e12,
        "bwd_tflops": (bwd_flops / ((kernel_ms["bwd_dq"]["avg_ms"] + kernel_ms["bwd_dkdv"]["avg_ms"]) * 1e-3) / 1e12
                       if do_bwd else None),
        "kernels_ms": {n: round(v["avg_ms"], 4) for n, v in kernel_ms.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
