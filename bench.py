#!/usr/bin/env python3
"""Throughput of gated GQA causal attention on one MI355X.

One step is one whole prefill pass (ga_prefill: the K-hat kernel, then the
fused attention kernel) over the paper-MoE-shaped long-context workload
(B=1, n=32768, H=32, G=4, d=128, RoPE on 32 dims, elementwise gate, bf16),
the largest single-GPU configuration. The other workloads are measured in the
same run as extra objects: the Qwen3.5-0.8B-shaped prefill (4096 tokens,
8/2/256), the Qwen3-0.6B-shaped batched prefill (4 x 2048, 16/8/128,
headwise gate), the fp32 toy (latency), decode over 64 long caches (GB/s),
and the adjacent paths (chunked prefill, fused [q | gate] input, a gate
variant, the backward).

Printed: one JSON line. ``value`` is prefill TFLOP/s counting only the
unmasked causal work 2*B*H*d*n*(n+1); ``roofline`` relates the attention
kernel's own duration (K launches back to back on its stream between two HIP
events, median of 5 such samples) to the bf16 dense MFMA peak;
``cpu_baseline`` times the fp64 CPU oracle on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HEADLINE = "moe_long_context_prefill"
EXTRA_PREFILL = {"qwen35_0p8b_prefill": 100, "qwen3_0p6b_batched_prefill": 100}  # workload: K launches per sample
VARIANT_WORKLOAD = "qwen35_0p8b_prefill"  # fused-input, gate-variant and backward measurements
MI355X_BF16_DENSE_TFLOPS = 2500.0
MI355X_HBM_GBS = 8000.0
METRIC = "gated GQA attn fwd TFLOP/s (prefill) + decode KV GB/s, % of MI355X roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE,
                    help="prefill workload of the headline line (default: the 32K-token one)")
    ap.add_argument("--only", action="store_true",
                    help="the headline prefill only (for profiler runs)")
    ap.add_argument("--no-extra-prefill", action="store_true",
                    help="skip the other prefill workloads and the toy")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-chunk", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-packed", action="store_true", help="skip the fused [q | gate] input measurement")
    ap.add_argument("--no-variant", action="store_true", help="skip the gate-variant epilogue measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--no-prefill", action="store_true", help="decode only (for counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--samples", type=int, default=5, help="timed samples of K launches (median reported)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--record-traffic", nargs=6,
                    metavar=("KERNEL", "WORKLOAD", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "counter_collection.csv files of a bench run and of a --copy-calibration run")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "gated_gqa_softmax_amd", "csrc")
# symbol of the kernel behind each name ga_prefill_attention_kernel returns
PREFILL_KERNEL_SYMBOL = {"wide": "prefill_wide_kernel", "mirror": "prefill_v2_kernel",
                         "simple": "prefill_mfma_kernel", "generic": "naive_kernel"}
KERNEL_SOURCES = {
    "prefill_v2_kernel": ["ga_prefill_v2.hip", "ga_prefill_tile.hpp", "ga_gate.hpp", "ga_common.hpp",
                          "ga_internal.hpp"],
    "prefill_wide_kernel": ["ga_prefill_wide.hip", "ga_prefill_tile.hpp", "ga_gate.hpp", "ga_common.hpp",
                            "ga_internal.hpp"],
    "decode_partials_kernel": ["ga_decode.hip", "ga_gate.hpp", "ga_common.hpp", "ga_internal.hpp"],
    "prefill_mfma_kernel": ["ga_prefill_mfma.hip", "ga_gate.hpp", "ga_common.hpp", "ga_internal.hpp"],
    "naive_kernel": ["ga_naive.hip", "ga_common.hpp", "ga_internal.hpp"],
}


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/hbm_traffic.json (rocprofv3 FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy of known size), or None when the record is
    missing or was measured on a different version of the kernel's source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[f"{kernel}@{workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"]


COPY_BYTES = 1 << 30
COPY_KERNEL = "neg_kernel"


def copy_calibration(torch):
    """A plain elementwise pass (y = -x, bf16) that reads and writes COPY_BYTES each."""
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": COPY_BYTES, "copy_calibration_bytes_written": COPY_BYTES,
                      "launches": 5}))


def counter_per_dispatch(csv_path: str, kernel: str, counter: str) -> float:
    """Mean over dispatches of one rocprofv3 counter (summed over its instances)
    for the kernels whose name contains `kernel`."""
    import csv
    per, names = {}, set()
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
                names.add(r["Kernel_Name"])
    if not per:
        raise SystemExit(f"{csv_path}: no {counter} rows for a kernel named *{kernel}*")
    if len(names) > 1:
        raise SystemExit(f"{csv_path}: *{kernel}* matches several kernels ({sorted(names)}); "
                         "profile a run with only the one workload")
    return sum(per.values()) / len(per)


def record_traffic(kernel, workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    fetch = counter_per_dispatch(fetch_csv, kernel, "FETCH_SIZE")
    write = counter_per_dispatch(write_csv, kernel, "WRITE_SIZE")
    cf = counter_per_dispatch(copy_fetch_csv, COPY_KERNEL, "FETCH_SIZE")
    cw = counter_per_dispatch(copy_write_csv, COPY_KERNEL, "WRITE_SIZE")
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            db = json.load(f)
    except (OSError, ValueError):
        db = {}
    rec = {"source_sha256": source_digest(kernel), "fetch_kib": fetch, "write_kib": write,
           "fetch_scale": COPY_BYTES / 1024 / cf, "write_scale": COPY_BYTES / 1024 / cw,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": COPY_BYTES}
    rec["bytes_per_launch"] = fetch * 1024 * rec["fetch_scale"] + write * 1024 * rec["write_scale"]
    db[f"{kernel}@{workload}"] = rec
    with open(path, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({f"{kernel}@{workload}": rec}))


def ramp(torch, fn, seconds=0.25):
    """Keep the GPU busy with untimed calls for a moment after the warmup
    steps: a handful of calls that follow seconds of host-side input
    generation still run at lower clocks (measured: +7 us on a 90 us step)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def timed_ms(torch, fn, stream, k, samples):
    """Median over ``samples`` of the mean ms per call of ``k`` calls of
    ``fn`` back to back between two HIP events on ``stream`` (each sample
    bracketed by synchronisations); also returns every sample."""
    res = []
    for _ in range(samples):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / k)
    return float(np.median(res)), res


def time_whole_and_kernel(torch, whole, attention, stream, steps, warmup, samples=5):
    """Median ms of ``whole`` (one step) and of ``attention`` (the attention
    kernel's launch), each from ``samples`` samples of ``steps`` calls."""
    for _ in range(warmup):
        whole()
    ramp(torch, whole)
    step_ms, step_s = timed_ms(torch, whole, stream, steps, samples)
    kernel_ms, kernel_s = timed_ms(torch, attention, stream, steps, samples)
    return {"step_ms": step_ms, "kernel_ms": kernel_ms, "step_samples_ms": step_s, "kernel_samples_ms": kernel_s}


def time_prefill(torch, api, inputs, accounting, wname, steps, warmup, samples=5):
    """Whole ga_prefill steps and the attention launch alone on one prefill workload."""
    w = inputs.WORKLOADS[wname]
    x = inputs.make_prefill(w)
    et = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dv = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt) if a is not None else None
    q, k, v = dv(x["q"], et), dv(x["k"], et), dv(x["v"], et)
    gate = dv(x["gate"], et)
    wq, wk, pos = dv(x["q_norm_w"]), dv(x["k_norm_w"]), dv(x["positions"])
    d = api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rot_dim, w.rope_base, w.rms_eps, 0.0, et,
                      w.gate_mode)
    khat = api.ga_prefill_keys(d, k, None, wk, pos)
    out = torch.empty((w.batch, w.seq_len, w.n_q_heads * w.head_dim), dtype=et, device="cuda")
    ws = torch.empty(api.ga_prefill_workspace_bytes(d, w.seq_len), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def whole():
        api.ga_prefill(d, q, k, v, gate, wq, wk, pos, out=out, workspace=ws, stream=stream)

    def attention():
        api.ga_prefill_attention(d, q, khat, v, gate, wq, pos, out=out, stream=stream, k_norm_w=wk)

    t0 = time.perf_counter()
    res = time_whole_and_kernel(torch, whole, attention, stream, steps, warmup, samples)
    wall = time.perf_counter() - t0
    kernel = PREFILL_KERNEL_SYMBOL[api.ga_prefill_attention_kernel(d, w.seq_len)]
    flops = accounting.causal_prefill_flops(w.batch, w.n_q_heads, w.head_dim, w.seq_len)
    del q, k, v, gate, khat, out, ws
    return dict(w=w, x=x, flops=flops, attn_ms=res["kernel_ms"], kernel=kernel, step_ms=res["step_ms"],
                step_samples_ms=res["step_samples_ms"], kernel_samples_ms=res["kernel_samples_ms"], wall_s=wall)


def prefill_config(w):
    return {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "n_q_heads": w.n_q_heads,
            "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "rot_dim": w.rot_dim, "gate": w.gate_mode}


def prefill_roofline(pre):
    w = pre["w"]
    achieved = pre["flops"] / (pre["attn_ms"] * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": pre["kernel"], "achieved": achieved, "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / MI355X_BF16_DENSE_TFLOPS,
            "traffic": measured_traffic(pre["kernel"], w.name), "kernel_ms": pre["attn_ms"],
            "kernel_samples_ms": pre["kernel_samples_ms"], "algorithmic_flops": pre["flops"]}


def prefill_object(pre, steps):
    return {"metric": METRIC, "value": pre["flops"] / (pre["step_ms"] * 1e-3) / 1e12, "unit": "TFLOP/s",
            "ms_per_step": pre["step_ms"], "step_samples_ms": pre["step_samples_ms"], "steps": steps,
            "dtype": "bf16" if pre["w"].dtype == "bf16" else "f32", "config": prefill_config(pre["w"]),
            "roofline": prefill_roofline(pre)}


def time_toy(torch, api, inputs, steps, warmup, samples=5):
    """The fp32 toy workload: latency of one whole ga_prefill call (8.7 kflop:
    launch-bound; no roofline claim)."""
    w = inputs.WORKLOADS["toy"]
    x = inputs.make_prefill(w)
    dv = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)
    f = torch.float32
    q, k, v, gate = dv(x["q"], f), dv(x["k"], f), dv(x["v"], f), dv(x["gate"], f)
    wq, wk, pos = dv(x["q_norm_w"]), dv(x["k_norm_w"]), dv(x["positions"])
    d = api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rot_dim, w.rope_base, w.rms_eps, 0.0, f,
                      w.gate_mode)
    out = torch.empty((w.batch, w.seq_len, w.n_q_heads * w.head_dim), dtype=f, device="cuda")
    ws = torch.empty(max(1, api.ga_prefill_workspace_bytes(d, w.seq_len)), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def whole():
        api.ga_prefill(d, q, k, v, gate, wq, wk, pos, out=out, workspace=ws, stream=stream)

    for _ in range(warmup):
        whole()
    ms, samples_ms = timed_ms(torch, whole, stream, steps, samples)
    return {"metric": "toy prefill latency", "value": ms * 1e3, "unit": "us per call", "higher_is_better": False,
            "samples_us": [t * 1e3 for t in samples_ms], "steps": steps, "dtype": "f32",
            "config": prefill_config(w), "kernel": api.ga_prefill_attention_kernel(d, w.seq_len),
            "note": "two launches (K-hat, attention) per call; latency-bound, no roofline claim"}


def time_decode(torch, api, inputs, accounting, steps, warmup, samples=5):
    w = inputs.WORKLOADS["decode_64seq"]
    x = inputs.make_decode(w)
    et = torch.bfloat16
    lens = x["cache_lens"]
    max_len = int(lens.max())
    cap = max_len + 1
    kc = torch.empty((w.batch, cap, w.n_kv_heads, w.head_dim), dtype=et, device="cuda")
    vc = torch.empty_like(kc)

    def put(b, kh, vv):
        kc[b, : len(kh)] = torch.from_numpy(kh).to("cuda", dtype=et)
        vc[b, : len(vv)] = torch.from_numpy(vv).to("cuda", dtype=et)

    inputs.for_each_cache_rows(w, lens, put, threads=min(16, os.cpu_count() or 1))
    dv = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)
    q, kn, vn, gate = dv(x["q"], et), dv(x["k_new"], et), dv(x["v_new"], et), dv(x["gate"], et)
    wq, wk, dl = dv(x["q_norm_w"]), dv(x["k_norm_w"]), dv(lens)
    d = api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rot_dim, w.rope_base, w.rms_eps, 0.0, et,
                      w.gate_mode)
    ws = torch.empty(api.ga_decode_workspace_bytes(d, max_len), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads * w.head_dim), dtype=et, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        api.ga_decode(d, q, kn, vn, kc, vc, dl, max_len, gate=gate, q_norm_w=wq, k_norm_w=wk, out=out, workspace=ws,
                      stream=stream)

    for _ in range(warmup):
        step()
    ramp(torch, step)
    # the step: whole ga_decode calls back to back between two events
    step_ms, step_s = timed_ms(torch, step, stream, steps, samples)
    # the partials kernel alone, back to back between two events
    part_ms, part_s = timed_ms(torch, lambda: api.ga_decode_partials(d, q, kc, vc, dl, max_len, ws, q_norm_w=wq,
                                                                     stream=stream), stream, steps, samples)
    total_bytes = accounting.decode_bytes(lens, w.n_q_heads, w.n_kv_heads, w.head_dim, 2, w.gate_mode)
    cache_bytes = int(lens.astype(np.int64).sum()) * 2 * w.n_kv_heads * w.head_dim * 2
    part_bytes = cache_bytes + w.batch * w.n_q_heads * w.head_dim * 2          # cache + q
    return {
        "metric": "decode KV GB/s",
        "value": total_bytes / (step_ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "ms_per_step": step_ms,
        "step_samples_ms": step_s,
        "steps": steps,
        "config": {"workload": w.name, "batch": w.batch, "cache_len_range": [w.cache_len_lo, w.cache_len_hi],
                   "sum_cache_len": int(lens.sum()), "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "rot_dim": w.rot_dim, "gate": w.gate_mode},
        "bytes_per_step": total_bytes,
        "roofline": {"bound": "hbm", "kernel": "decode_partials_kernel", "achieved": part_bytes / (part_ms * 1e-3) / 1e9,
                     "peak": MI355X_HBM_GBS, "unit": "GB/s",
                     "frac": part_bytes / (part_ms * 1e-3) / 1e9 / MI355X_HBM_GBS,
                     "traffic": measured_traffic("decode_partials_kernel", w.name),
                     "kernel_ms": part_ms, "kernel_samples_ms": part_s, "algorithmic_bytes": part_bytes},
    }


def _cpu_env():
    """Cores of this process, the CPU model and numpy's BLAS build; BLAS
    threads are set to the core count."""
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(cores)
    except Exception:  # pragma: no cover
        pass
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = ""
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '')} {b.get('version', '')}".strip()
    except Exception:  # pragma: no cover
        pass
    return cores, cpu, blas


def _median_wall(fn, reps=3):
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), times


def cpu_baseline(inputs, accounting, headline_x=None, decode_sample=8):
    """The fp64 CPU oracle, as it stands, timed on this host's cores.

    Headline: the 32K-token workload on a seeded sample of 16 query blocks of
    256 rows (all 32 heads, the last block included), one run, extrapolated
    to the whole workload by its share of the unmasked flops (the rate in
    TFLOP/s is the sample's). The other workloads: whole prefill workloads
    (toy, 4096-token, batched) and decode over a seeded sample of sequences of
    the 64-sequence batch (rate extrapolated by cached bytes), median of 3
    runs each."""
    from oracle import attention as oracle
    cores, cpu, blas = _cpu_env()
    per = {}

    def kw(w, x):
        return dict(gate_mode=w.gate_mode, q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], positions=x["positions"],
                    rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)

    # headline: sampled blocks of the 32K-token workload
    w = inputs.WORKLOADS[HEADLINE]
    x = headline_x if headline_x is not None else inputs.make_prefill(w)
    starts = inputs.sample_row_blocks(w, 16, 256)
    t0 = time.perf_counter()
    oracle.prefill_blocks(x["q"], x["k"], x["v"], x["gate"], [(0, r0) for r0 in starts], **kw(w, x))
    t_sample = time.perf_counter() - t0
    d, H = w.head_dim, w.n_q_heads
    sample_flops = sum(2.0 * H * d * sum(i + 1 for i in range(r0, min(w.seq_len, r0 + 256))) for r0 in starts)
    total_flops = accounting.causal_prefill_flops(w.batch, H, d, w.seq_len)
    rate = sample_flops / t_sample / 1e12
    head = {"value": rate, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{HEADLINE}: 16 seeded query blocks of 256 rows x all {H} heads (the last block included), "
                      f"{sample_flops:.3e} of the workload's {total_flops:.3e} unmasked flops, one run of "
                      f"{t_sample:.1f} s, fp64 NumPy oracle; whole-workload time extrapolated by flop share",
            "extrapolated_whole_s": total_flops / (rate * 1e12), "cpu": cpu, "blas": blas}
    del x
    # whole prefill workloads, median of 3
    for name in ("toy", "qwen35_0p8b_prefill", "qwen3_0p6b_batched_prefill"):
        w = inputs.WORKLOADS[name]
        x = inputs.make_prefill(w)
        t, ts = _median_wall(lambda: oracle.prefill(x["q"], x["k"], x["v"], x["gate"], **kw(w, x)))
        flops = accounting.causal_prefill_flops(w.batch, w.n_q_heads, w.head_dim, w.seq_len)
        per[name] = {"value": flops / t / 1e12, "unit": "TFLOP/s", "seconds": t, "runs_s": ts,
                     "sample": "whole workload, median of 3"}
    # decode: a seeded sample of the 64 sequences, median of 3, rate by cached bytes
    w = inputs.WORKLOADS["decode_64seq"]
    xd = inputs.make_decode(w)
    pick = sorted(np.random.default_rng(9).choice(w.batch, decode_sample, replace=False).tolist())
    rows = {b: inputs.decode_cache_rows(w, b, int(xd["cache_lens"][b])) for b in pick}
    sub = {k_: (v_[pick] if isinstance(v_, np.ndarray) and v_.shape[:1] == (w.batch,) else v_)
           for k_, v_ in xd.items()}
    lens = xd["cache_lens"][pick]
    t, ts = _median_wall(lambda: oracle.decode(
        sub["q"], sub["k_new"], sub["v_new"], sub["gate"], gate_mode=w.gate_mode, q_norm_w=sub["q_norm_w"],
        k_norm_w=sub["k_norm_w"], k_cache_rows=lambda i: rows[pick[i]], cache_lens=lens, rms_eps=w.rms_eps,
        rope_base=w.rope_base, rot_dim=w.rot_dim))
    nbytes = accounting.decode_bytes(lens, w.n_q_heads, w.n_kv_heads, w.head_dim, 2, w.gate_mode)
    per["decode_64seq"] = {"value": nbytes / t / 1e9, "unit": "GB/s", "seconds": t, "runs_s": ts,
                           "sample": f"sequences {pick} of 64 (sum L = {int(lens.sum())}), median of 3; "
                                     "bytes as the GPU step counts them"}
    head["per_workload"] = per
    return head


def time_chunk(torch, api, inputs, accounting, steps, warmup):
    """Chunked prefill against a KV cache: four 1024-token chunks of the
    Qwen3.5-0.8B attention shape after 0, 1024, 2048 and 3072 cached tokens."""
    w = inputs.WORKLOADS["qwen35_0p8b_chunk"]
    x = inputs.make_prefill(w)
    et = torch.bfloat16
    lens = np.array(w.extra["cache_lens"], dtype=np.int32)
    max_len = int(lens.max())
    cap = max_len + w.seq_len
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    shape = (w.batch, cap, w.n_kv_heads, w.head_dim)
    kc = torch.randn(shape, generator=gen, device="cuda").to(et)   # cached K-hat / V prefix (synthetic)
    vc = torch.randn(shape, generator=gen, device="cuda").to(et)
    dv = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)
    q, k, v, gate = dv(x["q"], et), dv(x["k"], et), dv(x["v"], et), dv(x["gate"], et)
    wq, wk, dl = dv(x["q_norm_w"]), dv(x["k_norm_w"]), dv(lens)
    d = api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rot_dim, w.rope_base, w.rms_eps, 0.0, et,
                      w.gate_mode)
    out = torch.empty((w.batch, w.seq_len, w.n_q_heads * w.head_dim), dtype=et, device="cuda")
    wsb = api.ga_prefill_chunk_workspace_bytes(d, w.seq_len, cap, max_len)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
    stream = torch.cuda.current_stream()

    def whole():
        api.ga_prefill_chunk(d, q, k, v, kc, vc, dl, max_len, gate=gate, q_norm_w=wq, k_norm_w=wk, out=out,
                             workspace=ws, stream=stream)

    def attention():
        api.ga_prefill_chunk_attention(d, q, kc, vc, dl, max_len, gate=gate, q_norm_w=wq, k_norm_w=wk, out=out,
                                       workspace=ws, stream=stream)

    res = time_whole_and_kernel(torch, whole, attention, stream, steps, warmup)
    flops = accounting.chunk_prefill_flops(lens, w.n_q_heads, w.head_dim, w.seq_len)
    achieved = flops / (res["kernel_ms"] * 1e-3) / 1e12
    kernel = PREFILL_KERNEL_SYMBOL[api.ga_prefill_chunk_kernel(d, w.seq_len, cap)]
    return {
        "metric": "chunked prefill TFLOP/s",
        "value": flops / (res["step_ms"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "ms_per_step": res["step_ms"],
        "steps": steps,
        "config": {"workload": w.name, "batch": w.batch, "chunk_len": w.seq_len, "cache_lens": lens.tolist(),
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "rot_dim": w.rot_dim, "gate": w.gate_mode},
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": achieved, "peak": MI355X_BF16_DENSE_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MI355X_BF16_DENSE_TFLOPS, "kernel_ms": res["kernel_ms"],
                     "traffic": measured_traffic(kernel, w.name), "algorithmic_flops": flops},
    }


def time_packed(torch, api, inputs, accounting, wname, steps, warmup):
    """A prefill workload with q and the gate read in place from a fused q
    projection's output: per-head [q | gate] rows, head stride 2d."""
    w = inputs.WORKLOADS[wname]
    x = inputs.make_prefill(w)
    et = torch.bfloat16
    dv = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)
    hd = w.head_dim
    qg = torch.cat([dv(x["q"], et), dv(x["gate"], et)], dim=-1)           # [B, n, H, 2d]
    q, gate = qg[..., :hd], qg[..., hd:]
    k, v = dv(x["k"], et), dv(x["v"], et)
    wq, wk, pos = dv(x["q_norm_w"]), dv(x["k_norm_w"]), dv(x["positions"])
    d = api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, hd, w.rot_dim, w.rope_base, w.rms_eps, 0.0, et,
                      w.gate_mode, q_head_stride=2 * hd, gate_head_stride=2 * hd)
    khat = torch.empty_like(k)
    api.ga_prefill_keys(d, k, None, wk, pos, k_hat=khat)
    out = torch.empty((w.batch, w.seq_len, w.n_q_heads * hd), dtype=et, device="cuda")
    ws = torch.empty(api.ga_prefill_workspace_bytes(d, w.seq_len), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def whole():
        api.ga_prefill(d, q, k, v, gate, wq, wk, pos, out=out, workspace=ws, stream=stream)

    def attention():
        api.ga_prefill_attention(d, q, khat, v, gate, wq, pos, out=out, stream=stream, k_norm_w=wk)

    res = time_whole_and_kernel(torch, whole, attention, stream, steps, warmup)
    flops = accounting.causal_prefill_flops(w.batch, w.n_q_heads, hd, w.seq_len)
    achieved = flops / (res["kernel_ms"] * 1e-3) / 1e12
    kernel = PREFILL_KERNEL_SYMBOL[api.ga_prefill_attention_kernel(d, w.seq_len)]
    return {
        "metric": METRIC,
        "value": flops / (res["step_ms"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "ms_per_step": res["step_ms"],
        "steps": steps,
        "config": {"workload": w.name, "layout": "fused q projection: per-head [q | gate], head stride 2d",
                   "batch": w.batch, "seq_len": w.seq_len, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": hd, "rot_dim": w.rot_dim, "gate": w.gate_mode},
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": achieved, "peak": MI355X_BF16_DENSE_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MI355X_BF16_DENSE_TFLOPS, "kernel_ms": res["kernel_ms"],
                     "algorithmic_flops": flops},
    }


def time_gate_variant(torch, api, inputs, accounting, wname, steps, warmup):
    """A prefill workload with the extended epilogue: SiLU gate,
    multiplicative, after a per-head RMSNorm of the attention output."""
    w = inputs.WORKLOADS[wname]
    x = inputs.make_prefill(w)
    et = torch.bfloat16
    dv = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)
    q, k, v, gate = dv(x["q"], et), dv(x["k"], et), dv(x["v"], et), dv(x["gate"], et)
    wq, wk, pos = dv(x["q_norm_w"]), dv(x["k_norm_w"]), dv(x["positions"])
    onw = torch.ones(w.head_dim, dtype=torch.float32, device="cuda")
    d = api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rot_dim, w.rope_base, w.rms_eps, 0.0, et,
                      w.gate_mode, gate_act="silu", gate_combine="mul", out_norm_w=onw, out_norm_eps=1e-6)
    khat = torch.empty_like(k)
    api.ga_prefill_keys(d, k, None, wk, pos, k_hat=khat)
    out = torch.empty((w.batch, w.seq_len, w.n_q_heads * w.head_dim), dtype=et, device="cuda")
    ws = torch.empty(api.ga_prefill_workspace_bytes(d, w.seq_len), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def whole():
        api.ga_prefill(d, q, k, v, gate, wq, wk, pos, out=out, workspace=ws, stream=stream)

    def attention():
        api.ga_prefill_attention(d, q, khat, v, gate, wq, pos, out=out, stream=stream, k_norm_w=wk)

    res = time_whole_and_kernel(torch, whole, attention, stream, steps, warmup)
    flops = accounting.causal_prefill_flops(w.batch, w.n_q_heads, w.head_dim, w.seq_len)
    achieved = flops / (res["kernel_ms"] * 1e-3) / 1e12
    kernel = PREFILL_KERNEL_SYMBOL[api.ga_prefill_attention_kernel(d, w.seq_len)]
    return {
        "metric": METRIC,
        "value": flops / (res["step_ms"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "ms_per_step": res["step_ms"],
        "steps": steps,
        "config": {"workload": w.name, "gate": "elementwise SiLU, multiplicative, after a per-head output RMSNorm",
                   "batch": w.batch, "seq_len": w.seq_len, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "rot_dim": w.rot_dim},
        "roofline": {"bound": "mfma", "kernel": kernel + " (extended epilogue)", "achieved": achieved,
                     "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MI355X_BF16_DENSE_TFLOPS,
                     "kernel_ms": res["kernel_ms"], "algorithmic_flops": flops},
    }


def time_backward(torch, api, inputs, accounting, wname, steps, warmup):
    """ga_prefill_backward on the prefill workload (all gradients, the norm
    weights' included), whole calls back to back between two events."""
    w = inputs.WORKLOADS[wname]
    x = inputs.make_prefill(w)
    et = torch.bfloat16
    dv = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)
    q, k, v, gate = dv(x["q"], et), dv(x["k"], et), dv(x["v"], et), dv(x["gate"], et)
    wq, wk, pos = dv(x["q_norm_w"]), dv(x["k_norm_w"]), dv(x["positions"])
    gen = torch.Generator(device="cuda").manual_seed(w.seed + 1000)
    dout = torch.randn((w.batch, w.seq_len, w.n_q_heads * w.head_dim), generator=gen, device="cuda").to(et)
    d = api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rot_dim, w.rope_base, w.rms_eps, 0.0, et,
                      w.gate_mode)
    ws = torch.empty(api.ga_prefill_backward_workspace_bytes(d, w.seq_len), dtype=torch.uint8, device="cuda")
    grads = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dgate=torch.empty_like(gate),
                 dq_norm_w=torch.empty_like(wq), dk_norm_w=torch.empty_like(wk))
    stream = torch.cuda.current_stream()

    def whole():
        api.ga_prefill_backward(d, q, k, v, dout, gate=gate, q_norm_w=wq, k_norm_w=wk, positions=pos, workspace=ws,
                                stream=stream, grads=grads)

    for _ in range(warmup):
        whole()
    ramp(torch, whole)
    step_ms, step_s = timed_ms(torch, whole, stream, steps, 5)
    flops = accounting.causal_backward_flops(w.batch, w.n_q_heads, w.head_dim, w.seq_len)
    achieved = flops / (step_ms * 1e-3) / 1e12

    # the training pair: the forward keeps each row's log-sum-exp, the backward reuses it
    fws = torch.empty(api.ga_prefill_lse_workspace_bytes(d, w.seq_len), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.seq_len, w.n_q_heads * w.head_dim), dtype=et, device="cuda")
    lse = torch.empty((w.batch, w.seq_len, w.n_q_heads), dtype=torch.float32, device="cuda")

    def fwd_lse():
        api.ga_prefill_lse(d, q, k, v, gate=gate, q_norm_w=wq, k_norm_w=wk, positions=pos, out=out, lse=lse,
                           workspace=fws, stream=stream)

    def bwd_lse():
        api.ga_prefill_backward(d, q, k, v, dout, gate=gate, q_norm_w=wq, k_norm_w=wk, positions=pos, workspace=ws,
                                stream=stream, grads=grads, out=out, lse=lse)

    fwd_lse()
    ramp(torch, bwd_lse)
    lse_ms, lse_s = timed_ms(torch, bwd_lse, stream, steps, 5)
    ramp(torch, fwd_lse)
    fwd_ms, fwd_s = timed_ms(torch, fwd_lse, stream, steps, 5)
    saved = {
        "backward_ms": lse_ms, "backward_samples_ms": lse_s,
        "backward_tflops": flops / (lse_ms * 1e-3) / 1e12,
        "backward_frac": flops / (lse_ms * 1e-3) / 1e12 / MI355X_BF16_DENSE_TFLOPS,
        "forward_ms": fwd_ms, "forward_samples_ms": fwd_s,
        "note": "ga_prefill_lse (out and row log-sum-exp; running-max softmax) then ga_prefill_backward_lse "
                "(no recomputed forward attention); whole calls back to back, median of 5 samples",
    }
    return {
        "metric": "prefill backward TFLOP/s",
        "value": achieved,
        "unit": "TFLOP/s",
        "ms_per_step": step_ms,
        "step_samples_ms": step_s,
        "steps": steps,
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "rot_dim": w.rot_dim, "gate": w.gate_mode,
                   "gradients": "q, k, v, gate, q_norm_w, k_norm_w"},
        "roofline": {"bound": "mfma", "kernel": "ga_prefill_backward (whole call: all its kernels)",
                     "achieved": achieved, "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MI355X_BF16_DENSE_TFLOPS, "kernel_ms": step_ms, "algorithmic_flops": flops},
        "saved_lse": saved,
    }


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding of this path is design-only)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from gated_gqa_softmax_amd import accounting, api, inputs

    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.no_prefill:
        dec = time_decode(torch, api, inputs, accounting, args.decode_steps, args.warmup, args.samples)
        print(json.dumps({"decode": dec}), flush=True)
        return
    print(f"[bench] {args.workload}: timing", file=sys.stderr, flush=True)
    pre = time_prefill(torch, api, inputs, accounting, args.workload, args.steps, args.warmup, args.samples)
    w = pre["w"]
    rec = {
        "metric": METRIC,
        "value": pre["flops"] / (pre["step_ms"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "samples": args.samples,
        "ms_per_step": pre["step_ms"],
        "step_samples_ms": pre["step_samples_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": dict(prefill_config(w), parallelism="single-gpu"),
        "roofline": prefill_roofline(pre),
    }
    headline_x = pre["x"] if w.name == HEADLINE else None
    if not args.only:
        if not args.no_extra_prefill:
            for name, k in EXTRA_PREFILL.items():
                if name == w.name:
                    continue
                print(f"[bench] {name}: timing", file=sys.stderr, flush=True)
                rec[name] = prefill_object(time_prefill(torch, api, inputs, accounting, name, k, args.warmup,
                                                        args.samples), k)
            print("[bench] toy: timing", file=sys.stderr, flush=True)
            rec["toy"] = time_toy(torch, api, inputs, 100, args.warmup, args.samples)
        if not args.no_decode:
            print("[bench] decode_64seq: timing", file=sys.stderr, flush=True)
            rec["decode"] = time_decode(torch, api, inputs, accounting, args.decode_steps, args.warmup, args.samples)
        if not args.no_chunk:
            print("[bench] chunk: timing", file=sys.stderr, flush=True)
            rec["chunk"] = time_chunk(torch, api, inputs, accounting, 50, args.warmup)
        if not args.no_packed:
            print("[bench] packed: timing", file=sys.stderr, flush=True)
            rec["packed"] = time_packed(torch, api, inputs, accounting, VARIANT_WORKLOAD, 50, args.warmup)
        if not args.no_variant:
            print("[bench] gate variant: timing", file=sys.stderr, flush=True)
            rec["gate_variant"] = time_gate_variant(torch, api, inputs, accounting, VARIANT_WORKLOAD, 50,
                                                    args.warmup)
        if not args.no_backward:
            print("[bench] backward: timing", file=sys.stderr, flush=True)
            rec["backward"] = time_backward(torch, api, inputs, accounting, VARIANT_WORKLOAD, 10, args.warmup)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(inputs, accounting, headline_x)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
