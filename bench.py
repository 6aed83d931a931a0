#!/usr/bin/env python3
"""Throughput of gated GQA causal attention on one MI355X.

One step is one prefill pass (ga_prefill: the K-hat kernel then the fused
attention kernel) over the Qwen3.5-0.8B-shaped workload (B=1, n=4096, H=8,
G=2, d=256, RoPE on 64 dims, elementwise gate, bf16). The decode half of the
metric (ga_decode over 64 sequences with cache lengths ~U[1024, 32768]) is
measured in the same run and reported under "decode".

Printed: one JSON line. ``value`` is prefill TFLOP/s counting only the
unmasked causal work 2*B*H*d*n*(n+1); ``roofline`` relates the attention
kernel's own duration (HIP events around each launch, on its stream) to the
bf16 dense MFMA peak; ``cpu_baseline`` times the CPU oracle on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

MI355X_BF16_DENSE_TFLOPS = 2500.0
MI355X_HBM_GBS = 8000.0
METRIC = "gated GQA attn fwd TFLOP/s (prefill) + decode KV GB/s, % of MI355X roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen35_0p8b_prefill",
                    help="prefill workload to time (default: the headline one)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-chunk", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-packed", action="store_true", help="skip the fused [q | gate] input measurement")
    ap.add_argument("--no-variant", action="store_true", help="skip the gate-variant epilogue measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--no-prefill", action="store_true", help="decode only (for counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=20)
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
PREFILL_KERNEL_SYMBOL = {"wide": "prefill_wide_kernel", "mirror": "prefill_v2_kernel", "split": "prefill_v2_kernel",
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


def time_whole_and_kernel(torch, whole, attention, stream, steps, warmup):
    """Mean ms of ``whole`` (one step) and of ``attention`` (the attention
    kernel's launch), each as ``steps`` calls back to back between two events."""
    for _ in range(warmup):
        whole()
    ramp(torch, whole)
    res = {}
    for name, fn in (("step_ms", whole), ("kernel_ms", attention)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    return res


def time_prefill(torch, api, inputs, accounting, wname, steps, warmup):
    w = inputs.WORKLOADS[wname]
    x = inputs.make_prefill(w)
    et = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dv = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt) if a is not None else None
    q, k, v = dv(x["q"], et), dv(x["k"], et), dv(x["v"], et)
    gate = dv(x["gate"], et)
    wq, wk, pos = dv(x["q_norm_w"]), dv(x["k_norm_w"]), dv(x["positions"])
    d = api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rot_dim, w.rope_base, w.rms_eps, 0.0, et,
                      w.gate_mode)
    khat = torch.empty_like(k)
    out = torch.empty((w.batch, w.seq_len, w.n_q_heads * w.head_dim), dtype=et, device="cuda")
    ws_attn = torch.empty(max(1, api.ga_prefill_attention_workspace_bytes(d, w.seq_len)), dtype=torch.uint8,
                          device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev0=None, ev1=None):
        # exactly what ga_prefill does, with events around the attention kernel
        api.ga_prefill_keys(d, k, None, wk, pos, k_hat=khat, stream=stream)
        if ev0 is not None:
            ev0.record(stream)
        api.ga_prefill_attention(d, q, khat, v, gate, wq, pos, out=out, workspace=ws_attn, stream=stream)
        if ev1 is not None:
            ev1.record(stream)

    for _ in range(warmup):
        step()
    ramp(torch, step)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(*ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms_events = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # The attention kernel's launch duration: the same launches back to back
    # between two events on its stream (per-launch event pairs add several
    # microseconds of event overhead to a ~0.1 ms kernel).
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    k0.record(stream)
    for _ in range(steps):
        api.ga_prefill_attention(d, q, khat, v, gate, wq, pos, out=out, workspace=ws_attn, stream=stream)
    k1.record(stream)
    torch.cuda.synchronize()
    attn_ms = k0.elapsed_time(k1) / steps
    kernel = PREFILL_KERNEL_SYMBOL[api.ga_prefill_attention_kernel(d, w.seq_len)]
    # whole ga_prefill calls, for the step figure
    ws = torch.empty(api.ga_prefill_workspace_bytes(d, w.seq_len), dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        api.ga_prefill(d, q, k, v, gate, wq, wk, pos, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    flops = accounting.causal_prefill_flops(w.batch, w.n_q_heads, w.head_dim, w.seq_len)
    return dict(w=w, x=x, flops=flops, attn_ms=attn_ms, attn_ms_events=attn_ms_events, kernel=kernel,
                step_ms=step_ms, wall_s=wall)


def time_decode(torch, api, inputs, accounting, steps, warmup):
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

    def step(ev0=None, ev1=None):
        if ev0 is not None:
            ev0.record(stream)
        api.ga_decode_partials(d, q, kc, vc, dl, max_len, ws, q_norm_w=wq, stream=stream)
        if ev1 is not None:
            ev1.record(stream)
        api.ga_decode_merge(d, q, kn, vn, kc, vc, dl, max_len, ws, gate=gate, q_norm_w=wq, k_norm_w=wk, out=out,
                            stream=stream)

    for _ in range(warmup):
        step()
    ramp(torch, step)
    # per-launch event pairs around the partials kernel (a diagnostic: each
    # pair adds event overhead, so neither figure below comes from this loop)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(*ev[i])
    torch.cuda.synchronize()
    part_ms_events = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # the step: whole ga_decode calls back to back between two events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        api.ga_decode(d, q, kn, vn, kc, vc, dl, max_len, gate=gate, q_norm_w=wq, k_norm_w=wk, out=out, workspace=ws,
                      stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    # the partials kernel alone, back to back between two events
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    k0.record(stream)
    for _ in range(steps):
        api.ga_decode_partials(d, q, kc, vc, dl, max_len, ws, q_norm_w=wq, stream=stream)
    k1.record(stream)
    torch.cuda.synchronize()
    part_ms = k0.elapsed_time(k1) / steps
    total_bytes = accounting.decode_bytes(lens, w.n_q_heads, w.n_kv_heads, w.head_dim, 2, w.gate_mode)
    cache_bytes = int(lens.astype(np.int64).sum()) * 2 * w.n_kv_heads * w.head_dim * 2
    part_bytes = cache_bytes + w.batch * w.n_q_heads * w.head_dim * 2          # cache + q
    return {
        "metric": "decode KV GB/s",
        "value": total_bytes / (step_ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "ms_per_step": step_ms,
        "steps": steps,
        "config": {"workload": w.name, "batch": w.batch, "cache_len_range": [w.cache_len_lo, w.cache_len_hi],
                   "sum_cache_len": int(lens.sum()), "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "rot_dim": w.rot_dim, "gate": w.gate_mode},
        "bytes_per_step": total_bytes,
        "roofline": {"bound": "hbm", "kernel": "decode_partials_kernel", "achieved": part_bytes / (part_ms * 1e-3) / 1e9,
                     "peak": MI355X_HBM_GBS, "unit": "GB/s",
                     "frac": part_bytes / (part_ms * 1e-3) / 1e9 / MI355X_HBM_GBS,
                     "traffic": measured_traffic("decode_partials_kernel", w.name),
                     "kernel_ms": part_ms, "kernel_ms_event_pairs": part_ms_events,
                     "algorithmic_bytes": part_bytes},
    }


def cpu_baseline(w, x, flops, budget_s=15.0):
    """The CPU oracle, as it stands, on the whole prefill workload, repeated
    until about budget_s seconds of work (at least once)."""
    from oracle import attention as oracle
    try:
        import threadpoolctl
        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.prefill(x["q"], x["k"], x["v"], x["gate"], gate_mode=w.gate_mode, q_norm_w=x["q_norm_w"],
                       k_norm_w=x["k_norm_w"], positions=x["positions"], rms_eps=w.rms_eps, rope_base=w.rope_base,
                       rot_dim=w.rot_dim)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    t = float(np.median(times))
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"whole {w.name} workload, fp64 NumPy oracle, median of {len(times)} runs "
                      f"({t:.2f} s each)", "cpu": cpu}


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
    ws = torch.empty(max(1, api.ga_prefill_chunk_workspace_bytes(d, w.seq_len, cap, max_len)), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def whole():
        api.ga_prefill_chunk(d, q, k, v, kc, vc, dl, max_len, gate=gate, q_norm_w=wq, k_norm_w=wk, out=out,
                             workspace=ws, stream=stream)

    def attention():
        api.ga_prefill_chunk_attention(d, q, kc, vc, dl, max_len, gate=gate, q_norm_w=wq, out=out, workspace=ws,
                                       stream=stream)

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
        "roofline": {"bound": "mfma", "kernel": kernel + (" (key ranges split in two)" if ws.numel() > 1 else ""),
                     "achieved": achieved, "peak": MI355X_BF16_DENSE_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MI355X_BF16_DENSE_TFLOPS, "kernel_ms": res["kernel_ms"],
                     "algorithmic_flops": flops},
    }


def time_packed(torch, api, inputs, accounting, wname, steps, warmup):
    """The headline prefill with q and the gate read in place from a fused q
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
    ws_attn = torch.empty(max(1, api.ga_prefill_attention_workspace_bytes(d, w.seq_len)), dtype=torch.uint8,
                          device="cuda")
    stream = torch.cuda.current_stream()

    def whole():
        api.ga_prefill(d, q, k, v, gate, wq, wk, pos, out=out, workspace=ws, stream=stream)

    def attention():
        api.ga_prefill_attention(d, q, khat, v, gate, wq, pos, out=out, workspace=ws_attn, stream=stream)

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
    """The headline prefill with the extended epilogue: SiLU gate,
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
        api.ga_prefill_attention(d, q, khat, v, gate, wq, pos, out=out, stream=stream)

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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        whole()
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    flops = accounting.causal_backward_flops(w.batch, w.n_q_heads, w.head_dim, w.seq_len)
    achieved = flops / (step_ms * 1e-3) / 1e12
    return {
        "metric": "prefill backward TFLOP/s",
        "value": achieved,
        "unit": "TFLOP/s",
        "ms_per_step": step_ms,
        "steps": steps,
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "rot_dim": w.rot_dim, "gate": w.gate_mode,
                   "gradients": "q, k, v, gate, q_norm_w, k_norm_w"},
        "roofline": {"bound": "mfma", "kernel": "ga_prefill_backward (whole call: all its kernels)",
                     "achieved": achieved, "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MI355X_BF16_DENSE_TFLOPS, "kernel_ms": step_ms, "algorithmic_flops": flops},
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
        dec = time_decode(torch, api, inputs, accounting, args.decode_steps, args.warmup)
        print(json.dumps({"decode": dec}), flush=True)
        return
    pre = time_prefill(torch, api, inputs, accounting, args.workload, args.steps, args.warmup)
    w = pre["w"]
    achieved = pre["flops"] / (pre["attn_ms"] * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": pre["flops"] / (pre["step_ms"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "rot_dim": w.rot_dim, "gate": w.gate_mode,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "kernel": pre["kernel"], "achieved": achieved,
                     "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MI355X_BF16_DENSE_TFLOPS,
                     "traffic": measured_traffic(pre["kernel"], w.name), "kernel_ms": pre["attn_ms"],
                     "kernel_ms_event_pairs": pre["attn_ms_events"],
                     "algorithmic_flops": pre["flops"]},
    }
    if not args.no_decode:
        rec["decode"] = time_decode(torch, api, inputs, accounting, args.decode_steps, args.warmup)
    if not args.no_chunk:
        rec["chunk"] = time_chunk(torch, api, inputs, accounting, args.steps, args.warmup)
    if not args.no_packed and w.gate_mode == "elementwise" and w.dtype == "bf16":
        rec["packed"] = time_packed(torch, api, inputs, accounting, args.workload, args.steps, args.warmup)
    if not args.no_variant and w.gate_mode == "elementwise" and w.dtype == "bf16":
        rec["gate_variant"] = time_gate_variant(torch, api, inputs, accounting, args.workload, args.steps,
                                                args.warmup)
    if not args.no_backward and w.gate_mode == "elementwise" and w.dtype == "bf16":
        rec["backward"] = time_backward(torch, api, inputs, accounting, args.workload, max(5, args.steps // 5),
                                        args.warmup)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, pre["x"], pre["flops"])
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
