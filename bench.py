#!/usr/bin/env python3
"""Benchmark of libswattn on one MI355X: prints ONE JSON line.

A step is one forward + backward of causal attention on the "small" training
workload (B8 H6 T2048 D128, bf16, full causal; seeded synthetic data), issued as
the library's three kernels in order (forward; dQ pass, which also computes
delta; dK/dV pass), exactly what swattn_fwd + swattn_bwd launch.  ``--config``
picks another training workload; one with several windows (mid-alt: 512, 2048,
512, 2048) runs that many layers per step, forwards first, then backwards in
reverse order.  ``value`` is window-masked TFLOP/s of the whole step: forward
4*D*N_vis*B*H per layer, backward 2.5x that (the usual five-product
accounting), with N_vis = sum_i min(i+1, W) visible (query, key) pairs per head.

Also measured in the same run:
* per-kernel average durations from HIP events recorded on the stream the
  kernels run on, and the roofline of the dominant kernel;
* the same step cold (median of 50, each after a 1 GiB fill) and under the
  12*D*N_vis model-FLOP count;
* a 1 GiB device copy and an 8192^3 bf16 GEMM (torch) as measured ceilings next
  to the published peaks;
* KV-cache decode (32 sequences, H12 D128 bf16, lengths 512..4096 from seed 7;
  full causal and window 1024) in HBM GB/s, cold cache (a 1 GiB buffer is
  written before every timed call so the 256 MB MALL holds none of the cache);
* the fp64 CPU oracle timed on a bounded sample of the same workload
  (``cpu_baseline``).

Only this file's ``cpu_baseline`` leg imports the oracle.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (AMD public spec)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (AMD public spec)
METRIC = "attn fwd+bwd TFLOP/s (masked FLOPs) and % bf16 MFMA peak; decode HBM GB/s"
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = sorted(glob.glob(os.path.join(ROOT, "causal_sliding_window_amd", "csrc", "*")))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- accounting
def visible_pairs(T: int, W: int) -> int:
    """sum_{i<T} min(i+1, W): visible (query, key) pairs of one head."""
    if W < 0 or W >= T:
        return T * (T + 1) // 2
    return W * (W + 1) // 2 + (T - W) * W


def train_accounting(B, H, T, D, W, elem=2):
    n = visible_pairs(T, W) * B * H
    act = B * T * H * D * elem          # one [B,T,H,D] tensor
    vec = B * H * T * 4                 # one [B,H,T] fp32 vector
    return {
        "pairs": n,
        "flops_fwd": 4 * D * n,
        "flops_bwd": 10 * D * n,
        # algorithmic products per kernel: forward S, PV; dK/dV pass S, dP, dV, dK;
        # dQ pass S, dP, dQ (2*D flops per visible pair each) plus delta = dO . o
        "kernel_flops": {"fwd": 4 * D * n, "bwd_dkdv": 8 * D * n,
                         "bwd_dq": 6 * D * n + 2 * B * T * H * D},
        # algorithmic HBM bytes per kernel: every operand read once, result written once
        # (dQ pass: q, k, v, o, dO, lse in; dq, delta out.  dK/dV: q, k, v, dO, lse,
        # delta in; dk, dv out)
        "kernel_bytes": {"fwd": 4 * act + vec, "bwd_dkdv": 6 * act + 2 * vec,
                         "bwd_dq": 6 * act + 2 * vec},
    }


def step_accounting(B, H, T, D, windows):
    """train_accounting summed over the layers of one step (one layer per window)."""
    per = [train_accounting(B, H, T, D, W) for W in windows]
    out = {k: sum(a[k] for a in per) for k in ("pairs", "flops_fwd", "flops_bwd")}
    for k in ("kernel_flops", "kernel_bytes"):
        out[k] = {n: sum(a[k][n] for a in per) for n in per[0][k]}
    return out


def decode_bytes(lengths, H, D, W, elem=2, Hkv=None):
    """Visible K and V rows of the Hkv cache heads read once, q and o of the H query heads,
    and lse."""
    Hkv = H if Hkv is None else Hkv
    vis = sum(min(int(L), W) if W > 0 else int(L) for L in lengths)
    B = len(lengths)
    return 2 * vis * Hkv * D * elem + 2 * B * H * D * elem + B * H * 4


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        if p.endswith((".hip", ".h", ".cpp")):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- GPU legs
def bench_training(torch, swattn, inputs, cfg_name, steps, warmup, cold_steps=50):
    """Times `steps` training steps of workload `cfg_name`.  A step runs every layer of the
    workload's window schedule (one layer per entry of its `windows`, each with its own
    seeded inputs): the forwards in layer order, then the backwards in reverse order, as a
    model's training step issues them."""
    c = inputs.CONFIGS[cfg_name]
    B, H, T, D = c["B"], c["H"], c["T"], c["D"]
    windows = list(c["windows"])
    scale = 1.0 / math.sqrt(D)
    lib = swattn.lib()
    P = swattn._ptr
    stream = torch.cuda.current_stream()
    sh = swattn.ctypes.c_void_p(stream.cuda_stream)
    ws = torch.empty(swattn.swattn_bwd_workspace_size(B, H, T, D), dtype=torch.uint8, device="cuda:0")
    layers = []
    for i, W in enumerate(windows):
        x = {n: t.to("cuda:0") for n, t in inputs.config_inputs(cfg_name, layer=i).items()}
        q = x["q"]
        layers.append(dict(W=W, q=q, k=x["k"], v=x["v"], do=x["do"], o=torch.empty_like(q),
                           lse=torch.empty((B, H, T), dtype=torch.float32, device="cuda:0"),
                           dq=torch.empty_like(q), dk=torch.empty_like(q), dv=torch.empty_like(q)))

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {swattn.status_string(rc)}")

    def step(ev=None):
        # ev[i] holds four events per layer: before forward, forward | dQ, dQ | dK/dV, after
        for i, L in enumerate(layers):
            if ev is not None:
                ev[i][0].record(stream)
            check(lib.swattn_fwd(P(L["q"]), P(L["k"]), P(L["v"]), P(L["o"]), P(L["lse"]), B, H, T,
                                 D, L["W"], scale, sh), "fwd")
            if ev is not None:
                ev[i][1].record(stream)
        for i in reversed(range(len(layers))):
            L = layers[i]
            if ev is not None:
                ev[i][2].record(stream)
            # swattn_bwd is exactly these two passes; the dQ pass also writes delta
            check(lib.swattn_bwd_dq(P(L["q"]), P(L["k"]), P(L["v"]), P(L["o"]), P(L["do"]),
                                    P(L["lse"]), P(ws), P(L["dq"]), B, H, T, D, L["W"], scale, sh),
                  "bwd_dq")
            if ev is not None:
                ev[i][3].record(stream)
            check(lib.swattn_bwd_dkdv(P(L["q"]), P(L["k"]), P(L["v"]), P(L["do"]), P(L["lse"]),
                                      P(ws), P(L["dk"]), P(L["dv"]), B, H, T, D, L["W"], scale, sh),
                  "bwd_dkdv")
            if ev is not None:
                ev[i][4].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in layers]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # cold: a 1 GiB fill before each step, so the 256 MB MALL holds none of the inputs
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    cold = []
    for _ in range(cold_steps):
        flush.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    spans = {"fwd": (0, 1), "bwd_dq": (2, 3), "bwd_dkdv": (3, 4)}
    # per-kernel time of one step: summed over the layers, averaged over the steps
    per = {n: statistics.fmean(sum(e[i][a].elapsed_time(e[i][b]) for i in range(len(layers)))
                               for e in evs) for n, (a, b) in spans.items()}
    return {"B": B, "H": H, "T": T, "D": D, "windows": windows, "wall_s": wall, "kernel_ms": per,
            "cold_ms": statistics.median(cold) if cold else None,
            "acct": step_accounting(B, H, T, D, windows)}


def bench_decode(torch, swattn, inputs, iters, hkv=None):
    """Cold decode of the 32-sequence workload at each of its windows; with ``hkv`` the
    same workload with that many K/V heads (grouped-query decode)."""
    c = inputs.CONFIGS["decode"]
    B, H, D, Tmax = c["B"], c["H"], c["D"], c["Tmax"]
    lengths = inputs.decode_lengths(B, c["len_seed"], c["len_lo"], c["len_hi"])
    d = inputs.decode_inputs(B, H, D, Tmax, c["dtype"], c["seed"], lengths, Hkv=hkv)
    lengths = d["seqlens"].tolist()
    g = {n: t.to("cuda:0") for n, t in d.items()}
    scale = 1.0 / math.sqrt(D)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
    out = {}
    for W in c["windows"]:
        ws = torch.empty(swattn.swattn_decode_workspace_size(B, H, D, Tmax, W), dtype=torch.uint8,
                         device="cuda:0")
        o = torch.empty_like(g["q"])
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda:0")
        entry = swattn.swattn_decode if hkv is None else swattn.swattn_decode_gqa

        def call():
            entry(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], o, lse, W, scale, ws)

        for _ in range(3):
            call()
        cold, warm = [], []
        for _ in range(iters):
            flush.fill_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        for _ in range(iters):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            warm.append(a.elapsed_time(b))
        nbytes = decode_bytes(lengths, H, D, W, Hkv=hkv)
        ms = statistics.median(cold)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["causal" if W < 0 else f"window{W}"] = {
            "bytes": nbytes, "us_cold_median": round(ms * 1e3, 2),
            "us_warm_median": round(statistics.median(warm) * 1e3, 2),
            "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        }
    return out


def bench_prologue(torch, swattn, inputs, iters, cfg_name="small"):
    """QK-norm + rotary prologue on a training workload's raw q and k (one launch for
    both), forward and backward, cold (a 1 GiB fill before each call).  Bytes: the
    forward reads q, k and writes q', k'; the backward reads q, k, dq', dk' and writes
    dq, dk."""
    c = inputs.CONFIGS[cfg_name]
    B, T, H, D = c["B"], c["T"], c["H"], c["D"]
    x = inputs.training_inputs(B, T, H, D, c["dtype"], c["seeds"][0], qk_norm=False)
    # distinct gradient buffers for q' and k' (dO and v of the workload serve)
    q, k, dyq, dyk = (x[n].to("cuda:0") for n in ("q", "k", "do", "v"))
    yq, yk = torch.empty_like(q), torch.empty_like(k)
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    calls = {"forward": lambda: swattn.swattn_qk_norm_rope(q, k, yq, yk),
             "backward": lambda: swattn.swattn_qk_norm_rope_bwd(q, k, dyq, dyk, dq, dk)}
    tensor_bytes = q.numel() * q.element_size()
    res = {"workload": f"{cfg_name}: q and k [{B},{T},{H},{D}] bf16, raw"}
    for name, call in calls.items():
        for _ in range(3):
            call()
        ts = []
        for _ in range(iters):
            flush.fill_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        nb = (4 if name == "forward" else 6) * tensor_bytes
        ms = statistics.median(ts)
        res[name] = {"bytes": nb, "us_cold_median": round(ms * 1e3, 2),
                     "GB_per_s": round(nb / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del flush
    return res


def bench_prefill(torch, swattn, inputs, iters, tq=512):
    """Chunked prefill on the decode workload's caches: each of the 32 sequences appends a
    chunk of ``tq`` tokens at (its decode length - tq) and attends the chunk's queries to
    its cache, full causal.  Cold (a 1 GiB fill before each call); TFLOP/s counts the
    visible (query, key) pairs, 4*D per pair."""
    c = inputs.CONFIGS["decode"]
    B, H, D, Tmax = c["B"], c["H"], c["D"], c["Tmax"]
    lens = [max(int(L) - tq, 0) for L in inputs.decode_lengths(B, c["len_seed"], c["len_lo"],
                                                                c["len_hi"])]
    d = inputs.decode_inputs(B, H, D, Tmax, c["dtype"], c["seed"], lens)
    x = inputs.training_inputs(B, tq, H, D, c["dtype"], seed=c["seed"] + 10)
    g = {n: t.to("cuda:0") for n, t in d.items()}
    q, kn, vn = (x[n].to("cuda:0") for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, tq), dtype=torch.float32, device="cuda:0")
    scale = 1.0 / math.sqrt(D)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")

    def call():
        swattn.swattn_prefill(q, kn, vn, g["k_cache"], g["v_cache"], g["seqlens"], o, lse, -1,
                              scale)

    for _ in range(3):
        call()
    ts = []
    for _ in range(iters):
        flush.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    del flush
    pairs = H * sum(tq * L0 + tq * (tq + 1) // 2 for L0 in lens)
    ms = statistics.median(ts)
    return {"workload": f"{B} sequences, H{H} D{D}, chunks of {tq} tokens appended at "
                        f"(decode length - {tq}), cache of {Tmax} rows, full causal",
            "us_cold_median": round(ms * 1e3, 2),
            "TFLOP_per_s": round(4 * D * pairs / (ms * 1e-3) / 1e12, 1)}


def bench_training_gqa(torch, swattn, inputs, cfg_name, hkv, steps, warmup):
    """The training workload with ``hkv`` K/V heads shared by its query heads in groups:
    forward and backward of every layer through the grouped-query entry points (the
    backward as one call: dQ, the per-head dK/dV pass and the group sum)."""
    c = inputs.CONFIGS[cfg_name]
    B, H, T, D = c["B"], c["H"], c["T"], c["D"]
    scale = 1.0 / math.sqrt(D)
    layers = []
    for i, W in enumerate(c["windows"]):
        x = {n: t.to("cuda:0") for n, t in inputs.training_inputs(
            B, T, H, D, c["dtype"], c["seeds"][i], c["qk_norm"], Hkv=hkv).items()}
        layers.append(dict(W=W, **x, o=torch.empty_like(x["q"]),
                           lse=torch.empty((B, H, T), dtype=torch.float32, device="cuda:0"),
                           dq=torch.empty_like(x["q"]), dk=torch.empty_like(x["k"]),
                           dv=torch.empty_like(x["v"])))
    ws = torch.empty(swattn.swattn_bwd_gqa_workspace_size(B, H, hkv, T, D), dtype=torch.uint8,
                     device="cuda:0")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        for i, L in enumerate(layers):
            if ev is not None:
                ev[i][0].record(stream)
            swattn.swattn_fwd_gqa(L["q"], L["k"], L["v"], L["o"], L["lse"], L["W"], scale)
            if ev is not None:
                ev[i][1].record(stream)
        for i in reversed(range(len(layers))):
            L = layers[i]
            if ev is not None:
                ev[i][2].record(stream)
            swattn.swattn_bwd_gqa(L["q"], L["k"], L["v"], L["o"], L["do"], L["lse"], L["dq"],
                                  L["dk"], L["dv"], L["W"], scale, ws)
            if ev is not None:
                ev[i][3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in layers]
           for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: statistics.fmean(sum(e[i][a].elapsed_time(e[i][b]) for i in range(len(layers)))
                               for e in evs) for n, (a, b) in {"fwd": (0, 1), "bwd": (2, 3)}.items()}
    acct = step_accounting(B, H, T, D, list(c["windows"]))
    ms = wall / steps * 1e3
    return {"workload": f"{cfg_name} with {hkv} K/V heads for {H} query heads",
            "ms_per_step": round(ms, 4),
            "TFLOP_per_s": round((acct["flops_fwd"] + acct["flops_bwd"]) / (ms * 1e-3) / 1e12, 2),
            "fwd_ms": round(per["fwd"], 4), "bwd_ms": round(per["bwd"], 4),
            "fwd_TFLOP_per_s": round(acct["flops_fwd"] / (per["fwd"] * 1e-3) / 1e12, 1),
            "bwd_TFLOP_per_s": round(acct["flops_bwd"] / (per["bwd"] * 1e-3) / 1e12, 1)}


def measured_refs(torch):
    """Practical ceilings measured on this GPU, reported next to the published peaks: a
    1 GiB device copy (read + write bytes) and an 8192^3 bf16 GEMM (torch.matmul)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(n):
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return statistics.median(ts)

    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del src, dst
    m = 8192
    g = torch.Generator(device="cuda:0")
    g.manual_seed(0)
    x = torch.randn(m, m, device="cuda:0", generator=g).to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda:0", generator=g).to(torch.bfloat16)
    t_mm = timed(lambda: torch.matmul(x, y))
    del x, y
    return {"copy_GB_per_s": round(2 * n * 4 / t_copy / 1e9, 1),
            "gemm_bf16_TFLOP_per_s": round(2 * m ** 3 / t_mm / 1e12, 1),
            "what": "1 GiB device copy (read + write bytes); 8192^3 bf16 torch.matmul"}


# ----------------------------------------------------------------------------- CPU oracle leg
def cpu_baseline(inputs, budget_s=12.0):
    import numpy as np
    from oracle import attention as orc
    threads, blas = 1, "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            threads = max(i.get("num_threads", 1) for i in libs)
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs)
    except Exception:  # pragma: no cover
        pass
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    c = inputs.CONFIGS["small"]
    B, H, T, D, W = c["B"], c["H"], c["T"], c["D"], c["windows"][0]
    x = inputs.config_inputs("small")
    a = {n: inputs.to_f64(t) for n, t in x.items()}
    scale = 1.0 / math.sqrt(D)
    done, t_f, t_b = 0, 0.0, 0.0
    pairs = visible_pairs(T, W)
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(H):
            t1 = time.perf_counter()
            orc.head_fwd(a["q"][b, :, h], a["k"][b, :, h], a["v"][b, :, h], W, scale)
            t2 = time.perf_counter()
            orc.head_bwd(a["q"][b, :, h], a["k"][b, :, h], a["v"][b, :, h], a["do"][b, :, h], W, scale)
            t3 = time.perf_counter()
            t_f, t_b = t_f + (t2 - t1), t_b + (t3 - t2)
            done += 1
            if t3 - t0 > budget_s:
                break
        else:
            continue
        break
    el = t_f + t_b
    return {"value": round(14 * D * pairs * done / el / 1e12, 5), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "fwd_TFLOP_per_s": round(4 * D * pairs * done / t_f / 1e12, 5),
            "bwd_TFLOP_per_s": round(10 * D * pairs * done / t_b / 1e12, 5),
            "cpu": cpu, "blas": blas,
            "sample": f"{done} of {B * H} heads of the small workload (T={T}, D={D}, full causal): "
                      f"NumPy fp64 oracle forward ({t_f:.1f} s) + backward ({t_b:.1f} s), "
                      f"same masked-FLOP count"}


# ----------------------------------------------------------------------------- counters
def traffic_for(kernel: str):
    """HBM bytes per launch from stored rocprofv3 FETCH_SIZE/WRITE_SIZE counters, scaled by a
    plain copy kernel's reading; None when missing or taken on different kernel sources."""
    try:
        data = json.load(open(COUNTERS))
    except Exception:
        return None
    if data.get("source_hash") != source_hash():
        return None
    k = data.get("kernels", {}).get(kernel)
    if not k:
        return None
    return int(k["fetch_bytes"] * data["fetch_factor"] + k["write_bytes"] * data["write_factor"])


def ingest_counters(fetch_csv, write_csv, copy_bytes):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into
    profiles/counters.json.  The copy kernel (torch copy of `copy_bytes`) calibrates
    each counter: factor = known bytes / counter bytes."""
    import csv

    def read(path, counter):
        rows = {}
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") != counter:
                continue
            rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: statistics.fmean(v) for k, v in rows.items()}

    fe, wr = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    pick = lambda d, key: next((v for k, v in d.items() if key in k), None)  # noqa: E731

    def copy_reading(path, counter):
        # the calibration copy is the largest copy dispatch (the runtime issues small
        # copies of its own)
        vals = [float(r["Counter_Value"]) * 1024.0 for r in csv.DictReader(open(path))
                if r.get("Counter_Name") == counter and "copy" in r["Kernel_Name"]]
        return max(vals) if vals else None

    copy_f = copy_reading(fetch_csv, "FETCH_SIZE")
    copy_w = copy_reading(write_csv, "WRITE_SIZE")
    # the training and decode kernels of the small and decode workloads (not the grouped
    # or prefill instantiations, which the same run also launches)
    names = {"fwd": "fwd_bf16_kernel<128, false>",
             "bwd_dkdv": "bwd_dkdv_bf16_kernel<128, false>", "bwd_dq": "bwd_dq_bf16_kernel<128>",
             "decode_split": "decode_split_kernel<unsigned short, 128, false>"}
    out = {"source_hash": source_hash(), "copy_bytes": copy_bytes,
           "fetch_factor": copy_bytes / copy_f if copy_f else 1.0,
           "write_factor": copy_bytes / copy_w if copy_w else 1.0, "kernels": {}}
    for n, sub in names.items():
        f, w = pick(fe, sub), pick(wr, sub)
        if f is not None and w is not None:
            out["kernels"][n] = {"fetch_bytes": f, "write_bytes": w}
    os.makedirs(os.path.dirname(COUNTERS), exist_ok=True)
    json.dump(out, open(COUNTERS, "w"), indent=1)
    print(json.dumps(out))


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # ~0.3 ms per step: the defaults give the GPU ~0.3 s of load before timing (it
    # reaches its steady clocks after a few hundred milliseconds; 10 warm-up steps
    # measured 10% slower) and time ~0.6 s
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", default="small", help="training workload (default: small)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hkv", type=int, default=0,
                    help="also time the training workload with this many K/V heads "
                         "(grouped-query entry points)")
    ap.add_argument("--no-refs", action="store_true",
                    help="skip the measured copy-bandwidth and GEMM references")
    ap.add_argument("--decode-iters", type=int, default=20)
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="also run one torch copy of this many bytes (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_BYTES"))
    args = ap.parse_args()

    if args.ingest_counters:
        f, w, n = args.ingest_counters
        ingest_counters(f, w, int(n))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              f"multi-GPU path: run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    from causal_sliding_window_amd import inputs, swattn
    if not torch.cuda.is_available():
        print("no GPU visible: bench.py needs an MI355X", file=sys.stderr)
        return 1
    swattn.lib()  # fail loudly if the HIP library is missing

    if args.copy_probe:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    tr = bench_training(torch, swattn, inputs, args.config, args.steps, args.warmup)
    acct = tr["acct"]
    ms_step = tr["wall_s"] / args.steps * 1e3
    flops_step = acct["flops_fwd"] + acct["flops_bwd"]
    value = flops_step / (ms_step * 1e-3) / 1e12
    kernels = {}
    for n, ms in tr["kernel_ms"].items():
        f, by = acct["kernel_flops"][n], acct["kernel_bytes"][n]
        kernels[n] = {"ms": round(ms, 4), "TFLOP_per_s": round(f / (ms * 1e-3) / 1e12, 1),
                      "GB_per_s": round(by / (ms * 1e-3) / 1e9, 1)}
    dom = max(tr["kernel_ms"], key=lambda n: tr["kernel_ms"][n])
    dom_ms = tr["kernel_ms"][dom]
    achieved = acct["kernel_flops"][dom] / (dom_ms * 1e-3) / 1e12
    model_tflops = 12 * tr["D"] * acct["pairs"] / (ms_step * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms (cold {tr['cold_ms']:.3f} ms), {value:.1f} TFLOP/s; "
        f"kernels {kernels}")

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), RMS-normalised q/k)",
        "config": {"workload": f"{args.config}: B{tr['B']} H{tr['H']} T{tr['T']} D{tr['D']} "
                               f"bf16, {len(tr['windows'])} layer(s), windows {tr['windows']} "
                               f"(-1 = full causal), forward + backward",
                   "B": tr["B"], "H": tr["H"], "T": tr["T"], "D": tr["D"],
                   "windows": tr["windows"],
                   "parallelism": "none (1 GPU)"},
        "pct_bf16_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        # the same step under the 12*D*N_vis "model FLOP" count (no recompute of S)
        "model_TFLOP_per_s": round(model_tflops, 2),
        # median of 50 steps, each after a 1 GiB fill (inputs not in the MALL)
        "cold_ms_per_step": round(tr["cold_ms"], 4),
        "kernels": kernels,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     # stored counters are taken on the default (small) workload
                     "traffic": traffic_for(dom) if args.config == "small" else None,
                     "algorithmic_bytes": acct["kernel_bytes"][dom]},
    }
    if not args.no_decode:
        res["decode"] = bench_decode(torch, swattn, inputs, args.decode_iters)
        log(f"decode {res['decode']}")
        # grouped-query decode: the same 32 sequences with 4 K/V heads (3 query heads
        # each) and with one (multi-query); bytes count the Hkv cache heads
        res["decode_gqa"] = {f"hkv{n}": bench_decode(torch, swattn, inputs, args.decode_iters, n)
                             for n in (4, 1)}
        log(f"decode gqa {res['decode_gqa']}")
        res["prefill"] = bench_prefill(torch, swattn, inputs, args.decode_iters)
        log(f"prefill {res['prefill']}")
        res["qk_prologue"] = bench_prologue(torch, swattn, inputs, args.decode_iters)
        log(f"qk prologue {res['qk_prologue']}")
    if args.hkv:
        res["training_gqa"] = bench_training_gqa(torch, swattn, inputs, args.config, args.hkv,
                                                 max(50, args.steps // 4), max(50, args.warmup // 2))
        log(f"training gqa {res['training_gqa']}")
    if not args.no_refs:
        refs = measured_refs(torch)
        res["measured_refs"] = refs
        res["roofline"]["frac_of_measured_gemm"] = round(achieved / refs["gemm_bf16_TFLOP_per_s"], 4)
        for d in res.get("decode", {}).values():
            d["frac_of_measured_copy"] = round(d["GB_per_s"] / refs["copy_GB_per_s"], 4)
        log(f"measured refs {refs}")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inputs)
        log(f"cpu baseline {res['cpu_baseline']}")
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
