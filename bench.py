"""Benchmark of the attention hot path on one MI355X.

One step runs every stage of the path once on seeded synthetic inputs that
are already resident in device memory:
  1. masked prefill with LSE, bf16, B1 H16 P11,616 D64, last 16 keys padded
     (attn_fwd_lse; the ~3 MP patch self-attention case),
  2. chunked-KV attention: Q 8,192 x H24 x D128 against two 8,192-key
     chunks (2 x attn_fwd_lse) and their LSE merge (attn_merge_lse),
  3. one decode step: kv_append + attn_decode, bf16 GQA B32, 32 query / 8 KV
     heads, D128, cached lengths U[512, 8192] (then +1 appended).
The cache lengths are restored before every step so each step is the same
workload.

The headline value is the prefill's algorithmic throughput (4·D·H·Tq·n_valid
FLOP over the prefill call's duration, from HIP events on the launch stream
over the timed steps); the decode's algorithmic HBM rate (K and V bytes of
every cached token, plus q and o, over the attn_decode duration) and the
merge's rate are reported beside it.  `cpu_baseline` times the float64 CPU
oracle on a bounded sample of the prefill workload.

Timing: HIP events on the launch stream around every call of every timed step (K >= 50
by default), reported as the mean and the 10th / 50th / 90th percentiles per kernel.  The
decodes timed on their own read a 512 MiB scratch buffer before each call, so the 256 MB
last-level cache (MALL) holds none of the cache they read.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
Prints one JSON line.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E (published)
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 matrix peak (published)
PEAK_FP32_VECTOR_TFLOPS = 157.3   # MI355X fp32 vector peak (published; packed fp32 FMA)
# The E4M3 prefill runs Q·Kᵀ (half its FLOP) at the fp8 rate and P·V (the other half) at
# the bf16 rate: its matrix-core bound is 1 / (0.5 / fp8 peak + 0.5 / bf16 peak).
PEAK_FP8_PREFILL_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PREFILL_SRCS = [os.path.join(ROOT, "masked_attention_attn_amd", "csrc", f)
                for f in ("fwd_bf16.cuh", "fwd_bf16_d64.hip", "mfma_lds.cuh")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_p11616_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle", type=float, default=0.5,
                   help="seconds of untimed steps before the warm-up (clock ramp)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the sections measured outside the step: the P-sweep of the prefill "
                        "(memory and TFLOP/s at P = 1,944 .. 32,122), the packed varlen calls, "
                        "the paged decode, the causal GQA prefill and the FP8-cache decode")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time budget of the oracle baseline")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run 3 plain device-to-device copies of MIB MiB (reference kernel "
                        "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    p.add_argument("--decode-calls", type=int, default=0, metavar="N",
                   help="only run the decode workload on its bf16, E4M3 and INT8 caches N times each, "
                        "each call after a 512 MiB read (MALL flushed), and exit: the window the "
                        "decode counter profiles cover")
    p.add_argument("--api-calls", type=int, default=0, metavar="N",
                   help="only call every entry point of the step (and the allocation-free decode) N "
                        "times on preallocated buffers, between two device synchronisations, and "
                        "exit: the window a HIP runtime trace inspects for allocations and syncs")
    return p.parse_args()


def decode_calls(n):
    """The decode workload (B32, 32/8 heads, D128, 0.58 GB bf16 cache) on its bf16, E4M3 and INT8
    caches, n calls each, each after a 512 MiB read so that the MALL holds none of the cache."""
    import torch
    import masked_attention_attn_amd as ma
    import workloads as W
    ma.load()
    dev = torch.device("cuda:0")
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    for fmt in ("bf16", "fp8", "int8"):
        w = {"bf16": W.gqa_decode_b32, "fp8": W.gqa_decode_b32_fp8, "int8": W.gqa_decode_b32_int8}[fmt]()
        kc, vc, q = w.k_cache.to(dev), w.v_cache.to(dev), w.q.to(dev)
        lens = (w.lens + 1).to(dev)
        B, Hq, _, D = q.shape
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        ws = torch.empty(ma.attn_decode_workspace_bytes(B, Hq, kc.shape[1], kc.shape[2], D), dtype=torch.uint8,
                         device=dev)
        if fmt == "bf16":
            call = lambda: ma.attn_decode(q, kc, vc, lens, w.scale, out=o, lse=lse, workspace=ws, want_lse=True)
        else:
            ks, vs = w.k_scale.to(dev), w.v_scale.to(dev)
            fn = ma.attn_decode_fp8kv if fmt == "fp8" else ma.attn_decode_int8kv
            call = lambda: fn(q, kc, vc, ks, vs, lens, w.scale, out=o, lse=lse, workspace=ws, want_lse=True)
        for _ in range(n):
            flush.sum()
            call()
        torch.cuda.synchronize()
    print(json.dumps({"decode_calls": {"per_cache": n, "caches": ["bf16", "fp8", "int8"]}}))


def calibrate_copy(mib):
    import torch
    n = mib * 2**20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "copies": 3}))


LIB_SRCS = sorted(os.path.join(ROOT, "masked_attention_attn_amd", "csrc", f)
                  for f in os.listdir(os.path.join(ROOT, "masked_attention_attn_amd", "csrc")))


def file_sha(path):
    h = hashlib.sha256()
    with open(path, "rb") as f:
        for chunk in iter(lambda: f.read(1 << 20), b""):
            h.update(chunk)
    return h.hexdigest()[:16]


def src_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the prefill kernel from the committed rocprofv3 PMC
    summary, or None if it is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != src_hash(PREFILL_SRCS):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s):
    """Time the float64 oracle on whole heads of the prefill workload until the
    time budget is used (at least one head)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info()) if threadpool_info() else os.cpu_count()
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    B, H, Tq, D = w.q.shape
    n_valid = int((w.mask[0] == 0).sum())
    heads, t0 = 0, time.perf_counter()
    while heads < H:
        oracle.attention(w.q[:, heads:heads + 1], w.k[:, heads:heads + 1], w.v[:, heads:heads + 1],
                         w.mask, w.scale)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = oracle.attention_flops(heads, D, Tq, [n_valid])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {H} heads of the P=11,616 prefill (all {Tq} query rows each), "
                      f"float64 NumPy with the full masked softmax per head; {dt:.1f} s",
            "seconds": dt}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


SWEEP_P = (1944, 3952, 7776, 11616, 32122)   # the pages' patch counts, up to their OOM point
FLUSH_BYTES = 512 * 2**20                     # > the 256 MB MALL


def pct(xs, f):
    """The f-quantile of xs (nearest rank on the sorted values)."""
    ys = sorted(xs)
    return ys[min(len(ys) - 1, int(f * (len(ys) - 1) + 0.5))]


def dist_us(us):
    """mean / p10 / p50 / p90 of per-call durations in microseconds."""
    return {"mean": round(sum(us) / len(us), 2), "p10": round(pct(us, 0.1), 2), "p50": round(pct(us, 0.5), 2),
            "p90": round(pct(us, 0.9), 2), "n": len(us)}


def _time_call(torch, call, n=50, settle=0.3, flush=None):
    """Per-call durations (us) of n calls, each between two HIP events on the current stream,
    after `settle` seconds of untimed calls (the clocks drop while the host prepares the next
    inputs and need ~30 ms of work to ramp).  flush(), if given, runs before each timed call,
    outside its events.  Returns (mean seconds per call, mean/p10/p50/p90 in us)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle:
        for _ in range(3):
            call()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in ev:
        if flush is not None:
            flush()
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
    return sum(us) / len(us) / 1e6, dist_us(us)


def make_flush(torch, dev):
    """A read of FLUSH_BYTES of scratch (a sum over it): afterwards the MALL holds none of a
    decode's cache.  A read, not a write: written lines would stay dirty in the MALL and their
    write-back would run during the next timed call."""
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def flush():
        buf.sum()
    return flush


def smi_clocks(props=None):
    """Current sclk / mclk levels (the lines marked current in the amdgpu driver's pp_dpm_sclk and
    pp_dpm_mclk files) of the card whose PCI bus matches the device, else of the only AMD card
    listed; None where sysfs does not show them.  Read from sysfs, no child process: under a
    profiler that preloads itself into every process, a started tool would initialise the GPU."""
    import glob
    bus = getattr(props, "pci_bus_id", None)
    cards = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
        except OSError:
            continue
        addr = os.path.basename(os.path.realpath(dev))      # e.g. 0000:75:00.0
        if dev not in cards:
            cards.append((dev, addr))
    if bus is not None:
        match = [c for c in cards if int(c[1].split(":")[1], 16) == int(bus)]
    else:
        match = cards if len(cards) == 1 else []
    if not match:
        return None
    out = {"pci": match[0][1]}
    for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
        try:
            with open(os.path.join(match[0][0], name)) as f:
                cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
            out[name] = cur[0] if cur else None
        except OSError:
            out[name] = None
    return out


def gpu_info(torch, dev, busy_step):
    """Device name, CU count and memory, plus the clock levels read while the GPU runs
    queued bench steps (so they are the clocks under this load, not idle ones)."""
    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "total_memory_bytes": int(p.total_memory)}
    for _ in range(200):       # ~0.4 s of queued work
        busy_step()
    info["clocks_under_load"] = smi_clocks(p)
    torch.cuda.synchronize()
    return info


def p_sweep(torch, ma, dev):
    """Masked prefill with LSE, bf16, B1 H16 D64, last 16 keys padded, at each P: measured peak
    extra device memory of one call, its time, and the score matrix a materialising path holds.

    Around one call (O and LSE allocated by the caller, as a user would), after the inputs
    are resident: torch's peak allocated and reserved bytes above the pre-call level
    (reset_peak_memory_stats first), and the drop in the device's free memory (mem_get_info),
    which would also show any allocation made outside torch, i.e. by the library.  The
    library's own share is that drop minus torch's reserve growth.  The line fitted over P is
    through the measured peak allocated bytes."""
    rows = []
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    H, D = 16, 64
    for P in SWEEP_P:
        q, k, v = (torch.randn(1, H, P, D, device=dev, generator=g).mul_(0.5).to(torch.bfloat16)
                   for _ in range(3))
        mask = torch.zeros(1, P, dtype=torch.uint8, device=dev)
        mask[0, P - 16:] = 1
        ma.attn_fwd_lse(q, k, v, mask, D ** -0.5)      # code objects loaded, then the outputs freed
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base_alloc, base_res = torch.cuda.memory_allocated(dev), torch.cuda.memory_reserved(dev)
        free0 = torch.cuda.mem_get_info(dev)[0]
        o = torch.empty_like(q)
        lse = torch.empty(1, H, P, dtype=torch.float32, device=dev)
        ma.attn_fwd_lse(q, k, v, mask, D ** -0.5, out=o, lse=lse)
        torch.cuda.synchronize()
        peak_alloc = torch.cuda.max_memory_allocated(dev) - base_alloc
        peak_res = torch.cuda.max_memory_reserved(dev) - base_res
        drop = free0 - torch.cuda.mem_get_info(dev)[0]
        lib_bytes = drop - (torch.cuda.memory_reserved(dev) - base_res)
        call = lambda: ma.attn_fwd_lse(q, k, v, mask, D ** -0.5, out=o, lse=lse)
        t, d = _time_call(torch, call)
        flop = 4 * D * H * P * (P - 16)
        rows.append({"P": P, "us": d, "tflops": round(flop / t / 1e12, 1),
                     "measured_peak_allocated_bytes": int(peak_alloc),
                     "measured_peak_reserved_bytes": int(peak_res),
                     "measured_device_free_drop_bytes": int(drop),
                     "library_allocated_bytes": int(lib_bytes),
                     "o_plus_lse_bytes": o.numel() * 2 + lse.numel() * 4,
                     "score_matrix_bytes_avoided": H * P * P * 2})
        del q, k, v, mask, o, lse
        torch.cuda.empty_cache()
    # measured peak bytes against P: least-squares line and its worst residual
    xs = [r["P"] for r in rows]
    ys = [r["measured_peak_allocated_bytes"] for r in rows]
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    a = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    c = my - a * mx
    resid = max(abs(y - (a * x + c)) for x, y in zip(xs, ys))
    return {"workload": "masked prefill with LSE, bf16, B1 H16 D64, last 16 keys padded, N(0,1)*0.5",
            "rows": rows, "fit_measured_peak_bytes_per_P": round(a, 3),
            "fit_measured_peak_intercept_bytes": round(c, 1), "fit_max_abs_residual_bytes": round(resid, 1),
            "score_matrix_bytes_per_P_at_32122": 16 * 32122 * 2}


def fp32_section(torch, ma, W, dev):
    """The fp32 masked forward with LSE (B1 H16 T512 D64, last 48 keys padded), timed on its own.
    It runs on the vector ALU (fp32 fma, one product per instruction): against the published fp32
    vector peak, whose figure counts packed fp32 FMAs, twice what unpacked instructions reach.
    FLOP are algorithmic: 4·D·H·Tq·n_valid."""
    w = W.fp32_masked_t512()
    q, k, v, m = (t.to(dev) for t in (w.q, w.k, w.v, w.mask))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    t, d = _time_call(torch, lambda: ma.attn_fwd_lse(q, k, v, m, w.scale, out=o, lse=lse))
    B, H, Tq, D = q.shape
    n_valid = int((w.mask[0] == 0).sum())
    flop = 4 * D * H * Tq * n_valid
    return {"workload": "fp32 masked prefill with LSE, B1 H16 T512 D64, last 48 keys padded", "us": d,
            "tflops": round(flop / t / 1e12, 2), "bound": "alu",
            "frac_alu": round(flop / t / 1e12 / PEAK_FP32_VECTOR_TFLOPS, 4),
            "peak_tflops": PEAK_FP32_VECTOR_TFLOPS, "algorithmic_flop": flop}


def varlen_section(torch, ma, W, dev):
    """Packed variable-length calls (attn_fwd_varlen), each timed on its own:
      * the P = 1,944 pair (1,944 and 1,700 patches, H16 D64) packed, beside the same pair
        through the masked [B, H, T, D] path, where the 244 padded query rows and the padded
        keys of the second sequence are computed or skipped per block;
      * one ring hop: 8,192 packed queries against an 8,192-key chunk, H24 D128, with LSE.
    FLOP are algorithmic: 4·D·H·sum_b len_q,b·len_k,b."""
    res = {}
    for name, w in (("p1944_packed", W.varlen_p1944_packed()), ("ring_hop_8192", W.varlen_ring_hop_8192())):
        q, k, v, cq, ck = (t.to(dev) for t in (w.q, w.k, w.v, w.cu_q, w.cu_k))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=dev)
        t, d = _time_call(torch, lambda: ma.attn_fwd_varlen(q, k, v, cq, ck, w.max_q, w.scale, out=o, lse=lse))
        H, D = q.shape[1], q.shape[2]
        flop = 4 * D * H * sum(a * b for a, b in zip(w.lens_q, w.lens_k))
        res[name] = {"workload": w.name, "us": d, "tflops": round(flop / t / 1e12, 1),
                     "frac_mfma": round(flop / t / 1e12 / PEAK_BF16_TFLOPS, 4), "algorithmic_flop": flop}
        del q, k, v, cq, ck, o, lse
    pd = W.patch_p1944()
    q, k, v, m = (t.to(dev) for t in (pd.q, pd.k, pd.v, pd.mask))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    t, d = _time_call(torch, lambda: ma.attn_fwd_lse(q, k, v, m, pd.scale, out=o, lse=lse))
    res["p1944_padded_masked_us"] = d
    return res


def paged_section(torch, ma, W, dev, flush):
    """The decode workload (B32, H_q 32 / H_kv 8, D128, len U[512, 8192] + 1) with its cache in a
    shuffled page pool (attn_decode_paged), per page size, and with an E4M3 cache in 16-token
    pages (attn_decode_fp8kv_paged), each timed on its own; bytes as the contiguous decodes (K
    and V of every cached token, plus q and o)."""
    res = {}
    for ps in (16, 64):
        pg = W.gqa_decode_b32_paged(ps)
        w = pg.dec
        kp, vp, bt = pg.k_pages.to(dev), pg.v_pages.to(dev), pg.block_table.to(dev)
        lens = (w.lens + 1).to(dev)
        q = w.q.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        B, Hq, _, D = q.shape
        Hkv = kp.shape[1]
        ws = torch.empty(ma.attn_decode_workspace_bytes(B, Hq, Hkv, bt.shape[1] * ps, D), dtype=torch.uint8,
                         device=dev)
        t, d = _time_call(torch, lambda: ma.attn_decode_paged(q, kp, vp, bt, lens, w.scale, out=o, lse=lse,
                                                              workspace=ws, want_lse=True), flush=flush)
        nbytes = int((w.lens + 1).sum()) * 2 * Hkv * D * 2 + 2 * q.numel() * 2
        res[f"page_{ps}"] = {"us": d, "gbps": round(nbytes / t / 1e9, 1),
                             "frac_hbm": round(nbytes / t / 1e9 / PEAK_HBM_GBPS, 4)}
        del kp, vp, bt, lens, q, o, lse, ws
    # the same workload with an E4M3 cache in 16-token pages (attn_decode_fp8kv_paged)
    w = W.gqa_decode_b32_fp8()
    pg = W.to_paged(w, 16)
    kp, vp, bt = pg.k_pages.to(dev), pg.v_pages.to(dev), pg.block_table.to(dev)
    ks, vs, lens, q = w.k_scale.to(dev), w.v_scale.to(dev), (w.lens + 1).to(dev), w.q.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    B, Hq, _, D = q.shape
    Hkv = kp.shape[1]
    ws = torch.empty(ma.attn_decode_workspace_bytes(B, Hq, Hkv, bt.shape[1] * 16, D), dtype=torch.uint8, device=dev)
    t, d = _time_call(torch, lambda: ma.attn_decode_fp8kv_paged(q, kp, vp, ks, vs, bt, lens, w.scale, out=o,
                                                                lse=lse, workspace=ws, want_lse=True), flush=flush)
    nbytes = int((w.lens + 1).sum()) * 2 * Hkv * D + 2 * q.numel() * 2
    res["fp8_page_16"] = {"us": d, "gbps": round(nbytes / t / 1e9, 1),
                          "frac_hbm": round(nbytes / t / 1e9 / PEAK_HBM_GBPS, 4)}
    return res


def fp8_section(torch, ma, W, dev, flush, int8=False):
    """The decode workload with an E4M3 cache (attn_decode_fp8kv; per-(sequence, KV head) scales),
    or an INT8 cache (attn_decode_int8kv), timed on its own after the append; bytes: one byte per
    cached K and V element, plus q and o."""
    w = W.gqa_decode_b32_int8() if int8 else W.gqa_decode_b32_fp8()
    decode_fn = ma.attn_decode_int8kv if int8 else ma.attn_decode_fp8kv
    kc, vc, ks, vs = w.k_cache.to(dev), w.v_cache.to(dev), w.k_scale.to(dev), w.v_scale.to(dev)
    lens = (w.lens + 1).to(dev)
    q = w.q.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    B, Hq, _, D = q.shape
    Hkv, Tm = kc.shape[1], kc.shape[2]
    ws = torch.empty(ma.attn_decode_workspace_bytes(B, Hq, Hkv, Tm, D), dtype=torch.uint8, device=dev)
    t, d = _time_call(torch, lambda: decode_fn(q, kc, vc, ks, vs, lens, w.scale, out=o, lse=lse,
                                               workspace=ws, want_lse=True), flush=flush)
    nbytes = int((w.lens + 1).sum()) * 2 * Hkv * D + 2 * q.numel() * 2
    return {"workload": w.name, "us": d, "gbps": round(nbytes / t / 1e9, 1),
            "frac_hbm": round(nbytes / t / 1e9 / PEAK_HBM_GBPS, 4), "algorithmic_bytes": nbytes}


def fp8_prefill_section(torch, ma, W, dev):
    """E4M3-input prefill with LSE, each timed on its own: the P = 11,616 patch shape (non-causal,
    padded keys) and the causal GQA 8,192-token prompt (attn_prefill_fp8), and the packed ring hop
    (attn_prefill_varlen_fp8).  FLOP are algorithmic
    as for the bf16 calls; frac_mfma is against the split fp8 / bf16 matrix-core bound."""
    res = {}
    for key, w, causal in (("p11616", W.patch_p11616_fp8(), False),
                           ("causal_prompt_8192", W.gqa_causal_prefill_8192_fp8(), True)):
        q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
        qs, ks, vs = w.q_scale.to(dev), w.k_scale.to(dev), w.v_scale.to(dev)
        m = w.mask.to(dev) if w.mask is not None else None
        B, Hq, T, D = q.shape
        o = torch.empty((B, Hq, T, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
        t, d = _time_call(torch, lambda: ma.attn_prefill_fp8(q, k, v, qs, ks, vs, m, causal, w.scale, out=o, lse=lse))
        if causal:
            flop = 4 * D * Hq * B * T * (T + 1) // 2
        else:
            n_valid = [int((w.mask[b] == 0).sum()) if w.mask is not None else T for b in range(B)]
            flop = 4 * D * Hq * T * sum(n_valid)
        res[key] = {"workload": w.name, "us": d, "tflops": round(flop / t / 1e12, 1),
                    "frac_mfma": round(flop / t / 1e12 / PEAK_FP8_PREFILL_TFLOPS, 4),
                    "peak_tflops": round(PEAK_FP8_PREFILL_TFLOPS, 1), "algorithmic_flop": flop}
        del q, k, v, o, lse
    # the packed ring hop (attn_prefill_varlen_fp8)
    w = W.varlen_ring_hop_8192_fp8()
    q, k, v, qs, ks, vs, cq, ck = (t_.to(dev) for t_ in (w.q, w.k, w.v, w.q_scale, w.k_scale, w.v_scale, w.cu_q,
                                                          w.cu_k))
    tq, Hq, D = q.shape
    o = torch.empty((tq, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, tq), dtype=torch.float32, device=dev)
    t, d = _time_call(torch, lambda: ma.attn_prefill_varlen_fp8(q, k, v, qs, ks, vs, cq, ck, w.max_q, False,
                                                                w.scale, out=o, lse=lse))
    flop = 4 * D * Hq * sum(a * b for a, b in zip(w.cu_q.diff().tolist(), w.cu_k.diff().tolist()))
    res["ring_hop_8192"] = {"workload": w.name, "us": d, "tflops": round(flop / t / 1e12, 1),
                            "frac_mfma": round(flop / t / 1e12 / PEAK_FP8_PREFILL_TFLOPS, 4),
                            "peak_tflops": round(PEAK_FP8_PREFILL_TFLOPS, 1), "algorithmic_flop": flop}
    return res


def causal_section(torch, ma, W, dev):
    """Causal GQA prompt passes (attn_prefill / attn_prefill_varlen, H_q 32 / H_kv 8, D128), each
    timed on its own: one 8,192-token prompt, and 8 packed prompts of 1,024 .. 4,096 tokens.
    FLOP are algorithmic: 4·D·H_q per (query, visible key) pair, T(T+1)/2 pairs per prompt."""
    res = {}
    w = W.gqa_causal_prefill_8192()
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    t, d = _time_call(torch, lambda: ma.attn_prefill(q, k, v, None, True, w.scale, out=o, lse=lse))
    B, Hq, T, D = q.shape
    flop = 4 * D * Hq * B * T * (T + 1) // 2
    res["prompt_8192"] = {"workload": w.name, "us": d, "tflops": round(flop / t / 1e12, 1),
                          "frac_mfma": round(flop / t / 1e12 / PEAK_BF16_TFLOPS, 4), "algorithmic_flop": flop}
    del q, k, v, o, lse
    w = W.gqa_causal_prompts_packed()
    q, k, v, cq, ck = (t_.to(dev) for t_ in (w.q, w.k, w.v, w.cu_q, w.cu_k))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=dev)
    t, d = _time_call(torch, lambda: ma.attn_prefill_varlen(q, k, v, cq, ck, w.max_q, True, w.scale, out=o,
                                                            lse=lse))
    flop = 4 * 128 * 32 * sum(n * (n + 1) // 2 for n in w.lens_q)
    res["packed_prompts"] = {"workload": w.name, "us": d, "tflops": round(flop / t / 1e12, 1),
                             "frac_mfma": round(flop / t / 1e12 / PEAK_BF16_TFLOPS, 4), "algorithmic_flop": flop}
    return res


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.decode_calls:
        decode_calls(args.decode_calls)
        return

    import torch
    import masked_attention_attn_amd as ma
    import workloads as W

    if not os.path.exists(ma.LIB_PATH):
        raise SystemExit(f"{ma.LIB_PATH} is not built: run python __graft_entry__.py first")
    ma.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs (host generation, then resident on the device)
    pf = W.patch_p11616()
    ch = W.chunked_kv_2x8192()
    dc = W.gqa_decode_b32()
    q3, k3, v3, m3 = (t.to(dev) for t in (pf.q, pf.k, pf.v, pf.mask))
    o3 = torch.empty_like(q3)
    l3 = torch.empty(q3.shape[:3], dtype=torch.float32, device=dev)
    q4 = ch.q.to(dev)
    k4 = [t.to(dev) for t in ch.k_chunks]
    v4 = [t.to(dev) for t in ch.v_chunks]
    o4 = [torch.empty_like(q4) for _ in range(2)]
    l4 = [torch.empty(q4.shape[:3], dtype=torch.float32, device=dev) for _ in range(2)]
    om4 = torch.empty_like(q4)
    lm4 = torch.empty(q4.shape[:3], dtype=torch.float32, device=dev)
    kc, vc = dc.k_cache.to(dev), dc.v_cache.to(dev)
    kn, vn, q5 = dc.k_new.to(dev), dc.v_new.to(dev), dc.q.to(dev)
    lens0 = dc.lens.to(dev)
    lens = lens0.clone()
    o5 = torch.empty_like(q5)
    l5 = torch.empty(q5.shape[:2], dtype=torch.float32, device=dev)
    B5, Hq5, _, D5 = q5.shape
    Hkv5, Tmax5 = kc.shape[1], kc.shape[2]
    ws = torch.empty(ma.attn_decode_workspace_bytes(B5, Hq5, Hkv5, Tmax5, D5), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    n_ev = 6

    if args.api_calls:
        # Warm-up (the library's one-time set-up: kernel attributes, occupancy query, the
        # static scratch's address), then the window: nothing but entry-point calls on
        # buffers allocated above, between two device synchronisations.
        def calls():
            ma.attn_fwd_lse(q3, k3, v3, m3, pf.scale, out=o3, lse=l3)
            for i in range(2):
                ma.attn_fwd_lse(q4, k4[i], v4[i], None, ch.scale, out=o4[i], lse=l4[i])
            ma.attn_merge_lse(o4, l4, out=om4, lse_out=lm4)
            ma.kv_append(kc, vc, lens, kn, vn)
            ma.attn_decode(q5, kc, vc, lens, dc.scale, out=o5, lse=l5, workspace=ws, want_lse=True)
            ma.attn_decode_noalloc(q5, kc, vc, lens, o5, l5, scale=dc.scale)
        calls()
        torch.cuda.synchronize()
        for _ in range(args.api_calls):
            calls()
        torch.cuda.synchronize()
        print(json.dumps({"api_call_window": {"iterations": args.api_calls,
                                              "entry_points_per_iteration": 7}}))
        return

    def step(ev=None):
        lens.copy_(lens0)
        if ev: ev[0].record(stream)
        ma.attn_fwd_lse(q3, k3, v3, m3, pf.scale, out=o3, lse=l3)
        if ev: ev[1].record(stream)
        for i in range(2):
            ma.attn_fwd_lse(q4, k4[i], v4[i], None, ch.scale, out=o4[i], lse=l4[i])
        if ev: ev[2].record(stream)
        ma.attn_merge_lse(o4, l4, out=om4, lse_out=lm4)
        if ev: ev[3].record(stream)
        ma.kv_append(kc, vc, lens, kn, vn)
        if ev: ev[4].record(stream)
        ma.attn_decode(q5, kc, vc, lens, dc.scale, out=o5, lse=l5, workspace=ws, want_lse=True)
        if ev: ev[5].record(stream)

    # The GPU clocks ramp up over the first ~30 ms of continuous work and drop
    # again after idling; run untimed steps for --settle seconds first so the
    # timed steps see the steady-state clock.
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < args.settle:
        step()
        n_settle += 1
        if n_settle % 4 == 0:
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()       # with W >= 1, code objects are loaded before free memory is read
    free_before = torch.cuda.mem_get_info()[0]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    free_after = torch.cuda.mem_get_info()[0]

    def spans(a, b):
        return [events[s_][a].elapsed_time(events[s_][b]) * 1e3 for s_ in range(args.steps)]   # us per step

    d_prefill, d_chunks, d_merge, d_append, d_decode = (spans(0, 1), spans(1, 2), spans(2, 3), spans(3, 4),
                                                        spans(4, 5))
    mean_s = lambda us: sum(us) / len(us) / 1e6
    t_prefill, t_chunks, t_merge, t_append, t_decode = (mean_s(d) for d in (d_prefill, d_chunks, d_merge,
                                                                              d_append, d_decode))
    # ---- algorithmic work
    B, H, P, D = pf.q.shape
    n_valid = int((pf.mask[0] == 0).sum())
    flop_prefill = 4 * D * H * P * n_valid
    tf_prefill = flop_prefill / t_prefill / 1e12
    Hc, Tqc, Dc = ch.q.shape[1], ch.q.shape[2], ch.q.shape[3]
    flop_chunks = 2 * 4 * Dc * Hc * Tqc * ch.k_chunks[0].shape[2]
    merge_bytes = (2 * (om4.numel() * 2 + lm4.numel() * 4)) + om4.numel() * 2 + lm4.numel() * 4
    lens_after = dc.lens.long() + 1
    kv_bytes = int(lens_after.sum().item()) * 2 * Hkv5 * D5 * 2
    decode_bytes = kv_bytes + q5.numel() * 2 + o5.numel() * 2
    decode_gbps = decode_bytes / t_decode / 1e9
    traffic = measured_traffic()

    # ---- the decode on its own, with the MALL flushed before every call
    flush = make_flush(torch, dev)
    lens_ready = (lens0 + 1).to(torch.int32)
    t_dec_flushed, d_dec_flushed = _time_call(
        torch, lambda: ma.attn_decode(q5, kc, vc, lens_ready, dc.scale, out=o5, lse=l5, workspace=ws, want_lse=True),
        flush=flush)

    # ---- device identity and clocks under this load (outside the timed region)
    gpu = gpu_info(torch, dev, step)

    prefill_extra = o3.numel() * o3.element_size() + l3.numel() * 4
    out = {
        "metric": "masked attn prefill TFLOP/s @P=11,616 (frac MFMA peak); decode HBM GB/s",
        "value": round(tf_prefill, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"seconds": args.settle, "untimed_steps": n_settle},
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs in the shapes the pages measure)",
        "config": {
            "workload": "masked patch self-attention prefill with LSE, bf16, B1 H16 P11616 D64, "
                        "last 16 keys padded, inputs N(0,1)*0.5",
            "B": B, "H": H, "P": P, "D": D, "n_valid_keys": n_valid,
            "also_in_step": ["chunked KV: Q 8192 x H24 x D128 vs 2 x 8192 keys + LSE merge",
                             "decode: kv_append + attn_decode, B32 Hq32 Hkv8 D128, len U[512,8192]+1"],
        },
        "roofline": {
            "bound": "mfma", "kernel": "fwd_bf16_kernel<64, LSE>",
            "achieved": round(tf_prefill, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf_prefill / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
            "algorithmic_flop_per_launch": flop_prefill, "avg_launch_us": round(t_prefill * 1e6, 2),
            "launch_us": dist_us(d_prefill),
            "exps_per_launch": H * P * n_valid,
            "exp_rate_Gexp_per_s": round(H * P * n_valid / t_prefill / 1e9, 1),
        },
        "decode": {
            "metric": "decode HBM GB/s", "value": round(decode_gbps, 1), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(decode_gbps, 1), "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(decode_gbps / PEAK_HBM_GBPS, 4),
                         "algorithmic_bytes_per_launch": decode_bytes},
            "attn_decode_us": dist_us(d_decode), "kv_append_us": dist_us(d_append),
            "standalone_mall_flushed": {"us": d_dec_flushed,
                                        "gbps": round(decode_bytes / t_dec_flushed / 1e9, 1),
                                        "frac_hbm": round(decode_bytes / t_dec_flushed / 1e9 / PEAK_HBM_GBPS, 4)},
            "cached_tokens": int(lens_after.sum().item()),
        },
        "chunked": {
            "fwd_lse_x2_us": dist_us(d_chunks),
            "tflops": round(flop_chunks / t_chunks / 1e12, 2),
            "frac_mfma": round(flop_chunks / t_chunks / 1e12 / PEAK_BF16_TFLOPS, 4),
            "merge_us": dist_us(d_merge),
            "merge_gbps": round(merge_bytes / t_merge / 1e9, 1),
            "merge_frac_hbm": round(merge_bytes / t_merge / 1e9 / PEAK_HBM_GBPS, 4),
        },
        "memory": {
            "device_free_drop_across_timed_steps_bytes": int(free_before - free_after),
            "prefill_call_extra_bytes": int(prefill_extra),
            "prefill_call_extra_GB": round(prefill_extra / 1e9, 4),
            "avoided_score_matrix_bytes": H * P * P * 2,
            "decode_workspace_bytes": int(ws.numel()),
        },
        "library": {"path": os.path.relpath(ma.LIB_PATH, ROOT), "sha256_16": file_sha(ma.LIB_PATH),
                    "kernel_sources_sha256_16": src_hash(LIB_SRCS),
                    "prefill_kernel_sources_sha256_16": src_hash(PREFILL_SRCS)},
        "gpu": gpu,
    }
    if not args.no_sweep:
        out["p_sweep"] = p_sweep(torch, ma, dev)
        out["fp32_prefill"] = fp32_section(torch, ma, W, dev)
        out["varlen"] = varlen_section(torch, ma, W, dev)
        out["paged_decode"] = paged_section(torch, ma, W, dev, flush)
        out["causal_gqa_prefill"] = causal_section(torch, ma, W, dev)
        out["fp8_kv_decode"] = fp8_section(torch, ma, W, dev, flush)
        out["int8_kv_decode"] = fp8_section(torch, ma, W, dev, flush, int8=True)
        out["fp8_prefill"] = fp8_prefill_section(torch, ma, W, dev)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(pf, args.cpu_seconds)
        cb.pop("seconds", None)
        cb["cpu_model"] = cpu_model()
        out["cpu_baseline"] = cb
    print(json.dumps(out))


if __name__ == "__main__":
    main()
