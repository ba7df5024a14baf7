#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one attn_fwd call over the whole workload (every step of the
method runs inside it): the default workload is causal GQA, B=4, Hq=32,
Hkv=8, S=4096, d=128, bf16. Inputs are seeded synthetic N(0,1) tensors already
resident in HBM before timing starts. Prints one JSON line with the
causal-adjusted TFLOP/s, the roofline of the kernel (achieved / peak dense
MFMA rate, from HIP events around every launch on the launch stream) and the
fp64 CPU oracle timed on a bounded sample of the same workload.

Timing mirrors the codelab's benchmark helper ("Accelerate attention on GPU
with cuDNN and TransformerEngine", section 8: warm-up calls first, inputs
already on the device, warm caches), with device events instead of host time.

--workload takes any name of sdpa_inputs.WORKLOADS. The decode workload runs
the split-KV path (one step = the chunk kernel plus the merge kernel), the
backward workload one attn_bwd call (delta, dQ and dK/dV kernels; its FLOP are
the five products of the backward pass, 2.5 times the forward's); a
workload whose arithmetic intensity is below the ridge point reports the HBM
roofline (algorithmic bytes per launch over the launch time) instead of the
matrix-core one.

Before timing, --warmup calls run and then more calls until --warm-seconds
(default 1 s) of launches have passed, so the clocks are those of a
sustained run. The line also carries the distribution of single launches
(median / min / p90, events around each call), the CU count and peak clock,
the achieved clock and matrix-core / vector-unit / LDS utilisation from the
committed counter summary of the same kernel sources, and the seed. The CPU baseline runs the oracle on a pool of host
threads and reports the GPU output's error on the heads it computed.

Other modes:
    --no-cpu-baseline        skip the oracle timing
    --copy-calibration MIB   run a plain device copy of MIB MiB (to calibrate HBM byte counters)
    --sweep                  the codelab's own benchmark shapes (one JSON line per shape, see sweep_shapes)
    --eager                  time forward steps as K separate calls with events around each (default: one HIP
                             graph of the K launches, replayed once)
    --mfma-peak              the matrix-core ceiling: bf16, fp8 and fp32 MFMA streams on register operands, one and
                             two waves per SIMD (libmfmapeak.so), one JSON line per case
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (causal-adjusted) and % of MFMA peak, 1 MI355X"
METRIC_BWD = "attention bwd TFLOP/s (causal-adjusted, five products) and % of MFMA peak, 1 MI355X"

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0

CSRC = os.path.join(ROOT, "scaled_dot_product_18_amd", "csrc")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# Source file of each kernel family; its counter summaries are keyed on it.
KERNEL_SOURCES = {"attn_fwd_bf16_pp_kernel": "attn_fwd_bf16_pp.hip", "attn_fwd_bf16_kernel": "attn_fwd_bf16.hip",
                  "attn_fwd_ppk_kernel": "attn_fwd_ppk.hip",
                  "attn_fwd_fp8_pp_kernel": "attn_fwd_fp8_pp.hip",
                  "attn_fwd_mfma_kernel": "attn_fwd_mfma.hip", "attn_fwd_f32_kernel": "attn_fwd_f32.hip",
                  "attn_fwd_f32_split_kernel": "attn_fwd_f32.hip",
                  "attn_fwd_splitkv_kernel": "attn_fwd_splitkv.hip", "attn_bwd_dkdv_kernel": "attn_bwd.hip"}
SHARED_SOURCES = ("kernel_common.h", "launch.h", "attn_api.cpp")


def kernel_source_hash(kernel: str) -> str:
    """sha256 (16 hex digits) over a kernel's source file and the sources every
    launch shares: a counter summary taken on other sources no longer
    describes the kernel."""
    h = hashlib.sha256()
    for fn in (KERNEL_SOURCES[kernel],) + SHARED_SOURCES:
        h.update(fn.encode())
        with open(os.path.join(CSRC, fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_name(w) -> str:
    if w.path == "splitkv":
        return "attn_fwd_splitkv_kernel"
    if w.path == "bwd":
        return "attn_bwd_dkdv_kernel"
    if w.dtype in ("bf16", "fp8") and w.d == 128 and (w.Sq + 127) // 128 * w.B * w.Hq <= (512 if w.causal else 256):
        return "attn_fwd_ppk_kernel"  # small grids of 128-row tiles: key halves
    if w.dtype == "bf16" and w.d == 128:
        return "attn_fwd_bf16_pp_kernel"
    if w.d == 64 and w.Sk >= 1024 and (w.dtype == "fp8" or (w.dtype == "bf16" and (w.Sq + 127) // 128 * w.B * w.Hq <= 768)):
        return "attn_fwd_ppk_kernel"  # d = 64 over 1024+ keys (bf16: grids of up to 768 workgroups)
    if w.dtype == "fp8" and w.d == 128:
        return "attn_fwd_fp8_pp_kernel"
    if w.dtype == "f32" and (w.Sq + 127) // 128 * w.B * w.Hq <= 128 and w.Sk > 32:
        return "attn_fwd_f32_split_kernel"  # grids up to 128 workgroups of 128 rows split the keys
    return {"f32": "attn_fwd_f32_kernel", "bf16": "attn_fwd_bf16_kernel", "fp8": "attn_fwd_mfma_kernel"}[w.dtype]


def traffic_from_profiles(w):
    """HBM bytes per launch from the committed counter summary
    profiles/<kernel>_<workload>_hbm.txt, or None when it is missing or was
    taken on other kernel sources. The file holds 'key: value' lines; the
    ones read here are kernel_source_sha and hbm_bytes_per_launch."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name(w)}_{w.name}_hbm.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            key, sep, val = line.partition(":")
            if sep:
                rec[key.strip()] = val.strip()
    if rec.get("kernel_source_sha") != kernel_source_hash(kernel_name(w)):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def counters_from_profiles(w):
    """Achieved clock and unit utilisation of the kernel from the committed
    counter summary profiles/<kernel>_<workload>_sq.txt (one rocprofv3 --pmc
    pass of GRBM_GUI_ACTIVE and SQ counters), or None when it is missing or was
    taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name(w)}_{w.name}_sq.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            key, sep, val = line.partition(":")
            if sep and not key.startswith("#"):
                rec[key.strip()] = val.strip()
    if rec.get("kernel_source_sha") != kernel_source_hash(kernel_name(w)):
        return None
    out = {}
    for key in ("achieved_clock_mhz", "mfma_busy_pct", "valu_busy_pct", "lds_active_pct", "lds_bank_conflict_pct",
                "mfma_valu_coexec_pct"):
        try:
            out[key] = float(rec[key])
        except (KeyError, ValueError):
            out[key] = None
    out["source"] = os.path.relpath(path, ROOT)
    return out


def cpu_baseline(w, inp, budget_s: float = 15.0, gpu_out=None, gpu_lse=None) -> dict:
    """Time the fp64 oracle on whole (batch, head) pairs of the same inputs, on a
    pool of host threads (one (b, h) pair per task, one BLAS thread each), until
    the budget is spent. When the GPU's output is given, also report its max and
    mean |GPU - oracle| over the pairs the oracle computed."""
    import threading
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    import oracle
    from oracle import e4m3

    workers = max(1, min(16, os.cpu_count() or 1))
    G = w.Hq // w.Hkv

    def as64(t, name):
        if w.dtype == "fp8":
            return e4m3.dequantise(t.numpy(), inp["descale_" + name])
        return t.to(torch.float64).numpy()

    o_cpu = gpu_out.to(torch.float64).cpu() if gpu_out is not None else None
    l_cpu = gpu_lse.to(torch.float64).cpu() if gpu_lse is not None else None
    lock = threading.Lock()
    done = {"heads": 0, "t_last": 0.0, "err_max": 0.0, "err_sum": 0.0, "err_n": 0, "lse_max": 0.0}
    t0 = time.perf_counter()

    def one(b, h):
        if time.perf_counter() - t0 >= budget_s:
            return
        q = as64(inp["q"][b, h], "q")[None, None]
        k = as64(inp["k"][b, h // G], "k")[None, None]
        v = as64(inp["v"][b, h // G], "v")[None, None]
        if w.path == "bwd":
            oracle.attention_backward(q, k, v, inp["dout"][b, h].to(torch.float64).numpy()[None, None],
                                      w.scale, w.causal)
            o_ref = lse_ref = None
        else:
            o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal)
        t = time.perf_counter() - t0
        with lock:
            done["heads"] += 1
            done["t_last"] = max(done["t_last"], t)
            if o_ref is not None and o_cpu is not None:
                err = np.abs(o_cpu[b, h].numpy() - o_ref[0, 0])
                done["err_max"] = max(done["err_max"], float(err.max()))
                done["err_sum"] += float(err.sum())
                done["err_n"] += err.size
                if l_cpu is not None:
                    done["lse_max"] = max(done["lse_max"], float(np.abs(l_cpu[b, h].numpy() - lse_ref[0, 0]).max()))

    try:
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits(1)
    except Exception:
        limit = None
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(lambda bh: one(*bh), [(b, h) for b in range(w.B) for h in range(w.Hq)]))
    finally:
        if limit is not None:
            limit.unregister() if hasattr(limit, "unregister") else limit.__exit__(None, None, None)
    elapsed = max(done["t_last"], 1e-9)
    heads = done["heads"]
    flop_per_head = w.flops() / (w.B * w.Hq)
    rec = {"value": flop_per_head * heads / elapsed / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
           "sample": f"{heads} of {w.B * w.Hq} (batch, head) pairs of the same workload, full fp64 oracle, "
                     f"{workers} host threads (one pair per task, one BLAS thread each), {elapsed:.1f} s wall; "
                     "FLOP counted causal-adjusted like the GPU value",
           "cpu": platform.processor() or platform.machine(), "os_cpu_count": os.cpu_count()}
    if done["err_n"]:
        rec["gpu_vs_oracle"] = {"heads": heads, "max_abs_err_o": done["err_max"],
                                "mean_abs_err_o": done["err_sum"] / done["err_n"],
                                "max_abs_err_lse": done["lse_max"] if l_cpu is not None else None}
    return rec


def hip_clock_rate_mhz():
    """Peak clock the HIP runtime reports for device 0 (hipDeviceAttributeClockRate, kHz)."""
    try:
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0:  # 5 = hipDeviceAttributeClockRate
            return val.value / 1000.0
    except Exception:
        pass
    return None


def percentile(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(math.ceil(q * len(xs))) - 1))]


def copy_calibration(mib: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))


def sweep_shapes():
    """The benchmark cells of the codelab ("Accelerate attention on GPU with cuDNN
    and TransformerEngine"): its base shape is B=4, N=8 heads, head dim 64
    (section 3); section 8 sweeps the sequence length over 64..1024 and the batch
    over 1..16 at T=256, unmasked, in fp32 and bf16; the TransformerEngine cell
    sweeps causal bf16 over T=128..2048; the FP8 cell runs causal attention at
    T=2048. Its closing next steps try head dimensions 32, 64 and 128 (here in
    fp32, bf16 and fp8 at T=1024, unmasked and causal) and re-run the MHA / GQA /
    MQA cell (8 query heads against 8, 2 and 1 KV heads; section 9's cell is
    B=2, T=64) at longer sequences. Seeds follow the cells' key numbers (sl,
    bs + 100, sl + 1000, 9000, 42). Returns (sweep name, Workload) pairs in the
    library's [B, H, S, d] layout."""
    import sdpa_inputs
    B, N, H = 4, 8, 64
    out = []
    for dtype in ("f32", "bf16"):
        for sl in (64, 128, 256, 512, 1024):
            out.append(("seq_len", sdpa_inputs.custom(B, N, N, sl, sl, H, dtype, False, seed=sl,
                                                      name=f"seq_len_{dtype}_b{B}_t{sl}")))
        for bs in (1, 2, 4, 8, 16):
            out.append(("batch", sdpa_inputs.custom(bs, N, N, 256, 256, H, dtype, False, seed=bs + 100,
                                                    name=f"batch_{dtype}_b{bs}_t256")))
    for sl in (128, 256, 512, 1024, 2048):
        out.append(("causal_bf16", sdpa_inputs.custom(B, N, N, sl, sl, H, "bf16", True, seed=sl + 1000,
                                                      name=f"causal_bf16_b{B}_t{sl}")))
    out.append(("fp8", sdpa_inputs.custom(B, N, N, 2048, 2048, H, "fp8", True, seed=9000, name=f"fp8_causal_b{B}_t2048")))
    for dtype in ("f32", "bf16", "fp8"):
        for hd in (32, 64, 128):
            for causal in (False, True):
                out.append(("head_dim", sdpa_inputs.custom(B, N, N, 1024, 1024, hd, dtype, causal, seed=1024,
                                                           name=f"head_dim_{dtype}_d{hd}_t1024_{'c' if causal else 'n'}")))
    for sl in (1024, 4096):
        for hkv in (8, 2, 1):
            out.append(("mha_gqa_mqa", sdpa_inputs.custom(2, N, hkv, sl, sl, H, "bf16", True, seed=42,
                                                          name=f"kv_heads_{hkv}_bf16_b2_t{sl}")))
    return out


MFMA_KINDS = [  # (kind, instruction, FLOP per instruction, published dense peak TFLOP/s)
    (0, "v_mfma_f32_32x32x16_bf16", 32768, PEAK_TFLOPS["bf16"]),
    (1, "v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3)", 131072, PEAK_TFLOPS["fp8"]),
    (2, "v_mfma_f32_32x32x2_f32", 4096, PEAK_TFLOPS["f32"]),
]


def run_mfma_peak(warm_seconds: float = 1.0, repeats: int = 5) -> int:
    """The matrix-core ceiling the attention kernels are measured against: every
    wave streams MFMAs on register operands (libmfmapeak.so, built beside the
    attention library), one and two waves per SIMD. One JSON line per case:
    achieved TFLOP/s (median of `repeats` launches of about 20 ms, after
    `warm_seconds` of launches) and its fraction of the published dense peak."""
    import ctypes
    import torch
    from scaled_dot_product_18_amd import build as _build
    if not os.path.exists(_build.PEAK_LIB_PATH):
        raise SystemExit(f"{_build.PEAK_LIB_PATH} is missing: build first (python -m scaled_dot_product_18_amd.build)")
    lib = ctypes.CDLL(_build.PEAK_LIB_PATH)
    lib.mfma_peak_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_peak_launch.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    for kind, instr, flop, peak in MFMA_KINDS:
        for wps in (1, 2):
            blocks = cus * wps
            sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")

            def launch(iters):
                rc = lib.mfma_peak_launch(kind, blocks, iters, sink.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"mfma_peak_launch: status {rc}")

            def timed(iters):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                launch(iters)
                e1.record(stream)
                e1.synchronize()
                return e0.elapsed_time(e1) * 1e-3

            iters = 1000
            for _ in range(3):  # about 20 ms per launch, once the clock has left its idle state
                iters = max(1000, int(iters * 0.02 / max(timed(iters), 1e-6)))
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < warm_seconds:
                timed(iters)
            ts = sorted(timed(iters) for _ in range(repeats))
            t = ts[len(ts) // 2]
            total = blocks * 4 * iters * 8 * flop
            print(json.dumps({"mfma_peak": instr, "waves_per_simd": wps, "workgroups": blocks, "iters": iters,
                              "launch_ms": round(t * 1e3, 3), "tflops": round(total / t / 1e12, 1),
                              "published_peak_tflops": peak, "frac_of_published": round(total / t / 1e12 / peak, 4)}),
                  flush=True)
    return 0


def run_sweep(warmup: int = 2, repeats: int = 20) -> int:
    """Time every sweep shape like the codelab's helper (warm-up calls, then the
    median of the timed calls, each with HIP events on the launch stream around
    the Python call, so launch overhead is included), and also as one HIP graph
    of the same number of launches (the kernel time per launch, which the
    roofline fraction uses)."""
    import torch
    import sdpa_inputs
    import scaled_dot_product_18_amd as sdpa
    sdpa.require_library()
    stream = torch.cuda.current_stream()
    for sweep, w in sweep_shapes():
        inp = sdpa_inputs.make_inputs(w)
        dev = {n: inp[n].cuda() for n in ("q", "k", "v")}
        out = torch.empty((w.B, w.Hq, w.Sq, w.d), dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16,
                          device="cuda")

        def call():
            if w.dtype == "fp8":
                sdpa.fwd_fp8(dev["q"], dev["k"], dev["v"], inp["descale_q"], inp["descale_k"], inp["descale_v"],
                             causal=w.causal, scale=w.scale, out=out)
            else:
                sdpa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale, out=out)

        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        times = []
        for _ in range(repeats):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            b.synchronize()
            times.append(a.elapsed_time(b))
        med = sorted(times)[len(times) // 2]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(repeats):
                call()
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.replay()
        b.record(stream)
        b.synchronize()
        per_launch = a.elapsed_time(b) / repeats
        peak = PEAK_TFLOPS[w.dtype]
        print(json.dumps({"sweep": sweep, "workload": w.name, "B": w.B, "T": w.Sq, "N": w.Hq, "K": w.Hkv, "H": w.d,
                          "dtype": w.dtype, "causal": w.causal, "ms_median": round(med, 5),
                          "tflops": round(w.flops() / (med * 1e-3) / 1e12, 3),
                          "tokens_per_s": round(w.B * w.Sq / (med * 1e-3), 1),
                          "graph_us_per_launch": round(per_launch * 1e3, 2),
                          "graph_tflops": round(w.flops() / (per_launch * 1e-3) / 1e12, 2),
                          "graph_pct_of_peak": round(100 * w.flops() / (per_launch * 1e-3) / 1e12 / peak, 2),
                          "kernel": kernel_name(w)}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="measure the matrix-core ceiling (MFMA streams on register operands) instead")
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="after --warmup calls, keep launching for this long before timing")
    ap.add_argument("--eager-launches", type=int, default=50,
                    help="single launches timed after the graph replay (median / min / p90)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0
    if args.sweep:
        return run_sweep()
    if args.mfma_peak:
        return run_mfma_peak()

    import sdpa_inputs
    import scaled_dot_product_18_amd as sdpa
    sdpa.require_library()

    name = args.workload or sdpa_inputs.HEADLINE
    w = sdpa_inputs.WORKLOADS[name]
    log(f"[bench] workload {name}: generating inputs")
    inp = sdpa_inputs.make_inputs(w)
    dev = {n: inp[n].cuda() for n in ("q", "k", "v")}
    out = torch.empty((w.B, w.Hq, w.Sq, w.d), dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16,
                      device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda") if w.want_lse else None

    workspace = None
    if w.path == "splitkv":
        _, nbytes = sdpa.splitkv_plan(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    if w.path == "bwd":
        # The backward step's inputs: the forward's O and lse (computed here, before timing) and a seeded dO.
        inp["dout"] = sdpa_inputs.draw_grad(w)
        dev["dout"] = inp["dout"].cuda()
        dev["o"], dev["lse"] = sdpa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale,
                                        want_lse=True)
        from scaled_dot_product_18_amd import _lib
        st, nbytes = _lib.attn_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d)
        if st != 0:
            raise RuntimeError(f"attn_bwd_workspace_size: status {st}")
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")

    def step():
        if w.path == "bwd":
            sdpa.bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["lse"], dev["dout"], causal=w.causal, scale=w.scale,
                     workspace=workspace)
        elif w.path == "splitkv":
            sdpa.fwd_splitkv(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale, out=out, lse_out=lse,
                             workspace=workspace)
        elif w.dtype == "fp8":
            sdpa.fwd_fp8(dev["q"], dev["k"], dev["v"], inp["descale_q"], inp["descale_k"], inp["descale_v"],
                         causal=w.causal, scale=w.scale, out=out, lse_out=lse)
        else:
            sdpa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale, out=out, lse_out=lse)

    props = torch.cuda.get_device_properties(0)

    # Warm-up: --warmup calls; then (for forward steps) the graph of K launches
    # is captured and checked; then more launches until --warm-seconds have
    # passed, right before the timed region, so it starts at the clocks a
    # sustained run holds.
    log(f"[bench] warmup {args.warmup} calls + {args.warm_seconds:.1f} s of launches")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Forward steps are timed as one HIP graph of K launches (the library only
    # enqueues kernels on the caller's stream, so a graph captures them): from
    # Python each call costs more host time than a short kernel runs, and the
    # graph keeps the GPU fed. The replayed output must equal the eager one.
    # The backward step allocates its gradients per call and is timed eagerly,
    # with events around every launch.
    use_graph = w.path != "bwd" and not args.eager
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    if use_graph:
        eager_out = out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step()
        torch.cuda.synchronize()
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, eager_out):
            raise RuntimeError("the graph replay's output differs from the eager call's")
    stream = torch.cuda.current_stream()

    t_w0 = time.perf_counter()
    chunk, n_warm = 1, args.warmup
    while time.perf_counter() - t_w0 < args.warm_seconds:
        t_c = time.perf_counter()
        for _ in range(chunk):
            if use_graph:
                graph.replay()
            else:
                step()
        torch.cuda.synchronize()
        n_warm += chunk * (args.steps if use_graph else 1)
        if time.perf_counter() - t_c < 0.02:
            chunk *= 2

    def eager_launches(n):
        """n launches, each between two events on the launch stream; sorted durations in ms."""
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for i in range(n):
            starts[i].record(stream)
            step()
            ends[i].record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in zip(starts, ends))

    log(f"[bench] timing {args.steps} steps" + (" (one graph replay)" if use_graph else ""))
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    region0.record(stream)
    if use_graph:
        graph.replay()
    else:
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for i in range(args.steps):
            starts[i].record(stream)
            step()
            ends[i].record(stream)
    region1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0

    region_ms = region0.elapsed_time(region1)
    if use_graph:
        per_launch = [region_ms / args.steps]
    else:
        per_launch = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    avg_launch_ms = sum(per_launch) / len(per_launch)
    ms_per_step = region_ms / args.steps

    # Distribution of single launches (events around each call), beside the graph value.
    dist = eager_launches(args.eager_launches) if use_graph else per_launch

    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step, launch avg {avg_launch_ms * 1e3:.1f} us; single launches: "
        f"median {percentile(dist, 0.5) * 1e3:.1f}, min {dist[0] * 1e3:.1f}, p90 {percentile(dist, 0.9) * 1e3:.1f} us; "
        f"host wall {t_wall / args.steps * 1e3:.1f} us/step")

    # The roofline that bounds the workload: below the ridge point (peak FLOP/s
    # over peak bytes/s) it is HBM bandwidth, above it the matrix cores.
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / w.hbm_bytes() < ridge:
        bound, unit_r, peak_r = "hbm", "GB/s", PEAK_HBM_GBS
        achieved_r = w.hbm_bytes() / (avg_launch_ms * 1e-3) / 1e9
    else:
        bound, unit_r, peak_r, achieved_r = "mfma", "TFLOP/s", peak, achieved
    rec = {
        "metric": METRIC_BWD if w.path == "bwd" else METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) q/k/v" + (", per-tensor amax e4m3fn" if w.dtype == "fp8" else "")
                + (", N(0,1) dO; O and lse from the forward kernel" if w.path == "bwd" else ""),
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Sk": w.Sk, "d": w.d,
                   "causal": w.causal, "lse": w.want_lse, "in_dtype": w.dtype, "path": w.path,
                   "out_dtype": "f32" if w.dtype == "f32" else "bf16", "seed": w.seed,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "tokens_per_s": round(w.B * w.Sq / (ms_per_step * 1e-3), 1),
        "hbm_gbs_algorithmic": round(w.hbm_bytes() / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": bound,
            "kernel": kernel_name(w),
            "achieved": round(achieved_r, 2),
            "peak": peak_r,
            "unit": unit_r,
            "frac": round(achieved_r / peak_r, 4),
            "traffic": traffic_from_profiles(w),
            "algorithmic_flop_per_launch": flops,
            "algorithmic_bytes_per_launch": w.hbm_bytes(),
            "avg_launch_us": round(avg_launch_ms * 1e3, 2),
        },
        "single_launch_us": {"n": len(dist), "median": round(percentile(dist, 0.5) * 1e3, 2),
                             "min": round(dist[0] * 1e3, 2), "p90": round(percentile(dist, 0.9) * 1e3, 2),
                             "method": "events around each of n eager calls after the timed region"},
        "device": {"name": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
                   "cu_count": props.multi_processor_count, "peak_clock_mhz": hip_clock_rate_mhz(),
                   "warmup_launches": n_warm},
        "counters": counters_from_profiles(w),
        "cpu_baseline": None,
        "kernel_source_sha": kernel_source_hash(kernel_name(w)),
        "timing": "one HIP graph of the K launches, replayed once" if use_graph else "events around each of K launches",
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle on a bounded sample ({args.cpu_budget:.0f} s budget)")
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget, gpu_out=out if w.path != "bwd" else None,
                                           gpu_lse=lse if w.path != "bwd" else None)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
