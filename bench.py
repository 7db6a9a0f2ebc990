#!/usr/bin/env python3
"""Benchmark of the online MXFP4 W4A4 linear layer on one MI355X.

A step is one pass of the whole online layer over one batch: the activation
transform + MXFP4 quantization kernel, then the MXFP4 GEMM against weights
prepared offline (untimed, like the pages' offline weight preparation).
The default workload is the MLP down-projection prefill M4096 N4096 K14336
with bf16 activations, the largest layer (481 GFLOP per step).  Inputs are seeded synthetic tensors (module `workloads`)
resident in HBM before the timed region; R replicas of (x, W', y) are
cycled so that the working set exceeds the 256 MB Infinity Cache.

Prints one JSON line:
  value        = 2*M*N*K / (wall time per step)      [TFLOP/s]
  act_transform= algorithmic bytes / act-kernel time  [GB/s]
  roofline     = the GEMM kernel (dominant) against the dense MXFP4 MFMA peak
  cpu_baseline = the CPU oracle on a bounded sample of the same layer: its
                 transform + quantization (GB/s) and its fp64 GEMM
                 (TFLOP/s), combined into the layer's TFLOP/s
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 linear TFLOP/s + act-transform GB/s, % of MI355X roofline, 1 GPU"
PEAK_MXFP4_TFLOPS = 10100.0   # MI355X dense FP4/FP6 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
MALL_BYTES = 256 << 20

WORKLOADS = {
    # name: (config, variant, M, description)
    "tiny": (1, 0, None, "tiny M16 N128 K256 fp32 (latency-bound)"),
    "attn": (2, 0, None, "attn-proj M2048 N4096 K4096 bf16"),
    "down": (3, 0, None, "down-prefill M4096 N4096 K14336 bf16"),
    "decode-gateup-m1": (4, 0, 1, "decode gate/up M1 N25600 K5120 bf16"),
    "decode-gateup-m8": (4, 0, 8, "decode gate/up M8 N25600 K5120 bf16"),
    "decode-gateup-m32": (4, 0, 32, "decode gate/up M32 N25600 K5120 bf16"),
    "decode-down-m1": (4, 1, 1, "decode down M1 N5120 K25600 bf16"),
    "decode-down-m8": (4, 1, 8, "decode down M8 N5120 K25600 bf16"),
    "decode-down-m32": (4, 1, 32, "decode down M32 N5120 K25600 bf16"),
    "moe": (5, 0, None, "MoE E64 T8192 N1024 K3072 bf16, Zipf(1.1) per-expert routing"),
    "moe-token": (5, 0, None, "MoE E64 T8192 N1024 K3072 bf16, per-token Zipf(1.1) routing"),
}

# Offline weight preparation with the Hessian exponent search (Hessian of the
# transformed calibration input, then the per-group scale search): the layer
# weights of a workload above and its calibration draw.
OFFLINE = {
    "prep-gateup": (4, 0, "gate/up weights N25600 K5120, 4096 calibration rows, bf16"),
    "prep-moe": (5, 0, "MoE weights E64 N1024 K3072, 512 calibration rows per expert, bf16"),
}
OFFLINE_METRIC = ("offline W4A4 weight preparation (Hessian, exponent search, Flip-Refinement), "
                  "ms per layer, 1 GPU")
PEAK_FP64_TFLOPS = 78.6   # MI355X vector fp64, a fused multiply-add counted as 2
PEAK_FP64_TOPS = 39.3     # separate fp64 add or multiply: 256 CUs x 64 lanes x 2.4 GHz
SEARCH_OPS_PER_GROUP = 2 * (2 * 32 * 32 + 2 * 32)   # two candidates' quadratic forms


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="down", choices=sorted(WORKLOADS) + sorted(OFFLINE))
    p.add_argument("--scale-rule", default="smooth", choices=["smooth", "literal"],
                   help="per-channel factor of the synthetic layer: smooth s = 1/sigma (default) or literal "
                        "s = sigma, sigma = sqrt(max|x_cal| / max|w|) per channel")
    p.add_argument("--path", default="auto", choices=["auto", "fused", "unfused"])
    p.add_argument("--out", default="f32", choices=["f32", "bf16"], help="dtype of y")
    p.add_argument("--epilogue", default="none", choices=["none", "swiglu"],
                   help="swiglu: weight rows are (gate, up) pairs and y is [M][N/2] = silu(gate) * up")
    p.add_argument("--w-layout", default="auto", choices=["auto", "tiled", "rowmajor"],
                   help="prepared weights as macaq_prepare_weights writes them (row-major), or repacked offline by "
                        "macaq_tile_weights (contiguous GEMM copies); auto: tiled for M > 32 when N %% 32 == 0 and "
                        "K %% 128 == 0 (the decode kernels read row-major weights)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ablation", action="store_true", help="skip the pure-MXFP4 comparison")
    p.add_argument("--cpu-rows", type=int, default=256, help="activation rows of the CPU oracle baseline")
    p.add_argument("--cpu-wrows", type=int, default=512, help="weight rows of the CPU oracle baseline's GEMM")
    p.add_argument("--flip-rounds", type=int, default=4096,
                   help="offline workloads: at most this many Flip-Refinement moves per weight row")
    p.add_argument("--library-compare", action="store_true",
                   help="only time our prefill GEMM against the vendor library's MXFP4 GEMM (hipBLASLt through "
                        "torch._scaled_mm) on the same operands, attn-proj and down-prefill, bf16 output")
    p.add_argument("--mfma-probe", action="store_true",
                   help="time the block-scaled FP4 MFMA alone (from registers, random and zero operands): "
                        "the MFMA throughput the chip sustains, next to the 10.1 PFLOP/s datasheet figure")
    p.add_argument("--tune", action="append", default=[], metavar="KNOB=VALUE",
                   help="override a launch shape for this run (macaq_set_tuning), e.g. GEMM_GROUP_M=8 or "
                        "ACT_SEGMENT=32; repeatable; recorded in the line's config")
    p.add_argument("--stream-calibration", action="store_true",
                   help="only run plain HBM streams (reads only, writes only, 4:1 and 1:1 read:write) through "
                        "macaq_probe_stream: the achievable rate for each traffic mix")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 512 MiB device-to-device copy (5 times) so that HBM byte "
                        "counters can be scaled against a transfer of known size")
    return p.parse_args()


def copy_calibration():
    """A plain 512 MiB device-to-device copy (torch's copy kernel): the
    reference transfer of known size that scales the HBM byte counters, and
    the achievable streaming bandwidth (read + write) on this GPU, which
    bounds what an HBM-bound kernel can reach in practice."""
    import torch
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": n, "bytes_written_per_copy": n, "copies": 5 + reps,
                                           "us_per_copy": round(us, 2),
                                           "GBps_read_plus_write": round(2 * n / us / 1e3, 1),
                                           "frac_of_hbm_peak": round(2 * n / us / 1e3 / PEAK_HBM_GBPS, 4)}}))


def stream_calibration(reps=10):
    """macaq_probe_stream: plain HBM streams of known size with the read/write
    mixes of the bandwidth-bound kernels: reads only (the decode GEMM's weight
    stream), writes only, four bytes read per byte written (the online
    transform reads about 3.8 bytes per byte of codes and scales it writes)
    and one to one (a copy), 2 GiB read or 512 MiB written per launch, past
    the 256 MB Infinity Cache; and 4:1 at the down-prefill transform's own
    byte counts, each launch on the next window of the buffers.  Non-temporal
    loads; a few grid sizes, each timed with HIP events around `reps` (or four
    rounds of windows) launches on the launch stream."""
    import torch
    import mxfp4_w4a4_quantized_channel_amd as mx
    dev = "cuda:0"
    L = mx.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    src = torch.empty(2 << 30, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    forms = {"read only": (2 << 30, 0), "write only": (0, 512 << 20),
             "read:write 4:1": (2 << 30, 512 << 20), "read:write 1:1": (512 << 20, 512 << 20)}
    # the down-prefill transform's own traffic: 117.4 MB of bf16 read, 29.4 MB
    # of codes written (4:1); consecutive launches take the next window of src
    # and dst (17 windows), so no launch finds its bytes in the Infinity Cache
    act_rb, act_wb = 4096 * 14336 * 2, 4096 * 14336 // 2
    forms["read:write 4:1, down-prefill transform size"] = (act_rb, act_wb)
    res = {}
    for name, (rb, wb) in forms.items():
        best = None
        windows = min((2 << 30) // rb, (512 << 20) // wb) if 0 < rb < (512 << 20) and wb > 0 else 1
        for blocks in (2048, 8192, 32768) if windows == 1 else (512, 1024, 2048, 4096, 8192):
            out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
            count = [0]

            def launch():
                w = count[0] % windows
                count[0] += 1
                if L.macaq_probe_stream(ctypes.c_void_p(src.data_ptr() + w * rb), rb,
                                        ctypes.c_void_p(dst.data_ptr() + w * wb), wb,
                                        blocks, ctypes.c_void_p(out.data_ptr()), sp) != 0:
                    raise RuntimeError(L.macaq_last_error().decode())
            launch()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            n = reps if windows == 1 else 4 * windows
            for _ in range(n):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / n * 1e3
            gbps = (rb + wb) / us / 1e3
            res[f"{name}, {blocks} blocks"] = {"us": round(us, 2), "GBps": round(gbps, 1)}
            if best is None or gbps > best:
                best = gbps
        res[f"{name}, best"] = {"GBps": round(best, 1), "frac_of_hbm_peak": round(best / PEAK_HBM_GBPS, 4)}
    print(json.dumps({"stream_calibration": res, "read_bytes": {k: v[0] for k, v in forms.items()},
                      "write_bytes": {k: v[1] for k, v in forms.items()}, "launches": reps}), flush=True)


STREAM_SRC_BYTES, STREAM_DST_BYTES = 2 << 30, 512 << 20   # the live ceilings' stream buffers


def stream_windows(read_bytes, write_bytes, cap=64):
    """Windows of the stream buffers for a transform-sized plain stream: the
    number of disjoint (read_bytes, write_bytes) windows that fit in both
    buffers, at most `cap`, or 0 when the stream is too small (< 8 MiB read)
    or too large (> 1 GiB) to measure this way, or its sizes do not suit
    macaq_probe_stream (multiples of 16, reads a whole multiple of writes)."""
    if not ((8 << 20) <= read_bytes <= (1 << 30)) or write_bytes <= 0:
        return 0
    if read_bytes % 16 or write_bytes % 16 or read_bytes % write_bytes:
        return 0
    return max(1, min(STREAM_SRC_BYTES // read_bytes, STREAM_DST_BYTES // write_bytes, cap))


def live_ceilings(L, sp, stream, act_read, act_us, gemm_flops, gemm_us, a_codes, w_codes):
    """What the chip sustains for the same work, timed in the same run, next
    to the kernels' times: a plain stream of the transform's traffic (its
    activation bytes read, a quarter of that written: macaq_probe_stream,
    each launch on the next window of a 2 GiB buffer, best of three grids)
    and, for an MFMA-bound GEMM, the block-scaled FP4 MFMA alone on the
    layer's own codes with the GEMM's MFMA count per SIMD (macaq_probe_mfma,
    one 4-wave block per CU)."""
    import torch
    dev = "cuda:0"
    res = {}

    def timed(launch, n):
        launch(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            launch(i + 1)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    windows = stream_windows(act_read, act_read // 4) if act_us is not None and act_read % 64 == 0 else 0
    if windows:
        rb, wb = act_read, act_read // 4
        src = torch.empty(STREAM_SRC_BYTES, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty(STREAM_DST_BYTES, dtype=torch.uint8, device=dev)
        best = None
        for blocks in (1024, 2048, 4096):
            out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)

            def launch(i, blocks=blocks, out=out):
                w = i % windows
                if L.macaq_probe_stream(ctypes.c_void_p(src.data_ptr() + w * rb), rb,
                                        ctypes.c_void_p(dst.data_ptr() + w * wb), wb, blocks,
                                        ctypes.c_void_p(out.data_ptr()), sp) != 0:
                    raise RuntimeError(L.macaq_last_error().decode())
            us = timed(launch, 4 * windows)
            best = us if best is None else min(best, us)
        del src, dst
        res["act_plain_stream"] = {"read_bytes": rb, "write_bytes": wb, "us": round(best, 2),
                                   "transform_frac_of_it": round(best / act_us, 4)}
    if gemm_flops is not None:
        per_simd = gemm_flops / 131072 / 1024
        iters = max(1, int(round(per_simd / 16)))
        # lane l: 64 bytes of the layer's activation codes, then 64 of its weight codes
        ops = torch.stack([a_codes.reshape(-1)[:4096].reshape(64, 64), w_codes.reshape(-1)[:4096].reshape(64, 64)],
                          1).reshape(-1).contiguous()
        out = torch.empty(256 * 4 * 64, dtype=torch.float32, device=dev)

        def launch(i):
            if L.macaq_probe_mfma(ctypes.c_void_p(ops.data_ptr()), 256, 4, iters, ctypes.c_void_p(out.data_ptr()),
                                  sp) != 0:
                raise RuntimeError(L.macaq_last_error().decode())
        us = timed(launch, 20)
        res["mfma_only"] = {"mfmas_per_simd": iters * 16, "us": round(us, 2), "gemm_frac_of_it": round(us / gemm_us, 4)}
    return res


def library_compare(steps):
    """Our prefill GEMM next to the vendor library's MXFP4 GEMM (hipBLASLt, as
    torch._scaled_mm runs it for float4_e2m1fn_x2 operands with e8m0 block
    scales) on the same operands: the attn-proj and down-prefill layers'
    activation codes (from macaq_quant_act) and prepared weights, row-major
    as the library takes them; ours also on the tiled layouts the layer
    itself uses (macaq_tile_weights offline, macaq_quant_act_tiled online).
    A comparison leg only; nothing of the layer runs through the library.

    The library call spends longer on the host than its kernel takes on the
    GPU, so both sides are timed behind a GPU busy-wait long enough to hide
    the host: the K launches queue up and run back to back between the two
    events."""
    import torch
    import workloads
    import mxfp4_w4a4_quantized_channel_amd as mx
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows = []
    for name in ("attn", "down"):
        cfg, variant, _, desc = WORKLOADS[name]
        wl = workloads.make(cfg, variant=variant)
        M, N, K = wl.M, wl.N, wl.K
        s = wl.s.to(dev)
        ac, asc = mx.quant_act(wl.x.to(dev), s)
        wc, wsc = mx.prepare_weights(wl.w.to(dev), s)
        a4 = ac.view(torch.float4_e2m1fn_x2)
        w4 = wc.reshape(N, K // 2).view(torch.float4_e2m1fn_x2)
        sa = asc.view(torch.float8_e8m0fnu)
        sw = wsc.reshape(N, K // 32).view(torch.float8_e8m0fnu)
        y16 = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        y32 = torch.empty(M, N, dtype=torch.float32, device=dev)
        ours16 = lambda: mx.gemm(ac, asc, wc, wsc, out=y16, out_dtype=torch.bfloat16)
        ours32 = lambda: mx.gemm(ac, asc, wc, wsc, out=y32, out_dtype=torch.float32)
        tc, ts = mx.tile_weights(wc, wsc)
        atc, ats = mx.quant_act_tiled(wl.x.to(dev), s)
        yt16 = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        yt32 = torch.empty(M, N, dtype=torch.float32, device=dev)
        tiled = mx.W_TILED | mx.A_TILED
        tiled16 = lambda: mx.gemm(atc, ats, tc, ts, out=yt16, out_dtype=torch.bfloat16, epilogue=tiled, M=M)
        tiled32 = lambda: mx.gemm(atc, ats, tc, ts, out=yt32, out_dtype=torch.float32, epilogue=tiled, M=M)
        lib16 = lambda: torch._scaled_mm(a4, w4.t(), scale_a=sa, scale_b=sw, out_dtype=torch.bfloat16)

        def gpu_us(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            host_us = (time.perf_counter() - t0) * 1e6
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(int(2.5e3 * host_us * steps))   # about (steps x host time) at 2.5 GHz, doubled below
            torch.cuda._sleep(int(2.5e3 * host_us * steps))
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps * 1e3

        ours32()
        y_lib = lib16()
        ours16()
        tiled32()
        torch.cuda.synchronize()
        rel = ((y_lib.float() - y32).abs() / y32.abs().clamp_min(1e-30))
        t = {k: [] for k in ("ours_bf16", "library_bf16", "ours_fp32", "ours_tiled_bf16", "ours_tiled_fp32")}
        for _ in range(3):   # interleaved, to share clock and thermal conditions
            t["ours_bf16"].append(gpu_us(ours16))
            t["library_bf16"].append(gpu_us(lib16))
            t["ours_fp32"].append(gpu_us(ours32))
            t["ours_tiled_bf16"].append(gpu_us(tiled16))
            t["ours_tiled_fp32"].append(gpu_us(tiled32))
        flops = 2.0 * M * N * K
        med = {k: sorted(v)[1] for k, v in t.items()}
        rows.append({"workload": desc, "M": M, "N": N, "K": K,
                     **{f"{k}_us": round(v, 2) for k, v in med.items()},
                     **{f"{k}_tflops": round(flops / v / 1e6, 1) for k, v in med.items()},
                     "library_over_ours_bf16": round(med["library_bf16"] / med["ours_bf16"], 3),
                     "library_over_ours_tiled_bf16": round(med["library_bf16"] / med["ours_tiled_bf16"], 3),
                     "agreement": {"ours_bf16_is_rne_of_ours_fp32": bool(torch.equal(y16, y32.to(torch.bfloat16))),
                                   "ours_tiled_fp32_equal_to_ours_fp32": bool(torch.equal(yt32, y32)),
                                   "library_max_rel_diff_vs_ours_fp32": round(float(rel.max()), 5),
                                   "library_bf16_equal_to_ours_bf16": round(float((y_lib == y16).float().mean()), 4)}})
    print(json.dumps({"library_compare": rows, "library": "hipBLASLt via torch._scaled_mm "
                      f"(torch {torch.__version__}, HIP {torch.version.hip}), MXFP4 x MXFP4, bf16 output",
                      "steps": steps, "timing": "median of 3 interleaved rounds, each K launches behind a "
                      "GPU busy-wait, HIP events"}), flush=True)


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where unreadable)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


_SMI = {}


def gpu_state():
    """Clock, power and temperature of the first GPU as the AMD SMI library
    reports them at this moment, read in-process (no child process), or None
    where the library is missing or fails.  A snapshot, not an average: the
    clock under load is the counters' figure."""
    try:
        import amdsmi as smi
        if "h" not in _SMI:
            smi.amdsmi_init()
            _SMI["h"] = smi.amdsmi_get_processor_handles()[0]
        h = _SMI["h"]
        power = smi.amdsmi_get_power_info(h)
        return {"sclk_mhz": smi.amdsmi_get_clock_info(h, smi.AmdSmiClkType.GFX)["clk"],
                "mclk_mhz": smi.amdsmi_get_clock_info(h, smi.AmdSmiClkType.MEM)["clk"],
                "power_w": power.get("socket_power", power.get("current_socket_power")),
                "hotspot_c": smi.amdsmi_get_temp_metric(h, smi.AmdSmiTemperatureType.HOTSPOT,
                                                        smi.AmdSmiTemperatureMetric.CURRENT)}
    except Exception:
        return None


def sources_sha256(paths):
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_record(kernel_key):
    """HBM bytes per launch (counter-measured, copy-calibrated) from the
    committed summary profiles/hbm_traffic.json, or None when a source the
    kernel is built from changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))[kernel_key]
        if sources_sha256(rec["sources"]) != rec["sources_sha256"]:
            return None
    except (OSError, KeyError, ValueError):
        return None
    return rec["bytes_per_launch"]


def cpu_baseline(wl, rows, wrows, seconds=6.0):
    """The oracle as it stands, timed on a bounded sample of the same layer
    and scaled to the whole layer:
      * transform + MXFP4 quantization of `rows` activation rows, in GB/s
        of the kernel's algorithmic bytes (x read, codes and scales written);
      * the dequantized fp64 GEMM of those rows against `wrows` weight rows
        prepared by the oracle (untimed, like the offline preparation), in
        TFLOP/s of 2 * rows * wrows * K;
    each repeated for about `seconds`.  value = the layer's 2MNK over the
    time the two stages would take on all M rows and N weight rows at these
    rates.  The transform runs in numpy's single-threaded array operations,
    the GEMM in the BLAS thread pool."""
    import numpy as np
    import oracle
    import workloads
    from threadpoolctl import threadpool_info

    import torch
    M, N, K = wl.M, wl.N, wl.K
    rows, wrows = min(rows, M), min(wrows, N)
    xb = workloads.bf16_bits(wl.x[:rows]) if wl.x.dtype == torch.bfloat16 else wl.x[:rows].numpy()
    off = wl.offsets.numpy()
    e0 = int(np.searchsorted(off, 0, side="right") - 1)
    w = workloads.bf16_bits(wl.w[e0, :wrows]) if wl.w.dtype == torch.bfloat16 else wl.w[e0, :wrows].numpy()
    wc, ws = oracle.prepare_weights(w, wl.s[e0].numpy())
    s = wl.s[e0:e0 + 1].numpy()

    def timed(fn):
        t0, reps = time.perf_counter(), 0
        while True:
            out = fn()
            reps += 1
            el = time.perf_counter() - t0
            if el > seconds or reps >= 200:
                return out, el / reps, reps

    (ac, asc), t_act, n_act = timed(lambda: oracle.quant_act(xb, s))
    _, t_gemm, n_gemm = timed(lambda: oracle.gemm(ac, asc, wc, ws))
    xbytes = xb.dtype.itemsize
    act_bytes = rows * K * xbytes + rows * K // 2 + rows * K // 32 + 4 * K
    act_gbps = act_bytes / t_act / 1e9
    gemm_tflops = 2.0 * rows * wrows * K / t_gemm / 1e12
    layer_s = t_act * M / rows + t_gemm * (M / rows) * (N / wrows)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(2.0 * M * N * K / layer_s / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"transform+quant of {rows} of {M} rows ({n_act} reps), fp64 GEMM of those rows against "
                      f"{wrows} of {N} oracle-prepared weight rows ({n_gemm} reps); scaled to the layer",
            "act_transform": {"GBps": round(act_gbps, 4), "us_per_row": round(t_act / rows * 1e6, 2), "cores": 1},
            "gemm": {"TFLOPs": round(gemm_tflops, 6), "cores": int(threads)},
            "layer_s": round(layer_s, 3), "seconds": round(t_act * n_act + t_gemm * n_gemm, 2), "cpu": cpu_model(),
            "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_baseline_offline(wl, rows, cols, flip_rows, flip_rounds):
    """The oracle's offline chain on a bounded sample, scaled to one layer:
    the Hessian of `cols` input columns of expert 0's calibration rows (work
    grows with cols^2), the exponent search of `rows` weight rows, and the
    Flip-Refinement of `flip_rows` weight rows (their gradient over all K
    and their rounds, against the full Hessian)."""
    import numpy as np
    import oracle
    import workloads
    from threadpoolctl import threadpool_info

    K, N, E = wl.K, wl.N, wl.E
    co = wl.cal_offsets.numpy()
    xb = workloads.bf16_bits(wl.xcal[co[0]:co[1], :cols])
    s = wl.s[0].numpy()
    t0 = time.perf_counter()
    h = oracle.hessian(xb, s[None, :cols])[0]
    t_h = time.perf_counter() - t0
    hk = np.zeros((K, K), np.float32)
    hk[:cols, :cols] = h
    w = workloads.bf16_bits(wl.w[0, :rows])
    t0 = time.perf_counter()
    oracle.prepare_weights_hessian(w, s, hk)
    t_s = time.perf_counter() - t0
    hf = oracle.hessian(workloads.bf16_bits(wl.xcal[co[0]:co[1]]), s[None])[0].astype(np.float32)
    wf = workloads.bf16_bits(wl.w[0, :flip_rows])
    c0, s0 = oracle.prepare_weights_hessian(wf, s, hf)
    xp = oracle.transform(oracle.as_f32(wf), np.broadcast_to(oracle.weight_reciprocal(s), (flip_rows, K)))
    t0 = time.perf_counter()
    oracle.flip_refine(xp, c0, s0, hf, flip_rounds)
    t_f = time.perf_counter() - t0
    layer_s = E * (t_h * (K / cols) ** 2 + t_s * N / rows + t_f * N / flip_rows)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(layer_s * 1e3, 1), "unit": "ms per layer", "cores": int(threads), "kind": "oracle",
            "sample": f"Hessian of {cols} of {K} columns over {co[1] - co[0]} calibration rows ({t_h:.2f} s, "
                      f"scaled by (K/cols)^2) + search of {rows} of {N} weight rows ({t_s:.2f} s, scaled by "
                      f"N/rows) + Flip-Refinement of {flip_rows} rows, up to {flip_rounds} moves ({t_f:.2f} s, "
                      f"scaled by N/rows), times {E} expert(s)",
            "seconds": round(t_h + t_s + t_f, 2), "cpu": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0))}


def bench_offline(args):
    """One step = macaq_hessian over the calibration rows, then
    macaq_prepare_weights_hessian over all weight rows, then
    macaq_flip_refine of those codes, for every expert."""
    import numpy as np
    import torch
    import workloads
    import mxfp4_w4a4_quantized_channel_amd as mx

    cfg, variant, desc = OFFLINE[args.workload]
    wl = workloads.make(cfg, variant=variant, M=1 if cfg == 4 else None, keep_calib=True)
    N, K, E = wl.N, wl.K, wl.E
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mx.lib()
    xc = wl.xcal.to(dev)
    s0 = wl.s.to(dev)
    w = wl.w.to(dev)
    T = xc.shape[0]
    off = wl.cal_offsets.to(dev) if E > 1 else None
    h = torch.empty((E, K, K), dtype=torch.float32, device=dev)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device=dev)
    moves = torch.zeros((E, N), dtype=torch.int32, device=dev)
    ws = torch.empty(mx.flip_refine_workspace_bytes(E * N, K), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    p = ctypes.c_void_p
    off_p = p(off.data_ptr()) if off is not None else None
    xdt = mx.BF16 if xc.dtype == torch.bfloat16 else mx.F32

    def hess(i):
        if mx.macaq_hessian(p(xc.data_ptr()), xdt, p(s0.data_ptr()), off_p, E, T, K, p(h.data_ptr()), sp) != 0:
            raise RuntimeError(mx.lib().macaq_last_error().decode())

    def search(i):
        if mx.macaq_prepare_weights_hessian(p(w.data_ptr()), xdt, p(s0.data_ptr()), p(h.data_ptr()), E, N, K,
                                            p(codes.data_ptr()), p(scales.data_ptr()), sp) != 0:
            raise RuntimeError(mx.lib().macaq_last_error().decode())

    def flip(rounds):
        if mx.macaq_flip_refine(p(w.data_ptr()), xdt, p(s0.data_ptr()), p(h.data_ptr()), E, N, K, rounds,
                                p(codes.data_ptr()), p(scales.data_ptr()), p(moves.data_ptr()), p(ws.data_ptr()),
                                ws.numel(), sp) != 0:
            raise RuntimeError(mx.lib().macaq_last_error().decode())

    def search_flip(i):
        search(i)
        flip(args.flip_rounds)

    def chain(i):
        hess(i)
        search(i)
        flip(args.flip_rounds)

    state_before = gpu_state()
    for i in range(args.warmup):
        chain(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        chain(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    state_after = gpu_state()

    def kernel_us(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e3

    def search_grad(i):                        # flip with 0 rounds: the gradient kernel (the rounds
        search(i)                              # kernel exits at once), on the codes the chain refines
        flip(0)

    h_us = kernel_us(hess)
    s_us = kernel_us(search)
    sf_us = kernel_us(search_flip)
    g_us = kernel_us(search_grad) - s_us
    r_us = sf_us - s_us - g_us
    h_flops = float(T) * K * (K + 1)           # one FMA per row for each distinct entry of the symmetric H
    s_ops = float(E) * N * (K // 32) * SEARCH_OPS_PER_GROUP
    g_ops = 2.0 * E * N * K * K                # a multiply-add (2 flops) per (row, j, i)
    h_ach = h_flops / h_us / 1e6
    s_ach = s_ops / s_us / 1e6
    g_ach = g_ops / g_us / 1e6
    search(0)
    flip(args.flip_rounds)
    torch.cuda.synchronize()
    mv = moves.double()
    moved = None
    if E == 1:
        plain = mx.prepare_weights(w, s0)[1]
        moved = round(float((plain != scales).float().mean()), 4)
    out = {
        "metric": OFFLINE_METRIC, "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": desc, "N": N, "K": K, "experts": E, "calibration_rows": T,
                   "parallelism": "none (one GPU)"},
        "groups_moved_to_b0_plus_1": moved,
    }
    hk = {"kernel": "hessian_tile_kernel", "bound": "alu", "achieved": round(h_ach, 2), "peak": PEAK_FP64_TFLOPS,
          "unit": "TFLOP/s", "frac": round(h_ach / PEAK_FP64_TFLOPS, 4), "us": round(h_us, 2), "traffic": None}
    sk = {"kernel": "prep_hessian_kernel", "bound": "alu", "achieved": round(s_ach, 2), "peak": PEAK_FP64_TOPS,
          "unit": "T fp64 op/s", "frac": round(s_ach / PEAK_FP64_TOPS, 4), "us": round(s_us, 2), "traffic": None}
    # the gradient's multiply-adds are fused whenever that is exact (always for
    # round-to-nearest start codes), so its peak is the fp64 FMA rate
    gk = {"kernel": "flip_grad_kernel", "bound": "alu", "achieved": round(g_ach, 2), "peak": PEAK_FP64_TFLOPS,
          "unit": "TFLOP/s", "frac": round(g_ach / PEAK_FP64_TFLOPS, 4), "us": round(g_us, 2), "traffic": None}
    rk = {"kernel": "flip_rounds_kernel", "bound": "latency (one reduction and one H row per move)",
          "us": round(r_us, 2), "moves_per_row_mean": round(float(mv.mean()), 1),
          "moves_per_row_max": int(mv.max()), "moves_total": int(mv.sum()),
          "ns_per_move": round(r_us * 1e3 / max(float(mv.sum()), 1), 2),
          "rows_at_max_rounds": int((moves == args.flip_rounds).sum())}
    ks = {"hessian": hk, "search": sk, "flip_grad": gk, "flip_rounds": rk}
    dom = max(("hessian", h_us), ("search", s_us), ("flip_grad", g_us), key=lambda t: t[1])[0]
    out["roofline"] = ks[dom]     # the dominant kernel with a roofline
    out["kernels"] = ks
    out["config"]["flip_max_rounds"] = args.flip_rounds
    out["gpu_state"] = {"before": state_before, "after": state_after}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_offline(wl, rows=min(1024, N), cols=min(1024, K),
                                                   flip_rows=min(32, N), flip_rounds=args.flip_rounds)
    print(json.dumps(out), flush=True)


def transform_overhead(args, mx, L, wl, xs, wss, wcs, ys, s0, off_p, stream, sp, a_codes, a_scales, gemm_ws,
                       M, N, K, E, R, ydt, epi, tiled=False):
    """The pages quote MACaQ's cost over pure MXFP4 (same W4A4 layer without
    the scale and the block Hadamard).  Time the online layer both ways on the
    same inputs: MACaQ = transform+quant kernel, then the GEMM against W';
    pure = plain MXFP4 quantization kernel, then the same GEMM against plainly
    quantized W.  overhead = t_macaq / t_pure - 1 (layer level).  Both write
    y with the step's output dtype and epilogue (ydt, epi)."""
    import torch
    p = ctypes.c_void_p
    xdt = mx.BF16 if xs[0].dtype == torch.bfloat16 else mx.F32
    wp = wl.w.reshape(E * N, K).to(xs[0].device)
    pc, ps = mx.quant_mxfp4(wp)
    pc, ps = pc.reshape(E, N, K // 2), ps.reshape(E, N, K // 32)
    if tiled:   # the same weight layout as the MACaQ step
        pc, ps = mx.tile_weights(pc, ps)
    pcs = [pc.clone() for _ in range(R)]
    pss = [ps.clone() for _ in range(R)]

    def macaq_step(i):
        j = i % R
        st = mx.macaq_quant_act(p(xs[j].data_ptr()), xdt, p(s0.data_ptr()), off_p, E, M, K, p(a_codes.data_ptr()),
                                p(a_scales.data_ptr()), sp)
        st |= mx.macaq_gemm_ex(p(a_codes.data_ptr()), p(a_scales.data_ptr()), off_p, E, p(wcs[j].data_ptr()),
                               p(wss[j].data_ptr()), M, N, K, p(ys[j].data_ptr()), ydt, epi, p(gemm_ws.data_ptr()),
                               gemm_ws.numel(), sp)
        assert st == 0, mx.lib().macaq_last_error()

    def pure_step(i):
        j = i % R
        st = mx.macaq_quant_mxfp4(p(xs[j].data_ptr()), xdt, M, K, p(a_codes.data_ptr()), p(a_scales.data_ptr()), sp)
        st |= mx.macaq_gemm_ex(p(a_codes.data_ptr()), p(a_scales.data_ptr()), off_p, E, p(pcs[j].data_ptr()),
                               p(pss[j].data_ptr()), M, N, K, p(ys[j].data_ptr()), ydt, epi, p(gemm_ws.data_ptr()),
                               gemm_ws.numel(), sp)
        assert st == 0, mx.lib().macaq_last_error()

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    # alternate to share clock and thermal conditions
    tm1, tp1 = timed(macaq_step), timed(pure_step)
    tm2, tp2 = timed(macaq_step), timed(pure_step)
    tm, tp = min(tm1, tm2), min(tp1, tp2)
    return {"macaq_ms": round(tm, 5), "pure_mxfp4_ms": round(tp, 5), "overhead": round(tm / tp - 1.0, 4),
            "pages_figure": "2.3% end-to-end (Qwen3-32B, vLLM); about 8% on a 0.6B model"}


def mfma_probe(reps=50):
    """macaq_probe_mfma: 256 blocks (one per CU), each SIMD running 3584
    MFMAs (the down-prefill GEMM's count per SIMD: 481 GFLOP / 131072 FLOP
    / 1024 SIMDs) with one wave per SIMD, or two waves of half as many, and
    no memory traffic.  Operand codes: zeros, uniformly random bytes, or the
    codes of the down-prefill layer's own activation and prepared weight
    (a 64-row slice of the same synthetic distribution).  The clock under
    MFMA load follows the power drawn, which follows how many operand bits
    toggle."""
    import torch
    import workloads
    import mxfp4_w4a4_quantized_channel_amd as mx
    dev = "cuda:0"
    L = mx.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    gen = torch.Generator(device="cpu").manual_seed(7)
    wl = workloads.make(3, shape=(64, 64, 14336))
    ac, _ = mx.quant_act(wl.x.to(dev), wl.s.to(dev))
    wc, _ = mx.prepare_weights(wl.w.to(dev), wl.s.to(dev))
    # lane l: 64 bytes of activation codes, then 64 bytes of weight codes
    layer = torch.stack([ac.reshape(-1)[:4096].reshape(64, 64), wc.reshape(-1)[:4096].reshape(64, 64)], 1).reshape(-1)
    sources = {"zero": torch.zeros(8192, dtype=torch.uint8, device=dev),
               "random": torch.randint(0, 256, (8192,), dtype=torch.uint8, generator=gen).to(dev),
               "down-prefill codes": layer.contiguous()}
    res = {}
    for data, src in sources.items():
        for waves, iters, m in ((4, 224, 16), (8, 224, 8)):
            out = torch.empty(256 * waves * 64, dtype=torch.float32, device=dev)

            def launch():
                if L.macaq_probe_mfma(ctypes.c_void_p(src.data_ptr()), 256, waves, iters,
                                      ctypes.c_void_p(out.data_ptr()), sp) != 0:
                    raise RuntimeError(L.macaq_last_error().decode())
            for _ in range(5):
                launch()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            flops = 256 * waves * iters * m * 131072
            res[f"{data}, {waves // 4} wave(s) per SIMD"] = {
                "us": round(us, 2), "TFLOPs": round(flops / us / 1e6, 1),
                "frac_of_peak": round(flops / us / 1e6 / PEAK_MXFP4_TFLOPS, 4)}
    print(json.dumps({"mfma_probe": res, "mfmas_per_simd": 3584, "flop_per_launch": 256 * 4 * 224 * 16 * 131072,
                      "peak_TFLOPs": PEAK_MXFP4_TFLOPS, "launches": reps}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.mfma_probe:
        mfma_probe()
        return
    if args.stream_calibration:
        stream_calibration()
        return
    if args.library_compare:
        library_compare(min(args.steps, 100))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer is data-parallel: "
              f"run one process per GPU on its own rows)", file=sys.stderr)
        sys.exit(2)

    if args.workload in OFFLINE:
        bench_offline(args)
        return

    import torch
    import workloads
    import mxfp4_w4a4_quantized_channel_amd as mx

    cfg, variant, Mdec, desc = WORKLOADS[args.workload]
    kw = dict(variant=variant)
    if Mdec is not None:
        kw["M"] = Mdec
    if args.workload == "moe-token":
        kw["routing"] = "token_zipf"
    wl = workloads.make(cfg, scale_rule=args.scale_rule, **kw)
    M, N, K, E = wl.M, wl.N, wl.K, wl.E
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = mx.lib()
    flags = {"auto": mx.PATH_AUTO, "fused": mx.PATH_FUSED, "unfused": mx.PATH_UNFUSED}[args.path]
    tuned = {}
    for t in args.tune:
        knob, value = t.split("=")
        mx.set_tuning(getattr(mx, "TUNE_" + knob.upper()), int(value))
        tuned[knob.upper()] = int(value)

    # ---- resident inputs, R replicas so the rotation defeats the MALL
    x0 = wl.x.to(dev)
    s0 = wl.s.to(dev)
    off = wl.offsets.to(dev) if E > 1 else None
    wc0, ws0 = mx.prepare_weights(wl.w.to(dev), s0)
    tiled = args.w_layout == "tiled" or (args.w_layout == "auto" and M > 32 and N % 32 == 0 and K % 128 == 0)
    if tiled:   # offline repack, outside the timed region like the preparation itself
        wc0, ws0 = mx.tile_weights(wc0, ws0)
        flags |= mx.W_TILED
    set_bytes = x0.numel() * x0.element_size() + wc0.numel() + ws0.numel() + M * N * 4   # y at most fp32 [M][N]
    R = max(2, min(64, -(-(4 * MALL_BYTES) // set_bytes)))
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    wcs = [wc0] + [wc0.clone() for _ in range(R - 1)]
    wss = [ws0] + [ws0.clone() for _ in range(R - 1)]
    y_dtype = torch.float32 if args.out == "f32" else torch.bfloat16
    ydt = mx.F32 if args.out == "f32" else mx.BF16
    epi = mx.EPI_SWIGLU if args.epilogue == "swiglu" else mx.EPI_NONE
    gemm_epi = epi | (mx.W_TILED if tiled else 0)   # macaq_gemm_ex takes the layout bit with the epilogue
    y_cols = N // 2 if epi == mx.EPI_SWIGLU else N
    ys = [torch.empty((M, y_cols), dtype=y_dtype, device=dev) for _ in range(R)]
    need = L.macaq_linear_workspace_bytes(M, N, K, E, flags)
    ws_buf = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    # the linear call's staging of the activation: tiled (whole 32-row blocks)
    # for a dense layer with tiled weights, else row-major
    a_tiled = tiled
    stage_rows = int(L.macaq_quant_act_tiled_rows(M, E)) if a_tiled else M
    a_codes = ws_buf[: stage_rows * K // 2]
    fused = L.macaq_linear_path(M, N, K, E, flags) == mx.PATH_FUSED
    a_scales = ws_buf[(stage_rows * K // 2 + 255) // 256 * 256:]
    gemm_ws = torch.zeros(max(int(L.macaq_gemm_workspace_bytes(M, N, K, E)), 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    xdt = mx.BF16 if x0.dtype == torch.bfloat16 else mx.F32
    p = ctypes.c_void_p
    off_p = p(off.data_ptr()) if off is not None else None

    def step_args(i):
        j = i % R
        return (p(xs[j].data_ptr()), p(wcs[j].data_ptr()), p(wss[j].data_ptr()), p(ys[j].data_ptr()))

    def run_linear(i):
        xp, wcp, wsp, yp = step_args(i)
        st = mx.macaq_linear_ex(xp, xdt, p(s0.data_ptr()), off_p, E, wcp, wsp, M, N, K, yp, ydt, epi,
                                p(ws_buf.data_ptr()), ws_buf.numel(), flags, sp)
        if st != 0:
            raise RuntimeError(mx.lib().macaq_last_error().decode())

    state_before = gpu_state()
    # ---- warmup
    for i in range(args.warmup):
        run_linear(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps of the layer
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_linear(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    state_after = gpu_state()
    ms_per_step = wall / args.steps * 1e3
    flops = 2.0 * M * N * K
    value = flops / (wall / args.steps) / 1e12

    # ---- per-kernel durations: a timed region of K back-to-back launches of
    # one kernel on the launch stream, bracketed by HIP events (an unfused
    # step is the activation kernel then the GEMM, the two launches
    # macaq_linear makes on that path)
    def act_only(i):
        xp = step_args(i)[0]
        if a_tiled:
            st = mx.macaq_quant_act_tiled(xp, xdt, p(s0.data_ptr()), off_p, E, M, K, p(a_codes.data_ptr()),
                                          p(a_scales.data_ptr()), sp)
        else:
            st = mx.macaq_quant_act(xp, xdt, p(s0.data_ptr()), off_p, E, M, K, p(a_codes.data_ptr()),
                                    p(a_scales.data_ptr()), sp)
        if st != 0:
            raise RuntimeError(mx.lib().macaq_last_error().decode())

    gemm_layout = gemm_epi | (mx.A_TILED if a_tiled else 0)

    def gemm_only(i):
        _, wcp, wsp, yp = step_args(i)
        if mx.macaq_gemm_ex(p(a_codes.data_ptr()), p(a_scales.data_ptr()), off_p, E, wcp, wsp, M, N, K, yp, ydt,
                            gemm_layout, p(gemm_ws.data_ptr()), gemm_ws.numel(), sp) != 0:
            raise RuntimeError(mx.lib().macaq_last_error().decode())

    def kernel_us(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e3

    # per-kernel timing: back-to-back launches of each kernel of the step (an
    # unfused step's two kernels are macaq_quant_act(_tiled) and macaq_gemm,
    # the launches macaq_linear makes on that path); events between the
    # launches inside layer steps would add a few microseconds to each
    act_us = None
    if fused:
        timing = "back-to-back launches of the fused kernel"
        gemm_us = kernel_us(run_linear)
    else:
        timing = "back-to-back launches of each kernel"
        act_us = kernel_us(act_only)
        gemm_us = kernel_us(gemm_only)

    # algorithmic bytes
    xb = M * K * x0.element_size()
    act_alg = xb + M * K // 2 + M * K // 32 + 4 * E * K
    if E > 1:
        counts = wl.offsets.diff().numpy()
        w_alg = int((counts > 0).sum()) * N * K * 17 // 32
    else:
        w_alg = N * K * 17 // 32
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": desc, "M": M, "N": N, "K": K, "experts": E, "x_dtype": str(x0.dtype).split(".")[-1],
                   "path": "fused" if fused else "unfused", "replicas": R,
                   "w_layout": "tiled" if tiled else "row-major",
                   "act_staging": "tiled" if a_tiled else ("none (fused)" if fused else "row-major"),
                   "y": f"{args.out} [{M}][{y_cols}]" + (" swiglu" if epi == mx.EPI_SWIGLU else ""),
                   "scale_rule": {"smooth": "s = 1/sigma", "literal": "s = sigma"}[args.scale_rule],
                   "kernel_timing": timing,
                   **({"tuning": tuned} if tuned else {}),
                   "parallelism": "none (one GPU)"},
    }
    if act_us is not None:
        out["act_transform"] = {"GBps": round(act_alg / act_us / 1e3, 1), "us": round(act_us, 2),
                                "bytes": act_alg, "frac_of_hbm_peak": round(act_alg / act_us / 1e3 / PEAK_HBM_GBPS, 4),
                                "traffic": traffic_record(f"{args.workload}:act")}
    # counter records are keyed by workload, kernel and (when not fp32 / no epilogue) the output variant
    out_key = "" if (args.out == "f32" and epi == mx.EPI_NONE) else f":{args.out}:{args.epilogue}"
    gemm_name = "fused transform+GEMM" if fused else "MXFP4 GEMM"
    if fused or M <= 32:
        # the kernel's algorithmic HBM bytes: W' codes+scales, its activation
        # input (x and s when fused, else the MXFP4 codes+scales), y
        a_in = xb + 4 * K if fused else M * K // 2 + M * K // 32
        gemm_bytes = w_alg + a_in + M * y_cols * ys[0].element_size()
        ach = gemm_bytes / gemm_us / 1e3
        out["roofline"] = {"kernel": gemm_name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4), "us": round(gemm_us, 2),
                           "traffic": traffic_record(f"{args.workload}:{'fused' if fused else 'gemm'}{out_key}")}
    else:
        # the roofline is the larger of the MFMA time and the HBM time of the
        # kernel's algorithmic bytes (A codes + scales, the active experts' W',
        # y): dense prefill layers are MFMA-bound, the MoE layers HBM-bound
        gemm_bytes = w_alg + M * K // 2 + M * K // 32 + M * y_cols * ys[0].element_size()
        t_mfma, t_hbm = flops / PEAK_MXFP4_TFLOPS / 1e6, gemm_bytes / PEAK_HBM_GBPS / 1e3   # us
        if t_mfma >= t_hbm:
            ach = flops / gemm_us / 1e6
            out["roofline"] = {"kernel": gemm_name, "bound": "mfma", "achieved": round(ach, 1),
                               "peak": PEAK_MXFP4_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_MXFP4_TFLOPS, 4)}
        else:
            ach = gemm_bytes / gemm_us / 1e3
            out["roofline"] = {"kernel": gemm_name, "bound": "hbm", "achieved": round(ach, 1),
                               "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4),
                               "tflops": round(flops / gemm_us / 1e6, 1)}
        out["roofline"].update({"us": round(gemm_us, 2), "roofline_us": {"mfma": round(t_mfma, 2), "hbm": round(t_hbm, 2)},
                                "traffic": traffic_record(f"{args.workload}:gemm{out_key}")})
    if not fused:
        mfma_bound = out["roofline"]["bound"] == "mfma"
        ceil = live_ceilings(L, sp, stream, xb, act_us, flops if mfma_bound else None, gemm_us, a_codes, wcs[0])
        if ceil:
            out["ceilings"] = ceil
    if not args.no_ablation:
        # both sides row-major activation codes into the same GEMM kernel:
        # the comparison isolates the transform against the plain quantizer.
        # The plain quantizer has no fused form, so a layer that runs fused
        # is compared on the two-launch path on both sides.
        if fused:
            rm_buf = torch.zeros(int(L.macaq_quant_act_bytes(M, K)), dtype=torch.uint8, device=dev)
        else:
            rm_buf = ws_buf
        rm_codes = rm_buf[: M * K // 2]
        rm_scales = rm_buf[(M * K // 2 + 255) // 256 * 256:]
        out["transform_overhead"] = transform_overhead(args, mx, L, wl, xs, wss, wcs, ys, s0, off_p, stream, sp,
                                                       rm_codes, rm_scales, gemm_ws, M, N, K, E, R, ydt, gemm_epi,
                                                       tiled=tiled)
        if fused:
            out["transform_overhead"]["path"] = "two launches on both sides (the layer itself runs fused)"
    out["gpu_state"] = {"before": state_before, "after": state_after}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows, args.cpu_wrows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
