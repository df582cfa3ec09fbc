#!/usr/bin/env python3
"""Benchmark of the fused low-bit DiT linear layer on one MI355X.

One step = the whole hot path on one batch of synthetic activations that are
already resident in HBM: the on-the-fly FP4 activation quantizer followed by the
fused FP4 GEMM + epilogue, for the DiT MLP up-projection workload (M=4608 tokens,
K=3072, N=2x8192 gate/up pairs, gated-SiLU epilogue, bf16 output 4608x8192).
Weights are packed once before timing (an offline step).  Before the W warm-up
steps the same steps run back to back, untimed, for --settle seconds (0.3 s by
default): the power-managed shader clock takes ~100 steps to leave its idle
state, and timing that ramp would measure the power manager, not the kernels.
The K timed steps follow the warm-up.  Input/output sets
rotate over more than the 256 MB Infinity Cache, so every step reads its
operands from HBM rather than from a warm cache.

Prints one JSON line:
  value        = 2*M*N*K / (quantize + GEMM time per step), TFLOP/s
  roofline     = the GEMM kernel alone: 2*M*N*K / its average duration (HIP events
                 around each launch in the timed region) against the MI355X dense
                 FP4 MFMA peak; traffic = HBM bytes per launch from rocprofv3
                 counters recorded under profiles/ (null if the kernel source has
                 changed since)
  cpu_baseline = the CPU oracle (float64) on a bounded row sample of the same
                 workload, timed on this host's cores
  kernels      = per-kernel figures: the GEMM's mean and p10 / p50 / p90 event
                 times, the quantizer's time and HBM rate, and two fusion
                 comparisons (quantized output against GEMM + quantizer; gated-SiLU
                 in the epilogue against an identity GEMM + a separate gated-SiLU
                 pass over its bf16 output)
  mfma_probe   = the FP4 MFMA rate of a register-only probe kernel on every CU,
                 with the shader clock it ran at, and the GEMM's fraction of it
  power        = socket power and GFX clock (amdsmi) sampled while ~1.5 s of the
                 same steps run back to back, and the steps' TFLOP/s per watt
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused FP4 GEMM+epilogue TFLOP/s and % of MI355X FP4 MFMA peak, M=4608 K=3072"
# MI355X dense MFMA peaks of the instruction each format's products run on (MXFP8 at
# the FP8 rate; NVFP4 is dequantized in registers onto the f16 MFMA)
PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "mx8": 5000.0, "nv4": 2500.0}
HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_fp4_mlp_gated_silu.txt")
GEMM_SRC = os.path.join(ROOT, "bit_gemm_dit_amd", "csrc", "gemm.hip")


def code_only(text: str) -> str:
    """C++ source without its comments, trailing blanks and empty lines, so that an
    edit of the comments alone leaves the hash of the kernel source unchanged (the
    sources hold no string literal with a comment marker in it)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash() -> str:
    """Hash of the GEMM kernel's code (gemm.hip + common.hpp, comments excluded): the
    counter summaries record it, and the traffic they give is used only while it
    still matches."""
    h = hashlib.sha256()
    for f in (GEMM_SRC, os.path.join(ROOT, "bit_gemm_dit_amd", "csrc", "common.hpp")):
        with open(f, encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def read_traffic() -> float | None:
    """HBM bytes per GEMM launch from the committed counter summary, if it still
    describes the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split("=", 1) for line in f.read().splitlines() if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("source_hash", "").strip() != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_sets(ditq, torch, wl, n_sets: int, epi: int):
    from workloads import make_inputs
    d = make_inputs(wl.name, seed=0)
    x0 = torch.from_numpy(d["x"].view("int16")).cuda().view(torch.bfloat16)
    w = torch.from_numpy(d["w"].view("int16")).cuda().view(torch.bfloat16)
    blob0 = ditq.pack_weights(w, ditq.FMT_FP4, epi)
    del w
    sets = []
    for i in range(n_sets):
        x = x0 if i == 0 else x0.clone()
        blob = blob0 if i == 0 else blob0.clone()
        codes = torch.empty((wl.K // 128, wl.M, 64), dtype=torch.uint8, device="cuda")
        scales = torch.empty((wl.K // 128, wl.M, 4), dtype=torch.uint8, device="cuda")
        out = torch.empty((wl.M, wl.N // 2), dtype=torch.bfloat16, device="cuda")
        sets.append((x, blob, codes, scales, out))
    return d, sets


def run_gpu(args):
    import torch
    import bit_gemm_dit_amd as ditq
    from workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    epi = ditq.EPI_GATED_SILU
    d, sets = build_sets(ditq, torch, wl, args.rotate, epi)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    M, N, K = wl.M, wl.N, wl.K

    def step(i, ev=None):
        x, blob, codes, scales, out = sets[i % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        ditq.dit_quantize_act(ditq.FMT_FP4, x.data_ptr(), M, K, K, codes.data_ptr(), scales.data_ptr(), sptr)
        if ev is not None:
            ev[1].record(stream)
        ditq.dit_gemm_q4_epilogue(codes.data_ptr(), scales.data_ptr(), blob.data_ptr(), M, N, K, epi, None,
                                  out.data_ptr(), N // 2, sptr)
        if ev is not None:
            ev[2].record(stream)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    # Untimed settle: the power-managed shader clock leaves its idle state over the
    # first ~100 steps of a cold start (GEMM 147-152 us in steps 5-50, 125 us from
    # step 100 on, same box), so the same steps first run back to back for
    # --settle seconds; then the W warm-up steps and the K timed steps.
    t_end = time.perf_counter() + args.settle
    i_settle = 0
    while time.perf_counter() < t_end:
        for _ in range(32):
            step(i_settle)
            i_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_ms = [e[0].elapsed_time(e[1]) for e in events]
    g_ms = [e[1].elapsed_time(e[2]) for e in events]
    flops = wl.flops
    ms_per_step = wall * 1e3 / args.steps
    gemm_ms = sum(g_ms) / len(g_ms)
    quant_ms = sum(q_ms) / len(q_ms)
    g_sorted = sorted(g_ms)

    def pct(q):
        return round(g_sorted[min(len(g_sorted) - 1, int(q * len(g_sorted)))] * 1e3, 2)
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    quant_bytes = M * K * 2 + M * K // 2 + M * K // 32
    traffic = read_traffic()
    res = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": i_settle,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": M, "N": N, "K": K, "epilogue": "gated_silu",
                   "format": "fp4_e2m1_e8m0_block32", "output": f"bf16 {M}x{N // 2}",
                   "rotating_sets": len(sets)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["fp4"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["fp4"], 4), "traffic": traffic},
        "kernels": {
            "gemm_fp4_gated_silu_us": round(gemm_ms * 1e3, 2),
            "gemm_fp4_gated_silu_us_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
            "quant_fp4_us": round(quant_ms * 1e3, 2),
            "quant_fp4_GBps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
            "quant_fp4_hbm_frac": round(quant_bytes / (quant_ms * 1e-3) / 1e9 / HBM_GBPS, 4),
        },
    }
    if not args.no_fusion_compare:
        res["kernels"].update(time_quantizer_back_to_back(ditq, torch, wl, sets, quant_bytes, args))
        res["kernels"].update(time_quantized_output(ditq, torch, wl, sets, epi, args))
        res["kernels"].update(time_unfused_epilogue(ditq, torch, wl, d, sets, epi, args))
    if not args.no_power:
        res["power"] = sample_power_and_clock(torch, step, wl.flops)
    if not args.no_probe:
        res["mfma_probe"] = time_mfma_probe(ditq, torch)
        res["mfma_probe"]["gemm_frac_of_probe"] = round(achieved / res["mfma_probe"]["tflops"], 4)
    if args.all_configs:
        res["other_configs"] = time_other_configs(ditq, torch, args)
    return res, d


def time_quantizer_back_to_back(ditq, torch, wl, sets, quant_bytes, args):
    """The FP4 quantizer launched n times back to back between one event pair (no
    per-launch event gap, no GEMM write-back in flight), beside a plain device copy
    that moves the same bytes (half read, half written) under the same rotation over
    the input sets: the copy is the rate HBM gives a streaming kernel of this size."""
    M, K = wl.M, wl.K
    sptr = torch.cuda.current_stream().cuda_stream
    n = max(40, args.steps // 2)
    half = quant_bytes // 2 // 16 * 16
    srcs = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in sets]
    dsts = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in sets]
    for t in srcs:
        t.fill_(1)

    def quantize(i):
        x, _, codes, scales, _ = sets[i % len(sets)]
        ditq.dit_quantize_act(ditq.FMT_FP4, x.data_ptr(), M, K, K, codes.data_ptr(), scales.data_ptr(), sptr)

    def copy(i):
        dsts[i % len(sets)].copy_(srcs[i % len(sets)])

    out = {}
    for name, fn in (("quant", quantize), ("copy", copy)):
        for i in range(n // 2):
            fn(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        out[name] = a.elapsed_time(b) / n * 1e3
    del srcs, dsts
    q_gbps = quant_bytes / (out["quant"] * 1e-6) / 1e9
    c_gbps = 2 * half / (out["copy"] * 1e-6) / 1e9
    return {
        "quant_fp4_back_to_back_us": round(out["quant"], 2),
        "quant_fp4_back_to_back_hbm_frac": round(q_gbps / HBM_GBPS, 4),
        "copy_same_bytes_us": round(out["copy"], 2),
        "copy_same_bytes_hbm_frac": round(c_gbps / HBM_GBPS, 4),
        "quant_fp4_rate_vs_copy": round(q_gbps / c_gbps, 4),
    }


def time_quantized_output(ditq, torch, wl, sets, epi, args):
    """The same GEMM when its output feeds another FP4 GEMM: fused (the epilogue
    writes FP4 codes + E8M0 scales, no bf16) against unfused (bf16 output, then a
    separate activation-quantizer pass over it).  Back-to-back sustained runs."""
    M, N, K = wl.M, wl.N, wl.K
    width = N // 2
    sptr = torch.cuda.current_stream().cuda_stream
    qc = torch.empty((width // 128, M, 64), dtype=torch.uint8, device="cuda")
    qs = torch.empty((width // 128, M, 4), dtype=torch.uint8, device="cuda")
    n = max(20, args.steps // 4)

    def fused(i):
        _, blob, codes, scales, _ = sets[i % len(sets)]
        ditq.dit_gemm_q4_epilogue_q4(codes.data_ptr(), scales.data_ptr(), blob.data_ptr(), M, N, K, epi, None,
                                     None, 0, qc.data_ptr(), qs.data_ptr(), sptr)

    def unfused(i):
        _, blob, codes, scales, out = sets[i % len(sets)]
        ditq.dit_gemm_q4_epilogue(codes.data_ptr(), scales.data_ptr(), blob.data_ptr(), M, N, K, epi, None,
                                  out.data_ptr(), width, sptr)
        ditq.dit_quantize_act(ditq.FMT_FP4, out.data_ptr(), M, width, width, qc.data_ptr(), qs.data_ptr(), sptr)

    times = {}
    for name, fn in (("fused", fused), ("unfused", unfused)):
        for i in range(n // 2):
            fn(i)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        times[name] = sum(a.elapsed_time(b) for a, b in ev) / n * 1e3
    return {
        "gemm_q4out_fused_us": round(times["fused"], 2),
        "gemm_then_quantize_us": round(times["unfused"], 2),
        "q4out_fusion_saving_us": round(times["unfused"] - times["fused"], 2),
    }


def time_unfused_epilogue(ditq, torch, wl, d, sets, epi, args):
    """The gated-SiLU GEMM fused (the small op on the accumulators, one bf16 store of
    [M, N/2]) against unfused: an identity GEMM that stores C = [gate | up] as bf16
    [M, N] (weights packed for the identity epilogue), then the separate gated-SiLU
    pass that reads C back and writes [M, N/2].  Back-to-back sustained runs."""
    M, N, K = wl.M, wl.N, wl.K
    sptr = torch.cuda.current_stream().cuda_stream
    w = torch.from_numpy(d["w"].view("int16")).cuda().view(torch.bfloat16)
    blob_id0 = ditq.pack_weights(w, ditq.FMT_FP4, ditq.EPI_IDENTITY)
    blob_ids = [blob_id0] + [blob_id0.clone() for _ in range(len(sets) - 1)]   # rotated like the fused blobs
    del w
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    n = max(20, args.steps // 4)

    def fused(i):
        _, blob, codes, scales, out = sets[i % len(sets)]
        ditq.dit_gemm_q4_epilogue(codes.data_ptr(), scales.data_ptr(), blob.data_ptr(), M, N, K, epi, None,
                                  out.data_ptr(), N // 2, sptr)

    def identity_gemm(i):
        _, _, codes, scales, _ = sets[i % len(sets)]
        ditq.dit_gemm_q4_epilogue(codes.data_ptr(), scales.data_ptr(), blob_ids[i % len(sets)].data_ptr(), M, N, K,
                                  ditq.EPI_IDENTITY, None, c.data_ptr(), N, sptr)

    def separate_pass(i):
        out = sets[i % len(sets)][4]
        ditq.dit_gated_silu_bf16(c.data_ptr(), M, N, N, out.data_ptr(), N // 2, sptr)

    def timed(fns):
        for i in range(n // 2):
            for f in fns:
                f(i)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            for j, f in enumerate(fns):
                f(i)
                ev[i][j + 1].record()
        torch.cuda.synchronize()
        return [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / n * 1e3 for j in range(len(fns))]

    t_fused, = timed([fused])
    t_gemm, t_pass = timed([identity_gemm, separate_pass])
    del blob_ids, blob_id0, c
    return {
        "unfused_identity_gemm_us": round(t_gemm, 2),
        "unfused_gated_silu_pass_us": round(t_pass, 2),
        "unfused_total_us": round(t_gemm + t_pass, 2),
        "fused_gated_silu_gemm_us": round(t_fused, 2),
        "epilogue_fusion_saving_us": round(t_gemm + t_pass - t_fused, 2),
    }


def sample_power_and_clock(torch, step, flops, seconds=1.5):
    """Socket power and GFX clock from amdsmi, sampled every 20 ms by a thread while
    the benchmark's step (quantize + GEMM) runs back to back for about `seconds`
    (after 0.3 s of warm-up at load).  Read-only queries; null where amdsmi is absent."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # no amdsmi on this host: report it, do not fail
        return {"error": f"{type(e).__name__}: {str(e)[:160]}"}
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                pw = amdsmi.amdsmi_get_power_info(h)
                ck = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
                samples.append((float(pw["current_socket_power"]), float(ck["clk"])))
            except Exception:
                pass
            time.sleep(0.02)

    i = 0

    def run_for(sec):
        nonlocal i
        t_end = time.perf_counter() + sec
        while time.perf_counter() < t_end:
            for _ in range(32):
                step(i)
                i += 1
            torch.cuda.synchronize()

    run_for(0.3)
    th = threading.Thread(target=sampler, daemon=True)
    i0, t0 = i, time.perf_counter()
    th.start()
    run_for(seconds)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not samples:
        return {"error": "no samples"}
    watts = sum(p for p, _ in samples) / len(samples)
    mhz = sum(c for _, c in samples) / len(samples)
    tflops = flops * (i - i0) / elapsed / 1e12
    return {"socket_power_w": round(watts, 1), "gfx_clock_mhz": round(mhz, 1), "samples": len(samples),
            "steps": i - i0, "step_tflops": round(tflops, 1), "tflops_per_w": round(tflops / watts, 2)}


def time_mfma_probe(ditq, torch):
    """Register-only FP4 MFMA probe on every CU: sustained TFLOP/s (median of 5
    launches of ~2 ms) and the shader clock from its s_memtime cycle counts."""
    wg = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 16000
    flop = wg * 4 * iters * 8 * 2 * 32 * 32 * 64
    for _ in range(2):
        ditq.mfma_fp4_probe(wg, iters)
    res = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out = ditq.mfma_fp4_probe(wg, iters)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3
        cyc = sorted(out[:, 0].cpu().tolist())[wg // 2]
        res.append((flop / sec / 1e12, cyc / sec / 1e9))
    res.sort()
    tflops, ghz = res[len(res) // 2]
    return {"tflops": round(tflops, 1), "clock_ghz": round(ghz, 3), "workgroups": wg, "iters": iters,
            "frac_of_spec_peak": round(tflops / PEAK_TFLOPS["fp4"], 4)}


def time_other_configs(ditq, torch, args):
    """GEMM-only and quantizer timings of the other full-size workloads (informational)."""
    from workloads import WORKLOADS, make_inputs
    out = {}
    # (workload, epilogue, format: None = the workload's own)
    plans = [("qkv_rmsnorm_hd128", "qk_rmsnorm", None), ("qkv_rmsnorm_hd256", "qk_rmsnorm", None),
             ("fp8_cfg_pair", "identity", None), ("fp8_cfg_pair", "gated_silu", None),
             ("qkv_rmsnorm_hd128", "qk_rmsnorm", "fp8"), ("qkv_rmsnorm_hd256", "qk_rmsnorm", "fp8"),
             ("mlp_gated_silu", "gated_silu", "mx8"), ("qkv_rmsnorm_hd128", "qk_rmsnorm", "mx8"),
             ("fp8_cfg_pair", "identity", "mx8"), ("mlp_gelu_tanh", "gelu_tanh", None),
             ("mlp_down_gate_residual", "gate_residual", None), ("mlp_gated_silu", "gated_silu", "nv4")]
    epis = {"identity": 0, "gated_silu": 1, "qk_rmsnorm": 2, "gelu_tanh": 3, "gate_residual": 4}
    fmts = {"fp4": ditq.FMT_FP4, "fp8": ditq.FMT_FP8, "mx8": ditq.FMT_MX8, "nv4": ditq.FMT_NV4}
    for name, epi_name, fmt_name in plans:
        wl = WORKLOADS[name]
        d = make_inputs(name, seed=0)
        fmt_name = fmt_name or wl.fmt
        fmt = fmts[fmt_name]
        epi = epis[epi_name]
        x = torch.from_numpy(d["x"].view("int16")).cuda().view(torch.bfloat16)
        w = torch.from_numpy(d["w"].view("int16")).cuda().view(torch.bfloat16)
        blob = ditq.pack_weights(w, fmt, epi)
        del w
        rms = None
        keep = []
        if epi == 2:
            gq = torch.from_numpy(d["gamma_q"]).cuda()
            gk = torch.from_numpy(d["gamma_k"]).cuda()
            keep = [gq, gk]
            rms = ditq.rmsnorm_params(gq, gk, wl.n_heads, wl.eps)
        codes, scales = ditq.quantize_act(x, fmt)
        if epi == 4:
            res = torch.from_numpy(d["residual"].view("int16")).cuda().view(torch.bfloat16)
            gate = torch.from_numpy(d["gate"]).cuda()
            keep = [res, gate]

            def run_gemm(out=None):
                return ditq.gemm_gate_residual(codes, scales, blob, wl.N, wl.K, fmt, res, gate, wl.rows_per_gate,
                                               out=out)
        else:
            def run_gemm(out=None):
                return ditq.gemm(codes, scales, blob, wl.N, wl.K, fmt, epi, rms=rms, out=out)
        o = run_gemm()
        # evict the Infinity Cache between launches by reading a 512 MB buffer (a read
        # leaves clean lines behind; writing it would leave dirty ones whose write-back
        # then competes with the timed kernels for HBM)
        flush = torch.zeros(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        times_g, times_q = [], []
        for _ in range(max(3, args.steps // 2)):
            flush.sum()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            ditq.dit_quantize_act(fmt, x.data_ptr(), wl.M, wl.K, wl.K, codes.data_ptr(), scales.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
            e[1].record()
            run_gemm(out=o)
            e[2].record()
            torch.cuda.synchronize()
            times_q.append(e[0].elapsed_time(e[1]))
            times_g.append(e[1].elapsed_time(e[2]))
        times_g.sort()
        times_q.sort()
        g = times_g[len(times_g) // 2]
        q = times_q[len(times_q) // 2]
        qbytes = wl.M * wl.K * 2 + {1: wl.M * wl.K // 2 + wl.M * wl.K // 32, 2: wl.M * wl.K + 4 * wl.M,
                                    3: wl.M * wl.K + wl.M * wl.K // 32, 4: wl.M * wl.K // 2 + wl.M * wl.K // 16}[fmt]
        key = f"{name}/{epi_name}" + ("" if fmt_name == wl.fmt else f"/{fmt_name}")
        out[key] = {
            "gemm_us": round(g * 1e3, 2),
            "tflops": round(wl.flops / (g * 1e-3) / 1e12, 1),
            "frac_of_peak": round(wl.flops / (g * 1e-3) / 1e12 / PEAK_TFLOPS[fmt_name], 4),
            "quant_us": round(q * 1e3, 2),
            "quant_GBps": round(qbytes / (q * 1e-3) / 1e9, 1),
        }
        del keep, flush, blob, x, codes, scales, o
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            # the oracle on the host cores, for the same format and epilogue (the
            # default run times it on the headline workload only)
            out[key]["cpu_baseline"] = oracle_rate(d, fmt_name, epi_name, args.cpu_budget / 4)
        print(f"other config {key} done", file=sys.stderr, flush=True)
    return out


def oracle_rate(d, fmt: str, epi: str, budget_s: float):
    """The CPU oracle on a bounded row sample of one of the other workloads, the same
    way as cpu_baseline: the weights quantized and decoded once beforehand, then
    activation quantize + decode + float64 GEMM + the epilogue on as many token rows
    as fit about budget_s / 3 seconds, repeated to about budget_s, median reported."""
    import numpy as np
    from oracle import epilogue, quant
    q = {"fp4": quant.quantize_fp4, "fp8": quant.quantize_fp8, "mx8": quant.quantize_mx8,
         "nv4": quant.quantize_nv4}[fmt]
    dq = {"fp4": quant.dequantize_fp4, "fp8": quant.dequantize_fp8, "mx8": quant.dequantize_mx8,
          "nv4": quant.dequantize_nv4}[fmt]
    M, K = d["x"].shape
    N = d["w"].shape[0]
    WdT = np.ascontiguousarray(dq(*q(d["w"])).T)
    kw = {}
    if epi == "qk_rmsnorm":
        kw = dict(n_heads=d["n_heads"], head_dim=d["head_dim"], gamma_q=d["gamma_q"], gamma_k=d["gamma_k"],
                  eps=d["eps"])

    def run(rows):
        acc = dq(*q(d["x"][:rows])) @ WdT
        if epi == "gate_residual":
            return epilogue.apply(epi, acc, residual=d["residual"], gate=d["gate"],
                                  rows_per_gate=d["rows_per_gate"], row_ids=np.arange(rows))
        return epilogue.apply(epi, acc, **kw)

    t = time.perf_counter()
    run(64)
    dt = time.perf_counter() - t
    rows = max(64, int(min(M, max(64, 64 * (budget_s / 3) / max(dt, 1e-3)))) // 64 * 64)
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start < budget_s and len(times) < 50):
        t = time.perf_counter()
        run(rows)
        times.append(time.perf_counter() - t)
    times.sort()
    med = times[len(times) // 2]
    return {"value": round(2.0 * rows * N * K / med / 1e12, 4), "unit": "TFLOP/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{rows} of {M} token rows; median of {len(times)} repetitions, {med:.2f} s each"}


def cpu_baseline(d, budget_s: float):
    """Time the CPU oracle (quantize the activation rows, decode, float64 GEMM,
    gated-SiLU) on a bounded sample of the workload: as many token rows as fit
    about budget_s / 3 seconds (all rows when the host is fast enough), repeated
    until about budget_s seconds of work, median repetition reported.  Weights are
    quantized and decoded once beforehand, as packing is offline."""
    import numpy as np
    from oracle import epilogue, quant
    cores = len(os.sched_getaffinity(0))
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    M, K = d["x"].shape
    N = d["w"].shape[0]
    wc, ws = quant.quantize_fp4(d["w"])
    WdT = np.ascontiguousarray(quant.dequantize_fp4(wc, ws).T)

    def run(rows):
        ac, as_ = quant.quantize_fp4(d["x"][:rows])
        acc = quant.dequantize_fp4(ac, as_) @ WdT
        return epilogue.gated_silu(acc)

    t = time.perf_counter()
    run(64)
    dt = time.perf_counter() - t
    rows = int(min(M, max(64, 64 * (budget_s / 3) / max(dt, 1e-3))))
    rows = max(64, rows // 64 * 64)
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start < budget_s and len(times) < 50):
        t = time.perf_counter()
        run(rows)
        times.append(time.perf_counter() - t)
    times.sort()
    med = times[len(times) // 2]
    flops = 2.0 * rows * N * K
    return {"value": round(flops / med / 1e12, 4), "unit": "TFLOP/s", "cores": cores, "cpu": cpu, "kind": "oracle",
            "sample": f"{rows} of {M} token rows of the same workload (activation quantize + decode + float64 "
                      f"GEMM + gated-SiLU; weights quantized beforehand); median of {len(times)} repetitions, "
                      f"{med:.2f} s each"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mlp_gated_silu")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed back-to-back steps before the warm-up, so the power-managed "
                         "clock has left its idle state")
    ap.add_argument("--rotate", type=int, default=4, help="input/output sets cycled through (> cache size)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-configs", action="store_true", help="also time the other workloads' kernels")
    ap.add_argument("--no-fusion-compare", action="store_true",
                    help="skip the fused vs unfused timings (quantized output, gated-SiLU pass), which keeps a "
                         "kernel trace to the timed steps")
    ap.add_argument("--no-probe", action="store_true", help="skip the register-only MFMA probe")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the power / clock sampling run (keeps a kernel trace to the timed steps)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of this many MiB first (the reference dispatch that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this layer runs on one GPU; multi-GPU runs are not part of this benchmark "
                                   "(the path would shard over token rows with replicated weights)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.workload != "mlp_gated_silu":
        raise SystemExit("the headline step is the mlp_gated_silu workload; use --all-configs for the others")
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res, d = run_gpu(args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, args.cpu_budget)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
