#!/usr/bin/env python3
"""Benchmark of the FP8 weight-quantized linear path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

Prints ONE JSON line.  The headline workload is Llama-3-8B q_proj decode:
W [4096, 4096] E4M3 with per-channel scales, bf16 X with M in {1, 8, 32, 64},
fp8_w_bf16_a (W8A16).  One step = one linear call per M (4 calls), each on a
different copy of the quantized weight from a rotating pool larger than the
256 MB Infinity Cache, so every step streams its weights from HBM.  The steps
are captured in HIP graphs (as a decode loop would run them) and timed with
HIP events on the launch stream.  `value` is the algorithmic weight-stream
throughput: (N*K codes + 4N scale bytes + 2MK activation bytes + 2MN output
bytes) summed over the step's calls, divided by the step time.

Unless --quick, the same line carries measurements of the other rows of the
path on their own workloads ("rows"): the Tiny workload, weight quantization,
activation quantization, the W8A8 prefill GEMM (Llama-3-8B gate+up and
Llama-3-70B down_proj), the Llama-3-70B decoder layer's seven linears at
M = 12, and the next rows (fp16 and fused-quantization fp8 activations,
held/EMA scales, the FP8 KV cache, per-group scales).  Prefill GEMM and
activation-cast rows rotate through copies of their inputs whose other copies
together exceed the 256 MB Infinity Cache, so each call reads HBM.

`cpu_baseline` is the CPU oracle (tests' checker) timed on this host on full
decode steps; `cpu_oracle_by_config` times it on every workload (quantization
in full, the GEMM in full or on 64 seeded rows of the prefill GEMMs).  Inputs
are seeded synthetic data (workloads.py).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16 / bf16 MFMA, published
MALL_BYTES = 256 << 20         # Infinity Cache
DECODE_MS = (1, 8, 32, 64)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=12)
    ap.add_argument("--quick", action="store_true", help="headline only (no extra rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pool-mb", type=int, default=1024,
                    help="size of the rotating pool of quantized weight copies")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time spent repeating the headline oracle decode step")
    ap.add_argument("--sections", default="all",
                    help="comma-separated rows to run after the headline: decode-next, tiny, "
                         "prefill, layer, kv (default all); e.g. a profiler run of one section")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(json.dumps({"error": "this benchmark runs on exactly one GPU: the FP8 linear "
                              "path is data-parallel (each GPU would hold whole weights and take "
                              "its own share of the tokens), so one MI355X's share is what it "
                              "measures", "n_gpus": args.gpus}), flush=True)
        return 2
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")

    import numpy as np
    import torch

    import fp8_weight_quantized_amd as fq
    import workloads
    from fp8_weight_quantized_amd import _lib

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda:0")
    L = _lib.lib()
    log("library", fq.library_path(), "device", torch.cuda.get_device_name(dev))

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def ptr(t):
        return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)

    # ------------------------------------------------------------------ decode
    wl = workloads.WORKLOADS["q_proj_decode"]
    lin = wl.linears[0]
    N, K = lin.n, lin.k
    t0 = time.time()
    w_bits = workloads.weight(wl, lin)
    xs_bits = {m: workloads.activation(wl, m, K) for m in DECODE_MS}
    log(f"generated q_proj inputs in {time.time() - t0:.1f}s")
    wq0, w_scale = fq.quantize_weight(up_bf16(w_bits))
    copies_n = max(8, (args.pool_mb << 20) // (N * K))
    copies_n = (copies_n + len(DECODE_MS) - 1) // len(DECODE_MS) * len(DECODE_MS)
    pool = torch.empty((copies_n, N, K), dtype=torch.uint8, device=dev)
    pool[:] = wq0.unsqueeze(0)
    xs = {m: up_bf16(xs_bits[m]) for m in DECODE_MS}
    ys = {m: torch.empty((m, N), dtype=torch.bfloat16, device=dev) for m in DECODE_MS}
    wsn = {m: L.fp8q_linear_workspace_size(0, m, N, K) for m in DECODE_MS}
    wsp = {m: (torch.zeros(wsn[m], dtype=torch.uint8, device=dev) if wsn[m] else None) for m in DECODE_MS}
    step_bytes = sum(N * K + 4 * N + 2 * m * K + 2 * m * N for m in DECODE_MS)
    rot = copies_n // len(DECODE_MS)          # steps per full rotation of the pool

    def decode_step(i: int, stream: int):
        for j, m in enumerate(DECODE_MS):
            c = (len(DECODE_MS) * i + j) % copies_n
            st = L.fp8q_linear(0, ptr(xs[m]), m, K, K, None, ptr(pool[c]), N, K, ptr(w_scale),
                               ptr(ys[m]), N, ptr(wsp[m]), wsn[m], stream)
            if st != 0:
                raise RuntimeError(_lib.last_error())

    def capture(nsteps: int):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
            h = torch.cuda.current_stream(dev).cuda_stream
            for i in range(nsteps):
                decode_step(i, h)
        torch.cuda.current_stream(dev).wait_stream(s)
        return g

    cur = torch.cuda.current_stream(dev).cuda_stream
    for i in range(args.warmup):                       # eager warm-up steps
        decode_step(i, cur)
    n_full, rem = divmod(args.steps, rot)
    g_full = capture(rot) if n_full else None
    g_rem = capture(rem) if rem else None
    for g in (g_full, g_rem):                          # first replay uploads the graph
        if g is not None:
            g.replay()
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(n_full):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"decode step {ms_per_step * 1e3:.2f} us, {value:.1f} GB/s")

    # spread of the step time, outside the timed region: one event pair per
    # replay of a whole rotation of the weight pool
    g_dist = g_full if g_full is not None else capture(rot)
    if g_full is None:
        g_dist.replay()
    samples = []
    for _ in range(20):
        a_ev = torch.cuda.Event(enable_timing=True)
        b_ev = torch.cuda.Event(enable_timing=True)
        a_ev.record()
        g_dist.replay()
        b_ev.record()
        b_ev.synchronize()
        samples.append(a_ev.elapsed_time(b_ev) * 1e3 / rot)
    samples.sort()

    def pct(q: float) -> float:
        return round(samples[min(len(samples) - 1, int(q * (len(samples) - 1) + 0.5))], 3)
    step_spread = {"median_us": pct(0.5), "p10_us": pct(0.1), "p90_us": pct(0.9),
                   "samples": len(samples), "steps_per_sample": rot}
    log("step spread", step_spread)

    # per-M breakdown (each call alone, graph of one rotation)
    per_m = {}
    for j, m in enumerate(DECODE_MS):
        def one_m(i, stream, m=m):
            c = i % copies_n
            st = L.fp8q_linear(0, ptr(xs[m]), m, K, K, None, ptr(pool[c]), N, K, ptr(w_scale),
                               ptr(ys[m]), N, ptr(wsp[m]), wsn[m], stream)
            if st != 0:
                raise RuntimeError(_lib.last_error())
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
            h = torch.cuda.current_stream(dev).cuda_stream
            for i in range(copies_n):
                one_m(i, h)
        torch.cuda.current_stream(dev).wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        start.record()
        g.replay()
        end.record()
        end.synchronize()
        us = start.elapsed_time(end) * 1e3 / copies_n
        b = N * K + 4 * N + 2 * m * K + 2 * m * N
        desc = fq.describe_linear(0, m, N, K)
        per_m[str(m)] = {"us": round(us, 3), "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                         "bytes": b, "kernel": desc, "kernel_symbol": desc[:desc.index(">") + 1]}
    log("per-M", per_m)

    result = {
        "metric": "FP8 linear TFLOPS (prefill M) and weight-stream GB/s (decode M); % of roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded heavy-tail N(0,0.1)+3% +-U(2,4) weights, N(0,1) activations",
        "config": {
            "workload": "Llama-3-8B q_proj decode, fp8_w_bf16_a (W8A16)",
            "N": N, "K": K, "M": list(DECODE_MS),
            "weight_copies_rotated": copies_n,
            "weight_pool_MB": round(copies_n * N * K / 1e6, 1),
            "timing": "HIP graphs of whole steps, HIP events on the launch stream",
            "arithmetic": "E4M3 weight codes widened exactly to bf16 in registers, bf16 MFMA, "
                          "fp32 accumulation, fp32 per-channel scale, bf16 output",
        },
        "per_m": per_m,
        "step_spread": step_spread,
        "roofline": roofline_decode(per_m, N, K),
    }
    # secondary denominator: what a plain device copy reaches on this GPU
    copy_gbs = measured_copy_gbs(torch, dev)
    result["roofline"]["measured_copy_GBps"] = round(copy_gbs, 1)
    result["roofline"]["frac_of_measured_copy"] = round(result["roofline"]["achieved"] / copy_gbs, 4)
    log("device copy", round(copy_gbs, 1), "GB/s (read + write)")

    # --------------------------------------------------------------- other rows
    sections = {"decode-next", "tiny", "prefill", "layer", "kv"} if args.sections == "all" \
        else set(args.sections.split(","))
    if not args.quick:
        rows = {}
        if "decode-next" in sections:
            # fp8_w_fp16_a on the same decode step: fp16 copies of the activations
            xs16 = {m: xs[m].to(torch.float16) for m in DECODE_MS}
            ys16 = {m: torch.empty((m, N), dtype=torch.float16, device=dev) for m in DECODE_MS}

            def decode_step_f16(i: int, stream: int):
                for j, m in enumerate(DECODE_MS):
                    c = (len(DECODE_MS) * i + j) % copies_n
                    st = L.fp8q_linear(2, ptr(xs16[m]), m, K, K, None, ptr(pool[c]), N, K, ptr(w_scale),
                                       ptr(ys16[m]), N, ptr(wsp[m]), wsn[m], stream)
                    if st != 0:
                        raise RuntimeError(_lib.last_error())
            g16 = torch.cuda.CUDAGraph()
            s16 = torch.cuda.Stream(device=dev)
            s16.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.graph(g16, stream=s16, capture_error_mode="relaxed"):
                h = torch.cuda.current_stream(dev).cuda_stream
                for i in range(rot):
                    decode_step_f16(i, h)
            torch.cuda.current_stream(dev).wait_stream(s16)
            g16.replay()
            torch.cuda.synchronize()
            start.record()
            g16.replay()
            end.record()
            end.synchronize()
            us16 = start.elapsed_time(end) * 1e3 / rot
            rows["f1_w8a16_f16_q_proj_decode"] = {
                "shape": "N=K=4096, M=1,8,32,64 per step", "us_per_step": round(us16, 3),
                "GB/s": round(step_bytes / (us16 * 1e-6) / 1e9, 1),
                "frac_hbm": round(step_bytes / (us16 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "mode": "fp8_w_fp16_a (fp16 activations and output)"}
            log(rows["f1_w8a16_f16_q_proj_decode"])

            # fp8_w_fp8_a at decode sizes: the same step on per-tensor E4M3 activations
            # (quantized once, outside the timed region)
            xq8 = {}
            for m in DECODE_MS:
                xq8[m] = fq.quantize_act(xs[m])
            wsn8 = {m: L.fp8q_linear_workspace_size(1, m, N, K) for m in DECODE_MS}
            wsp8 = {m: (torch.empty(wsn8[m], dtype=torch.uint8, device=dev) if wsn8[m] else None)
                    for m in DECODE_MS}

            def decode_step_f8(i: int, stream: int):
                for j, m in enumerate(DECODE_MS):
                    c = (len(DECODE_MS) * i + j) % copies_n
                    q, sc = xq8[m]
                    st = L.fp8q_linear(1, ptr(q), m, K, q.stride(0), ptr(sc), ptr(pool[c]), N, K,
                                       ptr(w_scale), ptr(ys[m]), N, ptr(wsp8[m]), wsn8[m], stream)
                    if st != 0:
                        raise RuntimeError(_lib.last_error())
            g8 = torch.cuda.CUDAGraph()
            s8 = torch.cuda.Stream(device=dev)
            s8.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.graph(g8, stream=s8, capture_error_mode="relaxed"):
                h = torch.cuda.current_stream(dev).cuda_stream
                for i in range(rot):
                    decode_step_f8(i, h)
            torch.cuda.current_stream(dev).wait_stream(s8)
            g8.replay()
            torch.cuda.synchronize()
            start.record()
            g8.replay()
            end.record()
            end.synchronize()
            us8 = start.elapsed_time(end) * 1e3 / rot
            bytes8 = sum(N * K + 4 * N + m * K + 4 + 2 * m * N for m in DECODE_MS)
            rows["f1_w8a8_codes_q_proj_decode"] = {
                "shape": "N=K=4096, M=1,8,32,64 per step", "us_per_step": round(us8, 3),
                "GB/s": round(bytes8 / (us8 * 1e-6) / 1e9, 1),
                "frac_hbm": round(bytes8 / (us8 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "mode": "fp8_w_fp8_a GEMM alone, on E4M3 codes and a scale made outside the timed "
                        "region (not the mode's whole per-call cost: see f1_w8a8_dynamic_q_proj_decode)"}
            log(rows["f1_w8a8_codes_q_proj_decode"])

            # fp8_w_fp8_a from bf16 activations: the per-tensor quantization folded
            # into the GEMM (absmax kernel + GEMM kernel per call), the mode's
            # whole per-call cost
            wsnd = {m: L.fp8q_linear_w8a8_dynamic_workspace_size(m, N, K) for m in DECODE_MS}
            wspd = {m: torch.empty(wsnd[m], dtype=torch.uint8, device=dev) for m in DECODE_MS}

            def decode_step_dyn(i: int, stream: int):
                for j, m in enumerate(DECODE_MS):
                    c = (len(DECODE_MS) * i + j) % copies_n
                    st = L.fp8q_linear_w8a8_dynamic(ptr(xs[m]), m, K, K, ptr(pool[c]), N, K,
                                                    ptr(w_scale), ptr(ys[m]), N, None, ptr(wspd[m]),
                                                    wsnd[m], None, stream)
                    if st != 0:
                        raise RuntimeError(_lib.last_error())
            usd = time_graph(torch, dev, [lambda h, i=i: decode_step_dyn(i, h) for i in range(rot)])
            bytesd = sum(N * K + 4 * N + 2 * m * K + 4 + 2 * m * N for m in DECODE_MS)
            rows["f1_w8a8_dynamic_q_proj_decode"] = {
                "shape": "N=K=4096, M=1,8,32,64 per step", "us_per_step": round(usd, 3),
                "GB/s": round(bytesd / (usd * 1e-6) / 1e9, 1),
                "frac_hbm": round(bytesd / (usd * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "mode": "fp8_w_fp8_a from bf16 X (fp8q_linear_w8a8_dynamic): up to 16 rows the "
                        "decode GEMM taking the absmax and casting X to E4M3 in registers (one "
                        "launch up to 32768 activation values, else after an absmax launch); "
                        "17-64 rows the quantizer, then the GEMM on the codes",
                "kernels": {str(m): fq.describe_linear(1, m, N, K, dynamic=True) for m in DECODE_MS}}
            log(rows["f1_w8a8_dynamic_q_proj_decode"])
            del wspd

            # per-group weight scales (groups of 128) on the same decode step
            G = 128
            wqg, wsg = fq.quantize_weight_grouped(up_bf16(w_bits), G)
            pool_g = torch.empty((copies_n, N, K), dtype=torch.uint8, device=dev)
            pool_g[:] = wqg.unsqueeze(0)
            del wqg
            wsng = {m: L.fp8q_linear_grouped_workspace_size(0, m, N, K, G) for m in DECODE_MS}
            wspg = {m: (torch.zeros(wsng[m], dtype=torch.uint8, device=dev) if wsng[m] else None)
                    for m in DECODE_MS}

            def decode_step_g(i: int, stream: int):
                for j, m in enumerate(DECODE_MS):
                    c = (len(DECODE_MS) * i + j) % copies_n
                    st = L.fp8q_linear_grouped(0, ptr(xs[m]), m, K, K, None, ptr(pool_g[c]), N, K,
                                               ptr(wsg), G, ptr(ys[m]), N, ptr(wspg[m]), wsng[m],
                                               stream)
                    if st != 0:
                        raise RuntimeError(_lib.last_error())
            gg = torch.cuda.CUDAGraph()
            sg = torch.cuda.Stream(device=dev)
            sg.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.graph(gg, stream=sg, capture_error_mode="relaxed"):
                h = torch.cuda.current_stream(dev).cuda_stream
                for i in range(rot):
                    decode_step_g(i, h)
            torch.cuda.current_stream(dev).wait_stream(sg)
            gg.replay()
            torch.cuda.synchronize()
            start.record()
            gg.replay()
            end.record()
            end.synchronize()
            usg = start.elapsed_time(end) * 1e3 / rot
            bytes_g = sum(N * K + 4 * N * (K // G) + 2 * m * K + 2 * m * N for m in DECODE_MS)
            rows["f4_grouped_q_proj_decode"] = {
                "shape": "N=K=4096, M=1,8,32,64 per step, groups of 128", "us_per_step": round(usg, 3),
                "GB/s": round(bytes_g / (usg * 1e-6) / 1e9, 1),
                "frac_hbm": round(bytes_g / (usg * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "mode": "fp8_w_bf16_a with per-group weight scales",
                "kernels": {str(m): fq.describe_linear(0, m, N, K, G) for m in DECODE_MS}}
            log(rows["f4_grouped_q_proj_decode"])
            del pool_g, gg
            torch.cuda.empty_cache()

            # 128 and 256 rows on the same weight (batched decode): the decode
            # kernels in 64-row groups, which the host picks over the prefill
            # GEMMs for a weight this narrow
            mid = {}
            for mode in (0, 1):
                for m in (128, 256):
                    xm = up_bf16(workloads.activation(wl, m, K))
                    xs_m = None
                    if mode == 1:
                        xm, xs_m = fq.quantize_act(xm)
                    ym = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                    nwm = L.fp8q_linear_workspace_size(mode, m, N, K)
                    wsm = torch.empty(nwm, dtype=torch.uint8, device=dev) if nwm else None

                    def call_mid(i: int, stream: int, mode=mode, m=m, xm=xm, xs_m=xs_m, ym=ym,
                                 nwm=nwm, wsm=wsm):
                        st = L.fp8q_linear(mode, ptr(xm), m, K, K, None if xs_m is None else ptr(xs_m),
                                           ptr(pool[i % copies_n]), N, K, ptr(w_scale), ptr(ym), N,
                                           ptr(wsm), nwm, stream)
                        if st != 0:
                            raise RuntimeError(_lib.last_error())
                    usm = time_graph(torch, dev, [lambda h, i=i: call_mid(i, h) for i in range(copies_n)])
                    bm = N * K + 4 * N + (2 if mode == 0 else 1) * m * K + 2 * m * N
                    mid[f"{'fp8_w_bf16_a' if mode == 0 else 'fp8_w_fp8_a'} M={m}"] = {
                        "us": round(usm, 2), "GB/s": round(bm / (usm * 1e-6) / 1e9, 1),
                        "kernel": fq.describe_linear(mode, m, N, K)}
            rows["mid_rows_q_proj"] = {
                "shape": "N=K=4096 (Llama-3-8B q_proj), 128 and 256 rows", "calls": mid,
                "timing": "HIP graph of calls on weight copies rotated past the Infinity Cache",
                "note": "beyond the decode configs: 65..1024 rows on a narrow weight run the decode "
                        "kernels where a cost estimate says they beat the prefill GEMMs"}
            log(rows["mid_rows_q_proj"])
        cpu = None if args.no_cpu_baseline else {}
        if "tiny" in sections:
            rows.update(tiny_rows(fq, L, up_bf16, ptr, workloads, torch, dev, cpu))
        rows.update(other_rows(args, fq, L, up_bf16, ptr, workloads, np, torch, dev, cpu, sections))
        result["rows"] = rows
        if cpu is not None:
            for key in ("mlp_prefill", "down_prefill_70b"):
                if key in cpu and f"a6a7_w8a8_{key}" in rows:
                    g_us = rows[f"a6a7_w8a8_{key}"]["us"]
                    cpu[key]["gpu_us_gemm"] = g_us
                    cpu[key]["speedup_gemm_extrapolated"] = round(
                        cpu[key]["gemm_full_s_extrapolated"] * 1e6 / g_us, 1)
            result["cpu_oracle_by_config"] = {
                "cores": cpu_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                "note": "the fp64 oracle as the tests use it, on this host's cores; quantization "
                        "in full for every workload, the GEMM in full for Tiny, q_proj decode and "
                        "the 70B layer, on 64 seeded rows for the prefill GEMMs (full size "
                        "extrapolated linearly in M, labelled)",
                **cpu}

    if args.copy_calibration:
        # a plain elementwise copy of known size (1 GiB read + 1 GiB written) whose
        # FETCH_SIZE / WRITE_SIZE readings scale the counters of the kernels above
        nbytes = 1 << 30
        a = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        torch.mul(a, 1, out=b)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = nbytes
        del a, b

    # ------------------------------------------------------------ CPU baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, lin, w_bits, xs_bits, step_bytes,
                                              args.cpu_seconds)
        if "rows" in result and "cpu_oracle_by_config" in result:
            result["cpu_oracle_by_config"]["q_proj_decode"] = {
                "gemm_step_s": result["cpu_baseline"]["seconds_per_step"],
                "quantize_weight_s": result["cpu_baseline"]["quantize_weight_s"],
                "gpu_us_step": round(ms_per_step * 1e3, 3),
                "speedup_gemm": round(result["cpu_baseline"]["seconds_per_step"] * 1e3 / ms_per_step, 1)}

    print(json.dumps(result), flush=True)
    return 0


KERNEL_SOURCES = ("fp8_weight_quantized_amd/csrc/kernels/w8a16.hip",
                  "fp8_weight_quantized_amd/csrc/kernels/device_common.hpp",
                  "fp8_weight_quantized_amd/csrc/kernels/e4m3_div.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_w8a16_q_proj_decode_hbm_traffic.txt")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(m: int):
    """HBM bytes per launch of the decode kernel at this M, from the committed
    FETCH_SIZE / WRITE_SIZE summary, or None when there is none or the kernel
    source has changed since the counters were taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    fields = {}
    for ln in lines:
        if ":" in ln and not ln.startswith(("#", " ", "|")):
            key, val = ln.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    val = fields.get(f"traffic_bytes_per_launch_m{m}")
    return float(val) if val else None


def measured_copy_gbs(torch, dev, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Read + write bandwidth of a plain 1 GiB device-to-device copy (torch),
    after a warm-up: a measured ceiling for streaming kernels, reported beside
    the published 8 TB/s."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def roofline_decode(per_m: dict, n: int, k: int) -> dict:
    """Roofline of the step's dominant kernel: the decode instantiation with the
    longest launches.  achieved = its algorithmic bytes per launch (N*K codes +
    4N scale bytes + 2MK activation + 2MN output bytes) / its average launch
    time, timed with HIP events around a graph of launches on their stream."""
    m = max(per_m, key=lambda key: per_m[key]["us"])
    rec = per_m[m]
    achieved = rec["GB/s"]
    return {
        "bound": "hbm",
        "kernel": f"{rec['kernel_symbol']} (M={m}, N={n}, K={k})",
        "achieved": achieved,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(int(m)),
        "algorithmic_bytes_per_launch": rec["bytes"],
        "us_per_launch": rec["us"],
        "kernel_source_sha256": kernel_source_hash(),
    }


def cpu_threads() -> int:
    """Threads the oracle's OpenMP loops use: the affinity mask, capped by
    OMP_NUM_THREADS when that is set."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    return cores


def cpu_time(fn, min_s: float = 0.3, max_reps: int = 50) -> float:
    """Seconds per call of fn() on the host: at least one call, repeated until
    min_s has passed (or max_reps calls)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or reps >= max_reps:
            return dt / reps


def time_graph(torch, dev, calls, reps: int = 3) -> float:
    """Average us per call of a list of no-argument launch functions (each takes
    the stream handle), captured once into a HIP graph and replayed; the best
    of `reps` replays after one untimed replay."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
        h = torch.cuda.current_stream(dev).cuda_stream
        for c in calls:
            c(h)
    torch.cuda.current_stream(dev).wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(reps):
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        best = min(best, a.elapsed_time(b) * 1e3 / len(calls))
    del g
    return best


def rotation_sets(nbytes_per_set: int) -> int:
    """Input copies to rotate through so that every call finds its inputs
    evicted from the 256 MB Infinity Cache: the other copies together exceed
    it."""
    return max(2, -(-MALL_BYTES // max(1, nbytes_per_set)) + 1)


def time_eager(torch, fn, iters: int, warm: int = 2, warm_ms: float = 30.0) -> float:
    """Average ms per call of fn() over `iters` calls, HIP events on the current stream.

    Warm-up runs at least `warm` calls and at least `warm_ms` of GPU time: under
    sustained matrix-core load the clock drops after the first few calls and
    recovers over the next ~20 ms (seen in kernel traces of the prefill GEMM),
    so timing right after a short warm-up would measure that transient instead
    of the sustained rate."""
    for _ in range(max(1, warm)):
        fn()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    fn()
    e.record()
    e.synchronize()
    once = max(s.elapsed_time(e), 1e-3)
    for _ in range(min(500, int(warm_ms / once))):
        fn()
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def other_rows(args, fq, L, up_bf16, ptr, workloads, np, torch, dev, cpu, sections) -> dict:
    """The rows besides the headline; `cpu` (a dict, or None to skip) collects
    the oracle's timings on the same host inputs."""
    rows = {}
    iters = max(3, min(args.steps, 20))
    stream = lambda: torch.cuda.current_stream(dev).cuda_stream  # noqa: E731

    # prefill: activation quantization + W8A8 GEMM.  Every timed call finds
    # its inputs outside the Infinity Cache: calls rotate through copies of
    # the inputs whose other copies together exceed its 256 MB.
    for key in ("mlp_prefill", "down_prefill_70b") if "prefill" in sections else ():
        wl = workloads.WORKLOADS[key]
        lin = wl.linears[0]
        m = wl.ms[0]
        n, k = lin.n, lin.k
        t0 = time.time()
        w_bits = workloads.weight(wl, lin)
        x_bits = workloads.activation(wl, m, lin.k)
        log(f"generated {key} inputs in {time.time() - t0:.1f}s")
        if cpu is not None:
            cpu[key] = cpu_prefill(key, w_bits, x_bits, m, n, k)
            log("oracle", key, cpu[key])
        w = up_bf16(w_bits)
        x = up_bf16(x_bits)
        del w_bits, x_bits
        wq, ws = fq.quantize_weight(w)
        xq, xsc = fq.quantize_act(x)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

        nset = rotation_sets(xq.numel() + wq.numel())
        sets = [(xq, wq)] + [(xq.clone(), wq.clone()) for _ in range(nset - 1)]
        ctr = [0]

        def gemm():
            xq_, wq_ = sets[ctr[0] % nset]
            ctr[0] += 1
            st = L.fp8q_linear(1, ptr(xq_), m, k, xq_.stride(0), ptr(xsc), ptr(wq_), n, wq_.stride(0),
                               ptr(ws), ptr(y), n, None, 0, stream())
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
        ms = time_eager(torch, gemm, iters)
        flops = 2.0 * m * n * k
        tf = flops / (ms * 1e-3) / 1e12
        rows[f"a6a7_w8a8_{key}"] = {
            "shape": f"M={m} N={n} K={k}", "us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
            "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4), "kernel": fq.describe_linear(1, m, n, k),
            "input_sets_rotated": nset}
        log(key, rows[f"a6a7_w8a8_{key}"])

        # the write-up's prefill mode, fp8_w_fp16_a: fp16 activations (the
        # same values, rounded to fp16) on the 16-bit MFMA, and bf16 too
        if key == "mlp_prefill":
            for mode, dt, tag in ((2, torch.float16, "f16"), (0, torch.bfloat16, "bf16")):
                x16 = x.to(dt)
                y16 = torch.empty((m, n), dtype=dt, device=dev)
                s16 = [(x16, wq)] + [(x16.clone(), sets[i][1]) for i in range(1, nset)]

                def gemm16(mode=mode, s16=s16, y16=y16):
                    x_, wq_ = s16[ctr[0] % nset]
                    ctr[0] += 1
                    st = L.fp8q_linear(mode, ptr(x_), m, k, k, None, ptr(wq_), n, wq_.stride(0),
                                       ptr(ws), ptr(y16), n, None, 0, stream())
                    if st != 0:
                        raise RuntimeError(fq._lib.last_error())
                ms16 = time_eager(torch, gemm16, iters)
                tf16 = flops / (ms16 * 1e-3) / 1e12
                rows[f"f1_w8a16_{tag}_prefill_{key}"] = {
                    "shape": f"M={m} N={n} K={k}", "us": round(ms16 * 1e3, 2),
                    "TFLOP/s": round(tf16, 1), "frac_16bit_peak": round(tf16 / F16_PEAK_TFLOPS, 4),
                    "kernel": fq.describe_linear(mode, m, n, k), "input_sets_rotated": nset,
                    "mode": ("fp8_w_fp16_a" if mode == 2 else "fp8_w_bf16_a") +
                            ": E4M3 weights widened exactly on the 16-bit MFMA"}
                log(key, rows[f"f1_w8a16_{tag}_prefill_{key}"])
                del x16, y16, s16

        # the same GEMM with per-group weight scales (groups of 128)
        wqg, wsg = fq.quantize_weight_grouped(w, 128)
        gsets = [(xq, wqg)] + [(xq.clone(), wqg.clone()) for _ in range(nset - 1)]

        def gemm_g():
            xq_, wq_ = gsets[ctr[0] % nset]
            ctr[0] += 1
            st = L.fp8q_linear_grouped(1, ptr(xq_), m, k, xq_.stride(0), ptr(xsc), ptr(wq_), n,
                                       wq_.stride(0), ptr(wsg), 128, ptr(y), n, None, 0, stream())
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
        ms = time_eager(torch, gemm_g, iters)
        tf = flops / (ms * 1e-3) / 1e12
        rows[f"f4_grouped_w8a8_{key}"] = {
            "shape": f"M={m} N={n} K={k}, groups of 128", "us": round(ms * 1e3, 2),
            "TFLOP/s": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
            "kernel": fq.describe_linear(1, m, n, k, 128), "input_sets_rotated": nset,
            "note": "accumulators rescaled by s[g-1]/s[g] as each group opens"}
        log(key, rows[f"f4_grouped_w8a8_{key}"])
        del wqg, wsg, gsets, sets

        # weight quantization (offline in deployment; timed for completeness)
        wqb = torch.empty((n, k), dtype=torch.uint8, device=dev)
        wsb_ = torch.empty(n, dtype=torch.float32, device=dev)

        def wquant():
            st = L.fp8q_quantize_weight(ptr(w), n, k, k, ptr(wqb), k, ptr(wsb_), None, stream())
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
        ms = time_eager(torch, wquant, iters)
        b = 3.0 * n * k + 4 * n
        rows[f"a1a2_quantize_weight_{key}"] = {
            "shape": f"N={n} K={k}", "us": round(ms * 1e3, 2),
            "GB/s": round(b / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(key, rows[f"a1a2_quantize_weight_{key}"])
        del w, wqb, wsb_

        aws_n = L.fp8q_quantize_act_workspace_size(m, k)
        aws = torch.empty(aws_n, dtype=torch.uint8, device=dev)
        aset = rotation_sets(x.numel() * 2 + xq.numel())
        asets = [(x, xq)] + [(x.clone(), torch.empty_like(xq)) for _ in range(aset - 1)]

        def actq():
            x_, q_ = asets[ctr[0] % aset]
            ctr[0] += 1
            st = L.fp8q_quantize_act(ptr(x_), m, k, k, ptr(q_), q_.stride(0), ptr(xsc), ptr(aws),
                                     aws_n, None, stream())
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
        ms = time_eager(torch, actq, iters)
        b = 3.0 * m * k + 4
        rows[f"a3a4_quantize_act_{key}"] = {
            "shape": f"M={m} K={k}", "us": round(ms * 1e3, 2),
            "GB/s": round(b / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "input_sets_rotated": aset, "note": "two kernels (absmax, cast); X is re-read by the cast"}
        log(key, rows[f"a3a4_quantize_act_{key}"])

        # the whole prefill linear from bf16 X: the dynamic fp8_w_fp8_a entry
        # point (quantizer into its workspace, then the FP8 MFMA GEMM)
        dws_n = L.fp8q_linear_w8a8_dynamic_workspace_size(m, n, k)
        dws = torch.empty(dws_n, dtype=torch.uint8, device=dev)
        dsets = [(x, wq)] + [(asets[i % aset][0], wq.clone()) for i in range(1, nset)]

        def dyn():
            x_, wq_ = dsets[ctr[0] % nset]
            ctr[0] += 1
            st = L.fp8q_linear_w8a8_dynamic(ptr(x_), m, k, k, ptr(wq_), n, wq_.stride(0), ptr(ws),
                                            ptr(y), n, None, ptr(dws), dws_n, None, stream())
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
        ms = time_eager(torch, dyn, iters)
        tf = flops / (ms * 1e-3) / 1e12
        rows[f"a3a7_w8a8_dynamic_{key}"] = {
            "shape": f"M={m} N={n} K={k}", "us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
            "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4), "input_sets_rotated": nset,
            "note": "fp8q_linear_w8a8_dynamic from bf16 X: absmax + cast + FP8 MFMA GEMM (3 kernels)"}
        log(key, rows[f"a3a7_w8a8_dynamic_{key}"])
        del dsets, dws

        # held (static) and EMA scales: one read of X per call
        held = xsc.clone()
        state = torch.zeros(1, dtype=torch.float32, device=dev)
        if L.fp8q_quantize_act_ema(ptr(x), m, k, k, ptr(xq), xq.stride(0), ptr(xsc), ptr(state),
                                   0.9999, 0.0, 1, ptr(aws), aws_n, None, stream()) != 0:
            raise RuntimeError(fq._lib.last_error())

        def actq_static():
            x_, q_ = asets[ctr[0] % aset]
            ctr[0] += 1
            st = L.fp8q_quantize_act_static(ptr(x_), m, k, k, ptr(held), ptr(q_), q_.stride(0),
                                            None, stream())
            if st != 0:
                raise RuntimeError(fq._lib.last_error())

        def actq_ema():
            x_, q_ = asets[ctr[0] % aset]
            ctr[0] += 1
            st = L.fp8q_quantize_act_ema(ptr(x_), m, k, k, ptr(q_), q_.stride(0), ptr(xsc),
                                         ptr(state), 0.9999, 0.1, 0, ptr(aws), aws_n, None,
                                         stream())
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
        for name, fn, note in (
                ("static", actq_static, "one kernel: cast with a held scale"),
                ("ema", actq_ema, "cast with the EMA state, absmax from the same loads, "
                                  "then a one-workgroup update")):
            ms = time_eager(torch, fn, iters)
            b = 3.0 * m * k + 8
            rows[f"f2_quantize_act_{name}_{key}"] = {
                "shape": f"M={m} K={k}", "us": round(ms * 1e3, 2),
                "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "input_sets_rotated": aset, "note": note}
            log(key, rows[f"f2_quantize_act_{name}_{key}"])
        del x, wq, ws, xq, y, asets
        torch.cuda.empty_cache()

    if "layer" in sections:
        rows.update(layer_rows(fq, L, up_bf16, ptr, workloads, torch, dev, cpu, iters, stream))
    if "kv" in sections:
        rows.update(kv_rows(fq, L, up_bf16, ptr, workloads, np, torch, dev, iters, stream))
    return rows


def layer_rows(fq, L, up_bf16, ptr, workloads, torch, dev, cpu, iters, stream) -> dict:
    """The Llama-3-70B decoder layer's seven linears at decode M = 12
    (W8A16), unfused, fused and with per-group scales, and the weight
    quantization of its matrices."""
    rows = {}
    # 70B decoder layer at decode M = 12 (W8A16), plus weight quantization of gate_proj
    wl = workloads.WORKLOADS["layer_decode_70b"]
    m = wl.ms[0]
    t0 = time.time()
    layer = []
    wq_us = 0.0
    cpu_layer = {"quantize_weight_s": 0.0, "gemm_s": 0.0} if cpu is not None else None
    for lin in wl.linears:
        w_bits = workloads.weight(wl, lin)
        x_bits = workloads.activation(wl, m, lin.k)
        if cpu_layer is not None:
            import oracle
            oracle.build()
            oq = {}
            cpu_layer["quantize_weight_s"] += cpu_time(
                lambda: oq.update(zip(("q", "s", "f"), oracle.quantize_weight(w_bits))), min_s=0.0)
            cpu_layer["gemm_s"] += cpu_time(lambda: oracle.linear(0, x_bits, oq["q"], oq["s"]),
                                            min_s=0.0)
            del oq
        w = up_bf16(w_bits)
        del w_bits
        qb = torch.empty((lin.n, lin.k), dtype=torch.uint8, device=dev)
        sb = torch.empty(lin.n, dtype=torch.float32, device=dev)

        def wq_one(w=w, q=qb, s=sb, lin=lin):
            st = L.fp8q_quantize_weight(ptr(w), lin.n, lin.k, lin.k, ptr(q), lin.k, ptr(s), None, stream())
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
        wq_us += time_eager(torch, wq_one, 3) * 1e3
        del qb, sb
        if lin.name == "gate_proj":
            q = torch.empty((lin.n, lin.k), dtype=torch.uint8, device=dev)
            s = torch.empty(lin.n, dtype=torch.float32, device=dev)

            def wquant(w=w, q=q, s=s, lin=lin):
                st = L.fp8q_quantize_weight(ptr(w), lin.n, lin.k, lin.k, ptr(q), lin.k, ptr(s), None, stream())
                if st != 0:
                    raise RuntimeError(fq._lib.last_error())
            ms = time_eager(torch, wquant, iters)
            b = 3.0 * lin.n * lin.k + 4 * lin.n
            rows["a1a2_quantize_weight_gate_proj_70b"] = {
                "shape": f"N={lin.n} K={lin.k}", "us": round(ms * 1e3, 2),
                "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(rows["a1a2_quantize_weight_gate_proj_70b"])
            sg_ = torch.empty((lin.n, lin.k // 128), dtype=torch.float32, device=dev)

            def wquant_g(w=w, q=q, s=sg_, lin=lin):
                st = L.fp8q_quantize_weight_grouped(ptr(w), lin.n, lin.k, lin.k, 128, ptr(q), lin.k,
                                                    ptr(s), None, stream())
                if st != 0:
                    raise RuntimeError(fq._lib.last_error())
            ms = time_eager(torch, wquant_g, iters)
            b = 3.0 * lin.n * lin.k + 4 * lin.n * (lin.k // 128)
            rows["f4_quantize_weight_grouped_gate_proj_70b"] = {
                "shape": f"N={lin.n} K={lin.k}, groups of 128", "us": round(ms * 1e3, 2),
                "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(rows["f4_quantize_weight_grouped_gate_proj_70b"])
            del sg_
        wq, ws = fq.quantize_weight(w)
        del w
        x = up_bf16(x_bits)
        del x_bits
        y = torch.empty((m, lin.n), dtype=torch.bfloat16, device=dev)
        nws = L.fp8q_linear_workspace_size(0, m, lin.n, lin.k)
        wsb = torch.zeros(nws, dtype=torch.uint8, device=dev) if nws else None
        layer.append((lin, wq, ws, x, y, wsb, nws))
    log(f"prepared 70B layer in {time.time() - t0:.1f}s")
    torch.cuda.empty_cache()
    nel = sum(lin.n * lin.k for lin in wl.linears)
    rows["a1a2_quantize_weight_layer_70b"] = {
        "shape": "7 matrices, 855,638,016 weights", "us": round(wq_us, 2),
        "GB/s": round((3.0 * nel) / (wq_us * 1e-6) / 1e9, 1),
        "frac_hbm": round((3.0 * nel) / (wq_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "note": "sum of the seven matrices' quantization times"}
    log(rows["a1a2_quantize_weight_layer_70b"])
    if cpu_layer is not None:
        cpu_layer["gpu_us"] = None       # filled in below from the layer step
        cpu["layer_decode_70b"] = cpu_layer

    def layer_step(h):
        for lin, wq, ws, x, y, wsb, nws in layer:
            st = L.fp8q_linear(0, ptr(x), m, lin.k, lin.k, None, ptr(wq), lin.n, wq.stride(0), ptr(ws),
                               ptr(y), lin.n, ptr(wsb), nws, h)
            if st != 0:
                raise RuntimeError(fq._lib.last_error())

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
        layer_step(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.current_stream(dev).wait_stream(s)
    ms = time_eager(torch, g.replay, iters)
    b = sum(lin.n * lin.k + 4 * lin.n + 2 * m * lin.k + 2 * m * lin.n for lin, *_ in layer)
    per = {}
    for lin, wq, ws, x, y, wsb, nws in layer:
        # the C call as a caller holding raw pointers makes it: arguments
        # marshalled once, so the time is the library's host path + the GPU's
        args = (0, ptr(x), m, lin.k, lin.k, None, ptr(wq), lin.n, wq.stride(0), ptr(ws), ptr(y),
                lin.n, ptr(wsb), nws, stream())

        def one(args=args):
            if L.fp8q_linear(*args) != 0:
                raise RuntimeError(fq._lib.last_error())
        mso = time_eager(torch, one, iters)
        bb = lin.n * lin.k + 4 * lin.n + 2 * m * lin.k + 2 * m * lin.n
        per[lin.name] = {"us": round(mso * 1e3, 2), "GB/s": round(bb / (mso * 1e-3) / 1e9, 1)}
    # the same layer with the weights that share an input concatenated along
    # N, as serving engines store them: q/k/v -> qkv [10240, 8192] and
    # gate/up -> gate_up [57344, 8192]; the same bytes in 4 launches, not 7
    by_name = {lin.name: (lin, wq, ws, x) for lin, wq, ws, x, *_ in layer}
    fused = []
    for name, parts in (("qkv_proj", ("q_proj", "k_proj", "v_proj")), ("o_proj", ("o_proj",)),
                        ("gate_up_proj", ("gate_proj", "up_proj")), ("down_proj", ("down_proj",))):
        lins = [by_name[p_][0] for p_ in parts]
        nf, kf = sum(l_.n for l_ in lins), lins[0].k
        wqf = torch.cat([by_name[p_][1] for p_ in parts]) if len(parts) > 1 else by_name[parts[0]][1]
        wsf = torch.cat([by_name[p_][2] for p_ in parts]) if len(parts) > 1 else by_name[parts[0]][2]
        xf = by_name[parts[0]][3]
        yf = torch.empty((m, nf), dtype=torch.bfloat16, device=dev)
        nwf = L.fp8q_linear_workspace_size(0, m, nf, kf)
        wsbf = torch.zeros(nwf, dtype=torch.uint8, device=dev) if nwf else None
        fused.append((name, nf, kf, wqf, wsf, xf, yf, wsbf, nwf))

    def layer_step_fused(h):
        for name, nf, kf, wqf, wsf, xf, yf, wsbf, nwf in fused:
            st = L.fp8q_linear(0, ptr(xf), m, kf, kf, None, ptr(wqf), nf, wqf.stride(0), ptr(wsf),
                               ptr(yf), nf, ptr(wsbf), nwf, h)
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
    gf = torch.cuda.CUDAGraph()
    sfs = torch.cuda.Stream(device=dev)
    sfs.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(gf, stream=sfs, capture_error_mode="relaxed"):
        layer_step_fused(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.current_stream(dev).wait_stream(sfs)
    msf = time_eager(torch, gf.replay, iters)
    bf = sum(nf * kf + 4 * nf + 2 * m * kf + 2 * m * nf for _, nf, kf, *_ in fused)
    rows["a5_layer_decode_70b_fused"] = {
        "shape": "qkv [10240,8192], o [8192,8192], gate_up [57344,8192], down [8192,28672], M=12",
        "us": round(msf * 1e3, 2), "GB/s": round(bf / (msf * 1e-3) / 1e9, 1),
        "frac_hbm": round(bf / (msf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "timing": "one HIP graph per layer step",
        "kernels": {name: fq.describe_linear(0, m, nf, kf) for name, nf, kf, *_ in fused}}
    log(rows["a5_layer_decode_70b_fused"])
    del fused, gf

    # the same layer with per-group weight scales (groups of 128)
    G = 128
    layer_g = []
    for lin, wq, ws, x, y, wsb, nws in layer:
        wsg = torch.ones((lin.n, lin.k // G), dtype=torch.float32, device=dev) * ws[:, None]
        nwg = L.fp8q_linear_grouped_workspace_size(0, m, lin.n, lin.k, G)
        wsbg = torch.zeros(nwg, dtype=torch.uint8, device=dev) if nwg else None
        layer_g.append((lin, wq, wsg.contiguous(), x, y, wsbg, nwg))

    def layer_step_g(h):
        for lin, wq, wsg, x, y, wsb, nws in layer_g:
            st = L.fp8q_linear_grouped(0, ptr(x), m, lin.k, lin.k, None, ptr(wq), lin.n,
                                       wq.stride(0), ptr(wsg), G, ptr(y), lin.n, ptr(wsb), nws, h)
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
    gg = torch.cuda.CUDAGraph()
    sgs = torch.cuda.Stream(device=dev)
    sgs.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(gg, stream=sgs, capture_error_mode="relaxed"):
        layer_step_g(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.current_stream(dev).wait_stream(sgs)
    msg = time_eager(torch, gg.replay, iters)
    bg = sum(lin.n * lin.k + 4 * lin.n * (lin.k // G) + 2 * m * lin.k + 2 * m * lin.n
             for lin, *_ in layer_g)
    rows["f4_grouped_layer_decode_70b"] = {
        "shape": "7 linears, M=12, groups of 128", "us": round(msg * 1e3, 2),
        "GB/s": round(bg / (msg * 1e-3) / 1e9, 1),
        "frac_hbm": round(bg / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "timing": "one HIP graph per layer step",
        "kernels": {lin.name: fq.describe_linear(0, m, lin.n, lin.k, G) for lin, *_ in layer_g}}
    log(rows["f4_grouped_layer_decode_70b"])
    del layer_g, gg

    rows["a5_layer_decode_70b"] = {
        "shape": "7 linears, M=12", "weight_MB": round(b / 1e6, 1), "us": round(ms * 1e3, 2),
        "GB/s": round(b / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "timing": "one HIP graph per layer step (856 MB of weights: no Infinity Cache reuse)",
        "kernels": {lin.name: fq.describe_linear(0, m, lin.n, lin.k) for lin, *_ in layer},
        "per_linear_eager": per,
        "per_linear_eager_note": "one eager C call after another on the same weights (arguments "
                                 "marshalled once): the library's host path included, and weights "
                                 "under 256 MB may be served from the Infinity Cache (a latency "
                                 "figure, not an HBM one)"}
    log(rows["a5_layer_decode_70b"])
    if cpu is not None and "layer_decode_70b" in cpu:
        c = cpu["layer_decode_70b"]
        c["gpu_us"] = {"gemm_step": round(ms * 1e3, 2), "quantize_weight": round(wq_us, 2)}
        c["speedup_gemm"] = round(c["gemm_s"] * 1e6 / (ms * 1e3), 1)
        c["quantize_weight_s"] = round(c["quantize_weight_s"], 3)
        c["gemm_s"] = round(c["gemm_s"], 3)
        c["sample"] = "all 7 matrices in full: quantization, and the fp64 GEMM at M=12"
    del layer
    torch.cuda.empty_cache()
    return rows


def kv_rows(fq, L, up_bf16, ptr, workloads, np, torch, dev, iters, stream) -> dict:
    """FP8 KV-cache writes of Llama-3-70B (8 KV heads x 128): a calibrating
    8192-token prefill chunk, and one decode step (12 tokens) over 80 layers."""
    rows = {}
    heads, hd, layers = 8, 128, 80
    width = heads * hd

    def make_call(k, v, t, slot, kc, vc, run, sc, ws, nws, cal):
        def call(h=None):
            st = L.fp8q_kv_cache_write(ptr(k), ptr(v), t, heads, hd, width, ptr(slot), ptr(kc),
                                       ptr(vc), kc.shape[1], ptr(run), ptr(sc), cal, ptr(ws), nws,
                                       None, stream() if h is None else h)
            if st != 0:
                raise RuntimeError(fq._lib.last_error())
        return call

    t, s_rows = 8192, 8192
    k = up_bf16(workloads.outlier_act(t, width, 901))
    v = up_bf16(workloads.normal_act(t, width, 902))
    slot = torch.arange(t, dtype=torch.int64, device=dev)
    kc = torch.zeros((heads, s_rows, hd), dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    run = torch.zeros(2, dtype=torch.float32, device=dev)
    sc = torch.zeros(2, dtype=torch.float32, device=dev)
    nws = L.fp8q_kv_cache_workspace_size(t, heads, hd)
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev)
    b = 2 * (3.0 * t * width) + 8 * t
    for name, cal, note in (("prefill_calibrate", 1, "K and V, 8192 tokens: absmax pass, "
                             "then the cast with the raised running max"),
                            ("prefill_held", 0, "K and V, 8192 tokens: one cast pass")):
        ms = time_eager(torch, make_call(k, v, t, slot, kc, vc, run, sc, ws, nws, cal), iters)
        rows[f"f3_kv_cache_write_{name}_70b"] = {
            "shape": f"T={t} heads={heads} head_dim={hd}", "us": round(ms * 1e3, 2),
            "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "note": note}
        log(rows[f"f3_kv_cache_write_{name}_70b"])
    del k, v, kc, vc, ws

    # decode: 12 sequences append one token each, in every one of 80 layers
    t = 12
    per_layer = []
    for layer in range(layers):
        k = up_bf16(workloads.outlier_act(t, width, 1000 + layer))
        v = up_bf16(workloads.normal_act(t, width, 2000 + layer))
        kc = torch.zeros((heads, s_rows, hd), dtype=torch.uint8, device=dev)
        vc = torch.zeros_like(kc)
        run = torch.full((2,), 4.0, dtype=torch.float32, device=dev)
        sc = torch.zeros(2, dtype=torch.float32, device=dev)
        slot = torch.arange(t, dtype=torch.int64, device=dev) * 600 + 7
        nws = L.fp8q_kv_cache_workspace_size(t, heads, hd)
        ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev)
        per_layer.append(make_call(k, v, t, slot, kc, vc, run, sc, ws, nws, 0))
        per_layer[-1].keep = (k, v, kc, vc, run, sc, slot, ws)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
        for call in per_layer:
            call(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.current_stream(dev).wait_stream(s)
    ms = time_eager(torch, g.replay, iters)
    b = layers * (2 * (3.0 * t * width) + 8 * t)
    rows["f3_kv_cache_write_decode_step_70b"] = {
        "shape": f"{layers} layers x T={t} heads={heads} head_dim={hd}", "us": round(ms * 1e3, 2),
        "us_per_layer": round(ms * 1e3 / layers, 2), "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
        "timing": "one HIP graph of 80 single-launch writes",
        "note": "launch-bound: 24 KB in and 24 KB out per layer"}
    log(rows["f3_kv_cache_write_decode_step_70b"])
    del per_layer, g
    torch.cuda.empty_cache()
    return rows


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, lin, w_bits, xs_bits, step_bytes, seconds: float = 10.0) -> dict:
    """The CPU oracle (unchanged, fp64) on one full decode step: the four
    q_proj calls M = 1, 8, 32, 64 on the oracle-quantized weight."""
    import oracle
    oracle.build()
    t0 = time.perf_counter()
    wq, ws, _ = oracle.quantize_weight(w_bits)
    tq = time.perf_counter() - t0
    reps = 0
    t0 = time.perf_counter()
    while True:                         # repeat whole steps for about `seconds` of CPU work
        for m in DECODE_MS:
            oracle.linear(0, xs_bits[m], wq, ws)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    return {"value": round(step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cpu_threads(),
            "kind": "oracle", "cpu_model": cpu_model(), "seconds_per_step": round(dt, 4),
            "steps_timed": reps, "quantize_weight_s": round(tq, 4),
            "sample": f"{reps} full decode steps (q_proj W[4096,4096], M=1,8,32,64), fp64 oracle "
                      "GEMM; weight quantization timed once, apart"}


def cpu_prefill(key, w_bits, x_bits, m, n, k) -> dict:
    """The oracle on a prefill workload: weight and activation quantization in
    full, and the fp64 W8A8 GEMM on 64 seeded rows x all N columns, with its
    linear extrapolation to all M rows (labelled as such)."""
    import numpy as np
    import oracle
    oracle.build()
    oq = {}
    tw = cpu_time(lambda: oq.update(w=oracle.quantize_weight(w_bits)), min_s=0.0)
    tx = cpu_time(lambda: oq.update(x=oracle.quantize_act(x_bits)), min_s=0.0)
    rows = np.sort(np.random.default_rng(64).choice(m, 64, replace=False))
    wq, ws, _ = oq["w"]
    xq, xs, _ = oq["x"]
    tg = cpu_time(lambda: oracle.linear(1, xq, wq, ws, xs, rows=rows), min_s=0.0)
    return {"quantize_weight_s": round(tw, 3), "quantize_act_s": round(tx, 3),
            "gemm_64_rows_s": round(tg, 3),
            "gemm_full_s_extrapolated": round(tg * m / 64, 2),
            "sample": f"M={m} N={n} K={k}: quantizers in full; GEMM measured on 64 seeded rows, "
                      "full size extrapolated linearly in M"}


def tiny_rows(fq, L, up_bf16, ptr, workloads, torch, dev, cpu) -> dict:
    """The Tiny workload (W [256, 512], X [16, 512], seed 0): weight
    quantization and the W8A16 linear, each as a HIP graph of 64 calls (both
    are launch-bound), and the oracle on the same inputs."""
    wl = workloads.WORKLOADS["tiny"]
    lin = wl.linears[0]
    m, n, k = wl.ms[0], lin.n, lin.k
    w_bits = workloads.weight(wl, lin)
    x_bits = workloads.activation(wl, m, k)
    w, x = up_bf16(w_bits), up_bf16(x_bits)
    q = torch.empty((n, k), dtype=torch.uint8, device=dev)
    sc = torch.empty(n, dtype=torch.float32, device=dev)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

    def tq(h):
        if L.fp8q_quantize_weight(ptr(w), n, k, k, ptr(q), k, ptr(sc), None, h) != 0:
            raise RuntimeError(fq._lib.last_error())

    def tl(h):
        if L.fp8q_linear(0, ptr(x), m, k, k, None, ptr(q), n, k, ptr(sc), ptr(y), n, None, 0, h) != 0:
            raise RuntimeError(fq._lib.last_error())
    tq(torch.cuda.current_stream(dev).cuda_stream)
    us_q = time_graph(torch, dev, [tq] * 64)
    us_l = time_graph(torch, dev, [tl] * 64)
    row = {"shape": f"W[{n},{k}] X[{m},{k}] seed 0", "quantize_weight_us": round(us_q, 3),
           "linear_us": round(us_l, 3), "linear_kernel": fq.describe_linear(0, m, n, k),
           "timing": "HIP graph of 64 calls each; launch-bound (0.16 MB of data)"}
    log("tiny", row)
    if cpu is not None:
        import oracle
        oracle.build()
        oq = {}
        cq = cpu_time(lambda: oq.update(w=oracle.quantize_weight(w_bits)))
        cl = cpu_time(lambda: oracle.linear(0, x_bits, oq["w"][0], oq["w"][1]))
        cpu["tiny"] = {"quantize_weight_s": round(cq, 6), "gemm_s": round(cl, 6),
                       "gpu_us": {"quantize_weight": row["quantize_weight_us"],
                                  "gemm": row["linear_us"]},
                       "sample": "the whole workload, repeated for at least 0.3 s"}
    return {"tiny": row}


if __name__ == "__main__":
    sys.exit(main())
