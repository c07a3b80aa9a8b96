"""Benchmark of the block-scaled quantized GEMM / dequant matvec path on one MI355X.

Prints ONE JSON line. The headline step is one MXFP8 GEMM of the prefill shape M=2048 (tokens),
K=4096, N=14336 (E4M3 data, E8M0 scales per 32 along K, fp32 accumulation, fp16 C): `value` is
its throughput in TFLOP/s (2*M*N*K per step over the HIP-event time of the timed steps, inputs
already resident in HBM). The other workloads of the path are measured in the same run and
reported under "detail": the MXFP4 GEMM (M=4096, N=8192, K=8192), the mixed E4M3 x E2M1 GEMM and
the E5M2 x E5M2 GEMM at the prefill shape (against the fp8 peak), the prefill GEMM with binary16
activations quantised inside the GEMM against mx_pack_run + GEMM, the FP6 E2M3 x E2M3 GEMM at the
prefill shape (against the fp6 peak, equal to fp4's), the fp16 GEMM (4096^3), the
small MXFP8 GEMM (128x256x128, a latency figure), the int8/int4 dequant matvec (M=1 and M=8,
K=4096, N=14336; GB/s of algorithmic bytes), the same int8/int4-weight product at M=128 (N=12288)
and M=64 (N=4096) with K=4096 (TFLOP/s against the fp16 peak) and the GPU pack/unpack codecs.

Timing: per workload, --settle seconds (default 0.5) of untimed calls so that the shader clock
reaches its sustained-load level, W warm-up steps, then K steps between two HIP events recorded
on the stream the kernels are launched on, bracketed by device synchronisation. Inputs rotate over several copies so that
repeats are not served by the 256 MB Infinity Cache (3 sets for GEMMs, >= 384 MB of weights for
the matvec). The CPU baseline is the oracle timed on the host cores on every workload measured: the
whole output where small, else whole rows for about --cpu-seconds each, extrapolated.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# The pages' own throughput figures, on other hardware: context for the fp16 GEMM detail line, not a
# target (they print none for a block-scaled GEMM or a dequant matvec). "TileLang Metal Backend
# Internals", section 5.6 (current performance snapshot): fp16 in and out, fp32 accumulation, full
# tiles, mean of 100 timed runs, Apple M5 with a 10-core GPU.
PAGES_CONTEXT = {
    "note": "the pages' figures on Apple M5 (10-core GPU), other hardware: context, not a target",
    "source": "TileLang Metal Backend Internals, section 5.6",
    "fp16_gemm_4096x4096x4096_tflops": {"pytorch_mps": 13.6, "mlx": 12.7, "tilelang": 12.9},
    "compare_with_detail": "fp16_gemm_4096x4096x4096",
}

PEAK = {  # MI355X dense peaks (256 CUs x 2.4 GHz x flop/clk/CU) and HBM bandwidth
    "mxfp8": 5033.2, "mxfp6": 10066.3, "mxfp4": 10066.3, "fp16": 2516.6, "hbm_gbs": 8000.0,
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def hbm_traffic(kernel, tile, shape):
    """HBM bytes per launch of the headline kernel, as measured by the rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes summarised under profiles/ (a line "traffic_record: {json}" naming kernel,
    tile and shape). None when no record matches the kernel this run uses."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None, None
    for name in sorted(os.listdir(pdir)):
        if not name.endswith((".md", ".txt")):
            continue
        with open(os.path.join(pdir, name)) as f:
            for line in f:
                if not line.startswith("traffic_record: "):
                    continue
                rec = json.loads(line[len("traffic_record: "):])
                if rec.get("kernel") == kernel and rec.get("tile") == tile and tuple(rec.get("shape", ())) == shape:
                    return rec["bytes_per_launch"], f"profiles/{name}"
    return None, None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_info(torch):
    """The GPU the run used: name, architecture and compute-unit count (the peaks above assume
    256 CUs at 2.4 GHz, AMD's MI355X figures)."""
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "gcn_arch": getattr(pr, "gcnArchName", ""), "cus": pr.multi_processor_count,
            "memory_gib": round(pr.total_memory / 2**30, 1)}


def host_pack_times(np, synth):
    """The library's host codec (mx_pack_host, one thread) packing the fp32 sources of each GEMM
    workload and the matvec weights: context beside the oracle timings."""
    import ctypes
    from block_scaled_quantized_amd import api
    out = {}
    for name, fmt, shapes in (("mxfp8_gemm_128x256x128", api.MX_E4M3, ((128, 128), (256, 128))),
                              ("mxfp8_gemm_2048x14336x4096", api.MX_E4M3, ((2048, 4096), (14336, 4096))),
                              ("mxfp4_gemm_4096x8192x8192", api.MX_E2M1, ((4096, 8192), (8192, 8192))),
                              ("matvec_int8_4096x14336", api.MX_INT8, ((4096, 14336),)),
                              ("matvec_int4_4096x14336", api.MX_INT4, ((4096, 14336),))):
        secs, nbytes = 0.0, 0
        for rows, cols in shapes:
            src = np.ascontiguousarray(synth.normal((rows, cols), 1.0, 7), dtype=np.float32)
            if fmt in (api.MX_INT8, api.MX_INT4):
                cs, ss = api.int_shapes(fmt, rows, cols)
                codes, scales = np.empty(cs, np.uint8), np.empty(ss, np.float16)
            else:
                cs, ss = api.mx_shapes(fmt, rows, cols)
                codes, scales = np.empty(cs, np.uint8), np.empty(ss, np.uint8)
            t0 = time.perf_counter()
            api.mx_pack_host(fmt, src, rows, cols, codes, scales)
            secs += time.perf_counter() - t0
            nbytes += src.nbytes
        out[name] = {"seconds": secs, "source_gbs": nbytes / secs / 1e9, "threads": 1}
    return out


def cpu_baseline(np, synth, C_prefill, keep, budget_s):
    """The oracle (oracle/, plain C, fp64) timed on the host on every workload whose GPU output this
    run kept: the whole output where it is small (the 128x256x128 GEMM, the matvecs), else whole
    rows of C computed in chunks of one row per thread until `budget_s` seconds have passed, with
    the full-output time extrapolated (rows are independent and cost the same). The oracle
    quantises the fp32 sources itself. Each checked GPU row is compared with the acceptance bound;
    the E4M3 pack's rows (the oracle's quantiser on the same fp32 source) are compared bit for bit."""
    import oracle as orc
    affinity = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(affinity, int(env)) if env.isdigit() and int(env) > 0 else affinity
    orc.set_threads(threads)
    threads = orc.num_threads()
    configs = {}

    def rows_leg(name, M, N, K, flops_row, run_rows, R, gpu, unit_flops=True):
        done, t, worst = 0, 0.0, 0.0
        while done < M and (t < budget_s or done == 0):
            n = min(threads, M - done)
            t0 = time.perf_counter()
            ref = run_rows(done, n)
            t += time.perf_counter() - t0
            _, ratio, _ = orc.check(gpu[done:done + n].cpu().numpy().astype(np.float64), ref, K, R)
            worst = max(worst, ratio)
            done += n
        configs[name] = {"rows": done, "of_rows": M, "seconds": t, "extrapolated": done < M,
                         "full_output_seconds": t * M / done,
                         "tflops": flops_row * done / t / 1e12, "gpu_worst_err_over_bound": worst}

    def mx_leg(name, fmt, M, N, K, wl, sigma_b, gpu):
        a_src = synth.normal((M, K), 1.0, synth.seed_for(wl, 0))
        b_src = synth.normal((N, K), sigma_b, synth.seed_for(wl, 1))
        oA, oSA = orc.mx_quantize(fmt, a_src)
        oB, oSB = orc.mx_quantize(fmt, b_src)
        del a_src, b_src
        R = orc.rms_ab(orc.dequant(fmt, oA, oSA, M, K), orc.dequant(fmt, oB, oSB, N, K).T)
        rows_leg(name, M, N, K, 2.0 * N * K,
                 lambda r0, n: orc.mxgemm(fmt, fmt, oA, oSA, oB, oSB, M, N, K, row0=r0, nrows=n), R, gpu)

    log_ = lambda m: print(f"[bench] cpu: {m}", file=sys.stderr, flush=True)
    if "mxfp8_small" in keep:
        log_("mxfp8 128x256x128")
        mx_leg("mxfp8_gemm_128x256x128", orc.E4M3, 128, 256, 128, synth.MXFP8_SMALL, 1.0, keep["mxfp8_small"])
    if "fp16" in keep:
        log_("fp16 4096^3")
        A16 = synth.uniform_pm1((4096, 4096), synth.seed_for(synth.F16_SQUARE, 0)).astype(np.float16)
        B16 = synth.uniform_pm1((4096, 4096), synth.seed_for(synth.F16_SQUARE, 1)).astype(np.float16)
        R = orc.rms_ab(A16.astype(np.float64), B16.astype(np.float64))
        rows_leg("fp16_gemm_4096x4096x4096", 4096, 4096, 4096, 2.0 * 4096 * 4096,
                 lambda r0, n: orc.gemm_f16(A16, B16, row0=r0, nrows=n), R, keep["fp16"])
        del A16, B16
    log_("mxfp8 prefill 2048x14336x4096")
    mx_leg("mxfp8_gemm_2048x14336x4096", orc.E4M3, 2048, 14336, 4096, synth.MXFP8_PREFILL, 0.02, C_prefill)
    if any(k.startswith("matvec_") for k in keep):
        Km, Nm = 4096, 14336
        w = synth.normal((Km, Nm), 0.02, synth.seed_for(synth.MATVEC, 1))
        x8 = synth.normal((8, Km), 1.0, synth.seed_for(synth.MATVEC, 0)).astype(np.float16)
        for fw, name in ((orc.INT8, "int8"), (orc.INT4, "int4")):
            q, s = orc.int_quantize(fw, w)
            oW = q.view(np.uint8) if fw == orc.INT8 else orc.pack_int4(q)
            wdeq = orc.dequant(fw, oW, s, Km, Nm)
            for Mv in (1, 8):
                key = f"matvec_{name}_M{Mv}"
                if key not in keep:
                    continue
                log_(key)
                x = x8[:Mv]
                t0 = time.perf_counter()
                ref = orc.matvec(fw, x, oW, s, Km, Nm)
                t = time.perf_counter() - t0
                _, ratio, _ = orc.check(keep[key].cpu().numpy().astype(np.float64), ref, Km,
                                        orc.rms_ab(x.astype(np.float64), wdeq))
                nbytes = oW.size + 2 * s.size + 2 * Mv * Km + 2 * Mv * Nm
                configs[key] = {"rows": Mv, "of_rows": Mv, "seconds": t, "extrapolated": False,
                                "full_output_seconds": t, "gbs": nbytes / t / 1e9,
                                "gpu_worst_err_over_bound": ratio}
        del w
    if "mxfp4" in keep:
        log_("mxfp4 4096x8192x8192")
        mx_leg("mxfp4_gemm_4096x8192x8192", orc.E2M1, 4096, 8192, 8192, synth.MXFP4_LARGE, 1.0, keep["mxfp4"])
    for Mq, Nq, Kq in ((128, 12288, 4096), (64, 4096, 4096)):   # the small-M weight GEMM, row by row
        if not any(k.startswith(f"wq_gemm_") and k.endswith(f"_{Mq}x{Nq}x{Kq}") for k in keep):
            continue
        w = synth.normal((Kq, Nq), 0.02, synth.seed_for(synth.WQ_PREFILL, 1))
        xq = synth.normal((Mq, Kq), 1.0, synth.seed_for(synth.WQ_PREFILL, 0)).astype(np.float16)
        for fw, name in ((orc.INT4, "int4"), (orc.INT8, "int8")):
            key = f"wq_gemm_{name}_{Mq}x{Nq}x{Kq}"
            if key not in keep:
                continue
            log_(key)
            q, s = orc.int_quantize(fw, w)
            oW = q.view(np.uint8) if fw == orc.INT8 else orc.pack_int4(q)
            R = orc.rms_ab(xq.astype(np.float64), orc.dequant(fw, oW, s, Kq, Nq))
            rows_leg(key, Mq, Nq, Kq, 2.0 * Nq * Kq,
                     lambda r0, n: orc.matvec(fw, xq[r0:r0 + n], oW, s, Kq, Nq), R, keep[key])
        del w
    if "pack_e4m3" in keep:   # the quantiser (brute-force nearest code per element), row by row
        log_("pack e4m3 2048x4096")
        src = synth.normal((2048, 4096), 1.0, synth.seed_for(synth.MXFP8_PREFILL, 0))
        g_codes, g_scales = (t.cpu().numpy() for t in keep["pack_e4m3"])
        done, t, exact = 0, 0.0, True
        while done < 2048 and (t < budget_s or done == 0):
            n = min(threads, 2048 - done)
            t0 = time.perf_counter()
            oc, osc = orc.mx_quantize(orc.E4M3, src[done:done + n])
            t += time.perf_counter() - t0
            exact = exact and np.array_equal(oc, g_codes[done:done + n]) and np.array_equal(osc, g_scales[done:done + n])
            done += n
        configs["pack_e4m3_2048x4096"] = {"rows": done, "of_rows": 2048, "seconds": t, "extrapolated": done < 2048,
                                          "full_output_seconds": t * 2048 / done,
                                          "source_gbs": done * 4096 * 4 / t / 1e9, "gpu_bit_exact": bool(exact)}
    head = configs["mxfp8_gemm_2048x14336x4096"]
    return {"value": head["tflops"], "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{head['rows'] - 1} of C for the MXFP8 GEMM M=2048,N=14336,K=4096 "
                      f"({head['rows']}x14336x4096 MACs in {head['seconds']:.1f} s, fp64, closed-form decode per "
                      f"element); the other workloads under 'configs'",
            "cpu_model": cpu_model(), "affinity_cpus": affinity, "omp_threads": threads,
            "budget_s_per_config": budget_s, "configs": configs}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle", type=float, default=0.5,
                   help="seconds of untimed load before each workload's warm-up steps (clock ramp)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=4.0,
                   help="oracle seconds per large workload in the CPU baseline (whole rows, extrapolated)")
    p.add_argument("--only", default="", help="comma list of detail workloads to run (default all)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs the kernels on one GPU; multi-GPU runs are not implemented (--gpus must be 1)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from block_scaled_quantized_amd import api, synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def settle(fn, seconds=0.5):
        """Run fn until `seconds` of wall time have passed: under sustained MFMA load the shader
        clock takes a few hundred ms to reach its steady state, and a timed region of a few ms
        that starts cold measures the ramp, not the kernel."""
        t_end = time.perf_counter() + seconds
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn(i)
                i += 1
            torch.cuda.synchronize()

    def timed(fn, steps, warmup):
        """Mean ms per call of fn(i) over `steps` calls, HIP events on the launch stream."""
        settle(fn, args.settle)
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def mx_operands(fmt, M, N, K, wl, sigma_b, copies):
        a_src = synth.normal((M, K), 1.0, synth.seed_for(wl, 0))
        b_src = synth.normal((N, K), sigma_b, synth.seed_for(wl, 1))
        cs, ss = api.mx_shapes(fmt, M, K)
        A = torch.empty(cs, dtype=torch.uint8, device=dev)
        SA = torch.empty(ss, dtype=torch.uint8, device=dev)
        api.mx_pack_run(fmt, d(a_src), M, K, A, SA)
        cs, ss = api.mx_shapes(fmt, N, K)
        B = torch.empty(cs, dtype=torch.uint8, device=dev)
        SB = torch.empty(ss, dtype=torch.uint8, device=dev)
        api.mx_pack_run(fmt, d(b_src), N, K, B, SB)
        sets = [(A, SA, B, SB)] + [(A.clone(), SA.clone(), B.clone(), SB.clone()) for _ in range(copies - 1)]
        torch.cuda.synchronize()
        return sets, a_src, b_src

    # ---------------- headline: MXFP8 prefill GEMM ----------------------------------------
    M, N, K = 2048, 14336, 4096
    sets, a_src, b_src = mx_operands(api.MX_E4M3, M, N, K, synth.MXFP8_PREFILL, 0.02, 3)
    plan = api.mxgemm_create(M, N, K, api.MX_E4M3, api.MX_E4M3)
    tile = api.mxgemm_plan_info(plan)
    Cs = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(3)]

    def step(i):
        A, SA, B, SB = sets[i % 3]
        api.mxgemm_run(plan, A, SA, B, SB, Cs[i % 3], stream)

    log("timing mxfp8 prefill GEMM")
    ms = timed(step, args.steps, args.warmup)
    flops = 2.0 * M * N * K
    tflops = flops / (ms * 1e-3) / 1e12
    C0 = Cs[0]
    # a separate pass with an event pair around every call: the median per call beside the mean
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    median_ms = per_call[len(per_call) // 2]

    detail = {}
    keep = {}  # GPU outputs the CPU baseline checks, by workload
    only = set(filter(None, args.only.split(",")))  # "none" skips every detail workload

    def want(name):
        return not only or name in only

    # ---------------- MXFP4 GEMM -------------------------------------------------------------
    if want("mxfp4_large"):
        log("timing mxfp4 GEMM")
        M4, N4, K4 = 4096, 8192, 8192
        s4, _, _ = mx_operands(api.MX_E2M1, M4, N4, K4, synth.MXFP4_LARGE, 1.0, 3)
        p4 = api.mxgemm_create(M4, N4, K4, api.MX_E2M1, api.MX_E2M1)
        C4 = [torch.empty((M4, N4), dtype=torch.float16, device=dev) for _ in range(3)]
        t = timed(lambda i: api.mxgemm_run(p4, *s4[i % 3], C4[i % 3], stream), args.steps, args.warmup)
        keep["mxfp4"] = C4[0]
        tf = 2.0 * M4 * N4 * K4 / (t * 1e-3) / 1e12
        detail["mxfp4_gemm_4096x8192x8192"] = {"ms": t, "tflops": tf, "frac_peak": tf / PEAK["mxfp4"],
                                               "tile": api.mxgemm_plan_info(p4)}
        del s4, C4

    # ---------------- mixed MX pair: E4M3 activations x E2M1 weights at the prefill shape -----------
    if want("mixed_prefill"):
        log("timing mixed E4M3 x E2M1 GEMM")
        sa, _, _ = mx_operands(api.MX_E4M3, M, 64, K, synth.MXFP8_PREFILL, 1.0, 1)   # A (E4M3) only
        sb, _, _ = mx_operands(api.MX_E2M1, 64, N, K, synth.MXFP4_LARGE, 0.02, 1)    # B (E2M1) only
        A8, SA8 = sa[0][0], sa[0][1]
        B4, SB4 = sb[0][2], sb[0][3]
        msets = [(A8, SA8, B4, SB4)] + [(A8.clone(), SA8.clone(), B4.clone(), SB4.clone()) for _ in range(2)]
        pm = api.mxgemm_create(M, N, K, api.MX_E4M3, api.MX_E2M1)
        Cm = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(3)]
        t = timed(lambda i: api.mxgemm_run(pm, *msets[i % 3], Cm[i % 3], stream), args.steps, args.warmup)
        tf = flops / (t * 1e-3) / 1e12
        detail["mixed_e4m3_x_e2m1_gemm_2048x14336x4096"] = {"ms": t, "tflops": tf, "frac_peak": tf / PEAK["mxfp8"],
                                                            "tile": api.mxgemm_plan_info(pm)}
        del sa, sb, msets
        # the other order: E2M1 activations (A) with E4M3 weights (B)
        log("timing mixed E2M1 x E4M3 GEMM")
        sa, _, _ = mx_operands(api.MX_E2M1, M, 64, K, synth.MXFP8_PREFILL, 1.0, 1)   # A (E2M1) only
        sb, _, _ = mx_operands(api.MX_E4M3, 64, N, K, synth.MXFP4_LARGE, 0.02, 1)    # B (E4M3) only
        A4, SA4 = sa[0][0], sa[0][1]
        B8, SB8 = sb[0][2], sb[0][3]
        msets = [(A4, SA4, B8, SB8)] + [(A4.clone(), SA4.clone(), B8.clone(), SB8.clone()) for _ in range(2)]
        pm2 = api.mxgemm_create(M, N, K, api.MX_E2M1, api.MX_E4M3)
        t = timed(lambda i: api.mxgemm_run(pm2, *msets[i % 3], Cm[i % 3], stream), args.steps, args.warmup)
        tf = flops / (t * 1e-3) / 1e12
        detail["mixed_e2m1_x_e4m3_gemm_2048x14336x4096"] = {"ms": t, "tflops": tf, "frac_peak": tf / PEAK["mxfp8"],
                                                            "tile": api.mxgemm_plan_info(pm2)}
        api.mxgemm_destroy(pm2)
        del sa, sb, msets, Cm

    # ---------------- E5M2 x E5M2 at the prefill shape -------------------------------------------------
    if want("e5m2_prefill"):
        log("timing E5M2 GEMM")
        s5, _, _ = mx_operands(api.MX_E5M2, M, N, K, synth.MXFP8_PREFILL, 0.02, 3)
        p5 = api.mxgemm_create(M, N, K, api.MX_E5M2, api.MX_E5M2)
        C5 = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(3)]
        t = timed(lambda i: api.mxgemm_run(p5, *s5[i % 3], C5[i % 3], stream), args.steps, args.warmup)
        tf = flops / (t * 1e-3) / 1e12
        detail["mxfp8_e5m2_gemm_2048x14336x4096"] = {"ms": t, "tflops": tf, "frac_peak": tf / PEAK["mxfp8"],
                                                     "tile": api.mxgemm_plan_info(p5)}
        del s5, C5

    # ---------------- FP6 E2M3 x E2M3 at the prefill shape ----------------------------------------------
    if want("fp6_prefill"):
        log("timing FP6 GEMM")
        s6, _, _ = mx_operands(api.MX_E2M3, M, N, K, synth.MXFP8_PREFILL, 0.02, 3)
        p6 = api.mxgemm_create(M, N, K, api.MX_E2M3, api.MX_E2M3)
        C6 = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(3)]
        t = timed(lambda i: api.mxgemm_run(p6, *s6[i % 3], C6[i % 3], stream), args.steps, args.warmup)
        tf = flops / (t * 1e-3) / 1e12
        detail["mxfp6_e2m3_gemm_2048x14336x4096"] = {"ms": t, "tflops": tf, "frac_peak": tf / PEAK["mxfp6"],
                                                     "tile": api.mxgemm_plan_info(p6)}
        del s6, C6

    # ---------------- fp16 activations quantised inside the GEMM, against pack + GEMM ---------------
    if want("quant_a"):
        log("timing quantise-on-load GEMM")
        a16 = [d(a_src.astype(np.float16)) for _ in range(3)]
        a32 = [d(a_src) for _ in range(3)]
        pq = api.mxgemm_create(M, N, K, api.MX_E4M3, api.MX_E4M3, api.MXGEMM_QUANT_A)
        Cq = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(3)]
        t_f = timed(lambda i: api.mxgemm_run(pq, a16[i % 3], None, sets[i % 3][2], sets[i % 3][3], Cq[i % 3], stream),
                    args.steps, args.warmup)

        def pack_gemm(i):
            A_, SA_, B_, SB_ = sets[i % 3]
            api.mx_pack_run(api.MX_E4M3, a32[i % 3], M, K, A_, SA_, stream)
            api.mxgemm_run(plan, A_, SA_, B_, SB_, Cq[i % 3], stream)
        t_pg = timed(pack_gemm, args.steps, args.warmup)
        detail["mxfp8_quant_a_2048x14336x4096"] = {
            "fused_us": t_f * 1e3, "fused_tflops": flops / (t_f * 1e-3) / 1e12,
            "pack_fp32_plus_gemm_us": t_pg * 1e3, "pack_plus_gemm_tflops": flops / (t_pg * 1e-3) / 1e12,
            "default": "pack + GEMM" if t_pg <= t_f else "fused",
            "note": "fused: binary16 A quantised to E4M3 inside the GEMM (MXGEMM_QUANT_A); pack + GEMM: "
                    "mx_pack_run from fp32 A, then the GEMM on the codes"}
        del a16, a32, Cq

    # ---------------- fp16 GEMM ----------------------------------------------------------------
    if want("f16_square"):
        log("timing fp16 GEMM")
        Mf = Nf = Kf = 4096
        Af = d(synth.uniform_pm1((Mf, Kf), synth.seed_for(synth.F16_SQUARE, 0)).astype(np.float16))
        Bf = d(synth.uniform_pm1((Kf, Nf), synth.seed_for(synth.F16_SQUARE, 1)).astype(np.float16))
        fsets = [(Af, Bf)] + [(Af.clone(), Bf.clone()) for _ in range(2)]
        pf = api.mxgemm_create(Mf, Nf, Kf, api.MX_F16, api.MX_F16)
        Cf = [torch.empty((Mf, Nf), dtype=torch.float16, device=dev) for _ in range(3)]
        t = timed(lambda i: api.mxgemm_run(pf, fsets[i % 3][0], None, fsets[i % 3][1], None, Cf[i % 3], stream),
                  args.steps, args.warmup)
        keep["fp16"] = Cf[0]
        tf = 2.0 * Mf * Nf * Kf / (t * 1e-3) / 1e12
        detail["fp16_gemm_4096x4096x4096"] = {"ms": t, "tflops": tf, "frac_peak": tf / PEAK["fp16"],
                                              "tile": api.mxgemm_plan_info(pf)}
        del fsets, Cf

    # ---------------- small MXFP8 GEMM (latency) -----------------------------------------------
    if want("mxfp8_small"):
        log("timing small mxfp8 GEMM")
        Ms, Ns, Ks = 128, 256, 128
        ss_, _, _ = mx_operands(api.MX_E4M3, Ms, Ns, Ks, synth.MXFP8_SMALL, 1.0, 1)
        ps = api.mxgemm_create(Ms, Ns, Ks, api.MX_E4M3, api.MX_E4M3)
        Csm = torch.empty((Ms, Ns), dtype=torch.float16, device=dev)
        t = timed(lambda i: api.mxgemm_run(ps, *ss_[0], Csm, stream), args.steps, args.warmup)
        keep["mxfp8_small"] = Csm
        detail["mxfp8_gemm_128x256x128"] = {"us": t * 1e3, "tflops": 2.0 * Ms * Ns * Ks / (t * 1e-3) / 1e12,
                                            "tile": api.mxgemm_plan_info(ps)}

    # ---------------- dequant matvec ---------------------------------------------------------------
    if want("matvec"):
        log("timing matvec")
        Km, Nm = 4096, 14336
        w = synth.normal((Km, Nm), 0.02, synth.seed_for(synth.MATVEC, 1))
        x8 = synth.normal((8, Km), 1.0, synth.seed_for(synth.MATVEC, 0)).astype(np.float16)
        wd = d(w)
        xd = d(x8)
        for fw, name, copies in ((api.MX_INT8, "int8", 7), (api.MX_INT4, "int4", 12)):
            cs, ss = api.int_shapes(fw, Km, Nm)
            W = torch.empty(cs, dtype=torch.uint8, device=dev)
            Ws = torch.empty(ss, dtype=torch.float16, device=dev)
            api.mx_pack_run(fw, wd, Km, Nm, W, Ws)
            wsets = [(W, Ws)] + [(W.clone(), Ws.clone()) for _ in range(copies - 1)]
            for Mv in (1, 8):
                y = torch.empty((Mv, Nm), dtype=torch.float16, device=dev)
                xv = xd[:Mv].contiguous()
                need = api.mxmatvec_workspace_size(Mv, Nm, Km, fw)
                ws = torch.zeros(max(16, need), dtype=torch.uint8, device=dev)
                nbytes = W.numel() + Ws.numel() * 2 + Mv * Km * 2 + Mv * Nm * 2
                for label, wsp in (("", ws), ("_single_pass", None)):
                    t = timed(lambda i: api.mxmatvec_run(Mv, Nm, Km, xv, wsets[i % copies][0], fw, wsets[i % copies][1],
                                                         y, wsp, None, stream), args.steps, args.warmup)
                    gbs = nbytes / (t * 1e-3) / 1e9
                    keep[f"matvec_{name}_M{Mv}"] = y.clone()
                    detail[f"matvec_{name}_M{Mv}{label}"] = {"us": t * 1e3, "gbs": gbs, "frac_hbm": gbs / PEAK["hbm_gbs"],
                                                            "bytes": nbytes, "weight_copies": copies,
                                                            "workspace_bytes": need if wsp is not None else 0}
            del wsets
        del wd

    # ---------------- int8 / int4-weight GEMM with fp16 block scales at small M ----------------------
    if want("wq_gemm"):
        log("timing small-M weight-quantised GEMM")
        # M=160 leaves a second round of 64 x 128 tiles part-filled: with a workspace its blocks are
        # dealt out in equal runs
        for Mq, Nq, Kq in ((128, 12288, 4096), (64, 4096, 4096), (160, 12288, 4096)):
            wq = d(synth.normal((Kq, Nq), 0.02, synth.seed_for(synth.WQ_PREFILL, 1)))
            xq = d(synth.normal((Mq, Kq), 1.0, synth.seed_for(synth.WQ_PREFILL, 0)).astype(np.float16))
            yq = torch.empty((Mq, Nq), dtype=torch.float16, device=dev)
            for fw, name in ((api.MX_INT4, "int4"), (api.MX_INT8, "int8")):
                cs, ss = api.int_shapes(fw, Kq, Nq)
                W = torch.empty(cs, dtype=torch.uint8, device=dev)
                Ws = torch.empty(ss, dtype=torch.float16, device=dev)
                api.mx_pack_run(fw, wq, Kq, Nq, W, Ws)
                # enough weight copies (>= 384 MB) that repeats are not served by the Infinity Cache
                nq = max(3, -(-(384 << 20) // (W.numel() + 2 * Ws.numel())))
                qsets = [(W, Ws)] + [(W.clone(), Ws.clone()) for _ in range(nq - 1)]
                # with a workspace K is split across workgroups where the unsplit grid is small (the
                # default a caller with a workspace gets); without one, the unsplit kernel
                need = api.mxmatvec_workspace_size(Mq, Nq, Kq, fw)
                wsq = torch.zeros(max(16, need), dtype=torch.uint8, device=dev) if need else None
                nbytes = W.numel() + Ws.numel() * 2 + Mq * Kq * 2 + Mq * Nq * 2
                for label, wsp in (("", wsq), ("_no_workspace", None)):
                    if label and need == 0:
                        continue
                    t = timed(lambda i: api.mxmatvec_run(Mq, Nq, Kq, xq, qsets[i % nq][0], fw, qsets[i % nq][1], yq,
                                                         wsp, None, stream), args.steps, args.warmup)
                    if not label:
                        keep[f"wq_gemm_{name}_{Mq}x{Nq}x{Kq}"] = yq.clone()
                    tf = 2.0 * Mq * Nq * Kq / (t * 1e-3) / 1e12
                    detail[f"wq_gemm_{name}_{Mq}x{Nq}x{Kq}{label}"] = {
                        "us": t * 1e3, "tflops": tf, "frac_peak_fp16": tf / PEAK["fp16"],
                        "gbs": nbytes / (t * 1e-3) / 1e9, "weight_copies": nq,
                        "workspace_bytes": need if wsp is not None else 0}
                del qsets
            del wq, xq, yq

    # ---------------- codecs -------------------------------------------------------------------------
    if want("codec"):
        log("timing codecs")
        rows, cols = 2048, 4096
        src = d(a_src)
        A8 = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        S8 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        t = timed(lambda i: api.mx_pack_run(api.MX_E4M3, src, rows, cols, A8, S8, stream), args.steps, args.warmup)
        nbytes = rows * cols * 4 + rows * cols + rows * cols // 32
        detail["pack_e4m3_2048x4096"] = {"us": t * 1e3, "gbs": nbytes / (t * 1e-3) / 1e9}
        keep["pack_e4m3"] = (A8.clone(), S8.clone())
        out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
        t = timed(lambda i: api.mx_unpack_run(api.MX_E4M3, A8, S8, rows, cols, out, stream), args.steps, args.warmup)
        detail["unpack_e4m3_2048x4096"] = {"us": t * 1e3, "gbs": nbytes / (t * 1e-3) / 1e9}

    # ---------------- plain device copy (HBM reference and traffic-counter calibration) ------------
    if want("copy"):
        log("timing device copy")
        nbytes = 256 << 20
        csrc = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        cdst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        csrc.fill_(1)
        t = timed(lambda i: cdst.copy_(csrc), args.steps, args.warmup)
        detail["device_copy_256MiB"] = {"us": t * 1e3, "gbs": 2 * nbytes / (t * 1e-3) / 1e9,
                                        "bytes_read": nbytes, "bytes_written": nbytes}
        del csrc, cdst

    # ---------------- CPU baseline: the oracle on each workload ------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        torch.cuda.synchronize()
        cpu = cpu_baseline(np, synth, C0, keep, args.cpu_seconds)
        cpu["host_pack"] = host_pack_times(np, synth)

    kname = {4: "gemm_pp_ring_kernel", 3: "gemm_ring_kernel", 2: "gemm_pp_kernel"}.get(tile[3], "gemm_kernel")
    traffic, traffic_src = hbm_traffic(kname, list(tile), (M, N, K))

    out = {
        "metric": "block-scaled GEMM TFLOPS & % MFMA peak (MXFP8/MXFP4); int8 matvec GB/s",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 (e4m3 x e8m0/32, fp32 accumulate, fp16 out)",
        "data": "synthetic: seeded PCG64, activations N(0,1), weights 0.02*N(0,1), quantised on the GPU",
        "median_ms_per_call": median_ms,
        "config": {"workload": "mxfp8_gemm_prefill M=2048 N=14336 K=4096", "M": M, "N": N, "K": K,
                   "tile_m_n_k": list(tile), "input_sets_rotated": 3},
        "device": device_info(torch),
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK["mxfp8"], "unit": "TFLOP/s",
                     "frac": tflops / PEAK["mxfp8"], "traffic": traffic,
                     "kernel": f"{kname}<E4M3, {tile[0]}x{tile[1]}>",
                     "flops_per_launch": flops, "traffic_source": traffic_src},
        "cpu_baseline": cpu,
        "detail": detail,
        "context": PAGES_CONTEXT,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
