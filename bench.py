"""Benchmark of the NVFP4 MoE hot path on one MI355X.

One step = one full MoE layer: route + permute, NVFP4 quantisation of the tokens, gate/up
grouped GEMM with SwiGLU, requantisation, down grouped GEMM, FINALIZE.  Default workload:
the decode layer at ~32 rows per expert (1024 tokens, 256 experts, top-8, hidden 6144,
intermediate 2048).  Inputs are seeded synthetic data (see synth/), resident in HBM before
the timed region.  Prints one JSON line.

value = grouped-GEMM FLOPs of the step (2 * sum_e M_e * N * K over both GEMMs, real rows
only) / step time, in TFLOPS.  The roofline object is for the dominant kernel (the gate/up
grouped GEMM), timed with HIP events on the stream it is launched on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE grouped-GEMM TFLOPS + weight HBM GB/s (% roofline) at ~32 tok/expert"
HBM_PEAK_GBPS = 8000.0
F16_PEAK_TFLOPS = 2500.0   # dense fp16 MFMA: the ceiling of the exact NVFP4 path
FP4_PEAK_TFLOPS = 10100.0  # dense FP4 MFMA (power-of-two scales per 32 only): context
WORKLOADS = {"layer_decode": "LAYER_DECODE", "layer_skewed": "LAYER_SKEWED", "layer_prefill": "LAYER_PREFILL",
             "layer_tiny": "TINY", "layer_ep8": "LAYER_EP8", "layer_tp8": "LAYER_TP8",
             "gemm_e8_m32": "GEMM_DECODE"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="layer_decode", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the named workload (no further configurations or measured peaks); "
                         "for short profiler runs")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB three times (to scale HBM "
                         "byte counters against a kernel of known traffic) and exit")
    ap.add_argument("--power-sample", action="store_true",
                    help="only run the decode layer's GEMMs back to back for a few seconds each while "
                         "amd-smi samples board power and clocks midway; print one JSON line and exit")
    return ap.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "layer_decode_t1024_e256_k8_hbm_traffic.md")


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy of known size), or None when the summary is missing or the
    kernel sources changed since the counters were taken."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    blob = json.loads(m.group(1))
    h = hashlib.sha256()
    for p in blob["kernel_sources"]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != blob["kernel_sources_sha256"] or kernel not in blob["per_launch"]:
        return None
    return blob["per_launch"][kernel]["bytes"]


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


_probe = None


def probes():
    """The measurement kernels, streaming read and MFMA throughput
    (block_scaled_fp4_02_amd/libmoe_probes.so)."""
    global _probe
    if _probe is None:
        import ctypes as C
        path = os.path.join(ROOT, "block_scaled_fp4_02_amd", "libmoe_probes.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(path)
        L.moe_probe_stream_read_variants.restype = C.c_int
        L.moe_probe_stream_read_variant_info.restype = C.c_int
        L.moe_probe_stream_read_variant_info.argtypes = [C.c_int]
        L.moe_probe_stream_read_groups.restype = C.c_int64
        L.moe_probe_stream_read_groups.argtypes = [C.c_int64, C.c_int, C.c_int64]
        L.moe_probe_stream_read.restype = C.c_int
        L.moe_probe_stream_read.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_int64, C.c_void_p, C.c_void_p]
        L.moe_probe_mfma_kinds.restype = C.c_int
        L.moe_probe_mfma_flops_per_wave_iter.restype = C.c_double
        L.moe_probe_mfma_flops_per_wave_iter.argtypes = [C.c_int]
        L.moe_probe_mfma_expected_sink.restype = C.c_double
        L.moe_probe_mfma_expected_sink.argtypes = [C.c_int, C.c_int]
        L.moe_probe_mfma_peak.restype = C.c_int
        L.moe_probe_mfma_peak.argtypes = [C.c_int, C.c_int64, C.c_int, C.c_void_p, C.c_void_p]
        _probe = L
    return _probe


MFMA_KINDS = ("f16_16x16x32", "fp4_16x16x128")


def mfma_peak(torch, iters: int = 2048, launches: int = 5) -> dict:
    """Measured dense MFMA throughput per kind (fp16 16x16x32, FP4 16x16x128 with unit block
    scales): back-to-back MFMAs on register operands over 4, 8 or 16 workgroups of four waves
    per CU, HIP events on the launch stream; the fastest grid is the measured peak at the
    clock the board holds under that load.  Each launch's sums are checked against their
    exact value."""
    import ctypes as C
    L = probes()
    stream = torch.cuda.current_stream()
    sp = C.c_void_p(stream.cuda_stream)
    out = {}
    for kind, name in enumerate(MFMA_KINDS):
        best = None
        for groups in (256 * 4, 256 * 8, 256 * 16):
            sink = torch.empty(groups * 4, dtype=torch.float32, device="cuda")

            def launch():
                rc = L.moe_probe_mfma_peak(kind, groups, iters, C.c_void_p(sink.data_ptr()), sp)
                if rc != 0:
                    raise RuntimeError(f"moe_probe_mfma_peak: hipError {rc}")
            launch()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(launches):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            want = L.moe_probe_mfma_expected_sink(kind, iters)
            if not bool((sink == want).all()):
                raise RuntimeError(f"MFMA probe {name}: sums differ from {want}")
            us = e0.elapsed_time(e1) * 1e3 / launches
            tf = groups * 4 * L.moe_probe_mfma_flops_per_wave_iter(kind) * iters / (us * 1e-6) / 1e12
            if best is None or tf > best["TFLOPs"]:
                best = {"TFLOPs": round(tf, 1), "avg_launch_us": round(us, 1), "workgroups": groups,
                        "workgroups_per_cu": groups // 256}
        out[name] = best
    return out


def stream_read(torch, nbytes: int, copies: int, launches: int) -> dict:
    """The streaming-read kernel over one of `copies` distinct buffers of `nbytes` each, cycled
    (together larger than the 256 MB of on-die cache when copies > 1, so every launch reads
    HBM), HIP events on the launch stream.  Every variant (loads in flight per lane, cache
    policy) and grid (one round over the buffer, or 1, 2, 4 or 8 looping workgroups per CU) is
    timed; the fastest is the measured read rate at this size."""
    import ctypes as C
    L = probes()
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(copies)]
    sink = torch.empty(4 * (1 << 19), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = C.c_void_p(stream.cuda_stream)
    best = None
    for v in range(L.moe_probe_stream_read_variants()):
        for max_groups in (1 << 19, 256 * 8, 256 * 4, 256 * 2, 256):
            groups = int(L.moe_probe_stream_read_groups(nbytes, v, max_groups))

            def launch(i):
                rc = L.moe_probe_stream_read(C.c_void_p(bufs[i % copies].data_ptr()), nbytes, v, groups,
                                             C.c_void_p(sink.data_ptr()), sp)
                if rc != 0:
                    raise RuntimeError(f"moe_probe_stream_read: hipError {rc}")
            for i in range(2 * copies):
                launch(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(launches):
                launch(i)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / launches
            if best is None or us < best[0]:
                info = L.moe_probe_stream_read_variant_info(v)
                best = (us, {"loads_in_flight_per_lane": info & 255, "non_temporal": bool(info & 256),
                             "workgroups": groups})
    del bufs, sink
    torch.cuda.empty_cache()
    us, how = best
    return {"bytes_per_launch": nbytes, "copies_rotated": copies, "avg_launch_us": round(us, 2),
            "GBps": round(nbytes / us / 1e3, 1), "best_variant": how}


def power_sample(moe, torch):
    """Decode layer: each grouped GEMM launched back to back for ~5 s while `amd-smi metric`
    (a child process) samples socket power and clocks once, 2 s in."""
    import subprocess
    import synth
    L = synth.LAYER_DECODE
    W1, W2 = make_weights(L, moe, torch)
    logits = torch.from_numpy(synth.router_logits(L)).cuda()
    x = torch.from_numpy(synth.layer_activations(L).view(np.int16)).cuda().view(torch.bfloat16)
    plan = moe.MoELayerPlan(L.T, L.E, L.k, L.H, L.I, W1, W2)
    plan.forward(logits, x)
    torch.cuda.synchronize()
    out = {"workload": L.name}
    for tag, fn in (("gemm1", plan.gemm1), ("gemm2", plan.gemm2)):
        t0, n, proc = time.time(), 0, None
        while time.time() - t0 < 5:
            for _ in range(20):
                fn()
            n += 20
            if proc is None and time.time() - t0 > 2:
                proc = subprocess.Popen(["amd-smi", "metric", "-p", "-c", "-g", "0", "--json"],
                                        stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        torch.cuda.synchronize()
        rec = {"avg_launch_us": round((time.time() - t0) / n * 1e6, 1), "launches": n}
        try:
            rec["amd_smi"] = json.loads(proc.communicate(timeout=60)[0]) if proc else None
        except (ValueError, subprocess.TimeoutExpired, OSError) as err:
            rec["amd_smi"] = f"unavailable: {err}"
        out[tag] = rec
    print(json.dumps(out), flush=True)


def make_weights(L, moe, torch):
    """Seeded f32 weights per expert (host threads), uploaded and NVFP4-quantised on the GPU
    by the library's own quantiser, one dynamic global scale per expert matrix, then packed
    once into the layout the grouped GEMM streams (moe_pack_weights_nvfp4)."""
    import synth
    from concurrent.futures import ThreadPoolExecutor
    dev = torch.device("cuda")
    out = {}
    for name, rows, cols, fn in (("W1", 2 * L.I, L.H, synth.layer_w1), ("W2", L.H, L.I, synth.layer_w2)):
        q = torch.empty(L.E, rows, cols // 2, dtype=torch.uint8, device=dev)
        sf = torch.empty(L.E, rows, cols // 16, dtype=torch.uint8, device=dev)
        gs = torch.empty(L.E, dtype=torch.float32, device=dev)
        ws = torch.empty(max(moe.lib().moe_quantize_nvfp4_workspace(rows, cols), 16), dtype=torch.uint8, device=dev)
        staging = torch.empty(rows, cols, dtype=torch.float32, device=dev)
        with ThreadPoolExecutor(16) as ex:
            futs = [ex.submit(fn, L, e) for e in range(min(L.E, 32))]
            for e in range(L.E):
                w = futs[e].result()
                futs[e] = None
                if e + 32 < L.E:
                    futs.append(ex.submit(fn, L, e + 32))
                staging.copy_(torch.from_numpy(w))
                moe.moe_quantize_nvfp4(staging, q[e], sf[e], gs[e:e + 1], moe.MOE_GS_DYNAMIC, None, ws)
        torch.cuda.synchronize()
        packed = moe.pack_weights(moe.NVFP4Tensor(q, sf, gs))   # one-time layout preparation
        torch.cuda.synchronize()
        del q, sf, staging
        out[name] = packed
    return out["W1"], out["W2"]


def grouped_gemm_decode(moe, torch, steps: int, copies: int = 8, with_stream_read: bool = True) -> dict:
    """The single grouped GEMM at decode shape (8 groups x 32 rows, K 6144, N 2048, NONE
    epilogue) on packed weights.  `copies` distinct weight copies (8 x 56.6 MB, more than
    the 256 MB Infinity Cache) are cycled so that every launch streams its weights from HBM."""
    import synth
    G = synth.GEMM_DECODE
    dev = torch.device("cuda")
    wq = torch.empty(G.E, G.N, G.K // 2, dtype=torch.uint8, device=dev)
    wsf = torch.empty(G.E, G.N, G.K // 16, dtype=torch.uint8, device=dev)
    wgs = torch.empty(G.E, dtype=torch.float32, device=dev)
    for e in range(G.E):
        w = torch.from_numpy(synth.gemm_b(G, e)).to(dev)
        moe.moe_quantize_nvfp4(w, wq[e], wsf[e], wgs[e:e + 1], moe.MOE_GS_DYNAMIC)
    packed = moe.pack_weights(moe.NVFP4Tensor(wq, wsf, wgs))
    Ws = [packed] + [moe.PackedWeights(packed.data.clone(), wgs, G.N, G.K) for _ in range(copies - 1)]
    a_bits = torch.from_numpy(synth.gemm_a_bf16(G).view(np.int16)).to(dev).view(torch.bfloat16)
    A = moe.quantize_alloc(a_bits)
    off = torch.arange(0, (G.E + 1) * G.M, G.M, dtype=torch.int32, device=dev)
    R = G.E * G.M
    D = torch.empty(R, G.N, dtype=torch.bfloat16, device=dev)
    args = [moe._gemm_args_for(A, W, off, R, moe.MOE_EPI_NONE, D, None) for W in Ws]
    ws = moe._ws(moe.moe_grouped_gemm_nvfp4_workspace(args[0]), dev)
    for _ in range(2):   # warm-up: every copy twice (16 launches)
        for a in args:
            moe.moe_grouped_gemm_nvfp4(a, ws)
    torch.cuda.synchronize()
    n = max(steps, 13) * copies   # at least 100 timed launches
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        moe.moe_grouped_gemm_nvfp4(args[i % copies], ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    w_bytes = G.E * G.N * (G.K // 2 + G.K // 16)
    alg = w_bytes + R * (G.K // 2 + G.K // 16) + R * G.N * 2
    flops = 2.0 * R * G.N * G.K
    del Ws, args, packed, A, D, ws
    torch.cuda.empty_cache()
    # the streaming-read kernel over exactly as many bytes per launch, cycled over as many
    # copies: the read rate this working-set size reaches, launch start and drain included
    rec = {"workload": G.name, "avg_launch_us": round(us, 2), "tflops": round(flops / us / 1e6, 2),
            "alg_bytes_per_launch": alg, "GBps": round(alg / us / 1e3, 1),
            "hbm_frac": round(alg / us / 1e3 / HBM_PEAK_GBPS, 4), "weight_copies_rotated": copies}
    if with_stream_read:
        sr = stream_read(torch, (alg + 15) // 16 * 16, copies, n)
        rec["stream_read_same_bytes"] = sr
        rec["frac_of_stream_read_same_bytes"] = round(sr["avg_launch_us"] / us, 4)
    return rec


def dense_gemm(moe, torch, launches: int = 20) -> dict:
    """The dense special case (one group, 8192^3, NONE epilogue) on packed weights."""
    import synth
    G = synth.GEMM_DENSE
    dev = torch.device("cuda")
    w = torch.from_numpy(synth.gemm_b(G, 0)).to(dev)
    wq = torch.empty(1, G.N, G.K // 2, dtype=torch.uint8, device=dev)
    wsf = torch.empty(1, G.N, G.K // 16, dtype=torch.uint8, device=dev)
    wgs = torch.empty(1, dtype=torch.float32, device=dev)
    moe.moe_quantize_nvfp4(w, wq[0], wsf[0], wgs, moe.MOE_GS_DYNAMIC)
    del w
    W = moe.pack_weights(moe.NVFP4Tensor(wq, wsf, wgs))
    del wq, wsf
    a_bits = torch.from_numpy(synth.gemm_a_bf16(G).view(np.int16)).to(dev).view(torch.bfloat16)
    A = moe.quantize_alloc(a_bits)
    del a_bits
    off = torch.tensor([0, G.M], dtype=torch.int32, device=dev)
    D = torch.empty(G.M, G.N, dtype=torch.bfloat16, device=dev)
    args = moe._gemm_args_for(A, W, off, G.M, moe.MOE_EPI_NONE, D, None)
    ws = moe._ws(moe.moe_grouped_gemm_nvfp4_workspace(args), dev)
    for _ in range(3):
        moe.moe_grouped_gemm_nvfp4(args, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        moe.moe_grouped_gemm_nvfp4(args, ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    flops = 2.0 * G.M * G.N * G.K
    del A, W, D, args, ws
    torch.cuda.empty_cache()
    ref_tflops = torch_f16_matmul_tflops(torch, G.M, launches)
    return {"workload": G.name, "avg_launch_us": round(us, 1), "tflops": round(flops / us / 1e6, 1),
            "frac_of_f16_dense_peak": round(flops / us / 1e6 / F16_PEAK_TFLOPS, 4),
            "torch_f16_matmul_tflops": round(ref_tflops, 1),
            "frac_of_torch_f16_matmul": round(flops / us / 1e6 / ref_tflops, 4)}


def torch_f16_matmul_tflops(torch, n: int = 8192, launches: int = 20) -> float:
    """The library fp16 GEMM (torch.matmul on fp16 operands) at n^3: the f16 MFMA rate a tuned
    dense kernel reaches on this machine, a measured companion to the 2.5 PFLOP/s spec peak."""
    dev = torch.device("cuda")
    a = torch.randn(n, n, dtype=torch.float16, device=dev)
    b = torch.randn(n, n, dtype=torch.float16, device=dev)
    for _ in range(3):
        c = torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        c = torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    del a, b, c
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / us / 1e6


def cpu_baseline(L, offsets, row_src, seconds):
    """The oracle's grouped GEMMs (gate/up then down) over the routed rows of the first
    experts, one expert at a time until `seconds` of CPU time is spent; FLOPs / time."""
    import oracle
    import synth
    logits_x = synth.layer_activations(L)
    xq = oracle.quantize_bf16(logits_x)
    flops, spent, experts, rows_done = 0.0, 0.0, 0, 0
    rng = np.random.default_rng(0)
    for e in range(L.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w1 = oracle.quantize(synth.layer_w1(L, e))
        w2 = oracle.quantize(synth.layer_w2(L, e))
        off1 = np.array([0, hi - lo], np.int32)
        act_bits = synth.bf16_bits(rng.standard_normal((hi - lo, L.I)).astype(np.float32))
        aq = oracle.quantize_bf16(act_bits)
        t0 = time.perf_counter()
        oracle.grouped_gemm(xq, w1.q[None], w1.sf[None], np.array([w1.g], np.float32), off1,
                            A_rows=row_src[lo:hi])
        oracle.grouped_gemm(aq, w2.q[None], w2.sf[None], np.array([w2.g], np.float32), off1)
        spent += time.perf_counter() - t0
        flops += 2.0 * (hi - lo) * (2 * L.I * L.H + L.H * L.I)
        experts += 1
        rows_done += hi - lo
        if spent >= seconds:
            break
    rec = {"value": flops / spent / 1e12, "unit": "TFLOPS", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"oracle grouped GEMMs (gate/up {2 * L.I}x{L.H} then down {L.H}x{L.I}) over the "
                     f"{rows_done} routed rows of the first {experts} experts of the same workload, "
                     f"{spent:.1f} s of CPU time"}
    # the same GEMMs on one thread, over the first few experts (about a quarter of the time)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        f1, s1, n1, e = 0.0, 0.0, 0, 0
        while s1 < seconds / 4 and e < L.E:
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            e += 1
            if hi == lo:
                continue
            w1 = oracle.quantize(synth.layer_w1(L, e - 1))
            t0 = time.perf_counter()
            oracle.grouped_gemm(xq, w1.q[None], w1.sf[None], np.array([w1.g], np.float32),
                                np.array([0, hi - lo], np.int32), A_rows=row_src[lo:hi])
            s1 += time.perf_counter() - t0
            f1 += 2.0 * (hi - lo) * 2 * L.I * L.H
            n1 += hi - lo
    finally:
        oracle.set_num_threads(threads)
    rec["single_thread"] = {"value": f1 / s1 / 1e12, "unit": "TFLOPS",
                            "sample": f"oracle gate/up GEMMs over {n1} routed rows, {s1:.1f} s on one thread"}
    rec["host"] = {"cpu": host_cpu_model(), "nproc": os.cpu_count()}
    return rec


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_layer(L, moe, torch, steps: int, warmup: int, weights=None, fused: bool = False) -> dict:
    """Time `steps` full layer steps (after `warmup`) with HIP events around every stage on
    the launch stream; returns the stage times and the derived GEMM figures.  fused: requantise
    the SwiGLU output in the gate/up GEMM's epilogue with a static global scale, calibrated
    as a caller would, from one dynamic pass."""
    import synth
    dev = torch.device("cuda")
    t_setup = time.time()
    W1, W2 = weights if weights is not None else make_weights(L, moe, torch)
    logits = torch.from_numpy(synth.router_logits(L)).to(dev)
    x = torch.from_numpy(synth.layer_activations(L).view(np.int16)).to(dev).view(torch.bfloat16)
    plan = moe.MoELayerPlan(L.T, L.E, L.k, L.H, L.I, W1, W2)
    if fused:
        plan.forward(logits, x)
        g2 = plan.actq.gs.clone()
        plan = moe.MoELayerPlan(L.T, L.E, L.k, L.H, L.I, W1, W2, static_g2=g2)
    torch.cuda.synchronize()
    print(f"# {L.name}: setup {time.time() - t_setup:.1f}s", file=sys.stderr, flush=True)

    stages = ["route", "quantize_input", "gemm1", "requantize", "gemm2", "finalize"]
    calls = [lambda: plan.route(logits), lambda: plan.quantize_input(x), plan.gemm1, plan.requantize,
             plan.gemm2, plan.finalize]
    for _ in range(warmup):
        plan.forward(logits, x)
    torch.cuda.synchronize()

    # stage breakdown: the six calls one after another on one stream, events between them
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        evs[s][0].record(stream)
        for i, c in enumerate(calls):
            c()
            evs[s][i + 1].record(stream)
    torch.cuda.synchronize()
    stage_us = {st: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)]) * 1e3)
                for i, st in enumerate(stages)}
    # the timed steps: whole forward passes on one stream, bracketed by device synchronisation
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        plan.forward(logits, x)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    # the same steps replayed from a HIP graph of one forward pass (no host launch work)
    g = plan.graph(logits, x)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        g.replay()
    torch.cuda.synchronize()
    graph_ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    del g

    off = plan.off.cpu().numpy()
    sizes = np.diff(off)
    active = int((sizes > 0).sum())
    R = int(off[-1])
    gemm1_flops = 2.0 * R * (2 * L.I) * L.H
    gemm2_flops = 2.0 * R * L.H * L.I
    w1_bytes = active * (2 * L.I) * (L.H // 2 + L.H // 16)
    w2_bytes = active * L.H * (L.I // 2 + L.I // 16)
    x_bytes = L.T * (L.H // 2 + L.H // 16)
    act_bytes = R * L.I * 2
    g1_alg_bytes = w1_bytes + x_bytes + act_bytes
    # the down GEMM reads the requantised act and writes one bf16 row of H per routed row
    # (at a small I, e.g. a tensor-parallel share, these writes are a large part of its bytes)
    g2_alg_bytes = w2_bytes + R * (L.I // 2 + L.I // 16) + R * L.H * 2
    g1_s = stage_us["gemm1"] * 1e-6
    g2_s = stage_us["gemm2"] * 1e-6
    weight_gbps = (w1_bytes + w2_bytes) / (g1_s + g2_s) / 1e9
    gemm_alg_gbps = (g1_alg_bytes + g2_alg_bytes) / (g1_s + g2_s) / 1e9
    return {"plan": plan, "weights": (W1, W2), "off": off, "sizes": sizes, "ms_per_step": ms_per_step,
            "graph_ms_per_step": graph_ms_per_step, "stage_us": stage_us,
            "value": (gemm1_flops + gemm2_flops) / (ms_per_step * 1e-3) / 1e12,
            "gemm_tflops": (gemm1_flops + gemm2_flops) / (g1_s + g2_s) / 1e12,
            "weight_gbps": weight_gbps, "gemm_alg_gbps": gemm_alg_gbps, "g1_alg_bytes": g1_alg_bytes,
            "g2_alg_bytes": g2_alg_bytes, "g1_s": g1_s, "g1_flops": gemm1_flops}


def roofline_record(L, r) -> dict:
    """Roofline of the dominant kernel, the gate/up grouped GEMM: at tens of rows per expert
    the four-wave kernel streams weights (HBM-bound); at >= 96 rows per expert (and 2I a
    multiple of 512, the library's own rule) the 8-wave kernel is MFMA-bound, against the fp16
    dense peak -- exact E2M1 x E4M3 products are formed in fp16, so that is the contraction's
    own dtype (the FP4 peak fraction is given beside it for context)."""
    import synth
    g1_s = r["g1_s"]
    if (L.T * L.k) / L.E >= 96 and (2 * L.I) % 512 == 0:
        tf = r["g1_flops"] / g1_s / 1e12
        return {"kernel": "gemm_lds_wide_kernel<1> (gate/up + SwiGLU)", "bound": "mfma",
                "achieved": round(tf, 1), "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / F16_PEAK_TFLOPS, 4), "traffic": None,
                "flops_per_launch": int(r["g1_flops"]), "avg_launch_us": round(g1_s * 1e6, 2),
                "peak_dtype": "f16 (the exact E2M1 x E4M3 products are formed in fp16)",
                "frac_of_fp4_dense_peak": round(tf / FP4_PEAK_TFLOPS, 4)}
    return {"kernel": "gemm_lds_kernel<1> (gate/up + SwiGLU)", "bound": "hbm",
            "achieved": round(r["g1_alg_bytes"] / g1_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(r["g1_alg_bytes"] / g1_s / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic("moe::gemm::gemm_lds_kernel<1>") if L is synth.LAYER_DECODE else None,
            "alg_bytes_per_launch": int(r["g1_alg_bytes"]), "avg_launch_us": round(g1_s * 1e6, 2)}


def shard_record(L, moe, torch, steps: int, weights=None) -> dict:
    """A further layer configuration on the full path (one GPU's share of the decode layer
    under expert or tensor parallelism, or the skewed decode layer); `weights` reuses packed
    weights of the same shape."""
    r = run_layer(L, moe, torch, steps, 2, weights=weights)
    out = {"workload": L.name, "ms_per_step": round(r["ms_per_step"], 4),
           "graph_ms_per_step": round(r["graph_ms_per_step"], 4), "tflops": round(r["value"], 2),
           "gemm_tflops": round(r["gemm_tflops"], 2), "weight_hbm_GBps": round(r["weight_gbps"], 1),
           "weight_hbm_frac": round(r["weight_gbps"] / HBM_PEAK_GBPS, 4),
           "gemm_alg_hbm_GBps": round(r["gemm_alg_gbps"], 1),
           "gemm_alg_hbm_frac": round(r["gemm_alg_gbps"] / HBM_PEAK_GBPS, 4),
           "stage_us": {k: round(v, 2) for k, v in r["stage_us"].items()},
           "offsets": [int(v) for v in r["off"]]}
    del r
    torch.cuda.empty_cache()
    return out


def prefill_record(L, moe, torch, steps: int, weights) -> dict:
    """The prefill layer on the full path, with the roofline of its two GEMMs against the
    fp16 dense MFMA peak (and the FP4 peak beside it)."""
    r = run_layer(L, moe, torch, steps, 2, weights=weights)
    g1_s, g2_s = r["stage_us"]["gemm1"] * 1e-6, r["stage_us"]["gemm2"] * 1e-6
    g2_flops = 2.0 * int(r["off"][-1]) * L.H * L.I
    tf1, tf2 = r["g1_flops"] / g1_s / 1e12, g2_flops / g2_s / 1e12
    sizes = r["sizes"]
    out = {"workload": L.name, "steps": steps, "ms_per_step": round(r["ms_per_step"], 4),
           "graph_ms_per_step": round(r["graph_ms_per_step"], 4),
           "tflops": round(r["value"], 2), "gemm_tflops": round(r["gemm_tflops"], 2),
           "rows_per_expert_min_median_max": [int(sizes.min()), int(np.median(sizes)), int(sizes.max())],
           "stage_us": {k: round(v, 2) for k, v in r["stage_us"].items()},
           "roofline": roofline_record(L, r),
           "gemm2": {"kernel": "gemm_lds_wide_kernel<0> (down, NONE)", "achieved": round(tf2, 1),
                     "unit": "TFLOP/s", "frac": round(tf2 / F16_PEAK_TFLOPS, 4),
                     "frac_of_fp4_dense_peak": round(tf2 / FP4_PEAK_TFLOPS, 4)},
           "gemms_frac_of_f16_dense_peak": round(r["gemm_tflops"] / F16_PEAK_TFLOPS, 4),
           "gemms_frac_of_fp4_dense_peak": round(r["gemm_tflops"] / FP4_PEAK_TFLOPS, 4)}
    del r
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.power_sample:
        import torch

        import block_scaled_fp4_02_amd as moe
        torch.cuda.set_device(0)
        power_sample(moe, torch)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_scaled_fp4_02_amd as moe
    import synth
    L = getattr(synth, WORKLOADS[args.workload])
    torch.cuda.set_device(0)
    if args.workload == "gemm_e8_m32":
        # the single grouped GEMM alone (8 groups x 32 rows, K 6144, N 2048, NONE epilogue)
        print(json.dumps(grouped_gemm_decode(moe, torch, args.steps, with_stream_read=not args.no_extras)), flush=True)
        return
    r = run_layer(L, moe, torch, args.steps, args.warmup)
    sizes, g1_s = r["sizes"], r["g1_s"]
    rec = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": L.name, "tokens": L.T, "experts": L.E, "top_k": L.k, "hidden": L.H,
                   "intermediate": L.I, "rows_per_expert_min_median_max": [int(sizes.min()), int(np.median(sizes)),
                                                                           int(sizes.max())],
                   "operands": "NVFP4 (e2m1, e4m3 scale per 16, f32 global) dequantised exactly to fp16 MFMA, fp32 accumulate",
                   "weights_layout": "packed"},
        "roofline": roofline_record(L, r),
        "graph_ms_per_step": round(r["graph_ms_per_step"], 4),
        "gemm_tflops": round(r["gemm_tflops"], 2),
        "weight_hbm_GBps": round(r["weight_gbps"], 1),
        "weight_hbm_frac": round(r["weight_gbps"] / HBM_PEAK_GBPS, 4),
        "gemm_alg_hbm_GBps": round(r["gemm_alg_gbps"], 1),
        "gemm_alg_hbm_frac": round(r["gemm_alg_gbps"] / HBM_PEAK_GBPS, 4),
        "stage_us": {k: round(v, 2) for k, v in r["stage_us"].items()},
    }
    off, row_src = r["off"], r["plan"].row_src.cpu().numpy()
    extras = not args.no_extras
    if L is synth.LAYER_DECODE and extras:
        f = run_layer(L, moe, torch, args.steps, args.warmup, weights=r["weights"], fused=True)
        rec["layer_decode_fused_static_g2"] = {
            "ms_per_step": round(f["ms_per_step"], 4), "graph_ms_per_step": round(f["graph_ms_per_step"], 4),
            "tflops": round(f["value"], 2),
            "stage_us": {k: round(v, 2) for k, v in f["stage_us"].items()},
            "note": "SwiGLU output requantised in the gate/up GEMM epilogue (MOE_EPI_SWIGLU_NVFP4) with a "
                    "static global scale calibrated from one dynamic pass; requantize stage is empty"}
        del f
        # skewed decode (512 tokens, Zipf-biased router: 0-200+ rows per expert, some empty), the
        # same expert weights; its weight rate counts active experts only
        sk = shard_record(synth.LAYER_SKEWED, moe, torch, args.steps, weights=r["weights"])
        sizes_sk = np.diff(np.asarray(sk.pop("offsets")))
        sk["rows_per_expert_min_median_max"] = [int(sizes_sk.min()), int(np.median(sizes_sk)), int(sizes_sk.max())]
        sk["active_experts"] = int((sizes_sk > 0).sum())
        rec["layer_skewed"] = sk
        # prefill (16384 tokens, ~512 rows per expert): the MFMA-bound configuration, on the
        # same expert weights (same expert count, hidden and intermediate sizes)
        rec["layer_prefill"] = prefill_record(synth.LAYER_PREFILL, moe, torch, min(args.steps, 10), r["weights"])
    del r
    torch.cuda.empty_cache()
    if extras and rec["roofline"]["bound"] == "hbm":
        # measured companion to the spec peak: the streaming-read kernel over 1 GiB buffers
        sr = stream_read(torch, 1 << 30, 2, 20)
        rec["roofline"]["measured_stream_read_GBps"] = sr["GBps"]
        rec["roofline"]["frac_of_measured_stream_read"] = round(rec["roofline"]["achieved"] / sr["GBps"], 4)
    elif extras:
        mm = torch_f16_matmul_tflops(torch)
        rec["roofline"]["measured_f16_matmul_TFLOPs"] = round(mm, 1)
        rec["roofline"]["frac_of_measured_f16_matmul"] = round(rec["roofline"]["achieved"] / mm, 4)
        mp = mfma_peak(torch)
        rec["measured_mfma_peak"] = mp
        rec["roofline"]["measured_f16_mfma_TFLOPs"] = mp["f16_16x16x32"]["TFLOPs"]
        rec["roofline"]["frac_of_measured_f16_mfma"] = round(
            rec["roofline"]["achieved"] / mp["f16_16x16x32"]["TFLOPs"], 4)
    if L is synth.LAYER_DECODE and extras:
        rec["grouped_gemm_decode_8x32"] = grouped_gemm_decode(moe, torch, args.steps)
        rec["dense_gemm_8192"] = dense_gemm(moe, torch)
        # measured companions to the spec MFMA peaks, for the MFMA-bound records above
        mp = mfma_peak(torch)
        rec["measured_mfma_peak"] = mp
        f16 = mp["f16_16x16x32"]["TFLOPs"]
        pr = rec["layer_prefill"]["roofline"]
        pr["measured_f16_mfma_TFLOPs"] = f16
        pr["frac_of_measured_f16_mfma"] = round(pr["achieved"] / f16, 4)
        pr["frac_of_measured_fp4_mfma"] = round(pr["achieved"] / mp["fp4_16x16x128"]["TFLOPs"], 4)
        dg = rec["dense_gemm_8192"]
        dg["frac_of_measured_f16_mfma"] = round(dg["tflops"] / f16, 4)
        for key, Ls in (("shard_ep8", synth.LAYER_EP8), ("shard_tp8", synth.LAYER_TP8)):
            rec[key] = shard_record(Ls, moe, torch, args.steps)
            del rec[key]["offsets"]
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(L, off, row_src, args.cpu_baseline_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
