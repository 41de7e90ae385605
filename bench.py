#!/usr/bin/env python3
"""Benchmark of the chunked gated-delta-rule forward on one MI355X.

Workload: the long-context configuration B=1, T=65536, Hq=4, Hv=8, K=V=128,
bf16 q/k/v with fp32 g/beta, 64-token chunks, no initial state, automatic
context-parallel split.  One step = one full forward pass (plan, intra-chunk
WY, serial state, output) through the C ABI on resident device buffers.

Prints ONE JSON line: tokens/s and ms per step (K steps between device
syncs, nothing else in the timed region, after about 0.25 s of untimed
steps and the W warmup steps so that the GPU clocks have settled; with --graph the step is also captured once in a HIP
graph, checked bitwise against an eager step and replayed, and the replay
rate is the value), the same step timed one call at a time after a 1 GiB
cache flush ("flushed"), the roofline of the dominant kernel (its mean
HIP-event duration on the launch stream over K more steps, against the
method's algorithmic bytes and flops for the workload: q, k, v, g, beta in,
o and the final state out, and the chunk GEMMs) as HBM and MFMA fractions of
the published peaks and of peaks measured in the same run by a copy kernel
and an MFMA loop, and the fp64 CPU oracle's throughput on the host.
The line also carries "configs_report": the other parity configurations (tiny
fp32, edge prefill, varlen forward and the backward), each timed per call
with a cache flush between calls and set against the method's roofline
(essential I/O and chunk-GEMM flops per token x value head); and
"train_step_sweep": training-step (forward + backward) and backward latency
against tokens per update step for value-head counts 64, 48, 32, 24, 16, 8
(the head configurations the pages benchmark the backward on).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_long_context.json")
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16 MFMA
MFMA_F32_PEAK_TFS = 157.3      # dense fp32 MFMA
METRIC = "GDN chunked-prefill fwd tokens/s (B=1,T=64K,Hv=8) + % MFMA/HBM roofline"


def per_kernel_work(w, G):
    """Algorithmic bytes and flops per token x value head for each kernel of
    the forward (each input read once, each output written once; bf16 = 2 B).
    Returns {kernel: (bytes, flops)} per token*value-head."""
    K, V, C, e = w.K, w.V, 64, 2
    return {
        # k, g, beta in; A diag(beta) rows (compact: the 10 lower 16 x 16
        # blocks, 80 of 128 bytes per row on average) and g_cum out; K K^T and the inverse
        "intra_wy": (K * e / G + 8 + C * e * 5 / 8 + 4,
                     2 * C * K + C * C // 3),
        # A diag(beta) (compact), v, k, q, g_cum in; o out (states and Vnew
        # stay on chip); K h, A''(V - Gamma K h), K^T Vnew, Q h, Q K^T, P Vnew
        "chunk_fused": (C * e * 5 / 8 + V * e + 2 * K * e / G + 4 + V * e,
                        4 * K * V + 2 * K * V + 2 * C * K + 4 * C * V),
    }


def sources_sha256() -> str:
    """Hash of the kernel sources; counter-derived traffic is valid only for it."""
    import hashlib
    d = os.path.join(ROOT, "gated_deltanet_chunked_rule_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h", ".cpp")) and name != "gdr_peaks.hip":
            h.update(name.encode())
            h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, each scaled by what
    the counter reads for a device copy of known size), or None when the
    summary is missing or was taken on different kernel sources."""
    import json
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256() or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return 1024.0 * (k["fetch_kib"] * rec["fetch_scale"] + k["write_kib"] * rec["write_scale"])


def method_work(K, V, G, esize, backward):
    """The method's flops and essential bytes per token x value head (64-token
    chunks): forward 6KV + 6CK + 4CV + C^2/3 flops and q, k (shared by the G
    value heads), v, o, g, beta bytes; backward 16KV + 18CK + 10CV + C^2 flops
    and q, k, v, do, dq, dk, dv, g, beta, dg, dbeta bytes."""
    C = 64
    if backward:
        return (16 * K * V + 18 * C * K + 10 * C * V + C * C,
                4 * K * esize / G + 3 * V * esize + 16)
    return (6 * K * V + 6 * C * K + 4 * C * V + C * C / 3,
            2 * K * esize / G + 2 * V * esize + 8)


def config_report(torch, gdr, gi, dev):
    """Per-call time of the other parity configurations against the method's
    roofline; a 1 GiB buffer is rewritten between calls so that no input is
    served from the last-level cache."""
    flush = torch.empty(1 << 28, device=dev, dtype=torch.float32)
    out = {}
    for name, backward, iters in (("tiny_fp32", False, 50), ("edge_prefill", False, 50),
                                  ("varlen", False, 50), ("backward", True, 50)):
        w = gi.WORKLOADS[name]
        inp = gi.make_inputs(w)
        d = {n: (x.to(dev) if hasattr(x, "to") and n != "cu_seqlens" else x) for n, x in inp.items()}
        cu = inp.get("cu_seqlens")
        h0 = d.get("initial_state")
        if backward:
            args = (d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["do"], d["dht"], d["scale"], h0, cu)
            call = lambda: gdr.gdr_chunk_bwd(*args)
        else:
            call = lambda: gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], h0, cu)
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        times = []
        for _ in range(iters):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        gdr.timing.reset()   # per-kernel durations from a second pass (events off the timed calls)
        gdr.timing.enable(True)
        for _ in range(iters):
            flush.zero_()
            call()
        torch.cuda.synchronize()
        gdr.timing.enable(False)
        kern = gdr.timing.collect()
        ms = sorted(times)[len(times) // 2]
        tokens = w.B * w.T
        tv = tokens * w.Hv
        esize = 4 if w.dtype == "f32" else 2
        flops_tv, bytes_tv = method_work(w.K, w.V, w.Hv // w.Hq, esize, backward)
        state_bytes = 0
        nseq = len(cu) - 1 if cu is not None else w.B
        if h0 is not None:
            state_bytes += nseq * w.Hv * w.K * w.V * 4
        state_bytes += nseq * w.Hv * w.K * w.V * 4 * (2 if backward else 1)  # final_state / dht, dh0
        flops, nbytes = flops_tv * tv, bytes_tv * tv + state_bytes
        peak = MFMA_F32_PEAK_TFS if w.dtype == "f32" else MFMA_BF16_PEAK_TFS
        t_mfma, t_hbm = flops / (peak * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)
        t_roof = max(t_mfma, t_hbm)
        t = ms * 1e-3
        out[name] = {
            "pass": "bwd" if backward else "fwd", "tokens": tokens, "ms": round(ms, 4),
            "tokens_per_s": round(tokens / t),
            "roof": {"bound": "mfma" if t_mfma > t_hbm else "hbm", "t_roof_us": round(t_roof * 1e6, 2),
                     "frac": round(t_roof / t, 4), "mfma_frac": round(t_mfma / t, 4),
                     "hbm_frac": round(t_hbm / t, 4), "mfma_peak_tfs": peak,
                     "gflop": round(flops / 1e9, 3), "mbytes": round(nbytes / 1e6, 2)},
            "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in kern.items()},
        }
        del d, inp
        torch.cuda.empty_cache()
    return out


SWEEP_HV = (64, 48, 32, 24, 16, 8)          # value heads per GPU (TP1 .. TP8 shares)
SWEEP_TOKENS = (8192, 16384, 32768, 65536)   # tokens per update step, as 8192-token sequences


def train_step_sweep(torch, gdr, dev):
    """Training-step latency against tokens per update step for each value-head
    count: one forward + backward through the autograd wrapper (the backward
    recomputes A), and the backward entry point alone (given the forward's A).  Hq = Hv/2,
    K = V = 128, bf16; inputs drawn on the device (q, k L2-normalised N(0,1),
    v and do N(0,1), g = log U(0.85, 1), beta = sigmoid(N(0,1)), no initial
    state), median of 5 calls with a cache flush before each."""
    flush = torch.empty(1 << 28, device=dev, dtype=torch.float32)
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    K = V = 128
    rows = []
    for hv in SWEEP_HV:
        hq = hv // 2
        for tokens in SWEEP_TOKENS:
            B, T = tokens // 8192, 8192
            nrm = lambda x: x / x.norm(dim=-1, keepdim=True)
            q = nrm(torch.randn(B, T, hq, K, device=dev, generator=gen)).to(torch.bfloat16)
            k = nrm(torch.randn(B, T, hq, K, device=dev, generator=gen)).to(torch.bfloat16)
            v = torch.randn(B, T, hv, V, device=dev, generator=gen).to(torch.bfloat16)
            do = torch.randn(B, T, hv, V, device=dev, generator=gen).to(torch.bfloat16)
            g = torch.log(0.85 + 0.15 * torch.rand(B, T, hv, device=dev, generator=gen))
            beta = torch.sigmoid(torch.randn(B, T, hv, device=dev, generator=gen))
            scale = K ** -0.5
            leaves = [x.detach().requires_grad_(True) for x in (q, k, v, g, beta)]

            def step():
                o, _ = gdr.chunk_gated_delta_rule(*leaves, scale)
                return torch.autograd.grad(o, leaves, do)

            _, _, _, A = gdr.gdr_chunk_fwd(q, k, v, g, beta, scale, output_A=True)
            bwd = lambda: gdr.gdr_chunk_bwd(q, k, v, g, beta, A, do, None, scale, None, None)

            def timed(fn, iters=5):
                for _ in range(2):
                    fn()
                torch.cuda.synchronize()
                ts = []
                for _ in range(iters):
                    flush.zero_()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fn()
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1))
                return sorted(ts)[len(ts) // 2]

            ms_step, ms_bwd = timed(step), timed(bwd)
            tv = tokens * hv
            ff, fb = method_work(K, V, 2, 2, False)
            bf, bb = method_work(K, V, 2, 2, True)
            roof = lambda fl, by: max(fl * tv / (MFMA_BF16_PEAK_TFS * 1e12), by * tv / (HBM_PEAK_GBS * 1e9))
            rows.append({"hv": hv, "hq": hq, "tokens": tokens, "ms_step": round(ms_step, 3),
                         "ms_bwd": round(ms_bwd, 3),
                         "step_tokens_per_s": round(tokens / (ms_step * 1e-3)),
                         "step_roof_frac": round(roof(ff + bf, fb + bb) / (ms_step * 1e-3), 4),
                         "bwd_roof_frac": round(roof(bf, bb) / (ms_bwd * 1e-3), 4)})
            del q, k, v, do, g, beta, leaves, A
            torch.cuda.empty_cache()
    return rows


def measure_peaks(torch, dev):
    """Peaks measured on this device by the probes of libgdr_peaks.so: a 1 GiB
    device copy (2 GiB of HBM traffic per kernel, non-temporal 16-byte
    accesses) and loops of independent bf16 MFMA instructions over 2048
    workgroups (8 waves per SIMD), in the 32x32x16 form (the one that reaches
    the published rate) and the 16x16x32 form (about half of it on gfx950)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_deltanet_chunked_rule_amd", "libgdr_peaks.so"))
    lib.gdr_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    lib.gdr_peak_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    nbytes = 1 << 30
    src = torch.empty(nbytes, device=dev, dtype=torch.uint8).fill_(1)
    dst = torch.empty_like(src)
    ms = ctypes.c_float()
    if lib.gdr_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, 10, st,
                         ctypes.byref(ms)) != 0:
        raise RuntimeError("copy probe failed")
    copy_gbs = 2 * nbytes / (ms.value * 1e-3) / 1e9
    del src, dst
    wgs, iters = 2048, 20000
    sink = torch.empty(wgs * 256, device=dev, dtype=torch.float32)
    tfs = {}
    for tile in (32, 16):
        if lib.gdr_peak_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), tile, iters, wgs, 5, st, ctypes.byref(ms)) != 0:
            raise RuntimeError("MFMA probe failed")
        tfs[tile] = wgs * 4 * iters * 131072 / (ms.value * 1e-3) / 1e12
    return {"hbm_copy_GBs": round(copy_gbs, 1), "mfma_bf16_TFs": round(tfs[32], 1),
            "mfma_bf16_16x16x32_TFs": round(tfs[16], 1),
            "how": "1 GiB device copy, non-temporal 16-byte accesses (read + write bytes); bf16 MFMA loops, "
                   "2048 workgroups x 4 waves, independent chains (32x32x16 and 16x16x32 forms)"}


def host_cpu():
    """CPU model and core count of the host the oracle ran on."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults long enough for the GPU clocks to reach their sustained state
    # (a 20-step window right after a cold start reads ~20 % slow); the timed
    # work is still well under a second
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration report")
    ap.add_argument("--no-sweep", action="store_true", help="skip the training-step sweep")
    ap.add_argument("--settle-s", type=float, default=0.25,
                    help="untimed steps for this many seconds before the warmup steps (GPU clocks)")
    ap.add_argument("--precise-vnew", action="store_true",
                    help="time the forward with the precise_vnew option (Vnew as two bf16 terms; the default "
                         "value is measured without it)")
    ap.add_argument("--graph", action="store_true",
                    help="also time a HIP-graph replay of the step and report it as the value (default: eager launches)")
    ap.add_argument("--flushed-steps", type=int, default=50,
                    help="steps timed one at a time after a 1 GiB cache flush")
    ap.add_argument("--no-peaks", action="store_true", help="skip the copy and MFMA peak probes")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (--gpus {args.gpus} requested); "
              "its kernels cover one GPU's share and it has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_chunked_rule_amd as gdr
    import gdr_inputs as gi

    w = gi.WORKLOADS["long_context"]
    inp = gi.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    g, beta = inp["g"].to(dev), inp["beta"].to(dev)
    scale = inp["scale"]
    G = w.Hv // w.Hq
    plan = gdr.gdr_chunk_fwd_plan(q, v)
    # workspace allocated once, outside the timed region
    ws = torch.empty(gdr.fwd_workspace_bytes(q, v), device=dev, dtype=torch.uint8)

    opts = gdr.Options(precise_vnew=1) if args.precise_vnew else None

    def step():
        return gdr.gdr_chunk_fwd(q, k, v, g, beta, scale, workspace=ws, options=opts)

    # untimed clock settle (about 0.25 s of steps) before the W warmup steps:
    # right after a cold start every kernel runs ~20 % slow until the GPU
    # clocks reach their sustained state
    settle0 = time.perf_counter()
    while time.perf_counter() - settle0 < args.settle_s:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # eager launches: each step enqueues its kernels from the host
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eager_ms = (t1 - t0) * 1e3 / args.steps
    o_ref, ht_ref, _, _ = step()
    graph_ms = None
    if args.graph:
        # the same step captured once in a HIP graph and replayed (fixed shapes
        # and buffers, as in a serving loop): no host launch gaps between the
        # kernels.  Every replay recomputes the whole forward; its output is
        # checked bitwise against the eager step.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            o_g, ht_g, _, _ = step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(o_g, o_ref) and torch.equal(ht_g, ht_ref)):
            raise RuntimeError("graph replay differs from the eager forward")
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        graph_ms = (t1 - t0) * 1e3 / args.steps
    # per-kernel durations: the same number of steps again, with the
    # library's HIP events recorded around every launch on its stream (the
    # events add a few us per launch, so they stay out of the timed region)
    gdr.timing.reset()
    gdr.timing.enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    gdr.timing.enable(False)
    kern = gdr.timing.collect()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens = w.B * w.T
    value = tokens / (ms_per_step * 1e-3)

    if args.calib_copy_mb > 0:
        nbytes = args.calib_copy_mb << 20
        src = torch.empty(nbytes // 4, device=dev, dtype=torch.float32).uniform_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    # the same step one call at a time, each after a 1 GiB cache flush (the
    # inputs are then read from HBM, not from the 256 MB last-level cache)
    flush = torch.empty(1 << 28, device=dev, dtype=torch.float32)
    flushed = []
    for _ in range(args.flushed_steps):
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        flushed.append(e0.elapsed_time(e1))
    del flush
    flushed_ms = sorted(flushed)[len(flushed) // 2] if flushed else None

    # Roofline of the dominant kernel against the method's work for the whole
    # workload: its essential bytes (q and k shared by the G value heads, v,
    # g, beta in; o out; the final state) and its chunk-GEMM flops, divided by
    # the kernel's mean duration, as fractions of the published HBM and bf16
    # MFMA peaks (and of the peaks measured below).  The kernel's own bytes
    # (with the A diag(beta) intermediate and the re-reads of the two-kernel
    # split) are reported separately under "kernel_own".
    work = per_kernel_work(w, G)
    tv = w.B * w.T * w.Hv
    dom = max((n for n in kern if n in work), key=lambda n: kern[n][0])
    avg_ms = kern[dom][0] / kern[dom][1]
    mflops_tv, mbytes_tv = method_work(w.K, w.V, G, 2, False)
    state_bytes = w.B * w.Hv * w.K * w.V * 4                         # final_state out
    m_bytes, m_flops = mbytes_tv * tv + state_bytes, mflops_tv * tv
    t_hbm = m_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = m_flops / (MFMA_BF16_PEAK_TFS * 1e12)
    gbs, tfs = m_bytes / (avg_ms * 1e-3) / 1e9, m_flops / (avg_ms * 1e-3) / 1e12
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": tfs, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom)
    roof["kernel"] = dom
    roof["kernel_avg_us"] = avg_ms * 1e3
    roof["work"] = {"bytes": m_bytes, "flops": m_flops, "bytes_per_tv": mbytes_tv, "flops_per_tv": mflops_tv,
                    "basis": "method: q, k (shared by the G value heads), v, g, beta in, o and final_state out; "
                             "chunk GEMMs 6KV + 6CK + 4CV + C^2/3 per token x value head"}
    roof["hbm_frac"] = gbs / HBM_PEAK_GBS
    roof["mfma_frac"] = tfs / MFMA_BF16_PEAK_TFS
    kb_tv, kf_tv = work[dom]
    roof["kernel_own"] = {"bytes_per_tv": kb_tv, "flops_per_tv": kf_tv,
                          "hbm_frac": kb_tv * tv / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "mfma_frac": kf_tv * tv / (avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS}
    step_s = ms_per_step * 1e-3
    roof["step"] = {"hbm_frac": m_bytes / step_s / 1e9 / HBM_PEAK_GBS,
                    "mfma_frac": m_flops / step_s / 1e12 / MFMA_BF16_PEAK_TFS,
                    "flushed_hbm_frac": None if flushed_ms is None else m_bytes / (flushed_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks(torch, dev)
        roof["measured_peaks"] = peaks
        roof["vs_measured"] = {"hbm_frac": gbs / peaks["hbm_copy_GBs"], "mfma_frac": tfs / peaks["mfma_bf16_TFs"],
                               "step_hbm_frac": m_bytes / step_s / 1e9 / peaks["hbm_copy_GBs"]}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        t_sample = w.T
        f = lambda x: x.to(torch.float64).numpy()
        c0 = time.perf_counter()
        oracle.gdr_fwd(f(inp["q"][:, :t_sample]), f(inp["k"][:, :t_sample]), f(inp["v"][:, :t_sample]),
                       f(inp["g"][:, :t_sample]), f(inp["beta"][:, :t_sample]), scale, threads=threads)
        c1 = time.perf_counter()
        cpu = {"value": t_sample / (c1 - c0), "unit": "tokens/s", "cores": min(threads, w.Hv),
               "kind": "oracle",
               "sample": f"fp64 token recurrence over the whole workload ({t_sample} tokens x {w.Hv} "
                         f"value heads), one thread per head",
               **host_cpu()}

    # the whole step against the method's roofline time for this workload
    method_roof = {"bound": "mfma" if t_mfma > t_hbm else "hbm", "t_roof_us": round(max(t_mfma, t_hbm) * 1e6, 2),
                   "frac": round(max(t_mfma, t_hbm) / (ms_per_step * 1e-3), 4),
                   "frac_flushed": None if flushed_ms is None else round(max(t_mfma, t_hbm) / (flushed_ms * 1e-3), 4)}

    configs = None
    if not args.no_configs:
        del q, k, v, g, beta, ws
        torch.cuda.empty_cache()
        configs = config_report(torch, gdr, gi, dev)
    sweep = None
    if not args.no_sweep:
        sweep = train_step_sweep(torch, gdr, dev)

    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "long_context", "B": w.B, "T": w.T, "Hq": w.Hq, "Hv": w.Hv, "K": w.K,
                   "V": w.V, "chunk": 64, "cp_segment_chunks": plan["segment_chunks"],
                   "cp_max_warmup_chunks": plan["warmup_chunks"], "state_workgroups": plan["state_workgroups"],
                   "launch": "hip_graph" if args.graph else "eager", "precise_vnew": bool(args.precise_vnew)},
        "eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms, "settle_s": args.settle_s,
        "flushed": None if flushed_ms is None else {
            "ms_per_step": flushed_ms, "tokens_per_s": tokens / (flushed_ms * 1e-3), "steps": args.flushed_steps,
            "how": "median of single steps, each timed with events after rewriting a 1 GiB buffer"},
        "kernels_us": {n: 1e3 * t / c for n, (t, c) in kern.items()},
        "roofline": roof,
        "method_roofline": method_roof,
        "cpu_baseline": cpu,
        "configs_report": configs,
        "train_step_sweep": sweep,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
