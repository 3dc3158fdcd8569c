"""Benchmark of the quantized-linear hot path on one MI355X.

One step is the linear layer's forward: quantize the bf16 activation with the
scheme's activation rule (amax, scale, round-to-nearest-even cast, pack), then
the scaled GEMM against the weight, quantized once before timing (as a layer
does at load), bf16 out.  Every workload runs in turn; the headline, printed
last, is the largest one: FP8 block-128 scales (activations 1x128 per token,
weights 128x128), M=8192 tokens, K=5120, N=13824.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--only WORKLOAD] [--no-cpu]

Prints one JSON line per workload (``"kind": "workload"``) and then the
headline line with the contract's fields, the roofline of the dominant kernel
(the block-128 GEMM, its launches timed with HIP events on the stream it runs
on), a summary of every workload, and the CPU oracle's per-phase timings on the
same workload.  Per-launch statistics are the mean (the roofline's figure),
median, p10 and p90 of the timed launches.

Activation inputs rotate over enough copies (>= 1 GiB) that every step reads
them from HBM rather than from the 256 MB Infinity Cache; weight-quantize and
W4A16 timings rotate weight copies the same way.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0, "bf16": 2500.0, "int8": 5000.0}   # MI355X dense matrix peaks
PEAK_HBM_GBS = 8000.0
CPU_GEMM_ROWS = 512                   # rows of the headline GEMM the CPU oracle recomputes
HEADLINE = ("fp8_block_dit", "fp8_block128")
# every workload, the headline last (the largest GEMM: 1.16 TFLOP)
RUNS = (("fp8_tensor_small", "fp8_tensor"), ("fp8_row_dit", "fp8_row"), ("mx_video_dit", "mxfp8"),
        ("mx_video_dit", "mxfp4"), ("mx_video_dit", "mxfp4_dual"), ("w4a16_dit", "w4a16_asym"),
        ("fp8_decode", "fused"), HEADLINE)
# --all adds the NEXT variants before the headline: int8 W8A8, the alpha / bias epilogue, static FP8 scales
EXTRA = (("fp8_row_dit", "int8_row"), ("fp8_row_dit", "fp8_row+epilogue"), ("fp8_row_dit", "int8_row+epilogue"),
         ("fp8_block_dit", "fp8_block128+epilogue"), ("fp8_block_dit", "fp8_block128+static"),
         ("fp8_tensor_small", "fp8_tensor+static"), ("load_and_dequant", "w4a16_asym+fp8_block128"))
DESCRIPTION = {
    "fp8_tensor_small": "FP8 e4m3 per-tensor dynamic scales, M=256 K=512 N=512",
    "fp8_row_dit": "FP8 e4m3 per-token activation x per-channel weight scales, M=4096 K=3072 N=12288, "
                   "1% K-channel outliers x20",
    "fp8_block_dit": "FP8 e4m3 block-128 dynamic scales (activation 1x128 per token, weight 128x128), "
                     "M=8192 K=5120 N=13824",
    "mx_video_dit": "OCP MX (E8M0 per 32 K), M=20280 K=5120 N=5120, 0.5% K-channel outliers x50",
    "w4a16_dit": "W4A16 int4 group-128 asymmetric, K=3072 N=12288",
    "fp8_decode": "FP8 per-token / block-128 qlinear for 1 and 16 tokens (fused activation quantize + GEMM), "
                  "K=3072 N=12288",
    "load_and_dequant": "the int4 RTN weight quantizer on the W4A16 weight (N=12288 K=3072, once at load) and "
                        "dequantize of that weight and of the block-128 activation (M=8192 K=5120)",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--only", default=None, help="time only this workload (NAME or NAME:SCHEME; its line is then "
                                                "the last)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--all", action="store_true", help="also time int8 W8A8, the alpha / bias epilogue, static "
                                                      "FP8 scales, the load-time int4 quantizer and dequantize "
                                                      "(before the headline)")
    p.add_argument("--copy-reference", action="store_true",
                   help="time torch's own bf16 -> fp8 cast at every quantizer size (the same bytes a quantizer "
                        "moves, without the scale arithmetic) and a cold read of the W4A16 weight, then exit")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a plain 1 GiB device copy (read 1 GiB, write 1 GiB) three times, the "
                        "reference dispatch that scales FETCH_SIZE / WRITE_SIZE counters to bytes")
    return p.parse_args()


def gpu_setup():
    import torch
    import precision_quantized_linear_amd as pql
    pql.lib()                       # raises if the HIP library is missing: there is no fallback
    torch.cuda.set_device(0)
    return torch, pql


def up(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def copies_for(nbytes: int, cap: int = 64) -> int:
    return max(2, min(cap, math.ceil((1 << 30) / max(1, nbytes))))


def settle(torch, tensors) -> None:
    """Read every byte of the rotated copies once, untimed, with a torch reduction (so it
    never mixes into a library kernel's trace).  Freshly cloned copies leave the caches
    full of written lines and a first pass over them runs slower than every later one (the
    W4A16 GEMV at M = 1: 9.4 us in a 10-step run against 6.4-6.9 us after); the timed
    steps then measure the steady rotation."""
    for t in tensors:
        if t is not None and t.numel():
            torch.sum(t.reshape(-1).view(torch.uint8), dtype=torch.int64)
    torch.cuda.synchronize()


def quant_bytes(pql, scheme: str, role: str, rows: int, cols: int) -> int:
    """Algorithmic HBM bytes of one quantize call: bf16 read once, codes and scales
    written once (per-tensor reads the input twice: the scale needs the whole tensor)."""
    c, s, z = pql.quantized_sizes(scheme, role, rows, cols)
    reads = 2 if scheme == "fp8_tensor" else 1
    return reads * 2 * rows * cols + c + s + z


def stats_us(ms_list):
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return {"mean_us": float(a.mean()), "median_us": float(np.median(a)), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90))}


class Events:
    """Per-launch HIP events recorded on the current (launching) stream, made ahead of
    the timed loop so that timing allocates nothing inside it."""

    def __init__(self, torch, n):
        self.pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(n)]
        self.used = 0

    def __call__(self, fn):
        s, e = self.pairs[self.used]
        self.used += 1
        s.record()
        fn()
        e.record()

    def ms(self):
        return [s.elapsed_time(e) for s, e in self.pairs[:self.used]]


def timed(torch, fn, steps, warmup):
    """Run fn(i) for warmup untimed then `steps` timed iterations; returns (total ms,
    per-launch ms list).  fn(i, ev) records its own launches into `ev`."""
    for i in range(warmup):
        fn(i, None)
    torch.cuda.synchronize()
    ev = Events(torch, steps * 2)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i, ev)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end), ev


def _rate(x, unit_scale):
    return round(x * unit_scale, 2)


# ----------------------------------------------------------------------------- one FP8 / MX workload
def run_quantized(torch, pql, name, scheme, steps, warmup):
    """One FP8 / MX / int8 workload.  ``scheme`` may carry a variant: "+epilogue" (the GEMM
    with alpha = 0.5 and a bf16 bias), "+static" (the activation quantized with supplied
    scales: the dynamic scales of the same input, as a calibrated scale would be)."""
    import workloads as wl
    scheme, _, variant = scheme.partition("+")
    w = wl.WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    a_bits, w_bits = wl.activation(w), wl.weight(w)
    a0, w0 = up(torch, a_bits), up(torch, w_bits)
    acts = [a0] + [a0.clone() for _ in range(copies_for(a0.numel() * 2) - 1)]
    wts = [w0] + [w0.clone() for _ in range(copies_for(w0.numel() * 2, 16) - 1)]
    settle(torch, acts + wts)
    qws = torch.empty(max(1, pql.workspace_size("quantize", scheme, "activation")), dtype=torch.uint8, device="cuda")
    wq = pql.quantize(w0, scheme, "weight", workspace=qws)
    aq = pql.quantize(a0, scheme, "activation", workspace=qws)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    static = aq.scales.clone() if variant == "static" else None
    bias = up(torch, wl.small_case(7, 1, N, 0.5)[0]) if variant == "epilogue" else None
    alpha = 0.5 if variant == "epilogue" else 1.0

    # weight quantize (done once at load in a layer; timed here for its bandwidth)
    def wstep(i, ev):
        f = lambda: pql.quantize(wts[i % len(wts)], scheme, "weight", workspace=qws, out=wq)
        ev(f) if ev else f()
    _, evw = timed(torch, wstep, steps, warmup)

    # the step: quantize A, then the GEMM
    def step(i, ev):
        if static is None:
            fq = lambda: pql.quantize(acts[i % len(acts)], scheme, "activation", workspace=qws, out=aq)
        else:
            fq = lambda: pql.quantize_static(acts[i % len(acts)], scheme, "activation", static, out=aq)
        fg = lambda: pql.qgemm(aq, wq, out=out, alpha=alpha, bias=bias)
        if ev:
            ev(fq)
            ev(fg)
        else:
            fq()
            fg()
    total_ms, ev = timed(torch, step, steps, warmup)
    ms = ev.ms()
    q_ms, g_ms = ms[0::2], ms[1::2]
    flops = 2.0 * M * N * K
    peak = PEAK_TFLOPS["fp4" if scheme.startswith("mxfp4") else "int8" if scheme == "int8_row" else "fp8"]
    ba, bw = quant_bytes(pql, scheme, "activation", M, K), quant_bytes(pql, scheme, "weight", N, K)
    qa, qw, gg = stats_us(q_ms), stats_us(evw.ms()), stats_us(g_ms)
    step_ms = total_ms / steps
    line = {
        "kind": "workload", "workload": name, "scheme": scheme + (f"+{variant}" if variant else ""),
        "M": M, "N": N, "K": K,
        "step_us": round(step_ms * 1e3, 2), "step_tflops": round(flops / (step_ms * 1e-3) / 1e12, 1),
        "gemm": {"kernel": pql.kernel_name("qgemm", scheme, "activation", M, N, K) + ("+epilogue" if bias is not None else ""),
                 **{k: round(v, 2) for k, v in gg.items()},
                 "tflops": round(flops / (gg["mean_us"] * 1e-6) / 1e12, 1),
                 "mfma_frac": round(flops / (gg["mean_us"] * 1e-6) / 1e12 / peak, 4),
                 "mfma_frac_median": round(flops / (gg["median_us"] * 1e-6) / 1e12 / peak, 4), "peak_tflops": peak},
        "quant_a": {"kernel": pql.kernel_name("quantize", scheme, "activation", M, N, K) if static is None
                    else "k_fp8_static",
                    **{k: round(v, 2) for k, v in qa.items()}, "bytes": ba,
                    "gbs_median": round(ba / (qa["median_us"] * 1e-6) / 1e9, 1),
                    "hbm_frac_median": round(ba / (qa["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "quant_w": {"kernel": pql.kernel_name("quantize", scheme, "weight", M, N, K),
                    **{k: round(v, 2) for k, v in qw.items()}, "bytes": bw,
                    "gbs_median": round(bw / (qw["median_us"] * 1e-6) / 1e9, 1),
                    "hbm_frac_median": round(bw / (qw["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
    }
    keep = {}
    if (name, scheme) == HEADLINE and not variant:   # the output rows the CPU oracle leg recomputes (every copy of A is equal)
        keep = {"a_bits": a_bits, "w_bits": w_bits,
                "c_rows": out[:CPU_GEMM_ROWS].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)}
    del acts, wts, aq, wq, out, static, bias
    torch.cuda.empty_cache()
    return line, keep


# ----------------------------------------------------------------------------- W4A16 sweep
def run_w4a16(torch, pql, steps, warmup):
    import workloads as wl
    w = wl.WORKLOADS["w4a16_dit"]
    codes, zeros, scales = wl.int4_weight_parts(w)
    wq = pql.from_numpy({"scheme": "w4a16_asym", "role": "weight", "rows": w.N, "cols": w.K,
                         "codes": wl.pack_int4_codes(codes), "scales": scales, "zeros": zeros}, "cuda")
    wbytes = w.N * w.K // 2 + w.N * (w.K // 128) * 3
    wcopies = [wq] + [pql.QTensor(wq.scheme, wq.role, wq.rows, wq.cols, wq.codes.clone(), wq.scales.clone(),
                                  wq.zeros.clone()) for _ in range(copies_for(wbytes) - 1)]
    settle(torch, [t for c in wcopies for t in (c.codes, c.scales, c.zeros)])
    lines = []
    for M in w.m_sweep:
        a0 = up(torch, wl.activation(w, M))
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device="cuda")

        def step(i, ev):
            f = lambda: pql.qgemm(a0, wcopies[i % len(wcopies)], out=out)
            ev(f) if ev else f()
        total_ms, ev = timed(torch, step, steps, warmup)
        gg = stats_us(ev.ms())
        flops = 2.0 * M * w.N * w.K
        byts = wbytes + 2 * M * w.K + 2 * M * w.N
        lines.append({"kind": "workload", "workload": "w4a16_dit", "scheme": "w4a16_asym", "M": M, "N": w.N,
                      "K": w.K, "step_us": round(total_ms / steps * 1e3, 2),
                      "gemm": {"kernel": pql.kernel_name("qgemm", "w4a16_asym", "activation", M, w.N, w.K),
                               **{k: round(v, 2) for k, v in gg.items()},
                               "tflops": round(flops / (gg["mean_us"] * 1e-6) / 1e12, 2),
                               "mfma_frac_bf16": round(flops / (gg["mean_us"] * 1e-6) / 1e12 / PEAK_TFLOPS["bf16"], 4),
                               "gbs_median": round(byts / (gg["median_us"] * 1e-6) / 1e9, 1),
                               "hbm_frac_median": round(byts / (gg["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                               "bytes": byts}})
        del a0, out
    del wcopies
    torch.cuda.empty_cache()
    return lines


# ----------------------------------------------------------------------------- load-time quantize, dequantize
def run_load_and_dequant(torch, pql, steps, warmup):
    """The two steps outside the per-call path: the int4 round-to-nearest weight quantizer (run once at
    load) on the W4A16 weight, and dequantize (codes and scales back to bf16) of that weight and of the
    block-128 activation.  Inputs rotate over >= 1 GiB of copies; HIP events per call; GB/s against the
    algorithmic bytes (the input read once, the output written once)."""
    import workloads as wl
    lines = []

    def line(scheme, role, op, rows, cols, kernel, byts, ms):
        st = stats_us(ms)
        return {"kind": "workload", "workload": "load_and_dequant", "scheme": scheme, "role": role, "op": op,
                "M": rows, "N": 0, "K": cols, "kernel": kernel, **{k: round(v, 2) for k, v in st.items()},
                "gbs_median": round(byts / (st["median_us"] * 1e-6) / 1e9, 1),
                "hbm_frac_median": round(byts / (st["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "bytes": byts}

    # int4 RTN quantize of the W4A16 weight (bf16 [12288, 3072] -> codes, scales, zero-points)
    w = wl.WORKLOADS["w4a16_dit"]
    w_bits = wl.weight(w)
    byts = quant_bytes(pql, "w4a16_asym", "weight", w.N, w.K)
    xs = [up(torch, w_bits)]
    xs += [xs[0].clone() for _ in range(copies_for(2 * w.N * w.K) - 1)]
    out = pql.quantize(xs[0], "w4a16_asym", "weight")
    settle(torch, xs)

    def qstep(i, ev):
        f = lambda: pql.quantize(xs[i % len(xs)], "w4a16_asym", "weight", out=out)
        ev(f) if ev else f()
    _, ev = timed(torch, qstep, steps, warmup)
    lines.append(line("w4a16_asym", "weight", "quantize", w.N, w.K, pql.kernel_name("quantize", "w4a16_asym", "weight"),
                      byts, ev.ms()))
    del xs

    # dequantize: that weight, then the block-128 activation of the headline workload
    wa = wl.WORKLOADS["fp8_block_dit"]
    for scheme, role, q in (("w4a16_asym", "weight", out),
                            ("fp8_block128", "activation", pql.quantize(up(torch, wl.activation(wa)), "fp8_block128",
                                                                        "activation"))):
        c, sc, z = pql.quantized_sizes(scheme, role, q.rows, q.cols)
        byts = c + sc + z + 2 * q.rows * q.cols
        qs = [q] + [pql.QTensor(q.scheme, q.role, q.rows, q.cols, q.codes.clone(), q.scales.clone(),
                                None if q.zeros is None else q.zeros.clone())
                    for _ in range(copies_for(c + sc + z) - 1)]
        y = torch.empty((q.rows, q.cols), dtype=torch.bfloat16, device="cuda")
        settle(torch, [t for x in qs for t in (x.codes, x.scales, x.zeros)])

        def dstep(i, ev):
            f = lambda: pql.dequantize(qs[i % len(qs)], out=y)
            ev(f) if ev else f()
        _, ev = timed(torch, dstep, steps, warmup)
        lines.append(line(scheme, role, "dequantize", q.rows, q.cols, pql.kernel_name("dequantize", scheme, role),
                          byts, ev.ms()))
        del qs, y
    del out
    torch.cuda.empty_cache()
    return lines


# ----------------------------------------------------------------------------- few-token qlinear
def run_decode(torch, pql, steps, warmup):
    """qlinear for 1 and 16 tokens on the per-token FP8 workload's weight (N=12288, K=3072):
    one fused launch that quantizes the activation inside the GEMM.  Weight copies rotate
    (>= 1 GiB) so every call streams the weight from HBM; timed per call with HIP events."""
    import workloads as wl
    w = wl.WORKLOADS["fp8_row_dit"]
    w0 = up(torch, wl.weight(w))
    lines = []
    for scheme in ("fp8_row", "fp8_block128"):
        wq = pql.quantize(w0, scheme, "weight")
        wbytes = wq.codes.numel() * wq.codes.element_size() + wq.scales.numel() * 4
        copies = [wq] + [pql.QTensor(wq.scheme, wq.role, wq.rows, wq.cols, wq.codes.clone(), wq.scales.clone(),
                                     None) for _ in range(copies_for(wbytes) - 1)]
        settle(torch, [t for c in copies for t in (c.codes, c.scales)])
        for M in (1, 16):
            a0 = up(torch, wl.activation(w, M))
            out = torch.empty((M, w.N), dtype=torch.bfloat16, device="cuda")

            def step(i, ev):
                f = lambda: pql.qlinear(a0, copies[i % len(copies)], out=out)
                ev(f) if ev else f()
            total_ms, ev = timed(torch, step, steps, warmup)
            gg = stats_us(ev.ms())
            byts = wbytes + 2 * M * w.K + 2 * M * w.N
            lines.append({"kind": "workload", "workload": "fp8_decode", "scheme": scheme, "M": M, "N": w.N,
                          "K": w.K, "step_us": round(total_ms / steps * 1e3, 2),
                          "gemm": {"kernel": pql.kernel_name("qlinear", scheme, "activation", M, w.N, w.K),
                                   **{k: round(v, 2) for k, v in gg.items()},
                                   "gbs_median": round(byts / (gg["median_us"] * 1e-6) / 1e9, 1),
                                   "hbm_frac_median": round(byts / (gg["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                                   "bytes": byts}})
            del a0, out
        del copies, wq
    del w0
    torch.cuda.empty_cache()
    return lines


# ----------------------------------------------------------------------------- CPU oracle
def host_info():
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            blas = f"{infos[0].get('internal_api')} {infos[0].get('version')}"
            threads = max(int(i.get("num_threads", 1)) for i in infos)
    except Exception:
        pass
    return model, blas, threads, len(os.sched_getaffinity(0))


def cpu_baseline(a_bits, w_bits, name, scheme, c_rows=None, gemm_rows=None):
    """The oracle, as it stands, on the headline workload: quantize A (full size, NumPy,
    one core), quantize W (full size, one core) and the float64 GEMM on a row sample
    (BLAS threads), each timed once.  value = the oracle's step rate (quantize A + the
    GEMM extrapolated from the sample to all M rows), in the metric's TFLOP/s.  With the
    GPU's output rows given, the similarity report of those rows against the oracle's
    (cosine, MAE, MSE / RMSE, max |diff|, L2, relative L2, PSNR) is added."""
    import oracle
    from oracle import metrics
    gemm_rows = gemm_rows or CPU_GEMM_ROWS
    M, K = a_bits.shape
    N = w_bits.shape[0]
    model, blas, threads, affinity = host_info()
    t0 = time.perf_counter()
    aq = oracle.quantize(a_bits, scheme, "activation")
    t_qa = time.perf_counter() - t0
    t0 = time.perf_counter()
    wq = oracle.quantize(w_bits, scheme, "weight")
    t_qw = time.perf_counter() - t0
    rows = min(gemm_rows, M)
    a_rows = dict(aq, codes=aq["codes"][:rows], scales=aq["scales"][:rows], rows=rows)
    t0 = time.perf_counter()
    c64 = oracle.gemm_ref(a_rows, wq)
    t_g = time.perf_counter() - t0
    t_g_full = t_g * M / rows
    flops = 2.0 * M * N * K
    return {"value": round(flops / (t_qa + t_g_full) / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{name}: oracle quantize A ({M}x{K}, full size, 1 core), quantize W ({N}x{K}, full size, "
                      f"1 core), float64 GEMM on the first {rows} of {M} rows ({threads} BLAS threads), "
                      f"extrapolated to all rows; value = 2MNK / (quantize A + GEMM)",
            "quantize_a_s": round(t_qa, 3), "quantize_w_s": round(t_qw, 3), "gemm_sample_s": round(t_g, 3),
            "gemm_full_s_est": round(t_g_full, 2), "host_cpu": model, "blas": blas, "blas_threads": threads,
            "affinity_cpus": affinity,
            **({"similarity_gpu_vs_oracle": {
                "rows": rows, **{k: float(f"{v:.6g}") for k, v in metrics.similarity(
                    oracle.bf16_to_f32(c_rows[:rows]).astype(np.float64), c64).items()},
                "meets_starting_thresholds": bool(metrics.meets_starting_thresholds(metrics.similarity(
                    oracle.bf16_to_f32(c_rows[:rows]).astype(np.float64), c64)))}} if c_rows is not None else {})}


def measured_traffic(profile: str, key: str = "traffic_bytes_per_launch"):
    """HBM bytes per launch of a kernel from its committed FETCH_SIZE / WRITE_SIZE summary
    under profiles/ (the line `key: bytes`), or None when that summary was taken on a
    different kernel source."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(root, "profiles", profile)).read().splitlines()
        fields = dict(line.split(": ", 1) for line in text if ": " in line and line.split(": ", 1)[0] in
                      (key, "kernel_source", "kernel_source_sha256_16"))
        src = os.path.join(root, fields["kernel_source"])
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        return int(fields[key]) if sha == fields["kernel_source_sha256_16"] else None
    except (OSError, KeyError, ValueError):
        return None


def summary_of(line):
    s = {"step_us": line["step_us"], "gemm_kernel": line["gemm"]["kernel"], "gemm_median_us": line["gemm"]["median_us"]}
    if "mfma_frac" in line["gemm"]:
        s.update({"gemm_mfma_frac": line["gemm"]["mfma_frac"],
                  "quant_a_hbm_frac_median": line["quant_a"]["hbm_frac_median"],
                  "quant_w_hbm_frac_median": line["quant_w"]["hbm_frac_median"]})
    else:
        s.update({"gemm_hbm_frac_median": line["gemm"]["hbm_frac_median"]})
        if line["gemm"].get("mfma_frac_bf16") is not None:
            s["gemm_bf16_mfma_frac"] = line["gemm"]["mfma_frac_bf16"]
    return s


def copy_reference(torch, steps):
    """Achievable-bandwidth references on this machine, from torch's own kernels (no libpql):
    the elementwise bf16 -> fp8 e4m3 cast at each quantizer shape (reads 2 bytes and writes
    1 byte per element, like a quantizer without its scale arithmetic) and a sum over the
    W4A16 weight's bytes read once (an amax) and copied.  Inputs rotate over >= 1 GiB of copies."""
    shapes = [("fp8_row_dit A", 4096, 3072), ("fp8_row_dit W", 12288, 3072), ("fp8_block_dit A", 8192, 5120),
              ("fp8_block_dit W", 13824, 5120), ("mx_video_dit A", 20280, 5120), ("mx_video_dit W", 5120, 5120)]
    for name, rows, cols in shapes:
        x0 = torch.randn(rows, cols, device="cuda").to(torch.bfloat16)
        xs = [x0] + [x0.clone() for _ in range(copies_for(x0.numel() * 2) - 1)]
        y = torch.empty(rows, cols, device="cuda", dtype=torch.float8_e4m3fn)

        def step(i, ev):
            f = lambda: y.copy_(xs[i % len(xs)])
            ev(f) if ev else f()
        _, ev = timed(torch, step, steps, 5)
        st = stats_us(ev.ms())
        byts = 3 * rows * cols
        print(json.dumps({"kind": "copy_reference", "what": f"torch bf16->fp8 cast, {name} ({rows}x{cols})",
                          "bytes": byts, **{k: round(v, 2) for k, v in st.items()},
                          "tbs_median": round(byts / (st["median_us"] * 1e-6) / 1e12, 2)}), flush=True)
        del xs, x0, y
    nbytes = 12288 * 3072 // 2 + 12288 * 24 * 3            # int4 codes, bf16 scales, u8 zero-points
    w0 = torch.randn(nbytes // 4, device="cuda")
    ws = [w0] + [w0.clone() for _ in range(copies_for(nbytes) - 1)]
    cp = torch.empty_like(w0)
    out = torch.empty((), device="cuda")
    for what, fn, byts in (("torch amax over the W4A16 weight's bytes as fp32 (one cold read)",
                            lambda i: torch.amax(ws[i % len(ws)], dim=0, out=out), nbytes),
                           ("torch copy of the W4A16 weight's bytes (cold read + write)",
                            lambda i: cp.copy_(ws[i % len(ws)]), 2 * nbytes)):
        def rstep(i, ev, fn=fn):
            f = lambda: fn(i)
            ev(f) if ev else f()
        _, ev = timed(torch, rstep, steps, 5)
        st = stats_us(ev.ms())
        print(json.dumps({"kind": "copy_reference", "what": what, "bytes": byts,
                          **{k: round(v, 2) for k, v in st.items()},
                          "tbs_median": round(byts / (st["median_us"] * 1e-6) / 1e12, 2)}), flush=True)


def select_runs(only, all_):
    """The (workload, scheme) runs of one invocation, the headline last: every default run, the --all
    entries before the headline when asked for, or the one --only names (NAME or NAME:SCHEME).  --only
    reaches an --all entry by its exact NAME:SCHEME, or by NAME when no default run has that name."""
    extra = EXTRA if all_ else tuple(
        r for r in EXTRA if only is not None and (only == f"{r[0]}:{r[1]}" or (
            only == r[0] and all(x[0] != r[0] for x in RUNS))))
    every = RUNS[:-1] + extra + RUNS[-1:]
    return [r for r in every if only is None or only in (r[0], f"{r[0]}:{r[1]}")]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              f"run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    torch, pql = gpu_setup()
    if args.copy_reference:
        copy_reference(torch, args.steps)
        return
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    runs = select_runs(args.only, args.all)
    if not runs:
        print(f"unknown workload {args.only!r}", file=sys.stderr)
        sys.exit(2)
    summary, head, keep = {}, None, {}
    for name, scheme in runs:
        if name == "load_and_dequant":
            for line in run_load_and_dequant(torch, pql, args.steps, args.warmup):
                summary[f"{name} {line['op']} {line['scheme']} {line['role']}"] = {
                    "kernel": line["kernel"], "median_us": line["median_us"],
                    "hbm_frac_median": line["hbm_frac_median"]}
                print(json.dumps(line), flush=True)
            continue
        if name in ("w4a16_dit", "fp8_decode"):
            lines = (run_w4a16 if name == "w4a16_dit" else run_decode)(torch, pql, args.steps, args.warmup)
            for line in lines:
                summary[f"{name} {line['scheme']} M={line['M']}"] = summary_of(line)
                print(json.dumps(line), flush=True)
                head = line
            continue
        line, k = run_quantized(torch, pql, name, scheme, args.steps, args.warmup)
        summary[f"{name} {scheme}"] = summary_of(line)
        keep.update(k)
        head = line
        if (name, scheme) != runs[-1]:
            print(json.dumps(line), flush=True)
    if head is None:   # only the load-time quantizer and dequantize lines were asked for
        return
    name, scheme = head["workload"], head["scheme"]
    g = head["gemm"]
    flops = 2 * head["M"] * head["N"] * head["K"]
    step_ms = head["step_us"] * 1e-3
    is_mx4 = scheme.startswith("mxfp4")
    result = {
        "metric": "qlinear TFLOP/s & quantize GB/s on 1 MI355X, % of MFMA/HBM peak",
        "value": round(flops / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4" if is_mx4 else "bf16" if scheme.startswith("w4a16") else "fp8",
        "data": "synthetic",
        "config": {"workload": f"{name}: {DESCRIPTION[name]}, bf16 out", "M": head["M"], "N": head["N"],
                   "K": head["K"], "scheme": scheme,
                   "step": "quantize A (per call) + GEMM; W quantized once at load" if "quant_a" in head
                           else "W4A16 GEMM (bf16 activation used as is)"},
    }
    if "quant_a" in head:
        result["quantize"] = {k: head["quant_a"][k] for k in ("kernel", "mean_us", "median_us", "p10_us", "p90_us",
                                                              "gbs_median", "hbm_frac_median", "bytes")}
        result["quantize_weight"] = {k: head["quant_w"][k] for k in ("kernel", "median_us", "gbs_median",
                                                                     "hbm_frac_median", "bytes")}
        peak = g["peak_tflops"]
        achieved = flops / (g["mean_us"] * 1e-6) / 1e12
        prof = {"k_gemm_block256": ("k_gemm_block256__fp8_block_dit.md", "traffic_bytes_per_launch"),
                "k_gemm32_fp8": ("k_gemm32_fp8__fp8_row_dit.md", "traffic_bytes_per_launch"),
                "k_gemm32<mxfp4>": ("k_gemm32_mx__mx_video_dit.md", "traffic_bytes_per_launch_mxfp4"),
                "k_gemm32<mxfp8>": ("k_gemm32_mx__mx_video_dit.md", "traffic_bytes_per_launch_mxfp8"),
                }.get(g["kernel"]) if (name, scheme) in (("fp8_block_dit", "fp8_block128"), ("fp8_row_dit", "fp8_row"),
                                                          ("mx_video_dit", "mxfp4"), ("mx_video_dit", "mxfp8")) else None
        result["roofline"] = {"kernel": g["kernel"], "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                              "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                              "traffic": measured_traffic(*prof) if prof else None,
                              "avg_us": g["mean_us"], "median_us": g["median_us"], "p10_us": g["p10_us"],
                              "p90_us": g["p90_us"], "algorithmic_flops": flops}
    result["workloads"] = summary
    if not args.no_cpu and keep:
        result["cpu_baseline"] = cpu_baseline(keep["a_bits"], keep["w_bits"], name, scheme, keep.get("c_rows"))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
