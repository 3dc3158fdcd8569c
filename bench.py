"""Benchmark of the quantized-linear hot path on one MI355X.

One step is the linear layer's forward on the DiT-shaped FP8 workload
(per-token activation scales x per-output-channel weight scales, M=4096 tokens,
K=3072, N=12288, 1% of the activation's K-channels x20): quantize the bf16
activation (amax, scale, round-to-nearest-even cast, pack), then the FP8 GEMM
with the scales applied in its epilogue, bf16 out.  The weight is quantized
once, before timing, as a layer does at load.

    python bench.py [--gpus 1] [--steps 50] [--warmup 100] [--all] [--no-cpu]

Prints one JSON line: qlinear TFLOP/s (value), the quantize kernel's GB/s, a
roofline object for the dominant kernel (the GEMM, timed with HIP events on
the stream it runs on) and the CPU oracle timed on a bounded sample.  ``--all``
first prints one extra JSON line per workload and kernel (quantize A / W,
GEMM, qlinear) for the tables in the design notes.

Activation inputs rotate over enough copies (>= 1 GiB) that every step reads
them from HBM rather than from the 256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0, "bf16": 2500.0, "int8": 5000.0}   # MI355X dense matrix peaks (int8: TOP/s)
EPI_SCHEMES = ("fp8_tensor", "fp8_row", "fp8_block128", "int8_row")           # GEMMs with the alpha / bias epilogue
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # The GPU's clock settles over the first ~15 ms of load (measured: the GEMM takes
    # ~137 us after 20 untimed steps, 127 us after 50, 121-123 us after 100-200), so
    # 100 untimed steps come before the timed ones.
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--all", action="store_true", help="also time every workload and kernel")
    p.add_argument("--workload", default=None, help="with --all: only this workload")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a plain 1 GiB device copy (read 1 GiB, write 1 GiB) three times, the "
                        "reference dispatch that scales FETCH_SIZE / WRITE_SIZE counters to bytes")
    return p.parse_args()


def gpu_setup():
    import torch
    import precision_quantized_linear_amd as pql
    pql.lib()
    torch.cuda.set_device(0)
    return torch, pql


def up(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def rotation(nbytes: int) -> int:
    return max(2, math.ceil((1 << 30) / max(1, nbytes)))


def quant_bytes(scheme: str, role: str, rows: int, cols: int) -> int:
    """Algorithmic HBM bytes of one quantize call: bf16 read once, codes and scales
    written once (per-tensor reads the input twice: the scale needs the whole tensor)."""
    import precision_quantized_linear_amd as pql
    c, s, z = pql.quantized_sizes(scheme, role, rows, cols)
    reads = 2 if scheme == "fp8_tensor" else 1
    return reads * 2 * rows * cols + c + s + z


class EventTimer:
    """Per-launch durations from HIP events recorded on the launching (current) stream.
    Events are made ahead of time (``reserve``), so timing adds no allocation."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []
        self.spare = []

    def reserve(self, n):
        t = self.torch
        self.spare = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(n)]

    def __call__(self, fn):
        if self.spare:
            s, e = self.spare.pop()
        else:
            s, e = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self):
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs])) if self.pairs else float("nan")


def time_loop(torch, fn, steps, warmup):
    """Mean duration of one launch: `steps` launches back to back between two HIP events
    on the launching stream, so the host's launch latency overlaps the GPU's work."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


# ----------------------------------------------------------------------------- headline step
def headline(torch, pql, steps, warmup):
    import workloads as wl
    w = wl.WORKLOADS["fp8_row_dit"]
    M, N, K = w.M, w.N, w.K
    scheme = "fp8_row"
    a0 = up(torch, wl.activation(w))
    wq = pql.quantize(up(torch, wl.weight(w)), scheme, "weight")
    R = rotation(a0.numel() * 2)
    acts = [a0] + [a0.clone() for _ in range(R - 1)]
    aq = pql.quantize(a0, scheme, "activation")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    tq, tg = EventTimer(torch), EventTimer(torch)

    def step(i):
        tq(lambda: pql.quantize(acts[i % R], scheme, "activation", out=aq))
        tg(lambda: pql.qgemm(aq, wq, out=out))

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    tq.pairs.clear()
    tg.pairs.clear()
    tq.reserve(steps)
    tg.reserve(steps)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / steps
    flops = 2.0 * M * N * K
    q_ms, g_ms = tq.mean_ms(), tg.mean_ms()
    qb = quant_bytes(scheme, "activation", M, K)
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    return {
        "step_ms": step_ms, "tflops": flops / (step_ms * 1e-3) / 1e12,
        "gemm_ms": g_ms, "gemm_tflops": gemm_tflops,
        "quant_ms": q_ms, "quant_gbs": qb / (q_ms * 1e-3) / 1e9, "quant_bytes": qb,
        "M": M, "N": N, "K": K, "rotation": R,
        "gemm_kernel": pql.kernel_name("qgemm", scheme, "activation", M, N, K),
        "quant_kernel": pql.kernel_name("quantize", scheme, "activation", M, N, K),
    }


# ----------------------------------------------------------------------------- every workload
def all_workloads(torch, pql, steps, warmup, only=None):
    import workloads as wl
    lines = []
    # int8 W8A8 has no workload of its own on the pages; it runs on the per-token /
    # per-channel FP8 workload's shape and data, the scheme it mirrors.
    for name, scheme in (("fp8_tensor_small", "fp8_tensor"), ("fp8_row_dit", "fp8_row"),
                         ("fp8_row_dit", "int8_row"), ("fp8_block_dit", "fp8_block128"),
                         ("mx_video_dit", "mxfp8"), ("mx_video_dit", "mxfp4")):
        if only and name != only:
            continue
        w = wl.WORKLOADS[name]
        a0, w0 = up(torch, wl.activation(w)), up(torch, wl.weight(w))
        Ra, Rw = rotation(a0.numel() * 2), rotation(w0.numel() * 2)
        acts = [a0] + [a0.clone() for _ in range(Ra - 1)]
        wts = [w0] + [w0.clone() for _ in range(Rw - 1)]
        aq = pql.quantize(a0, scheme, "activation")
        wq = pql.quantize(w0, scheme, "weight")
        out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(1, pql.workspace_size("qlinear", scheme, "activation", w.M, w.N, w.K)),
                         dtype=torch.uint8, device="cuda")
        qws = torch.empty(max(1, pql.workspace_size("quantize", scheme, "activation")), dtype=torch.uint8,
                          device="cuda")
        ta = time_loop(torch, lambda i: pql.quantize(acts[i % Ra], scheme, "activation", workspace=qws, out=aq),
                       steps, warmup)
        tw = time_loop(torch, lambda i: pql.quantize(wts[i % Rw], scheme, "weight", workspace=qws, out=wq),
                       steps, warmup)
        tg = time_loop(torch, lambda i: pql.qgemm(aq, wq, out=out), steps, warmup)
        tl = time_loop(torch, lambda i: pql.qlinear(acts[i % Ra], wq, out=out, workspace=ws), steps, warmup)
        flops = 2.0 * w.M * w.N * w.K
        ba, bw = quant_bytes(scheme, "activation", w.M, w.K), quant_bytes(scheme, "weight", w.N, w.K)
        peak = PEAK_TFLOPS["fp4" if scheme == "mxfp4" else "int8" if scheme == "int8_row" else "fp8"]
        extra = {}
        if scheme in EPI_SCHEMES:   # the fused epilogue alpha * (A W^T) + bias
            bias = torch.randn(w.N, device="cuda").to(torch.bfloat16)
            te = time_loop(torch, lambda i: pql.qgemm(aq, wq, out=out, alpha=0.5, bias=bias), steps, warmup)
            extra.update({"gemm_epi_us": te * 1e3, "gemm_epi_tflops": flops / (te * 1e-3) / 1e12})
        if scheme in pql.STATIC_SCHEMES:   # static activation scales
            sa = aq.scales.clone()
            aqs = pql.quantize_static(a0, scheme, "activation", sa)
            ts = time_loop(torch, lambda i: pql.quantize_static(acts[i % Ra], scheme, "activation", sa, out=aqs),
                           steps, warmup)
            tls = time_loop(torch, lambda i: pql.qlinear(acts[i % Ra], wq, out=out, workspace=ws, alpha=0.5,
                                                         bias=bias, act_scales=sa), steps, warmup)
            bs = 2 * w.M * w.K + aq.codes.numel() + sa.numel() * 4   # bf16 in, codes out, scales in
            extra.update({"quant_a_static_us": ts * 1e3, "quant_a_static_gbs": bs / (ts * 1e-3) / 1e9,
                          "quant_a_static_hbm_frac": bs / (ts * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "qlinear_static_bias_us": tls * 1e3})
        lines.append({"workload": name, "scheme": scheme, "M": w.M, "N": w.N, "K": w.K, **extra,
                      "quant_a_us": ta * 1e3, "quant_a_gbs": ba / (ta * 1e-3) / 1e9,
                      "quant_a_hbm_frac": ba / (ta * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "quant_w_us": tw * 1e3, "quant_w_gbs": bw / (tw * 1e-3) / 1e9,
                      "quant_w_hbm_frac": bw / (tw * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "gemm_us": tg * 1e3, "gemm_tflops": flops / (tg * 1e-3) / 1e12,
                      "gemm_mfma_frac": flops / (tg * 1e-3) / 1e12 / peak,
                      "qlinear_us": tl * 1e3, "qlinear_tflops": flops / (tl * 1e-3) / 1e12})
        del acts, wts, aq, wq, out, ws, extra
        torch.cuda.empty_cache()
    if only and only != "w4a16_dit":
        return lines
    w = wl.WORKLOADS["w4a16_dit"]
    codes, zeros, scales = wl.int4_weight_parts(w)
    wq = pql.QTensor("w4a16_asym", "weight", w.N, w.K,
                     torch.from_numpy(wl.pack_int4_codes(codes).view(np.int32)).cuda(),
                     torch.from_numpy(np.ascontiguousarray(scales.T).view(np.int16)).view(torch.bfloat16).cuda(),
                     torch.from_numpy(np.ascontiguousarray(zeros.T)).cuda())   # group-major
    for M in w.m_sweep:
        a0 = up(torch, wl.activation(w, M))
        R = rotation(a0.numel() * 2 + w.N * w.K // 2)
        wcopies = [wq] + [pql.QTensor(wq.scheme, wq.role, wq.rows, wq.cols, wq.codes.clone(), wq.scales.clone(),
                                      wq.zeros.clone()) for _ in range(min(R, 64) - 1)]
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device="cuda")
        tl = time_loop(torch, lambda i: pql.qgemm(a0, wcopies[i % len(wcopies)], out=out), steps, warmup)
        flops = 2.0 * M * w.N * w.K
        byts = w.N * w.K // 2 + w.N * (w.K // 128) * 3 + 2 * M * w.K + 2 * M * w.N
        lines.append({"workload": "w4a16_dit", "scheme": "w4a16_asym", "M": M, "N": w.N, "K": w.K,
                      "gemm_us": tl * 1e3, "gemm_tflops": flops / (tl * 1e-3) / 1e12,
                      "gemm_mfma_frac": flops / (tl * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
                      "gemm_gbs": byts / (tl * 1e-3) / 1e9,
                      "gemm_hbm_frac": byts / (tl * 1e-3) / 1e9 / PEAK_HBM_GBS})
        del wcopies
        torch.cuda.empty_cache()
    return lines


# ----------------------------------------------------------------------------- CPU oracle
def cpu_baseline(seconds: float):
    """The oracle, as it stands, on a bounded row sample of the same workload: quantize
    the activation rows, then the float64 GEMM against the (pre-quantized) weight."""
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    w = wl.WORKLOADS["fp8_row_dit"]
    rows = 256
    a = wl.activation(w)[:rows]
    wq = oracle.quantize(wl.weight(w), "fp8_row", "weight")
    flops = 2.0 * rows * w.N * w.K
    done, t0 = 0, time.perf_counter()
    while True:
        aq = oracle.quantize(a, "fp8_row", "activation")
        oracle.gemm_ref(aq, wq)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= 50:
            break
    return {"value": flops * done / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {w.M} activation rows of the same FP8 per-token workload (N={w.N}, K={w.K}): "
                      f"oracle quantize + float64 GEMM, {done} repetitions in {el:.1f} s; weight quantized "
                      f"once before timing", "seconds": el}


def measured_traffic(kernel_source: str):
    """HBM bytes per launch of the GEMM from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None when that summary was taken on a different kernel source."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    prof = os.path.join(root, "profiles", "k_gemm32_fp8__fp8_row_dit.md")
    try:
        fields = dict(line.split(": ", 1) for line in open(prof).read().splitlines() if ": " in line
                      and line.split(": ", 1)[0] in ("traffic_bytes_per_launch", "kernel_source",
                                                     "kernel_source_sha256_16"))
        src = os.path.join(root, fields["kernel_source"])
        if fields["kernel_source"] != kernel_source:
            return None
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        return int(fields["traffic_bytes_per_launch"]) if sha == fields["kernel_source_sha256_16"] else None
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    torch, pql = gpu_setup()
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.all:
        for line in all_workloads(torch, pql, args.steps, args.warmup, args.workload):
            print(json.dumps(line), flush=True)
    h = headline(torch, pql, args.steps, args.warmup)
    peak = PEAK_TFLOPS["fp8"]
    result = {
        "metric": "qlinear TFLOP/s & quantize GB/s on 1 MI355X, % of MFMA/HBM peak",
        "value": round(h["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "fp8_row_dit: FP8 e4m3 per-token activation x per-channel weight scales, "
                               "M=4096 K=3072 N=12288, 1% K-channel outliers x20, bf16 out",
                   "M": h["M"], "N": h["N"], "K": h["K"], "scheme": "fp8_row",
                   "step": "quantize A (per-token) + FP8 GEMM; W quantized once at load"},
        "quantize": {"kernel": h["quant_kernel"], "us": round(h["quant_ms"] * 1e3, 2),
                     "GB/s": round(h["quant_gbs"], 1), "hbm_frac": round(h["quant_gbs"] / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": h["quant_bytes"]},
        "roofline": {"kernel": h["gemm_kernel"], "bound": "mfma", "achieved": round(h["gemm_tflops"], 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(h["gemm_tflops"] / peak, 4),
                     "traffic": measured_traffic("precision_quantized_linear_amd/csrc/gemm32.hip"),
                     "avg_us": round(h["gemm_ms"] * 1e3, 2),
                     "algorithmic_flops": 2 * h["M"] * h["N"] * h["K"]},
    }
    if not args.no_cpu:
        cb = cpu_baseline(args.cpu_seconds)
        cb.pop("seconds", None)
        cb["value"] = round(cb["value"], 5)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
