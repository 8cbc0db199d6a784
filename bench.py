"""Throughput of the ROCmFP2 hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the path over one batch of synthetic input that is
already resident in HBM: int8 quantization of the fp32 activations
(rfp2_quantize_acts) followed by the product against ROCmFP2 weights
(rfp2_gemv, rfp2_moe_gemv or rfp2_gemm, by workload).  The weights are
quantized on the GPU (rfp2_quantize_weights) before timing, and the step
rotates over enough distinct copies of them (>= 1 GiB in all) that every
step reads its weights from HBM rather than from the 256 MB last-level cache.

One JSON line is printed.  `value` is whole-job throughput (algorithmic bytes
of the step / wall time of the step for GEMV workloads, 2*M*N*K / step time
for the GEMM workload).  `roofline` describes the product kernel alone, from
HIP events recorded around each of its launches on the bench stream.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
I8_PEAK_TOPS = 5000.0          # MI355X dense int8 matrix cores, 5.0 POP/s
COLD_BYTES = 1 << 30           # distinct weight bytes rotated through
DEFAULT_WORKLOAD = "gemv_4096x4096"
KERNEL_SOURCES = ["rfp2_device.h", "gemv_kernel.h", "gemv.hip", "gemm.hip",
                  "quantize.hip"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic(cfg) -> dict:
    """Bytes the method must move (and int8 ops) per step, by workload."""
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    w_row = K // 32 * 10
    quant = 4 * M * K + M * K + 4 * M * (K // 32)        # a in, q and d out
    if cfg["op"] == "moe":
        tk = cfg["top_k"]
        prod = tk * N * w_row + K + 4 * (K // 32) + 4 * tk + 4 * tk * N
        ops = 2 * tk * N * K
    else:
        prod = N * w_row + M * K + 4 * M * (K // 32) + 4 * M * N
        ops = 2 * M * N * K
    return {"quant_bytes": quant, "product_bytes": prod, "ops": ops}


def traffic_from_profiles(workload: str, khash: str):
    """HBM bytes per launch of the product kernel, from the committed counter
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_hash") != khash:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, budget_s: float = 12.0) -> dict:
    """The CPU oracle on a bounded sample of the workload: the first `rows`
    weight rows (quantized by the oracle, untimed), then timed repetitions of
    activation quantization + fp64 product until `budget_s` is spent."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()
                            if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = 1
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    rows = min(N, 256)
    if cfg["op"] == "moe":
        W = synth.expert_weights(int(synth.routing(cfg["E"], cfg["top_k"])[0]), N, K,
                                 cfg["sigma"], seed=cfg["wseed"])[:rows]
    else:
        W = synth.weights(N, K, cfg["sigma"], seed=cfg["wseed"])[:rows]
    packed = oracle.quantize_weights(W)
    Mb = min(M, 64)
    a = synth.activations(M, K)[:Mb]
    reps, t0 = 0, time.perf_counter()
    while True:
        q, d = oracle.quantize_acts(a)
        oracle.ref_gemv(packed, rows, K, q, d)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / reps
    w_row = K // 32 * 10
    sample_bytes = (rows * w_row + Mb * K + 4 * Mb * (K // 32) + 4 * Mb * rows
                    + 4 * Mb * K + Mb * K + 4 * Mb * (K // 32))
    sample_ops = 2 * Mb * rows * K
    out = {"cores": int(blas_threads), "kind": "oracle",
           "sample": f"{rows} weight rows x {Mb} token(s) of {cfg['name']}, "
                     f"{reps} timed repetitions of quantize_acts + ref_gemv (fp64, numpy)"}
    if cfg["op"] == "gemm":
        out.update(value=sample_ops / per / 1e12, unit="TOPS")
    else:
        out.update(value=sample_bytes / per / 1e9, unit="GB/s")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the product kernels run on a single MI355X; no multi-GPU path exists)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import bit_gemv_amd as rf
    import synth

    cfg = dict(synth.WORKLOADS[args.workload], name=args.workload)
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    alg = algorithmic(cfg)
    w_row = K // 32 * 10

    with torch.cuda.stream(stream):
        # ---- weights, quantized on the GPU, then copied until >= 1 GiB
        if cfg["op"] == "moe":
            E, top_k = cfg["E"], cfg["top_k"]
            per_copy = E * N * w_row
            master = torch.empty(per_copy, dtype=torch.uint8, device=dev)
            for e in range(E):
                We = torch.from_numpy(synth.expert_weights(e, N, K, cfg["sigma"],
                                                           seed=cfg["wseed"])).to(dev)
                rf.rfp2_quantize_weights(We, N, K, master[e * N * w_row:(e + 1) * N * w_row])
            ids = torch.from_numpy(synth.routing(E, top_k)).to(dev)
        else:
            per_copy = N * w_row
            master = torch.empty(per_copy, dtype=torch.uint8, device=dev)
            rf.rfp2_quantize_weights(
                torch.from_numpy(synth.weights(N, K, cfg["sigma"], seed=cfg["wseed"])).to(dev),
                N, K, master)
        copies = max(2, -(-COLD_BYTES // per_copy))
        bank = [master] + [master.clone() for _ in range(copies - 1)]
        a = torch.from_numpy(synth.activations(M, K)).to(dev)
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
        d = torch.empty((M, K // 32), dtype=torch.float32, device=dev)
        rows_out = cfg["top_k"] if cfg["op"] == "moe" else M
        y = torch.empty((rows_out, N), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

        def product(i):
            w = bank[i % copies]
            if cfg["op"] == "moe":
                rf.rfp2_moe_gemv(w, cfg["E"], N, K, ids, cfg["top_k"], q, d, y, None, stream)
            elif cfg["op"] == "gemm":
                rf.rfp2_gemm(w, N, K, q, d, M, y, stream)
            else:
                rf.rfp2_gemv(w, N, K, q, d, M, y, stream)

        def step(i, ev=None):
            rf.rfp2_quantize_acts(a, M, K, q, d, stream)
            if ev is not None:
                ev[0].record(stream)
            product(i)
            if ev is not None:
                ev[1].record(stream)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()

        # whole-job timing (no per-kernel events inside)
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for i in range(args.steps):
            step(args.warmup + i)
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_total = t_start.elapsed_time(t_end)

        # product-kernel timing: events around each launch on the same stream
        n_ev = min(args.steps, 500)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_ev)]
        for i in range(n_ev):
            step(i, evs[i])
        torch.cuda.synchronize()
        kern_ms = np.array([b.elapsed_time(e) for b, e in evs])

    ms_step = ms_total / args.steps
    kern_avg_s = float(np.mean(kern_ms)) * 1e-3
    khash = kernel_hash()
    if cfg["op"] == "gemm":
        value = alg["ops"] / (ms_step * 1e-3) / 1e12
        unit, metric = "TOPS", "ROCmFP2 M=512 GEMM int8 TOPS"
        achieved = alg["ops"] / kern_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": I8_PEAK_TOPS,
                "unit": "TOPS", "frac": achieved / I8_PEAK_TOPS}
    else:
        value = (alg["quant_bytes"] + alg["product_bytes"]) / (ms_step * 1e-3) / 1e9
        unit, metric = "GB/s", "ROCmFP2 GEMV effective HBM GB/s"
        achieved = alg["product_bytes"] / kern_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS}
    roof["traffic"] = traffic_from_profiles(args.workload, khash)
    roof["kernel"] = {"moe": "rfp2_moe_gemv", "gemm": "rfp2_gemm"}.get(cfg["op"], "rfp2_gemv")
    roof["kernel_us"] = {"mean": float(np.mean(kern_ms)) * 1e3,
                         "p10": float(np.percentile(kern_ms, 10)) * 1e3,
                         "p50": float(np.percentile(kern_ms, 50)) * 1e3,
                         "p90": float(np.percentile(kern_ms, 90)) * 1e3}
    roof["algorithmic_bytes"] = alg["product_bytes"]

    out = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K,
                   **({"experts": cfg["E"], "top_k": cfg["top_k"]} if cfg["op"] == "moe" else {}),
                   "weight_copies": copies, "weight_bytes_per_copy": per_copy,
                   "step": "rfp2_quantize_acts + " + roof["kernel"],
                   "kernel_hash": khash},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
