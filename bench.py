"""Throughput of the ROCmFP2 hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the path over one batch of synthetic input that is
already resident in HBM: int8 quantization of the fp32 activations and the
product against ROCmFP2 weights.  For one token that is the single
quantizing launch (rfp2_quant_gemv / rfp2_quant_moe_gemv; --two-launch
splits it); otherwise rfp2_quantize_acts followed by the product
(rfp2_gemv, rfp2_moe_gemv_tokens, rfp2_gemm, rfp2_gemm_f16, or
rfp2_moe_sort + the grouped routed GEMM, by workload).  The weights are
quantized on the GPU (rfp2_quantize_weights) before timing, and consecutive
steps read distinct copies of them: a copy comes back only after >= 1 GiB of
other weight bytes that the steps actually read (the routed experts only, for
the MoE workloads), so every step reads its weights from HBM rather than from
the 256 MB last-level cache.

The K timed steps are replayed from one HIP graph (checked bit for bit
against an eager step) right behind a graph of a few untimed lead-in steps,
with HIP events on the bench stream between them: the host submits the timed
graph while the lead-in runs, so neither host launch cost nor the graph's
start-up enters the figure.  A read of 2 GiB of unrelated memory precedes the
timed replay.  One JSON line is printed.  `value` is whole-job
throughput (algorithmic bytes of the step / wall time of the step for GEMV
workloads, 2*M*N*K / step time for the GEMM workload).  `roofline` describes
the product kernel alone: HIP events on the bench stream around K
back-to-back launches of that kernel replayed the same way (so the average
includes the small gap between consecutive kernels).  For the HBM-bound products it also
carries `cold_isolated`: 100 single launches, each after a cache flush,
median and p10 / p90 (see isolated_cold_us), with the plain read timed the
same way in `ceiling`.
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
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16 matrix cores, 2.5 PFLOP/s
COLD_BYTES = 1 << 30           # distinct weight bytes rotated through
# The large-layer GEMV is the workload on which an HBM fraction is meaningful
# (25 MiB of weights; the 5 MiB projection is latency-bound on this GPU).
DEFAULT_WORKLOAD = "gemv_16384x5120"
SECONDARY = ["gemv_512x2048", "gemv_4096x4096", "moe_128x1536x4096_top8",
             "gemv_16384x5120_m4", "moe_128x1536x4096_top8_t4", "gemm_512x14336x4096",
             "gemm_f16_512x14336x4096", "moe_gemm_128x1536x4096_top8_t512"]
MAX_COPY_BYTES = 40 << 30      # device memory the weight copies may take
KERNEL_SOURCES = ["rfp2_device.h", "gemv_kernel.h", "gemv.hip", "gemv_moe.hip", "gemm.hip",
                  "gemm_f16.hip", "f16_decode.h", "moe_sort.hip", "quantize.hip"]
# the sources of the GEMV kernels (one-token, multi-column and routed forms):
# a counter record taken on them stays valid while these are unchanged
GEMV_SOURCES = ["rfp2_device.h", "gemv_kernel.h", "gemv.hip", "gemv_moe.hip", "gemv_m34.hip"]
# the sources of the routed prompt-batch product (sort + fp16 grouped GEMM)
MOE_GEMM_SOURCES = ["rfp2_device.h", "f16_decode.h", "gemm_f16.hip", "moe_sort.hip"]
# the sources of the dense prompt-batch products (int8 and fp16 matrix cores)
GEMM_SOURCES = ["rfp2_device.h", "rfp2_internal.h", "gemm.hip"]
GEMM_F16_SOURCES = ["rfp2_device.h", "f16_decode.h", "rfp2_internal.h", "gemm_f16.hip"]


def kernel_hash(sources=None) -> str:
    """Hash of the kernel sources (all of them by default)."""
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def fused(cfg, two_launch: bool = False) -> bool:
    """One-token workloads run as one launch that quantizes the activations
    inside the product (rfp2_quant_gemv / rfp2_quant_moe_gemv)."""
    return not two_launch and cfg["op"] in ("gemv", "moe") and cfg["M"] == 1


def algorithmic(cfg, one_launch: bool = False) -> dict:
    """Bytes the method must move (and int8 ops) per step, by workload.
    Two launches: quantization (a in, q and d out), then the product (weights,
    q and d in, y out).  One launch: weights and a in, q, d and y out."""
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    w_row = K // 32 * 10
    quant = 4 * M * K + M * K + 4 * M * (K // 32)        # a in, q and d out
    if cfg["op"] == "moe":
        tk = cfg["top_k"]
        weights_y = tk * N * w_row + 4 * tk + 4 * tk * N
        ops = 2 * tk * N * K
    elif cfg["op"] in ("moe_tokens", "moe_gemm"):
        # every distinct routed expert once, ids, and one y row per slot
        import synth
        ids = synth.routing_tokens(cfg["E"], cfg["top_k"], M, cfg["share"])
        slots = M * cfg["top_k"]
        weights_y = len(set(ids.reshape(-1).tolist())) * N * w_row + 4 * slots + 4 * slots * N
        ops = 2 * slots * N * K
    else:
        weights_y = N * w_row + 4 * M * N
        ops = 2 * M * N * K
    if cfg["op"] == "moe":
        import synth
        wbytes = len(set(synth.routing(cfg["E"], cfg["top_k"]).tolist())) * N * w_row
    elif cfg["op"] in ("moe_tokens", "moe_gemm"):
        wbytes = len(set(ids.reshape(-1).tolist())) * N * w_row
    else:
        wbytes = N * w_row
    if one_launch:
        return {"quant_bytes": 0, "product_bytes": weights_y + quant, "ops": ops,
                "weight_bytes": wbytes}
    prod = weights_y + M * K + 4 * M * (K // 32)
    return {"quant_bytes": quant, "product_bytes": prod, "ops": ops, "weight_bytes": wbytes}


def traffic_from_profiles(workload: str):
    """HBM bytes per launch of the product kernel, from the committed counter
    summary, if it was taken on the current sources of the GEMV kernels."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    w = rec.get("workloads", {}).get(workload)
    if not w:
        return None
    # an entry carries the hash of the sources it was taken on (older entries:
    # the file's GEMV hash)
    sources = w.get("hash_sources", rec.get("hash_sources"))
    if w.get("kernel_hash", rec.get("kernel_hash")) != kernel_hash(sources):
        return None
    return w.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, budget_s: float = 12.0) -> dict:
    """The CPU oracle on a bounded sample of the workload: the first `rows`
    weight rows (quantized by the oracle, untimed), then timed repetitions of
    activation quantization + fp64 product until `budget_s` is spent (at
    least 3); the figure is the median repetition."""
    import numpy as np
    import oracle
    import synth
    blas_lib = "unknown"
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        blas_threads = max([p.get("num_threads", 1) for p in blas] or [1])
        if blas:
            blas_lib = f"{blas[0].get('internal_api', '?')} {blas[0].get('version', '')}".strip()
    except Exception:
        blas_threads = 1
    host = (f"host: os.cpu_count()={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}, "
            f"numpy {np.__version__}, BLAS {blas_lib} with {blas_threads} threads "
            f"(the unpack/dequantize steps are single-threaded numpy)")
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
    times, t_all = [], time.perf_counter()
    while True:
        t0 = time.perf_counter()
        q, d = oracle.quantize_acts(a)
        oracle.ref_gemv(packed, rows, K, q, d)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all >= budget_s and len(times) >= 3:
            break
    reps = len(times)
    per = sorted(times)[reps // 2]
    w_row = K // 32 * 10
    sample_bytes = (rows * w_row + Mb * K + 4 * Mb * (K // 32) + 4 * Mb * rows
                    + 4 * Mb * K + Mb * K + 4 * Mb * (K // 32))
    sample_ops = 2 * Mb * rows * K
    out = {"cores": int(blas_threads), "kind": "oracle",
           "sample": f"{rows} weight rows x {Mb} token(s) of {cfg['name']}, "
                     f"median of {reps} timed repetitions of quantize_acts + ref_gemv "
                     f"(fp64, numpy); "
                     + host}
    if cfg["op"] in ("gemm", "gemm_f16"):
        out.update(value=sample_ops / per / 1e12, unit="TOPS")
    else:
        out.update(value=sample_bytes / per / 1e9, unit="GB/s")
    return out


LEAD = 8                       # untimed launches at the head of a timed graph


def ring_slots(weight_bytes: int) -> int:
    """Data slots a timed loop rotates through: a slot is read again only
    after >= 1 GiB of other slots."""
    return max(2, -(-COLD_BYTES // weight_bytes))


def flush_caches(nbytes: int = 2 * COLD_BYTES) -> None:
    """Read `nbytes` of an unrelated buffer (torch's max): the caches then
    hold clean lines of nothing the timed launches read."""
    import torch
    junk = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")
    junk.max()
    torch.cuda.synchronize()
    del junk


def timed_graph(launch, steps: int, stream):
    """Two HIP graphs: LEAD untimed launches launch(0 .. LEAD-1), then the
    `steps` timed launches launch(LEAD + i).  -> (lead graph, timed graph)."""
    import torch
    g_lead = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_lead, stream=stream):
        for i in range(LEAD):
            launch(i, stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            launch(LEAD + i, stream)
    return g_lead, g


def replay_timed_us(tg, steps: int, stream) -> float:
    """Mean us per timed launch of a timed_graph: one untimed replay of both
    graphs and a cache flush, then the lead graph, the start event, the timed
    graph and the end event, enqueued back to back on `stream`: the host
    submits the timed graph while the lead graph still runs, so the events
    bracket back-to-back kernels rather than the graph's start-up."""
    import torch
    g_lead, g = tg
    with torch.cuda.stream(stream):
        g_lead.replay()
        g.replay()
        torch.cuda.synchronize()
        flush_caches()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        g_lead.replay()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def graph_time_us(launch, steps: int, ring: int = 1) -> float:
    """Mean time of launch(i, stream) over `steps` back-to-back launches
    timed inside a HIP graph (as the products are timed); launch i should use
    data slot i % ring."""
    import torch
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        launch(0, stream)
        torch.cuda.synchronize()
        tg = timed_graph(launch, steps, stream)
        us = replay_timed_us(tg, steps, stream)
        del tg
    return us


def isolated_cold_us(launch, stream, launches: int = 100) -> dict:
    """One call at a time from cold caches: before each launch a 1 GiB
    buffer is read and written (torch's in-place add) and then a second
    1 GiB buffer is only read (torch's max), so the caches end up full of
    clean lines of neither the weights nor the inputs; HIP events on the same
    stream bracket the single launch (dispatch included).  The read-only
    pass matters: lines the add leaves dirty are written back while the timed
    launch evicts them, which adds the flush's own write traffic to the
    launch (about 4 us at 26 MB of weights).  Median, p10 and p90 over
    `launches` launches."""
    import torch
    dev = torch.device("cuda:0")
    rw = torch.zeros(COLD_BYTES, dtype=torch.uint8, device=dev)
    ro = torch.zeros(COLD_BYTES // 4, dtype=torch.int32, device=dev)
    times = []
    with torch.cuda.stream(stream):
        for _ in range(launches):
            rw.add_(1)
            ro.max()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(stream)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
    del rw, ro
    times.sort()
    n = len(times)
    return {"median_us": times[n // 2], "p10_us": times[n // 10], "p90_us": times[(9 * n) // 10],
            "launches": n,
            "note": "each launch alone after a 1 GiB read-write and a 1 GiB read-only flush; "
                    "HIP events around the one launch, dispatch included"}


def measure_ceiling(nbytes: int, steps: int, isolated: bool = False) -> dict:
    """The read ceiling at a product's byte count: rfp2_read_ceiling (plain
    coalesced 16-byte loads) over distinct slices of >= 1 GiB, so every read
    comes from HBM as the products' weights do; and one read of 1 GiB.  With
    `isolated`, also the median of single launches timed as isolated_cold_us
    times the products."""
    import torch
    import bit_gemv_amd as rf
    dev = torch.device("cuda:0")
    nb = max(16, nbytes // 16 * 16)
    slot = -(-nb // 4096) * 4096             # slices start page-aligned, as allocations do
    slots = ring_slots(slot)
    buf = torch.zeros(max(slots * slot, COLD_BYTES // 16 * 16), dtype=torch.uint8, device=dev)
    out = torch.empty(rf.READ_CEILING_OUTPUTS, dtype=torch.int32, device=dev)
    us = graph_time_us(lambda i, st: rf.rfp2_read_ceiling(buf[(i % slots) * slot:], nb, out, stream=st),
                       steps, slots)
    big = COLD_BYTES // 16 * 16
    us_big = graph_time_us(lambda i, st: rf.rfp2_read_ceiling(buf, big, out, stream=st),
                           min(steps, 16))
    iso = None
    if isolated:
        iso = isolated_cold_us(lambda st: rf.rfp2_read_ceiling(buf, nb, out, stream=st),
                               torch.cuda.Stream())["median_us"]
    del buf, out
    torch.cuda.empty_cache()
    res = {"kernel": "rfp2_read_ceiling", "bytes": nb, "us": us, "GBps": nb / us / 1e3,
           "GBps_1GiB": big / us_big / 1e3}
    if iso is not None:
        res["isolated_median_us"] = iso
    return res


def measure_quantizer(workload: str, reps: int = 5) -> dict:
    """Weight-quantizer throughput on the workload's matrix: the plain and
    the importance-weighted scale search on the GPU (weights per second,
    graph-free back-to-back launches between events), and the CPU oracle on
    a 16-row sample of the same matrix."""
    import numpy as np
    import torch
    import bit_gemv_amd as rf
    import oracle
    import synth

    cfg = synth.workload(workload)
    N, K = cfg["N"], cfg["K"]
    dev = torch.device("cuda:0")
    W = synth.weights(N, K, cfg["sigma"], seed=cfg["wseed"])
    imp = synth.importance(K)
    x = torch.from_numpy(W).to(dev)
    imp_g = torch.from_numpy(imp).to(dev)
    w = torch.empty(N * K // 32 * 10, dtype=torch.uint8, device=dev)
    out = {"workload": workload, "weights": N * K}
    for name, call in (("plain", lambda: rf.rfp2_quantize_weights(x, N, K, w)),
                       ("imatrix", lambda: rf.rfp2_quantize_weights_imatrix(x, N, K, imp_g, w))):
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"gpu_{name}_ms"] = ms
        out[f"gpu_{name}_gweights_per_s"] = N * K / (ms * 1e-3) / 1e9
    rows = 16
    t0 = time.perf_counter()
    oracle.quantize_weights(W[:rows])
    t_plain = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.quantize_weights(W[:rows], imp)
    t_imp = time.perf_counter() - t0
    out.update(cpu_oracle_plain_mweights_per_s=rows * K / t_plain / 1e6,
               cpu_oracle_imatrix_mweights_per_s=rows * K / t_imp / 1e6,
               cpu_sample=f"{rows} rows of {workload}, numpy fp64, one thread for the search")
    return out


def measure(workload: str, steps: int, warmup: int, two_launch: bool = False,
            per_token: bool = False) -> dict:
    """Time one workload on cuda:0; returns the fields of its bench line."""
    import torch
    import bit_gemv_amd as rf
    import synth

    cfg = dict(synth.workload(workload), name=workload)
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    one = fused(cfg, two_launch)
    alg = algorithmic(cfg, one)
    w_row = K // 32 * 10

    with torch.cuda.stream(stream):
        # ---- weights, quantized on the GPU, then copied until >= 1 GiB
        if cfg["op"] in ("moe", "moe_tokens", "moe_gemm"):
            E, top_k = cfg["E"], cfg["top_k"]
            per_copy = E * N * w_row
            master = torch.empty(per_copy, dtype=torch.uint8, device=dev)
            for e in range(E):
                We = torch.from_numpy(synth.expert_weights(e, N, K, cfg["sigma"],
                                                           seed=cfg["wseed"])).to(dev)
                rf.rfp2_quantize_weights(We, N, K, master[e * N * w_row:(e + 1) * N * w_row])
            if cfg["op"] == "moe":
                ids = torch.from_numpy(synth.routing(E, top_k)).to(dev)
            else:
                ids = torch.from_numpy(
                    synth.routing_tokens(E, top_k, M, cfg["share"]).reshape(-1)).to(dev)
        else:
            per_copy = N * w_row
            master = torch.empty(per_copy, dtype=torch.uint8, device=dev)
            rf.rfp2_quantize_weights(
                torch.from_numpy(synth.weights(N, K, cfg["sigma"], seed=cfg["wseed"])).to(dev),
                N, K, master)
        # consecutive steps read consecutive copies; a copy comes back only
        # after >= 1 GiB of the weight bytes the steps actually read
        copies = ring_slots(alg["weight_bytes"])
        footprint = copies * alg["weight_bytes"]
        if footprint < COLD_BYTES:
            raise RuntimeError(f"{workload}: ring footprint {footprint} B below 1 GiB")
        if copies * per_copy > MAX_COPY_BYTES:
            raise RuntimeError(f"{workload}: {copies} weight copies exceed the copy budget")
        bank = [master] + [master.clone() for _ in range(copies - 1)]
        a = torch.from_numpy(synth.activations(M, K)).to(dev)
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
        d = torch.empty((M, K // 32), dtype=torch.float32, device=dev)
        rows_out = {"moe": cfg.get("top_k"), "moe_tokens": M * cfg.get("top_k", 1),
                    "moe_gemm": M * cfg.get("top_k", 1)}.get(cfg["op"], M)
        ws = None
        if cfg["op"] == "moe_gemm":
            ws = torch.empty(rf.rfp2_moe_gemm_workspace_bytes(cfg["E"], M, cfg["top_k"]),
                             dtype=torch.uint8, device=dev)
        y = torch.empty((rows_out, N), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

        def product(i, st):
            w = bank[i % copies]
            if one and cfg["op"] == "moe":
                rf.rfp2_quant_moe_gemv(w, cfg["E"], N, K, ids, cfg["top_k"], a, q, d, y, None,
                                       st)
            elif one:
                rf.rfp2_quant_gemv(w, N, K, a, q, d, y, st)
            elif cfg["op"] == "moe":
                rf.rfp2_moe_gemv(w, cfg["E"], N, K, ids, cfg["top_k"], q, d, y, None, st)
            elif cfg["op"] == "moe_tokens" and per_token:
                tk = cfg["top_k"]
                for t in range(M):   # one single-token call per token
                    rf.rfp2_moe_gemv(w, cfg["E"], N, K, ids[t * tk:(t + 1) * tk], tk, q[t],
                                     d[t], y[t * tk:(t + 1) * tk], None, st)
            elif cfg["op"] == "moe_tokens":
                rf.rfp2_moe_gemv_tokens(w, cfg["E"], N, K, ids, M, cfg["top_k"], q, d, y,
                                        None, st)
            elif cfg["op"] == "moe_gemm":
                rf.rfp2_moe_gemm(w, cfg["E"], N, K, ids, M, cfg["top_k"], q, d, y, None, ws,
                                 st)
            elif cfg["op"] == "gemm":
                rf.rfp2_gemm(w, N, K, q, d, M, y, st)
            elif cfg["op"] == "gemm_f16":
                rf.rfp2_gemm_f16(w, N, K, q, d, M, y, st)
            else:
                rf.rfp2_gemv(w, N, K, q, d, M, y, st)

        def step(i, st):
            if not one:
                rf.rfp2_quantize_acts(a, M, K, q, d, st)
            product(i, st)

        # eager warm-up and the reference result of one step
        for i in range(warmup):
            step(i, stream)
        step(0, stream)
        torch.cuda.synchronize()
        y_eager = y.clone()

        # The timed loops are HIP graphs (timed_graph): LEAD untimed steps,
        # then exactly `steps` steps between two event-record nodes, step i on
        # copy i % copies, replayed after a cache flush, so neither the host's
        # launch cost nor the graph's start-up enters the figure and every step
        # reads its weights from HBM.
        g_step = timed_graph(step, steps, stream)
        g_prod = timed_graph(product, steps, stream)
        torch.cuda.synchronize()
        # a replay must reproduce the eager result exactly (all weight copies
        # are byte-identical)
        for _ in range(2):
            y.zero_()
            torch.cuda.synchronize()
            g_step[1].replay()
            torch.cuda.synchronize()
            if not torch.equal(y, y_eager):
                raise RuntimeError(f"{workload}: graph replay differs from the eager step")

        ms_step = replay_timed_us(g_step, steps, stream) * 1e-3
        # product kernel alone: events around back-to-back launches of it
        kern_ms = replay_timed_us(g_prod, steps, stream) * 1e-3
        if not torch.equal(y, y_eager):
            raise RuntimeError(f"{workload}: product graph result differs from the eager step")
        # context only: the same weights every launch, so they stay in the
        # caches (the last-level cache holds 256 MB) -- not an HBM figure
        warm_us = None
        isolated = None
        if cfg["op"] not in ("gemm", "gemm_f16", "moe_gemm"):
            warm_us = graph_time_us(lambda i, st: product(0, st), steps)
            isolated = isolated_cold_us(lambda st: product(0, st), stream)
        del g_step, g_prod, bank, master
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    khash = kernel_hash()
    kernel = {"moe": "rfp2_moe_gemv", "gemm": "rfp2_gemm", "gemm_f16": "rfp2_gemm_f16",
              "moe_tokens": f"{M} x rfp2_moe_gemv" if per_token else "rfp2_moe_gemv_tokens",
              "moe_gemm": "rfp2_moe_gemm (sort + grouped GEMM)",
              }.get(cfg["op"], "rfp2_gemv")
    if one:
        kernel = "rfp2_quant_moe_gemv" if cfg["op"] == "moe" else "rfp2_quant_gemv"
    if cfg["op"] in ("gemm", "gemm_f16", "moe_gemm"):
        value = alg["ops"] / (ms_step * 1e-3) / 1e12
        unit, metric = "TOPS", {
            "gemm": "ROCmFP2 M=512 GEMM int8 TOPS",
            "gemm_f16": "ROCmFP2 M=512 GEMM TOPS (int8 x ROCmFP2 product on fp16 matrix cores)",
            "moe_gemm": "ROCmFP2 prompt-batch MoE GEMM TOPS (int8 x ROCmFP2 product on fp16 "
                        "matrix cores)"}[cfg["op"]]
        achieved = alg["ops"] / (kern_ms * 1e-3) / 1e12
        # the contraction's own dtype sets the peak: int8 5.0 POP/s, fp16 2.5 PFLOP/s
        peak = I8_PEAK_TOPS if cfg["op"] == "gemm" else F16_PEAK_TFLOPS
        compute = {"bound": "mfma", "achieved": achieved, "peak": peak,
                   "unit": "TOPS" if cfg["op"] == "gemm" else "TFLOP/s",
                   "frac": achieved / peak}
        # the roofline's binding limit: ops per algorithmic byte against the
        # ridge point (peak ops / 8 TB/s).  The dense GEMMs (~1200 ops/B) sit
        # above it; the routed product, which reads every expert's weights
        # for ~32 tokens each (~185 ops/B), below it: HBM-bound
        intensity = alg["ops"] / alg["product_bytes"]
        ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
        if intensity >= ridge:
            roof = dict(compute)
        else:
            gbs = alg["product_bytes"] / (kern_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": gbs / HBM_PEAK_GBS, "compute": compute}
        roof.update(ops_per_byte=intensity, ridge_ops_per_byte=ridge)
    else:
        value = (alg["quant_bytes"] + alg["product_bytes"]) / (ms_step * 1e-3) / 1e9
        unit, metric = "GB/s", "ROCmFP2 GEMV effective HBM GB/s"
        achieved = alg["product_bytes"] / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS}
    roof.update(traffic=traffic_from_profiles(workload), kernel=kernel,
                kernel_us=kern_ms * 1e3, algorithmic_bytes=alg["product_bytes"],
                algorithmic_ops=alg["ops"])
    if warm_us is not None:
        roof["warm"] = {"kernel_us": warm_us, "GBps": alg["product_bytes"] / warm_us / 1e3,
                        "note": "same weights every launch: cache-resident, not HBM"}
    if isolated is not None:
        isolated["GBps"] = alg["product_bytes"] / isolated["median_us"] / 1e3
        roof["cold_isolated"] = isolated
    if roof["bound"] == "hbm":
        # what a plain read of the same bytes reaches: the product's bandwidth
        # is reported against it besides the HBM peak
        ceil = measure_ceiling(alg["product_bytes"], steps, isolated is not None)
        ceil["frac_of_ceiling"] = roof["achieved"] / ceil["GBps"]
        if isolated is not None:
            isolated["frac_of_ceiling"] = ceil["isolated_median_us"] / isolated["median_us"]
        roof["ceiling"] = ceil
    config = {"workload": workload, "M": M, "N": N, "K": K}
    if cfg["op"] in ("moe", "moe_tokens", "moe_gemm"):
        config.update(experts=cfg["E"], top_k=cfg["top_k"])
    if cfg["op"] in ("moe_tokens", "moe_gemm"):
        config.update(tokens=M, expert_share=cfg["share"])
    config.update(weight_copies=copies, weight_bytes_per_copy=per_copy,
                  weight_bytes_read_per_step=alg["weight_bytes"],
                  ring_footprint_bytes=footprint,
                  step=kernel if one else "rfp2_quantize_acts + " + kernel,
                  timed_graph=f"{LEAD} untimed + {steps} timed steps",
                  kernel_hash=khash)
    return {"metric": metric, "value": value, "unit": unit, "ms_per_step": ms_step,
            "steps": steps, "config": config, "roofline": roof, "cfg": cfg}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--secondary", default=",".join(SECONDARY),
                    help="comma-separated workloads also measured (empty: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-token", action="store_true",
                    help="multi-token MoE workloads as one single-token call per token")
    ap.add_argument("--quantizer", action="store_true",
                    help="also time the weight quantizers (plain and importance-weighted)")
    ap.add_argument("--two-launch", action="store_true",
                    help="one-token workloads as rfp2_quantize_acts + the product "
                         "(default: the single quantizing launch)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the product kernels run on a single MI355X; no multi-GPU path exists)",
              file=sys.stderr)
        return 2

    r = measure(args.workload, args.steps, args.warmup, args.two_launch, args.per_token)
    print(f"[bench] {args.workload} measured", file=sys.stderr, flush=True)
    out = {
        "metric": r["metric"], "value": r["value"], "unit": r["unit"], "n_gpus": 1,
        "steps": r["steps"], "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic", "config": r["config"],
        "roofline": r["roofline"],
    }
    secondary = []
    for wl in [w for w in args.secondary.split(",") if w and w != args.workload]:
        s = measure(wl, args.steps, args.warmup, args.two_launch, args.per_token)
        print(f"[bench] {wl} measured", file=sys.stderr, flush=True)
        secondary.append({"workload": wl, "metric": s["metric"], "value": s["value"],
                          "unit": s["unit"], "ms_per_step": s["ms_per_step"],
                          "roofline": {k: s["roofline"][k] for k in
                                       ("bound", "achieved", "peak", "unit", "frac",
                                        "kernel", "kernel_us", "traffic", "ceiling", "warm",
                                        "cold_isolated", "compute", "ops_per_byte",
                                        "ridge_ops_per_byte")
                                       if k in s["roofline"]}})
    if secondary:
        out["secondary"] = secondary
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(r["cfg"])
    if args.quantizer:
        out["weight_quantizer"] = measure_quantizer(args.workload)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
