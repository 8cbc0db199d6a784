"""HBM traffic per launch of the products' kernels, from rocprofv3 counters.

Runs on a GPU machine with rocprofv3.  For each workload, bench.py runs twice
under `rocprofv3 --pmc`, once with FETCH_SIZE and once with WRITE_SIZE (each
pass its own run: one TCC counter group per pass).  The product kernel is
the kernel of the step with the most dispatches; its per-dispatch counter
values (summed over the counter's instances) are medianed.  Counter KiB are
scaled to bytes by what the same counters read, in the same runs, for the HIP
runtime's plain device-to-device copy kernel of known size (the bench's
weight copies); the scale of the largest copies over all runs is used.

Each workload's entry records the hash of the sources of its kernels (the
GEMV kernels, the routed prompt-batch product or a dense GEMM); an existing
OUT_JSON keeps its other workloads' entries.

usage: python -m bit_gemv_amd.hbm_counters OUT_JSON WORKLOAD [WORKLOAD ...]
"""
from __future__ import annotations

import json
import os
import shutil
import sqlite3
import statistics
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def bench_cmd(workload: str) -> list[str]:
    return [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", workload,
            "--secondary", "", "--no-cpu-baseline", "--steps", "32", "--warmup", "1"]


def run_pass(workload: str, counter: str, out_dir: str) -> str:
    cmd = ["timeout", "-s", "KILL", "240", "rocprofv3", "--pmc", counter, "-d", out_dir, "-o",
           "run", "--"] + bench_cmd(workload)
    print("[counters]", workload, counter, flush=True)
    subprocess.run(cmd, check=True, cwd="/tmp", stdout=subprocess.DEVNULL,
                   env=dict(os.environ, TMPDIR="/tmp"))
    for dirpath, _, files in os.walk(out_dir):
        for f in files:
            if f.endswith("_results.db"):
                return os.path.join(dirpath, f)
    raise RuntimeError(f"no results database under {out_dir}")


def per_dispatch(db: str, counter: str):
    con = sqlite3.connect(db)
    cur = con.cursor()
    names = {did: n for did, n in cur.execute("select dispatch_id, name from kernels")}
    vals = {}
    for did, v in cur.execute(
            "select dispatch_id, counter_value from pmc_events where counter_name = ?", (counter,)):
        vals[did] = vals.get(did, 0.0) + v
    con.close()
    out = {}
    for did, v in vals.items():
        out.setdefault(names[did], []).append(v)
    return out


def main(argv):
    out_json, workloads = argv[0], argv[1:]
    import bench
    import synth
    res, copies = {}, []
    for wl in workloads:
        cfg = dict(synth.workload(wl), name=wl)
        alg = bench.algorithmic(cfg, bench.fused(cfg))
        per_copy = cfg.get("E", 1) * cfg["N"] * cfg["K"] // 32 * 10
        got = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            tmp = tempfile.mkdtemp(prefix="pmc_", dir="/tmp")
            try:
                got[counter] = per_dispatch(run_pass(wl, counter, tmp), counter)
            finally:
                shutil.rmtree(tmp, ignore_errors=True)
        prods = {n: v for n, v in got["FETCH_SIZE"].items()
                 if any(k in n for k in ("gemv_kernel", "gemm_kernel", "gemm_f16_kernel"))}
        kernel = max(prods, key=lambda n: len(prods[n]))
        fetch = statistics.median(got["FETCH_SIZE"][kernel])
        write = statistics.median(got["WRITE_SIZE"][kernel])
        for n, v in got["FETCH_SIZE"].items():
            if "copyBuffer" in n:
                big = [x for x in v if x > 0.9 * max(v)]
                wv = [x for x in got["WRITE_SIZE"].get(n, []) if x > 0.9 * max(got["WRITE_SIZE"][n])]
                copies.append((per_copy, statistics.median(big), statistics.median(wv)))
        sources = {"moe_gemm": bench.MOE_GEMM_SOURCES, "gemm": bench.GEMM_SOURCES,
                   "gemm_f16": bench.GEMM_F16_SOURCES}.get(cfg["op"], bench.GEMV_SOURCES)
        res[wl] = {"kernel": kernel, "dispatches": len(got["FETCH_SIZE"][kernel]),
                   "fetch_kib_median": fetch, "write_kib_median": write,
                   "algorithmic_bytes_per_launch": alg["product_bytes"],
                   "kernel_hash": bench.kernel_hash(sources), "hash_sources": sources}
    nbytes, f_copy, w_copy = max(copies)
    rf, wf = nbytes / 1024 / f_copy, nbytes / 1024 / w_copy
    for wl, r in res.items():
        rd = round(r["fetch_kib_median"] * 1024 * rf)
        wr = round(r["write_kib_median"] * 1024 * wf)
        r.update(hbm_read_bytes_per_launch=rd, hbm_write_bytes_per_launch=wr,
                 hbm_bytes_per_launch=rd + wr,
                 ratio_to_algorithmic=(rd + wr) / r["algorithmic_bytes_per_launch"],
                 read_factor=rf, write_factor=wf)
    try:
        with open(out_json) as f:
            kept = json.load(f).get("workloads", {})
    except (OSError, ValueError):
        kept = {}
    res = {**kept, **res}
    out = {"copy_calibration": {"kernel": "__amd_rocclr_copyBuffer", "bytes": nbytes,
                                "fetch_kib": f_copy, "write_kib": w_copy,
                                "read_factor": rf, "write_factor": wf},
           "kernel_hash": bench.kernel_hash(bench.GEMV_SOURCES),
           "hash_sources": bench.GEMV_SOURCES, "workloads": res,
           "commands": [f"rocprofv3 --pmc {c} -d <out> -o run -- python3 -u <repo>/bench.py "
                        "--workload <workload> --secondary \"\" --no-cpu-baseline --steps 32 "
                        "--warmup 1" for c in ("FETCH_SIZE", "WRITE_SIZE")]}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({wl: round(r["ratio_to_algorithmic"], 4) for wl, r in res.items()}))


if __name__ == "__main__":
    main(sys.argv[1:])
