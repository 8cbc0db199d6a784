"""Host-side checks of bench.py (no GPU): it refuses more than one GPU, and
its algorithmic byte and op counts are the ones the workloads' definitions
give (the weight payload of every row read at 10 bytes per 32 weights, plus
q, d, ids and y), worked out here from the shapes by hand."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def product_bytes(name):
    cfg = dict(synth.WORKLOADS[name], name=name)
    return bench.algorithmic(cfg, one_launch=False)


def test_gemv_bytes():
    # 512 rows of 2048: 512*64 blocks*10 B + q 2048 + d 64*4 + y 512*4
    assert product_bytes("gemv_512x2048")["product_bytes"] == 327_680 + 2_048 + 256 + 2_048
    assert product_bytes("gemv_4096x4096")["product_bytes"] == 5_242_880 + 4_096 + 512 + 16_384
    assert product_bytes("gemv_16384x5120")["product_bytes"] == \
        26_214_400 + 5_120 + 640 + 65_536
    # four tokens on the same matrix: q, d and y four times
    assert product_bytes("gemv_16384x5120_m4")["product_bytes"] == \
        26_214_400 + 20_480 + 2_560 + 262_144


def test_moe_bytes_count_the_routed_experts_and_ids():
    # 8 routed experts of 1536x4096 (1,966,080 B each), q, d, 8 ids, 8 rows of y
    b = product_bytes("moe_128x1536x4096_top8")
    assert b["product_bytes"] == 8 * 1_966_080 + 4_096 + 512 + 32 + 8 * 1536 * 4
    assert b["ops"] == 2 * 8 * 1536 * 4096


def test_gemm_ops_and_bytes():
    b = product_bytes("gemm_512x14336x4096")
    assert b["ops"] == 60_129_542_144                 # 2 * 512 * 14336 * 4096
    assert b["product_bytes"] == 18_350_080 + 2_097_152 + 262_144 + 29_360_128


def test_one_launch_adds_the_fp32_activations_and_the_written_q_d():
    cfg = dict(synth.WORKLOADS["gemv_16384x5120"], name="gemv_16384x5120")
    one = bench.algorithmic(cfg, one_launch=True)
    # weights and y, fp32 a read, q and d written
    assert one["product_bytes"] == 26_214_400 + 65_536 + 4 * 5120 + 5120 + 4 * 160
    assert one["quant_bytes"] == 0


def test_any_dense_gemv_shape_is_a_workload():
    import pytest
    assert synth.workload("gemv_16384x5120") is synth.WORKLOADS["gemv_16384x5120"]
    cfg = synth.workload("gemv_8192x4096")
    assert (cfg["op"], cfg["M"], cfg["N"], cfg["K"]) == ("gemv", 1, 8192, 4096)
    assert synth.workload("gemv_8192x4096_m4")["M"] == 4
    # 8192 rows of 4096: 8192 * 128 blocks * 10 B + q + d + y
    b = bench.algorithmic(dict(cfg, name="gemv_8192x4096"), one_launch=False)
    assert b["product_bytes"] == 10_485_760 + 4_096 + 512 + 32_768
    for bad in ("gemm_8x8", "gemv_8192", "gemv_8x8_x2"):
        with pytest.raises(KeyError):
            synth.workload(bad)


def test_every_timed_loop_reads_a_gib_before_reusing_a_weight_copy():
    # consecutive steps read consecutive weight copies; there are enough
    # copies that >= 1 GiB of the bytes the steps actually read (the routed
    # experts only, for MoE) passes before a copy comes back
    for wl in [bench.DEFAULT_WORKLOAD] + bench.SECONDARY:
        cfg = dict(synth.workload(wl), name=wl)
        alg = bench.algorithmic(cfg, bench.fused(cfg))
        copies = bench.ring_slots(alg["weight_bytes"])
        assert copies >= 2 and copies * alg["weight_bytes"] >= bench.COLD_BYTES, wl
        per_copy = cfg.get("E", 1) * cfg["N"] * cfg["K"] // 32 * 10
        assert copies * per_copy <= bench.MAX_COPY_BYTES, wl
    one = dict(synth.WORKLOADS["moe_128x1536x4096_top8"], name="moe")
    assert bench.algorithmic(one, True)["weight_bytes"] == 8 * 1_966_080
