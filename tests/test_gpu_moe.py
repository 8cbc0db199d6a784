"""GPU parity of rfp2_moe_gemv (routed experts, one token) against the oracle."""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, assert_within_bound, device, empty, host, sample_rows, to_dev, torch
from test_gpu_decode import random_blocks

pytestmark = pytest.mark.gpu


def run_moe(bank, E, N, K, ids, q, d, with_err=True):
    top_k = len(ids)
    y = empty((top_k, N), torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device=y.device) if with_err else None
    rf.rfp2_moe_gemv(to_dev(bank.reshape(-1)), E, N, K, to_dev(np.asarray(ids, np.int32)),
                     top_k, to_dev(q), to_dev(d), y, err)
    return host(y), (int(host(err)[0]) if with_err else None)


def small_bank(E, N, K, seed):
    return np.stack([random_blocks(N, K, seed=seed + e, scale_hi=0x28) for e in range(E)])


@pytest.mark.parametrize("ids", [[5, 0, 5, 2], [3], [0, 1, 2, 3, 4, 5, 0, 1]])
def test_moe_rows_follow_ids(ids):
    announce("moe small", ids)
    E, N, K = 6, 300, 1024
    bank = small_bank(E, N, K, seed=40)
    q, d = oracle.quantize_acts(synth.activations(1, K))
    y, err = run_moe(bank, E, N, K, ids, q, d)
    assert err == 0
    ref = oracle.ref_moe_gemv(bank.reshape(-1), E, N, K, ids, q, d)
    for j, e in enumerate(ids):
        assert_within_bound(y[j], ref[j], oracle.abs_product_sums(bank[e], N, K, q, d)[0],
                            f"slot {j} expert {e}")


def test_moe_bad_ids_give_nan_rows_and_flag():
    announce("moe bad ids")
    E, N, K = 6, 100, 512
    bank = small_bank(E, N, K, seed=70)
    q, d = oracle.quantize_acts(synth.activations(1, K))
    ids = [1, 7, -1, 3, 2 ** 31 - 1]
    y, err = run_moe(bank, E, N, K, ids, q, d)
    assert err == 1
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all() and np.isnan(y[4]).all()
    for j in (0, 3):
        e = ids[j]
        assert_within_bound(y[j], oracle.ref_gemv(bank[e], N, K, q, d)[0],
                            oracle.abs_product_sums(bank[e], N, K, q, d)[0], f"slot {j}")
    y2, _ = run_moe(bank, E, N, K, [0, 9], q, d, with_err=False)   # no flag buffer
    assert np.isnan(y2[1]).all() and np.isfinite(y2[0]).all()


def test_moe_full_size_sampled_rows():
    # 128 experts of 1536x4096, top-8 routing: the routed experts are drawn
    # from the workload's generator and quantized on the GPU; the others hold
    # random blocks (they are never read).
    cfg = synth.WORKLOADS["moe_128x1536x4096_top8"]
    E, N, K, top_k = cfg["E"], cfg["N"], cfg["K"], cfg["top_k"]
    dev = device()
    announce("moe full", E, N, K, top_k)
    ids = synth.routing(E, top_k)
    rb = N * K // 32 * 10
    bank = torch.empty(E * rb, dtype=torch.uint8, device=dev)
    bank.random_(0, 0x7F)
    weights = {}
    for e in ids.tolist():
        weights[e] = synth.expert_weights(e, N, K, cfg["sigma"], seed=cfg["wseed"])
        rf.rfp2_quantize_weights(to_dev(weights[e]), N, K, bank[e * rb:(e + 1) * rb])
    a = synth.activations(1, K)
    q_g = empty((1, K), torch.int8)
    d_g = empty((1, K // 32), torch.float32)
    rf.rfp2_quantize_acts(to_dev(a), 1, K, q_g, d_g)
    y_g = empty((top_k, N), torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    rf.rfp2_moe_gemv(bank, E, N, K, to_dev(ids), top_k, q_g, d_g, y_g, err)
    y = host(y_g)
    assert int(host(err)[0]) == 0
    q, d = oracle.quantize_acts(a)
    rows = sample_rows(N, 16, seed=13)
    bank_h = host(bank).reshape(E, N, rb // N)
    for j, e in enumerate(ids.tolist()):
        packed_rows = oracle.quantize_weights(weights[e][rows])
        assert np.array_equal(bank_h[e][rows], packed_rows)
        assert_within_bound(y[j, rows], oracle.ref_gemv(packed_rows, len(rows), K, q, d)[0],
                            oracle.abs_product_sums(packed_rows, len(rows), K, q, d)[0],
                            f"expert {e}")
