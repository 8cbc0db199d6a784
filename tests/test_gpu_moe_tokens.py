"""GPU parity of rfp2_moe_gemv_tokens (routed experts for several tokens,
each expert's rows expanded once for every token routed to it) against the
oracle: row s of y is expert ids[s] applied to token s / top_k."""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, assert_within_bound, device, empty, host, sample_rows, to_dev, torch
from test_gpu_decode import random_blocks

pytestmark = pytest.mark.gpu


def run_tokens(bank, E, N, K, ids, q, d):
    T, top_k = ids.shape
    y = empty((T * top_k, N), torch.float32)
    y.fill_(12345.0)
    err = torch.zeros(1, dtype=torch.int32, device=y.device)
    rf.rfp2_moe_gemv_tokens(to_dev(bank.reshape(-1)), E, N, K, to_dev(ids.reshape(-1)), T,
                            top_k, to_dev(q), to_dev(d), y, err)
    return host(y), int(host(err)[0])


def check_rows(y, bank, E, N, K, ids, q, d):
    T, top_k = ids.shape
    refs = {}                   # expert -> (oracle products, |w a| sums) for every token
    for t in range(T):
        for j in range(top_k):
            s, e = t * top_k + j, int(ids[t, j])
            if not 0 <= e < E:
                assert np.isnan(y[s]).all(), f"slot {s}: bad id {e} not NaN"
                continue
            if e not in refs:
                refs[e] = (oracle.ref_gemv(bank[e], N, K, q, d),
                           oracle.abs_product_sums(bank[e], N, K, q, d))
            assert_within_bound(y[s], refs[e][0][t], refs[e][1][t],
                                f"token {t} slot {j} expert {e}")


def make_ids(kind, E, T, top_k, rng):
    if kind == "independent":
        return np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    if kind == "shared":
        return np.tile(rng.choice(E, top_k, replace=False), (T, 1)).astype(np.int32)
    if kind == "duplicates":
        return rng.integers(0, 3, (T, top_k)).astype(np.int32)
    if kind == "one_expert":
        return np.full((T, top_k), 4, np.int32)
    ids = rng.integers(0, E, (T, top_k)).astype(np.int32)     # with bad ids
    ids[0, 0] = E
    ids[-1, -1] = -3
    return ids


# (8, 8, 4096): four groups per lane, 70 KB of LDS; (8, 4, 8192): 100 KB, the
# direct loads land above 64 KB; (8, 2, 16384): 7 tokens then 1 (the one-token
# kernel); (5, 2, 32768): chunks of 3 and 2 tokens
@pytest.mark.parametrize("T,top_k,K", [(2, 3, 1024), (3, 8, 2048), (4, 8, 4096),
                                       (8, 8, 1024), (5, 1, 512), (8, 8, 4096),
                                       (8, 4, 8192), (8, 2, 16384), (5, 2, 32768)])
@pytest.mark.parametrize("kind", ["independent", "shared", "duplicates", "one_expert", "bad"])
def test_moe_tokens_against_oracle(T, top_k, K, kind):
    announce("moe_tokens", T, top_k, K, kind)
    E, N = 10, 300
    rng = np.random.default_rng(T * 100 + top_k + K)
    bank = np.stack([random_blocks(N, K, seed=7 * e + K, scale_hi=0x28) for e in range(E)])
    ids = make_ids(kind, E, T, top_k, rng)
    q, d = oracle.quantize_acts(synth.activations(T, K, seed=T + K))
    y, err = run_tokens(bank, E, N, K, ids, q, d)
    assert err == (1 if ((ids < 0) | (ids >= E)).any() else 0)
    check_rows(y, bank, E, N, K, ids, q, d)


def test_moe_tokens_single_token_is_moe_gemv():
    announce("moe_tokens T=1")
    E, N, K, top_k = 6, 200, 2048, 4
    bank = np.stack([random_blocks(N, K, seed=50 + e, scale_hi=0x28) for e in range(E)])
    ids = np.array([[3, 0, 3, 5]], np.int32)
    q, d = oracle.quantize_acts(synth.activations(1, K))
    y1, _ = run_tokens(bank, E, N, K, ids, q, d)
    y2 = empty((top_k, N), torch.float32)
    rf.rfp2_moe_gemv(to_dev(bank.reshape(-1)), E, N, K, to_dev(ids[0]), top_k, to_dev(q),
                     to_dev(d), y2)
    assert np.array_equal(y1.view(np.uint32), host(y2).view(np.uint32))


def test_moe_tokens_shape_limits():
    device()
    E, N, K = 2, 8, 256
    w = empty(E * N * K // 32 * 10, torch.uint8)
    ids = torch.zeros(72, dtype=torch.int32, device=w.device)
    q, d = empty((9, K), torch.int8), empty((9, K // 32), torch.float32)
    y = empty((72 * N,), torch.float32)
    with pytest.raises(rf.Rfp2Error):       # T * top_k above 64
        rf.rfp2_moe_gemv_tokens(w, E, N, K, ids, 8, 9, q, d, y)
    with pytest.raises(rf.Rfp2Error):       # T above 8
        rf.rfp2_moe_gemv_tokens(w, E, N, K, ids, 9, 1, q, d, y)


def test_moe_tokens_full_size_sampled_rows():
    # 128 experts of 1536x4096, 4 consecutive tokens, top-8, half of each
    # token's experts kept from the token before
    cfg = synth.WORKLOADS["moe_128x1536x4096_top8"]
    E, N, K, top_k, T = cfg["E"], cfg["N"], cfg["K"], cfg["top_k"], 4
    dev = device()
    announce("moe_tokens full", E, N, K, top_k, T)
    ids = synth.routing_tokens(E, top_k, T, 0.5)
    rb = N * K // 32 * 10
    bank = torch.empty(E * rb, dtype=torch.uint8, device=dev)
    bank.random_(0, 0x7F)
    weights = {}
    for e in sorted(set(ids.reshape(-1).tolist())):
        weights[e] = synth.expert_weights(e, N, K, cfg["sigma"], seed=cfg["wseed"])
        rf.rfp2_quantize_weights(to_dev(weights[e]), N, K, bank[e * rb:(e + 1) * rb])
    a = synth.activations(T, K)
    q_g, d_g = empty((T, K), torch.int8), empty((T, K // 32), torch.float32)
    rf.rfp2_quantize_acts(to_dev(a), T, K, q_g, d_g)
    y_g = empty((T * top_k, N), torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    rf.rfp2_moe_gemv_tokens(bank, E, N, K, to_dev(ids.reshape(-1)), T, top_k, q_g, d_g, y_g, err)
    y = host(y_g)
    assert int(host(err)[0]) == 0
    q, d = oracle.quantize_acts(a)
    rows = sample_rows(N, 12, seed=14)
    for t in range(T):
        for j in range(top_k):
            e = int(ids[t, j])
            packed_rows = oracle.quantize_weights(weights[e][rows])
            assert_within_bound(y[t * top_k + j, rows],
                                oracle.ref_gemv(packed_rows, len(rows), K, q[t:t + 1],
                                                d[t:t + 1])[0],
                                oracle.abs_product_sums(packed_rows, len(rows), K, q[t:t + 1],
                                                        d[t:t + 1])[0],
                                f"token {t} expert {e}")
