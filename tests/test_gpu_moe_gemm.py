"""GPU parity of the prompt-batch routed-expert path: rfp2_moe_sort (slots
grouped by expert, bit-exact against the oracle's stable grouping) and
rfp2_moe_gemm (each slot's row against the oracle within the fp32 bound,
and bit for bit against rfp2_gemm_f16 applied to the slot's expert: an
output does not depend on which other tokens share its tile)."""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, assert_within_bound, device, empty, host, sample_rows, to_dev, torch
from test_gpu_decode import random_blocks

pytestmark = pytest.mark.gpu


def gpu_sort(ids, E):
    S = ids.size
    offsets = empty(E + 1, torch.int32)
    order = empty(max(S, 1), torch.int32)
    order.fill_(-7)
    err = torch.zeros(1, dtype=torch.int32, device=offsets.device)
    rf.rfp2_moe_sort(to_dev(ids.reshape(-1).astype(np.int32)), S, E, offsets, order, err)
    off = host(offsets)
    return off, host(order)[:off[-1]], int(host(err)[0])


def routing(kind, E, T, top_k, rng):
    if kind == "uniform":       # top_k distinct experts per token
        return np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    if kind == "skewed":        # most slots on expert 1: several tiles of one expert
        ids = rng.integers(0, E, (T, top_k))
        ids[rng.random((T, top_k)) < 0.7] = 1
        return ids.astype(np.int32)
    if kind == "duplicates":    # repeated experts inside a token
        return rng.integers(0, 2, (T, top_k)).astype(np.int32)
    ids = rng.integers(0, E, (T, top_k)).astype(np.int32)      # "bad"
    ids[0, 0] = E
    ids[T // 2, -1] = -1
    ids[-1, 0] = 1 << 30
    return ids


@pytest.mark.parametrize("S,E,kind", [(1, 1, "uniform"), (120, 6, "uniform"),
                                      (4096, 128, "uniform"), (5000, 2048, "uniform"),
                                      (3000, 16, "skewed"), (70000, 64, "uniform"), (16384, 256, "uniform"),
                                      (16385, 256, "uniform"),
                                      (999, 10, "bad")])
def test_moe_sort_matches_oracle(S, E, kind):
    announce("moe_sort", S, E, kind)
    rng = np.random.default_rng(S + E)
    if kind == "uniform":
        ids = rng.integers(0, E, S)
    elif kind == "skewed":
        ids = np.where(rng.random(S) < 0.8, 3, rng.integers(0, E, S))
    else:
        ids = rng.integers(-2, E + 2, S)
    ids = ids.astype(np.int32)
    off, order, err = gpu_sort(ids, E)
    off_ref, order_ref = oracle.sort_by_expert(ids, E)
    assert np.array_equal(off, off_ref)
    assert np.array_equal(order, order_ref)
    assert err == int(((ids < 0) | (ids >= E)).any())


def run_moe_gemm(bank, E, N, K, ids, q, d, workspace=None):
    T, top_k = ids.shape
    y = empty((T * top_k, N), torch.float32)
    y.fill_(12345.0)
    err = torch.zeros(1, dtype=torch.int32, device=y.device)
    w = bank if isinstance(bank, torch.Tensor) else to_dev(bank.reshape(-1))
    rf.rfp2_moe_gemm(w, E, N, K, to_dev(ids.reshape(-1)), T, top_k,
                     q if isinstance(q, torch.Tensor) else to_dev(q),
                     d if isinstance(d, torch.Tensor) else to_dev(d), y, err, workspace)
    return y, int(host(err)[0])


def dense_rows(w_e, N, K, q_g, d_g, T):
    """rfp2_gemm_f16 of one expert over all T tokens (GPU tensor [T, N])."""
    y = empty((T, N), torch.float32)
    rf.rfp2_gemm_f16(w_e, N, K, q_g, d_g, T, y)
    return y


@pytest.mark.parametrize("T,top_k,K", [(40, 3, 512), (200, 2, 1024), (7, 8, 2048),
                                       (130, 1, 256)])
@pytest.mark.parametrize("kind", ["uniform", "skewed", "duplicates", "bad"])
def test_moe_gemm_against_oracle_and_dense(T, top_k, K, kind):
    announce("moe_gemm", T, top_k, K, kind)
    E, N = 8, 300                       # 300 rows: a ragged last row tile
    if kind == "uniform" and top_k > E:
        pytest.skip("top_k distinct experts need E >= top_k")
    rng = np.random.default_rng(T * 10 + top_k + K)
    bank = np.stack([random_blocks(N, K, seed=11 * e + K, scale_hi=0x28) for e in range(E)])
    ids = routing(kind, E, T, top_k, rng)
    q, d = oracle.quantize_acts(synth.activations(T, K, seed=T + K))
    y_g, err = run_moe_gemm(bank, E, N, K, ids, q, d)
    y = host(y_g)
    bad = (ids < 0) | (ids >= E)
    assert err == int(bad.any())
    q_g, d_g = to_dev(q), to_dev(d)
    flat = ids.reshape(-1)
    for e in range(E):
        slots = np.flatnonzero(flat == e)
        if slots.size == 0:
            continue
        ref = oracle.ref_gemv(bank[e], N, K, q, d)
        absum = oracle.abs_product_sums(bank[e], N, K, q, d)
        toks = slots // top_k
        assert_within_bound(y[slots], ref[toks], absum[toks], f"expert {e}")
        dense = host(dense_rows(to_dev(bank[e].reshape(-1)), N, K, q_g, d_g, T))
        assert np.array_equal(y[slots].view(np.uint32), dense[toks].view(np.uint32)), \
            f"expert {e}: routed rows differ from the dense product"
    assert np.isnan(y[np.flatnonzero(bad.reshape(-1))]).all()


@pytest.mark.parametrize("E,T,top_k,K,N", [(2048, 4096, 2, 256, 130),   # long sort chunks
                                          (40, 300, 2, 16384, 200),      # 64 stages of K
                                          # tiles of more than 32 slots started first:
                                          # 2 .. 4 groups of 64 experts, then the
                                          # first expert count that keeps the sort's order
                                          (130, 1200, 4, 512, 200),
                                          (256, 2048, 8, 256, 130),
                                          (257, 1024, 4, 256, 130)])
def test_moe_gemm_large_shapes_against_dense(E, T, top_k, K, N):
    # every routed row bit for bit against rfp2_gemm_f16 of its expert, and
    # sampled rows against the oracle
    announce("moe_gemm large", E, T, top_k, K, N)
    dev = device()
    rng = np.random.default_rng(E + T + K)
    ids = rng.integers(0, E, (T, top_k)).astype(np.int32)
    ids[rng.random((T, top_k)) < 0.3] = 5                  # one crowded expert
    rb = N * (K // 32) * 10
    bank = torch.randint(0, 0x28, (E * rb,), dtype=torch.uint8, device=dev)
    q, d = oracle.quantize_acts(synth.activations(T, K, seed=E))
    q_g, d_g = to_dev(q), to_dev(d)
    y_g, err = run_moe_gemm(bank, E, N, K, ids, q_g, d_g)
    assert err == 0
    flat = ids.reshape(-1)
    bank_h = None
    for e in sorted(set(flat.tolist())):
        slots = np.flatnonzero(flat == e)
        toks = slots // top_k
        dense = dense_rows(bank[e * rb:(e + 1) * rb], N, K, q_g, d_g, T)
        assert torch.equal(y_g[torch.from_numpy(slots).to(dev)],
                           dense[torch.from_numpy(toks).to(dev)]), f"expert {e}"
        if e == 5 or e == int(flat[0]):
            if bank_h is None:
                bank_h = host(bank).reshape(E, N, -1)
            rows = sample_rows(N, 6, seed=e)
            y = host(y_g)
            ref = oracle.ref_gemv(bank_h[e][rows], len(rows), K, q[toks], d[toks])
            absum = oracle.abs_product_sums(bank_h[e][rows], len(rows), K, q[toks], d[toks])
            assert_within_bound(y[np.ix_(slots, rows)], ref, absum, f"expert {e}")


def test_moe_gemm_workspace_and_limits():
    device()
    E, N, K, T, top_k = 4, 64, 256, 10, 2
    need = rf.rfp2_moe_gemm_workspace_bytes(E, T, top_k)
    assert need >= 4 * (2 * (E + 1) + T * top_k) and need % 256 == 0
    assert rf.rfp2_moe_gemm_workspace_bytes(4096, T, top_k) == 0      # E above 2048
    w = empty(E * N * K // 32 * 10, torch.uint8)
    ids = torch.zeros(T * top_k, dtype=torch.int32, device=w.device)
    q, d = empty((T, K), torch.int8), empty((T, K // 32), torch.float32)
    y = empty((T * top_k, N), torch.float32)
    small = empty(need - 256, torch.uint8)
    with pytest.raises(ValueError):                 # the binding sees the short buffer
        rf.rfp2_moe_gemm(w, E, N, K, ids, T, top_k, q, d, y, None, small)
    big = empty(need, torch.uint8)                  # the library checks the byte count
    assert rf.lib().rfp2_moe_gemm(w.data_ptr(), E, N, K, ids.data_ptr(), T, top_k,
                                  q.data_ptr(), d.data_ptr(), y.data_ptr(), None,
                                  big.data_ptr(), need - 4, None) == rf.RFP2_E_SHAPE
    with pytest.raises(rf.Rfp2Error):
        rf.rfp2_moe_sort(ids, T * top_k, 3000, empty(3001, torch.int32),
                         empty(T * top_k, torch.int32))


def test_moe_gemm_graph_replays_match_eager():
    announce("moe_gemm graph")
    E, N, K, T, top_k = 8, 256, 1024, 64, 4
    rng = np.random.default_rng(3)
    bank = to_dev(np.stack([random_blocks(N, K, seed=300 + e, scale_hi=0x28)
                            for e in range(E)]).reshape(-1))
    ids = to_dev(routing("uniform", E, T, top_k, rng).reshape(-1))
    q, d = oracle.quantize_acts(synth.activations(T, K, seed=8))
    q, d = to_dev(q), to_dev(d)
    ws = empty(rf.rfp2_moe_gemm_workspace_bytes(E, T, top_k), torch.uint8)
    y = empty((T * top_k, N), torch.float32)
    torch.cuda.synchronize()          # the inputs were written on the default stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        rf.rfp2_moe_gemm(bank, E, N, K, ids, T, top_k, q, d, y, None, ws, s)
        torch.cuda.synchronize()
        y_eager = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            rf.rfp2_moe_gemm(bank, E, N, K, ids, T, top_k, q, d, y, None, ws, s)
        for _ in range(3):
            y.zero_()
            ws.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, y_eager)


def test_moe_gemm_full_size():
    # 128 experts of 1536x4096, a 512-token prompt, top-8 routing (uniform,
    # without replacement per token); every expert quantized on the GPU from
    # the workload's generator
    cfg = synth.WORKLOADS["moe_128x1536x4096_top8"]
    E, N, K, top_k, T = cfg["E"], cfg["N"], cfg["K"], cfg["top_k"], 512
    dev = device()
    announce("moe_gemm full", E, N, K, top_k, T)
    rng = np.random.default_rng(2)
    ids = routing("uniform", E, T, top_k, rng)
    rb = N * K // 32 * 10
    bank = torch.empty(E * rb, dtype=torch.uint8, device=dev)
    rows = sample_rows(N, 6, seed=15)
    packed_rows = {}
    for e in range(E):
        W = synth.expert_weights(e, N, K, cfg["sigma"], seed=cfg["wseed"])
        rf.rfp2_quantize_weights(to_dev(W), N, K, bank[e * rb:(e + 1) * rb])
        packed_rows[e] = oracle.quantize_weights(W[rows])
    a = synth.activations(T, K)
    q_g, d_g = empty((T, K), torch.int8), empty((T, K // 32), torch.float32)
    rf.rfp2_quantize_acts(to_dev(a), T, K, q_g, d_g)
    y_g, err = run_moe_gemm(bank, E, N, K, ids, q_g, d_g)
    assert err == 0
    q, d = oracle.quantize_acts(a)
    assert np.array_equal(host(q_g), q)
    y = host(y_g)
    flat = ids.reshape(-1)
    for e in range(E):
        slots = np.flatnonzero(flat == e)
        toks = slots // top_k
        dense = dense_rows(bank[e * rb:(e + 1) * rb], N, K, q_g, d_g, T)
        assert torch.equal(y_g[torch.from_numpy(slots).to(dev)],
                           dense[torch.from_numpy(toks).to(dev)]), f"expert {e}"
        ref = oracle.ref_gemv(packed_rows[e], len(rows), K, q[toks], d[toks])
        absum = oracle.abs_product_sums(packed_rows[e], len(rows), K, q[toks], d[toks])
        assert_within_bound(y[np.ix_(slots, rows)], ref, absum, f"expert {e}")
