"""GPU test of rfp2_moe_gemm_noalloc (the allocation-free form of the
prompt-batch routed-expert product): through the C ABI, two calls in a row
(the second with a smaller batch and fewer experts) must give exactly what
rfp2_moe_gemm gives on the same inputs, and both are held to the fp32 bound
against the oracle."""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, assert_within_bound, empty, host, to_dev, torch
from test_gpu_decode import random_blocks

pytestmark = pytest.mark.gpu


def _case(E, N, K, T, top_k, seed):
    rng = np.random.default_rng(seed)
    bank = np.stack([random_blocks(N, K, seed=seed + e, scale_hi=0x7E) for e in range(E)])
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[T // 2, 0] = E                                  # one bad id: NaN row, err set
    q, d = oracle.quantize_acts(synth.activations(T, K, seed=seed + 1))
    return bank, ids, q, d


def _run(fn, bank, E, N, K, ids, T, top_k, q, d, **kw):
    y = empty((T * top_k, N), torch.float32)
    y.fill_(-3.0)
    err = torch.zeros(1, dtype=torch.int32, device=y.device)
    fn(to_dev(bank.reshape(-1)), E, N, K, to_dev(ids), T, top_k, to_dev(q), to_dev(d), y,
       err, **kw)
    return host(y), int(host(err)[0])


@pytest.mark.parametrize("first,second", [((12, 256, 1024, 96, 4), (5, 128, 512, 10, 2)),
                                          ((128, 192, 2048, 512, 8), (64, 192, 2048, 37, 8))])
def test_noalloc_matches_workspace_form_on_two_calls(first, second):
    for i, (E, N, K, T, top_k) in enumerate((first, second)):
        announce("moe_gemm_noalloc call", i, E, N, K, T, top_k)
        bank, ids, q, d = _case(E, N, K, T, top_k, seed=100 * i + E)
        y_ws, err_ws = _run(rf.rfp2_moe_gemm, bank, E, N, K, ids, T, top_k, q, d)
        y_na, err_na = _run(rf.rfp2_moe_gemm_noalloc, bank, E, N, K, ids, T, top_k, q, d)
        assert err_ws == err_na == 1
        assert np.array_equal(y_ws.view(np.uint32), y_na.view(np.uint32))
        ref = oracle.ref_moe_batch(bank.reshape(-1), E, N, K, ids, q, d)
        ok = ~np.isnan(ref[:, 0])
        assert np.isnan(y_na[~ok]).all()
        rows = np.flatnonzero(ok)[:: max(1, ok.sum() // 64)]
        absum = np.stack([oracle.abs_product_sums(bank[ids.reshape(-1)[s]], N, K,
                                                  q[s // top_k:s // top_k + 1],
                                                  d[s // top_k:s // top_k + 1])[0]
                          for s in rows])
        assert_within_bound(y_na[rows], ref[rows], absum, f"moe_gemm_noalloc call {i}")


def test_noalloc_refuses_sizes_beyond_its_array():
    announce("moe_gemm_noalloc size limit")
    E, N, K, top_k = 128, 64, 256, 8
    T = 32736                                   # 261,888 slots: 8 bytes over 1 MiB
    assert rf.rfp2_moe_gemm_workspace_bytes(E, T, top_k) > rf.MOE_GEMM_NOALLOC_MAX_BYTES
    assert rf.rfp2_moe_gemm_workspace_bytes(E, T - 1, top_k) <= rf.MOE_GEMM_NOALLOC_MAX_BYTES
    w = empty(E * N * K // 32 * 10, torch.uint8)
    ids = torch.zeros(T * top_k, dtype=torch.int32, device=w.device)
    q, d = empty((T, K), torch.int8), empty((T, K // 32), torch.float32)
    y = empty((T * top_k, N), torch.float32)    # full size: nothing may be written anyway
    st = rf.lib().rfp2_moe_gemm_noalloc(w.data_ptr(), E, N, K, ids.data_ptr(), T, top_k,
                                        q.data_ptr(), d.data_ptr(), y.data_ptr(), None,
                                        torch.cuda.current_stream().cuda_stream)
    assert st == rf.RFP2_E_SHAPE
