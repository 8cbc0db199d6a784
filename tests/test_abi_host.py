"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/rfp2.h declares, and
reject bad arguments with the documented status before touching the GPU.
"""
import pytest

import bit_gemv_amd as rf


def test_library_exports_every_declared_symbol():
    L = rf.lib()
    names = rf.header_symbols()
    assert set(names) == set(rf._SIGNATURES)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert rf.rfp2_abi_version() == 1
    assert rf.rfp2_status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert rf.rfp2_status_string(s) != "unknown status"
    assert rf.rfp2_status_string(-99) == "unknown status"


P = 0x10000          # an aligned fake device address: never dereferenced
MIS = P + 2          # misaligned for 16-byte arguments


def _gemv(w=P, N=4, K=256, q=P, d=P, M=1, y=P):
    return rf.lib().rfp2_gemv(w, N, K, q, d, M, y, None)


def test_gemv_argument_checks():
    assert _gemv(w=None) == rf.RFP2_E_NULL
    assert _gemv(y=None) == rf.RFP2_E_NULL
    assert _gemv(K=288) == rf.RFP2_E_SHAPE        # K % 256 != 0
    assert _gemv(K=0) == rf.RFP2_E_SHAPE
    assert _gemv(K=32768 + 256) == rf.RFP2_E_SHAPE
    assert _gemv(M=0) == rf.RFP2_E_SHAPE
    assert _gemv(M=9) == rf.RFP2_E_SHAPE
    assert _gemv(N=0) == rf.RFP2_E_SHAPE
    assert _gemv(w=MIS) == rf.RFP2_E_ALIGN
    assert _gemv(q=MIS) == rf.RFP2_E_ALIGN
    assert _gemv(d=P + 1) == rf.RFP2_E_ALIGN


def test_gemm_moe_quantize_argument_checks():
    L = rf.lib()
    assert L.rfp2_gemm(P, 4, 256, P, P, 0, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_gemm(P, 4, 100, P, P, 4, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_gemm(P, 4, 256, MIS, P, 4, P, None) == rf.RFP2_E_ALIGN
    assert L.rfp2_moe_gemv(P, 8, 4, 256, None, 2, P, P, P, None, None) == rf.RFP2_E_NULL
    assert L.rfp2_moe_gemv(P, 0, 4, 256, P, 2, P, P, P, None, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_moe_gemv(P, 8, 4, 256, P, 0, P, P, P, None, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_moe_gemv(P, 8, 4, 256, P, 2, P, P, P, P + 1, None) == rf.RFP2_E_ALIGN
    assert L.rfp2_quantize_acts(P, 1, 48, P, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_quantize_acts(P + 4, 1, 64, P, P, None) == rf.RFP2_E_ALIGN
    assert L.rfp2_quantize_acts(None, 1, 64, P, P, None) == rf.RFP2_E_NULL
    assert L.rfp2_quantize_weights(P, 1, 40, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_quantize_weights(P, 1, 64, P + 1, None) == rf.RFP2_E_ALIGN
    assert L.rfp2_debug_decode(P, 1, 33, P, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_debug_half_dots(P, 1, 64, P, 0, P, None) == rf.RFP2_E_SHAPE
    # M * N * (K/32) beyond 2^40 half-sum pairs is refused before any launch
    assert L.rfp2_debug_half_dots(P, 1 << 20, 1 << 20, P, 1 << 20, P, None) == rf.RFP2_E_SHAPE
    # the matrix-core half sums: whole 8-block groups per row only
    assert L.rfp2_debug_half_sums_mf(P, 1, 64, P, 1, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_debug_half_sums_mf(P, 1, 288, P, 1, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_debug_half_sums_mf(P, 1, 256, P, 0, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_debug_half_sums_mf(P, 1 << 20, 1 << 20, P, 1 << 20, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_debug_half_sums_mf(P, 1, 256, P, 1, None, None) == rf.RFP2_E_NULL
    assert L.rfp2_debug_half_sums_mf(P, 1, 256, P + 2, 1, P, None) == rf.RFP2_E_ALIGN
    assert L.rfp2_debug_decode_f16(P, 1, 64, 2, P, None) == rf.RFP2_E_SHAPE    # form 0 or 1
    assert L.rfp2_debug_decode_f16(P, 1, 48, 0, P, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_debug_decode_f16(P, 1, 64, 1, None, None) == rf.RFP2_E_NULL
    assert L.rfp2_debug_decode_f16(P + 1, 1, 64, 1, P, None) == rf.RFP2_E_ALIGN


def test_moe_sort_and_moe_gemm_argument_checks():
    L = rf.lib()
    assert L.rfp2_moe_sort(None, 10, 4, P, P, None, None) == rf.RFP2_E_NULL
    assert L.rfp2_moe_sort(P, 0, 4, P, P, None, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_moe_sort(P, 10, 0, P, P, None, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_moe_sort(P, 10, 2049, P, P, None, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_moe_sort(P, (1 << 24) + 1, 4, P, P, None, None) == rf.RFP2_E_SHAPE
    assert L.rfp2_moe_sort(P, 10, 4, P + 2, P, None, None) == rf.RFP2_E_ALIGN
    need = L.rfp2_moe_gemm_workspace_bytes(8, 512, 8)
    assert need >= 4 * (2 * 9 + 4096) and need % 256 == 0
    assert L.rfp2_moe_gemm_workspace_bytes(0, 1, 1) == 0
    assert L.rfp2_moe_gemm_workspace_bytes(2049, 1, 1) == 0
    assert L.rfp2_moe_gemm_workspace_bytes(8, 1 << 20, 17) == 0      # above 2^24 slots

    def gemm(E=8, N=64, K=256, T=512, top_k=8, ws=P, ws_bytes=need, q=P, err=None):
        return L.rfp2_moe_gemm(P, E, N, K, P, T, top_k, q, P, P, err, ws, ws_bytes, None)
    assert gemm(ws=None) == rf.RFP2_E_NULL
    assert gemm(ws_bytes=need - 4) == rf.RFP2_E_SHAPE
    assert gemm(K=320) == rf.RFP2_E_SHAPE
    assert gemm(N=0) == rf.RFP2_E_SHAPE
    assert gemm(E=4096) == rf.RFP2_E_SHAPE
    assert gemm(ws=P + 64) == rf.RFP2_E_ALIGN                  # workspace: 256 bytes
    assert gemm(q=MIS) == rf.RFP2_E_ALIGN
    assert gemm(err=P + 1) == rf.RFP2_E_ALIGN

    # the allocation-free form: the same checks, and no batch whose sorted
    # slots exceed its 1 MiB array (refused before any HIP call)
    def noalloc(E=8, N=64, K=256, T=512, top_k=8, ids=P, q=P):
        return L.rfp2_moe_gemm_noalloc(P, E, N, K, ids, T, top_k, q, P, P, None, None)
    assert noalloc(ids=None) == rf.RFP2_E_NULL
    assert noalloc(K=320) == rf.RFP2_E_SHAPE
    assert noalloc(E=2049) == rf.RFP2_E_SHAPE
    assert noalloc(E=128, T=32736) == rf.RFP2_E_SHAPE        # 261,888 slots: over 1 MiB
    assert L.rfp2_moe_gemm_workspace_bytes(128, 32735, 8) <= rf.MOE_GEMM_NOALLOC_MAX_BYTES
    assert noalloc(q=MIS) == rf.RFP2_E_ALIGN


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        rf._ptr(x, torch.uint8, 16, "w")
    with pytest.raises(TypeError):
        rf._ptr(x.numpy(), torch.uint8, 16, "w")
