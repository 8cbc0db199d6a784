"""Python binding of librfp2 (ROCmFP2 GEMV / GEMM for MI355X).

Argument marshalling only: every function here has the name and argument
order of the C entry point declared in include/rfp2.h, takes torch tensors
that live on the GPU, checks that each tensor has the dtype, layout and size
the call will touch (so that no kernel reads or writes outside a buffer), and
passes raw device pointers plus the current HIP stream to the library.  All
computation happens in the library's HIP kernels; there is no fallback path:
if librfp2.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librfp2.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "rfp2.h")

RFP2_OK, RFP2_E_NULL, RFP2_E_SHAPE, RFP2_E_ALIGN, RFP2_E_LAUNCH = 0, -1, -2, -3, -4
GEMV_MAX_M = 8

_lib = None

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p
_SIGNATURES = {
    "rfp2_abi_version": ([], ctypes.c_int),
    "rfp2_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "rfp2_quantize_acts": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p], ctypes.c_int),
    "rfp2_quantize_weights": ([_c_p, _c_i64, _c_i64, _c_p, _c_p], ctypes.c_int),
    "rfp2_quantize_weights_imatrix": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p], ctypes.c_int),
    "rfp2_gemv": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_p], ctypes.c_int),
    "rfp2_gemm": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_p], ctypes.c_int),
    "rfp2_gemm_f16": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_p], ctypes.c_int),
    "rfp2_moe_gemv": ([_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p, _c_p,
                       _c_p, _c_p], ctypes.c_int),
    "rfp2_moe_gemv_tokens": ([_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_i64, _c_i64, _c_p, _c_p,
                              _c_p, _c_p, _c_p], ctypes.c_int),
    "rfp2_moe_sort": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p], ctypes.c_int),
    "rfp2_moe_gemm_workspace_bytes": ([_c_i64, _c_i64, _c_i64], ctypes.c_size_t),
    "rfp2_moe_gemm": ([_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p,
                       _c_p, _c_p, ctypes.c_size_t, _c_p], ctypes.c_int),
    "rfp2_moe_gemm_noalloc": ([_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_i64, _c_i64, _c_p, _c_p,
                               _c_p, _c_p, _c_p], ctypes.c_int),
    "rfp2_read_ceiling": ([_c_p, _c_i64, ctypes.c_uint32, _c_p, _c_p], ctypes.c_int),
    "rfp2_quant_gemv": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p], ctypes.c_int),
    "rfp2_quant_moe_gemv": ([_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p, _c_p,
                             _c_p, _c_p, _c_p], ctypes.c_int),
    "rfp2_debug_decode": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p], ctypes.c_int),
    "rfp2_debug_half_dots": ([_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p], ctypes.c_int),
    "rfp2_debug_half_sums_mf": ([_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p], ctypes.c_int),
    "rfp2_debug_decode_f16": ([_c_p, _c_i64, _c_i64, ctypes.c_int, _c_p, _c_p], ctypes.c_int),
    "rfp2_debug_decode_i8": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p], ctypes.c_int),
}


class Rfp2Error(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call}: status {status}: {rfp2_status_string(status)}")


def lib() -> ctypes.CDLL:
    """The loaded librfp2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import "
                "__graft_entry__ as g; g.build()'` (ROCm hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Names of the functions declared in include/rfp2.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(rfp2_\w+)\s*\(", text, re.M)))


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t, dtype, numel: int, name: str):
    """Device pointer of `t` after checking what the call will touch."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {numel}")
    return t.data_ptr()


def _check(call: str, status: int):
    if status != RFP2_OK:
        raise Rfp2Error(call, status)


def _blocks(K: int) -> int:
    return K // 32


# ---------------------------------------------------------------------------
# entry points (same names and argument order as the C ABI)
# ---------------------------------------------------------------------------
def rfp2_abi_version() -> int:
    return lib().rfp2_abi_version()


def rfp2_status_string(status: int) -> str:
    return lib().rfp2_status_string(int(status)).decode()


def rfp2_quantize_acts(a, M: int, K: int, q, d, stream=None) -> None:
    import torch
    _check("rfp2_quantize_acts", lib().rfp2_quantize_acts(
        _ptr(a, torch.float32, M * K, "a"), M, K, _ptr(q, torch.int8, M * K, "q"),
        _ptr(d, torch.float32, M * _blocks(K), "d"), _stream(stream)))


def rfp2_quantize_weights(x, N: int, K: int, w, stream=None) -> None:
    import torch
    _check("rfp2_quantize_weights", lib().rfp2_quantize_weights(
        _ptr(x, torch.float32, N * K, "x"), N, K,
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), _stream(stream)))


def rfp2_quantize_weights_imatrix(x, N: int, K: int, importance, w, stream=None) -> None:
    import torch
    _check("rfp2_quantize_weights_imatrix", lib().rfp2_quantize_weights_imatrix(
        _ptr(x, torch.float32, N * K, "x"), N, K,
        _ptr(importance, torch.float32, K, "importance"),
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), _stream(stream)))


def rfp2_gemv(w, N: int, K: int, q, d, M: int, y, stream=None) -> None:
    import torch
    _check("rfp2_gemv", lib().rfp2_gemv(
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), N, K,
        _ptr(q, torch.int8, M * K, "q"), _ptr(d, torch.float32, M * _blocks(K), "d"), M,
        _ptr(y, torch.float32, M * N, "y"), _stream(stream)))


def rfp2_gemm(w, N: int, K: int, q, d, M: int, y, stream=None) -> None:
    import torch
    _check("rfp2_gemm", lib().rfp2_gemm(
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), N, K,
        _ptr(q, torch.int8, M * K, "q"), _ptr(d, torch.float32, M * _blocks(K), "d"), M,
        _ptr(y, torch.float32, M * N, "y"), _stream(stream)))


def rfp2_gemm_f16(w, N: int, K: int, q, d, M: int, y, stream=None) -> None:
    import torch
    _check("rfp2_gemm_f16", lib().rfp2_gemm_f16(
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), N, K,
        _ptr(q, torch.int8, M * K, "q"), _ptr(d, torch.float32, M * _blocks(K), "d"), M,
        _ptr(y, torch.float32, M * N, "y"), _stream(stream)))


def rfp2_moe_gemv(w, E: int, N: int, K: int, ids, top_k: int, q, d, y, err=None,
                  stream=None) -> None:
    import torch
    errp = None if err is None else _ptr(err, torch.int32, 1, "err")
    _check("rfp2_moe_gemv", lib().rfp2_moe_gemv(
        _ptr(w, torch.uint8, E * N * _blocks(K) * 10, "w"), E, N, K,
        _ptr(ids, torch.int32, top_k, "ids"), top_k,
        _ptr(q, torch.int8, K, "q"), _ptr(d, torch.float32, _blocks(K), "d"),
        _ptr(y, torch.float32, top_k * N, "y"), errp, _stream(stream)))


def rfp2_moe_gemv_tokens(w, E: int, N: int, K: int, ids, T: int, top_k: int, q, d, y,
                         err=None, stream=None) -> None:
    import torch
    errp = None if err is None else _ptr(err, torch.int32, 1, "err")
    _check("rfp2_moe_gemv_tokens", lib().rfp2_moe_gemv_tokens(
        _ptr(w, torch.uint8, E * N * _blocks(K) * 10, "w"), E, N, K,
        _ptr(ids, torch.int32, T * top_k, "ids"), T, top_k,
        _ptr(q, torch.int8, T * K, "q"), _ptr(d, torch.float32, T * _blocks(K), "d"),
        _ptr(y, torch.float32, T * top_k * N, "y"), errp, _stream(stream)))


def rfp2_moe_sort(ids, S: int, E: int, offsets, order, err=None, stream=None) -> None:
    import torch
    errp = None if err is None else _ptr(err, torch.int32, 1, "err")
    _check("rfp2_moe_sort", lib().rfp2_moe_sort(
        _ptr(ids, torch.int32, S, "ids"), S, E, _ptr(offsets, torch.int32, E + 1, "offsets"),
        _ptr(order, torch.int32, S, "order"), errp, _stream(stream)))


def rfp2_moe_gemm_workspace_bytes(E: int, T: int, top_k: int) -> int:
    return int(lib().rfp2_moe_gemm_workspace_bytes(E, T, top_k))


def rfp2_moe_gemm(w, E: int, N: int, K: int, ids, T: int, top_k: int, q, d, y, err=None,
                  workspace=None, stream=None) -> None:
    """workspace: a uint8 GPU tensor of at least rfp2_moe_gemm_workspace_bytes
    bytes; when None, one is allocated for this call."""
    import torch
    need = rfp2_moe_gemm_workspace_bytes(E, T, top_k)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=y.device)
    errp = None if err is None else _ptr(err, torch.int32, 1, "err")
    _check("rfp2_moe_gemm", lib().rfp2_moe_gemm(
        _ptr(w, torch.uint8, E * N * _blocks(K) * 10, "w"), E, N, K,
        _ptr(ids, torch.int32, T * top_k, "ids"), T, top_k,
        _ptr(q, torch.int8, T * K, "q"), _ptr(d, torch.float32, T * _blocks(K), "d"),
        _ptr(y, torch.float32, T * top_k * N, "y"), errp,
        _ptr(workspace, torch.uint8, need, "workspace"), workspace.numel(), _stream(stream)))


READ_CEILING_OUTPUTS = 524288


MOE_GEMM_NOALLOC_MAX_BYTES = 1 << 20


def rfp2_moe_gemm_noalloc(w, E: int, N: int, K: int, ids, T: int, top_k: int, q, d, y,
                          err=None, stream=None) -> None:
    import torch
    errp = None if err is None else _ptr(err, torch.int32, 1, "err")
    _check("rfp2_moe_gemm_noalloc", lib().rfp2_moe_gemm_noalloc(
        _ptr(w, torch.uint8, E * N * _blocks(K) * 10, "w"), E, N, K,
        _ptr(ids, torch.int32, T * top_k, "ids"), T, top_k,
        _ptr(q, torch.int8, T * K, "q"), _ptr(d, torch.float32, T * _blocks(K), "d"),
        _ptr(y, torch.float32, T * top_k * N, "y"), errp, _stream(stream)))


def read_ceiling_threads(nbytes: int) -> int:
    """Threads of the read helper's grid for nbytes (256 per workgroup)."""
    return 256 * min(2048, max(1, -(-(nbytes // 16) // 256)))


def rfp2_read_ceiling(buf, nbytes: int, out, magic: int = 0x9E3779B9, stream=None) -> None:
    """Measurement helper: read nbytes of buf with plain 16-byte loads; a
    thread whose XOR of what it read equals `magic` writes it to out[thread]."""
    import torch
    _check("rfp2_read_ceiling", lib().rfp2_read_ceiling(
        _ptr(buf, torch.uint8, nbytes, "buf"), nbytes, int(magic) & 0xFFFFFFFF,
        _ptr(out, torch.int32, read_ceiling_threads(nbytes), "out"), _stream(stream)))


def rfp2_quant_gemv(w, N: int, K: int, a, q, d, y, stream=None) -> None:
    import torch
    _check("rfp2_quant_gemv", lib().rfp2_quant_gemv(
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), N, K,
        _ptr(a, torch.float32, K, "a"), _ptr(q, torch.int8, K, "q"),
        _ptr(d, torch.float32, _blocks(K), "d"), _ptr(y, torch.float32, N, "y"),
        _stream(stream)))


def rfp2_quant_moe_gemv(w, E: int, N: int, K: int, ids, top_k: int, a, q, d, y, err=None,
                        stream=None) -> None:
    import torch
    errp = None if err is None else _ptr(err, torch.int32, 1, "err")
    _check("rfp2_quant_moe_gemv", lib().rfp2_quant_moe_gemv(
        _ptr(w, torch.uint8, E * N * _blocks(K) * 10, "w"), E, N, K,
        _ptr(ids, torch.int32, top_k, "ids"), top_k,
        _ptr(a, torch.float32, K, "a"), _ptr(q, torch.int8, K, "q"),
        _ptr(d, torch.float32, _blocks(K), "d"),
        _ptr(y, torch.float32, top_k * N, "y"), errp, _stream(stream)))


def rfp2_debug_decode(w, N: int, K: int, codes_out, scales_out, stream=None) -> None:
    import torch
    _check("rfp2_debug_decode", lib().rfp2_debug_decode(
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), N, K,
        _ptr(codes_out, torch.int8, N * K, "codes_out"),
        _ptr(scales_out, torch.float32, N * K // 16, "scales_out"), _stream(stream)))


def rfp2_debug_half_dots(w, N: int, K: int, q, M: int, sums_out, stream=None) -> None:
    import torch
    _check("rfp2_debug_half_dots", lib().rfp2_debug_half_dots(
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), N, K,
        _ptr(q, torch.int8, M * K, "q"), M,
        _ptr(sums_out, torch.int32, M * N * _blocks(K) * 2, "sums_out"), _stream(stream)))


def rfp2_debug_half_sums_mf(w, N: int, K: int, q, M: int, sums_out, stream=None) -> None:
    import torch
    _check("rfp2_debug_half_sums_mf", lib().rfp2_debug_half_sums_mf(
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), N, K,
        _ptr(q, torch.int8, M * K, "q"), M,
        _ptr(sums_out, torch.int32, M * N * _blocks(K) * 2, "sums_out"), _stream(stream)))


def rfp2_debug_decode_f16(w, N: int, K: int, form: int, h_out, stream=None) -> None:
    """h_out: int16 tensor [N, K] receiving IEEE half-precision bit patterns."""
    import torch
    _check("rfp2_debug_decode_f16", lib().rfp2_debug_decode_f16(
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), N, K, int(form),
        _ptr(h_out, torch.int16, N * K, "h_out"), _stream(stream)))


def rfp2_debug_decode_i8(w, N: int, K: int, wa_out, wb_out, scales_out, stream=None) -> None:
    """wa_out, wb_out: int8 [N, K]; scales_out: fp32 [N, K/32, 6]."""
    import torch
    _check("rfp2_debug_decode_i8", lib().rfp2_debug_decode_i8(
        _ptr(w, torch.uint8, N * _blocks(K) * 10, "w"), N, K,
        _ptr(wa_out, torch.int8, N * K, "wa_out"),
        _ptr(wb_out, torch.int8, N * K, "wb_out"),
        _ptr(scales_out, torch.float32, N * _blocks(K) * 6, "scales_out"), _stream(stream)))
