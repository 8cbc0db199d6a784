"""Plain fp64 / exact-integer statement of the ROCmFP2 format and its products.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow on purpose: every
step is written the way the page states it, with numpy used only to repeat a
step over many blocks at once.  No blocking, fusion or reordering beyond what
the definitions say.

Source: "ROCmFP2 codebook research report" (llm.ciru.ai, 2026-07-13).

Readings taken where the page is silent (each one is also listed with its
reason in the design notes of the repository):

R1  The scale search tests all 127 legal bytes, in the order start, start-1,
    start+1, start-2, start+2, ...; a candidate replaces the best so far only
    when its squared error is strictly lower.  The result is therefore the
    global minimum; ties go to the candidate visited first.
R2  "Start near max|x|/4" = the legal byte whose scale is nearest to
    max|x|/4, the lower byte on a tie (above 224 this is 0x7E).
R3  The inner/outer decision compares |x| <= 2.5*s (no division), so an
    exact midpoint is inner and x = 0 at s = 0 is inner.
R4  The sign rule sends x < 0 to the negative side; +0 and -0 go to +1.
R5  Byte 0x00 is legal and decodes to 0.0.  Bytes 0x7F..0xFF are invalid.
R6  The squared error of a candidate is summed in fp64 over the 16 values in
    index order: e = x - xhat; sse = sse + e*e, one rounding per operation.
R7  Activations: per 32-element block, amax = max|a|, d = fl32(amax/127)
    (IEEE fp32 division), q = clamp(round_half_away(fl32(a/d)), -127, 127).
    When d == 0 (amax == 0, or amax so small that amax/127 underflows)
    every q of the block is 0.  Non-finite activations are rejected.
R8  Rows are stored back to back, each row being K/32 blocks back to back.
R14 Importance-weighted search ("05 · Completed experiment"): the error of a
    candidate is sum_i w_i * (x_i - xhat_i)^2 with w_i = importance of the
    value's input channel * sqrt(sigma^2 + x_i^2).  The page leaves sigma
    undefined; here sigma^2 is the mean of x^2 over the 16-value half being
    searched (the unit the search works on).  Each term is w * (e*e), summed
    in index order, every step rounded once; the weights are computed once
    per half (x*x summed in index order, /16, + x_i*x_i, sqrt, * importance).
    The codes stay the nearest levels (a positive weight does not move a
    value's nearest level); only the winning scale changes.  All-zero
    importance makes every candidate score 0: the start byte wins.
"""
from __future__ import annotations

import numpy as np

# "02 · Quantization", codebook table: code 00 -> -4 (negative outer),
# 01 -> -1 (negative inner), 10 -> +1 (positive inner), 11 -> +4 (positive
# outer).  Four signed levels, no zero.
CODEBOOK = (-4, -1, 1, 4)
_CB = np.array(CODEBOOK, dtype=np.int64)

# "02 · Quantization", "One scale byte, 127 legal values": 0x00..0x7E.
UE4M3_MAX_BYTE = 0x7E

BLOCK_WEIGHTS = 32      # "01 · Storage": a block covers 32 weights
HALF_WEIGHTS = 16       # ... split into two 16-weight halves, one scale each
BLOCK_BYTES = 10        # 8 code bytes + 2 scale bytes


def row_bytes(K: int) -> int:
    """Bytes of one stored row of K weights ("01 · Storage": 10 B / 32)."""
    if K % BLOCK_WEIGHTS:
        raise ValueError("K must be a multiple of 32")
    return K // BLOCK_WEIGHTS * BLOCK_BYTES


def matrix_bytes(N: int, K: int) -> int:
    return N * row_bytes(K)


# --------------------------------------------------------------------------
# UE4M3 scale byte  ("02 · Quantization", "One scale byte, 127 legal values")
# --------------------------------------------------------------------------
def ue4m3_decode(b: int) -> float:
    """Decode one UE4M3 scale byte exactly.

    E = b >> 3, M = b & 7; E == 0 gives M * 2^-10, E > 0 gives
    (8 + M) * 2^(E - 11).  Only 0x00..0x7E are legal; anything else raises.
    """
    b = int(b)
    if b < 0 or b > UE4M3_MAX_BYTE:
        raise ValueError(f"illegal UE4M3 scale byte 0x{b:02X}")
    E = b >> 3
    M = b & 7
    if E == 0:
        return M * 2.0 ** -10
    return (8 + M) * 2.0 ** (E - 11)


def ue4m3_table() -> np.ndarray:
    """fp64 scale of every legal byte, indexed by the byte (127 entries)."""
    return np.array([ue4m3_decode(b) for b in range(UE4M3_MAX_BYTE + 1)],
                    dtype=np.float64)


# --------------------------------------------------------------------------
# Selector rule  ("02 · Quantization", codebook table and midpoint rule)
# --------------------------------------------------------------------------
def select_code(x: float, s: float) -> int:
    """Code (0..3) of one weight x at scale s.

    Sign picks the side; |x/s| <= 2.5 picks the inner level (1), else the
    outer level (4).  Compared as |x| <= 2.5*s (R3, R4).
    """
    outer = abs(x) > 2.5 * s
    if x < 0:
        return 0 if outer else 1
    return 3 if outer else 2


def _select_codes(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """`select_code` applied elementwise (x and s broadcast together)."""
    outer = np.abs(x) > 2.5 * s
    neg = x < 0
    return np.where(neg, np.where(outer, 0, 1), np.where(outer, 3, 2))


# --------------------------------------------------------------------------
# Block packing  ("01 · Storage", serialized layout)
# --------------------------------------------------------------------------
def pack_block(codes, e0: int, e1: int) -> bytes:
    """32 codes + two scale bytes -> 10 stored bytes.

    Byte j (0..7) holds weights 4j..4j+3, weight 4j+i in bits 2i..2i+1
    (four 2-bit selectors packed little-endian).  Byte 8 = e0 (weights
    0..15), byte 9 = e1 (weights 16..31).
    """
    codes = [int(c) for c in codes]
    if len(codes) != BLOCK_WEIGHTS or any(c < 0 or c > 3 for c in codes):
        raise ValueError("a block needs 32 codes in 0..3")
    out = bytearray(BLOCK_BYTES)
    for j in range(8):
        v = 0
        for i in range(4):
            v |= codes[4 * j + i] << (2 * i)
        out[j] = v
    out[8] = int(e0) & 0xFF
    out[9] = int(e1) & 0xFF
    return bytes(out)


def unpack_block(blk: bytes):
    """Inverse of `pack_block`: 10 bytes -> (codes[32], e0, e1)."""
    if len(blk) != BLOCK_BYTES:
        raise ValueError("a block is 10 bytes")
    codes = []
    for j in range(8):
        for i in range(4):
            codes.append((blk[j] >> (2 * i)) & 3)
    return codes, blk[8], blk[9]


def pack_matrix(codes: np.ndarray, ebytes: np.ndarray) -> np.ndarray:
    """codes uint8 [N,K] (0..3) + scale bytes uint8 [N,K/16] -> uint8 [N, 10K/32].

    The same layout as `pack_block`, block after block along each row (R8).
    """
    codes = np.asarray(codes, dtype=np.int64)
    N, K = codes.shape
    B = K // BLOCK_WEIGHTS
    c = codes.reshape(N, B, 8, 4)
    qbytes = (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6))
    e = np.asarray(ebytes, dtype=np.int64).reshape(N, B, 2)
    blocks = np.concatenate([qbytes, e], axis=2)          # [N, B, 10]
    return blocks.reshape(N, B * BLOCK_BYTES).astype(np.uint8)


def unpack_matrix(packed: np.ndarray, N: int, K: int):
    """Inverse of `pack_matrix`: -> (codes uint8 [N,K], ebytes uint8 [N,K/16])."""
    B = K // BLOCK_WEIGHTS
    blocks = np.asarray(packed, dtype=np.int64).reshape(N, B, BLOCK_BYTES)
    q = blocks[..., :8]
    c = np.stack([(q >> (2 * i)) & 3 for i in range(4)], axis=-1)  # [N,B,8,4]
    codes = c.reshape(N, K).astype(np.uint8)
    ebytes = blocks[..., 8:10].reshape(N, 2 * B).astype(np.uint8)
    return codes, ebytes


# --------------------------------------------------------------------------
# Per-half scale search  ("02 · Quantization", how a block is chosen)
# --------------------------------------------------------------------------
def start_byte(amax: np.ndarray) -> np.ndarray:
    """Byte whose scale is nearest to max|x|/4; the lower byte on a tie (R2)."""
    table = ue4m3_table()
    target = np.asarray(amax, dtype=np.float64) / 4.0
    dist = np.abs(table[None, :] - target.reshape(-1, 1))
    return np.argmin(dist, axis=1).astype(np.int64).reshape(np.shape(amax))


def _visit_offsets():
    """0, -1, +1, -2, +2, ..., -126, +126: the search order around the start."""
    yield 0
    for k in range(1, UE4M3_MAX_BYTE + 1):
        yield -k
        yield k


def importance_weights(X: np.ndarray, IMP: np.ndarray) -> np.ndarray:
    """Per-value weights of the importance-weighted objective ("05 · Completed
    experiment": importance_i * sqrt(sigma^2 + x_i^2)), fp64 [H,16].

    X: fp64 [H,16] halves; IMP: fp64 [H,16] importance of each value's input
    channel.  sigma^2 is the mean of x^2 over the half (R14), summed in index
    order; every step rounds once (x*x, sum, /16, +, sqrt, *)."""
    s2 = np.zeros(X.shape[0])
    for i in range(HALF_WEIGHTS):
        s2 = s2 + X[:, i] * X[:, i]
    sigma2 = s2 / 16.0
    return IMP * np.sqrt(sigma2[:, None] + X * X)


def _search_halves(X: np.ndarray, WT: np.ndarray | None = None):
    """Scale search on H halves at once.  X: fp64 [H,16].  WT: per-value
    weights of the objective (None: the plain squared error).
    -> (bytes, codes)."""
    H = X.shape[0]
    table = ue4m3_table()
    start = start_byte(np.abs(X).max(axis=1))
    best_sse = np.full(H, np.inf)
    best_b = start.copy()
    for off in _visit_offsets():
        b = start + off
        legal = (b >= 0) & (b <= UE4M3_MAX_BYTE)
        if not legal.any():
            continue
        s = table[np.clip(b, 0, UE4M3_MAX_BYTE)][:, None]
        xhat = _CB[_select_codes(X, s)] * s              # map all 16 values
        sse = np.zeros(H)
        for i in range(HALF_WEIGHTS):                      # R6: index order
            e = X[:, i] - xhat[:, i]
            t = e * e
            if WT is not None:
                t = WT[:, i] * t                           # weighted: w * (e*e)
            sse = sse + t
        better = legal & (sse < best_sse)                  # R1: strictly lower
        best_sse[better] = sse[better]
        best_b[better] = b[better]
    codes = _select_codes(X, table[best_b][:, None])
    return best_b.astype(np.uint8), codes.astype(np.uint8)


def _check_importance(imp, K: int) -> np.ndarray:
    imp = np.asarray(imp)
    if imp.dtype != np.float32 or imp.shape != (K,):
        raise TypeError(f"importance must be float32 [{K}]")
    if not (np.isfinite(imp).all() and (imp >= 0).all()):
        raise ValueError("importance must be finite and >= 0")
    return imp.astype(np.float64)


def quantize_half(x, importance=None) -> tuple[int, list[int]]:
    """Choose the scale byte and the 16 codes of one 16-weight half; with an
    importance vector (fp32 [16], >= 0) the error is the weighted one."""
    X = np.asarray(x, dtype=np.float32).astype(np.float64).reshape(1, HALF_WEIGHTS)
    if not np.isfinite(X).all():
        raise ValueError("non-finite weight")
    WT = None
    if importance is not None:
        IMP = _check_importance(importance, HALF_WEIGHTS).reshape(1, HALF_WEIGHTS)
        WT = importance_weights(X, IMP)
    b, c = _search_halves(X, WT)
    return int(b[0]), [int(v) for v in c[0]]


def quantize_weights(W: np.ndarray, importance=None) -> np.ndarray:
    """fp32 [N,K] -> packed ROCmFP2 bytes [N, 10K/32] (scale search per half).

    importance: None (plain squared error, "02 · Quantization") or fp32 [K],
    finite and >= 0, the importance of each input channel (column); the
    search then minimises the weighted error of "05 · Completed experiment".
    The codes are the nearest levels either way; only the scale choice
    changes."""
    W = np.asarray(W)
    if W.dtype != np.float32:
        raise TypeError("weights must be float32")
    N, K = W.shape
    row_bytes(K)
    X = W.astype(np.float64).reshape(-1, HALF_WEIGHTS)
    if not np.isfinite(X).all():
        raise ValueError("non-finite weight")
    WT = None
    if importance is not None:
        imp = _check_importance(importance, K)
        IMP = np.broadcast_to(imp.reshape(1, K), (N, K)).reshape(-1, HALF_WEIGHTS)
        WT = importance_weights(X, IMP)
    ebytes, codes = _search_halves(X, WT)
    return pack_matrix(codes.reshape(N, K), ebytes.reshape(N, K // HALF_WEIGHTS))


def dequantize_weights(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Reconstructed weights codebook[code] * scale, exact, fp64 [N,K]."""
    codes, ebytes = unpack_matrix(packed, N, K)
    if (ebytes > UE4M3_MAX_BYTE).any():
        raise ValueError("illegal UE4M3 scale byte in the matrix")
    scales = ue4m3_table()[ebytes]                       # [N, K/16]
    return (_CB[codes].reshape(N, K // HALF_WEIGHTS, HALF_WEIGHTS)
            * scales[:, :, None]).reshape(N, K)


def decoded_int8(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """The signed int8 lanes a code byte expands to ("03 · Runtime"), [N,K]."""
    codes, _ = unpack_matrix(packed, N, K)
    return _CB[codes].astype(np.int8)


# --------------------------------------------------------------------------
# int8 activations ("03 · Runtime": Q8_1 activations, one scale per 32)
# --------------------------------------------------------------------------
def quantize_acts(a: np.ndarray):
    """fp32 [M,K] -> (q int8 [M,K], d fp32 [M,K/32]) following R7."""
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("activations must be float32")
    if not np.isfinite(a).all():
        raise ValueError("non-finite activation")
    M, K = a.shape
    if K % BLOCK_WEIGHTS:
        raise ValueError("K must be a multiple of 32")
    A = a.reshape(M, K // BLOCK_WEIGHTS, BLOCK_WEIGHTS)
    amax = np.abs(A).max(axis=2)                                  # exact
    d = (amax / np.float32(127.0)).astype(np.float32)             # fl32 division
    q = np.zeros(A.shape, dtype=np.int8)
    nz = d > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (A / np.where(nz, d, np.float32(1.0))[..., None]).astype(np.float32)
    r64 = r.astype(np.float64)                          # exact widening
    rounded = np.sign(r64) * np.floor(np.abs(r64) + 0.5)  # half away from zero
    rounded = np.clip(rounded, -127, 127)
    q[nz] = rounded[nz].astype(np.int8)
    return q.reshape(M, K), d


def dequantize_acts(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """q * d per 32-block, exact in fp64, [M,K]."""
    q = np.asarray(q, dtype=np.int64)
    M, K = q.shape
    d64 = np.asarray(d, dtype=np.float32).astype(np.float64)
    return (q.reshape(M, K // BLOCK_WEIGHTS, BLOCK_WEIGHTS)
            * d64.reshape(M, K // BLOCK_WEIGHTS, 1)).reshape(M, K)


# --------------------------------------------------------------------------
# Products ("03 · Runtime": int8 lanes x Q8_1, int32 per half, then scales)
# --------------------------------------------------------------------------
def half_sums(packed: np.ndarray, N: int, K: int, q: np.ndarray) -> np.ndarray:
    """Integer dot of each 16-weight half with the int8 activations.

    -> int64 [M, N, K/32, 2]: S[m,n,b,h] = sum over the 16 weights of half h of
    block b of codebook[code] * q[m,k].
    """
    c8 = decoded_int8(packed, N, K).astype(np.int64)
    q = np.asarray(q, dtype=np.int64)
    M = q.shape[0]
    B = K // BLOCK_WEIGHTS
    return np.einsum("nbhi,mbhi->mnbh", c8.reshape(N, B, 2, HALF_WEIGHTS),
                     q.reshape(M, B, 2, HALF_WEIGHTS))


def ref_gemv(packed: np.ndarray, N: int, K: int, q: np.ndarray,
             d: np.ndarray) -> np.ndarray:
    """y[m,n] = sum_k w[n,k] * a[m,k] in fp64, with w the reconstructed weights
    and a = q*d the int8 activations (the exact value the integer pipeline
    re-associates).  -> fp64 [M,N]."""
    W = dequantize_weights(packed, N, K)
    A = dequantize_acts(q, d)
    return A @ W.T


ref_gemm = ref_gemv


def abs_product_sums(packed: np.ndarray, N: int, K: int, q: np.ndarray,
                     d: np.ndarray) -> np.ndarray:
    """sum_k |w[n,k] * a[m,k]|, fp64 [M,N]: the scale of the output tolerance."""
    W = np.abs(dequantize_weights(packed, N, K))
    A = np.abs(dequantize_acts(q, d))
    return A @ W.T


def ref_moe_gemv(bank: np.ndarray, E: int, N: int, K: int, ids, q: np.ndarray,
                 d: np.ndarray) -> np.ndarray:
    """Routed-expert products for one token.

    bank: the E experts' packed matrices back to back (E*N*10K/32 bytes).
    Row j of the result is expert ids[j] applied to the token; an id outside
    [0, E) gives a NaN row.  -> fp64 [len(ids), N].
    """
    bank = np.asarray(bank, dtype=np.uint8).reshape(E, N, row_bytes(K))
    ids = [int(i) for i in np.asarray(ids).reshape(-1)]
    y = np.full((len(ids), N), np.nan)
    for j, e in enumerate(ids):
        if 0 <= e < E:
            y[j] = ref_gemv(bank[e], N, K, q, d)[0]
    return y


def sort_by_expert(ids, E: int):
    """Routed slots grouped by expert: the token order of a batched expert
    product ("04 · Measured evidence" / "07 · Recipe decision": prompt
    batches through the routed experts, where prefill dominates).

    ids: the expert of each slot, slot s = t*top_k + j for token t's j-th
    expert.  Every slot whose id lies in [0, E) is put in the bucket of its
    expert, buckets in expert order, slots inside a bucket in increasing slot
    order; slots with another id are left out.
    -> (offsets int64 [E+1], order int64 [offsets[E]]): expert e's slots are
    order[offsets[e]:offsets[e+1]].
    """
    ids = [int(i) for i in np.asarray(ids).reshape(-1)]
    buckets = [[] for _ in range(E)]
    for s, e in enumerate(ids):
        if 0 <= e < E:
            buckets[e].append(s)
    offsets = [0]
    for b in buckets:
        offsets.append(offsets[-1] + len(b))
    order = [s for b in buckets for s in b]
    return np.array(offsets, dtype=np.int64), np.array(order, dtype=np.int64)


def ref_moe_batch(bank: np.ndarray, E: int, N: int, K: int, ids, q: np.ndarray,
                  d: np.ndarray) -> np.ndarray:
    """Routed-expert products for T tokens (a prompt batch).

    ids: [T, top_k]; q, d: the T tokens' int8 activations and scales.  Row
    t*top_k + j of the result is expert ids[t, j] applied to token t (NaN for
    an id outside [0, E)): the one-token product of each token, stacked.
    -> fp64 [T*top_k, N].
    """
    T = q.shape[0]
    ids = np.asarray(ids).reshape(T, -1)
    top_k = ids.shape[1]
    y = np.empty((T * top_k, N))
    for t in range(T):
        y[t * top_k:(t + 1) * top_k] = ref_moe_gemv(bank, E, N, K, ids[t], q[t:t + 1],
                                                    d[t:t + 1])
    return y
