"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and nothing else: it holds none of the
ROCmFP2 arithmetic (no quantization, packing, decoding or products), so the CPU
oracle and the HIP library can both be fed from it without sharing code.

The workloads stand in for the expert and projection tensors of the MoE model
that the ROCmFP2 report measured on (its shapes are not published there):
fp32 weights drawn from N(0, sigma) with 0.1% of the entries multiplied by 8
(outliers), and activations drawn from N(0, 1).
"""
from __future__ import annotations

import numpy as np

# Named workloads.  Sizes are (M tokens, N output rows, K reduction length).
WORKLOADS = {
    # single GEMV, small enough for the oracle to finish in seconds
    "gemv_512x2048": dict(op="gemv", M=1, N=512, K=2048, sigma=0.02, wseed=0),
    # dense projection GEMV (~5.0 MiB of ROCmFP2 weights)
    "gemv_4096x4096": dict(op="gemv", M=1, N=4096, K=4096, sigma=0.02, wseed=0),
    # routed experts: 128 up-projections 1536x4096, one token, top-8
    "moe_128x1536x4096_top8": dict(op="moe", M=1, E=128, top_k=8, N=1536,
                                   K=4096, sigma=0.02, wseed=0),
    # the same bank for 4 consecutive tokens (e.g. a speculative-decoding
    # verification batch), half of each token's experts kept from the token
    # before: tokens grouped per expert, each expert decoded once
    "moe_128x1536x4096_top8_t4": dict(op="moe_tokens", M=4, E=128, top_k=8, N=1536,
                                      K=4096, sigma=0.02, wseed=0, share=0.5),
    # the same bank for a 512-token prompt: every token routed to 8 distinct
    # experts, independently of the others (4096 slots, ~32 per expert)
    "moe_gemm_128x1536x4096_top8_t512": dict(op="moe_gemm", M=512, E=128, top_k=8,
                                             N=1536, K=4096, sigma=0.02, wseed=0,
                                             share=0.0),
    # large layer GEMV (25.0 MiB of ROCmFP2 weights) at 1 and 4 tokens
    "gemv_16384x5120": dict(op="gemv", M=1, N=16384, K=5120, sigma=0.015,
                            wseed=0),
    "gemv_16384x5120_m4": dict(op="gemv", M=4, N=16384, K=5120, sigma=0.015,
                               wseed=0),
    # the same shape of row eight times taller (200 MiB of weights): large
    # enough that the launch is small against the transfer; context for the
    # 25 MiB figure, not one of the measured configurations
    "gemv_131072x5120": dict(op="gemv", M=1, N=131072, K=5120, sigma=0.015,
                             wseed=0),
    # prompt-batch GEMM (int8 matrix cores; the same product on fp16 ones)
    "gemm_512x14336x4096": dict(op="gemm", M=512, N=14336, K=4096, sigma=0.02,
                                wseed=0),
    "gemm_f16_512x14336x4096": dict(op="gemm_f16", M=512, N=14336, K=4096,
                                    sigma=0.02, wseed=0),
}

GENERIC_GEMV_SIGMA = 0.015


def workload(name: str) -> dict:
    """A named workload, or a dense GEMV of any shape named gemv_<N>x<K> (one
    token) or gemv_<N>x<K>_m<M> (M tokens), drawn like the large-layer GEMV:
    weights N(0, 0.015) with outliers, seed 0."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    import re
    m = re.fullmatch(r"gemv_(\d+)x(\d+)(?:_m(\d+))?", name)
    if m is None:
        raise KeyError(f"unknown workload {name!r}")
    return dict(op="gemv", M=int(m.group(3) or 1), N=int(m.group(1)), K=int(m.group(2)),
                sigma=GENERIC_GEMV_SIGMA, wseed=0)


ACT_SEED = 1
ROUTE_SEED = 2
OUTLIER_FRACTION = 0.001
OUTLIER_FACTOR = 8.0


def weights(N: int, K: int, sigma: float, seed=0) -> np.ndarray:
    """fp32 [N,K]: N(0, sigma) draws, then round(0.001*N*K) distinct entries
    (uniform, without replacement, drawn after the normal draws from the same
    generator) multiplied by 8."""
    rng = np.random.default_rng(seed)
    W = rng.normal(0.0, sigma, (N, K)).astype(np.float32)
    n_out = int(round(OUTLIER_FRACTION * N * K))
    if n_out:
        idx = rng.choice(N * K, n_out, replace=False)
        W.reshape(-1)[idx] *= np.float32(OUTLIER_FACTOR)
    return W


def expert_weights(e: int, N: int, K: int, sigma: float, seed=0) -> np.ndarray:
    """Weights of expert e of a bank: the generator is seeded with [seed, e]."""
    return weights(N, K, sigma, seed=[seed, e])


def activations(M: int, K: int, seed=ACT_SEED) -> np.ndarray:
    """fp32 [M,K] standard-normal activations (row 0 does not depend on M)."""
    return np.random.default_rng(seed).standard_normal((M, K)).astype(np.float32)


def routing(E: int, top_k: int, seed=ROUTE_SEED) -> np.ndarray:
    """int32 [top_k] distinct expert ids, uniform without replacement."""
    return np.random.default_rng(seed).choice(E, top_k, replace=False).astype(np.int32)


IMP_SEED = 3


def importance(K: int, seed=IMP_SEED, samples: int = 64) -> np.ndarray:
    """fp32 [K] per-channel importance: the mean square, over `samples`
    draws, of activations whose channels have log-normal gains (so channels
    differ in importance, as calibration statistics E[a^2] do)."""
    rng = np.random.default_rng(seed)
    gain = np.exp(rng.normal(0.0, 0.5, K))
    a = rng.standard_normal((samples, K)) * gain
    return (a * a).mean(axis=0).astype(np.float32)


def routing_tokens(E: int, top_k: int, T: int, share: float, seed=ROUTE_SEED) -> np.ndarray:
    """int32 [T, top_k] expert ids for T consecutive tokens.  Token 0 draws
    top_k distinct experts uniformly; each later token keeps each expert of
    the token before it with probability `share` and fills the rest with
    fresh distinct draws (share 0: independent tokens, 1: identical routing)."""
    rng = np.random.default_rng(seed)
    out = np.empty((T, top_k), np.int32)
    out[0] = rng.choice(E, top_k, replace=False)
    for t in range(1, T):
        keep = [e for e in out[t - 1] if rng.random() < share]
        rest = [e for e in rng.permutation(E) if e not in keep][:top_k - len(keep)]
        out[t] = np.array(keep + rest, np.int32)
    return out


def uniform_bytes(n: int, lo: int, hi: int, seed) -> np.ndarray:
    """uint8 [n] uniform in [lo, hi] (raw random bytes for edge-case tests)."""
    return np.random.default_rng(seed).integers(lo, hi + 1, n, dtype=np.int64).astype(np.uint8)
