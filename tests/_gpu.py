"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(*what):
    """Name the case on stdout before its GPU step (a faulting run then says
    which case it was running)."""
    print("[case]", *what, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device())


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device=device())


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_within_bound(y_gpu, y_ref, absum, what=""):
    """|y_gpu - y_ref| <= 1e-5 * sum_k |w_k a_k| + 1e-6 for every output."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    bound = 1e-5 * np.asarray(absum) + 1e-6
    err = np.abs(y_gpu - y_ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} outputs outside the bound; first {idx.tolist()} "
            f"err {err[bad][:5]} bound {np.broadcast_to(bound, err.shape)[bad][:5]}")
    return float(np.max(err / bound)) if err.size else 0.0


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct rows: the first, the last and random ones."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, min(count, N), replace=False).tolist())
    rows.update({0, N - 1})
    return np.array(sorted(rows), dtype=np.int64)
