"""Helpers for the GPU parity tests: device transfer, the per-row error bound
check, and canary guard bands after output buffers."""
import numpy as np
import pytest
import torch

gpu = pytest.mark.gpu

CANARY = 12345.678


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def guarded_empty(shape, dtype=torch.float32, guard=1024):
    """An output tensor followed by `guard` canary elements in one allocation."""
    n = int(np.prod(shape))
    buf = torch.full((n + guard,), CANARY, dtype=dtype, device="cuda")
    return buf[:n].view(*shape), buf


def check_guard(buf, n):
    tail = host(buf[n:])
    assert np.all(tail == np.float32(CANARY)), "write past the end of an output buffer"


def assert_within_bound(y_gpu, y_ref, bound, rel, what=""):
    """|y_gpu - y_ref| <= rel * bound element by element (the per-row bound
    sum_k |W[n][k] x'[m][k]| computed by the oracle)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    lim = rel * bound
    bad = err > lim
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outputs outside {rel}*bound; first at {tuple(i)}: "
            f"gpu {y_gpu[tuple(i)]!r} ref {y_ref[tuple(i)]!r} err {err[tuple(i)]:.3e} "
            f"bound {lim[tuple(i)]:.3e}; max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3e}")
    return float(np.max(err / np.maximum(bound, 1e-300)))
