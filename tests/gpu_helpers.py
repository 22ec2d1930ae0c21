"""Helpers shared by the GPU tests: device placement, oracle calls, tolerance checks."""
from __future__ import annotations

import os
from typing import Optional, Sequence

import numpy as np
import pytest
import torch

from oracle import oracle as O

TOL = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 2e-3}
THREADS = min(16, os.cpu_count() or 1)


def lib():
    """The package, or skip when no GPU is present (GPU tests are also marked 'gpu')."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_group_quantized_q4gsw_amd as q
    return q


def dev(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    return None if t is None else t.cuda().contiguous()


def pack(q, w):
    return q.pack(dev(w.codes), dev(w.scales), w.group_size)


def assert_within(got: torch.Tensor, ref: np.ndarray, norm: np.ndarray, tol: float, label: str,
                  rows: Optional[Sequence[int]] = None) -> float:
    """|got - ref| <= tol * R elementwise (plus a denormal-sized floor); returns max err / R."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g = g[list(rows)]
    assert g.shape == ref.shape, (label, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    err = np.abs(g - ref)
    bound = tol * norm + 1e-30
    bad = err > bound
    ratio = float(np.max(err / np.maximum(norm, 1e-300))) if err.size else 0.0
    if np.any(bad):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{label}: {int(bad.sum())} of {err.size} outside tol {tol}*R; worst at {i}: "
                             f"got {g[i]!r} want {ref[i]!r} R {norm[i]!r}; max err/R {ratio:.3e}")
    return ratio


def oracle_fwd(x: torch.Tensor, w, rows: Optional[Sequence[int]] = None):
    xs = x if rows is None else x[list(rows)].contiguous()
    return O.linear_fwd(xs, w.codes, w.scales, w.group_size, threads=THREADS)


def oracle_bwd(d_out: torch.Tensor, w, rows: Optional[Sequence[int]] = None):
    ds = d_out if rows is None else d_out[list(rows)].contiguous()
    return O.linear_bwd_input(ds, w.codes, w.scales, w.group_size, threads=THREADS)


def sample_rows(M: int, count: int = 12) -> list:
    """Rows spread over [0, M), always including the first and the last."""
    if M <= count:
        return list(range(M))
    idx = set(np.linspace(0, M - 1, count).round().astype(int).tolist())
    idx.update({0, M - 1, min(M - 1, 127), min(M - 1, 128)})
    return sorted(idx)
