"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Error metric: for each (b, h) slice (or each state), ||x - y||_inf / ||y||_inf, where y
is the fp64 oracle.  The bound is 2e-2 when q, k, v are bf16 and 1e-4 when they are
fp32 (fp32 state and accumulation throughout in both cases).
"""

import numpy as np
import torch

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def to64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def slice_rel(x, y, lead=2):
    """Max over leading slices of ||x-y||_inf/||y||_inf; returns (worst, per-slice array)."""
    x, y = to64(x), to64(y)
    assert x.shape == y.shape, (x.shape, y.shape)
    xs = x.reshape(int(np.prod(x.shape[:lead])), -1)
    ys = y.reshape(int(np.prod(y.shape[:lead])), -1)
    num = np.max(np.abs(xs - ys), axis=1)
    den = np.maximum(np.max(np.abs(ys), axis=1), 1e-30)
    r = num / den
    return float(r.max()), r


def assert_close(x, y, tol, lead=2, what=""):
    worst, _ = slice_rel(x, y, lead)
    print(f"    parity {what}: max slice rel err {worst:.3e} (bound {tol:.0e})", flush=True)
    assert worst <= tol, f"{what}: max slice rel err {worst:.3e} > {tol:.1e}"
    return worst
