"""Parity metrics between the HIP path and the fp64 oracle.

Tolerances of the layer (bf16 inputs, fp32 accumulation):
  * o: for every (b, t, h) row, e = ||o_gpu - o_ref||_2 / max(||o_ref||_2, floor),
    floor = 1e-2 * mean row norm of o_ref; pass if max e <= 2e-2.  The floor keeps
    rows whose reference nearly cancels (e.g. t = 0, where o_0 is one product)
    from dividing by ~0.
  * S: ||S_gpu - S_ref||_F / ||S_ref||_F <= 1e-2, overall and per (b, h).
"""
from __future__ import annotations

import numpy as np

O_ROW_TOL = 2e-2
S_FRO_TOL = 1e-2


def o_row_errors(o_gpu, o_ref):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    diff = np.linalg.norm(o_gpu - o_ref, axis=-1)
    ref = np.linalg.norm(o_ref, axis=-1)
    floor = 1e-2 * max(float(ref.mean()), 1e-30)
    e = diff / np.maximum(ref, floor)
    return {
        "max": float(e.max()),
        "p99": float(np.percentile(e, 99)),
        "median": float(np.median(e)),
        "fro": float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300)),
        "finite": bool(np.isfinite(o_gpu).all()),
    }


def s_errors(S_gpu, S_ref):
    S_gpu = np.asarray(S_gpu, dtype=np.float64)
    S_ref = np.asarray(S_ref, dtype=np.float64)
    assert S_gpu.shape == S_ref.shape
    d = S_gpu - S_ref
    per = np.linalg.norm(d, axis=(-2, -1)) / np.maximum(np.linalg.norm(S_ref, axis=(-2, -1)), 1e-300)
    return {
        "fro": float(np.linalg.norm(d) / max(np.linalg.norm(S_ref), 1e-300)),
        "per_bh_max": float(per.max()),
        "finite": bool(np.isfinite(S_gpu).all()),
    }


def assert_o_close(o_gpu, o_ref, tol=O_ROW_TOL, what="o"):
    e = o_row_errors(o_gpu, o_ref)
    assert e["finite"], f"{what}: non-finite values"
    assert e["max"] <= tol, f"{what}: max row error {e['max']:.3e} > {tol} ({e})"
    return e


def assert_S_close(S_gpu, S_ref, tol=S_FRO_TOL, what="S"):
    e = s_errors(S_gpu, S_ref)
    assert e["finite"], f"{what}: non-finite values"
    assert e["fro"] <= tol and e["per_bh_max"] <= tol, f"{what}: {e} > {tol}"
    return e


def to_np(t):
    """torch tensor (any device, bf16/fp32) -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_np32(t):
    """torch tensor -> float32 numpy (exact for bf16 and fp32 data)."""
    return t.detach().float().cpu().numpy()
