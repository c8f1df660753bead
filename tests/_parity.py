"""Comparison rules shared by the GPU parity tests.

Bar for bf16 inputs: max |O_gpu - O_ref| <= 2e-2 and max |LSE_gpu - LSE_ref|
<= 1e-3 over rows with a visible key; -inf in exactly the same LSE entries
(rows with no visible key), where O must be exactly 0; no NaN or Inf
anywhere else.  fp32 inputs are held to a tighter bar derived from fp32
rounding: the length-D dot products and a sum over at most Tk terms stay
below 1e-5 relative at these sizes, so 1e-4 on O and on LSE leaves margin.
"""

import numpy as np
import torch

TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-4, 1e-4)}


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype="bf16", what=""):
    """Assert the parity bar; return (max O error, max LSE error)."""
    o = to64(o_gpu) if isinstance(o_gpu, torch.Tensor) else np.asarray(o_gpu, np.float64)
    l = to64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else np.asarray(lse_gpu, np.float64)
    o_tol, l_tol = TOL[dtype]
    assert o.shape == o_ref.shape and l.shape == lse_ref.shape, what
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(l).any(), f"{what}: NaN in LSE"
    assert np.isfinite(o).all(), f"{what}: Inf in O"
    empty_ref = np.isneginf(lse_ref)
    empty = np.isneginf(l)
    assert np.array_equal(empty, empty_ref), (
        f"{what}: -inf LSE mismatch at {np.argwhere(empty != empty_ref)[:5].tolist()}")
    assert not np.isposinf(l).any(), f"{what}: +inf LSE"
    assert (o[empty] == 0).all(), f"{what}: O not zero on empty rows"
    live = ~empty
    o_err = float(np.abs(o - o_ref).max()) if o.size else 0.0
    l_err = float(np.abs(l[live] - lse_ref[live]).max()) if live.any() else 0.0
    assert o_err <= o_tol, f"{what}: max |dO| = {o_err:.3e} > {o_tol}"
    assert l_err <= l_tol, f"{what}: max |dLSE| = {l_err:.3e} > {l_tol}"
    return o_err, l_err
