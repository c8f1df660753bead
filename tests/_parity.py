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


# Gradient bar (bf16 inputs).  The backward rounds P and dS to bf16 (unit
# roundoff u = 2^-8) before the three gradient products and accumulates in
# fp32; a gradient element is a sum of such products, so its error is a sum of
# independent roundings of relative size <= u (RMS u/sqrt(3) ~ 2.3e-3 of the
# element's magnitude), plus the same again when the gradient itself is stored
# in bf16 and when O arrives in bf16 (through D = rowsum(dO * O)).  The bar is
# about 3x that estimate on the relative Frobenius error and 2e-2 of the
# tensor's largest magnitude element-wise.  Entries whose exact gradient is 0
# because no visible pair reaches them must come out exactly 0.  A gradient
# that is 0 only by cancellation (a row with a single visible key has
# dP = D) keeps the fp32 residue of dP - D, two differently ordered sums of
# the same products: ~1e-7 relative to |dP| ~ sqrt(D), so 1e-4 absolute.
GRAD_FRO = 1e-2
GRAD_MAX = 2e-2
GRAD_CANCEL_ATOL = 1e-4


def compare_grads(got, ref, what="", fro_tol=GRAD_FRO, max_tol=GRAD_MAX, exact_zero=None):
    """Assert the gradient bar; return (relative Frobenius error, max error / max |ref|)."""
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.isfinite(g).all(), f"{what}: NaN or Inf"
    if exact_zero is not None and exact_zero.any():
        bad = g[exact_zero] != 0
        assert not bad.any(), f"{what}: {int(bad.sum())} entries that no pair reaches are not 0"
    nref = float(np.linalg.norm(ref))
    mref = float(np.abs(ref).max()) if ref.size else 0.0
    err = g - ref
    if nref == 0.0:
        mx = float(np.abs(err).max()) if err.size else 0.0
        assert mx <= GRAD_CANCEL_ATOL, f"{what}: exact gradient is 0, got max |g| = {mx:.3e}"
        return 0.0, mx
    fro = float(np.linalg.norm(err)) / nref
    mx = float(np.abs(err).max()) / mref
    assert fro <= fro_tol, f"{what}: relative Frobenius error {fro:.3e} > {fro_tol}"
    assert mx <= max_tol, f"{what}: max error {mx:.3e} of max |ref| > {max_tol}"
    return fro, mx
