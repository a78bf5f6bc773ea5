"""Helpers for the GPU parity tests: moving seeded inputs to the device and
measuring the error against the oracle with the tolerances the tests use.

Tolerances (stated for the whole suite):
  fp32 inputs: max |out - ref| / max |ref| <= 1e-5
  bf16 / f16 inputs (fp32 accumulation, unit-variance V): max |out - ref| <= 2e-2
  outputs of larger magnitude (the layer-normalised rows, |out| up to ~10):
  |out - ref| <= 2e-2 + u * |ref| element by element, u the output type's
  rounding unit relative to magnitude (bf16 2^-8, f16 2^-11): rounding a value
  of magnitude |ref| to the output type alone can cost u * |ref|, which the
  flat bound covers only below |ref| ~ 4 (bf16).
  gradients (bf16 / f16): |g - ref| <= 2e-2 + 2u * A element by element, where
  A is the sum of the magnitudes of the terms whose sum is g (grad_bounds).
  Each term carries at most a relative error of about u: the weights P and
  dS = P (dP - D) are rounded to the input type (u/2) before their products,
  and P is recomputed from the forward's row statistic, itself a sum of
  rounded weights (u/2); D uses the rounded forward output, which A covers
  through |D|_i = sum_c |dout_ic out_ic|; the rounded result adds u/2 |g|
  <= u/2 A.  A flat bound fails when the terms are large and cancel (scale
  ~ 1 makes the weights peaked and dP of size ~ sqrt(d)).
"""
from __future__ import annotations

import contextlib
import os

import numpy as np

TOL_F32_REL = 1e-5
TOL_LOWP_ABS = 2e-2
ROUNDING_UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def to_dev(arr, dtype: str):
    """numpy array (values exactly representable in ``dtype``) -> device tensor."""
    import torch
    if arr is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device="cuda", dtype=torch_dtype(dtype))


def lens_dev(lens):
    import torch
    if lens is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to("cuda")


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref)))


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    """Check ``got`` against the oracle ``ref`` at the suite's tolerance; returns the
    error measure used."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = max_err(got, ref)
    if dtype == "f32":
        scale = float(np.max(np.abs(ref))) if ref.size else 0.0
        rel = err / scale if scale > 0 else err
        assert rel <= TOL_F32_REL, f"{what}: relative error {rel:.3g} > {TOL_F32_REL}"
        return rel
    assert err <= TOL_LOWP_ABS, f"{what}: abs error {err:.3g} > {TOL_LOWP_ABS}"
    return err


def assert_close_scaled(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    """Element-wise |got - ref| <= 2e-2 + u * |ref| for bf16/f16 outputs (see the
    module docstring); returns the largest ratio of error to bound."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    bound = TOL_LOWP_ABS + ROUNDING_UNIT[dtype] * np.abs(ref)
    ratio = float(np.max(np.abs(got - ref) / bound))
    assert ratio <= 1.0, f"{what}: error reaches {ratio:.3g} x the bound (max abs err {np.max(np.abs(got - ref)):.3g})"
    return ratio


def grad_bounds(q, k, v, dout, P, out, scale):
    """Magnitude sums (A_dq, A_dk, A_dv) of the gradient terms; see the module
    docstring.  All arguments fp64 numpy arrays of the oracle's shapes."""
    q, k, v, dout = (np.asarray(x, np.float64) for x in (q, k, v, dout))
    dP = dout @ np.swapaxes(v, -1, -2)                          # [B,H,Nq,Nk]
    dabs = np.sum(np.abs(dout * out), axis=-1, keepdims=True)   # [B,H,Nq,1]
    M = P * (np.abs(dP) + dabs)
    a = abs(scale)
    A_dv = np.swapaxes(P, -1, -2) @ np.abs(dout)
    A_dk = a * (np.swapaxes(M, -1, -2) @ np.abs(q))
    A_dq = a * (M @ np.abs(k))
    return A_dq, A_dk, A_dv


def assert_close_grad(got: np.ndarray, ref: np.ndarray, A: np.ndarray, dtype: str, what: str = "") -> float:
    """Element-wise |got - ref| <= 2e-2 + 2u * A (see the module docstring); returns
    the largest ratio of error to bound."""
    assert got.shape == ref.shape == A.shape, (got.shape, ref.shape, A.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    bound = TOL_LOWP_ABS + 2.0 * ROUNDING_UNIT[dtype] * A
    ratio = float(np.max(np.abs(got - ref) / bound))
    assert ratio <= 1.0, f"{what}: error reaches {ratio:.3g} x the bound (max abs err {np.max(np.abs(got - ref)):.3g})"
    return ratio


@contextlib.contextmanager
def attention_block(block):
    """Run the bf16/f16 attention calls inside the block with the kernel of
    ``block`` queries per workgroup (32: one-wave workgroups, 256 / 512: four-
    or eight-wave workgroups) through the library's MHA_ATTENTION_BLOCK
    override; None keeps
    the library's own choice (mha_forward_block_queries)."""
    old = os.environ.get("MHA_ATTENTION_BLOCK")
    if block is None:
        os.environ.pop("MHA_ATTENTION_BLOCK", None)
    else:
        os.environ["MHA_ATTENTION_BLOCK"] = str(block)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("MHA_ATTENTION_BLOCK", None)
        else:
            os.environ["MHA_ATTENTION_BLOCK"] = old

