"""Shared helpers for the GPU parity tests: the tolerance bar and tensor <-> numpy."""
import numpy as np
import torch

# bf16 inputs: max-abs error 2e-2 and relative Frobenius error 1e-2 against the
# fp64 oracle; fp32 inputs: max-abs error 1e-5.
BF16_MAX_ABS = 2e-2
BF16_REL_FRO = 1e-2
F32_MAX_ABS = 1e-5
LSE_BF16_ABS = 2e-2
LSE_F32_ABS = 1e-5


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_bf16_close(got, ref, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel = errors(got, ref)
    assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_FRO, \
        f"{what}: max_abs={max_abs:.3e} rel_fro={rel:.3e}"
    return max_abs, rel


def assert_f32_close(got, ref, what="", tol=F32_MAX_ABS):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, _ = errors(got, ref)
    assert max_abs <= tol, f"{what}: max_abs={max_abs:.3e}"
    return max_abs


def assert_lse_close(got, ref, tol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), f"{what}: -inf pattern differs"
    if fin.any():
        err = float(np.abs(got[fin] - ref[fin]).max())
        assert err <= tol, f"{what}: lse err {err:.3e}"


# FP8 attention (E4M3 products on the matrix cores) against the oracle's FP8
# recipe.  The hardware accumulates an FP8 product with an error of up to
# about 2^-15 of the sum of the magnitudes of its terms (measured: 2.6e-5),
# so a weight that lies that close to an E4M3 rounding boundary can round to
# the neighbouring code: one step, at most 2^-3 of the weight.  A flipped
# weight moves an output by at most 2^-3 of (its share of the row's weight)
# x |v|, so the elementwise bar is max(2e-2, max|v| / 8); the relative
# Frobenius bar stays 1e-2, and the log-sum-exp (from the unquantised
# denominator) keeps the bf16 bar.
FP8_ATTN_REL_FRO = 1e-2


def assert_fp8_attention_close(got, ref, vmax, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel = errors(got, ref)
    bound = max(BF16_MAX_ABS, vmax / 8.0)
    print(f"  {what}: max_abs={max_abs:.3e} (bound {bound:.3e}) rel_fro={rel:.3e}", flush=True)
    assert max_abs <= bound and rel <= FP8_ATTN_REL_FRO, \
        f"{what}: max_abs={max_abs:.3e} (bound {bound:.3e}) rel_fro={rel:.3e}"
    return max_abs, rel
