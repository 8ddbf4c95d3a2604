"""Comparison helpers for HIP-vs-oracle parity tests (no attention arithmetic).

Tolerances: bf16 outputs within max |err| <= 1e-2 of the unrounded fp64
oracle, widened to one bf16 ulp of the reference where that is larger (from
|O| >= 2, where the ulp is 2^-6; only very short KV reaches such values); fp32 LSE within 1e-3 relative
(|d| <= 1e-3 * max(1, |LSE|), since LSE can sit near 0); -inf must match
exactly and NaN always fails.
"""
import numpy as np

OUT_ATOL = 1e-2
LSE_RTOL = 1e-3


def bf16_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 0.0)


def assert_out_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    tol = np.maximum(OUT_ATOL, bf16_ulp(ref))
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} outputs out of tolerance; max err "
                             f"{err.max():.3e}; first at {idx.tolist()} got "
                             f"{[got[tuple(i)] for i in idx]} ref {[ref[tuple(i)] for i in idx]}")
    return float(err.max()) if err.size else 0.0


def assert_lse_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN in LSE"
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), f"{what}: -inf pattern differs"
    g, r = got[~ninf], ref[~ninf]
    err = np.abs(g - r)
    tol = LSE_RTOL * np.maximum(1.0, np.abs(r))
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} LSE values out of tolerance, max err {err.max():.3e}"
    return float(err.max()) if err.size else 0.0
