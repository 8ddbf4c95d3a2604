"""Comparison helpers for HIP-vs-oracle parity tests (no attention arithmetic).

Tolerances: bf16 outputs within max |err| <= 1e-2 of the unrounded fp64
oracle; only where |O_ref| >= 4, whose bf16 spacing (2^-5) makes a correctly
rounded value up to 2^-6 > 1e-2 away, the bound is one bf16 ulp of the
reference (only very short KV reaches such values). fp32 LSE within 1e-3
relative, |d| <= max(1e-3 |LSE_ref|, 1e-4): the absolute floor covers LSE
values near 0 (one key whose score is near 0), where the fp32 rounding of the
D-term score sum (about 2^-24 sqrt(D) sum|q_d k_d| scale, ~1e-5 for N(0, 1)
inputs at D <= 256) is not relative to the tiny result. -inf must match
exactly and NaN always fails.

Gradients (bf16 dq, dk, dv) against the unrounded fp64 oracle: every element
within 2e-2 * sqrt(n) * max(1, rms(ref)) + 2^-8 |ref|, where n is the number
of query heads whose contributions the element sums (1 for dq, G for dk and
dv) and rms(ref) the root mean square of the reference tensor, and the whole
tensor within 1e-2 relative in the Frobenius norm. The rms factor is 1 on
the long causal sequences the derivation below emulates; few keys seen by
many queries give gradients of rms well above 1, whose rounding errors grow
in proportion (emulated in tests/test_grad_tolerance_derivation.py: the
unscaled term fails there, the scaled one holds with a 1.25x margin). Derivation: the
kernels round the softmax weights and dS to bf16 as MFMA operands (2^-9
relative each, random), take <dO, O> from the forward's bf16 output, and
round the results to bf16 (the 2^-8 |ref| term); an fp64 emulation of exactly
these roundings (causal, L up to 2000, D 32 and 128, N(0,1) inputs) gives
per-head element errors beyond the output rounding of at most 0.0094 and
Frobenius ratios of 0.0021-0.0027; dk and dv add G independent per-head
errors, which grow as sqrt(G) (emulated: 0.0068 at G = 1, 0.020 at G = 16),
while the Frobenius ratio does not grow with G. Where the oracle's gradient
is zero everywhere the Frobenius ratio is 0/0; a result at the rounding level
of fp32 sums (every |x| <= 2^-10) is then accepted: a gradient that vanishes
by cancellation, e.g. dq and dk of a row whose only visible key has weight
1 (dS = p (dP - delta) with dP = delta exactly), comes out as the difference
of two fp32 sums of the same D bf16 products taken in different orders, at
most 2 D 2^-24 sum|dO v| before the scale and |k| factors (below 1e-3 at
D <= 256 for N(0,1) inputs). Rows that see no key are exactly zero by
construction; `assert_zero_rows` checks that separately.
"""
import numpy as np

OUT_ATOL = 1e-2
OUT_ULP_FROM = 4.0     # |O_ref| from which one bf16 ulp (2^-5 and up) is the bound
LSE_RTOL = 1e-3
LSE_ATOL = 1e-4
GRAD_ATOL = 2e-2
GRAD_RTOL = 2.0 ** -8
GRAD_FRO = 1e-2
GRAD_ZERO_ATOL = 2.0 ** -10  # all-zero reference: rounding level of fp32 sums


def bf16_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 0.0)


def assert_out_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    tol = np.where(np.abs(ref) >= OUT_ULP_FROM, np.maximum(OUT_ATOL, bf16_ulp(ref)), OUT_ATOL)
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
    tol = np.maximum(LSE_RTOL * np.abs(r), LSE_ATOL)
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} LSE values out of tolerance, max err {err.max():.3e}"
    return float(err.max()) if err.size else 0.0


def grad_scale(ref):
    """max(1, root mean square of the reference gradient tensor)."""
    ref = np.asarray(ref, dtype=np.float64)
    return max(1.0, float(np.sqrt(np.mean(ref ** 2)))) if ref.size else 1.0


def assert_grad_close(got, ref, what="", heads=1):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in gradient"
    err = np.abs(got - ref)
    bad = err > GRAD_ATOL * np.sqrt(heads) * grad_scale(ref) + GRAD_RTOL * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} gradients out of tolerance; max err "
                             f"{err.max():.3e}; first at {idx.tolist()} got "
                             f"{[got[tuple(i)] for i in idx]} ref {[ref[tuple(i)] for i in idx]}")
    nr = np.linalg.norm(ref)
    if nr > 0:
        fro = np.linalg.norm(got - ref) / nr
        assert fro <= GRAD_FRO, f"{what}: relative Frobenius error {fro:.3e}"
    else:
        assert (np.abs(got) <= GRAD_ZERO_ATOL).all(), \
            f"{what}: gradient above rounding level where the oracle has none"
    return float(err.max()) if err.size else 0.0


def assert_zero_rows(got, rows, what=""):
    """Gradient rows that no visible key (or query) reaches are exactly 0."""
    got = np.asarray(got, dtype=np.float64)
    assert (got[rows] == 0).all(), f"{what}: nonzero gradient in rows no key reaches"
