"""Where the gradient tolerance in tests/parity.py comes from (CPU).

No page states a tolerance for gradients, so the bound is derived from the
arithmetic the backward kernels perform. Besides fp32 accumulation (about
2^-24 per operation, negligible here) the kernels take three roundings to
bfloat16: the softmax weights P before the dV product, the score gradients
dS before the dQ and dK products, and the forward output O (bf16) from which
delta_i = <dO_i, O_i> is taken; each gradient is then stored as bf16.

This file emulates exactly those roundings in fp64 (round to nearest even,
oracle.bf16.round_bf16), per sequence and query head, on seeded N(0, 1)
inputs, and compares the result with the unrounded fp64 oracle. It checks
the three facts the tolerance rests on:

  * per query head the error beyond the gradient's own bf16 rounding stays
    well inside 2e-2 (dq sums over one head);
  * dk and dv sum the contributions of the G query heads of a KV head, whose
    rounding errors are independent, so their error grows with G (about as
    sqrt(G)): at G = 16 the emulated error alone comes close to a fixed 2e-2
    (0.0195 at D = 128 here; the kernels, whose fp32 sums and exp2 add a
    little more, measured 0.025 on one such case), while 2e-2 sqrt(G) keeps
    a wide margin;
  * the whole-tensor (Frobenius) relative error stays below 1e-2 and does
    not grow with G.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import backward as BW
from oracle.bf16 import round_bf16
from tests.parity import GRAD_ATOL, GRAD_FRO, GRAD_RTOL, grad_scale


def emulated_backward_rows(qh, kh, vh, doh, out_bf16, lse, visible, scale):
    """One query head's gradients with the kernels' bf16 roundings applied:
    P and dS rounded before their products, delta from the bf16 output.
    Accumulations are exact (fp64); results are left unrounded."""
    s = np.where(visible, scale * (qh @ kh.T), -np.inf)
    live = np.isfinite(lse)
    p = np.where(visible & live[:, None], np.exp(s - np.where(live, lse, 0.0)[:, None]), 0.0)
    dv = round_bf16(p).T @ doh
    dp = doh @ vh.T
    delta = (doh * out_bf16).sum(axis=1)
    ds = round_bf16(p * (dp - delta[:, None]))
    return scale * (ds @ kh), scale * (ds.T @ qh), dv


def few_key_errors(Lq, Lk, D, seed):
    """One non-causal sequence of Lq queries over Lk keys, one head: the
    largest ratio, per gradient, of the emulated element error (bf16-stored,
    beyond the GRAD_RTOL rounding term) to the bound's absolute term, with
    and without its scaling by the gradient's RMS."""
    rng = np.random.default_rng([97, Lq, Lk, D, seed])
    bf = lambda *shape: round_bf16(rng.standard_normal(shape))
    q, k, v, do = bf(Lq, 1, D), bf(Lk, 1, D), bf(Lk, 1, D), bf(Lq, 1, D)
    cq, ck = np.array([0, Lq]), np.array([0, Lk])
    out, lse, _ = A.attend_varlen(q, k, v, cq, ck, 1, False)
    refs = BW.attend_varlen_backward(q, k, v, do, cq, ck, 1, False)[:3]
    emu = emulated_backward_rows(q[:, 0], k[:, 0], v[:, 0], do[:, 0], round_bf16(out[:, 0]),
                                 lse[:, 0], A.visible_keys(Lq, Lk, False), 1.0 / np.sqrt(D))
    res = {}
    for name, got, ref in zip(("dq", "dk", "dv"), emu, refs):
        ref = ref[:, 0]
        err = np.abs(round_bf16(got) - ref) - GRAD_RTOL * np.abs(ref)
        res[name] = (float(err.max() / (GRAD_ATOL * grad_scale(ref))),
                     float(err.max() / GRAD_ATOL))
    return res


def one_sequence_errors(L, D, G, seed, causal=True):
    """Max element error (beyond output rounding) and Frobenius ratio of
    emulated dq, dk, dv against the exact oracle, for one sequence of L
    tokens with G query heads on one KV head."""
    rng = np.random.default_rng([91, L, D, G, seed])
    bf = lambda *shape: round_bf16(rng.standard_normal(shape))
    q, k, v, do = bf(L, G, D), bf(L, 1, D), bf(L, 1, D), bf(L, G, D)
    cu = np.array([0, L])
    out, lse, _ = A.attend_varlen(q, k, v, cu, cu, 1, causal)
    rq, rk, rv, _, _ = BW.attend_varlen_backward(q, k, v, do, cu, cu, 1, causal)
    vis = A.visible_keys(L, L, causal)
    scale = 1.0 / np.sqrt(D)
    eq = np.zeros_like(rq)
    ek = np.zeros_like(rk)
    ev = np.zeros_like(rv)
    for h in range(G):
        gq, gk, gv = emulated_backward_rows(q[:, h], k[:, 0], v[:, 0], do[:, h],
                                            round_bf16(out[:, h]), lse[:, h], vis, scale)
        eq[:, h] = gq
        ek[:, 0] += gk
        ev[:, 0] += gv
    res = {}
    for name, got, ref in (("dq", eq, rq), ("dk", ek, rk), ("dv", ev, rv)):
        # the stored gradient is bf16: its own rounding is the GRAD_RTOL term
        err = np.abs(round_bf16(got) - ref) - GRAD_RTOL * np.abs(ref)
        res[name] = (float(err.max()), float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
    return res


@pytest.mark.parametrize("D", [32, 128])
def test_gradient_bound_follows_from_the_roundings(D):
    worst = {}
    for G in (1, 4, 16):
        for seed in range(2):
            r = one_sequence_errors(640, D, G, seed)
            for name, (emax, fro) in r.items():
                n = 1 if name == "dq" else G
                # the derived bound holds with a margin of at least 1.5x
                assert emax * 1.5 <= GRAD_ATOL * np.sqrt(n), (G, name, emax)
                assert fro * 2 <= GRAD_FRO, (G, name, fro)
                key = (G, name)
                worst[key] = max(worst.get(key, (0, 0)), (emax, fro))
    for name in ("dk", "dv"):
        e1, f1 = worst[(1, name)]
        e16, f16 = worst[(16, name)]
        # summing 16 independent per-head errors: clearly larger (the
        # expected factor is sqrt(16) = 4) ...
        assert e16 >= 2.0 * e1, (name, e1, e16)
        # ... while the relative Frobenius error does not grow with G
        assert f16 <= 1.5 * f1, (name, f1, f16)
    # dq sums one head whatever G is: it stays within the one-head bound
    # (its maximum still rises a little with G, being taken over G times as
    # many elements)
    assert worst[(16, "dq")][0] * 1.5 <= GRAD_ATOL


def test_bound_scales_with_the_gradient_rms():
    """Few keys seen by many queries (non-causal) give dk and dv of RMS
    well above 1 (sums of many terms of weight about 1 / Lk), and rounding
    errors in proportion: there the unscaled absolute bound of 2e-2 fails
    (by up to 4.5x) while 2e-2 max(1, rms) holds with a 1.25x margin (dk and
    dv use under 0.4 of it; dq, whose RMS stays below 1, up to 0.7)."""
    unscaled = 0.0
    for Lq, Lk, D in ((451, 4, 256), (1000, 2, 64), (2000, 8, 128)):
        for seed in range(2):
            for name, (scaled, plain) in few_key_errors(Lq, Lk, D, seed).items():
                assert scaled * 1.25 <= 1.0, (Lq, Lk, D, name, scaled)
                unscaled = max(unscaled, plain)
    assert unscaled > 1.0
