"""Pins of the fp64 backward oracle against things other than itself.

oracle.backward writes out the chain rule through the softmax. It is pinned
to: central finite differences of the forward oracle (an independent
computation of the same derivative), PyTorch autograd through
scaled_dot_product_attention on the CPU in fp64 (a library routine), closed
forms, and invariants of the mathematics. test_oracle_backward_mutants.py
plants plausible mistakes in the formula and checks that one of these fails.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import backward as BW
from tests.test_oracle_attention import _rand_case


def _loss(q, k, v, dout, cu_q, cu_k, B, causal):
    out, _, written = A.attend_varlen(q, k, v, cu_q, cu_k, B, causal)
    return float((out[written] * dout[written]).sum())


def finite_difference_error(q, k, v, dout, cu_q, cu_k, B, causal, eps=1e-6):
    """Largest |analytic - central difference| over every input element,
    relative to max(1, |gradient|)."""
    dq, dk, dv, wq, wk = BW.attend_varlen_backward(q, k, v, dout, cu_q, cu_k, B, causal)
    worst = 0.0
    for name, x, g, w in (("q", q, dq, wq), ("k", k, dk, wk), ("v", v, dv, wk)):
        for idx in np.ndindex(x.shape):
            if not w[idx[0]]:
                continue
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, dout, cu_q, cu_k, B, causal)
            x[idx] = old - eps
            lm = _loss(q, k, v, dout, cu_q, cu_k, B, causal)
            x[idx] = old
            fd = (lp - lm) / (2 * eps)
            worst = max(worst, abs(fd - g[idx]) / max(1.0, abs(fd)))
    return worst


def _fd_case(seed):
    rng = np.random.default_rng([21, seed])
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3]))
    D = int(rng.choice([2, 3, 4]))
    B = int(rng.integers(1, 3))
    causal = bool(seed % 2)
    q, k, v, cu_q, cu_k = _rand_case(rng, B, Hkv * G, Hkv, D, 4, 5, causal,
                                     lead=int(rng.integers(0, 2)), tail=2)
    dout = rng.standard_normal(q.shape)
    return q, k, v, dout, cu_q, cu_k, B, causal


@pytest.mark.parametrize("seed", range(8))
def test_matches_central_finite_differences_of_the_forward(seed):
    args = _fd_case(seed)
    assert finite_difference_error(*args) < 1e-7


def autograd_error(q, k, v, dout, cu_q, cu_k, B, causal):
    """Largest |oracle - torch autograd| on the defined rows, where torch
    differentiates SDPA (CPU fp64, explicit boolean mask) with GQA expanded
    by repeat_interleave, so each KV head's gradient sums its G query heads.
    Sequences must have no query row without a visible key."""
    dq, dk, dv, wq, wk = BW.attend_varlen_backward(q, k, v, dout, cu_q, cu_k, B, causal)
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    worst = 0.0
    for b in range(B):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0 or Lk == 0:
            continue
        qt = torch.tensor(q[q0:q1].transpose(1, 0, 2), requires_grad=True)
        kt = torch.tensor(k[k0:k1].transpose(1, 0, 2), requires_grad=True)
        vt = torch.tensor(v[k0:k1].transpose(1, 0, 2), requires_grad=True)
        mask = torch.ones(Lq, Lk, dtype=torch.bool)
        if causal:
            mask = mask.tril(diagonal=Lk - Lq)
        assert bool(mask.any(1).all())
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.repeat_interleave(G, 0), vt.repeat_interleave(G, 0), attn_mask=mask)
        o.backward(torch.from_numpy(dout[q0:q1].transpose(1, 0, 2).copy()))
        for mine, ref in ((dq[q0:q1], qt.grad), (dk[k0:k1], kt.grad), (dv[k0:k1], vt.grad)):
            worst = max(worst, float(np.abs(mine - ref.numpy().transpose(1, 0, 2)).max()))
    return worst


def _autograd_case(seed, causal, G):
    rng = np.random.default_rng([22, seed, int(causal), G])
    Hkv, D, B = 2, 8, 3
    lq = rng.integers(1, 12, size=B)
    lk = lq + rng.integers(0, 6, size=B)     # Lk >= Lq: every causal row sees a key
    cu_q = np.concatenate([[2], 2 + np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[1], 1 + np.cumsum(lk)]).astype(np.int64)
    q = rng.standard_normal((int(cu_q[-1]) + 1, Hkv * G, D))
    k = rng.standard_normal((int(cu_k[-1]) + 1, Hkv, D))
    v = rng.standard_normal((int(cu_k[-1]) + 1, Hkv, D))
    dout = rng.standard_normal(q.shape)
    return q, k, v, dout, cu_q, cu_k, B, causal


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("seed", range(2))
def test_matches_torch_autograd_through_sdpa(seed, causal, G):
    assert autograd_error(*_autograd_case(seed, causal, G)) < 1e-11


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_single_key_gives_zero_dq_dk_and_summed_dout_for_dv():
    """With one key the softmax weight is 1 whatever q and k are."""
    rng = np.random.default_rng(5)
    Hq, Hkv, D, L = 6, 2, 5, 7
    q = rng.standard_normal((L, Hq, D))
    k = rng.standard_normal((1, Hkv, D))
    v = rng.standard_normal((1, Hkv, D))
    dout = rng.standard_normal((L, Hq, D))
    dq, dk, dv, _, _ = BW.attend_varlen_backward(q, k, v, dout, [0, L], [0, 1], 1, False)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-13
    for hk in range(Hkv):
        np.testing.assert_allclose(dv[0, hk], dout[:, 3 * hk:3 * hk + 3].sum(axis=(0, 1)),
                                   rtol=1e-13, atol=1e-13)


def test_zero_output_gradient_gives_zero_gradients():
    rng = np.random.default_rng(6)
    q, k, v, cu_q, cu_k = _rand_case(rng, 3, 4, 2, 6, 9, 9, True, lead=1, tail=1)
    dq, dk, dv, wq, wk = BW.attend_varlen_backward(q, k, v, np.zeros_like(q), cu_q, cu_k, 3, True)
    assert (dq[wq] == 0).all() and (dk[wk] == 0).all() and (dv[wk] == 0).all()


def test_equal_value_rows_give_zero_dq_dk():
    """O no longer depends on the weights, so it does not depend on q or k."""
    rng = np.random.default_rng(7)
    L, Hq, Hkv, D = 9, 4, 2, 6
    q = rng.standard_normal((L, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = np.broadcast_to(rng.standard_normal((1, Hkv, D)), (L, Hkv, D)).copy()
    dout = rng.standard_normal((L, Hq, D))
    dq, dk, dv, _, _ = BW.attend_varlen_backward(q, k, v, dout, [0, L], [0, L], 1, True)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def test_causal_first_query_has_zero_dq_and_feeds_only_the_first_key():
    """With Lq = Lk, query 0 sees only key 0 (weight 1): dq_0 = 0, and with
    dout zero elsewhere only key 0 receives dv = dout_0 (per head)."""
    rng = np.random.default_rng(8)
    L, Hq, Hkv, D = 6, 2, 1, 4
    q = rng.standard_normal((L, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    dout = np.zeros((L, Hq, D))
    dout[0] = rng.standard_normal((Hq, D))
    dq, dk, dv, _, _ = BW.attend_varlen_backward(q, k, v, dout, [0, L], [0, L], 1, True)
    assert np.abs(dq[0]).max() == 0
    np.testing.assert_allclose(dv[0, 0], dout[0].sum(axis=0), rtol=1e-14)
    assert np.abs(dv[1:]).max() == 0 and np.abs(dk).max() == 0


def test_rows_without_visible_keys_and_keys_without_queries():
    """Causal with Lq > Lk: the first Lq - Lk rows see nothing (dq = 0); a
    sequence with Lq = 0 gives its keys dk = dv = 0; rows outside every
    sequence stay undefined."""
    rng = np.random.default_rng(9)
    cu_q = np.array([1, 7, 7, 10])        # Lq = 6, 0, 3
    cu_k = np.array([0, 3, 8, 12])        # Lk = 3, 5, 4
    q = rng.standard_normal((11, 2, 4))
    k = rng.standard_normal((13, 1, 4))
    v = rng.standard_normal((13, 1, 4))
    dout = rng.standard_normal(q.shape)
    dq, dk, dv, wq, wk = BW.attend_varlen_backward(q, k, v, dout, cu_q, cu_k, 3, True)
    assert (dq[1:4] == 0).all() and np.abs(dq[4:7]).max() > 0
    assert (dk[3:8] == 0).all() and (dv[3:8] == 0).all()
    assert np.isnan(dq[0]).all() and np.isnan(dq[10]).all() and np.isnan(dk[12]).all()
    assert wq.tolist() == [False] + [True] * 9 + [False]


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def invariant_errors(q, k, v, dout, cu_q, cu_k, B, causal):
    """Per (sequence, KV head): the key gradients sum to zero (shifting every
    key by one vector shifts each row's scores by a constant); dv sums to the
    output gradients of the rows that see a key; and the q.dq total equals
    the k.dk total (both are sum ds * s). Returns the largest violation."""
    dq, dk, dv, _, _ = BW.attend_varlen_backward(q, k, v, dout, cu_q, cu_k, B, causal)
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    worst = 0.0
    for b in range(B):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 <= q0 or k1 <= k0:
            continue
        live = A.visible_keys(q1 - q0, k1 - k0, causal).any(axis=1)
        for hk in range(Hkv):
            hs = slice(hk * G, hk * G + G)
            worst = max(worst, float(np.abs(dk[k0:k1, hk].sum(axis=0)).max()))
            want = dout[q0:q1, hs][live].sum(axis=(0, 1))
            worst = max(worst, float(np.abs(dv[k0:k1, hk].sum(axis=0) - want).max()))
            qdq = float((q[q0:q1, hs] * dq[q0:q1, hs]).sum())
            kdk = float((k[k0:k1, hk] * dk[k0:k1, hk]).sum())
            worst = max(worst, abs(qdq - kdk))
    return worst


@pytest.mark.parametrize("seed", range(6))
def test_invariants(seed):
    rng = np.random.default_rng([23, seed])
    G = int(rng.choice([1, 2, 4]))
    q, k, v, cu_q, cu_k = _rand_case(rng, 3, 2 * G, 2, 8, 12, 14, bool(seed % 2), lead=2, tail=2)
    dout = rng.standard_normal(q.shape)
    assert invariant_errors(q, k, v, dout, cu_q, cu_k, 3, bool(seed % 2)) < 1e-11


def test_gqa_equals_mha_with_repeated_kv_heads_summed_back():
    rng = np.random.default_rng(10)
    G, Hkv = 3, 2
    q, k, v, cu_q, cu_k = _rand_case(rng, 2, G * Hkv, Hkv, 5, 7, 9, True, tail=1)
    dout = rng.standard_normal(q.shape)
    dq, dk, dv, wq, wk = BW.attend_varlen_backward(q, k, v, dout, cu_q, cu_k, 2, True)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    dq2, dk2, dv2, _, _ = BW.attend_varlen_backward(q, kr, vr, dout, cu_q, cu_k, 2, True)
    np.testing.assert_allclose(dq[wq], dq2[wq], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk[wk], dk2[wk].reshape(-1, Hkv, G, 5).sum(2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv[wk], dv2[wk].reshape(-1, Hkv, G, 5).sum(2), rtol=1e-12, atol=1e-13)
