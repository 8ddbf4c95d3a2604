"""Plant plausible mistakes in the oracle (on the CPU) and check a pin fails.

Each mutant replaces one piece of oracle.attention for the duration of a test
and re-runs the two independent references (scalar brute force and PyTorch
SDPA) against the direct and the split-KV forms. A mutant must disagree with at least one of them; otherwise the pins
would not protect against that mistake.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import brute
from tests.test_oracle_attention import _rand_case, _sdpa_reference


def _case():
    rng = np.random.default_rng(99)
    # G = 2, Hkv = 2, causal, Lq != Lk in some sequences, offset pack start
    q, k, v, cu_q, cu_k = _rand_case(rng, 3, 4, 2, 8, 5, 7, True, lead=1, tail=2)
    return q, k, v, cu_q, cu_k


def _agrees_with_references(q, k, v, cu_q, cu_k, B, causal):
    try:
        out, lse, written = A.attend_varlen(q, k, v, cu_q, cu_k, B, causal)
    except (ValueError, IndexError):
        return False          # a mutant that cannot even run is caught
    ref = brute.attend_scalar(q.tolist(), k.tolist(), v.tolist(), cu_q, cu_k, B, causal)
    for (row, h), (o, ls) in ref.items():
        if not written[row] or not np.allclose(out[row, h], o, rtol=1e-9, atol=1e-9):
            return False
        if np.isinf(ls) != np.isinf(lse[row, h]):
            return False
        if np.isfinite(ls) and abs(lse[row, h] - ls) > 1e-9:
            return False
    for q0, Lq, o, ls, live in _sdpa_reference(q, k, v, cu_q, cu_k, B, causal):
        rows = np.arange(Lq)[live]
        if not np.allclose(out[q0 + rows], o[rows], rtol=1e-9, atol=1e-9):
            return False
    # the split-KV form (partials over 3-key ranges + LSE merge) against the
    # same brute force
    try:
        out_s, lse_s, written_s = A.attend_varlen_split(q, k, v, cu_q, cu_k, B, causal, 3)
    except (ValueError, IndexError):
        return False
    for (row, h), (o, ls) in ref.items():
        if not written_s[row] or not np.allclose(out_s[row, h], o, rtol=1e-9, atol=1e-9):
            return False
        if np.isinf(ls) != np.isinf(lse_s[row, h]):
            return False
        if np.isfinite(ls) and abs(lse_s[row, h] - ls) > 1e-9:
            return False
    return True


def _top_left(Lq, Lk, causal):
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    return np.ones((Lq, Lk), bool) if not causal else (j <= i)


def _no_scale(qh, kh, vh, visible, scale):
    return _ORIG_ROWS(qh, kh, vh, visible, 1.0)


def _swap_kv(qh, kh, vh, visible, scale):
    return _ORIG_ROWS(qh, vh, kh, visible, scale)


def _unnormalised(qh, kh, vh, visible, scale):
    o, lse = _ORIG_ROWS(qh, kh, vh, visible, scale)
    return o * np.exp(lse - lse.max() if np.isfinite(lse).any() else 0)[:, None], lse


def _lse_drops_max(qh, kh, vh, visible, scale):
    o, lse = _ORIG_ROWS(qh, kh, vh, visible, scale)
    s = np.where(visible, scale * (qh @ kh.T), -np.inf)
    return o, lse - np.where(visible.any(1), s.max(1), 0)


def _lengths_from_start(cu, B, s_max=None):
    cu = np.asarray(cu, dtype=np.int64)
    return cu[:B].copy(), cu[1:B + 1] - cu[0], np.zeros(B, bool)


_ORIG_ROWS = A.attend_rows
_ORIG_MERGE = A.merge_partials


def _merge_weight_sign(o_parts, m_parts, l_parts):
    m = np.asarray(m_parts, dtype=np.float64)
    M = m.max(axis=0)
    # weights exp(M - m_s) instead of exp(m_s - M)
    return _ORIG_MERGE(o_parts, np.where(np.isfinite(m), 2 * np.where(np.isfinite(M), M, 0) - m, m),
                       l_parts)


def _merge_unweighted_l(o_parts, m_parts, l_parts):
    O, LSE, M, L = _ORIG_MERGE(o_parts, m_parts, l_parts)
    L2 = np.asarray(l_parts, dtype=np.float64).sum(axis=0)
    live = np.isfinite(M)
    O2 = np.where(live[..., None], O * (L / np.where(live, L2, 1.0))[..., None], 0.0)
    return O2, LSE, M, L2

MUTANTS = {
    "head map h % Hkv": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
    "causal top-left": ("visible_keys", _top_left),
    "scale dropped": ("attend_rows", _no_scale),
    "K and V swapped": ("attend_rows", _swap_kv),
    "output not normalised": ("attend_rows", _unnormalised),
    "LSE without the max": ("attend_rows", _lse_drops_max),
    "lengths from pack start": ("_lengths", _lengths_from_start),
    "merge weights exp(M - m)": ("merge_partials", _merge_weight_sign),
    "merge sums l unweighted": ("merge_partials", _merge_unweighted_l),
}


def test_unmutated_oracle_agrees():
    assert _agrees_with_references(*_case(), 3, True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    assert not _agrees_with_references(*_case(), 3, True), name
