"""Plant plausible mistakes in the backward oracle (on the CPU) and check that
a pin fails for each: finite differences of the forward oracle, torch
autograd through SDPA, or the invariants."""
import numpy as np
import pytest

from oracle import backward as BW
from tests.test_oracle_backward import (_autograd_case, _fd_case, autograd_error,
                                        finite_difference_error, invariant_errors)


def _rows(variant):
    def rows(qh, kh, vh, doh, visible, scale):
        Lq, D = qh.shape
        Lk = kh.shape[0]
        if Lq == 0 or Lk == 0:
            return np.zeros((Lq, D)), np.zeros((Lk, D)), np.zeros((Lk, vh.shape[1]))
        s = np.where(visible, scale * (qh @ kh.T), -np.inf)
        live = visible.any(axis=1)
        m = np.where(live, s.max(axis=1), 0.0)
        e = np.where(visible, np.exp(s - m[:, None]), 0.0)
        p = np.zeros_like(e)
        p[live] = e[live] / e[live].sum(axis=1)[:, None]
        dp = doh @ vh.T
        delta = (p * dp).sum(axis=1)
        ds = p * (dp - delta[:, None])
        dv = p.T @ doh
        dq = scale * (ds @ kh)
        dk = scale * (ds.T @ qh)
        if variant == "no_delta":
            ds = p * dp
            dq, dk = scale * (ds @ kh), scale * (ds.T @ qh)
        elif variant == "sign":
            dq, dk = -dq, -dk
        elif variant == "delta_without_p":
            ds = p * (dp - dp.sum(axis=1)[:, None])
            dq, dk = scale * (ds @ kh), scale * (ds.T @ qh)
        elif variant == "dk_from_p":
            dk = scale * (p.T @ qh)
        elif variant == "dq_no_scale":
            dq = ds @ kh
        elif variant == "dq_from_v":
            dq = scale * (ds @ vh)
        elif variant == "dv_from_ds":
            dv = ds.T @ doh
        elif variant == "dk_from_dout":
            dk = scale * (ds.T @ doh)
        elif variant == "dv_unmasked":                  # causal mask dropped for dv
            full = np.exp(scale * (qh @ kh.T))
            dv = (full / full.sum(axis=1, keepdims=True)).T @ doh
        return dq, dk, dv
    return rows


def _caught():
    for seed in range(4):
        if finite_difference_error(*_fd_case(seed)) > 1e-7:
            return True
    for causal in (False, True):
        if autograd_error(*_autograd_case(0, causal, 4)) > 1e-11:
            return True
    rng = np.random.default_rng(3)
    from tests.test_oracle_attention import _rand_case
    q, k, v, cu_q, cu_k = _rand_case(rng, 3, 4, 2, 8, 12, 14, True, lead=2, tail=2)
    return invariant_errors(q, k, v, rng.standard_normal(q.shape), cu_q, cu_k, 3, True) > 1e-11


ROW_MUTANTS = ["no_delta", "sign", "delta_without_p", "dk_from_p", "dq_no_scale", "dq_from_v",
               "dv_from_ds", "dk_from_dout", "dv_unmasked"]


def test_unmutated_rows_pass_every_pin(monkeypatch):
    monkeypatch.setattr(BW, "backward_rows", _rows(None))
    assert not _caught()


@pytest.mark.parametrize("variant", ROW_MUTANTS)
def test_row_mutant_is_caught(monkeypatch, variant):
    monkeypatch.setattr(BW, "backward_rows", _rows(variant))
    assert _caught()


def test_wrong_head_map_is_caught(monkeypatch):
    monkeypatch.setattr(BW, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
    assert _caught()


def test_top_left_causal_alignment_is_caught(monkeypatch):
    def top_left(Lq, Lk, causal):
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        return np.ones((Lq, Lk), bool) if not causal else j <= i
    monkeypatch.setattr(BW, "visible_keys", top_left)
    assert _caught()
