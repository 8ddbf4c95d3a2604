"""fp64 gradients of varlen grouped-query attention (oracle).

TEST INFRASTRUCTURE ONLY — see the package docstring. Pure NumPy, float64.

What is computed: the gradients of the scalar L = sum(dO * O) with respect to
q, k and v, where O is the attention of oracle.attention (same THD packing,
contiguous GQA head map, bottom-right causal visibility, scale 1/sqrt(D)) and
dO is the given output gradient. The pages name a THD backward with the same
packed/strided contract as the forward ([FROST#552] Related: the THD backward
contract) but give no formula; the formula is the derivative of the forward
definition, written out by the chain rule through the softmax, per sequence
and query head, over the visible pairs (i, j) only:

  s_ij   = scale * <q_i, k_j>
  p_ij   = exp(s_ij - LSE_i)            (the row's softmax weights)
  dv_j  += p_ij * dO_i                  (summed over the query heads of the
                                         group that reads this KV head)
  dp_ij  = <dO_i, v_j>
  delta_i = sum_j p_ij * dp_ij          (equals <dO_i, O_i>)
  ds_ij  = p_ij * (dp_ij - delta_i)
  dq_i   = scale * sum_j ds_ij * k_j
  dk_j  += scale * ds_ij * q_i          (summed over the group as for dv)

A query row with no visible key has O = 0 and no dependence on any input:
dq_i = 0 and it adds nothing to dk, dv. Keys of a sequence that no query sees
(a sequence with Lq = 0) get dk = dv = 0.
"""
from __future__ import annotations

import numpy as np

from oracle.attention import _lengths, kv_head_of, visible_keys


def backward_rows(qh, kh, vh, doh, visible, scale):
    """Gradients for one query head's rows against one KV head's keys.

    qh [Lq, D], kh/vh [Lk, D], doh [Lq, D], visible [Lq, Lk] bool.
    Returns (dq [Lq, D], dk [Lk, D], dv [Lk, D]) in fp64.
    """
    Lq, D = qh.shape
    Lk = kh.shape[0]
    dq = np.zeros((Lq, D))
    dk = np.zeros((Lk, D))
    dv = np.zeros((Lk, vh.shape[1]))
    if Lq == 0 or Lk == 0:
        return dq, dk, dv
    s = np.where(visible, scale * (qh @ kh.T), -np.inf)
    live = visible.any(axis=1)
    m = np.where(live, s.max(axis=1), 0.0)
    e = np.where(visible, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    p[live] = e[live] / l[live, None]        # softmax weights; 0 off the visible set
    dv = p.T @ doh
    dp = doh @ vh.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    return dq, dk, dv


def attend_varlen_backward(q, k, v, dout, cu_q, cu_kv, B, causal, scale=None,
                           s_max_q=None, s_max_kv=None):
    """Gradients of sum(dout * attention(q, k, v)) over a THD pack, fp64.

    q, dout: [Tq, Hq, D]; k, v: [Tkv, Hkv, D]; cu_q/cu_kv: offsets with at
    least B+1 entries (only 0..B are read). Lengths are clamped to
    [0, s_max] when s_max is given, as in the forward.

    Returns (dq, dk, dv, written_q, written_kv): dq [Tq, Hq, D], dk/dv
    [Tkv, Hkv, D] in fp64, NaN on rows that belong to no sequence; the
    written masks mark the rows the method defines.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    assert Hq % Hkv == 0 and dout.shape == q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    wq = np.zeros(Tq, dtype=bool)
    wk = np.zeros(Tk, dtype=bool)
    q0s, Lqs, _ = _lengths(cu_q, B, s_max_q)
    k0s, Lks, _ = _lengths(cu_kv, B, s_max_kv)
    for b in range(B):
        q0, Lq, k0, Lk = int(q0s[b]), int(Lqs[b]), int(k0s[b]), int(Lks[b])
        vis = visible_keys(Lq, Lk, causal)
        dk[k0:k0 + Lk] = 0.0
        dv[k0:k0 + Lk] = 0.0
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            gq, gk, gv = backward_rows(q[q0:q0 + Lq, h], k[k0:k0 + Lk, hk], v[k0:k0 + Lk, hk],
                                       dout[q0:q0 + Lq, h], vis, scale)
            dq[q0:q0 + Lq, h] = gq
            dk[k0:k0 + Lk, hk] += gk
            dv[k0:k0 + Lk, hk] += gv
        wq[q0:q0 + Lq] = True
        wk[k0:k0 + Lk] = True
    return dq, dk, dv, wq, wk

