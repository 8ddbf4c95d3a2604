"""fp64 varlen grouped-query attention over THD-packed sequences (oracle).

TEST INFRASTRUCTURE ONLY — see the package docstring. Pure NumPy, float64.

Definition followed (textbook scaled-dot-product attention, per sequence, per
query head):

  * THD packing: the tokens of all sequences lie back to back; sequence b owns
    rows [cu[b], cu[b+1]) of the packed tensor, and only entries 0..B of a
    cu_seqlens buffer are read — the buffer may be longer because callers
    allocate it for the maximum batch ([TE#24] Changes; [FROST#552] Context).
  * GQA head map: query head h reads KV head h // G with G = Hq / Hkv. This is
    the contiguous grouping under which [Tq, Hq, D] -> [Tq, Hkv, G, D] is the
    byte-conserving reshape that folds G into the matmul M dimension
    ([KERNBENCH] "GQA via M-fold" commit).
  * Causal visibility when Lq != Lk is aligned bottom-right: query i sees key
    j iff j <= i + (Lk - Lq). With Lq = 1 (decode) the query sees every key.
  * s_j = scale * <q_i, k_j>, scale = 1/sqrt(D); m = max s_j;
    l = sum exp(s_j - m); O = sum exp(s_j - m) v_j / l; LSE = m + ln l
    (natural log, in units of the scaled score).
  * An empty visible set gives O = 0 and LSE = -inf (ln of the empty sum,
    which is also the identity of the LSE merge below).

Split-KV partials and their merge follow [ASTRAI] (split-KV commit: blocks
emit unnormalised (O, m, l) partials that a combine kernel reduces) and
[SPLITK] (The Context: split kernel writes partial accumulator, max and
denominator; a combine kernel merges them by log-sum-exp).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _lengths(cu, B, s_max=None):
    """Offsets and lengths of sequences 0..B-1 from entries 0..B of cu.

    With s_max given, each length is clamped to [0, s_max] (the library's
    reading for invalid device data: out-of-range lengths are clamped, never
    read past). Returns (starts, lengths, clamped_flags) as int64 arrays.
    """
    cu = np.asarray(cu, dtype=np.int64)
    starts = cu[:B].copy()
    lens = cu[1:B + 1] - cu[:B]
    clamped = np.zeros(B, dtype=bool)
    if s_max is not None:
        clamped = (lens < 0) | (lens > s_max)
        lens = np.clip(lens, 0, s_max)
    return starts, lens, clamped


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: contiguous groups of G = Hq / Hkv."""
    return h // (Hq // Hkv)


def visible_keys(Lq: int, Lk: int, causal: bool) -> np.ndarray:
    """Boolean [Lq, Lk]: query i may attend key j (bottom-right causal)."""
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    if not causal:
        return np.ones((Lq, Lk), dtype=bool)
    return j <= i + (Lk - Lq)


def attend_rows(qh, kh, vh, visible, scale):
    """Attention of query rows qh [Lq, D] over keys kh/vh [Lk, D].

    Returns (O [Lq, D] fp64, LSE [Lq] fp64). Rows with no visible key give
    O = 0 and LSE = -inf.
    """
    Lq = qh.shape[0]
    D = vh.shape[1] if vh.ndim == 2 else qh.shape[1]
    out = np.zeros((Lq, D), dtype=np.float64)
    lse = np.full(Lq, NEG_INF, dtype=np.float64)
    if Lq == 0 or kh.shape[0] == 0:
        return out, lse
    s = scale * (qh @ kh.T)                       # [Lq, Lk] scores
    s = np.where(visible, s, NEG_INF)
    live = visible.any(axis=1)
    m = np.where(live, s.max(axis=1), 0.0)         # row max over visible keys
    p = np.where(visible, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    out[live] = (p[live] @ vh) / l[live, None]
    lse[live] = m[live] + np.log(l[live])
    return out, lse


def attend_varlen(q, k, v, cu_q, cu_kv, B, causal, scale=None,
                  s_max_q=None, s_max_kv=None):
    """Varlen GQA attention, fp64.

    q: [Tq, Hq, D], k/v: [Tkv, Hkv, D] (any real dtype; converted to fp64
    exactly), cu_q/cu_kv: integer offsets with at least B+1 entries.

    Returns (out, lse, written):
      out [Tq, Hq, D] fp64 and lse [Tq, Hq] fp64, NaN on rows that belong to
      no sequence; written [Tq] bool marks the rows the method defines.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((Tq, Hq, D), np.nan)
    lse = np.full((Tq, Hq), np.nan)
    written = np.zeros(Tq, dtype=bool)
    q0s, Lqs, _ = _lengths(cu_q, B, s_max_q)
    k0s, Lks, _ = _lengths(cu_kv, B, s_max_kv)
    for b in range(B):
        q0, Lq, k0, Lk = int(q0s[b]), int(Lqs[b]), int(k0s[b]), int(Lks[b])
        if Lq == 0:
            continue
        vis = visible_keys(Lq, Lk, causal)
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            o, ls = attend_rows(q[q0:q0 + Lq, h, :], k[k0:k0 + Lk, hk, :],
                                v[k0:k0 + Lk, hk, :], vis, scale)
            out[q0:q0 + Lq, h, :] = o
            lse[q0:q0 + Lq, h] = ls
        written[q0:q0 + Lq] = True
    return out, lse, written


# ---------------------------------------------------------------------------
# Split-KV partials and the log-sum-exp merge
# ---------------------------------------------------------------------------

def partial_rows(qh, kh, vh, visible, scale):
    """Unnormalised partial state of query rows over a key range.

    Returns (O_unnorm [Lq, D], m [Lq], l [Lq]) with m the max visible score,
    l = sum exp(s - m) and O_unnorm = sum exp(s - m) v. An empty range gives
    the merge identity (0, -inf, 0).
    """
    Lq = qh.shape[0]
    D = vh.shape[1]
    o = np.zeros((Lq, D))
    m = np.full(Lq, NEG_INF)
    l = np.zeros(Lq)
    if Lq == 0 or kh.shape[0] == 0:
        return o, m, l
    s = np.where(visible, scale * (qh @ kh.T), NEG_INF)
    live = visible.any(axis=1)
    m[live] = s[live].max(axis=1)
    p = np.where(visible, np.exp(s - np.where(live, m, 0.0)[:, None]), 0.0)
    l[live] = p[live].sum(axis=1)
    o[live] = p[live] @ vh
    return o, m, l


def merge_partials(o_parts, m_parts, l_parts):
    """LSE merge of partials along axis 0.

    o_parts [S, ..., D], m_parts/l_parts [S, ...]. Returns (O, LSE, M, L):
    M = max_s m_s; w_s = exp(m_s - M) (0 for an empty partial);
    L = sum w_s l_s; O = sum w_s O_s / L; LSE = M + ln L. If every partial is
    empty: O = 0, LSE = -inf.
    """
    m_parts = np.asarray(m_parts, dtype=np.float64)
    l_parts = np.asarray(l_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    M = m_parts.max(axis=0)
    live = np.isfinite(M)
    Msafe = np.where(live, M, 0.0)
    w = np.where(np.isfinite(m_parts), np.exp(m_parts - Msafe), 0.0)
    L = (w * l_parts).sum(axis=0)
    num = (w[..., None] * o_parts).sum(axis=0)
    O = np.where(live[..., None], num / np.where(live, L, 1.0)[..., None], 0.0)
    LSE = np.where(live, M + np.log(np.where(live, L, 1.0)), NEG_INF)
    return O, LSE, M, L


def merge_two(a, b):
    """Merge two partial states (O_unnorm, m, l) into one (O_unnorm, m, l).

    The associative, commutative operator whose identity is (0, -inf, 0):
    M = max(m_a, m_b); O = e^{m_a-M} O_a + e^{m_b-M} O_b; l likewise.
    """
    oa, ma, la = (np.asarray(x, dtype=np.float64) for x in a)
    ob, mb, lb = (np.asarray(x, dtype=np.float64) for x in b)
    M = np.maximum(ma, mb)
    live = np.isfinite(M)
    Ms = np.where(live, M, 0.0)
    wa = np.where(np.isfinite(ma), np.exp(ma - Ms), 0.0)
    wb = np.where(np.isfinite(mb), np.exp(mb - Ms), 0.0)
    return (wa[..., None] * oa + wb[..., None] * ob, M, wa * la + wb * lb)


def attend_varlen_split(q, k, v, cu_q, cu_kv, B, causal, chunk, scale=None,
                        s_max_q=None, s_max_kv=None):
    """Same result as attend_varlen, computed as split-KV partials + merge.

    Sequence b's keys are cut into contiguous ranges [s*chunk, (s+1)*chunk);
    each range yields a partial (O_unnorm, m, l) for every query row; the
    partials are merged by merge_partials. Returns (out, lse, written).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((Tq, Hq, D), np.nan)
    lse = np.full((Tq, Hq), np.nan)
    written = np.zeros(Tq, dtype=bool)
    q0s, Lqs, _ = _lengths(cu_q, B, s_max_q)
    k0s, Lks, _ = _lengths(cu_kv, B, s_max_kv)
    for b in range(B):
        q0, Lq, k0, Lk = int(q0s[b]), int(Lqs[b]), int(k0s[b]), int(Lks[b])
        if Lq == 0:
            continue
        vis = visible_keys(Lq, Lk, causal)
        nsplit = max(1, -(-Lk // chunk))
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            parts = []
            for s in range(nsplit):
                a, e = s * chunk, min((s + 1) * chunk, Lk)
                parts.append(partial_rows(q[q0:q0 + Lq, h, :],
                                          k[k0 + a:k0 + e, hk, :],
                                          v[k0 + a:k0 + e, hk, :],
                                          vis[:, a:e], scale))
            O, LSE, _, _ = merge_partials([p[0] for p in parts],
                                          [p[1] for p in parts],
                                          [p[2] for p in parts])
            out[q0:q0 + Lq, h, :] = O
            lse[q0:q0 + Lq, h] = LSE
        written[q0:q0 + Lq] = True
    return out, lse, written


def causal_pairs(cu_q, cu_kv, B, causal, s_max_q=None, s_max_kv=None):
    """Number of visible (query, key) pairs per head, summed over sequences.

    The algorithmic work of prefill is 4 * Hq * D * pairs flop (two
    contractions of 2*D flop per visible pair).
    """
    _, Lqs, _ = _lengths(cu_q, B, s_max_q)
    _, Lks, _ = _lengths(cu_kv, B, s_max_kv)
    total = 0
    for Lq, Lk in zip(Lqs.tolist(), Lks.tolist()):
        if not causal:
            total += Lq * Lk
            continue
        for i in range(Lq):
            total += max(0, min(Lk, i + (Lk - Lq) + 1))
    return total


def attend_selected(q, k, v, cu_q, cu_kv, causal, picks, scale=None):
    """Oracle values for selected (sequence b, query index i, head h) rows only.

    Same definition as attend_varlen, evaluated one row at a time so that a
    large workload can be checked on a sample. Returns a list of
    (row, h, O [D] fp64, LSE fp64).
    """
    D = q.shape[2]
    Hq, Hkv = q.shape[1], k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    res = []
    for b, i, h in picks:
        q0, Lq = int(cu_q[b]), int(cu_q[b + 1]) - int(cu_q[b])
        k0, Lk = int(cu_kv[b]), int(cu_kv[b + 1]) - int(cu_kv[b])
        hk = kv_head_of(h, Hq, Hkv)
        vis = visible_keys(Lq, Lk, causal)[i:i + 1]
        o, ls = attend_rows(np.asarray(q[q0 + i:q0 + i + 1, h, :], dtype=np.float64),
                            np.asarray(k[k0:k0 + Lk, hk, :], dtype=np.float64),
                            np.asarray(v[k0:k0 + Lk, hk, :], dtype=np.float64), vis, scale)
        res.append((q0 + i, h, o[0], ls[0]))
    return res


def attend_gathered(q, k, v, cu_q, cu_idx, kv_idx, B, scale=None, s_max_q=None,
                    s_max_kv=None, kv_rows=None):
    """Attention over gathered keys (split-K blog post, The Context: Why
    Split-K Matters -- each query head attends to a selected list of cached
    tokens): sequence b's query rows cu_q[b]..cu_q[b+1] attend, without
    causal masking, to the K/V rows kv_idx[cu_idx[b] .. cu_idx[b+1]) in that
    list's order (a row listed twice counts twice). Reading for invalid data,
    as for lengths: a row index outside [0, kv_rows) is clamped into range
    and reported. Returns (out, lse, written, index_clamped).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kv_idx = np.asarray(kv_idx, dtype=np.int64)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    if kv_rows is None:
        kv_rows = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((Tq, Hq, D), np.nan)
    lse = np.full((Tq, Hq), np.nan)
    written = np.zeros(Tq, dtype=bool)
    clamped_any = False
    q0s, Lqs, _ = _lengths(cu_q, B, s_max_q)
    i0s, Lks, _ = _lengths(cu_idx, B, s_max_kv)
    for b in range(B):
        q0, Lq, i0, Lk = int(q0s[b]), int(Lqs[b]), int(i0s[b]), int(Lks[b])
        if Lq == 0:
            continue
        rows = kv_idx[i0:i0 + Lk]
        bad = (rows < 0) | (rows >= kv_rows)
        clamped_any = clamped_any or bool(bad.any())
        rows = np.clip(rows, 0, kv_rows - 1)
        vis = np.ones((Lq, Lk), dtype=bool)
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            o, ls = attend_rows(q[q0:q0 + Lq, h, :], k[rows, hk, :], v[rows, hk, :], vis, scale)
            out[q0:q0 + Lq, h, :] = o
            lse[q0:q0 + Lq, h] = ls
        written[q0:q0 + Lq] = True
    return out, lse, written, clamped_any
