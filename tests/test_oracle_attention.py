"""Pins of the fp64 attention oracle against things other than itself.

Each test below pins oracle.attention to an independent statement of the
result: scalar brute force, PyTorch's scaled_dot_product_attention and
logsumexp (a library routine, CPU fp64), closed forms, and invariants of the
mathematics. Together they fail for a dropped scale, a wrong head map, a
top-left causal alignment, swapped K/V, a wrong offset or an un-normalised
output (see test_oracle_mutants.py, which plants those mistakes).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import brute
from oracle.bf16 import round_bf16, bf16_bits, bits_to_f64


def _rand_case(rng, B, Hq, Hkv, D, max_q, max_k, causal, lead=0, tail=0,
               equal_len=False):
    lq = rng.integers(0, max_q + 1, size=B)
    lk = lq.copy() if equal_len else rng.integers(0, max_k + 1, size=B)
    cu_q = np.concatenate([[lead], lead + np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[lead], lead + np.cumsum(lk)]).astype(np.int64)
    # trailing garbage entries beyond B must never be read
    cu_q = np.concatenate([cu_q, rng.integers(-5, 5, size=tail)])
    cu_k = np.concatenate([cu_k, rng.integers(-5, 5, size=tail)])
    Tq = int(cu_q[B]) + 2
    Tk = int(cu_k[B]) + 2
    q = rng.standard_normal((Tq, Hq, D))
    k = rng.standard_normal((Tk, Hkv, D))
    v = rng.standard_normal((Tk, Hkv, D))
    return q, k, v, cu_q, cu_k


@pytest.mark.parametrize("seed", range(12))
def test_matches_scalar_brute_force(seed):
    rng = np.random.default_rng([7, seed])
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3]))
    Hq = Hkv * G
    D = int(rng.choice([2, 3, 5, 8]))
    B = int(rng.integers(1, 4))
    causal = bool(seed % 2)
    q, k, v, cu_q, cu_k = _rand_case(rng, B, Hq, Hkv, D, 6, 8, causal,
                                     lead=int(rng.integers(0, 3)), tail=2)
    out, lse, written = A.attend_varlen(q, k, v, cu_q, cu_k, B, causal)
    ref = brute.attend_scalar(q.tolist(), k.tolist(), v.tolist(), cu_q, cu_k, B, causal)
    assert written.sum() == len(ref) // Hq
    for (row, h), (o, ls) in ref.items():
        assert written[row]
        np.testing.assert_allclose(out[row, h], o, rtol=1e-12, atol=1e-12)
        if math.isinf(ls):
            assert lse[row, h] == -np.inf
        else:
            assert abs(lse[row, h] - ls) <= 1e-12 * max(1.0, abs(ls))
    # rows that belong to no sequence are left undefined
    assert np.isnan(out[~written]).all() and np.isnan(lse[~written]).all()


@pytest.mark.parametrize("seed", range(6))
def test_selected_rows_match_scalar_brute_force(seed):
    """attend_selected (the row-at-a-time form used to sample large workloads)
    against the scalar triple loops, on every (sequence, query, head) triple
    of a tiny ragged pack, causal and not, with Lq != Lk."""
    rng = np.random.default_rng([8, seed])
    Hkv, G = int(rng.choice([1, 2])), int(rng.choice([1, 3]))
    Hq, D, B = Hkv * G, int(rng.choice([3, 8])), int(rng.integers(1, 4))
    causal = bool(seed % 2)
    q, k, v, cu_q, cu_k = _rand_case(rng, B, Hq, Hkv, D, 5, 7, causal, lead=1, tail=2)
    ref = brute.attend_scalar(q.tolist(), k.tolist(), v.tolist(), cu_q, cu_k, B, causal)
    picks = [(b, i, h) for b in range(B) for i in range(int(cu_q[b + 1] - cu_q[b]))
             for h in range(Hq)]
    picks = [picks[j] for j in rng.permutation(len(picks))]
    got = A.attend_selected(q, k, v, cu_q, cu_k, causal, picks)
    assert len(got) == len(picks) == len(ref)
    for (b, i, h), (row, hh, o, ls) in zip(picks, got):
        assert (row, hh) == (int(cu_q[b]) + i, h)
        ro, rl = ref[(row, h)]
        np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
        if math.isinf(rl):
            assert ls == -np.inf and not o.any()
        else:
            assert abs(ls - rl) <= 1e-12 * max(1.0, abs(rl))


def _sdpa_reference(q, k, v, cu_q, cu_k, B, causal):
    """PyTorch CPU fp64: SDPA with an explicit boolean mask, GQA expanded to
    MHA by repeating each KV head G times (head h reads KV head h // G)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    res = []
    for b in range(B):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        qt = torch.from_numpy(q[q0:q1]).permute(1, 0, 2)            # [Hq, Lq, D]
        kt = torch.from_numpy(k[k0:k1]).permute(1, 0, 2).repeat_interleave(G, 0)
        vt = torch.from_numpy(v[k0:k1]).permute(1, 0, 2).repeat_interleave(G, 0)
        if causal:
            mask = torch.ones(Lq, Lk, dtype=torch.bool).tril(diagonal=Lk - Lq)
        else:
            mask = torch.ones(Lq, Lk, dtype=torch.bool)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        s = (qt @ kt.transpose(1, 2)) / math.sqrt(q.shape[2])
        lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
        res.append((q0, Lq, o.permute(1, 0, 2).numpy(), lse.T.numpy(), mask.any(1).numpy()))
    return res


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G", [1, 4])
def test_matches_torch_sdpa(causal, G):
    rng = np.random.default_rng([11, G, int(causal)])
    Hkv, D, B = 2, 16, 3
    q, k, v, cu_q, cu_k = _rand_case(rng, B, Hkv * G, Hkv, D, 20, 30, causal, lead=1, tail=3)
    out, lse, _ = A.attend_varlen(q, k, v, cu_q, cu_k, B, causal)
    for q0, Lq, o, ls, live in _sdpa_reference(q, k, v, cu_q, cu_k, B, causal):
        rows = np.arange(Lq)[live]
        np.testing.assert_allclose(out[q0 + rows], o[rows], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse[q0 + rows], ls[rows], rtol=1e-12, atol=1e-12)
        dead = np.arange(Lq)[~live]
        assert (out[q0 + dead] == 0).all() and (lse[q0 + dead] == -np.inf).all()


def test_single_key_returns_that_value_row_exactly():
    rng = np.random.default_rng(3)
    D, Hq, Hkv = 64, 8, 2
    vals = bits_to_f64(bf16_bits(rng.standard_normal((4, Hkv, D))))
    q = bits_to_f64(bf16_bits(rng.standard_normal((4, Hq, D))))
    k = bits_to_f64(bf16_bits(rng.standard_normal((4, Hkv, D))))
    cu = np.arange(5)
    out, lse, _ = A.attend_varlen(q, k, vals, cu, cu, 4, causal=False)
    for t in range(4):
        for h in range(Hq):
            assert np.array_equal(bf16_bits(out[t, h]), bf16_bits(vals[t, h // (Hq // Hkv)]))
            s0 = float(q[t, h] @ k[t, h // (Hq // Hkv)]) / 8.0
            assert abs(lse[t, h] - s0) <= 1e-12 * max(1, abs(s0))


def test_equal_value_rows_give_that_row_after_rounding():
    rng = np.random.default_rng(4)
    D, L = 32, 300
    row = bits_to_f64(bf16_bits(rng.standard_normal(D)))
    v = np.broadcast_to(row, (L, 1, D)).copy()
    q = rng.standard_normal((1, 4, D))
    k = rng.standard_normal((L, 1, D))
    out, _, _ = A.attend_varlen(q, k, v, [0, 1], [0, L], 1, causal=False)
    for h in range(4):
        assert np.array_equal(bf16_bits(out[0, h]), bf16_bits(row))


@pytest.mark.parametrize("L", [1, 2, 7, 128, 32768])
def test_zero_query_gives_log_length_and_mean_value(L):
    rng = np.random.default_rng(L)
    D = 16
    q = np.zeros((1, 2, D))
    k = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    out, lse, _ = A.attend_varlen(q, k, v, [0, 1], [0, L], 1, causal=False)
    assert abs(lse[0, 0] - math.log(L)) <= 1e-12 * max(1.0, math.log(L))
    if L == 32768:
        assert abs(lse[0, 0] - 15 * math.log(2)) < 1e-12
    np.testing.assert_allclose(out[0, 0], v[:, 0].mean(axis=0), rtol=1e-11, atol=1e-13)


def test_causal_first_query_sees_only_first_key_and_last_query_sees_all():
    rng = np.random.default_rng(5)
    lens = [1, 5, 33, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, D = int(cu[-1]), 4, 2, 32
    q = bits_to_f64(bf16_bits(rng.standard_normal((T, Hq, D))))
    k = bits_to_f64(bf16_bits(rng.standard_normal((T, Hkv, D))))
    v = bits_to_f64(bf16_bits(rng.standard_normal((T, Hkv, D))))
    out, lse, _ = A.attend_varlen(q, k, v, cu, cu, len(lens), causal=True)
    for b, L in enumerate(lens):
        s0 = int(cu[b])
        for h in range(Hq):
            assert np.array_equal(bf16_bits(out[s0, h]), bf16_bits(v[s0, h // 2]))
        # last query of a causal sequence == decode of that query over all keys
        last = s0 + L - 1
        o_dec, l_dec, _ = A.attend_varlen(q[last:last + 1], k[s0:s0 + L], v[s0:s0 + L],
                                          [0, 1], [0, L], 1, causal=False)
        np.testing.assert_allclose(out[last], o_dec[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[last], l_dec[0], rtol=1e-13)


def test_causal_rows_with_no_visible_key():
    # Lq > Lk: the first Lq - Lk queries see nothing under bottom-right alignment
    rng = np.random.default_rng(6)
    q = rng.standard_normal((5, 2, 8))
    k = rng.standard_normal((2, 1, 8))
    v = rng.standard_normal((2, 1, 8))
    out, lse, _ = A.attend_varlen(q, k, v, [0, 5], [0, 2], 1, causal=True)
    assert (out[:3] == 0).all() and (lse[:3] == -np.inf).all()
    assert np.isfinite(lse[3:]).all()
    # empty KV sequence in decode
    out, lse, _ = A.attend_varlen(q[:1], k[:0], v[:0], [0, 1], [0, 0], 1, causal=False)
    assert (out[0] == 0).all() and (lse[0] == -np.inf).all()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("chunk", [1, 2, 3, 7, 32, 1000])
def test_split_merge_equals_direct(causal, chunk):
    rng = np.random.default_rng([8, chunk, int(causal)])
    q, k, v, cu_q, cu_k = _rand_case(rng, 4, 8, 2, 16, 1 if not causal else 12, 90,
                                     causal, equal_len=causal)
    o1, l1, w1 = A.attend_varlen(q, k, v, cu_q, cu_k, 4, causal)
    o2, l2, w2 = A.attend_varlen_split(q, k, v, cu_q, cu_k, 4, causal, chunk)
    assert (w1 == w2).all()
    np.testing.assert_allclose(o2[w1], o1[w1], rtol=1e-12, atol=1e-13)
    fin = np.isfinite(l1[w1])
    np.testing.assert_array_equal(np.isfinite(l2[w1]), fin)
    np.testing.assert_allclose(l2[w1][fin], l1[w1][fin], rtol=1e-12, atol=1e-13)


def test_merge_is_associative_commutative_with_identity():
    rng = np.random.default_rng(9)
    D = 8

    def part(n):
        s = rng.standard_normal(n) * 3
        vv = rng.standard_normal((n, D))
        m = s.max()
        p = np.exp(s - m)
        return (p @ vv, np.float64(m), np.float64(p.sum())), (s, vv)

    (a, ra), (b, rb), (c, rc) = part(5), part(9), part(2)
    ident = (np.zeros(D), np.float64(-np.inf), np.float64(0.0))
    ab_c = A.merge_two(A.merge_two(a, b), c)
    a_bc = A.merge_two(a, A.merge_two(b, c))
    for x, y in zip(ab_c, a_bc):
        np.testing.assert_allclose(x, y, rtol=1e-13)
    for x, y in zip(A.merge_two(a, b), A.merge_two(b, a)):
        np.testing.assert_allclose(x, y, rtol=1e-15)
    for x, y in zip(A.merge_two(a, ident), a):
        np.testing.assert_allclose(x, y, rtol=0)
    both = A.merge_two(ident, ident)
    assert both[1] == -np.inf and both[2] == 0 and (both[0] == 0).all()
    # merged state == state of the concatenated scores (closed form)
    s = np.concatenate([ra[0], rb[0], rc[0]])
    vv = np.concatenate([ra[1], rb[1], rc[1]])
    M = s.max()
    np.testing.assert_allclose(ab_c[1], M, rtol=0)
    np.testing.assert_allclose(ab_c[2], np.exp(s - M).sum(), rtol=1e-13)
    np.testing.assert_allclose(ab_c[0], np.exp(s - M) @ vv, rtol=1e-12)
    O, LSE, _, _ = A.merge_partials([a[0], b[0], c[0]], [a[1], b[1], c[1]], [a[2], b[2], c[2]])
    np.testing.assert_allclose(LSE, M + np.log(np.exp(s - M).sum()), rtol=1e-14)
    np.testing.assert_allclose(O, (np.exp(s - M) @ vv) / np.exp(s - M).sum(), rtol=1e-12)
    O, LSE, _, _ = A.merge_partials([ident[0]] * 3, [ident[1]] * 3, [ident[2]] * 3)
    assert LSE == -np.inf and (O == 0).all()


def test_noncausal_invariant_to_key_and_sequence_permutation():
    rng = np.random.default_rng(10)
    lens = [3, 0, 11, 6]
    B, Hq, Hkv, D = 4, 6, 3, 8
    cu_k = np.concatenate([[0], np.cumsum(lens)])
    cu_q = np.arange(B + 1)
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((int(cu_k[-1]), Hkv, D))
    v = rng.standard_normal((int(cu_k[-1]), Hkv, D))
    o, l, _ = A.attend_varlen(q, k, v, cu_q, cu_k, B, False)
    # permute keys inside each sequence
    perm = np.concatenate([cu_k[b] + rng.permutation(lens[b]) for b in range(B)]).astype(int)
    o2, l2, _ = A.attend_varlen(q, k[perm], v[perm], cu_q, cu_k, B, False)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l, rtol=1e-13)
    # permute sequences in the pack
    order = [2, 0, 3, 1]
    k3 = np.concatenate([k[cu_k[b]:cu_k[b + 1]] for b in order])
    v3 = np.concatenate([v[cu_k[b]:cu_k[b + 1]] for b in order])
    cu_k3 = np.concatenate([[0], np.cumsum([lens[b] for b in order])])
    o3, l3, _ = A.attend_varlen(q[order], k3, v3, cu_q, cu_k3, B, False)
    np.testing.assert_allclose(o3, o[order], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l3, l[order], rtol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(12)
    G, Hkv, D = 4, 2, 8
    q, k, v, cu_q, cu_k = _rand_case(rng, 2, G * Hkv, Hkv, D, 5, 9, True, equal_len=True)
    o, l, _ = A.attend_varlen(q, k, v, cu_q, cu_k, 2, True)
    o2, l2, _ = A.attend_varlen(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                                cu_q, cu_k, 2, True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_clamp_policy_for_out_of_range_lengths():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((4, 2, 8))
    k = rng.standard_normal((40, 1, 8))
    v = rng.standard_normal((40, 1, 8))
    # length 30 > s_max 16 is read as 16; a negative length as 0
    cu_q = [0, 1, 2]
    cu_k = [0, 30, 25]
    o, l, _ = A.attend_varlen(q, k, v, cu_q, cu_k, 2, False, s_max_kv=16)
    o_ref, l_ref, _ = A.attend_varlen(q, k, v, [0, 1], [0, 16], 1, False)
    np.testing.assert_array_equal(o[0], o_ref[0])
    assert (o[1] == 0).all() and (l[1] == -np.inf).all()


def test_causal_pair_count_closed_form():
    lens = [1, 2, 64, 4096, 100]
    cu = np.concatenate([[0], np.cumsum(lens)])
    assert A.causal_pairs(cu, cu, len(lens), True) == sum(L * (L + 1) // 2 for L in lens)
    assert A.causal_pairs(cu, cu, len(lens), False) == sum(L * L for L in lens)
    # decode (Lq = 1) sees every key
    cq = np.arange(len(lens) + 1)
    assert A.causal_pairs(cq, cu, len(lens), True) == sum(lens)


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(14)
    x32 = rng.standard_normal(20000).astype(np.float32) * np.float32(4.0) ** rng.integers(-20, 20, 20000)
    ties = (np.frombuffer(rng.bytes(4 * 5000), dtype=np.uint32) & 0x3FFF0000) | 0x8000
    x32 = np.concatenate([x32, ties.view(np.float32)])
    t = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x32.astype(np.float64)), t)


def test_bf16_rounding_is_single_rounding_of_fp64():
    # 1 + 2^-8 + 2^-40 lies just above the bf16 tie point between 1 and
    # 1 + 2^-7: correct rounding goes up. Rounding first to fp32 would land on
    # the tie and then round to even (down).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert round_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert round_bf16(np.array([3.5e38]))[0] == np.inf
    assert round_bf16(np.array([2.0 ** -133]))[0] == 2.0 ** -133



def _gather_case(rng, B, Hq, Hkv, D, n_rows, max_sel, dup=True):
    q_lens = rng.integers(0, 3, size=B)
    sel = rng.integers(0, max_sel + 1, size=B)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    cu_idx = np.concatenate([[0], np.cumsum(sel)]).astype(np.int64)
    idx = rng.integers(0, n_rows, size=int(cu_idx[-1]))
    if dup and idx.size > 2:
        idx[1] = idx[0]
    q = rng.standard_normal((max(1, int(cu_q[-1])), Hq, D))
    k = rng.standard_normal((n_rows, Hkv, D))
    v = rng.standard_normal((n_rows, Hkv, D))
    return q, k, v, cu_q, cu_idx, idx


@pytest.mark.parametrize("seed", range(5))
def test_gathered_matches_brute_force_on_gathered_copies(seed):
    """Gathering then attending equals the scalar triple loops run on
    contiguous copies of the gathered rows (duplicates included)."""
    rng = np.random.default_rng([9, seed])
    Hkv, G = int(rng.choice([1, 2])), int(rng.choice([1, 2]))
    Hq, D, B = Hkv * G, 4, int(rng.integers(1, 4))
    q, k, v, cu_q, cu_idx, idx = _gather_case(rng, B, Hq, Hkv, D, 9, 6)
    out, lse, written, clamped = A.attend_gathered(q, k, v, cu_q, cu_idx, idx, B)
    assert not clamped
    kg, vg = k[idx], v[idx]
    ref = brute.attend_scalar(q.tolist(), kg.tolist(), vg.tolist(), cu_q, cu_idx, B, False)
    assert written.sum() == len(ref) // Hq
    for (row, h), (o, ls) in ref.items():
        np.testing.assert_allclose(out[row, h], o, rtol=1e-12, atol=1e-12)
        if math.isinf(ls):
            assert lse[row, h] == -np.inf
        else:
            assert abs(lse[row, h] - ls) <= 1e-12 * max(1.0, abs(ls))


def test_identity_gather_equals_contiguous_attention():
    rng = np.random.default_rng(11)
    q, k, v, cu_q, cu_k = _rand_case(rng, 3, 4, 2, 8, 2, 9, False)
    idx = np.arange(int(cu_k[3]))
    o1, l1, w1, _ = A.attend_gathered(q, k, v, cu_q, cu_k[:4], idx, 3)
    o2, l2, w2 = A.attend_varlen(q, k, v, cu_q, cu_k, 3, False)
    assert (w1 == w2).all()
    np.testing.assert_allclose(o1[w1], o2[w2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1[w1], l2[w2], rtol=1e-12, atol=1e-12)


def test_gathered_is_invariant_to_index_order():
    rng = np.random.default_rng(12)
    q, k, v, cu_q, cu_idx, idx = _gather_case(rng, 3, 4, 2, 8, 20, 7)
    o1, l1, w, _ = A.attend_gathered(q, k, v, cu_q, cu_idx, idx, 3)
    perm = idx.copy()
    for b in range(3):
        a, e = int(cu_idx[b]), int(cu_idx[b + 1])
        perm[a:e] = rng.permutation(perm[a:e])
    o2, l2, _, _ = A.attend_gathered(q, k, v, cu_q, cu_idx, perm, 3)
    np.testing.assert_allclose(o1[w], o2[w], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1[w], l2[w], rtol=1e-12, atol=1e-12)


def test_gathered_clamps_out_of_range_rows():
    rng = np.random.default_rng(13)
    q, k, v, _, _, _ = _gather_case(rng, 1, 2, 1, 8, 10, 4)
    cu_q = np.array([0, 1])
    cu_idx = np.array([0, 3])
    o1, l1, _, c1 = A.attend_gathered(q, k, v, cu_q, cu_idx, np.array([-5, 4, 99]), 1)
    o2, l2, _, c2 = A.attend_gathered(q, k, v, cu_q, cu_idx, np.array([0, 4, 9]), 1)
    assert c1 and not c2
    np.testing.assert_array_equal(o1[:1], o2[:1])
    np.testing.assert_array_equal(l1[:1], l2[:1])
