"""Pins of the padding-mask oracle: the page's exhaustive equivalence protocol.

The vectorised formula and the per-sequence loop form are two independent
statements of the mask; the page compares them over every combination of
lengths and reports the number of cases. The enumeration here re-derives that
number by counting the cases it actually runs.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import mask as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "te24_mask_equivalence.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _cu_from_lengths(lens, extra, rng):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    if extra:
        # a buffer sized for a larger maximum batch; the tail is adversarial
        tail = rng.choice([-1, 2**31 - 1, int(cu[-1]), -2**31], size=extra)
        cu = np.concatenate([cu, tail])
    return cu


def test_case_count_formula_matches_pages():
    g = _golden()
    assert M.self_attention_case_count() == g["self_attention"]["cases"]
    assert M.cross_attention_case_count() == g["cross_attention"]["cases"]


def test_exhaustive_self_attention_equivalence():
    g = _golden()["self_attention"]
    rng = np.random.default_rng(0)
    lo, hi = g["max_seqlen"]
    blo, bhi = g["batch_size"]
    cases = 0
    for max_seqlen in range(lo, hi + 1):
        for B in range(blo, bhi + 1):
            for lens in itertools.product(range(max_seqlen + 1), repeat=B):
                for extra in (0, 3):
                    cu = _cu_from_lengths(lens, extra, rng)
                    a = M.padding_mask(cu, B, max_seqlen)
                    b = M.padding_mask_loop(cu, B, max_seqlen)
                    assert a.shape == (B, 1, 1, max_seqlen) and a.dtype == bool
                    assert np.array_equal(a, b), (lens, extra)
                    cases += 1
    assert cases == g["cases"]


def test_cross_attention_enumeration_count():
    g = _golden()["cross_attention"]
    cases = 0
    for mq in range(g["max_seqlen_q"][0], g["max_seqlen_q"][1] + 1):
        for mk in range(g["max_seqlen_kv"][0], g["max_seqlen_kv"][1] + 1):
            for B in range(g["batch_size"][0], g["batch_size"][1] + 1):
                cases += ((mq + 1) * (mk + 1)) ** B
    assert cases == g["cases"]


def test_length_above_max_gives_all_false_row_and_loop_fails():
    cu = np.array([0, 3, 12, 14])      # second sequence has 9 > max 8
    m = M.padding_mask(cu, 3, 8)
    assert not m[1].any()
    assert np.array_equal(m[0, 0, 0], [False] * 3 + [True] * 5)
    with pytest.raises(M.RaggedRows):
        M.padding_mask_loop(cu, 3, 8)


def test_negative_length_gives_all_true_row():
    cu = np.array([5, 2, 4])
    m = M.padding_mask(cu, 2, 4)
    assert m[0].all()
    assert np.array_equal(m[1, 0, 0], [False, False, True, True])


def test_int32_difference_wraps():
    cu = np.array([-2**31, 2**31 - 1], dtype=np.int64)   # difference wraps to -1
    assert M.seqlens_int32(cu, 1)[0] == -1
    assert M.padding_mask(cu, 1, 3).all()
