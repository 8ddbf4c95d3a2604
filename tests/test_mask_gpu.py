"""Padding mask on the GPU vs the oracle, bit-exact (the page's exhaustive
self-attention protocol, 35368 cases, plus a long-row case)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import mask as M
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_exhaustive_self_attention_cases():
    import varlen_gqa_attention_amd as V
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "te24_mask_equivalence.json")))["self_attention"]
    rng = np.random.default_rng(0)
    cases = []
    for max_seqlen in range(g["max_seqlen"][0], g["max_seqlen"][1] + 1):
        for B in range(g["batch_size"][0], g["batch_size"][1] + 1):
            for lens in itertools.product(range(max_seqlen + 1), repeat=B):
                for extra in (0, 3):
                    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
                    if extra:
                        cu = np.concatenate([cu, rng.choice([-1, 2**31 - 1, -2**31], size=extra)])
                    cases.append((B, max_seqlen, cu.astype(np.int32)))
    assert len(cases) == g["cases"]
    print(f"[mask] {len(cases)} cases", flush=True)
    # pack every case's cu vector and output at its own offset of one buffer each
    cu_off, out_off = [0], [0]
    for B, ms, cu in cases:
        cu_off.append(cu_off[-1] + cu.size)
        out_off.append(out_off[-1] + ((B * ms + 15) // 16) * 16)
    cu_all = torch.from_numpy(np.concatenate([c for _, _, c in cases])).cuda()
    out_all = torch.full((out_off[-1],), True, dtype=torch.bool, device="cuda")
    for i, (B, ms, cu) in enumerate(cases):
        V.padding_mask(cu_all[cu_off[i]:cu_off[i + 1]], B, ms,
                       out=out_all[out_off[i]:out_off[i] + B * ms])
    torch.cuda.synchronize()
    got = out_all.cpu().numpy()
    for i, (B, ms, cu) in enumerate(cases):
        ref = M.padding_mask(cu, B, ms).reshape(-1)
        assert np.array_equal(got[out_off[i]:out_off[i] + B * ms], ref), (B, ms, cu)


@pytest.mark.parametrize("offset", [0, 1, 3])
def test_long_rows_and_unaligned_output(offset):
    import varlen_gqa_attention_amd as V
    lens = I.edge_sweep_lengths(64)
    B, ms = len(lens), 16384
    cu = I.cu_from_lengths(lens, 65, [-1, 2**31 - 1, int(lens.sum())])
    cu_d = torch.from_numpy(cu).cuda()
    buf = torch.zeros(B * ms + 16, dtype=torch.bool, device="cuda")
    out = buf[offset:offset + B * ms]
    V.padding_mask(cu_d, B, ms, out=out)
    torch.cuda.synchronize()
    ref = M.padding_mask(cu, B, ms).reshape(-1)
    assert np.array_equal(out.cpu().numpy(), ref)
    assert not buf[:offset].any() and not buf[offset + B * ms:].any()


def test_invalid_lengths_follow_the_formula():
    import varlen_gqa_attention_amd as V
    cu = np.array([0, 3, 12, 14, 10, -2**31, 2**31 - 1], dtype=np.int32)
    B, ms = 6, 8
    out = V.padding_mask(torch.from_numpy(cu).cuda(), B, ms)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), M.padding_mask(cu, B, ms))
    assert out.shape == (B, 1, 1, ms) and out.dtype == torch.bool


def test_exhaustive_cross_attention_cases():
    """Every combination of query and key lengths for max_seqlen_q, max_seqlen_kv
    in 1..5 and batch 1..3 (the page's 202100 cases). The cases of one
    (max_q, max_kv, B) shape are laid end to end as one batch (a mask row
    depends only on its own sequence's length), one launch per shape."""
    import varlen_gqa_attention_amd as V
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "te24_mask_equivalence.json")))["cross_attention"]
    n_cases = 0
    for mq in range(g["max_seqlen_q"][0], g["max_seqlen_q"][1] + 1):
        for mk in range(g["max_seqlen_kv"][0], g["max_seqlen_kv"][1] + 1):
            for B in range(g["batch_size"][0], g["batch_size"][1] + 1):
                pairs = list(itertools.product(range(mq + 1), range(mk + 1)))
                combos = list(itertools.product(pairs, repeat=B))
                n_cases += len(combos)
                lq = np.array([p[0] for c in combos for p in c], dtype=np.int64)
                lk = np.array([p[1] for c in combos for p in c], dtype=np.int64)
                cu_q = I.cu_from_lengths(lq)
                cu_k = I.cu_from_lengths(lk)
                n = lq.size
                got_q, got_k = V.cross_padding_masks(torch.from_numpy(cu_q).cuda(),
                                                     torch.from_numpy(cu_k).cuda(), n, mq, mk)
                ref_q, ref_k = M.cross_padding_masks(cu_q, cu_k, n, mq, mk)
                assert np.array_equal(got_q.cpu().numpy(), ref_q), (mq, mk, B)
                assert np.array_equal(got_k.cpu().numpy(), ref_k), (mq, mk, B)
    assert n_cases == g["cases"]


def test_cross_masks_with_longer_buffers_and_invalid_lengths():
    import varlen_gqa_attention_amd as V
    cu_q = np.array([0, 3, 1, 9, -7, 100], dtype=np.int32)     # lengths 3, -2, 8; tail ignored
    cu_k = np.array([5, 5, 2**31 - 1, 0, 44, 3], dtype=np.int32)
    got_q, got_k = V.cross_padding_masks(torch.from_numpy(cu_q).cuda(),
                                         torch.from_numpy(cu_k).cuda(), 3, 6, 4)
    ref_q, ref_k = M.cross_padding_masks(cu_q, cu_k, 3, 6, 4)
    assert np.array_equal(got_q.cpu().numpy(), ref_q)
    assert np.array_equal(got_k.cpu().numpy(), ref_k)
