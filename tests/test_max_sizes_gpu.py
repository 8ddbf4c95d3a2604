"""Parity at the largest sizes the plans accept (GPU): the largest query-head
groups folded into one workgroup, the longest sequences, the largest batches.
Results are checked against the fp64 oracle, in full where it finishes in
seconds and on sampled rows otherwise."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.parity import assert_lse_close, assert_out_close
from tests.test_decode_gpu import _w, run_decode
from tests.test_prefill_gpu import _prefill_workload, run_prefill
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,G", [(128, 256), (64, 256), (256, 128)])
def test_prefill_largest_query_groups(D, G):
    """G = 256 query heads on one KV head at D <= 128 (one query token per
    256-row workgroup) and G = 128 at D = 256: the largest groups a prefill
    plan accepts."""
    lens = [1, 3, 70, 129]
    run_prefill(_prefill_workload(f"max G={G} D={D}", G, 1, D, lens, lens, True), 11)


def test_prefill_group_beyond_the_limit_is_refused():
    import varlen_gqa_attention_amd as V
    with pytest.raises(V.VattnError) as e:
        V.Plan(2, 64, 64, 512, 1, 128, True)
    assert e.value.status == V._lib.VATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("path", [1, 2])
def test_decode_largest_query_groups(path):
    """G = 128 and 256 query heads per KV head: several head blocks per unit
    on both decode paths."""
    for G in (128, 256):
        w = _w(f"decode max G={G}", 3, G, 1, 128, [1, 700, 2049], s_max_kv=4096)
        r = run_decode(w, 12, force_decode_path=path)
        assert r["info"]["head_blocks"] > 1


def test_decode_longest_sequence():
    """One sequence of 131072 keys (2048 tiles; 32 splits of 4096 keys), Hq=64,
    Hkv=8, D=128, in full against the oracle."""
    w = _w("decode 128k keys", 1, 64, 8, 128, [131072])
    r = run_decode(w, 13)
    assert r["info"]["nsplit"] == 32 and r["info"]["chunk_keys"] == 4096


def test_decode_largest_batch_in_one_plan():
    """B_max = B = 4096 sequences of 1..300 keys (seeded), Hq=32, Hkv=8:
    32768 units in one grid."""
    lens = np.random.default_rng(14).integers(1, 301, size=4096)
    w = _w("decode B=4096", 4096, 32, 8, 128, lens, s_max_kv=300)
    r = run_decode(w, 14)
    assert r["info"]["n_units"] == 4096 * 8


def test_prefill_long_sequence_sampled():
    """One causal sequence of 32768 tokens (512 query tiles), Hq=32, Hkv=8,
    D=128, with a short one beside it; sampled rows (first, tile edges,
    middle, last) against the oracle."""
    lens = [32768, 100]
    w = _prefill_workload("prefill 32k tokens", 32, 8, 128, lens, lens, True)
    picks = [(0, i, h) for i in (0, 1, 63, 64, 16383, 16384, 32766, 32767) for h in (0, 9, 31)]
    picks += [(1, i, h) for i in (0, 99) for h in (0, 31)]
    run_prefill(w, 15, picks=picks)
