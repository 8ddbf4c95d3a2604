"""Decode over gathered keys (an index list per sequence) vs the oracle (GPU)."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.parity import assert_lse_close, assert_out_close
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu


def _case(sizes, n_rows, seed, Hq, Hkv, D):
    rng = np.random.default_rng([6, seed])
    B = len(sizes)
    cu_idx = I.cu_from_lengths(sizes)
    idx = rng.integers(0, n_rows, size=max(1, int(cu_idx[-1]))).astype(np.int32)
    if idx.size > 3:
        idx[2] = idx[1]                      # a duplicate
    q = I.normal_bf16((B, Hq, D), 100 + seed, "cuda")
    k = I.normal_bf16((n_rows, Hkv, D), 200 + seed, "cuda")
    v = I.normal_bf16((n_rows, Hkv, D), 300 + seed, "cuda")
    cu_q = I.cu_from_lengths(np.ones(B, np.int64))
    return q, k, v, cu_q, cu_idx, idx


def _run(plan, q, k, v, cu_q, cu_idx, idx, B):
    out, lse = plan.gathered(q, k, v, torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_idx).cuda(),
                             torch.from_numpy(idx).cuda(), B=B)
    torch.cuda.synchronize()
    return out, lse


def _oracle(q, k, v, cu_q, cu_idx, idx, B, s_max):
    return A.attend_gathered(I.bf16_to_f64(q), I.bf16_to_f64(k), I.bf16_to_f64(v), cu_q, cu_idx,
                             idx, B, s_max_kv=s_max)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (8, 2)])      # MFMA path (G=8), wave path (G=4)
@pytest.mark.parametrize("nsplit", [0, 1, 3, 8])
@pytest.mark.parametrize("D", [64, 128])
def test_gathered_topk_lists(Hq, Hkv, nsplit, D):
    import varlen_gqa_attention_amd as V
    sizes = [1, 37, 600, 0, 256]
    print(f"[gathered] Hq={Hq} Hkv={Hkv} D={D} nsplit={nsplit} sizes={sizes}", flush=True)
    q, k, v, cu_q, cu_idx, idx = _case(sizes, 5000, D + nsplit, Hq, Hkv, D)
    plan = V.Plan(len(sizes), 1, 640, Hq, Hkv, D, False, force_nsplit=nsplit)
    out, lse = _run(plan, q, k, v, cu_q, cu_idx, idx, len(sizes))
    assert plan.read_error() == 0
    ro, rl, wr, clamped = _oracle(q, k, v, cu_q, cu_idx, idx, len(sizes), 640)
    assert not clamped
    assert_out_close(I.bf16_to_f64(out)[wr], ro[wr])
    assert_lse_close(lse.cpu().numpy()[wr], rl[wr])


@pytest.mark.parametrize("D", [32, 256])
def test_gathered_other_head_dims(D):
    import varlen_gqa_attention_amd as V
    sizes = [300, 5, 129]
    q, k, v, cu_q, cu_idx, idx = _case(sizes, 2000, D, 32, 2, D)
    plan = V.Plan(4, 1, 512, 32, 2, D, False)
    out, lse = _run(plan, q, k, v, cu_q, cu_idx, idx, 3)
    ro, rl, wr, _ = _oracle(q, k, v, cu_q, cu_idx, idx, 3, 512)
    assert_out_close(I.bf16_to_f64(out)[wr], ro[wr])
    assert_lse_close(lse.cpu().numpy()[wr], rl[wr])


@pytest.mark.parametrize("path", [1, 2])
def test_identity_gather_equals_contiguous_execute_bitwise(path):
    import varlen_gqa_attention_amd as V
    lens = [100, 1, 700]
    cu = I.cu_from_lengths(lens)
    T = int(cu[-1])
    q = I.normal_bf16((3, 16, 128), 7, "cuda")
    k = I.normal_bf16((T, 2, 128), 8, "cuda")
    v = I.normal_bf16((T, 2, 128), 9, "cuda")
    plan = V.Plan(3, 1, 1024, 16, 2, 128, False, force_decode_path=path, force_nsplit=4)
    cu_q = torch.from_numpy(I.cu_from_lengths([1, 1, 1])).cuda()
    cu_d = torch.from_numpy(cu).cuda()
    o1, l1 = plan(q, k, v, cu_q, cu_d)
    o2, l2 = plan.gathered(q, k, v, cu_q, cu_d, torch.arange(T, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_out_of_range_rows_are_clamped_and_flagged():
    import varlen_gqa_attention_amd as V
    q, k, v, cu_q, cu_idx, idx = _case([4, 60], 100, 3, 16, 2, 64)
    idx[0], idx[5] = -3, 100                 # below and at the row count
    plan = V.Plan(2, 1, 64, 16, 2, 64, False, force_nsplit=2)
    out, lse = _run(plan, q, k, v, cu_q, cu_idx, idx, 2)
    assert plan.read_error() == V.ERRBIT_INDEX
    ro, rl, wr, clamped = _oracle(q, k, v, cu_q, cu_idx, idx, 2, 64)
    assert clamped
    assert_out_close(I.bf16_to_f64(out)[wr], ro[wr])
    assert_lse_close(lse.cpu().numpy()[wr], rl[wr])


def test_fused_plan_merges_gathered_keys_in_the_combine_kernel():
    import varlen_gqa_attention_amd as V
    sizes = [500, 33]
    q, k, v, cu_q, cu_idx, idx = _case(sizes, 3000, 4, 16, 2, 128)
    plan = V.Plan(2, 1, 512, 16, 2, 128, False, force_nsplit=4, fuse_combine=1)
    for _ in range(2):
        out, lse = _run(plan, q, k, v, cu_q, cu_idx, idx, 2)
    ro, rl, wr, _ = _oracle(q, k, v, cu_q, cu_idx, idx, 2, 512)
    assert_out_close(I.bf16_to_f64(out)[wr], ro[wr])
    assert_lse_close(lse.cpu().numpy()[wr], rl[wr])


def test_gathered_needs_a_decode_plan():
    import varlen_gqa_attention_amd as V
    plan = V.Plan(2, 64, 64, 8, 2, 64, True)
    q = torch.zeros(2, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(10, 2, 64, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    with pytest.raises(V.VattnError) as e:
        plan.gathered(q, k, k, cu, cu, torch.zeros(2, dtype=torch.int32, device="cuda"))
    assert e.value.status == -2


def test_gathered_full_size_bench_configuration():
    """The benchmark's gathered workload at full size (16 sequences, each
    attending 2048 sorted rows of its own 32768-token history, Hq=32, Hkv=8,
    D=128, default plan): every output against the oracle, which receives
    the selected rows (gathered with torch indexing) and an identity list."""
    import varlen_gqa_attention_amd as V
    B, Hq, Hkv, D, hist, sel = 16, 32, 8, 128, 32768, 2048
    plan = V.Plan(B, 1, sel, Hq, Hkv, D, False)
    q = I.normal_bf16((B, Hq, D), 40, "cuda")
    k = I.normal_bf16((B * hist, Hkv, D), 41, "cuda")
    v = I.normal_bf16((B * hist, Hkv, D), 42, "cuda")
    rng = I.rng(7, 0)
    idx = np.concatenate([b * hist + np.sort(rng.choice(hist, sel, replace=False))
                          for b in range(B)]).astype(np.int32)
    cu_q = I.cu_from_lengths(np.ones(B, np.int64))
    cu_idx = I.cu_from_lengths(np.full(B, sel))
    print(f"[gathered full size] plan {plan.info['nsplit']} splits", flush=True)
    out, lse = _run(plan, q, k, v, cu_q, cu_idx, idx, B)
    assert plan.read_error() == 0
    rows = torch.from_numpy(idx).cuda().long()
    ks, vs = k[rows], v[rows]
    ro, rl, wr, clamped = A.attend_gathered(
        I.bf16_to_f64(q), I.bf16_to_f64(ks), I.bf16_to_f64(vs), cu_q, cu_idx,
        np.arange(B * sel, dtype=np.int64), B, s_max_kv=sel)
    assert not clamped and wr.all()
    assert_out_close(I.bf16_to_f64(out), ro)
    assert_lse_close(lse.cpu().numpy(), rl)
