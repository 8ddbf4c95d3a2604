"""Argument errors (status codes, nothing enqueued) and device-data errors
(clamped lengths flagged in the plan's error word)."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.parity import assert_lse_close, assert_out_close
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_plan_argument_errors():
    import varlen_gqa_attention_amd as V
    with pytest.raises(V.VattnError) as e:
        V.Plan(4, 1, 64, 6, 4, 64, False)          # Hq % Hkv != 0
    assert e.value.status == -1
    with pytest.raises(V.VattnError) as e:
        V.Plan(4, 1, 64, 8, 2, 96, False)          # unsupported D
    assert e.value.status == -2
    with pytest.raises(V.VattnError):
        V.Plan(0, 1, 64, 8, 2, 64, False)


def test_execute_argument_errors():
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import _lib
    L = _lib.load()
    plan = V.Plan(2, 1, 64, 8, 2, 64, False)
    q = torch.zeros(2, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(64, 2, 64, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    lse = torch.zeros(2, 8, device="cuda")
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    args = lambda B, qp: (plan._h, B, qp, P(k), P(k), P(cu), P(cu), P(out), P(lse), 2, 64, None)
    assert L.vattn_execute(*args(3, P(q))) == -1           # B > B_max
    assert L.vattn_execute(*args(-1, P(q))) == -1
    assert L.vattn_execute(*args(1, P(q, 2))) == -1        # misaligned q
    assert L.vattn_execute(*args(1, None)) == -1           # null q
    assert L.vattn_execute(*args(0, None)) == 0            # B = 0: no-op
    torch.cuda.synchronize()


def test_out_of_range_lengths_are_clamped_and_flagged():
    import varlen_gqa_attention_amd as V
    Hq, Hkv, D, smax = 8, 2, 64, 100
    k = I.normal_bf16((400, Hkv, D), 1, "cuda")
    v = I.normal_bf16((400, Hkv, D), 2, "cuda")
    q = I.normal_bf16((3, Hq, D), 3, "cuda")
    cu_q = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device="cuda")
    cu_kv_np = np.array([0, 250, 240, 300], dtype=np.int32)   # 250 > s_max, -10 < 0, 60 ok
    plan = V.Plan(3, 1, smax, Hq, Hkv, D, False)
    out, lse = plan(q, k, v, cu_q, torch.from_numpy(cu_kv_np).cuda(), B=3)
    torch.cuda.synchronize()
    assert plan.read_error() == V.ERRBIT_KV_LEN
    ref_o, ref_l, _ = A.attend_varlen(I.bf16_to_f64(q), I.bf16_to_f64(k), I.bf16_to_f64(v),
                                      [0, 1, 2, 3], cu_kv_np, 3, False, s_max_kv=smax)
    assert_out_close(I.bf16_to_f64(out), ref_o)
    assert_lse_close(lse.cpu().numpy(), ref_l)
    plan.clear_error()
    torch.cuda.synchronize()
    assert plan.read_error() == 0


def test_rows_past_capacity_are_cut_and_flagged():
    import varlen_gqa_attention_amd as V
    Hq, Hkv, D = 8, 2, 64
    k = I.normal_bf16((50, Hkv, D), 4, "cuda")
    q = I.normal_bf16((2, Hq, D), 5, "cuda")
    cu_q = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    cu_kv = torch.tensor([0, 30, 80], dtype=torch.int32, device="cuda")  # second runs past 50 rows
    plan = V.Plan(2, 1, 64, Hq, Hkv, D, False)
    out, lse = plan(q, k, k, cu_q, cu_kv, B=2)
    torch.cuda.synchronize()
    assert plan.read_error() & V.ERRBIT_ROWS
    ref_o, ref_l, _ = A.attend_varlen(I.bf16_to_f64(q), I.bf16_to_f64(k), I.bf16_to_f64(k),
                                      [0, 1, 2], [0, 30, 50], 2, False)
    assert_out_close(I.bf16_to_f64(out), ref_o)


def test_kernel_event_hook():
    """The measurement hook records its events around the main kernel only,
    leaves results unchanged, and rejects a half-set pair."""
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import _lib
    L = _lib.load()
    B, Hq, Hkv, D, Lk = 1, 16, 2, 64, 4096
    plan = V.Plan(B, 1, Lk, Hq, Hkv, D, False, force_nsplit=8)
    q = I.normal_bf16((B, Hq, D), 41, "cuda")
    k = I.normal_bf16((Lk, Hkv, D), 42, "cuda")
    v = I.normal_bf16((Lk, Hkv, D), 43, "cuda")
    cu_q = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    cu_kv = torch.tensor([0, Lk], dtype=torch.int32, device="cuda")
    out0, lse0 = plan(q, k, v, cu_q, cu_kv)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with pytest.raises(ValueError):
        plan.set_kernel_events(a, b)                       # not yet created
    a.record()
    b.record()
    torch.cuda.synchronize()
    assert L.vattn_plan_set_kernel_events(plan._h, ctypes.c_void_p(a.cuda_event), None) == -1
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    plan.set_kernel_events(a, b)
    t0.record()
    out1, lse1 = plan(q, k, v, cu_q, cu_kv)
    t1.record()
    plan.set_kernel_events(None, None)
    torch.cuda.synchronize()
    kern, whole = a.elapsed_time(b), t0.elapsed_time(t1)
    assert 0.0 < kern <= whole
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


@pytest.mark.parametrize("grid", [0, 1])
def test_prefill_flags_a_sequence_with_no_live_tile(grid):
    """A negative query length is clamped to 0 (no tile is ever scheduled for
    that sequence) and still sets the error word; the other sequences are
    computed as usual."""
    import varlen_gqa_attention_amd as V
    Hq, Hkv, D = 8, 2, 64
    q = I.normal_bf16((60, Hq, D), 6, "cuda")
    k = I.normal_bf16((60, Hkv, D), 7, "cuda")
    v = I.normal_bf16((60, Hkv, D), 8, "cuda")
    cu_q_np = np.array([0, 20, 50, 40], dtype=np.int32)        # sequence 2: query length -10
    cu_kv_np = np.array([0, 20, 50, 60], dtype=np.int32)
    plan = V.Plan(3, 64, 64, Hq, Hkv, D, True, prefill_grid=grid)
    out = torch.zeros_like(q)
    lse = torch.zeros(60, Hq, device="cuda")
    plan(q, k, v, torch.from_numpy(cu_q_np).cuda(), torch.from_numpy(cu_kv_np).cuda(), out=out,
         lse=lse, B=3)
    torch.cuda.synchronize()
    assert plan.read_error() == V.ERRBIT_Q_LEN
    ref_o, ref_l, wr = A.attend_varlen(I.bf16_to_f64(q), I.bf16_to_f64(k), I.bf16_to_f64(v),
                                       cu_q_np, cu_kv_np, 3, True, s_max_q=64, s_max_kv=64)
    assert wr.sum() == 50
    assert_out_close(I.bf16_to_f64(out)[wr], ref_o[wr])
    assert_lse_close(lse.cpu().numpy()[wr], ref_l[wr])
