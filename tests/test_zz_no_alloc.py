"""vattn_execute_noalloc (plan and scratch without any allocation) against
vattn_execute on a plan of the same shape (GPU).

Two calls in a row through the C ABI, the second on a smaller input, each
compared bit for bit with vattn_execute and within tolerance with the fp64
oracle; the static scratch keeps the first call's contents when the second
runs. Also: a plan whose scratch exceeds the static array is refused before
anything is enqueued, and the caller's error word receives clamp flags.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.parity import assert_lse_close, assert_out_close
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu


def _noalloc(shape, m, B, out, lse, err=None):
    """Call vattn_execute_noalloc through the C entry point."""
    from varlen_gqa_attention_amd import _lib
    L = _lib.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return L.vattn_execute_noalloc(*shape, B, P(m["q"]), P(m["k"]), P(m["v"]), P(m["cu_q"]),
                                   P(m["cu_kv"]), P(out), P(lse), m["q"].shape[0],
                                   m["k"].shape[0], P(err), st)


def _case(w, seed):
    import varlen_gqa_attention_amd as V
    shape = (w["B_max"], w["s_max_q"], w["s_max_kv"], w["Hq"], w["Hkv"], w["D"], int(w["causal"]))
    print(f"[noalloc] {w['name']} shape={shape} B={w['B']}", flush=True)
    m = I.materialise(w, seed, "cuda")
    plan = V.Plan(*shape)
    ref_out, ref_lse = plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], B=w["B"])
    out = torch.full_like(m["q"], 7.0)
    lse = torch.full(m["q"].shape[:2], 7.0, device="cuda")
    assert _noalloc(shape, m, w["B"], out, lse) == 0
    torch.cuda.synchronize()
    return plan, m, ref_out, ref_lse, out, lse


def _check(w, m, ref_out, ref_lse, out, lse):
    # same plan, same kernels: identical bits to vattn_execute
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), w["name"]
    assert torch.equal(lse, ref_lse), w["name"]
    q, k, v = (I.bf16_to_f64(m[n]) for n in ("q", "k", "v"))
    ro, rl, wr = A.attend_varlen(q, k, v, m["cu_q_np"], m["cu_kv_np"], w["B"], w["causal"])
    assert_out_close(I.bf16_to_f64(out)[wr], ro[wr], w["name"])
    assert_lse_close(lse.cpu().numpy().astype(np.float64)[wr], rl[wr], w["name"])


def _split_decode(name, B, Hq, Hkv, D, lens):
    lens = np.asarray(lens, dtype=np.int64)
    return dict(name=name, B=B, B_max=B, Hq=Hq, Hkv=Hkv, D=D, causal=False,
                q_lens=np.ones(B, np.int64), kv_lens=lens, s_max_q=1, s_max_kv=int(lens.max()))


def test_noalloc_matches_execute_two_calls_second_smaller():
    big = I.long_decode()                                   # 32 splits, 1.1 MB of partials
    small = _split_decode("split decode, 3 sequences", 3, 16, 2, 128, [1, 1000, 4097])
    plan_b, mb, rob, rlb, ob, lb = _case(big, 0)
    assert plan_b.info["nsplit"] == 32 and not plan_b.info["direct"]
    plan_s, ms, ros, rls, os_, ls = _case(small, 1)
    assert plan_s.info["nsplit"] > 1 and not plan_s.info["direct"]
    _check(big, mb, rob, rlb, ob, lb)
    _check(small, ms, ros, rls, os_, ls)


def test_noalloc_prefill_and_direct_decode():
    lens = np.array([1, 40, 129, 300])
    wp = dict(name="causal prefill", B=4, B_max=4, Hq=8, Hkv=2, D=64, causal=True,
              q_lens=lens, kv_lens=lens, s_max_q=300, s_max_kv=300)
    _, m, ro, rl, o, l = _case(wp, 2)
    _check(wp, m, ro, rl, o, l)
    wd = I.tiny_decode(0)                                   # one split: direct write
    plan, m, ro, rl, o, l = _case(wd, 3)
    assert plan.info["direct"]
    _check(wd, m, ro, rl, o, l)


def test_noalloc_refuses_plans_beyond_the_static_scratch():
    from varlen_gqa_attention_amd import _lib
    w = I.edge_sweep(128)     # B_max 64 x Hq 128 x 8 splits of fp32 partials: ~35 MB
    import varlen_gqa_attention_amd as V
    info = V.describe_plan(64, 1, 16384, 128, 8, 128, 0)
    assert info["scratch_bytes"] > 8 << 20
    m = I.materialise(w, 4, "cuda")
    out = torch.full_like(m["q"], 7.0)
    lse = torch.full(m["q"].shape[:2], 7.0, device="cuda")
    shape = (64, 1, 16384, 128, 8, 128, 0)
    assert _noalloc(shape, m, w["B"], out, lse) == _lib.VATTN_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())   # nothing enqueued


def test_noalloc_error_word_receives_clamp_flags():
    from varlen_gqa_attention_amd import ERRBIT_KV_LEN
    w = _split_decode("clamped", 2, 8, 1, 64, [100, 900])
    m = I.materialise(w, 5, "cuda")
    shape = (2, 1, 512, 8, 1, 64, 0)    # s_max_kv 512 < 900: the second length is clamped
    out = torch.empty_like(m["q"])
    lse = torch.empty(m["q"].shape[:2], device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert _noalloc(shape, m, 2, out, lse, err) == 0
    torch.cuda.synchronize()
    assert int(err.item()) == ERRBIT_KV_LEN
    q, k, v = (I.bf16_to_f64(m[n]) for n in ("q", "k", "v"))
    ro, rl, wr = A.attend_varlen(q, k, v, m["cu_q_np"], m["cu_kv_np"], 2, False, s_max_kv=512)
    assert_out_close(I.bf16_to_f64(out)[wr], ro[wr], "clamped")
