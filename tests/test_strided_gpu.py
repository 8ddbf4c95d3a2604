"""Token-row-strided views (q, k, v as slices of one fused QKV buffer, out as
a slice of a wider buffer): results equal the packed call bit for bit, the
parts of the buffers outside the views are untouched, and invalid strides are
rejected (GPU)."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.parity import assert_lse_close, assert_out_close
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

SENT = 0x4B80


def _fused(T, Hq, Hkv, D, seed):
    qkv = I.normal_bf16((T, Hq + 2 * Hkv, D), seed, "cuda")
    return qkv, qkv[:, :Hq], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:]


def _wide_out(T, Hq, D, extra=3):
    buf = torch.empty(T, Hq + extra, D, dtype=torch.bfloat16, device="cuda")
    buf.view(torch.int16).fill_(SENT)
    return buf, buf[:, 1:Hq + 1]


def _check(plan, q_lens, kv_lens, Hq, Hkv, D, causal, seed, B=None):
    cu_q = I.cu_from_lengths(q_lens)
    cu_k = I.cu_from_lengths(kv_lens)
    Tq, Tk = max(1, int(cu_q[-1])), max(1, int(cu_k[-1]))
    T = max(Tq, Tk)
    print(f"[strided] Hq={Hq} Hkv={Hkv} D={D} causal={causal} lens={list(q_lens)[:6]}",
          flush=True)
    qkv, q, k, v = _fused(T, Hq, Hkv, D, seed)
    q, k, v = q[:Tq], k[:Tk], v[:Tk]
    cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    B = len(q_lens) if B is None else B
    # packed reference call
    out_p, lse_p = plan(q.contiguous(), k.contiguous(), v.contiguous(), cq, ck, B=B)
    # strided call
    buf, out_s = _wide_out(Tq, Hq, D)
    lse_s = torch.empty(Tq, Hq, device="cuda")
    assert not q.is_contiguous() and not out_s.is_contiguous()
    plan(q, k, v, cq, ck, out=out_s, lse=lse_s, B=B)
    torch.cuda.synchronize()
    written = np.zeros(Tq, bool)
    for b in range(B):
        written[cu_q[b]:cu_q[b + 1]] = True
    w = torch.from_numpy(written).cuda()
    assert torch.equal(out_p[w].view(torch.int16), out_s[w].view(torch.int16))
    assert torch.equal(lse_p[w], lse_s[w])
    raw = buf.view(torch.int16)
    assert bool((raw[:, 0] == SENT).all()) and bool((raw[:, Hq + 1:] == SENT).all())
    assert bool((raw[~w] == SENT).all())
    # and against the oracle
    ro, rl, wr = A.attend_varlen(I.bf16_to_f64(q), I.bf16_to_f64(k), I.bf16_to_f64(v), cu_q,
                                 cu_k, B, causal)
    assert_out_close(I.bf16_to_f64(out_s)[wr], ro[wr])
    assert_lse_close(lse_s.cpu().numpy()[wr], rl[wr])


@pytest.mark.parametrize("path,nsplit,fuse", [(2, 4, 0), (2, 1, 0), (1, 3, 0), (1, 1, 0),
                                              (2, 5, 1)])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_on_fused_qkv_slices(path, nsplit, fuse, D):
    import varlen_gqa_attention_amd as V
    Hq, Hkv = 16, 2
    kv_lens = [1, 300, 64, 0, 1000]
    plan = V.Plan(len(kv_lens), 1, 1024, Hq, Hkv, D, False, force_decode_path=path,
                  force_nsplit=nsplit, fuse_combine=fuse)
    _check(plan, [1] * len(kv_lens), kv_lens, Hq, Hkv, D, False, 30 + D)


@pytest.mark.parametrize("grid", [0, 1])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_prefill_on_fused_qkv_slices(grid, D):
    import varlen_gqa_attention_amd as V
    Hq, Hkv = 8, 2
    lens = [70, 1, 129, 300]
    plan = V.Plan(len(lens), 512, 512, Hq, Hkv, D, True, prefill_grid=grid)
    _check(plan, lens, lens, Hq, Hkv, D, True, 40 + D)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_prefill_with_the_widest_kv_rows(D):
    """K and V rows 2^25 - 8 elements apart (64 MiB per token row), the widest
    a prefill plan accepts: the kernel's 32-bit tile offsets reach their
    largest values. Equal to the packed call bit for bit, and the oracle;
    rows 2^25 elements apart or more are rejected before anything is
    enqueued."""
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import _lib
    Hq, Hkv = 4, 1
    lens = [3, 2]
    cu = I.cu_from_lengths(lens)
    T = int(cu[-1])
    stride = (1 << 25) - 8
    print(f"[wide rows] D={D} stride={stride}", flush=True)
    plan = V.Plan(len(lens), 8, 8, Hq, Hkv, D, True)
    q = I.normal_bf16((T, Hq, D), 60 + D, "cuda")
    kp = I.normal_bf16((T, Hkv, D), 61 + D, "cuda")
    vp = I.normal_bf16((T, Hkv, D), 62 + D, "cuda")
    store = torch.zeros(2, (T - 1) * stride + Hkv * D, dtype=torch.bfloat16, device="cuda")
    k = store[0].as_strided((T, Hkv, D), (stride, D, 1))
    v = store[1].as_strided((T, Hkv, D), (stride, D, 1))
    k.copy_(kp)
    v.copy_(vp)
    c = torch.from_numpy(cu).cuda()
    out_p, lse_p = plan(q, kp, vp, c, c, B=len(lens))
    out_w, lse_w = plan(q, k, v, c, c, B=len(lens))
    torch.cuda.synchronize()
    assert torch.equal(out_p.view(torch.int16), out_w.view(torch.int16))
    assert torch.equal(lse_p, lse_w)
    ro, rl, wr = A.attend_varlen(I.bf16_to_f64(q), I.bf16_to_f64(kp), I.bf16_to_f64(vp), cu, cu,
                                 len(lens), True)
    assert_out_close(I.bf16_to_f64(out_w)[wr], ro[wr])
    assert_lse_close(lse_w.cpu().numpy()[wr], rl[wr])
    # one row 2^25 elements apart: rejected, out untouched
    L = _lib.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    out_r = torch.full_like(out_p, 7.0)
    for ks, vs in ((1 << 25, 0), (0, 1 << 25), ((1 << 25) + 8, (1 << 25) + 8)):
        st = L.vattn_execute_strided(plan._h, len(lens), P(q), 0, P(store[0]), ks, P(store[1]),
                                     vs, P(c), P(c), P(out_r), 0, P(lse_w), T, 2, None)
        assert st == -1, (ks, vs, st)
    torch.cuda.synchronize()
    assert bool((out_r == 7.0).all())
    del store


def test_invalid_strides_are_rejected():
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import _lib
    L = _lib.load()
    Hq, Hkv, D = 8, 2, 64
    plan = V.Plan(2, 1, 64, Hq, Hkv, D, False)
    q = torch.zeros(2, Hq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(64, Hkv, D, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    lse = torch.zeros(2, Hq, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    call = lambda qs, ks, vs, os_: L.vattn_execute_strided(
        plan._h, 2, P(q), qs, P(k), ks, P(k), vs, P(cu), P(cu), P(out), os_, P(lse), 2, 64, None)
    assert call(Hq * D - 8, 0, 0, 0) == -1            # rows would overlap
    assert call(0, Hkv * D + 4, 0, 0) == -1           # not 16-byte aligned
    assert call(0, 0, 0, Hq * D - 64) == -1
    assert call(0, 0, 0, 0) == 0                      # 0 = packed
    torch.cuda.synchronize()


def test_prefill_full_size_on_fused_qkv_equals_packed_bitwise():
    """The benchmark's causal varlen prefill at full size with q, k, v as
    slices of one fused QKV buffer and out inside a wider buffer: bit-equal
    to the packed call."""
    import varlen_gqa_attention_amd as V
    w = I.varlen_prefill(0)
    m = I.materialise(w, 0, "cuda")
    Hq, Hkv, D = w["Hq"], w["Hkv"], w["D"]
    plan = V.Plan(w["B_max"], w["s_max_q"], w["s_max_kv"], Hq, Hkv, D, True)
    out_p, lse_p = plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], B=w["B"])
    T = m["q"].shape[0]
    qkv = torch.empty(T, Hq + 2 * Hkv, D, dtype=torch.bfloat16, device="cuda")
    qkv[:, :Hq] = m["q"]
    qkv[:, Hq:Hq + Hkv] = m["k"]
    qkv[:, Hq + Hkv:] = m["v"]
    buf, out_s = _wide_out(T, Hq, D)
    lse_s = torch.empty(T, Hq, device="cuda")
    plan(qkv[:, :Hq], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:], m["cu_q"], m["cu_kv"], out=out_s,
         lse=lse_s, B=w["B"])
    torch.cuda.synchronize()
    assert torch.equal(out_p.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(lse_p, lse_s)
    raw = buf.view(torch.int16)
    assert bool((raw[:, 0] == SENT).all()) and bool((raw[:, Hq + 1:] == SENT).all())
