"""Backward (dq, dk, dv) through the C ABI vs the fp64 oracle (GPU).

The forward runs on the GPU (its out and lse feed the backward, as in
training); the oracle differentiates the exact attention of the same bf16
inputs. Covers ragged packs with empty sequences, Lq != Lk both ways, a
sequence without keys, several tiles per sequence, trailing cu entries past
B, row-strided views, determinism and the error statuses.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import backward as BW
from tests.parity import assert_grad_close
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

SENT = 0x4B80


def _setup(q_lens, kv_lens, Hq, Hkv, D, seed, lead=3, tail=(-1, 2**31 - 1)):
    B = len(q_lens)
    cu_q = I.cu_from_lengths(q_lens, capacity=B + 1 + len(tail), tail=tail, start=lead)
    cu_k = I.cu_from_lengths(kv_lens, capacity=B + 1 + len(tail), tail=tail, start=lead + 1)
    Tq = lead + int(np.sum(q_lens)) + 2
    Tk = lead + 1 + int(np.sum(kv_lens)) + 2
    q = I.normal_bf16((Tq, Hq, D), 10 + seed, "cuda")
    k = I.normal_bf16((Tk, Hkv, D), 20 + seed, "cuda")
    v = I.normal_bf16((Tk, Hkv, D), 30 + seed, "cuda")
    dout = I.normal_bf16((Tq, Hq, D), 40 + seed, "cuda")
    return B, cu_q, cu_k, q, k, v, dout


def _run(plan, B, cu_q, cu_k, q, k, v, dout):
    cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    out, lse = plan(q, k, v, cq, ck, B=B)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    for t in (dq, dk, dv):
        t.view(torch.int16).fill_(SENT)
    plan.backward(q, k, v, out, lse, dout, cq, ck, dq=dq, dk=dk, dv=dv, B=B)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def _check(B, cu_q, cu_k, q, k, v, dout, dq, dk, dv, causal, what):
    rq, rk, rv, wq, wk = BW.attend_varlen_backward(
        I.bf16_to_f64(q), I.bf16_to_f64(k), I.bf16_to_f64(v), I.bf16_to_f64(dout), cu_q, cu_k,
        B, causal)
    G = q.shape[1] // k.shape[1]
    assert_grad_close(I.bf16_to_f64(dq)[wq], rq[wq], what + " dq")
    assert_grad_close(I.bf16_to_f64(dk)[wk], rk[wk], what + " dk", heads=G)
    assert_grad_close(I.bf16_to_f64(dv)[wk], rv[wk], what + " dv", heads=G)
    # rows that belong to no sequence are not written
    for t, w in ((dq, wq), (dk, wk), (dv, wk)):
        raw = t.view(torch.int16).cpu().numpy()
        assert (raw[~w] == SENT).all()


# lengths: an empty query side, Lq < Lk, Lq > Lk, a sequence without keys,
# single tokens and tile boundaries +- 1
Q_LENS = [70, 1, 0, 129, 200, 33, 4, 64]
K_LENS = [70, 1, 5, 129, 250, 20, 0, 65]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_backward_matches_oracle(D, G, causal):
    import varlen_gqa_attention_amd as V
    Hkv = 2
    Hq = Hkv * G
    print(f"[backward] D={D} G={G} causal={causal}", flush=True)
    B, cu_q, cu_k, q, k, v, dout = _setup(Q_LENS, K_LENS, Hq, Hkv, D, D + G)
    plan = V.Plan(B + 2, 256, 256, Hq, Hkv, D, causal, backward=True)
    _, _, dq, dk, dv = _run(plan, B, cu_q, cu_k, q, k, v, dout)
    assert plan.read_error() == 0
    _check(B, cu_q, cu_k, q, k, v, dout, dq, dk, dv, causal, f"D={D} G={G}")


@pytest.mark.parametrize("G,D", [(8, 128), (2, 64), (16, 128), (4, 256)])
def test_backward_several_tiles_per_sequence(G, D):
    """Sequences spanning several query tiles, key tiles and 64-row steps."""
    import varlen_gqa_attention_amd as V
    Hkv = 1 if G == 16 else 2
    Hq = Hkv * G
    q_lens, kv_lens = [700, 300, 1025], [700, 513, 1025]
    print(f"[backward] long G={G} D={D}", flush=True)
    B, cu_q, cu_k, q, k, v, dout = _setup(q_lens, kv_lens, Hq, Hkv, D, 7 + G)
    plan = V.Plan(B, 1100, 1100, Hq, Hkv, D, True, backward=True)
    _, _, dq, dk, dv = _run(plan, B, cu_q, cu_k, q, k, v, dout)
    _check(B, cu_q, cu_k, q, k, v, dout, dq, dk, dv, True, f"long G={G} D={D}")


def test_backward_is_deterministic():
    import varlen_gqa_attention_amd as V
    B, cu_q, cu_k, q, k, v, dout = _setup([300, 77], [300, 90], 16, 2, 128, 3)
    plan = V.Plan(B, 300, 300, 16, 2, 128, True, backward=True)
    r1 = _run(plan, B, cu_q, cu_k, q, k, v, dout)
    r2 = _run(plan, B, cu_q, cu_k, q, k, v, dout)
    for a, b in zip(r1[2:], r2[2:]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_backward_on_fused_buffers_equals_packed_bitwise():
    """q/k/v as slices of one fused QKV buffer and dq/dk/dv as slices of one
    fused gradient buffer: bit-identical to packed copies, other bytes of the
    fused gradient buffer untouched."""
    import varlen_gqa_attention_amd as V
    Hq, Hkv, D = 8, 2, 64
    lens = [90, 1, 200]
    cu = I.cu_from_lengths(lens)
    T = int(cu[-1])
    qkv = I.normal_bf16((T, Hq + 2 * Hkv, D), 5, "cuda")
    q, k, v = qkv[:, :Hq], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:]
    dout = I.normal_bf16((T, Hq, D), 6, "cuda")
    cq = torch.from_numpy(cu).cuda()
    plan = V.Plan(3, 256, 256, Hq, Hkv, D, True, backward=True)
    out, lse = plan(q.contiguous(), k.contiguous(), v.contiguous(), cq, cq)
    dq0, dk0, dv0 = plan.backward(q.contiguous(), k.contiguous(), v.contiguous(), out, lse, dout,
                                  cq, cq)
    g = torch.empty(T, Hq + 2 * Hkv + 1, D, dtype=torch.bfloat16, device="cuda")
    g.view(torch.int16).fill_(SENT)
    dq, dk, dv = g[:, :Hq], g[:, Hq:Hq + Hkv], g[:, Hq + Hkv:Hq + 2 * Hkv]
    plan.backward(q, k, v, out, lse, dout, cq, cq, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for a, b in ((dq, dq0), (dk, dk0), (dv, dv0)):
        assert torch.equal(a.contiguous().view(torch.int16), b.view(torch.int16))
    assert bool((g[:, Hq + 2 * Hkv:].view(torch.int16) == SENT).all())


@pytest.mark.parametrize("D", [64, 128])
def test_backward_with_the_widest_rows(D):
    """Every tensor of the backward 2^24 - 8 elements per token row (32 MiB),
    the widest the backward accepts: the kernels' 32-bit in-tile and in-step
    byte offsets reach their largest values. Equal to the packed call bit for
    bit, and the oracle."""
    import varlen_gqa_attention_amd as V
    Hq, Hkv = 4, 2
    lens = [3, 2]
    cu = I.cu_from_lengths(lens)
    T = int(cu[-1])
    rs = (1 << 24) - 8
    print(f"[wide rows] backward D={D} stride={rs}", flush=True)
    plan = V.Plan(len(lens), 8, 8, Hq, Hkv, D, True, backward=True)
    q = I.normal_bf16((T, Hq, D), 70 + D, "cuda")
    k = I.normal_bf16((T, Hkv, D), 71 + D, "cuda")
    v = I.normal_bf16((T, Hkv, D), 72 + D, "cuda")
    dout = I.normal_bf16((T, Hq, D), 73 + D, "cuda")
    c = torch.from_numpy(cu).cuda()
    out, lse = plan(q, k, v, c, c, B=len(lens))
    dq0, dk0, dv0 = plan.backward(q, k, v, out, lse, dout, c, c, B=len(lens))

    def wide(t):
        store = torch.zeros((T - 1) * rs + t.shape[1] * D, dtype=torch.bfloat16, device="cuda")
        w = store.as_strided(tuple(t.shape), (rs, D, 1))
        w.copy_(t)
        return w
    qw, kw, vw, ow, dow = wide(q), wide(k), wide(v), wide(out), wide(dout)
    dqw, dkw, dvw = wide(torch.zeros_like(q)), wide(torch.zeros_like(k)), wide(torch.zeros_like(v))
    plan.backward(qw, kw, vw, ow, lse, dow, c, c, dq=dqw, dk=dkw, dv=dvw, B=len(lens))
    torch.cuda.synchronize()
    for a, b in ((dqw, dq0), (dkw, dk0), (dvw, dv0)):
        assert torch.equal(a.contiguous().view(torch.int16), b.view(torch.int16))
    _check(len(lens), cu, cu, q, k, v, dout, dq0, dk0, dv0, True, "wide rows")


def test_backward_needs_a_backward_plan_and_valid_strides():
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import _lib
    L = _lib.load()
    Hq, Hkv, D = 4, 2, 64
    q = torch.zeros(8, Hq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(8, Hkv, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(8, Hq, device="cuda")
    cu = torch.tensor([0, 8], dtype=torch.int32, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    plain = V.Plan(1, 8, 8, Hq, Hkv, D, True)
    with pytest.raises(V.VattnError) as e:
        plain.backward(q, k, k, q, lse, q, cu, cu)
    assert e.value.status == -2
    plan = V.Plan(1, 8, 8, Hq, Hkv, D, True, backward=True)

    def call(q_rs, dk_rs):
        return L.vattn_backward(plan._h, 1, P(q), q_rs, P(k), 0, P(k), 0, P(q), 0, P(q), 0,
                                P(lse), P(cu), P(cu), P(q), 0, P(k), dk_rs, P(k), 0, 8, 8, None)
    assert call(Hq * D - 8, 0) == -1         # rows would overlap
    assert call(0, Hkv * D + 4) == -1        # not 16-byte aligned
    assert call(1 << 24, 0) == -1            # beyond the 24-bit row offsets
    assert call(0, 0) == 0
    torch.cuda.synchronize()


def test_backward_full_size_varlen_prefill_sampled():
    """The benchmark's backward workload at full size (B=16, L~U[64,4096],
    Hq=32, Hkv=8, D=128, plan s_max 4096, the same launch configuration):
    for the longest and the shortest sequence and one KV head, every dq row
    of the G query heads and every dk / dv row against the oracle's per-head
    gradients, summed over the group."""
    import varlen_gqa_attention_amd as V
    w = I.varlen_prefill(0)
    m = I.materialise(w, 0, "cuda")
    plan = V.Plan(w["B_max"], w["s_max_q"], w["s_max_kv"], w["Hq"], w["Hkv"], w["D"], True,
                  backward=True)
    out, lse = plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], B=w["B"])
    dout = I.normal_bf16(tuple(m["q"].shape), 77, "cuda")
    dq, dk, dv = plan.backward(m["q"], m["k"], m["v"], out, lse, dout, m["cu_q"], m["cu_kv"],
                               B=w["B"])
    torch.cuda.synchronize()
    G = w["Hq"] // w["Hkv"]
    scale = 1.0 / np.sqrt(w["D"])
    lens = np.asarray(w["q_lens"])
    for b in (int(np.argmax(lens)), int(np.argmin(lens))):
        hk = 3
        q0, L = int(m["cu_q_np"][b]), int(lens[b])
        print(f"[backward full size] sequence {b} length {L} kv head {hk}", flush=True)
        sl = slice(q0, q0 + L)
        kh = I.bf16_to_f64(m["k"][sl, hk])
        vh = I.bf16_to_f64(m["v"][sl, hk])
        vis = np.tril(np.ones((L, L), dtype=bool))
        rk = np.zeros((L, w["D"]))
        rv = np.zeros((L, w["D"]))
        for h in range(hk * G, hk * G + G):
            gq, gk, gv = BW.backward_rows(I.bf16_to_f64(m["q"][sl, h]), kh, vh,
                                          I.bf16_to_f64(dout[sl, h]), vis, scale)
            assert_grad_close(I.bf16_to_f64(dq[sl, h]), gq, f"dq b={b} h={h}")
            rk += gk
            rv += gv
        assert_grad_close(I.bf16_to_f64(dk[sl, hk]), rk, f"dk b={b}", heads=G)
        assert_grad_close(I.bf16_to_f64(dv[sl, hk]), rv, f"dv b={b}", heads=G)


def test_backward_graph_replay_with_changing_lengths():
    """Forward + backward captured once in a graph and replayed with new
    device-side lengths (copied into the captured cu buffers between replays
    by the program's own eager work): every replay equals the eager call on
    the same lengths, bit for bit."""
    import varlen_gqa_attention_amd as V
    Hq, Hkv, D, smax, B = 8, 2, 64, 300, 4
    steps = 4
    lens = [I.uniform_lengths(B, 0, smax, 9, t) for t in range(steps)]
    T = smax * B
    q = I.normal_bf16((T, Hq, D), 1, "cuda")
    k = I.normal_bf16((T, Hkv, D), 2, "cuda")
    v = I.normal_bf16((T, Hkv, D), 3, "cuda")
    dout = I.normal_bf16((T, Hq, D), 4, "cuda")
    plan = V.Plan(B, smax, smax, Hq, Hkv, D, True, backward=True)
    cu = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    lse = torch.zeros(T, Hq, device="cuda")
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)

    def step():
        plan(q, k, v, cu, cu, out=out, lse=lse, B=B)
        plan.backward(q, k, v, out, lse, dout, cu, cu, dq=dq, dk=dk, dv=dv, B=B)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        step()
    torch.cuda.synchronize()
    for t in range(steps):
        cu.copy_(torch.from_numpy(I.cu_from_lengths(lens[t])).cuda())
        for x in (dq, dk, dv):
            x.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (dq, dk, dv)]
        for x in (dq, dk, dv):
            x.zero_()
        step()                                    # eager, same lengths
        torch.cuda.synchronize()
        for a, b in zip(got, (dq, dk, dv)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), t


def test_backward_clamps_and_flags_invalid_lengths_and_b0_is_a_noop():
    """A length above s_max is clamped (as in the forward) and flagged; the
    gradients equal the oracle's on the clamped sequence. B = 0 enqueues
    nothing."""
    import varlen_gqa_attention_amd as V
    Hq, Hkv, D = 4, 1, 64
    plan = V.Plan(2, 96, 96, Hq, Hkv, D, True, backward=True)
    q = I.normal_bf16((200, Hq, D), 11, "cuda")
    k = I.normal_bf16((200, Hkv, D), 12, "cuda")
    v = I.normal_bf16((200, Hkv, D), 13, "cuda")
    dout = I.normal_bf16((200, Hq, D), 14, "cuda")
    cu = np.array([0, 150, 190], dtype=np.int32)          # first length 150 > s_max 96
    cu_t = torch.from_numpy(cu).cuda()
    out, lse = plan(q, k, v, cu_t, cu_t, B=2)
    plan.clear_error()
    dq, dk, dv = (torch.zeros_like(x) for x in (q, k, v))
    plan.backward(q, k, v, out, lse, dout, cu_t, cu_t, dq=dq, dk=dk, dv=dv, B=2)
    torch.cuda.synchronize()
    assert plan.read_error() & V.ERRBIT_Q_LEN
    rq, rk, rv, wq, wk = BW.attend_varlen_backward(
        I.bf16_to_f64(q), I.bf16_to_f64(k), I.bf16_to_f64(v), I.bf16_to_f64(dout), cu, cu, 2,
        True, s_max_q=96, s_max_kv=96)
    assert_grad_close(I.bf16_to_f64(dq)[wq], rq[wq], "clamped dq")
    assert_grad_close(I.bf16_to_f64(dk)[wk], rk[wk], "clamped dk", heads=Hq // Hkv)
    assert_grad_close(I.bf16_to_f64(dv)[wk], rv[wk], "clamped dv", heads=Hq // Hkv)
    before = [x.clone() for x in (dq, dk, dv)]
    plan.backward(q, k, v, out, lse, dout, cu_t, cu_t, dq=dq, dk=dk, dv=dv, B=0)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(before, (dq, dk, dv)))
