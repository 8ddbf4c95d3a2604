"""Seeded random configurations through the C ABI vs the oracle (GPU).

Each case draws a batch size, ragged lengths (zeros, ones and tile
boundaries included), a GQA grouping, a head dimension, causal or full
attention, decode or prefill, a split count, a prefill grid option, and
whether q / k / v are slices of a fused buffer; prefill cases also run the
backward. Everything is compared with the fp64 oracle to the parity bounds.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import backward as BW
from tests.parity import assert_grad_close, assert_lse_close, assert_out_close
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

SPECIAL = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129]


def _lengths(rng, B, hi):
    out = []
    for _ in range(B):
        if rng.random() < 0.4:
            out.append(min(hi, int(rng.choice(SPECIAL))))
        else:
            out.append(int(rng.integers(0, hi + 1)))
    return np.array(out, dtype=np.int64)


def _case(seed):
    rng = np.random.default_rng([31, seed])
    D = int(rng.choice([32, 64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8, 16] if D < 256 else [1, 2, 4, 8]))
    decode = bool(rng.random() < 0.4)
    B = int(rng.integers(1, 7))
    B_max = B + int(rng.integers(0, 3))
    causal = bool(rng.random() < 0.7)
    s_max_kv = int(rng.choice([64, 129, 300]))
    if decode:
        q_lens = np.ones(B, np.int64)
        q_lens[rng.random(B) < 0.15] = 0
        s_max_q = 1
    else:
        s_max_q = s_max_kv
        q_lens = _lengths(rng, B, s_max_q)
    kv_lens = _lengths(rng, B, s_max_kv)
    if not decode and rng.random() < 0.5:
        kv_lens = q_lens.copy()                        # self-attention shape
    opts = {}
    if decode:
        opts["force_nsplit"] = int(rng.choice([0, 0, 1, 2, 3, 7]))
        opts["force_decode_path"] = int(rng.choice([0, 0, 1, 2]))
    else:
        opts["prefill_grid"] = int(rng.integers(0, 2))
        opts["backward"] = 1
    fused = bool(rng.random() < 0.3)
    return dict(D=D, Hkv=Hkv, Hq=Hkv * G, B=B, B_max=B_max, causal=causal, decode=decode,
                s_max_q=s_max_q, s_max_kv=s_max_kv, q_lens=q_lens, kv_lens=kv_lens, opts=opts,
                fused=fused)


@pytest.mark.parametrize("seed", range(120))
def test_random_configuration(seed):
    import varlen_gqa_attention_amd as V
    c = _case(seed)
    print(f"[sweep {seed}] D={c['D']} Hq={c['Hq']} Hkv={c['Hkv']} B={c['B']}/{c['B_max']} "
          f"decode={c['decode']} causal={c['causal']} fused={c['fused']} opts={c['opts']} "
          f"q={c['q_lens'].tolist()} kv={c['kv_lens'].tolist()}", flush=True)
    B, Hq, Hkv, D = c["B"], c["Hq"], c["Hkv"], c["D"]
    cu_q = I.cu_from_lengths(c["q_lens"], capacity=c["B_max"] + 1, tail=[-1, 2**31 - 1])
    cu_k = I.cu_from_lengths(c["kv_lens"], capacity=c["B_max"] + 1, tail=[-1, 2**31 - 1])
    Tq = max(1, int(c["q_lens"].sum()))
    Tk = max(1, int(c["kv_lens"].sum()))
    T = max(Tq, Tk)
    if c["fused"]:
        qkv = I.normal_bf16((T, Hq + 2 * Hkv, D), 1000 + seed, "cuda")
        q, k, v = qkv[:Tq, :Hq], qkv[:Tk, Hq:Hq + Hkv], qkv[:Tk, Hq + Hkv:]
    else:
        q = I.normal_bf16((Tq, Hq, D), 2000 + seed, "cuda")
        k = I.normal_bf16((Tk, Hkv, D), 3000 + seed, "cuda")
        v = I.normal_bf16((Tk, Hkv, D), 4000 + seed, "cuda")
    plan = V.Plan(c["B_max"], c["s_max_q"], c["s_max_kv"], Hq, Hkv, D, c["causal"], **c["opts"])
    cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    # zero-filled outputs: rows outside every sequence stay defined for the copy back
    out = torch.zeros(Tq, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(Tq, Hq, device="cuda")
    plan(q, k, v, cq, ck, out=out, lse=lse, B=B)
    torch.cuda.synchronize()
    assert plan.read_error() == 0
    qf, kf, vf = I.bf16_to_f64(q), I.bf16_to_f64(k), I.bf16_to_f64(v)
    ro, rl, wr = A.attend_varlen(qf, kf, vf, cu_q, cu_k, B, c["causal"])
    assert_out_close(I.bf16_to_f64(out)[wr], ro[wr], f"sweep {seed} out")
    assert_lse_close(lse.cpu().numpy()[wr], rl[wr], f"sweep {seed} lse")
    if c["decode"]:
        return
    dout = I.normal_bf16((Tq, Hq, D), 5000 + seed, "cuda")
    dq, dk, dv = (torch.zeros(t.shape, dtype=torch.bfloat16, device="cuda") for t in (q, k, v))
    plan.backward(q, k, v, out, lse, dout, cq, ck, dq=dq, dk=dk, dv=dv, B=B)
    torch.cuda.synchronize()
    gq, gk, gv, wq, wk = BW.attend_varlen_backward(qf, kf, vf, I.bf16_to_f64(dout), cu_q, cu_k,
                                                   B, c["causal"])
    assert_grad_close(I.bf16_to_f64(dq)[wq], gq[wq], f"sweep {seed} dq")
    assert_grad_close(I.bf16_to_f64(dk)[wk], gk[wk], f"sweep {seed} dk", heads=Hq // Hkv)
    assert_grad_close(I.bf16_to_f64(dv)[wk], gv[wk], f"sweep {seed} dv", heads=Hq // Hkv)
