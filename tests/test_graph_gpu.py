"""Continuous batching under graph capture: one capture of {advance lengths,
execute}, replayed with new device-side lengths each step, no host work in
between; sampled steps checked against the oracle."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.parity import assert_lse_close, assert_out_close
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nsplit,fuse", [(0, 0), (4, 0), (4, 1)])
def test_graph_replay_with_changing_lengths(nsplit, fuse):
    import varlen_gqa_attention_amd as V
    B, Hq, Hkv, D, smax, steps = 16, 32, 8, 128, 2048, 12
    lens = [I.uniform_lengths(B, 1, smax, 2, t) for t in range(steps)]
    cu_steps = torch.from_numpy(np.stack([I.cu_from_lengths(l) for l in lens])).cuda()
    pool = smax * B
    q = I.normal_bf16((B, Hq, D), 100, "cuda")
    k = I.normal_bf16((pool, Hkv, D), 101, "cuda")
    v = I.normal_bf16((pool, Hkv, D), 102, "cuda")
    cu_q = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    live = torch.zeros(1, B + 1, dtype=torch.int32, device="cuda")
    step = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.zeros_like(q)
    lse = torch.zeros(B, Hq, device="cuda")
    outs = torch.zeros(steps, B, Hq, D, dtype=torch.bfloat16, device="cuda")
    lses = torch.zeros(steps, B, Hq, device="cuda")
    plan = V.Plan(B, 1, smax, Hq, Hkv, D, False, force_nsplit=nsplit, fuse_combine=fuse)
    print(f"[graph] plan {plan.info}", flush=True)

    def one_step():
        torch.index_select(cu_steps, 0, step, out=live)
        plan(q, k, v, cu_q, live.view(-1), out=out, lse=lse, B=B)
        outs.index_copy_(0, step, out.unsqueeze(0))
        lses.index_copy_(0, step, lse.unsqueeze(0))
        step.add_(1)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        one_step()                       # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    step.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        one_step()
    torch.cuda.synchronize()
    step.zero_()
    for t in range(steps):
        g.replay()
        if t >= steps // 2:              # second half: eager work + syncs between replays
            torch.cuda.synchronize()
            _ = (q.float() * 2).sum()
    torch.cuda.synchronize()
    assert int(step.item()) == steps
    # every replay equals an eager execution of the same step, bit for bit
    for t in range(steps):
        o_e, l_e = plan(q, k, v, cu_q, cu_steps[t].contiguous(), B=B)
        torch.cuda.synchronize()
        assert torch.equal(o_e.view(torch.int16), outs[t].view(torch.int16)), f"step {t}"
        assert torch.equal(l_e, lses[t]), f"step {t}"
    qf, kf, vf = I.bf16_to_f64(q), I.bf16_to_f64(k), I.bf16_to_f64(v)
    for t in range(steps):
        ref_o, ref_l, _ = A.attend_varlen(qf, kf, vf, np.arange(B + 1), cu_steps[t].cpu().numpy(),
                                          B, False)
        assert_out_close(I.bf16_to_f64(outs[t]), ref_o, f"step {t}")
        assert_lse_close(lses[t].cpu().numpy(), ref_l, f"step {t}")
