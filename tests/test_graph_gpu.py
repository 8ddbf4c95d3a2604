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


@pytest.mark.timeout(400)
def test_continuous_batching_full_size_graph_replay():
    """The continuous-batching workload at its own size: B=64, Hq=32, Hkv=8,
    D=128, one plan with s_max_kv=8192, one capture of {select this step's
    cu_seqlens on the device, execute, keep the sampled steps' results},
    replayed 100 times with lengths U[128, 8192] per step (seed (2, t)). Steps
    0, 1, 50 and 99 are checked against the oracle and, bit for bit, against
    an eager execute of the same step."""
    import varlen_gqa_attention_amd as V
    steps, sampled = 100, (0, 1, 50, 99)
    ws = [I.batched_decode_step(t) for t in range(steps)]
    B, Hq, Hkv, D, smax = 64, 32, 8, 128, 8192
    cu_steps = torch.from_numpy(np.stack([I.cu_from_lengths(w["kv_lens"]) for w in ws])).cuda()
    pool = B * smax
    q = I.normal_bf16((B, Hq, D), 120, "cuda")
    k = I.normal_bf16((pool, Hkv, D), 121, "cuda")
    v = I.normal_bf16((pool, Hkv, D), 122, "cuda")
    cu_q = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    live = torch.zeros(1, B + 1, dtype=torch.int32, device="cuda")
    step = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.zeros_like(q)
    lse = torch.zeros(B, Hq, device="cuda")
    # slot of each step in the kept results: sampled steps 0..3, the rest 4
    slot_of = torch.full((steps,), len(sampled), dtype=torch.int64)
    for i, t in enumerate(sampled):
        slot_of[t] = i
    slot_of = slot_of.cuda()
    slot = torch.zeros(1, dtype=torch.int64, device="cuda")
    outs = torch.zeros(len(sampled) + 1, B, Hq, D, dtype=torch.bfloat16, device="cuda")
    lses = torch.zeros(len(sampled) + 1, B, Hq, device="cuda")
    plan = V.Plan(B, 1, smax, Hq, Hkv, D, False)
    print(f"[graph full size] plan {plan.info}", flush=True)

    def one_step():
        torch.index_select(cu_steps, 0, step, out=live)
        plan(q, k, v, cu_q, live.view(-1), out=out, lse=lse, B=B)
        torch.index_select(slot_of, 0, step, out=slot)
        outs.index_copy_(0, slot, out.unsqueeze(0))
        lses.index_copy_(0, slot, lse.unsqueeze(0))
        step.add_(1)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        one_step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        one_step()
    torch.cuda.synchronize()
    step.zero_()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    assert int(step.item()) == steps
    print("[graph full size] 100 replays done", flush=True)
    rows = int(cu_steps[list(sampled)].max().item())
    qf, kf, vf = I.bf16_to_f64(q), I.bf16_to_f64(k[:rows]), I.bf16_to_f64(v[:rows])
    for i, t in enumerate(sampled):
        cu_t = cu_steps[t].contiguous()
        o_e, l_e = plan(q, k, v, cu_q, cu_t, B=B)
        torch.cuda.synchronize()
        assert torch.equal(o_e.view(torch.int16), outs[i].view(torch.int16)), f"step {t}"
        assert torch.equal(l_e, lses[i]), f"step {t}"
        ref_o, ref_l, _ = A.attend_varlen(qf, kf, vf, np.arange(B + 1), cu_t.cpu().numpy(), B,
                                          False)
        assert_out_close(I.bf16_to_f64(outs[i]), ref_o, f"step {t}")
        assert_lse_close(lses[i].cpu().numpy(), ref_l, f"step {t}")
        print(f"[graph full size] step {t} matches the oracle", flush=True)


@pytest.mark.timeout(400)
def test_continuous_batching_hundred_steps_in_one_graph():
    """The continuous-batching workload as the benchmark times it: its 100
    steps (B=64, Hq=32, Hkv=8, D=128, s_max_kv=8192, lengths U[128, 8192]
    per step) captured back to back in one graph, each step reading its own
    cu_seqlens row and writing its own output slot; replayed twice. Steps 0,
    1, 50 and 99 match the oracle and, bit for bit, an eager execute."""
    import varlen_gqa_attention_amd as V
    steps, sampled = 100, (0, 1, 50, 99)
    ws = [I.batched_decode_step(t) for t in range(steps)]
    B, Hq, Hkv, D, smax = 64, 32, 8, 128, 8192
    cu_all = torch.from_numpy(np.stack([I.cu_from_lengths(w["kv_lens"]) for w in ws])).cuda()
    cu_rows = [cu_all[t] for t in range(steps)]
    pool = B * smax
    q = I.normal_bf16((B, Hq, D), 130, "cuda")
    k = I.normal_bf16((pool, Hkv, D), 131, "cuda")
    v = I.normal_bf16((pool, Hkv, D), 132, "cuda")
    cu_q = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    outs = torch.zeros(steps, B, Hq, D, dtype=torch.bfloat16, device="cuda")
    lses = torch.zeros(steps, B, Hq, device="cuda")
    plan = V.Plan(B, 1, smax, Hq, Hkv, D, False)
    print(f"[graph 100 steps] plan {plan.info}", flush=True)

    def all_steps():
        for t in range(steps):
            plan(q, k, v, cu_q, cu_rows[t], out=outs[t], lse=lses[t], B=B)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        all_steps()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        all_steps()
    torch.cuda.synchronize()
    outs.zero_()
    lses.zero_()
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
    print("[graph 100 steps] replays done", flush=True)
    rows = int(cu_all[list(sampled)].max().item())
    qf, kf, vf = I.bf16_to_f64(q), I.bf16_to_f64(k[:rows]), I.bf16_to_f64(v[:rows])
    for t in sampled:
        o_e, l_e = plan(q, k, v, cu_q, cu_rows[t], B=B)
        torch.cuda.synchronize()
        assert torch.equal(o_e.view(torch.int16), outs[t].view(torch.int16)), f"step {t}"
        assert torch.equal(l_e, lses[t]), f"step {t}"
        ref_o, ref_l, _ = A.attend_varlen(qf, kf, vf, np.arange(B + 1), cu_rows[t].cpu().numpy(), B,
                                          False)
        assert_out_close(I.bf16_to_f64(outs[t]), ref_o, f"step {t}")
        assert_lse_close(lses[t].cpu().numpy(), ref_l, f"step {t}")
        print(f"[graph 100 steps] step {t} matches the oracle", flush=True)


def test_plan_collected_inside_a_capture():
    """A plan that only a reference cycle keeps alive, collected by the garbage
    collector while a global-mode capture is open, must not free its scratch
    inside the capture: the capture completes and replays correctly."""
    import gc
    import varlen_gqa_attention_amd as V
    B, Hq, Hkv, D, smax = 4, 8, 2, 64, 256
    lens = I.uniform_lengths(B, 1, smax, 5, 0)
    cu_kv = torch.from_numpy(I.cu_from_lengths(lens)).cuda()
    q = I.normal_bf16((B, Hq, D), 110, "cuda")
    k = I.normal_bf16((B * smax, Hkv, D), 111, "cuda")
    v = I.normal_bf16((B * smax, Hkv, D), 112, "cuda")
    cu_q = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    plan = V.Plan(B, 1, smax, Hq, Hkv, D, False, force_nsplit=2)
    out = torch.zeros_like(q)
    lse = torch.zeros(B, Hq, device="cuda")
    plan(q, k, v, cu_q, cu_kv, out=out, lse=lse, B=B)   # warm-up outside capture
    torch.cuda.synchronize()
    gc.collect()
    doomed = V.Plan(B, 1, smax, Hq, Hkv, D, False)
    cycle = {"plan": doomed}
    cycle["self"] = cycle
    del doomed, cycle
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s, capture_error_mode="global"):
        gc.collect()                    # the cycle's plan is released here
        plan(q, k, v, cu_q, cu_kv, out=out, lse=lse, B=B)
    torch.cuda.synchronize()
    assert len(V._deferred_handles) == 1
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    o_e, l_e = plan(q, k, v, cu_q, cu_kv, B=B)
    torch.cuda.synchronize()
    assert torch.equal(o_e.view(torch.int16), out.view(torch.int16))
    assert torch.equal(l_e, lse)
    V._release_deferred()
    assert V._deferred_handles == []
