"""Prefill parity: HIP causal varlen prefill vs the fp64 oracle (GPU)."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.parity import assert_lse_close, assert_out_close
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

SENT_OUT = 0x4B80
SENT_LSE = 12345.0


def _prefill_workload(name, Hq, Hkv, D, q_lens, kv_lens, causal=True, B_max=None,
                      s_max_q=None, s_max_kv=None):
    q_lens = np.asarray(q_lens, np.int64)
    kv_lens = np.asarray(kv_lens, np.int64)
    B = len(q_lens)
    return dict(name=name, B=B, B_max=B_max or B, Hq=Hq, Hkv=Hkv, D=D, causal=causal,
                q_lens=q_lens, kv_lens=kv_lens, s_max_q=s_max_q or max(2, int(q_lens.max())),
                s_max_kv=s_max_kv or max(1, int(kv_lens.max())))


def run_prefill(w, seed=0, picks=None, **opts):
    import varlen_gqa_attention_amd as V
    print(f"[prefill] {w['name']} seed={seed} B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} D={w['D']} "
          f"causal={w['causal']} q_lens={list(w['q_lens'])[:8]} opts={opts}", flush=True)
    m = I.materialise(w, seed, "cuda")
    plan = V.Plan(w["B_max"], w["s_max_q"], w["s_max_kv"], w["Hq"], w["Hkv"], w["D"], w["causal"],
                  **opts)
    out = torch.empty_like(m["q"]).view(torch.int16).fill_(SENT_OUT).view(torch.bfloat16)
    lse = torch.full(m["q"].shape[:2], SENT_LSE, dtype=torch.float32, device="cuda")
    plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], out=out, lse=lse, B=w["B"])
    torch.cuda.synchronize()
    assert plan.read_error() == 0
    got_o = I.bf16_to_f64(out)
    got_l = lse.cpu().numpy().astype(np.float64)
    if picks is None:
        q, k, v = (I.bf16_to_f64(m[n]) for n in ("q", "k", "v"))
        ref_o, ref_l, written = A.attend_varlen(q, k, v, m["cu_q_np"], m["cu_kv_np"], w["B"],
                                                w["causal"])
        assert_out_close(got_o[written], ref_o[written], w["name"])
        assert_lse_close(got_l[written], ref_l[written], w["name"])
        raw = out.view(torch.int16).cpu().numpy()
        assert (raw[~written] == np.int16(SENT_OUT)).all()
        assert (lse.cpu().numpy()[~written] == SENT_LSE).all()
    else:
        q, k, v = (m[n].cpu() for n in ("q", "k", "v"))
        rows = A.attend_selected(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                 m["cu_q_np"], m["cu_kv_np"], w["causal"], picks)
        ro = np.stack([r[2] for r in rows])
        rl = np.array([r[3] for r in rows])
        go = np.stack([got_o[r[0], r[1]] for r in rows])
        gl = np.array([got_l[r[0], r[1]] for r in rows])
        assert_out_close(go, ro, w["name"] + " sampled")
        assert_lse_close(gl, rl, w["name"] + " sampled")
    return plan, m, out, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_small_varlen(causal, G):
    lens = [1, 33, 130, 64, 65]
    run_prefill(_prefill_workload(f"small G={G}", 2 * G, 2, 64, lens, lens, causal), 1)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_head_dims(D):
    lens = [31, 32, 33, 127, 129, 200]
    run_prefill(_prefill_workload(f"D={D}", 8, 2, D, lens, lens, True), 2)


@pytest.mark.parametrize("G", [3, 16, 32])
def test_odd_and_large_groups(G):
    lens = [5, 40, 77]
    run_prefill(_prefill_workload(f"G={G}", G, 1, 64, lens, lens, True), 3)


GRIDS = [0, 1]  # s_max grid with dead-tile exit; device-built schedule on a persistent grid


@pytest.mark.parametrize("grid", GRIDS)
def test_bottom_right_causal_with_unequal_lengths(grid):
    # includes Lq > Lk (leading rows see no key) and Lq = 0
    w = _prefill_workload("Lq != Lk", 8, 2, 128, [5, 70, 0, 9, 40], [100, 30, 7, 0, 40], True)
    run_prefill(w, 4, prefill_grid=grid)


def test_noncausal_unequal_lengths():
    w = _prefill_workload("non-causal Lq != Lk", 8, 2, 64, [5, 70, 3], [100, 30, 1], False)
    run_prefill(w, 5)


@pytest.mark.parametrize("grid", GRIDS)
def test_tile_boundaries(grid):
    lens = [31, 32, 33, 63, 64, 65, 95, 96, 97, 128]
    run_prefill(_prefill_workload("boundaries", 32, 8, 128, lens, lens, True), 6, prefill_grid=grid)


@pytest.mark.parametrize("grid", GRIDS)
def test_unused_batch_slots_and_longer_cu_buffer(grid):
    w = _prefill_workload("B < B_max", 8, 2, 64, [17, 50], [17, 50], True, B_max=6, s_max_q=64,
                          s_max_kv=64)
    w["cu_capacity"], w["cu_tail"] = 9, [-1, 2**31 - 1, 0]
    run_prefill(w, 7, prefill_grid=grid)


def test_schedule_with_more_sequences_than_schedule_threads():
    # 1500 sequences (the schedule kernel loops over them), many empty, lengths
    # spanning zero to several query tiles
    lens = np.random.default_rng([5, 1]).integers(0, 200, size=1500)
    lens[::7] = 0
    w = _prefill_workload("many sequences", 4, 1, 32, lens, lens, True, s_max_q=256, s_max_kv=256)
    run_prefill(w, 9, prefill_grid=1)


@pytest.mark.parametrize("D", [64, 256])
def test_persistent_grid_smaller_than_work(D):
    # few CUs' worth of workgroups walking many tiles each
    lens = [300, 5, 257, 64, 1, 128]
    run_prefill(_prefill_workload(f"n_cu=3 D={D}", 8, 2, D, lens, lens, True), 10,
                n_cu_override=3, prefill_grid=1)


def test_full_size_varlen_prefill_sampled():
    w = I.varlen_prefill(0)
    rng = np.random.default_rng(123)
    picks = []
    for b, L in enumerate(w["q_lens"]):
        for i in sorted({0, 1, 31, 32, int(L) // 2, int(L) - 1, int(rng.integers(0, L))}):
            if i < L:
                for h in (0, 5, 31):
                    picks.append((b, i, h))
    run_prefill(w, 0, picks=picks)


@pytest.mark.parametrize("growth", [0.05, 0.5, 4.0])
@pytest.mark.parametrize("D", [64, 128])
def test_growing_scores(growth, D):
    """Keys scaled up along each sequence (key j of a sequence by 1 + growth *
    j / 64), so a row's max score climbs tile after tile: by a few base-2
    units over the sequence (weights stay against the first reference), by
    tens (weights past 2^8 but under 2^30, still no rescale), and by hundreds
    (tiles redone with the row max and O rescaled). Against the oracle. V is
    scaled by 1/4: a softmax this peaked puts nearly all weight on one key,
    so |O| follows |v|, and for |O| in [2, 4) one bf16 rounding of the output
    (up to 2^-7) plus the rounding of the dominant weight exceeds 1e-2 for any
    kernel that rounds P to bf16."""
    import varlen_gqa_attention_amd as V
    lens = [300, 129, 64, 700]
    w = _prefill_workload(f"growing scores x{growth}", 8, 2, D, lens, lens, True)
    print(f"[prefill] growing scores growth={growth} D={D}", flush=True)
    m = I.materialise(w, 5, "cuda")
    cu = m["cu_kv_np"]
    scale = torch.ones(m["k"].shape[0], device="cuda")
    for b in range(len(lens)):
        j = torch.arange(int(cu[b + 1] - cu[b]), device="cuda", dtype=torch.float32)
        scale[int(cu[b]):int(cu[b + 1])] = 1.0 + growth * j / 64.0
    k = (m["k"].float() * scale[:, None, None]).to(torch.bfloat16)
    v = (m["v"].float() * 0.25).to(torch.bfloat16)
    plan = V.Plan(w["B_max"], w["s_max_q"], w["s_max_kv"], w["Hq"], w["Hkv"], D, True)
    out, lse = plan(m["q"], k, v, m["cu_q"], m["cu_kv"], B=w["B"])
    torch.cuda.synchronize()
    ref_o, ref_l, written = A.attend_varlen(I.bf16_to_f64(m["q"]), I.bf16_to_f64(k),
                                            I.bf16_to_f64(v), m["cu_q_np"], cu, w["B"], True)
    assert np.isfinite(ref_l[written]).all()
    assert_out_close(I.bf16_to_f64(out)[written], ref_o[written], w["name"])
    assert_lse_close(lse.cpu().numpy().astype(np.float64)[written], ref_l[written], w["name"])


def test_exact_grid_and_both_planned_grids_agree_bitwise():
    import varlen_gqa_attention_amd as V
    w = _prefill_workload("exact grid", 32, 8, 128, [100, 1, 700, 64], [100, 1, 700, 64], True,
                          s_max_q=1024, s_max_kv=1024)
    plan, m, out, lse = run_prefill(w, 8)
    assert plan.info["prefill_persistent"] == 0
    tq = plan.info["q_tokens_per_tile"]
    tiles = [(b << 16) | t for b, L in enumerate(w["q_lens"]) for t in range(-(-int(L) // tq))]
    tmap = torch.tensor(tiles[::-1], dtype=torch.int32, device="cuda")
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    plan.execute_exact_grid(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], tmap, out2, lse2, w["B"])
    plan1 = V.Plan(w["B_max"], w["s_max_q"], w["s_max_kv"], w["Hq"], w["Hkv"], w["D"], True,
                   prefill_grid=1)
    assert plan1.info["prefill_persistent"] == 1
    out3 = torch.empty_like(out)
    lse3 = torch.empty_like(lse)
    plan1(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], out=out3, lse=lse3, B=w["B"])
    torch.cuda.synchronize()
    for o, l in ((out2, lse2), (out3, lse3)):
        assert torch.equal(out.view(torch.int16), o.view(torch.int16))
        assert torch.equal(lse, l)


def test_repeated_executes_reuse_the_schedule_bitwise():
    # the schedule is rebuilt on every execute (new lengths, same plan)
    import varlen_gqa_attention_amd as V
    plan = V.Plan(4, 512, 512, 8, 2, 64, True, prefill_grid=1)
    for step, lens in enumerate(([500, 3, 0, 77], [1, 512, 130, 9], [64, 64, 64, 64])):
        w = _prefill_workload(f"step {step}", 8, 2, 64, lens, lens, True, s_max_q=512,
                              s_max_kv=512)
        m = I.materialise(w, 20 + step, "cuda")
        out, lse = plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], B=4)
        torch.cuda.synchronize()
        q, k, v = (I.bf16_to_f64(m[n]) for n in ("q", "k", "v"))
        ro, rl, wr = A.attend_varlen(q, k, v, m["cu_q_np"], m["cu_kv_np"], 4, True)
        assert_out_close(I.bf16_to_f64(out)[wr], ro[wr], f"step {step}")
        assert_lse_close(lse.cpu().numpy().astype(np.float64)[wr], rl[wr], f"step {step}")
