"""Decode parity: HIP split-KV / direct decode vs the fp64 oracle (GPU).

Every case fills out/lse with sentinels first, so rows the library must not
write are checked bit-exactly, and compares every written row with the oracle
(tolerances in tests/parity.py).
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.chooser import choose_decode_split
from tests.parity import assert_lse_close, assert_out_close
from varlen_gqa_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

SENT_OUT = 0x4B80   # bf16 bit pattern of 16777216.0
SENT_LSE = 12345.0


def _vattn():
    import varlen_gqa_attention_amd as V
    return V


def run_decode(w, seed=0, B=None, **opts):
    V = _vattn()
    B = w["B"] if B is None else B
    print(f"[decode] {w['name']} seed={seed} B={B} Hq={w['Hq']} Hkv={w['Hkv']} D={w['D']} "
          f"opts={opts}", flush=True)
    m = I.materialise(w, seed, "cuda")
    plan = V.Plan(w["B_max"], w["s_max_q"], w["s_max_kv"], w["Hq"], w["Hkv"], w["D"],
                  w["causal"], **opts)
    out = torch.empty_like(m["q"]).view(torch.int16).fill_(SENT_OUT).view(torch.bfloat16)
    lse = torch.full(m["q"].shape[:2], SENT_LSE, dtype=torch.float32, device="cuda")
    plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], out=out, lse=lse, B=B)
    torch.cuda.synchronize()
    err = plan.read_error()
    q, k, v = (I.bf16_to_f64(m[n]) for n in ("q", "k", "v"))
    ref_o, ref_l, written = A.attend_varlen(q, k, v, m["cu_q_np"], m["cu_kv_np"], B, w["causal"])
    got_o = I.bf16_to_f64(out)
    got_l = lse.cpu().numpy().astype(np.float64)
    e1 = assert_out_close(got_o[written], ref_o[written], w["name"])
    e2 = assert_lse_close(got_l[written], ref_l[written], w["name"])
    raw = out.view(torch.int16).cpu().numpy()
    assert (raw[~written] == np.int16(SENT_OUT)).all(), "wrote rows outside the sequences"
    assert (lse.cpu().numpy()[~written] == SENT_LSE).all(), "wrote LSE outside the sequences"
    info = plan.info
    plan.close()
    return dict(out_err=e1, lse_err=e2, err_word=err, info=info, out=out)


def _w(name, B, Hq, Hkv, D, kv_lens, s_max_kv=None, B_max=None, causal=False, cu_capacity=None,
       cu_tail=None):
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    d = dict(name=name, B=B, B_max=B_max or B, Hq=Hq, Hkv=Hkv, D=D, causal=causal,
             q_lens=np.ones(B, np.int64), kv_lens=kv_lens, s_max_q=1,
             s_max_kv=s_max_kv or max(1, int(kv_lens.max())))
    if cu_capacity:
        d["cu_capacity"], d["cu_tail"] = cu_capacity, cu_tail
    return d


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_decode_default_plan(seed):
    # 128 keys at most: below the work floor of one split, so a direct pass
    r = run_decode(I.tiny_decode(seed), seed)
    assert r["info"]["nsplit"] == 1 and r["info"]["direct"]
    assert r["err_word"] == 0


def _pages_rule_plan_matches_oracle(w, info):
    """The plan the library chose under the pages' split rule equals the
    oracle chooser's default (pages') rule."""
    want = choose_decode_split(w["B_max"], w["s_max_kv"], w["Hkv"] * info["head_blocks"],
                               info["n_cu"], info["block_n"])
    assert (info["nsplit"], info["chunk_keys"], info["direct"], info["grid"]) == \
        (want["nsplit"], want["chunk_keys"], want["direct"], want["grid"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_decode_pages_rule(seed):
    """Tiny decode under the pages' rule: the tile count (2 tiles of 64 keys)
    binds, so two splits and the LSE combine."""
    w = I.tiny_decode(seed)
    r = run_decode(w, seed, split_rule="pages")
    _pages_rule_plan_matches_oracle(w, r["info"])
    assert r["info"]["nsplit"] == 2 and r["info"]["combine_grid"] > 0
    assert r["err_word"] == 0


def test_long_decode_pages_rule():
    w = I.long_decode()
    r = run_decode(w, 3, split_rule="pages")
    _pages_rule_plan_matches_oracle(w, r["info"])
    assert r["info"]["nsplit"] == 32


def test_batched_decode_full_size_pages_rule():
    """Continuous batching under the pages' rule: 64 x 8 units fill the
    device, so one direct-write pass and no combine."""
    w = I.batched_decode_step(2)
    r = run_decode(w, 2, split_rule="pages")
    _pages_rule_plan_matches_oracle(w, r["info"])
    assert r["info"]["direct"] and r["info"]["combine_grid"] == 0


@pytest.mark.parametrize("D", [32, 64, 256])
def test_edge_sweep_pages_rule(D):
    w = I.edge_sweep(D)
    r = run_decode(w, D, split_rule="pages")
    _pages_rule_plan_matches_oracle(w, r["info"])
    assert r["info"]["direct"] and r["err_word"] == 0


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("nsplit", [1, 2])
def test_tiny_decode_paths(path, nsplit):
    run_decode(I.tiny_decode(5), 5, force_decode_path=path, force_nsplit=nsplit)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 32])
def test_split_count_sweep(path, nsplit):
    w = _w("split sweep", 3, 16, 2, 128, [1, 1000, 4097])
    r = run_decode(w, 11, force_decode_path=path, force_nsplit=nsplit)
    units = w["Hkv"] * r["info"]["head_blocks"]
    want = choose_decode_split(w["B_max"], w["s_max_kv"], units, r["info"]["n_cu"],
                               r["info"]["block_n"], force_nsplit=nsplit)
    assert r["info"]["nsplit"] == want["nsplit"]
    assert r["info"]["chunk_keys"] == want["chunk_keys"]


def test_split_results_agree_across_split_counts():
    w = _w("split agreement", 2, 16, 2, 128, [3000, 777])
    outs = [run_decode(w, 12, force_nsplit=n)["out"].float() for n in (1, 2, 7, 32)]
    for o in outs[1:]:
        # different split counts only change rounding: within 2 bf16 ulp
        diff = (o - outs[0]).abs()
        ulp = outs[0].abs().clamp_min(2 ** -20) * 2 ** -7
        assert bool((diff <= 2 * ulp + 2 ** -12).all())


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 8, 16, 32])
@pytest.mark.parametrize("path", [1, 2])
def test_group_sizes(G, path):
    w = _w(f"G={G}", 3, 2 * G, 2, 64, [65, 2, 300])
    run_decode(w, 13 + G, force_decode_path=path)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("nsplit", [1, 3])
def test_head_dims(D, path, nsplit):
    w = _w(f"D={D}", 4, 16, 2, D, [1, 63, 64, 1025])
    run_decode(w, 17 + D, force_decode_path=path, force_nsplit=nsplit)


def test_long_decode_full_size():
    r = run_decode(I.long_decode(), 0)
    assert r["info"]["nsplit"] == 32 and r["info"]["grid"] == 256


def test_one_gpu_share_of_long_decode_with_forced_splits():
    # the head-sharded long decode on one of 8 GPUs (Hq=8, Hkv=1), default
    # plan and the split count the grid needs to fill the CUs
    w = _w("shard", 1, 8, 1, 128, [32768])
    r = run_decode(w, 5)
    assert r["info"]["nsplit"] == 32 and r["info"]["grid"] == 32
    r = run_decode(w, 6, force_nsplit=256)
    assert r["info"]["nsplit"] == 256 and r["info"]["grid"] == 256


def test_batched_decode_full_size():
    # 512 (sequence, kv head) units at 16 workgroups per CU: 8 splits, MFMA path
    r = run_decode(I.batched_decode_step(0), 0)
    assert r["info"]["nsplit"] == 8 and r["info"]["decode_path"] == 2


def test_batched_decode_full_size_direct_wave():
    # the single-pass direct write on the wave path, at the same size
    r = run_decode(I.batched_decode_step(1), 1, force_nsplit=1, force_decode_path=1)
    assert r["info"]["direct"] and r["info"]["decode_path"] == 1


@pytest.mark.parametrize("D", [32, 64, 256])
@pytest.mark.parametrize("nsplit", [0, 2, 3, 32])
def test_edge_sweep(D, nsplit):
    w = I.edge_sweep(D)
    r = run_decode(w, D, force_nsplit=nsplit)
    assert r["err_word"] == 0


def test_empty_and_zero_length_sequences():
    w = _w("empty kv", 4, 8, 2, 64, [0, 5, 0, 0], s_max_kv=128)
    for ns in (0, 2):
        r = run_decode(w, 21, force_nsplit=ns)
        assert r["err_word"] == 0


def test_zero_query_length_writes_nothing():
    V = _vattn()
    w = _w("no query", 2, 8, 2, 64, [10, 20])
    m = I.materialise(w, 22, "cuda")
    cu_q = torch.tensor([0, 0, 1], dtype=torch.int32, device="cuda")  # sequence 0 has no query
    plan = V.Plan(2, 1, 20, 8, 2, 64, False)
    out = torch.empty_like(m["q"]).view(torch.int16).fill_(SENT_OUT).view(torch.bfloat16)
    lse = torch.full(m["q"].shape[:2], SENT_LSE, device="cuda")
    plan(m["q"], m["k"], m["v"], cu_q, m["cu_kv"], out=out, lse=lse, B=2)
    torch.cuda.synchronize()
    q, k, v = (I.bf16_to_f64(m[n]) for n in ("q", "k", "v"))
    ref_o, ref_l, written = A.attend_varlen(q, k, v, [0, 0, 1], m["cu_kv_np"], 2, False)
    assert written.tolist() == [True, False]
    assert_out_close(I.bf16_to_f64(out)[:1], ref_o[:1])
    assert (out.view(torch.int16)[1].cpu().numpy() == np.int16(SENT_OUT)).all()


def test_b_zero_is_noop():
    V = _vattn()
    plan = V.Plan(4, 1, 64, 8, 2, 64, False)
    q = torch.zeros(4, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(4, 2, 64, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(5, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 3.0)
    lse = torch.full((4, 8), 3.0, device="cuda")
    plan(q, k, k, cu, cu, out=out, lse=lse, B=0)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((lse == 3.0).all())


@pytest.mark.parametrize("B,lens", [(5, [0, 1, 700, 2049, 4000]),   # 10 units: coherent form
                                    (4, [0, 1, 2049, 4000])])         # 8 units: XCD-local form
@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("nsplit", [2, 7, 32])
def test_fused_merge_equals_combine_kernel_bitwise(path, nsplit, B, lens):
    """The in-kernel merge (last split workgroup) and the combine kernel use
    the same arithmetic order: identical bits. With a unit count that is a
    multiple of 8 the in-kernel merge reads the partials through the XCD's
    L2 (plain loads), otherwise with cache-bypassing loads."""
    w = _w("fused vs combine", B, 16, 2, 128, lens, s_max_kv=4096)
    a = run_decode(w, 31, force_decode_path=path, force_nsplit=nsplit, fuse_combine=2)
    assert a["info"]["fused_combine"] == 0 and a["info"]["combine_grid"] > 0
    b = run_decode(w, 31, force_decode_path=path, force_nsplit=nsplit, fuse_combine=1)
    assert b["info"]["fused_combine"] == 1
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))


@pytest.mark.parametrize("which", ["long", "batched"])
def test_fused_merge_full_size_equals_combine_kernel_bitwise(which):
    """At the long-decode size (8 units x 32 splits, in-kernel merge by
    default) and at the continuous-batching size (512 units, forced), the
    XCD-local in-kernel merge equals the combine kernel bit for bit and
    matches the oracle; repeated launches repeat exactly."""
    import varlen_gqa_attention_amd as V
    w = I.long_decode() if which == "long" else I.batched_decode_step(3)
    fuse = 0 if which == "long" else 1
    a = run_decode(w, 41, fuse_combine=2)
    b = run_decode(w, 41, fuse_combine=fuse)
    assert b["info"]["fused_combine"] == 1 and a["info"]["fused_combine"] == 0
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))
    m = I.materialise(w, 41, "cuda")
    plan = V.Plan(w["B_max"], 1, w["s_max_kv"], w["Hq"], w["Hkv"], w["D"], False,
                  fuse_combine=fuse)
    outs = [plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], B=w["B"]) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o.view(torch.int16), b["out"].view(torch.int16))


def test_fused_plan_repeats_exactly():
    import varlen_gqa_attention_amd as V
    w = _w("fused repeat", 3, 64, 8, 128, [5000, 3, 9000], s_max_kv=9000)
    m = I.materialise(w, 32, "cuda")
    plan = V.Plan(3, 1, 9000, 64, 8, 128, False, force_nsplit=13, fuse_combine=1)
    assert plan.info["fused_combine"] == 1
    outs = []
    for _ in range(4):
        o, l = plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], B=3)
        outs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])
