"""CPU checks of the C ABI: the library builds and loads, exports every
function include/vattn.h declares, and its host-only plan chooser equals the
oracle's split rule; plus the pure C++ chooser test (no HIP)."""
import os
import re
import subprocess

import pytest

from oracle.chooser import choose_decode_split, choose_prefill_grid

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vattn.h")


def _lib():
    from varlen_gqa_attention_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vattn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    from varlen_gqa_attention_amd._lib import EXPORTS
    assert declared_functions() == sorted(EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "varlen_gqa_attention_amd",
                                                                     "libvattn.so")],
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (vattn_\w+)", out))
    assert set(declared_functions()) <= exported
    assert L.vattn_abi_version() == 4


SWEEP = [(B, S, Hq, Hkv) for B in (1, 2, 33, 64, 300) for S in (1, 100, 4096, 32768)
         for Hq, Hkv in ((4, 1), (32, 8), (64, 8), (128, 8), (16, 16))]


@pytest.mark.parametrize("B,S,Hq,Hkv", SWEEP)
@pytest.mark.parametrize("n_cu", [256, 80])
def test_describe_equals_oracle_rule(B, S, Hq, Hkv, n_cu):
    import varlen_gqa_attention_amd as V
    _lib()
    info = V.describe_plan(B, 1, S, Hq, Hkv, 128, 0, n_cu_override=n_cu)
    units = Hkv * info["head_blocks"]
    want = choose_decode_split(B, S, units, n_cu, info["block_n"], target_blocks_per_cu=16,
                               min_chunk_tiles=16)
    for key in ("nsplit", "chunk_keys", "grid", "direct", "n_tiles"):
        assert info[key] == int(want[key]), key
    # the default target scales with 128 / D (64, 32, 16, 8 workgroups per CU)
    for D in (32, 64, 256):
        info = V.describe_plan(B, 1, S, Hq, Hkv, D, 0, n_cu_override=n_cu)
        want = choose_decode_split(B, S, Hkv * info["head_blocks"], n_cu, info["block_n"],
                                   target_blocks_per_cu=16 * 128 // D, min_chunk_tiles=16)
        for key in ("nsplit", "chunk_keys", "grid", "direct", "n_tiles"):
            assert info[key] == int(want[key]), (D, key)
    # the default s_max grid follows the oracle's grid rule; the scheduled
    # option (prefill_grid=1) is one workgroup per CU over a device-built list
    p = V.describe_plan(B, max(2, S), S, Hq, Hkv, 128, 1, n_cu_override=n_cu)
    g = choose_prefill_grid(B, max(2, S), Hkv, p["q_tokens_per_tile"])
    assert p["n_qtiles"] == g["n_qtiles"] and p["prefill_persistent"] == 0
    assert p["grid"] == 8 * -(-(B * Hkv) // 8) * g["n_qtiles"]
    d = V.describe_plan(B, max(2, S), S, Hq, Hkv, 128, 1, n_cu_override=n_cu, prefill_grid=1)
    assert d["n_qtiles"] == g["n_qtiles"]
    assert d["prefill_persistent"] == 1 and d["grid"] == n_cu
    assert d["scratch_bytes"] == 512 + 4 * B * g["n_qtiles"]


@pytest.mark.parametrize("B,S,Hq,Hkv", SWEEP)
@pytest.mark.parametrize("n_cu", [256, 80])
def test_describe_pages_rule_equals_oracle_default(B, S, Hq, Hkv, n_cu):
    """The pages' split rule (target 2 workgroups per CU, no work floor) is
    selectable through the plan options, and the library's chooser then equals
    the oracle's chooser at its defaults, bit for bit."""
    import varlen_gqa_attention_amd as V
    _lib()
    info = V.describe_plan(B, 1, S, Hq, Hkv, 128, 0, n_cu_override=n_cu,
                           target_blocks_per_cu=2, min_chunk_tiles=1)
    units = Hkv * info["head_blocks"]
    want = choose_decode_split(B, S, units, n_cu, info["block_n"])
    for key in ("nsplit", "chunk_keys", "grid", "direct", "n_tiles"):
        assert info[key] == int(want[key]), key
    # merge: in the split kernel when all split workgroups fit the device at
    # once and the units are a multiple of 8; else a combine kernel of one
    # workgroup per (sequence, two query heads) at D = 128
    fused = not want["direct"] and (B * units) % 8 == 0 and want["grid"] <= n_cu
    assert info["fused_combine"] == int(fused)
    assert info["combine_grid"] == (0 if want["direct"] or fused else B * -(-Hq // 2))
    same = V.describe_plan(B, 1, S, Hq, Hkv, 128, 0, n_cu_override=n_cu, split_rule="pages")
    assert same == info


@pytest.mark.parametrize("T,F", [(1, 1), (2, 16), (4, 4), (8, 1), (16, 8), (3, 2)])
@pytest.mark.parametrize("B,S,Hq,Hkv", SWEEP[::4])
def test_describe_any_target_and_floor_equals_oracle(T, F, B, S, Hq, Hkv):
    import varlen_gqa_attention_amd as V
    _lib()
    info = V.describe_plan(B, 1, S, Hq, Hkv, 64, 0, n_cu_override=256,
                           target_blocks_per_cu=T, min_chunk_tiles=F)
    want = choose_decode_split(B, S, Hkv * info["head_blocks"], 256, info["block_n"],
                               target_blocks_per_cu=T, min_chunk_tiles=F)
    for key in ("nsplit", "chunk_keys", "grid", "direct", "n_tiles"):
        assert info[key] == int(want[key]), key


def test_default_rule_constants():
    """All-zero options select the documented default (16 per CU at D = 128,
    scaled by 128 / D; 16 tiles)."""
    import varlen_gqa_attention_amd as V
    _lib()
    for B, S in ((1, 32768), (64, 8192), (16, 2048), (2, 128), (33, 16384)):
        for D in (32, 64, 128, 256):
            a = V.describe_plan(B, 1, S, 32, 8, D, 0, n_cu_override=256)
            b = V.describe_plan(B, 1, S, 32, 8, D, 0, n_cu_override=256,
                                target_blocks_per_cu=16 * 128 // D, min_chunk_tiles=16)
            assert a == b
    with pytest.raises(ValueError):
        V.describe_plan(1, 1, 64, 8, 8, 64, 0, n_cu_override=256, split_rule="pages",
                        target_blocks_per_cu=2)


@pytest.mark.parametrize("force", [1, 2, 3, 7, 32, 100])
def test_describe_forced_split_equals_oracle(force):
    import varlen_gqa_attention_amd as V
    _lib()
    info = V.describe_plan(3, 1, 4097, 16, 2, 128, 0, n_cu_override=256, force_nsplit=force)
    want = choose_decode_split(3, 4097, 2, 256, 64, force_nsplit=force)
    assert (info["nsplit"], info["chunk_keys"]) == (want["nsplit"], want["chunk_keys"])


def test_describe_status_codes():
    import varlen_gqa_attention_amd as V
    _lib()
    with pytest.raises(V.VattnError) as e:
        V.describe_plan(1, 1, 64, 6, 4, 64, 0, n_cu_override=256)
    assert e.value.status == -1
    with pytest.raises(V.VattnError) as e:
        V.describe_plan(1, 1, 64, 8, 2, 48, 0, n_cu_override=256)
    assert e.value.status == -2


def test_pure_cpp_plan_test(tmp_path):
    src = os.path.join(ROOT, "varlen_gqa_attention_amd", "csrc")
    exe = tmp_path / "test_plan"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-o", str(exe),
                    os.path.join(src, "tests", "test_plan.cpp"), os.path.join(src, "plan.cpp")],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(1, 100, 8, 8, 64), (16, 4096, 32, 8, 128),
                                          (3, 1000, 12, 4, 32), (64, 1, 128, 1, 128),
                                          (5, 700, 16, 2, 256)])
def test_describe_backward_grids(B, S, Hq, Hkv, D):
    """Backward plans: the dq grid follows the forward's grid rule at 256 rows
    per workgroup, the dk/dv grid covers 128-key tiles, and the plan's scratch
    grows by the row-wise <dout, out> buffer."""
    import varlen_gqa_attention_amd as V
    _lib()
    base = V.describe_plan(B, S, S, Hq, Hkv, D, 1, n_cu_override=256)
    d = V.describe_plan(B, S, S, Hq, Hkv, D, 1, n_cu_override=256, backward=1)
    G = Hq // Hkv
    rows, slices = (256, 1) if D <= 128 else (128, 2)   # 128-column slices at D = 256
    g = choose_prefill_grid(B, S, Hkv, rows // G)
    assert d["backward"] == 1 and d["bwd_q_tokens_per_tile"] == rows // G
    assert d["bwd_grid_dq"] == 8 * -(-(B * Hkv) // 8) * g["n_qtiles"] * slices
    assert d["bwd_grid_dkdv"] == 8 * -(-(B * Hkv) // 8) * -(-S // 128) * slices
    assert d["scratch_bytes"] == base["scratch_bytes"] + 256 + 4 * B * S * Hq
    assert base["backward"] == 0 and base["bwd_grid_dq"] == 0


@pytest.mark.parametrize("s_max_q,Hq,Hkv,D", [(1, 256, 1, 256), (1, 512, 1, 64)])
def test_backward_plan_limits(s_max_q, Hq, Hkv, D):
    """G above the dq workgroup's rows (128 at D = 256, else 256) has no
    backward; the (decode) forward plan is fine."""
    import varlen_gqa_attention_amd as V
    _lib()
    with pytest.raises(V.VattnError) as e:
        V.describe_plan(2, s_max_q, 64, Hq, Hkv, D, 1, n_cu_override=256, backward=1)
    assert e.value.status == -2
    V.describe_plan(2, s_max_q, 64, Hq, Hkv, D, 1, n_cu_override=256)


def test_plan_released_during_capture_is_freed_after_it(monkeypatch):
    """A plan handle released while the current stream captures a graph is not
    freed then (hipFree would invalidate a global-mode capture), but at the
    next release outside a capture; nothing is freed twice."""
    import varlen_gqa_attention_amd as V
    freed = []

    class FakeLib:
        def vattn_plan_destroy(self, h):
            freed.append(h)

    monkeypatch.setattr(V, "_LIB", FakeLib())
    monkeypatch.setattr(V, "_deferred_handles", [])
    capturing = [True]
    monkeypatch.setattr(V, "_capturing", lambda: capturing[0])
    V._destroy_handle("a")
    V._destroy_handle("b")
    assert freed == [] and V._deferred_handles == ["a", "b"]
    V._release_deferred()               # still capturing: nothing happens
    assert freed == []
    capturing[0] = False
    V._destroy_handle("c")
    assert sorted(freed) == ["a", "b", "c"] and V._deferred_handles == []
    V._release_deferred()
    assert sorted(freed) == ["a", "b", "c"]
