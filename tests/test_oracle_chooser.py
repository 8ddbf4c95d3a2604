"""Pins of the plan-time split rule: the properties the rule states.

"Fill the device with about two blocks per CU, capped by tile count and 32;
single-pass direct write when batch * kv_heads already saturates": each
property below is one clause of that sentence, checked over a sweep.
"""
import itertools

import pytest

from oracle.chooser import choose_decode_split, choose_prefill_grid


SWEEP = list(itertools.product([1, 2, 7, 16, 33, 64, 128, 600],      # B_max
                               [1, 2, 8, 16],                         # Hkv
                               [1, 63, 64, 65, 512, 8192, 32768],     # s_max_kv
                               [256, 80, 304],                        # n_cu
                               [32, 64]))                             # block_n


@pytest.mark.parametrize("B,Hkv,S,n_cu,bn", SWEEP)
def test_split_rule_properties(B, Hkv, S, n_cu, bn):
    p = choose_decode_split(B, S, Hkv, n_cu, bn)
    n_units = B * Hkv
    n_tiles = -(-S // bn)
    ns, ch = p["nsplit"], p["chunk_tiles"]
    assert 1 <= ns <= 32 and ns <= n_tiles
    # contiguous chunks cover all tiles and none is empty at s_max
    assert (ns - 1) * ch < n_tiles <= ns * ch
    # never more splits than ~2 blocks/CU, the tile count or 32 ask for
    want = -(-2 * n_cu // n_units)
    target = max(1, min(want, n_tiles, 32))
    assert ns <= target
    # the chunk is the smallest one that stays within that count, so the
    # device is filled as far as the caps allow
    if ch > 1:
        assert -(-n_tiles // (ch - 1)) > target
    assert 2 * ns > target
    if target == want and ns == target:
        assert n_units * ns >= 2 * n_cu
    # direct write exactly when one split results; saturation implies it
    assert p["direct"] == (ns == 1)
    if n_units >= 2 * n_cu:
        assert p["direct"]
    assert p["grid"] == n_units * ns


def test_split_rule_named_regimes():
    # one sequence, 8 KV heads, 32768 keys on 256 CUs: the 32 cap binds
    p = choose_decode_split(1, 32768, 8, 256, 64)
    assert p["nsplit"] == 32 and p["grid"] == 256 and p["chunk_keys"] == 1024
    # 64 sequences x 8 KV heads = 512 units = 2 per CU: direct write
    assert choose_decode_split(64, 8192, 8, 256, 64)["direct"]
    # tile count binds for short KV
    assert choose_decode_split(2, 128, 1, 256, 64)["nsplit"] == 2


def test_forced_split_count():
    p = choose_decode_split(1, 1000, 1, 256, 64, force_nsplit=3)
    assert p["nsplit"] == 3 and p["chunk_tiles"] == 6
    p = choose_decode_split(1, 100, 1, 256, 64, force_nsplit=7)
    assert p["nsplit"] == 2          # only two tiles exist
    p = choose_decode_split(1, 64 * 40, 1, 256, 64, force_nsplit=7)
    assert p["nsplit"] == 7 and p["chunk_tiles"] == 6


def test_prefill_grid():
    g = choose_prefill_grid(16, 4096, 8, 32)
    assert g["grid"] == 16 * 128 * 8
    assert choose_prefill_grid(3, 33, 2, 32)["n_qtiles"] == 2


def test_work_floor_per_split():
    # with at least 16 tiles per split: 2048 keys, 128 units -> 2 splits of 1024
    p = choose_decode_split(16, 2048, 8, 256, 64, target_blocks_per_cu=8, min_chunk_tiles=16)
    assert (p["nsplit"], p["chunk_keys"]) == (2, 1024)
    # 8192 keys, 512 units at 8 per CU -> 4 splits (the floor allows 8; the
    # library's default of 16 per CU takes all 8)
    p = choose_decode_split(64, 8192, 8, 256, 64, target_blocks_per_cu=8, min_chunk_tiles=16)
    assert (p["nsplit"], p["chunk_keys"]) == (4, 2048)
    # 128 keys: one split, direct write
    assert choose_decode_split(2, 128, 1, 256, 64, target_blocks_per_cu=8,
                               min_chunk_tiles=16)["direct"]
    # the floor never lowers a count below what the tile count allows
    for S in (1, 64, 1000, 5000, 32768):
        for m in (1, 4, 16):
            p = choose_decode_split(1, S, 1, 256, 64, target_blocks_per_cu=8, min_chunk_tiles=m)
            n_tiles = -(-S // 64)
            assert 1 <= p["nsplit"] <= max(1, -(-n_tiles // m))
            assert p["chunk_tiles"] * p["nsplit"] >= n_tiles


# (target workgroups per CU, work floor in tiles): the pages' rule (2, 1),
# this library's default (8, 16), and others around them
RULES = [(2, 1), (16, 16), (8, 16), (1, 1), (4, 4), (8, 1), (2, 16), (16, 8)]


def _brute_force_split(B, S, Hkv, n_cu, bn, T, F, cap=32):
    """The split rule by enumeration: among chunk sizes (in tiles) whose split
    count stays within the bound min(ceil(T n_cu / units), tiles, cap,
    ceil(tiles / F)), the smallest chunk; the count is what that chunk needs."""
    units = B * Hkv
    tiles = -(-S // bn)
    bound = max(1, min(-(-T * n_cu // units), tiles, cap, -(-tiles // F)))
    for ch in range(1, tiles + 1):
        if -(-tiles // ch) <= bound:
            return -(-tiles // ch), ch, bound
    raise AssertionError("unreachable")


@pytest.mark.parametrize("T,F", RULES)
@pytest.mark.parametrize("B,Hkv,S,n_cu,bn", SWEEP[::3])
def test_split_rule_properties_any_target_and_floor(T, F, B, Hkv, S, n_cu, bn):
    """The oracle's rule with its two parameters: the split count equals the
    enumeration above, never exceeds the target, the tile count, 32 or the
    floor's bound, covers every tile with no empty split at s_max, and writes
    directly exactly when one split results."""
    p = choose_decode_split(B, S, Hkv, n_cu, bn, target_blocks_per_cu=T, min_chunk_tiles=F)
    ns, ch = p["nsplit"], p["chunk_tiles"]
    want_ns, want_ch, bound = _brute_force_split(B, S, Hkv, n_cu, bn, T, F)
    assert (ns, ch) == (want_ns, want_ch)
    tiles = -(-S // bn)
    assert 1 <= ns <= bound and ns <= 32 and ns <= tiles and ns <= -(-tiles // F)
    assert (ns - 1) * ch < tiles <= ns * ch
    assert 2 * ns > bound
    assert p["direct"] == (ns == 1)
    if B * Hkv >= T * n_cu:
        assert p["direct"]      # the batch's units alone fill the target
    assert p["grid"] == B * Hkv * ns and p["chunk_keys"] == ch * bn


def test_split_rule_pages_regimes_of_the_workloads():
    """The pages' rule (target 2, no floor) on the five workload shapes at
    64-key tiles and 256 CUs."""
    # tiny decode: 2 units, 128 keys -> the tile count (2) binds: two splits
    p = choose_decode_split(2, 128, 1, 256, 64)
    assert (p["nsplit"], p["chunk_keys"], p["direct"]) == (2, 64, False)
    # long decode: 8 units -> 64 wanted, the cap binds: 32 splits of 1024 keys
    p = choose_decode_split(1, 32768, 8, 256, 64)
    assert (p["nsplit"], p["chunk_keys"], p["grid"]) == (32, 1024, 256)
    # continuous batching: 64 x 8 = 512 units >= 2 per CU -> direct write
    p = choose_decode_split(64, 8192, 8, 256, 64)
    assert p["direct"] and p["grid"] == 512
    # edge sweep: B_max 64 x 8 units -> direct write
    p = choose_decode_split(64, 16384, 8, 256, 64)
    assert p["direct"] and p["grid"] == 512
    # one GPU's share of the long decode at 8-way head sharding: 1 unit ->
    # 512 wanted, the cap binds
    p = choose_decode_split(1, 32768, 1, 256, 64)
    assert p["nsplit"] == 32 and p["grid"] == 32
