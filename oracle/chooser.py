"""Plan-time split-count and grid rule (oracle) — TEST INFRASTRUCTURE ONLY.

Source: [ASTRAI] split-KV commit — the split count is chosen to fill the device
with about two blocks per compute unit, capped by the number of KV tiles and
by 32, and the kernel falls back to a single-pass direct write when
batch * kv_heads already saturates the device. [SPLITK] (The Thinking Process;
Assumptions and Their Validity): the count depends only on plan-time
quantities so it can be fixed inside a captured graph. [FROST#552] (How the
other backends avoid this; Proposal to evaluate): the grid is sized from the
declared batch and s_max at plan time; tiles past a sequence's real length
exit on the device.

Readings where the pages leave the rule open:
  * "about two blocks per CU" -> want = ceil(target * n_cu / n_units) with
    n_units = B_max * Hkv and target = 2;
  * "tile count" -> ceil(s_max_kv / block_n), block_n being the kernel's KV
    tile (an implementation choice, passed in here);
  * splits are contiguous ranges of chunk_tiles tiles; after capping, the
    count is recomputed as ceil(n_tiles / chunk_tiles) so that no split is
    empty at s_max_kv;
  * "already saturates" -> the rule yields one split; that plan writes the
    output directly and runs no combine step.
Prefill grids are B_max * ceil(s_max_q / q_tokens_per_tile) * Hkv, each block
covering the G query heads of one KV head (heads folded into the row
dimension, [KERNBENCH] "GQA via M-fold").
"""
from __future__ import annotations


def _cdiv(a, b):
    return -(-a // b)


def choose_decode_split(B_max, s_max_kv, Hkv, n_cu, block_n,
                        target_blocks_per_cu=2, nsplit_cap=32, force_nsplit=0,
                        min_chunk_tiles=1):
    """Returns dict(nsplit, chunk_tiles, chunk_keys, n_tiles, grid, direct).

    The defaults are the pages' rule (about two blocks per SM, capped by the
    tile count and 32). min_chunk_tiles > 1 adds a floor on the work per
    split: at most ceil(n_tiles / min_chunk_tiles) splits.
    """
    n_units = B_max * Hkv
    n_tiles = _cdiv(s_max_kv, block_n)
    if force_nsplit > 0:
        nsplit = min(force_nsplit, n_tiles)
    else:
        want = _cdiv(target_blocks_per_cu * n_cu, n_units)
        nsplit = max(1, min(want, n_tiles, nsplit_cap, _cdiv(n_tiles, min_chunk_tiles)))
    chunk_tiles = _cdiv(n_tiles, nsplit)
    nsplit = _cdiv(n_tiles, chunk_tiles)
    return dict(nsplit=nsplit, chunk_tiles=chunk_tiles,
                chunk_keys=chunk_tiles * block_n, n_tiles=n_tiles,
                grid=n_units * nsplit, direct=(nsplit == 1))


def choose_prefill_grid(B_max, s_max_q, Hkv, q_tokens_per_tile):
    n_qtiles = _cdiv(s_max_q, q_tokens_per_tile)
    return dict(n_qtiles=n_qtiles, grid=B_max * n_qtiles * Hkv)
