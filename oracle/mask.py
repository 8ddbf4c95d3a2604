"""Padding mask from cu_seqlens (oracle) — TEST INFRASTRUCTURE ONLY.

Source: [TE#24] (Description; Changes; Equivalence).

  * Formula form (the page's vectorised construction): for b < B,
    seqlen[b] = cu[b+1] - cu[b]; mask[b, 0, 0, p] = (p >= seqlen[b]) for
    p < max_seqlen; True marks a padded position. Only cu[0..B] is read, so a
    buffer allocated for a larger maximum batch is fine.
  * Loop form (the per-sequence construction the page replaced, kept by it
    as reference-mask code on the test side): row b is
    [False] * seqlen + [True] * (max_seqlen - seqlen). It fails for a length
    above max_seqlen (rows of unequal length), where the formula instead
    yields an all-False row.

Reading for integer width: cu_seqlens is an int32 tensor, so the difference
is taken in int32 (two's-complement wraparound) and then compared with the
positions in a wider type, as tensor type promotion does.
"""
from __future__ import annotations

import numpy as np


def seqlens_int32(cu, B):
    cu = np.asarray(cu, dtype=np.int64)
    d = (cu[1:B + 1] - cu[:B]) & 0xFFFFFFFF
    return np.where(d >= 2**31, d - 2**32, d).astype(np.int64)


def padding_mask(cu, B, max_seqlen):
    """bool [B, 1, 1, max_seqlen]; True = padded position (p >= seqlen)."""
    lens = seqlens_int32(cu, B)
    pos = np.arange(max_seqlen, dtype=np.int64)
    return (pos[None, :] >= lens[:, None]).reshape(B, 1, 1, max_seqlen)


class RaggedRows(ValueError):
    """The loop form cannot build the mask (a length outside [0, max])."""


def padding_mask_loop(cu, B, max_seqlen):
    """Per-sequence list construction; raises RaggedRows where it cannot."""
    rows = []
    for b in range(B):
        n = int(cu[b + 1]) - int(cu[b])
        row = [False] * n + [True] * (max_seqlen - n)
        if len(row) != max_seqlen:
            raise RaggedRows(f"row {b} has {len(row)} entries, not {max_seqlen}")
        rows.append(row)
    return np.array(rows, dtype=bool).reshape(B, 1, 1, max_seqlen)


def cross_padding_masks(cu_q, cu_kv, B, max_q, max_kv):
    """Query-side and key-side padding masks for cross attention."""
    return padding_mask(cu_q, B, max_q), padding_mask(cu_kv, B, max_kv)


def self_attention_case_count(max_seqlens=range(1, 9), batches=range(1, 5),
                              buffer_variants=2):
    """Number of cases in the exhaustive self-attention comparison: every
    combination of lengths in [0, max_seqlen], for each max and batch, with and
    without a longer cu buffer."""
    return buffer_variants * sum((m + 1) ** b for m in max_seqlens for b in batches)


def cross_attention_case_count(max_q=range(1, 6), max_kv=range(1, 6),
                               batches=range(1, 4)):
    """Number of cases in the exhaustive cross-attention comparison: every
    combination of q and kv lengths for each (max_q, max_kv, batch)."""
    return sum(((mq + 1) * (mk + 1)) ** b
               for mq in max_q for mk in max_kv for b in batches)
