"""Seeded synthetic inputs for tests and benchmarks.

Holds no attention arithmetic: only random lengths, offsets and values. Both
the HIP path and the CPU oracle consume what these functions produce (the
oracle receives the exact bf16 values copied to the host).

Values are fp32 N(0, 1) draws rounded to bf16 (torch's conversion, round to
nearest even); lengths come from numpy's PCG64 seeded with [workload, step];
ranges [lo, hi] are inclusive.
"""
from __future__ import annotations

import numpy as np


def rng(*key):
    return np.random.default_rng(list(key))


def uniform_lengths(n, lo, hi, *key):
    return rng(*key).integers(lo, hi + 1, size=n).astype(np.int64)


def cu_from_lengths(lens, capacity=None, tail=None, start=0):
    """int32 prefix offsets [start, start+l0, ...]; with capacity > len+1 the
    extra entries are filled from `tail` (cycled) to model a buffer sized for
    a larger maximum batch."""
    cu = start + np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))])
    if capacity is not None and capacity > cu.size:
        fill = np.resize(np.asarray(tail if tail is not None else [-1], dtype=np.int64),
                         capacity - cu.size)
        cu = np.concatenate([cu, fill])
    return cu.astype(np.int32)


def normal_bf16(shape, seed, device="cpu"):
    """torch bf16 tensor of N(0,1) draws from a generator seeded on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def bf16_to_f64(t):
    """Exact fp64 numpy copy of a bf16 tensor (any device)."""
    import torch
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


# ---------------------------------------------------------------------------
# Named workloads: shapes and length recipes
# ---------------------------------------------------------------------------

def tiny_decode(seed=0):
    """B=2, Hq=4, Hkv=1, D=64, one query token each, KV lengths U[1, 128]."""
    lens = uniform_lengths(2, 1, 128, 0, seed)
    return dict(name="tiny decode", B=2, B_max=2, Hq=4, Hkv=1, D=64, causal=False,
                q_lens=np.ones(2, np.int64), kv_lens=lens, s_max_q=1, s_max_kv=128)


def long_decode():
    """B=1, Hq=64, Hkv=8, D=128, one query token, KV length 32768."""
    return dict(name="long decode", B=1, B_max=1, Hq=64, Hkv=8, D=128, causal=False,
                q_lens=np.ones(1, np.int64), kv_lens=np.array([32768]), s_max_q=1,
                s_max_kv=32768)


def batched_decode_step(step):
    """B=64, Hq=32, Hkv=8, D=128, plan s_max_kv=8192; step t draws KV lengths
    U[128, 8192]."""
    lens = uniform_lengths(64, 128, 8192, 2, step)
    return dict(name="continuous-batching decode", B=64, B_max=64, Hq=32, Hkv=8, D=128,
                causal=False, q_lens=np.ones(64, np.int64), kv_lens=lens, s_max_q=1,
                s_max_kv=8192)


def varlen_prefill(seed=0):
    """B=16, causal, q_len = kv_len U[64, 4096], Hq=32, Hkv=8, D=128, s_max 4096."""
    lens = uniform_lengths(16, 64, 4096, 3, seed)
    return dict(name="causal varlen prefill", B=16, B_max=16, Hq=32, Hkv=8, D=128, causal=True,
                q_lens=lens, kv_lens=lens, s_max_q=4096, s_max_kv=4096)


def edge_sweep_lengths(D):
    """33 KV lengths: 0, 1, 2, tile multiples +-1 up to 4096, 16383, 16384,
    and 4 draws from U[0, 16384], shuffled."""
    base = [0, 1, 2]
    for k in (16, 32, 64, 128, 256, 512, 1024, 4096):
        base += [k - 1, k, k + 1]
    base += [16383, 16384]
    r = rng(4, D)
    base += list(r.integers(0, 16385, size=4))
    lens = np.array(base, dtype=np.int64)
    r.shuffle(lens)
    return lens


def edge_sweep(D):
    """B=33 of B_max=64, Hq=128, Hkv=8 (G=16), one query token, lengths up to
    16384; cu buffers hold 65 entries with adversarial trailing values."""
    lens = edge_sweep_lengths(D)
    return dict(name=f"edge sweep D={D}", B=33, B_max=64, Hq=128, Hkv=8, D=D, causal=False,
                q_lens=np.ones(33, np.int64), kv_lens=lens, s_max_q=1, s_max_kv=16384,
                cu_capacity=65, cu_tail=[-1, 2**31 - 1, 0])


def materialise(w, seed, device):
    """Device tensors for a workload dict: q, k, v, cu_q, cu_kv (+ sizes)."""
    import torch
    cap = w.get("cu_capacity")
    tail = w.get("cu_tail")
    cu_q = cu_from_lengths(w["q_lens"], cap, tail if tail is None else [tail[0], tail[1], int(np.sum(w["q_lens"]))])
    cu_k = cu_from_lengths(w["kv_lens"], cap, tail if tail is None else [tail[0], tail[1], int(np.sum(w["kv_lens"]))])
    Tq = int(np.sum(w["q_lens"]))
    Tk = int(np.sum(w["kv_lens"]))
    q = normal_bf16((max(Tq, 1), w["Hq"], w["D"]), 3 * seed + 0, device)
    k = normal_bf16((max(Tk, 1), w["Hkv"], w["D"]), 3 * seed + 1, device)
    v = normal_bf16((max(Tk, 1), w["Hkv"], w["D"]), 3 * seed + 2, device)
    return dict(q=q, k=k, v=v,
                cu_q=torch.from_numpy(cu_q).to(device), cu_kv=torch.from_numpy(cu_k).to(device),
                cu_q_np=cu_q, cu_kv_np=cu_k, Tq=Tq, Tk=Tk)
