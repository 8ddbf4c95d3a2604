"""Scalar pure-Python attention (tiny inputs only) — TEST INFRASTRUCTURE ONLY.

Written without NumPy vector ops, one score at a time, straight from the
textbook definition of scaled-dot-product attention; used to pin
oracle.attention on tiny inputs. Same conventions as oracle.attention:
GQA head h reads KV head h // G, bottom-right causal alignment, empty visible
set -> O = 0, LSE = -inf, cu entries beyond B are never read.
"""
from __future__ import annotations

import math


def attend_scalar(q, k, v, cu_q, cu_kv, B, causal):
    """q, k, v: nested lists [T][H][D] of floats. Returns {(row, h): (O, lse)}."""
    Hq = len(q[0]) if q else 0
    Hkv = len(k[0]) if k else 1
    D = len(q[0][0]) if q else 0
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    res = {}
    for b in range(B):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_kv[b]), int(cu_kv[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        for i in range(Lq):
            for h in range(Hq):
                hk = h // G
                scores = []
                for j in range(Lk):
                    if causal and j > i + (Lk - Lq):
                        continue
                    dot = 0.0
                    for d in range(D):
                        dot += q[q0 + i][h][d] * k[k0 + j][hk][d]
                    scores.append((j, scale * dot))
                if not scores:
                    res[(q0 + i, h)] = ([0.0] * D, -math.inf)
                    continue
                mx = max(s for _, s in scores)
                den = 0.0
                num = [0.0] * D
                for j, s in scores:
                    e = math.exp(s - mx)
                    den += e
                    for d in range(D):
                        num[d] += e * v[k0 + j][hk][d]
                res[(q0 + i, h)] = ([x / den for x in num], mx + math.log(den))
    return res
