"""varlen_gqa_attention_amd — varlen grouped-query attention on MI355X (gfx950).

Thin Python binding over the C ABI of libvattn.so (include/vattn.h): it checks
tensor metadata (dtype, shape, contiguity, device) and passes data pointers
and the current HIP stream. Every step of the computation runs in the HIP
kernels; there is no fallback path: the first call into the library raises
ImportError when libvattn.so has not been built.

    plan = Plan(B_max, s_max_q, s_max_kv, Hq, Hkv, D, causal)
    out, lse = plan(q, k, v, cu_seqlens_q, cu_seqlens_kv, B=B)
    mask = padding_mask(cu_seqlens, B, max_seqlen)
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import (DECODE_AUTO, DECODE_MFMA, DECODE_WAVE, ERRBIT_KV_LEN, ERRBIT_Q_LEN,
                   ERRBIT_INDEX, ERRBIT_ROWS, PlanInfo, PlanOpts, VattnError)


class _LazyLib:
    """Loads libvattn.so on first use; raises ImportError if it is missing."""

    def __getattr__(self, name):
        return getattr(_lib.load(), name)


_LIB = _LazyLib()

__all__ = ["Plan", "execute_noalloc", "padding_mask", "cross_padding_masks", "describe_plan", "VattnError", "DECODE_AUTO",
           "DECODE_WAVE", "DECODE_MFMA", "ERRBIT_Q_LEN", "ERRBIT_KV_LEN", "ERRBIT_ROWS",
           "ERRBIT_INDEX"]


# Decode split rules (include/vattn.h, vattn_plan_opts): "pages" is the rule
# the split-K pages state (about two workgroups per CU, no work floor);
# "default" is this library's tuned default (16 per CU at D = 128, scaled by
# 128 / D; 16 tiles per split).
SPLIT_RULES = {"default": dict(target_blocks_per_cu=0, min_chunk_tiles=0),
               "pages": dict(target_blocks_per_cu=2, min_chunk_tiles=1)}


def _opts(target_blocks_per_cu=0, nsplit_cap=0, force_nsplit=0, force_decode_path=0,
          n_cu_override=0, fuse_combine=0, decode_waves=0, prefill_grid=0, backward=0,
          min_chunk_tiles=0, split_rule=None):
    if split_rule is not None:
        if split_rule not in SPLIT_RULES:
            raise ValueError(f"split_rule must be one of {sorted(SPLIT_RULES)}")
        if target_blocks_per_cu or min_chunk_tiles:
            raise ValueError("give split_rule or target_blocks_per_cu / min_chunk_tiles, not both")
        target_blocks_per_cu = SPLIT_RULES[split_rule]["target_blocks_per_cu"]
        min_chunk_tiles = SPLIT_RULES[split_rule]["min_chunk_tiles"]
    return PlanOpts(target_blocks_per_cu, nsplit_cap, force_nsplit, force_decode_path,
                    n_cu_override, fuse_combine, decode_waves, prefill_grid, int(backward),
                    min_chunk_tiles)


def describe_plan(B_max, s_max_q, s_max_kv, Hq, Hkv, D, causal, **opts):
    """Plan the library would build (host only when n_cu_override > 0)."""
    info = PlanInfo()
    o = _opts(**opts)
    _lib.check(_LIB.vattn_plan_describe(B_max, s_max_q, s_max_kv, Hq, Hkv, D, int(causal),
                                        ctypes.byref(o), ctypes.byref(info)), "vattn_plan_describe")
    return info.as_dict()


def _stream_of(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


# Plan handles released while the current stream is capturing a graph. Freeing
# a plan calls hipFree, which a global-mode capture forbids from every thread
# (the capture would be invalidated); a plan dropped there, for instance by a
# garbage-collector pass that runs inside the capture, is freed at the next
# release or plan creation outside a capture instead.
_deferred_handles = []


def _capturing():
    import torch
    try:
        return torch.cuda.is_current_stream_capturing()
    except Exception:
        return False


def _release_deferred():
    while _deferred_handles and not _capturing():
        _LIB.vattn_plan_destroy(_deferred_handles.pop())


def _destroy_handle(h):
    if _capturing():
        _deferred_handles.append(h)
        return
    _LIB.vattn_plan_destroy(h)
    _release_deferred()


class Plan:
    """A plan for up to B_max sequences (see vattn_plan in include/vattn.h)."""

    def __init__(self, B_max, s_max_q, s_max_kv, Hq, Hkv, D, causal=True, **opts):
        self._h = ctypes.c_void_p()
        _release_deferred()
        o = _opts(**opts)
        _lib.check(_LIB.vattn_plan_ex(ctypes.byref(self._h), B_max, s_max_q, s_max_kv, Hq, Hkv,
                                      D, int(causal), ctypes.byref(o)), "vattn_plan")
        info = PlanInfo()
        _lib.check(_LIB.vattn_plan_query(self._h, ctypes.byref(info)), "vattn_plan_query")
        self.info = info.as_dict()
        self.B_max, self.Hq, self.Hkv, self.D = B_max, Hq, Hkv, D

    # -- tensors -----------------------------------------------------------
    def _check(self, q, k, v, cu_q, cu_kv, out, lse, row_strided=False):
        """Metadata checks. With row_strided, q / k / v / out may be views whose
        token dimension has any stride (heads and head dims contiguous)."""
        import torch
        for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                            ("v", v, torch.bfloat16), ("out", out, torch.bfloat16),
                            ("lse", lse, torch.float32), ("cu_seqlens_q", cu_q, torch.int32),
                            ("cu_seqlens_kv", cu_kv, torch.int32)):
            if t.dtype != dt:
                raise TypeError(f"{name} must be {dt}, got {t.dtype}")
            if not t.is_cuda:
                raise ValueError(f"{name} must be a device tensor")
            if row_strided and name in ("q", "k", "v", "out") and t.dim() == 3:
                if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
                    raise ValueError(f"{name}: heads and head dims must be contiguous")
            elif not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if q.dim() != 3 or q.shape[1:] != (self.Hq, self.D):
            raise ValueError(f"q must be [T_q, {self.Hq}, {self.D}], got {tuple(q.shape)}")
        for name, t in (("k", k), ("v", v)):
            if t.dim() != 3 or t.shape[1:] != (self.Hkv, self.D):
                raise ValueError(f"{name} must be [T_kv, {self.Hkv}, {self.D}], got {tuple(t.shape)}")
        if k.shape != v.shape:
            raise ValueError("k and v must have the same shape")
        if out.shape != q.shape or lse.shape != q.shape[:2]:
            raise ValueError("out must match q and lse must be [T_q, Hq]")

    def __call__(self, q, k, v, cu_seqlens_q, cu_seqlens_kv, out=None, lse=None, B=None,
                 stream=None):
        """Enqueue attention for sequences 0..B-1 (B defaults to len(cu_q) - 1)."""
        import torch
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        if B is None:
            B = cu_seqlens_q.numel() - 1
        if cu_seqlens_q.numel() < B + 1 or cu_seqlens_kv.numel() < B + 1:
            raise ValueError("cu_seqlens buffers need at least B + 1 entries")
        self._check(q, k, v, cu_seqlens_q, cu_seqlens_kv, out, lse, row_strided=True)
        if all(t.is_contiguous() for t in (q, k, v, out)):
            _lib.check(_LIB.vattn_execute(self._h, B, _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), _ptr(out),
                                          _ptr(lse), q.shape[0], k.shape[0],
                                          _stream_of(q, stream)), "vattn_execute")
        else:
            # token-row-strided views (e.g. slices of a fused QKV buffer)
            _lib.check(_LIB.vattn_execute_strided(
                self._h, B, _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
                _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), _ptr(out), out.stride(0), _ptr(lse),
                q.shape[0], k.shape[0], _stream_of(q, stream)), "vattn_execute_strided")
        return out, lse

    def gathered(self, q, k, v, cu_seqlens_q, cu_idx, kv_idx, out=None, lse=None, B=None,
                 stream=None):
        """Decode over gathered keys: sequence b attends K/V rows
        kv_idx[cu_idx[b]:cu_idx[b+1]] (int32 device tensors)."""
        import torch
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        if B is None:
            B = cu_seqlens_q.numel() - 1
        if cu_seqlens_q.numel() < B + 1 or cu_idx.numel() < B + 1:
            raise ValueError("cu_seqlens_q and cu_idx need at least B + 1 entries")
        self._check(q, k, v, cu_seqlens_q, cu_idx, out, lse)
        if kv_idx.dtype != torch.int32 or not kv_idx.is_cuda or not kv_idx.is_contiguous():
            raise ValueError("kv_idx must be a contiguous int32 device tensor")
        _lib.check(_LIB.vattn_execute_gathered(
            self._h, B, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_idx),
            _ptr(kv_idx), _ptr(out), _ptr(lse), q.shape[0], k.shape[0], kv_idx.numel(),
            _stream_of(q, stream)), "vattn_execute_gathered")
        return out, lse

    def backward(self, q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_kv, dq=None, dk=None,
                 dv=None, B=None, stream=None):
        """Gradients (dq, dk, dv) of sum(dout * out) for a plan made with
        backward=True; out and lse are this plan's forward results. Tensors
        may be token-row-strided views (heads and head dims contiguous)."""
        import torch
        if dq is None:
            dq = torch.empty_like(q, memory_format=torch.contiguous_format)
        if dk is None:
            dk = torch.empty_like(k, memory_format=torch.contiguous_format)
        if dv is None:
            dv = torch.empty_like(v, memory_format=torch.contiguous_format)
        if B is None:
            B = cu_seqlens_q.numel() - 1
        if cu_seqlens_q.numel() < B + 1 or cu_seqlens_kv.numel() < B + 1:
            raise ValueError("cu_seqlens buffers need at least B + 1 entries")
        self._check(q, k, v, cu_seqlens_q, cu_seqlens_kv, out, lse, row_strided=True)
        for name, t, like in (("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            if t.dtype != torch.bfloat16 or not t.is_cuda or t.shape != like.shape:
                raise ValueError(f"{name} must be a bf16 device tensor shaped like {tuple(like.shape)}")
            if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
                raise ValueError(f"{name}: heads and head dims must be contiguous")
        _lib.check(_LIB.vattn_backward(
            self._h, B, _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
            _ptr(out), out.stride(0), _ptr(dout), dout.stride(0), _ptr(lse),
            _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), _ptr(dq), dq.stride(0), _ptr(dk),
            dk.stride(0), _ptr(dv), dv.stride(0), q.shape[0], k.shape[0],
            _stream_of(q, stream)), "vattn_backward")
        return dq, dk, dv

    def execute_exact_grid(self, q, k, v, cu_seqlens_q, cu_seqlens_kv, tile_map, out, lse, B,
                           stream=None):
        """Prefill over an exact list of live (b << 16 | q_tile) tiles."""
        import torch
        self._check(q, k, v, cu_seqlens_q, cu_seqlens_kv, out, lse)
        if tile_map.dtype != torch.int32 or not tile_map.is_cuda or not tile_map.is_contiguous():
            raise ValueError("tile_map must be a contiguous int32 device tensor")
        _lib.check(_LIB.vattn_execute_exact_grid(
            self._h, B, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv),
            _ptr(out), _ptr(lse), q.shape[0], k.shape[0], _ptr(tile_map), tile_map.numel(),
            _stream_of(q, stream)), "vattn_execute_exact_grid")
        return out, lse

    # -- error word --------------------------------------------------------
    def error_word_ptr(self):
        return _LIB.vattn_plan_error_word(self._h)

    def read_error(self):
        """Synchronising diagnostic read of the device error word."""
        v = ctypes.c_int32()
        _lib.check(_LIB.vattn_plan_read_error(self._h, ctypes.byref(v)), "vattn_plan_read_error")
        return v.value

    def clear_error(self, stream=None):
        import torch
        s = torch.cuda.current_stream() if stream is None else stream
        _lib.check(_LIB.vattn_plan_clear_error(self._h, ctypes.c_void_p(s.cuda_stream)),
                   "vattn_plan_clear_error")

    def set_kernel_events(self, start=None, stop=None):
        """Measurement hook: record the torch.cuda.Event pair `start` / `stop`
        around the plan's main kernel in later eager calls (None, None: off).
        The events must already have been recorded once (torch creates the
        underlying HIP event lazily, on first record)."""
        if (start is None) != (stop is None):
            raise ValueError("give both events or neither")
        hs = [ctypes.c_void_p(e.cuda_event if e is not None else 0) for e in (start, stop)]
        if start is not None and not (hs[0].value and hs[1].value):
            raise ValueError("record each event once before passing it")
        _lib.check(_LIB.vattn_plan_set_kernel_events(self._h, hs[0], hs[1]),
                   "vattn_plan_set_kernel_events")
        self._events = (start, stop)  # keep them alive while the hook is set

    def close(self):
        if self._h:
            _destroy_handle(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def execute_noalloc(B_max, s_max_q, s_max_kv, Hq, Hkv, D, causal, q, k, v, cu_seqlens_q,
                    cu_seqlens_kv, out, lse, B, err_word=None, stream=None):
    """One attention pass with no allocation (vattn_execute_noalloc): the plan
    is chosen per call and its scratch is a static device array shared by
    every call on the GPU. out / lse / err_word (one int32, or None) are
    caller-owned device tensors; inputs are packed and contiguous."""
    import torch
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("out", out, torch.bfloat16),
                        ("lse", lse, torch.float32), ("cu_seqlens_q", cu_seqlens_q, torch.int32),
                        ("cu_seqlens_kv", cu_seqlens_kv, torch.int32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    if q.shape[1:] != (Hq, D) or k.shape[1:] != (Hkv, D) or v.shape != k.shape:
        raise ValueError("q must be [T_q, Hq, D] and k, v [T_kv, Hkv, D]")
    if out.shape != q.shape or lse.shape != q.shape[:2]:
        raise ValueError("out must match q and lse must be [T_q, Hq]")
    if cu_seqlens_q.numel() < B + 1 or cu_seqlens_kv.numel() < B + 1:
        raise ValueError("cu_seqlens buffers need at least B + 1 entries")
    if err_word is not None and (err_word.dtype != torch.int32 or not err_word.is_cuda):
        raise ValueError("err_word must be an int32 device tensor")
    _lib.check(_LIB.vattn_execute_noalloc(
        B_max, s_max_q, s_max_kv, Hq, Hkv, D, int(causal), B, _ptr(q), _ptr(k), _ptr(v),
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), _ptr(out), _ptr(lse), q.shape[0], k.shape[0],
        _ptr(err_word) if err_word is not None else None, _stream_of(q, stream)),
        "vattn_execute_noalloc")
    return out, lse


def cross_padding_masks(cu_seqlens_q, cu_seqlens_kv, B, max_seqlen_q, max_seqlen_kv,
                        out_q=None, out_kv=None, stream=None):
    """(bool [B, 1, 1, max_seqlen_q], bool [B, 1, 1, max_seqlen_kv]): the
    query-side and key-side padding masks of a cross-attention batch."""
    import torch
    for cu in (cu_seqlens_q, cu_seqlens_kv):
        if cu.dtype != torch.int32 or not cu.is_cuda or not cu.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous int32 device tensors")
        if cu.numel() < B + 1:
            raise ValueError("cu_seqlens needs at least B + 1 entries")
    dev = cu_seqlens_q.device
    if out_q is None:
        out_q = torch.empty((B, 1, 1, max_seqlen_q), dtype=torch.bool, device=dev)
    if out_kv is None:
        out_kv = torch.empty((B, 1, 1, max_seqlen_kv), dtype=torch.bool, device=dev)
    for o, n in ((out_q, max_seqlen_q), (out_kv, max_seqlen_kv)):
        if o.dtype != torch.bool or not o.is_contiguous() or o.numel() != B * n:
            raise ValueError("outputs must be contiguous bool tensors of B * max_seqlen elements")
    _lib.check(_LIB.vattn_cross_padding_mask(_ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), B,
                                             max_seqlen_q, max_seqlen_kv, _ptr(out_q),
                                             _ptr(out_kv), _stream_of(cu_seqlens_q, stream)),
               "vattn_cross_padding_mask")
    return out_q, out_kv


def padding_mask(cu_seqlens, B, max_seqlen, out=None, stream=None):
    """bool [B, 1, 1, max_seqlen]: True where position >= cu[b+1] - cu[b]."""
    import torch
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 device tensor")
    if cu_seqlens.numel() < B + 1:
        raise ValueError("cu_seqlens needs at least B + 1 entries")
    if out is None:
        out = torch.empty((B, 1, 1, max_seqlen), dtype=torch.bool, device=cu_seqlens.device)
    if out.dtype != torch.bool or not out.is_contiguous() or out.numel() != B * max_seqlen:
        raise ValueError("out must be a contiguous bool tensor of B * max_seqlen elements")
    _lib.check(_LIB.vattn_padding_mask(_ptr(cu_seqlens), B, max_seqlen, _ptr(out),
                                       _stream_of(cu_seqlens, stream)), "vattn_padding_mask")
    return out
