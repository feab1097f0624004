"""PyTorch-facing binding of libws: argument marshalling only.

Tensors supply device memory and torch's current HIP stream supplies the
stream; every step of the computation runs in the library's gfx950 kernels.
Names follow include/ws.h without the ws_ prefix.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib as L

_BITS16 = (torch.bfloat16, torch.int16, torch.uint16)


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev16(t: torch.Tensor | None, name: str, shape=None) -> ctypes.c_void_p | None:
    if t is None:
        return None
    if t.dtype not in _BITS16:
        raise TypeError(f"{name} must hold bf16 bits (bfloat16/int16), got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


class KVCache:
    """One GPU's pre-allocated, head-major K/V cache bf16[heads][capacity][D]."""

    def __init__(self, heads: int, head_dim: int, capacity: int, device=None,
                 fill: float | None = None):
        dev = torch.device(device) if device is not None else torch.device("cuda")
        self.k = torch.empty((heads, capacity, head_dim), dtype=torch.bfloat16, device=dev)
        self.v = torch.empty_like(self.k)
        if fill is not None:
            self.k.fill_(fill)
            self.v.fill_(fill)
        self._c = L.WsKvCache(self.k.data_ptr(), self.v.data_ptr(), heads, head_dim, capacity, 0)

    @property
    def heads(self) -> int:
        return self._c.heads

    @property
    def head_dim(self) -> int:
        return self._c.head_dim

    @property
    def capacity(self) -> int:
        return self._c.capacity

    @property
    def len(self) -> int:
        return self._c.len

    def rewind(self, length: int) -> None:
        """Forget rows >= length (their bits stay until overwritten)."""
        if not 0 <= length <= self._c.len:
            raise ValueError("rewind length outside [0, len]")
        self._c.len = length

    @property
    def struct(self) -> L.WsKvCache:
        return self._c


def kv_append(cache: KVCache, k_src: torch.Tensor, v_src: torch.Tensor, head_begin: int = 0,
              layout: str = "token") -> None:
    """ws_kv_append: token-major [n][H][D] or head-major [H][n][D] source."""
    if layout not in ("token", "head"):
        raise ValueError("layout must be 'token' or 'head'")
    if k_src.dim() != 3 or k_src.shape != v_src.shape:
        raise ValueError("k_src/v_src must be equal 3-d tensors")
    n, h = (k_src.shape[0], k_src.shape[1]) if layout == "token" else (k_src.shape[1], k_src.shape[0])
    st = L.lib().ws_kv_append(ctypes.byref(cache.struct), _dev16(k_src, "k_src"),
                              _dev16(v_src, "v_src"), n, h, head_begin,
                              L.WS_TOKEN_MAJOR if layout == "token" else L.WS_HEAD_MAJOR,
                              _stream(k_src))
    L.check(st, "ws_kv_append")


def kv_append_segments(cache: KVCache, segments) -> None:
    """ws_kv_append_segments: segments = [(k_src, v_src, layout, head_begin)],
    layout 'token' ([n][H][D]) or 'head' ([H][n][D]); written to consecutive
    rows in one launch."""
    segs = (L.WsKvSegment * max(1, len(segments)))()
    stream = None
    for i, (k_src, v_src, layout, head_begin) in enumerate(segments):
        if layout not in ("token", "head"):
            raise ValueError("layout must be 'token' or 'head'")
        if k_src.dim() != 3 or k_src.shape != v_src.shape:
            raise ValueError("k_src/v_src must be equal 3-d tensors")
        n, h = ((k_src.shape[0], k_src.shape[1]) if layout == "token"
                else (k_src.shape[1], k_src.shape[0]))
        segs[i] = L.WsKvSegment(_dev16(k_src, "k_src").value, _dev16(v_src, "v_src").value, n, h,
                                head_begin, L.WS_TOKEN_MAJOR if layout == "token" else L.WS_HEAD_MAJOR)
        stream = _stream(k_src)
    st = L.lib().ws_kv_append_segments(ctypes.byref(cache.struct), segs, len(segments),
                                       stream if stream is not None else _stream_default())
    L.check(st, "ws_kv_append_segments")


def _stream_default() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def attn_default_splits(heads: int, n_q: int, head_dim: int, n_keys: int) -> int:
    return int(L.lib().ws_attn_default_splits(heads, n_q, head_dim, n_keys))


def attn_workspace_bytes(heads: int, n_q: int, head_dim: int, n_splits: int) -> int:
    return int(L.lib().ws_attn_workspace_bytes(heads, n_q, head_dim, n_splits))


def _units(n_q, n_keys, q_unit_begin, unit_kend):
    if q_unit_begin is None:
        q_unit_begin, unit_kend = [0, n_q], [n_keys]
    n_units = len(unit_kend)
    if len(q_unit_begin) != n_units + 1:
        raise ValueError("q_unit_begin must have len(unit_kend) + 1 entries")
    qb = (ctypes.c_int32 * (n_units + 1))(*[int(x) for x in q_unit_begin])
    ke = (ctypes.c_int32 * n_units)(*[int(x) for x in unit_kend])
    return n_units, qb, ke


class AttnCall:
    """Marshalled arguments of one attention call (shared by the entry points)."""

    def __init__(self, cache: KVCache, q, k_self=None, v_self=None, q_unit_begin=None,
                 unit_kend=None, scale=None, n_splits=0, out=None, workspace=None):
        hr, d = cache.heads, cache.head_dim
        if q.dim() != 3 or q.shape[0] != hr or q.shape[2] != d:
            raise ValueError(f"q must be [{hr}][n_q][{d}]")
        self.n_q = q.shape[1]
        self.n_self = 0 if k_self is None else k_self.shape[1]
        n_keys = cache.len + self.n_self
        self.n_units, self.qb, self.ke = _units(self.n_q, n_keys, q_unit_begin, unit_kend)
        self.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        self.splits = n_splits or attn_default_splits(hr, self.n_q, d, n_keys)
        if out is None:
            out = torch.empty_like(q, dtype=torch.bfloat16)
        need = attn_workspace_bytes(hr, self.n_q, d, self.splits)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        self.cache, self.q, self.k_self, self.v_self = cache, q, k_self, v_self
        self.out, self.workspace = out, workspace
        self.args = (
            ctypes.byref(cache.struct), _dev16(q, "q"), ctypes.c_int32(self.n_q),
            _dev16(k_self, "k_self", (hr, self.n_self, d)) if k_self is not None else None,
            _dev16(v_self, "v_self", (hr, self.n_self, d)) if v_self is not None else None,
            ctypes.c_int32(self.n_self), ctypes.c_int32(self.n_units), self.qb, self.ke,
            ctypes.c_float(self.scale), ctypes.c_int32(self.splits),
            _dev16(out, "out", tuple(q.shape)),
            ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None,
            ctypes.c_size_t(workspace.numel() * workspace.element_size()) if workspace is not None else 0)

    # the stream is torch's current one at each call (so a call made under
    # torch.cuda.stream(...) or inside graph capture lands on that stream)
    def run(self) -> torch.Tensor:
        L.check(L.lib().ws_block_causal_attn(*self.args, _stream(self.q)), "ws_block_causal_attn")
        return self.out

    def partial(self) -> None:
        L.check(L.lib().ws_attn_partial(*self.args, _stream(self.q)), "ws_attn_partial")

    def merge(self) -> torch.Tensor:
        ws = self.workspace
        L.check(L.lib().ws_attn_merge(
            self.cache.heads, self.n_q, self.cache.head_dim, self.splits,
            ctypes.c_void_p(ws.data_ptr()) if ws is not None else None,
            ws.numel() * ws.element_size() if ws is not None else 0,
            ctypes.c_void_p(self.out.data_ptr()), _stream(self.q)), "ws_attn_merge")
        return self.out


def block_causal_attn(cache: KVCache, q, k_self=None, v_self=None, q_unit_begin=None,
                      unit_kend=None, scale=None, n_splits=0, out=None, workspace=None):
    """ws_block_causal_attn; returns out (bf16 [heads][n_q][D])."""
    return AttnCall(cache, q, k_self, v_self, q_unit_begin, unit_kend, scale, n_splits,
                    out, workspace).run()


def block_causal_attn_noalloc(cache: KVCache, q, k_self=None, v_self=None, q_unit_begin=None,
                              unit_kend=None, scale=None, n_splits=0, out=None):
    """ws_block_causal_attn_noalloc: no workspace; the library's per-GPU
    scratch holds the split partials. Returns out."""
    hr, d = cache.heads, cache.head_dim
    if q.dim() != 3 or q.shape[0] != hr or q.shape[2] != d:
        raise ValueError(f"q must be [{hr}][n_q][{d}]")
    n_q = q.shape[1]
    n_self = 0 if k_self is None else k_self.shape[1]
    n_units, qb, ke = _units(n_q, cache.len + n_self, q_unit_begin, unit_kend)
    if out is None:
        out = torch.empty_like(q, dtype=torch.bfloat16)
    st = L.lib().ws_block_causal_attn_noalloc(
        ctypes.byref(cache.struct), _dev16(q, "q"), n_q,
        _dev16(k_self, "k_self", (hr, n_self, d)) if k_self is not None else None,
        _dev16(v_self, "v_self", (hr, n_self, d)) if v_self is not None else None,
        n_self, n_units, qb, ke, ctypes.c_float(1.0 / math.sqrt(d) if scale is None else scale),
        n_splits, _dev16(out, "out", tuple(q.shape)), _stream(q))
    L.check(st, "ws_block_causal_attn_noalloc")
    return out


def fm_euler_step(x: torch.Tensor, v: torch.Tensor, dt: float) -> torch.Tensor:
    """ws_fm_euler_step: x (float32, in place) += dt * v (bf16)."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    if v.numel() != x.numel():
        raise ValueError("v and x differ in size")
    st = L.lib().ws_fm_euler_step(ctypes.c_void_p(x.data_ptr()), _dev16(v, "v"), x.numel(),
                                  ctypes.c_float(dt), _stream(x))
    L.check(st, "ws_fm_euler_step")
    return x
