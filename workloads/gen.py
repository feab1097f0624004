"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

Every tensor is drawn per head from its own PCG64 stream keyed by
(seed, tensor tag, unit, denoise step, absolute head index), so any subset of
heads can be regenerated without drawing the others. Q/K/V and the velocity
are float32 N(0,1) draws (times the workload's data scale) rounded to bf16
with round-to-nearest-even on the host; the same bf16 bits go to the GPU and
to the oracle. The Euler state x0 is float32 N(0,1).

This module only draws and formats inputs: it holds no step of the method.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Workload

_POOL = None


def _pool() -> ThreadPoolExecutor:
    """Thread pool for per-head draws (NumPy releases the GIL while filling)."""
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL

# tensor tags (part of each stream's key)
TAG_CACHE_K = 1   # cache tokens of a unit (its slice, then its committed latents)
TAG_CACHE_V = 2
TAG_Q = 3         # queries of one denoise step
TAG_SELF_K = 4    # the unit's own latent tokens' keys of one denoise step
TAG_SELF_V = 5
TAG_VEL = 6       # velocity of one denoise step
TAG_X0 = 7        # initial latent (Euler state)
TAG_MISC = 8      # ad-hoc tensors in tests


def stream(seed: int, tag: int, unit: int, step: int, head: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, tag, unit, step, head])))


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    Inputs must be finite (the generators only make finite values)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_rne_bits: non-finite input")
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for display/uploads)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_heads(seed: int, tag: int, unit: int, step: int, heads, n: int, d: int,
                 scale: float = 1.0) -> np.ndarray:
    """float32 N(0,1)*scale, head-major [len(heads)][n][d], one stream per head."""
    heads = list(heads)
    out = np.empty((len(heads), n, d), dtype=np.float32)

    def one(i):
        stream(seed, tag, unit, step, heads[i]).standard_normal(
            (n, d), dtype=np.float32, out=out[i])
        if scale != 1.0:
            out[i] *= np.float32(scale)

    list(_pool().map(one, range(len(heads))))
    return out


def bf16_heads(seed: int, tag: int, unit: int, step: int, heads, n: int, d: int,
               scale: float = 1.0) -> np.ndarray:
    """bf16 bits, head-major [len(heads)][n][d]."""
    heads = list(heads)
    out = np.empty((len(heads), n, d), dtype=np.uint16)

    def one(i):
        x = stream(seed, tag, unit, step, heads[i]).standard_normal((n, d), dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[i] = bf16_rne_bits(x)

    list(_pool().map(one, range(len(heads))))
    return out


# ---------------------------------------------------------------- workloads

def cache_unit_tokens(w: Workload, unit: int, heads, n_tok: int | None = None):
    """K and V bits of the cache tokens of `unit`, head-major [len(heads)][n][D].

    A complete prior unit has w.unit_tokens tokens (its slice, then its
    committed latents); the current unit contributes only its first
    w.slice_tokens tokens (the slice) before attention.
    """
    n = w.unit_tokens if n_tok is None else n_tok
    k = bf16_heads(w.seed, TAG_CACHE_K, unit, 0, heads, n, w.head_dim, w.data_scale)
    v = bf16_heads(w.seed, TAG_CACHE_V, unit, 0, heads, n, w.head_dim, w.data_scale)
    return k, v


def token_major(head_major: np.ndarray) -> np.ndarray:
    """[H][n][D] -> [n][H][D] (the slice layout the thinker broadcasts)."""
    return np.ascontiguousarray(np.transpose(head_major, (1, 0, 2)))


def step_tensors(w: Workload, step: int, heads=None, unit: int | None = None):
    """Inputs of one denoise step for this GPU's heads (head-major bf16 bits):
    q [Hr][Nq][D], k_self/v_self [Hr][Ns][D], velocity [Hr][Nq][D]."""
    if heads is None:
        heads = range(w.head_begin, w.head_begin + w.heads)
    u = w.current_unit if unit is None else unit
    d = w.head_dim
    q = bf16_heads(w.seed, TAG_Q, u, step, heads, w.n_q, d, w.data_scale)
    ks = bf16_heads(w.seed, TAG_SELF_K, u, step, heads, w.n_self, d, w.data_scale)
    vs = bf16_heads(w.seed, TAG_SELF_V, u, step, heads, w.n_self, d, w.data_scale)
    vel = bf16_heads(w.seed, TAG_VEL, u, step, heads, w.n_q, d, 1.0)
    return q, ks, vs, vel


def x0(w: Workload, heads=None) -> np.ndarray:
    """Initial latent share, float32 [Hr][Nq][D]."""
    if heads is None:
        heads = range(w.head_begin, w.head_begin + w.heads)
    return normal_heads(w.seed, TAG_X0, w.current_unit, 0, heads, w.n_q, w.head_dim)


def history_unit_ids(w: Workload) -> np.ndarray:
    """Unit id of every valid cache row at attention time (construction log):
    prior units 0..U-1 in order, then the current unit's slice (unit U)."""
    ids = np.repeat(np.arange(w.cached_units, dtype=np.int64), w.unit_tokens)
    if w.prefill:
        return ids
    return np.concatenate([ids, np.full(w.slice_tokens, w.current_unit, dtype=np.int64)])


def history_bits(w: Workload, heads=None):
    """Full valid cache contents at attention time, head-major bf16 bits
    [Hr][L][D] for K and V, in construction order (as appended)."""
    if heads is None:
        heads = range(w.head_begin, w.head_begin + w.heads)
    heads = list(heads)
    L = w.cache_len
    k = np.empty((len(heads), L, w.head_dim), dtype=np.uint16)
    v = np.empty_like(k)
    pos = 0
    for u in range(w.cached_units):
        ku, vu = cache_unit_tokens(w, u, heads)
        k[:, pos:pos + w.unit_tokens] = ku
        v[:, pos:pos + w.unit_tokens] = vu
        pos += w.unit_tokens
    if not w.prefill:
        ku, vu = cache_unit_tokens(w, w.current_unit, heads, w.slice_tokens)
        k[:, pos:] = ku
        v[:, pos:] = vu
    return k, v


def prefill_queries(w: Workload, heads=None, units=None) -> np.ndarray:
    """Queries of the multi-unit form: the video tokens of every cached unit
    (or of `units`), unit by unit, head-major bf16 bits [len(heads)][n][D]."""
    if heads is None:
        heads = range(w.head_begin, w.head_begin + w.heads)
    units = range(w.cached_units) if units is None else units
    return np.concatenate([bf16_heads(w.seed, TAG_Q, u, 0, heads, w.video_tokens, w.head_dim,
                                      w.data_scale) for u in units], axis=1)
