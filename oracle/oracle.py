"""fp64 CPU oracle of the cached block-causal denoising step.

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
bench's CPU-baseline leg may import or run this module. The HIP library never
calls it, and it shares no code, constant or helper with the HIP path: it reads
bf16 bit patterns and float32 arrays and computes in float64 with NumPy.

What it computes, and where the pages state it (pages cited by title and
section; the pages print no formula, so each definition below is the plain
reading of the passage, written out):

* Cache append -- "Wan-Streamer v0.2：更高分辨率，相同延迟" (paper.rainbus.top
  structured summary), prerequisites, "K/V缓存预分片", and "方法步骤详情"; the
  English technical summary (gist.science), Methodology, "The Performer", K/V
  handling. A performer rank holds a cache that was split ahead of time; when a
  new K/V slice arrives it writes its own part of the slice straight into its
  local cache positions and nothing else moves. Reading: the rank's part is a
  contiguous block of heads (Ulysses head sharding) and the cache keeps the full
  history of those heads; the write is a bit copy.

* Block-causal attention -- "通义实验室发布 Wan-Streamer v0.2…" (remio.ai),
  section "为什么端到端模型对级联式 AI 智能体构成挑战": every streaming block may
  only use information already available when it is produced, so nothing
  depends on later frames. Reading: a query of unit u sees every key whose unit
  is <= u, and attention inside a unit is bidirectional. Softmax attention is
  the textbook definition: o_i = sum_j p_ij v_j with p_ij = exp(s_ij - m_i) /
  sum_j' exp(s_ij' - m_i) over visible keys, s_ij = scale * <q_i, k_j>.

* Flow-matching Euler update -- the structured summary, "核心方法" and
  "Thinker-Performer架构": the performer generates the next unit's latent by
  flow matching. Reading: one explicit Euler step x <- x + dt * v per denoise
  step, x held in float32, v in bf16.

Parity pins for every function live in tests/test_oracle_pins.py (brute force,
closed forms, library special cases and invariants); none is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

TOKEN_MAJOR = 0   # slice layout [n_tok][src_heads][D]
HEAD_MAJOR = 1    # slice layout [src_heads][n_tok][D]


# --------------------------------------------------------------- bf16 decode

def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: the 16 bits are the top half of an
    IEEE binary32 word whose low half is zero."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# -------------------------------------------------------------- cache append

def kv_append(cache_k, cache_v, length, k_src, v_src, head_begin, layout=TOKEN_MAJOR):
    """Write this rank's heads of one K/V slice into its local cache
    ("Wan-Streamer v0.2：更高分辨率，相同延迟" (structured summary), 前置知识
    K/V缓存预分片 and 方法步骤详情: the rank writes its part of the slice straight
    into its pre-split cache positions).

    cache_k, cache_v: uint16 bf16 bits [Hr][capacity][D] (not modified).
    k_src, v_src: uint16 bits, [n][H][D] (TOKEN_MAJOR) or [H][n][D] (HEAD_MAJOR).
    Rows [length, length + n) of heads [0, Hr) receive source heads
    [head_begin, head_begin + Hr); every other slot keeps its bits.
    Returns (new_k, new_v, length + n).
    """
    cache_k = np.asarray(cache_k, dtype=np.uint16)
    cache_v = np.asarray(cache_v, dtype=np.uint16)
    k_src = np.asarray(k_src, dtype=np.uint16)
    v_src = np.asarray(v_src, dtype=np.uint16)
    hr, cap, d = cache_k.shape
    if layout == TOKEN_MAJOR:
        n, h_src, d_src = k_src.shape
        part_k = k_src[:, head_begin:head_begin + hr, :].transpose(1, 0, 2)
        part_v = v_src[:, head_begin:head_begin + hr, :].transpose(1, 0, 2)
    elif layout == HEAD_MAJOR:
        h_src, n, d_src = k_src.shape
        part_k = k_src[head_begin:head_begin + hr]
        part_v = v_src[head_begin:head_begin + hr]
    else:
        raise ValueError("unknown slice layout")
    if d_src != d or v_src.shape != k_src.shape:
        raise ValueError("slice shape does not match the cache")
    if head_begin < 0 or head_begin + hr > h_src:
        raise ValueError("head block outside the slice")
    if length < 0 or length + n > cap:
        raise ValueError("append overflows the cache")
    new_k = cache_k.copy()
    new_v = cache_v.copy()
    new_k[:, length:length + n, :] = part_k
    new_v[:, length:length + n, :] = part_v
    return new_k, new_v, length + n


# ---------------------------------------------------- block-causal attention

def visible(q_unit, k_unit) -> np.ndarray:
    """Boolean [Nq][Nk]: key j is visible to query i iff unit(j) <= unit(i)
    ("通义实验室发布 Wan-Streamer v0.2…" (remio.ai), 为什么端到端模型对级联式 AI 智能体构成挑战:
    a block uses only what is available when it is produced)."""
    q_unit = np.asarray(q_unit, dtype=np.int64)
    k_unit = np.asarray(k_unit, dtype=np.int64)
    return k_unit[None, :] <= q_unit[:, None]


def attention_probs_head(q, k, q_unit, k_unit, scale) -> np.ndarray:
    """Softmax weights of one head, float64 [Nq][Nk]; masked entries are 0.
    The textbook softmax over the visible keys of visible().

    q: [Nq][D], k: [Nk][D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    mask = visible(q_unit, k_unit)
    if not np.all(mask.any(axis=1)):
        raise ValueError("a query has no visible key")
    s = float(scale) * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(s - m), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def attention(q, k, v, q_unit, k_unit, scale, row_chunk_elems=1 << 25) -> np.ndarray:
    """Block-causal softmax attention, float64 ("通义实验室发布 Wan-Streamer v0.2…" (remio.ai), 为什么端到端模型对级联式 AI 智能体构成挑战;
    "Wan-Streamer v0.2：更高分辨率，相同延迟" (structured summary), 方法步骤详情: each rank attends with its
    local full-history cache).

    q: [H][Nq][D], k and v: [H][Nk][D] (float64 or bf16 bits as uint16);
    q_unit: [Nq] unit of each query; k_unit: [Nk] unit of each key (taken
    from the order the keys were appended, not from any kernel argument).
    Returns o: [H][Nq][D] float64. Query rows are processed in independent
    chunks only to bound memory; each row is computed exactly as defined.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not np.all(np.isfinite(t)):
            raise ValueError(f"non-finite {name}")
    h, nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != h or k.shape[2] != d:
        raise ValueError("q/k/v shapes disagree")
    q_unit = np.asarray(q_unit, dtype=np.int64)
    k_unit = np.asarray(k_unit, dtype=np.int64)
    if q_unit.shape != (nq,) or k_unit.shape != (k.shape[1],):
        raise ValueError("unit id arrays disagree with q/k")
    out = np.empty((h, nq, d), dtype=np.float64)
    rows = max(1, row_chunk_elems // max(1, k.shape[1]))
    for hh in range(h):
        for r0 in range(0, nq, rows):
            r1 = min(nq, r0 + rows)
            p = attention_probs_head(q[hh, r0:r1], k[hh], q_unit[r0:r1], k_unit, scale)
            out[hh, r0:r1] = p @ v[hh]
    return out


def streaming_keys(cache_k, cache_v, length, cache_unit, k_self, v_self, self_unit):
    """Keys of a denoise step: valid cache rows [0, length) then the unit's own
    tokens, which belong to the unit itself (the cache holds the full history:
    "Wan-Streamer v0.2：更高分辨率，相同延迟" (structured summary), 方法步骤详情).
    Returns (k [H][Nk][D], v, k_unit [Nk]) as float64 / int64."""
    ck = _as_f64(np.asarray(cache_k)[:, :length])
    cv = _as_f64(np.asarray(cache_v)[:, :length])
    cu = np.asarray(cache_unit, dtype=np.int64)[:length]
    if cu.shape[0] != length:
        raise ValueError("construction log shorter than the cache")
    if k_self is None or np.asarray(k_self).shape[1] == 0:
        return ck, cv, cu
    sk = _as_f64(k_self)
    sv = _as_f64(v_self)
    su = np.full(sk.shape[1], int(self_unit), dtype=np.int64)
    return (np.concatenate([ck, sk], axis=1), np.concatenate([cv, sv], axis=1),
            np.concatenate([cu, su]))


# ------------------------------------------------------ flow-matching Euler

def fm_euler_step(x, v_bits, dt) -> np.ndarray:
    """One explicit Euler step x + dt * v in float64 from float32 x and bf16 v
    ("Wan-Streamer v0.2：更高分辨率，相同延迟" (structured summary), 核心方法 and Thinker-Performer架构:
    the performer generates the next unit's latent by flow matching).

    dt * v is exact in float64 (at most 24 + 8 significant bits), so the only
    rounding is that of the sum; the float32 state of the next step is this
    value rounded to nearest-even (fm_euler_state).
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    v64 = bf16_to_f64(v_bits)
    return x64 + np.float64(np.float32(dt)) * v64


def fm_euler_state(x, v_bits, dt) -> np.ndarray:
    """The float32 state after one step: fm_euler_step rounded to float32."""
    return fm_euler_step(x, v_bits, dt).astype(np.float32)


def fm_euler_unit(x0, v_steps, dt) -> np.ndarray:
    """All denoise steps of one unit: x_{s+1} = fp32(x_s + dt * v_s)."""
    x = np.asarray(x0, dtype=np.float32)
    for v in v_steps:
        x = fm_euler_state(x, v, dt)
    return x


# ------------------------------------------------------------------ helpers

def _as_f64(t) -> np.ndarray:
    t = np.asarray(t)
    if t.dtype == np.uint16:
        return bf16_to_f64(t)
    return t.astype(np.float64)
