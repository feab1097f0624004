"""ws_kv_append on the GPU against the oracle's bit copy (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from workloads import gen as G
from tests.gpu_common import POISON_BITS, dev_bits, host_bits, need_gpu, poisoned_cache

pytestmark = pytest.mark.gpu


def _poison_np(heads, cap, d):
    return np.full((heads, cap, d), POISON_BITS, dtype=np.uint16)


@pytest.mark.parametrize("w", W.STREAMING, ids=[w.name for w in W.STREAMING])
def test_unit_append_bit_exact(w):
    """The per-unit append of each workload: a full unit (slice + committed
    latents) from an all-heads token-major source, keeping this GPU's block,
    written behind existing rows; everything else keeps its bits."""
    need_gpu()
    from cached_block_causal_amd import kv_append
    print(f"append {w.name}", flush=True)
    d, hr = w.head_dim, w.heads
    n = w.unit_tokens
    start = 37                                   # rows already present
    cap = start + n + 11                         # room after the append
    cache = poisoned_cache(hr, d, cap)
    pre_k, pre_v = G.cache_unit_tokens(w, 999, range(w.head_begin, w.head_begin + hr), start)
    kv_append(cache, dev_bits(pre_k), dev_bits(pre_v), layout="head")
    k, v = G.cache_unit_tokens(w, 5, range(w.heads_total), n)
    ks, vs = G.token_major(k), G.token_major(v)
    kv_append(cache, dev_bits(ks), dev_bits(vs), head_begin=w.head_begin, layout="token")
    torch.cuda.synchronize()
    assert cache.len == start + n
    ek, ev, el = O.kv_append(_poison_np(hr, cap, d), _poison_np(hr, cap, d), 0, pre_k, pre_v, 0,
                             O.HEAD_MAJOR)
    ek, ev, el = O.kv_append(ek, ev, el, ks, vs, w.head_begin, O.TOKEN_MAJOR)
    assert np.array_equal(host_bits(cache.k), ek)
    assert np.array_equal(host_bits(cache.v), ev)


def test_rank_share_head_blocks():
    """Each of the 4 ranks of a 40-head slice receives its own 10 heads."""
    need_gpu()
    from cached_block_causal_amd import kv_append
    w = W.V02_RANK
    k, v = G.cache_unit_tokens(w, 3, range(40), w.slice_tokens)
    ks, vs = G.token_major(k), G.token_major(v)
    for r in range(4):
        cache = poisoned_cache(10, 128, 64)
        kv_append(cache, dev_bits(ks), dev_bits(vs), head_begin=10 * r)
        got = host_bits(cache.k)
        assert np.array_equal(got[:, :32], k[10 * r:10 * r + 10])
        assert np.all(got[:, 32:] == POISON_BITS)
        assert np.array_equal(host_bits(cache.v)[:, :32], v[10 * r:10 * r + 10])


def test_history_by_appends_equals_generator():
    """Building the tiny workload's cache unit by unit gives the construction
    log's contents."""
    need_gpu()
    from tests.gpu_common import fill_history
    w = W.TINY
    cache = poisoned_cache(w.heads, w.head_dim, w.capacity)
    fill_history(cache, w)
    k, v = G.history_bits(w)
    assert cache.len == w.cache_len
    assert np.array_equal(host_bits(cache.k)[:, :w.cache_len], k)
    assert np.array_equal(host_bits(cache.v)[:, :w.cache_len], v)
    assert np.all(host_bits(cache.k)[:, w.cache_len:] == POISON_BITS)


def test_overflow_is_rejected_without_writes():
    need_gpu()
    from cached_block_causal_amd import kv_append
    from cached_block_causal_amd._lib import WS_ERR_CAPACITY, WsError
    cache = poisoned_cache(2, 64, 10)
    src = dev_bits(np.arange(11 * 2 * 64, dtype=np.uint16).reshape(11, 2, 64))
    with pytest.raises(WsError) as e:
        kv_append(cache, src, src)
    assert e.value.status == WS_ERR_CAPACITY
    torch.cuda.synchronize()
    assert cache.len == 0
    assert np.all(host_bits(cache.k) == POISON_BITS)


def test_empty_append_is_noop():
    need_gpu()
    from cached_block_causal_amd import kv_append
    cache = poisoned_cache(2, 128, 4)
    src = dev_bits(np.zeros((0, 2, 128), dtype=np.uint16))
    kv_append(cache, src, src)
    assert cache.len == 0


@pytest.mark.parametrize("w", W.STREAMING, ids=[w.name for w in W.STREAMING])
def test_unit_end_fused_append_bit_exact(w):
    """A unit's end as one launch (ws_kv_append_segments): its committed
    latents (head-major, this GPU's heads) then the next unit's slice
    (token-major, all heads of the slice, keeping this GPU's block), written
    behind existing rows; equal bit for bit to the oracle's two appends in
    that order, everything else untouched."""
    need_gpu()
    from cached_block_causal_amd import kv_append, kv_append_segments
    print(f"fused append {w.name}", flush=True)
    d, hr = w.head_dim, w.heads
    own = range(w.head_begin, w.head_begin + hr)
    n_commit = w.unit_tokens - w.slice_tokens
    start = 29
    cap = start + n_commit + w.slice_tokens + 9
    cache = poisoned_cache(hr, d, cap)
    pre_k, pre_v = G.cache_unit_tokens(w, 998, own, start)
    kv_append(cache, dev_bits(pre_k), dev_bits(pre_v), layout="head")
    ck, cv = G.cache_unit_tokens(w, 6, own, w.unit_tokens)
    ck, cv = np.ascontiguousarray(ck[:, w.slice_tokens:]), np.ascontiguousarray(cv[:, w.slice_tokens:])
    sk, sv = G.cache_unit_tokens(w, 7, range(w.heads_total), w.slice_tokens)
    sk, sv = G.token_major(sk), G.token_major(sv)
    kv_append_segments(cache, [(dev_bits(ck), dev_bits(cv), "head", 0),
                               (dev_bits(sk), dev_bits(sv), "token", w.head_begin)])
    torch.cuda.synchronize()
    assert cache.len == start + n_commit + w.slice_tokens
    ek, ev, el = O.kv_append(_poison_np(hr, cap, d), _poison_np(hr, cap, d), 0, pre_k, pre_v, 0,
                             O.HEAD_MAJOR)
    ek, ev, el = O.kv_append(ek, ev, el, ck, cv, 0, O.HEAD_MAJOR)
    ek, ev, el = O.kv_append(ek, ev, el, sk, sv, w.head_begin, O.TOKEN_MAJOR)
    assert el == cache.len
    assert np.array_equal(host_bits(cache.k), ek)
    assert np.array_equal(host_bits(cache.v), ev)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_four_segments_with_an_empty_one(head_dim):
    """Four segments of mixed layouts and source head ranges, one of them
    empty with NULL buffers: bit-exact against the oracle's appends."""
    need_gpu()
    from cached_block_causal_amd import kv_append_segments
    from cached_block_causal_amd import _lib as L
    rng = np.random.default_rng(head_dim)
    hr, cap = 3, 250
    srcs = [("head", 5, 1, 17), ("token", 4, 1, 1), ("head", 3, 0, 0), ("token", 7, 4, 130)]
    cache = poisoned_cache(hr, head_dim, cap)
    segs, want_k, want_v, length = [], _poison_np(hr, cap, head_dim), _poison_np(hr, cap, head_dim), 0
    for layout, src_heads, hb, n in srcs:
        shape = (src_heads, n, head_dim) if layout == "head" else (n, src_heads, head_dim)
        k = rng.integers(0, 0x7F00, size=shape, dtype=np.uint16)
        v = rng.integers(0, 0x7F00, size=shape, dtype=np.uint16)
        segs.append((dev_bits(k), dev_bits(v), layout, hb))
        want_k, want_v, length = O.kv_append(want_k, want_v, length, k, v, hb,
                                             O.HEAD_MAJOR if layout == "head" else O.TOKEN_MAJOR)
    kv_append_segments(cache, segs)
    torch.cuda.synchronize()
    assert cache.len == length == 148
    assert np.array_equal(host_bits(cache.k), want_k)
    assert np.array_equal(host_bits(cache.v), want_v)
    # too many tokens in total: refused, nothing written
    with pytest.raises(L.WsError) as e:
        kv_append_segments(cache, segs)
    assert e.value.status == L.WS_ERR_CAPACITY
    torch.cuda.synchronize()
    assert cache.len == 148
    assert np.array_equal(host_bits(cache.k), want_k)
