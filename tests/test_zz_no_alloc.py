"""The allocation-free attention entry point (ws_block_causal_attn_noalloc)
against the workspace entry point (ws_block_causal_attn), through the C ABI.

The no-alloc call keeps its split partials and unit table in a scratch array
the library holds per GPU; at the same split count both entry points run the
same kernels on the same inputs, so their outputs agree bit for bit. Two and
three calls in a row (the later ones smaller, with another head_dim, and with
a unit table past the launch arguments) check that the shared scratch
carries nothing over from one call to the next. Oversized explicit split
counts are refused on the host before any GPU work.
"""
import ctypes

import numpy as np
import pytest

from workloads import gen as G
from tests.gpu_common import MAX_ABS, REL_FRO, dev_bits, host_bits, need_gpu, poisoned_cache

FAKE = 0x7F0000000000


def _case(heads, head_dim, unit_keys, unit_queries, n_self, seed):
    """A cache of the given units, queries per unit, and own tokens."""
    from cached_block_causal_amd import kv_append
    n_k = sum(unit_keys)
    k = G.bf16_heads(seed, G.TAG_CACHE_K, 0, 0, range(heads), n_k, head_dim)
    v = G.bf16_heads(seed, G.TAG_CACHE_V, 0, 0, range(heads), n_k, head_dim)
    q = G.bf16_heads(seed, G.TAG_Q, 0, 0, range(heads), sum(unit_queries), head_dim)
    ks = G.bf16_heads(seed, G.TAG_SELF_K, 0, 0, range(heads), n_self, head_dim) if n_self else None
    vs = G.bf16_heads(seed, G.TAG_SELF_V, 0, 0, range(heads), n_self, head_dim) if n_self else None
    cache = poisoned_cache(heads, head_dim, n_k + 7)
    kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    qb = np.concatenate([[0], np.cumsum(unit_queries)]).tolist()
    kend = np.cumsum(unit_keys).tolist()
    kend[-1] += n_self          # the last unit also sees the own tokens
    return (cache, dev_bits(q), dev_bits(ks) if n_self else None,
            dev_bits(vs) if n_self else None, qb, kend)


def _both(cache, q, ks, vs, qb, kend, n_splits):
    from cached_block_causal_amd import block_causal_attn, block_causal_attn_noalloc
    ref = host_bits(block_causal_attn(cache, q, ks, vs, q_unit_begin=qb, unit_kend=kend,
                                      n_splits=n_splits))
    got = host_bits(block_causal_attn_noalloc(cache, q, ks, vs, q_unit_begin=qb, unit_kend=kend,
                                              n_splits=n_splits))
    return ref, got


def _close(ref, got, what):
    a = ref.astype(np.uint32) << 16
    b = got.astype(np.uint32) << 16
    fa, fb = a.view(np.float32).astype(np.float64), b.view(np.float32).astype(np.float64)
    assert np.all(np.isfinite(fb)), what
    d = fb - fa
    max_abs = float(np.max(np.abs(d)))
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(fa), 1e-300))
    assert max_abs <= MAX_ABS and rel <= REL_FRO, f"{what}: {max_abs} {rel}"


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_on_consecutive_calls():
    need_gpu()
    import torch
    # call 1: rank-share-like shape (920 queries, 20,920 keys), 4 splits
    c1 = _case(10, 128, [20000], [920], 920, 41)
    print("noalloc call 1: 10 heads D 128 n_q 920 keys 20920 splits 4", flush=True)
    ref, got = _both(*c1, n_splits=4)
    assert np.array_equal(ref, got), "call 1 differs from the workspace entry point"
    # the default split count (lowered to fit the scratch if needed)
    from cached_block_causal_amd import block_causal_attn, block_causal_attn_noalloc
    cache, q, ks, vs, qb, kend = c1
    ref0 = host_bits(block_causal_attn(cache, q, ks, vs, q_unit_begin=qb, unit_kend=kend))
    got0 = host_bits(block_causal_attn_noalloc(cache, q, ks, vs, q_unit_begin=qb, unit_kend=kend))
    _close(ref0, got0, "call 1, default splits")
    # call 2: smaller, head_dim 64, a 72-row tail tile, 3 splits
    c2 = _case(4, 64, [3000], [200], 100, 43)
    print("noalloc call 2: 4 heads D 64 n_q 200 keys 3100 splits 3", flush=True)
    ref, got = _both(*c2, n_splits=3)
    assert np.array_equal(ref, got), "call 2 differs from the workspace entry point"
    # call 3: 90 units with queries (table in the scratch), 2 splits
    rng = np.random.default_rng(5)
    uk = rng.integers(8, 60, 90).tolist()
    uq = rng.integers(1, 5, 90).tolist()
    c3 = _case(3, 128, uk, uq, 0, 47)
    print(f"noalloc call 3: 90 units n_q {sum(uq)} keys {sum(uk)} splits 2", flush=True)
    ref, got = _both(*c3, n_splits=2)
    assert np.array_equal(ref, got), "call 3 differs from the workspace entry point"
    torch.cuda.synchronize()


def test_noalloc_refuses_split_counts_beyond_the_scratch():
    """Host-side: 40 heads x 920 queries at 8 splits needs ~152 MB of
    partials; refused before anything touches a GPU."""
    from cached_block_causal_amd import _lib as L
    lib = L.lib()
    c = L.WsKvCache(FAKE, FAKE + 4096, 40, 128, 61000, 60960)
    qb = (ctypes.c_int32 * 2)(0, 920)
    ke = (ctypes.c_int32 * 1)(60960)
    st = lib.ws_block_causal_attn_noalloc(ctypes.byref(c), FAKE, 920, None, None, 0, 1, qb, ke,
                                          ctypes.c_float(0.088), 8, FAKE, None)
    assert st == L.WS_ERR_WORKSPACE
    assert b"scratch" in lib.ws_last_error()
