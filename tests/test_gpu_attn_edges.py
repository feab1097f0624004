"""Edge cases of ws_block_causal_attn on the GPU: special values, ragged
sizes, partial visibility of the cache, empty inputs and error paths."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import gen as G
from tests.gpu_common import assert_close, dev_bits, host_bits, need_gpu, poisoned_cache

pytestmark = pytest.mark.gpu


def _bits(rng, shape, scale=1.0):
    return G.bf16_rne_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def _cache_with(ck, cv, extra=17):
    from cached_block_causal_amd import kv_append
    h, n, d = ck.shape
    cache = poisoned_cache(h, d, n + extra)
    if n:
        kv_append(cache, dev_bits(ck), dev_bits(cv), layout="head")
    return cache


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_splits", [0, 1, 3])
def test_single_visible_key_returns_v_bit_exact(d, n_splits):
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    rng = np.random.default_rng(d)
    ck, cv = _bits(rng, (3, 70, d)), _bits(rng, (3, 70, d))
    q = _bits(rng, (3, 5, d))
    cache = _cache_with(ck, cv)
    out = host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=[0, 5], unit_kend=[1],
                                      n_splits=n_splits))
    assert np.array_equal(out, np.broadcast_to(cv[:, :1], out.shape))


@pytest.mark.parametrize("d", [64, 128])
def test_identical_keys_give_mean_of_values(d):
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    rng = np.random.default_rng(1)
    row = _bits(rng, (d,))
    ck = np.broadcast_to(row, (2, 300, d)).copy()
    cv = _bits(rng, (2, 300, d))
    q = _bits(rng, (2, 40, d))
    cache = _cache_with(ck, cv)
    out = host_bits(block_causal_attn(cache, dev_bits(q)))
    want = np.broadcast_to(O.bf16_to_f64(cv).mean(axis=1, keepdims=True), (2, 40, d))
    assert_close(out, want, "identical keys")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", ["rising", "falling", "spike"])
@pytest.mark.parametrize("n_splits", [1, 3])
@pytest.mark.parametrize("nq", [40, 4])
def test_running_max_moves_across_tiles(d, shape, n_splits, nq):
    """Scores built along one direction: rising by about 10 log2 units per
    64-key tile (more than the running max may lag, so the output, the
    denominator and the score offset are rescaled at every tile or every
    other 32-key tile), falling (the first tile holds the max), or flat with
    one spike in a middle tile; plus random noise. 40 queries run the main
    kernel, 4 the narrow one. Every output against the oracle."""
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    rng = np.random.default_rng(d + len(shape))
    n, heads = 640, 2
    j = np.arange(n, dtype=np.float32)
    if shape == "rising":
        b = 0.01 * j * np.sqrt(128 / d)
    elif shape == "falling":
        b = 0.01 * (n - 1 - j) * np.sqrt(128 / d)
    else:
        b = np.where(j == 333, 4.0, 0.0).astype(np.float32)
    base = np.ones(d, np.float32)
    k = b[None, :, None] * base[None, None, :] + 0.05 * rng.standard_normal((heads, n, d)).astype(np.float32)
    ck = G.bf16_rne_bits(k.astype(np.float32))
    cv = _bits(rng, (heads, n, d))
    q = G.bf16_rne_bits((np.ones((heads, nq, d), np.float32)
                         + 0.05 * rng.standard_normal((heads, nq, d)).astype(np.float32)))
    cache = _cache_with(ck, cv)
    out = host_bits(block_causal_attn(cache, dev_bits(q), n_splits=n_splits))
    want = O.attention(q, ck, cv, np.zeros(nq), np.zeros(n), 1 / np.sqrt(d))
    assert_close(out, want, f"{shape} D {d} splits {n_splits} queries {nq}")


RAGGED = [
    # (d, heads, n_q, n_cache, n_self)
    (64, 3, 1, 1, 0),
    (64, 2, 31, 63, 5),
    (128, 2, 33, 65, 0),
    (128, 3, 32, 97, 3),     # the largest call of the narrow kernel
    (64, 2, 32, 130, 0),
    (128, 1, 129, 0, 200),
    (64, 5, 300, 500, 77),
    (128, 3, 257, 1000, 129),
]


@pytest.mark.parametrize("case", RAGGED, ids=[str(c) for c in RAGGED])
def test_ragged_streaming_sizes(case):
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    d, h, nq, nc, ns = case
    rng = np.random.default_rng(nq * 7 + nc)
    ck, cv = _bits(rng, (h, nc, d)), _bits(rng, (h, nc, d))
    q = _bits(rng, (h, nq, d))
    sk, sv = _bits(rng, (h, ns, d)), _bits(rng, (h, ns, d))
    cache = _cache_with(ck, cv)
    out = torch.full((h, nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    block_causal_attn(cache, dev_bits(q), dev_bits(sk) if ns else None,
                      dev_bits(sv) if ns else None, out=out)
    k = np.concatenate([ck, sk], axis=1)
    v = np.concatenate([cv, sv], axis=1)
    want = O.attention(q, k, v, np.zeros(nq), np.zeros(nc + ns), 1 / np.sqrt(d))
    assert_close(host_bits(out), want, str(case))


def test_units_seeing_part_of_the_cache():
    """Several query units whose visible ranges end inside the cache, inside
    the own tokens, and mid-tile, with an empty unit in between."""
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    rng = np.random.default_rng(5)
    d, h, nc, ns = 128, 2, 400, 90
    ck, cv = _bits(rng, (h, nc, d)), _bits(rng, (h, nc, d))
    sk, sv = _bits(rng, (h, ns, d)), _bits(rng, (h, ns, d))
    qb = [0, 70, 70, 200, 333]
    kend = [130, 250, 401, 490]
    q = _bits(rng, (h, qb[-1], d))
    cache = _cache_with(ck, cv)
    for n_splits in (0, 1, 5):
        out = host_bits(block_causal_attn(cache, dev_bits(q), dev_bits(sk), dev_bits(sv),
                                          q_unit_begin=qb, unit_kend=kend, n_splits=n_splits))
        k = np.concatenate([ck, sk], axis=1)
        v = np.concatenate([cv, sv], axis=1)
        # visibility by key index: key j carries unit id = first unit whose kend > j
        key_unit = np.searchsorted(np.array(kend), np.arange(nc + ns), side="right")
        q_unit = np.concatenate([np.full(qb[u + 1] - qb[u], u) for u in range(len(kend))])
        want = O.attention(q, k, v, q_unit, key_unit, 1 / np.sqrt(d))
        assert_close(out, want, f"partial visibility splits {n_splits}")


@pytest.mark.parametrize("d", [64, 128])
def test_narrow_call_with_units(d):
    """At most 32 queries (the narrow kernel): four units, one of them empty,
    whose visible ranges end inside the cache, mid-tile and inside the own
    tokens; default, one, five and 256 splits."""
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    rng = np.random.default_rng(32 + d)
    h, nc, ns = 3, 333, 41
    ck, cv = _bits(rng, (h, nc, d)), _bits(rng, (h, nc, d))
    sk, sv = _bits(rng, (h, ns, d)), _bits(rng, (h, ns, d))
    qb = [0, 4, 4, 17, 32]
    kend = [100, 250, 333 + 7, 374]
    q = _bits(rng, (h, qb[-1], d))
    cache = _cache_with(ck, cv)
    k = np.concatenate([ck, sk], axis=1)
    v = np.concatenate([cv, sv], axis=1)
    key_unit = np.searchsorted(np.array(kend), np.arange(nc + ns), side="right")
    q_unit = np.concatenate([np.full(qb[u + 1] - qb[u], u) for u in range(len(kend))])
    want = O.attention(q, k, v, q_unit, key_unit, 1 / np.sqrt(d))
    for n_splits in (0, 1, 5, 256):
        out = host_bits(block_causal_attn(cache, dev_bits(q), dev_bits(sk), dev_bits(sv),
                                          q_unit_begin=qb, unit_kend=kend, n_splits=n_splits))
        assert_close(out, want, f"narrow units D {d} splits {n_splits}")


@pytest.mark.parametrize("d", [64, 128])
def test_maximum_units_and_splits(d):
    """The largest unit table (64 units of 1 to 9 keys and 0 to 5 queries,
    so query and key tiles hold many units) and the largest split count
    (256, far more splits than key tiles: most splits are empty and must
    drop out of the merge)."""
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    rng = np.random.default_rng(64 + d)
    h = 2
    unit_keys = rng.integers(1, 10, 64)
    unit_queries = rng.integers(0, 6, 64)
    unit_queries[-1] = max(1, unit_queries[-1])
    nk, nq = int(unit_keys.sum()), int(unit_queries.sum())
    ck, cv = _bits(rng, (h, nk, d)), _bits(rng, (h, nk, d))
    q = _bits(rng, (h, nq, d))
    qb = np.concatenate([[0], np.cumsum(unit_queries)]).tolist()
    kend = np.cumsum(unit_keys).tolist()
    cache = _cache_with(ck, cv)
    ku = np.repeat(np.arange(64), unit_keys)
    qu = np.repeat(np.arange(64), unit_queries)
    want = O.attention(q, ck, cv, qu, ku, 1 / np.sqrt(d))
    for n_splits in (0, 256):
        out = host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=qb, unit_kend=kend,
                                          n_splits=n_splits))
        assert_close(out, want, f"64 units splits {n_splits}")


def test_empty_query_set_is_noop():
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    rng = np.random.default_rng(0)
    cache = _cache_with(_bits(rng, (2, 10, 64)), _bits(rng, (2, 10, 64)))
    q = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    out = block_causal_attn(cache, q)
    assert out.shape == (2, 0, 64)


def test_errors_are_reported_before_launch():
    need_gpu()
    from cached_block_causal_amd import AttnCall, block_causal_attn
    from cached_block_causal_amd._lib import WS_ERR_SHAPE, WS_ERR_WORKSPACE, WsError
    rng = np.random.default_rng(0)
    cache = _cache_with(_bits(rng, (2, 300, 64)), _bits(rng, (2, 300, 64)))
    q = dev_bits(_bits(rng, (2, 50, 64)))
    with pytest.raises(WsError) as e:                       # kend beyond the keys
        block_causal_attn(cache, q, q_unit_begin=[0, 50], unit_kend=[301])
    assert e.value.status == WS_ERR_SHAPE
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(WsError) as e:
        AttnCall(cache, q, n_splits=4, workspace=small).run()
    assert e.value.status == WS_ERR_WORKSPACE


LONG = [
    # (d, heads, n_q, n_cache, n_self, units): long caches outside the seven
    # workloads; the narrow kernel at D = 64 and with a unit table, and the
    # 128-row kernel at D = 64, at the library's default split counts
    (64, 16, 4, 60000, 4, 1),
    (64, 8, 32, 40000, 0, 8),
    (64, 6, 252, 20000, 252, 1),
]


@pytest.mark.parametrize("case", LONG, ids=[str(c) for c in LONG])
def test_long_caches_sampled_heads(case):
    """Every output of two heads (the first and the last) against the oracle."""
    need_gpu()
    from cached_block_causal_amd import attn_default_splits, block_causal_attn
    d, h, nq, nc, ns, units = case
    rng = np.random.default_rng(nc + nq)
    ck, cv = _bits(rng, (h, nc, d)), _bits(rng, (h, nc, d))
    q = _bits(rng, (h, nq, d))
    sk = _bits(rng, (h, ns, d)) if ns else None
    sv = _bits(rng, (h, ns, d)) if ns else None
    cache = _cache_with(ck, cv)
    nk = nc + ns
    if units == 1:
        qb, kend = [0, nq], [nk]
        q_unit, key_unit = np.zeros(nq), np.zeros(nk)
    else:
        # unit u: queries [4u, 4u + 4), keys up to an end spread over the cache
        qb = list(range(0, nq + 1, nq // units))
        kend = [int(nk * (u + 1) / units) - (7 if u + 1 < units else 0) for u in range(units)]
        key_unit = np.searchsorted(np.array(kend), np.arange(nk), side="right")
        q_unit = np.repeat(np.arange(units), nq // units)
    assert attn_default_splits(h, nq, d, nk) > 1
    out = host_bits(block_causal_attn(cache, dev_bits(q), dev_bits(sk) if ns else None,
                                      dev_bits(sv) if ns else None, q_unit_begin=qb,
                                      unit_kend=kend))
    k = np.concatenate([ck, sk], axis=1) if ns else ck
    v = np.concatenate([cv, sv], axis=1) if ns else cv
    for hh in (0, h - 1):
        want = O.attention(q[hh:hh + 1], k[hh:hh + 1], v[hh:hh + 1], q_unit, key_unit,
                           1 / np.sqrt(d))
        assert_close(out[hh:hh + 1], want, f"{case} head {hh}")
