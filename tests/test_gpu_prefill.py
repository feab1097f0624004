"""Multi-unit block-causal attention at scale against the fp64 oracle.

The queries of many units in one call, each unit seeing the cache up to its
own end: the general form of the pages' block-causal attention ("通义实验室
发布 Wan-Streamer v0.2…", section 为什么端到端模型对级联式 AI 智能体构成挑战:
a block may only use what is available when it is produced), here as the
re-encoding of a 64-unit history. The work is a block triangle: the kernel
skips key tiles past a query tile's last visible key and masks only the tiles
on the diagonal, so these tests cover every kind of tile: fully visible,
masked, straddling a unit boundary, and query tiles holding two units.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from workloads import gen as G
from tests.gpu_common import (all_finite_bits, assert_close, dev_bits, fill_history, host_bits,
                              need_gpu, poisoned_cache)

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(300)
def test_history_prefill_full_size_sampled_rows():
    """v02_history_prefill (58,880 queries x 60,928 keys, 10 heads): every
    output finite; on every head, every row of units 0 and 1 and rows sampled
    at unit and query-tile boundaries and at random, equal to the oracle."""
    need_gpu()
    from cached_block_causal_amd import AttnCall
    w = W.V02_PREFILL
    print(f"prefill {w.name} n_q {w.n_q} n_keys {w.n_keys}", flush=True)
    cache = poisoned_cache(w.heads, w.head_dim, w.capacity)
    fill_history(cache, w)
    assert cache.len == w.n_keys
    q = G.prefill_queries(w)
    call = AttnCall(cache, dev_bits(q), q_unit_begin=w.q_unit_begin(), unit_kend=w.unit_kend())
    out = host_bits(call.run())
    assert all_finite_bits(out)
    heads = list(range(w.heads))
    hk, hv = G.history_bits(w, [w.head_begin + h for h in heads])
    ids = G.history_unit_ids(w)
    vt = w.video_tokens
    rng = np.random.default_rng(7)
    edges = [u * vt + d for u in (1, 2, 31, 62, 63) for d in (-1, 0, 1)]
    tiles = [t * 128 + d for t in (7, 8, 229, 459) for d in (-1, 0)]
    rows = sorted(set(list(range(2 * vt)) + edges + tiles + [w.n_q - 1]
                      + list(rng.integers(0, w.n_q, 64))))
    rows = np.array([r for r in rows if 0 <= r < w.n_q])
    want = O.attention(q[heads][:, rows], hk, hv, rows // vt, ids, 1 / np.sqrt(w.head_dim))
    print(assert_close(out[heads][:, rows], want, "prefill sampled rows"), flush=True)


def _ragged_case(head_dim, unit_keys, unit_queries, seed):
    """Cache of units with the given key counts, queries with the given
    counts per unit (zero allowed), drawn from the seeded generator."""
    heads = 3
    n_k, n_q = sum(unit_keys), sum(unit_queries)
    k = G.bf16_heads(seed, G.TAG_CACHE_K, 0, 0, range(heads), n_k, head_dim)
    v = G.bf16_heads(seed, G.TAG_CACHE_V, 0, 0, range(heads), n_k, head_dim)
    q = G.bf16_heads(seed, G.TAG_Q, 0, 0, range(heads), n_q, head_dim)
    ku = np.repeat(np.arange(len(unit_keys)), unit_keys)
    qu = np.repeat(np.arange(len(unit_queries)), unit_queries)
    qb = np.concatenate([[0], np.cumsum(unit_queries)]).tolist()
    kend = np.cumsum(unit_keys).tolist()
    return k, v, q, ku, qu, qb, kend


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("n_splits", [0, 1, 3])
def test_ragged_units_every_output(head_dim, n_splits):
    """Units of 1..300 keys and 0..257 queries, so that query tiles hold up to
    four units, some units have no queries, and key tiles end mid-unit; all
    outputs compared with the oracle."""
    need_gpu()
    from cached_block_causal_amd import block_causal_attn, kv_append
    unit_keys = [7, 130, 1, 300, 64, 65, 2, 190]
    unit_queries = [3, 129, 1, 0, 257, 5, 40, 100]
    k, v, q, ku, qu, qb, kend = _ragged_case(head_dim, unit_keys, unit_queries, 11)
    print(f"ragged units D {head_dim} splits {n_splits}", flush=True)
    cache = poisoned_cache(3, head_dim, k.shape[1] + 17)
    kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    out = host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=qb, unit_kend=kend,
                                      n_splits=n_splits))
    want = O.attention(q, k, v, qu, ku, 1 / np.sqrt(head_dim))
    assert_close(out, want, f"ragged D {head_dim} splits {n_splits}")


def test_prefill_splits_agree_bitwise_per_split_count():
    """Same call twice gives the same bits; different split counts agree
    within the tolerance (they change only the rounding order)."""
    need_gpu()
    from cached_block_causal_amd import block_causal_attn, kv_append
    unit_keys = [952] * 6
    unit_queries = [920] * 6
    k, v, q, ku, qu, qb, kend = _ragged_case(128, unit_keys, unit_queries, 5)
    cache = poisoned_cache(3, 128, k.shape[1])
    kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    runs = {s: host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=qb, unit_kend=kend,
                                           n_splits=s)) for s in (1, 4)}
    again = host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=qb, unit_kend=kend,
                                        n_splits=4))
    assert np.array_equal(runs[4], again)
    want = O.attention(q, k, v, qu, ku, 1 / np.sqrt(128))
    for s, out in runs.items():
        assert_close(out, want, f"6 units splits {s}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("n_splits", [0, 1])
def test_256_units_audio_history_sampled_rows(n_splits):
    """Re-encoding of a 256-unit audio-era history in one call (each unit of
    956 keys; its 4 audio tokens as queries over the cache up to its own
    end): more units than the launch arguments carry, so the unit table goes
    through the workspace. Rows of the first, middle and last units and
    random rows on three heads against the oracle; every output finite."""
    need_gpu()
    from cached_block_causal_amd import block_causal_attn, kv_append
    unit_keys = [956] * 256
    unit_queries = [4] * 256
    k, v, q, ku, qu, qb, kend = _ragged_case(128, unit_keys, unit_queries, 17)
    print(f"256 units: n_q {q.shape[1]} n_keys {k.shape[1]} splits {n_splits}", flush=True)
    cache = poisoned_cache(3, 128, k.shape[1] + 64)
    kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    out = host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=qb, unit_kend=kend,
                                      n_splits=n_splits))
    assert all_finite_bits(out)
    rng = np.random.default_rng(3)
    rows = sorted(set(list(range(8)) + list(range(512, 516)) + list(range(1016, 1024))
                      + list(rng.integers(0, 1024, 24))))
    rows = np.array(rows)
    want = O.attention(q[:, rows], k, v, qu[rows], ku, 1 / np.sqrt(128))
    print(assert_close(out[:, rows], want, f"256 units splits {n_splits}"), flush=True)


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("n_splits", [0, 1, 3])
def test_over_200_ragged_units_every_output(head_dim, n_splits):
    """230 units of 1..40 keys and 0..6 queries (a quarter of them empty):
    more than 64 units with queries, so the table is in device memory and
    rows find their unit by binary search; every output against the oracle.
    A second call with the same queries gathered into 40 units (the rest
    empty) takes the in-argument table."""
    need_gpu()
    from cached_block_causal_amd import block_causal_attn, kv_append
    rng = np.random.default_rng(23)
    unit_keys = rng.integers(1, 41, 230).tolist()
    unit_queries = rng.integers(0, 7, 230)
    unit_queries[rng.random(230) < 0.25] = 0
    unit_queries = unit_queries.tolist()
    k, v, q, ku, qu, qb, kend = _ragged_case(head_dim, unit_keys, unit_queries, 29)
    live = sum(1 for n in unit_queries if n)
    print(f"{len(unit_keys)} units ({live} with queries) n_q {q.shape[1]} n_keys {k.shape[1]} "
          f"D {head_dim} splits {n_splits}", flush=True)
    assert live > 64
    cache = poisoned_cache(3, head_dim, k.shape[1] + 5)
    kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    out = host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=qb, unit_kend=kend,
                                      n_splits=n_splits))
    want = O.attention(q, k, v, qu, ku, 1 / np.sqrt(head_dim))
    assert_close(out, want, f"230 units D {head_dim} splits {n_splits}")
    # the same rows in at most 40 non-empty units: queries move to the last
    # unit whose key end is <= their own, so each row sees fewer keys
    keep = sorted(set(np.linspace(0, 229, 40).astype(int).tolist()))
    unit_of = np.array([max(u for u in keep if u <= x) for x in qu])
    uq2 = [int(np.sum(unit_of == u)) for u in range(230)]
    qb2 = np.concatenate([[0], np.cumsum(uq2)]).tolist()
    out2 = host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=qb2, unit_kend=kend,
                                       n_splits=n_splits))
    want2 = O.attention(q, k, v, unit_of, ku, 1 / np.sqrt(head_dim))
    assert_close(out2, want2, f"40 of 230 units D {head_dim} splits {n_splits}")
