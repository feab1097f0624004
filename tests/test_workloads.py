"""Input generator and workload bookkeeping (CPU)."""
import numpy as np
import pytest
import torch

import workloads as W
from workloads import gen as G


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        # exact ties: halfway between neighbouring bf16 values
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130 * 3], dtype=np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(G.bf16_rne_bits(x), want)
    assert G.bf16_rne_bits(np.array([1 + 2 ** -8], np.float32))[0] == 0x3F80   # tie -> even
    assert G.bf16_rne_bits(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 0x3F82


def test_bf16_rounding_rejects_nonfinite():
    with pytest.raises(ValueError):
        G.bf16_rne_bits(np.array([np.inf], np.float32))


def test_streams_are_deterministic_and_per_head():
    a = G.bf16_heads(0, G.TAG_Q, 3, 1, [0, 1, 2], 7, 8)
    b = G.bf16_heads(0, G.TAG_Q, 3, 1, [2], 7, 8)
    c = G.bf16_heads(0, G.TAG_Q, 3, 1, [0, 1, 2], 7, 8)
    assert np.array_equal(a, c)
    assert np.array_equal(a[2], b[0])           # a head's stream is independent of the others
    assert not np.array_equal(a[0], a[1])
    d = G.bf16_heads(1, G.TAG_Q, 3, 1, [0], 7, 8)
    assert not np.array_equal(a[0], d[0])


def test_workload_key_counts():
    want = {"tiny": 804, "v01_unit": 9372, "v02_rank_share": 61880,
            "v02_whole_performer": 61880, "audio_long_history": 244772,
            "v02_history_prefill": 60928, "joint_rank_share": 245692}
    for w in W.ALL:
        assert w.n_keys == want[w.name]
    assert W.TINY.cache_len == 552 and W.V02_RANK.cache_len == 60960
    assert W.AUDIO_LONG.cache_len == 244768
    assert W.V02_RANK.latent_elems == 920 * 10 * 128


def test_joint_unit_table():
    """Audio rows first: they see the cache and the unit's 4 audio tokens; the
    video rows also see the unit's 920 video tokens. The audio rows and keys
    are the audio workload's own draws (the same streams, first rows)."""
    w = W.JOINT_RANK
    assert w.q_unit_begin() == [0, 4, 924] and w.unit_kend() == [244772, 245692]
    assert w.visible_pairs() == 4 * 244772 + 920 * 245692
    q, ks, _, _ = G.step_tensors(w, 2, heads=[5])
    qa, ksa, _, _ = G.step_tensors(W.AUDIO_LONG, 2, heads=[5])
    assert np.array_equal(q[:, :4], qa) and np.array_equal(ks[:, :4], ksa)
    ids = G.history_unit_ids(w)
    assert np.array_equal(ids, G.history_unit_ids(W.AUDIO_LONG))


def test_prefill_unit_table():
    """The multi-unit form: unit u's 920 queries see the cache up to the end
    of unit u (952 tokens per unit), so the visible pairs are a block
    triangle; the streaming form is one unit seeing every key."""
    w = W.V02_PREFILL
    qb, ke = w.q_unit_begin(), w.unit_kend()
    assert len(qb) == 65 and qb[0] == 0 and qb[-1] == w.n_q == 58880
    assert ke[0] == 952 and ke[-1] == w.n_keys == w.cache_len == 60928
    assert w.visible_pairs() == 920 * 952 * (64 * 65 // 2)
    assert W.V02_RANK.visible_pairs() == 920 * 61880
    assert W.V02_RANK.q_unit_begin() == [0, 920] and W.V02_RANK.unit_kend() == [61880]
    ids = G.history_unit_ids(w)
    assert ids.shape == (60928,) and ids[-1] == 63
    q = G.prefill_queries(w, heads=[3], units=[0, 5])
    assert q.shape == (1, 1840, 128)
    assert np.array_equal(q[:, 920:], G.bf16_heads(w.seed, G.TAG_Q, 5, 0, [3], 920, 128))


def test_history_matches_unit_by_unit_construction():
    w = W.TINY
    k, v = G.history_bits(w)
    ids = G.history_unit_ids(w)
    assert k.shape == (4, w.cache_len, 64) and ids.shape == (w.cache_len,)
    k1, _ = G.cache_unit_tokens(w, 1, range(4))
    assert np.array_equal(k[:, 268:536], k1)
    ks, _ = G.cache_unit_tokens(w, 2, range(4), 16)
    assert np.array_equal(k[:, 536:], ks)
    assert list(np.unique(ids[536:])) == [2] and list(np.unique(ids[268:536])) == [1]


def test_data_scale_applied_before_rounding():
    w = W.TINY
    q, _, _, vel = G.step_tensors(w, 0)
    qf = G.bf16_bits_to_f32(q)
    assert 0.1 < qf.std() < 0.15                 # N(0,1)/8
    assert 0.9 < G.bf16_bits_to_f32(vel).std() < 1.1
