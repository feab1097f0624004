"""ws_block_causal_attn on the GPU against the fp64 oracle, on every workload.

Small workloads are compared on every output element; the full-size video
workloads, the audio workload and the joint call on every output of every
head at one denoise step, and on sampled heads and rows at the later steps
(the oracle computes each head independently).
Unused cache capacity is poisoned with NaN, so any read past the valid rows
would show up as a non-finite output.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from workloads import gen as G
from tests.gpu_common import (assert_close, dev_bits, fill_history, host_bits, need_gpu,
                              poisoned_cache)

pytestmark = pytest.mark.gpu


def _streaming_case(w, steps, heads_sampled=None, rows_sampled=None):
    """Run the streaming step of workload w on the GPU for the given denoise
    steps; compare all heads (heads_sampled None) or the sampled heads, on
    every query row (rows_sampled None) or the sampled rows (rows are
    independent, so the oracle computes just those)."""
    from cached_block_causal_amd import AttnCall
    print(f"attn {w.name} steps {steps} heads {heads_sampled}", flush=True)
    cache = poisoned_cache(w.heads, w.head_dim, w.capacity)
    fill_history(cache, w)
    assert cache.len == w.cache_len
    hist_heads = (list(range(w.head_begin, w.head_begin + w.heads)) if heads_sampled is None
                  else [w.head_begin + h for h in heads_sampled])
    hk, hv = G.history_bits(w, hist_heads)
    ids = G.history_unit_ids(w)
    sel = slice(None) if heads_sampled is None else list(heads_sampled)
    results = []
    for s in steps:
        q, ks, vs, _ = G.step_tensors(w, s)
        call = AttnCall(cache, dev_bits(q), dev_bits(ks), dev_bits(vs))
        out = host_bits(call.run())
        # the two-launch form gives the same bits
        call.out.view(torch.int16).fill_(0x7FC0)
        call.partial()
        call.merge()
        assert np.array_equal(host_bits(call.out), out)
        k, v, ku = O.streaming_keys(hk, hv, w.cache_len, ids, ks[sel], vs[sel], w.current_unit)
        rows = slice(None) if rows_sampled is None else list(rows_sampled)
        qs = q[sel][:, rows]
        want = O.attention(qs, k, v, np.full(qs.shape[1], w.current_unit), ku,
                           1 / np.sqrt(w.head_dim))
        results.append(assert_close(out[sel][:, rows], want, f"{w.name} step {s}"))
    print(results, flush=True)


def test_tiny_streaming_all_steps():
    need_gpu()
    _streaming_case(W.TINY, range(4))


def test_v01_unit_full():
    need_gpu()
    _streaming_case(W.V01_UNIT, [0, 3])


@pytest.mark.timeout(300)
def test_v02_rank_share_every_head():
    """All 10 heads x 920 queries x 61,880 keys of denoise step 0."""
    need_gpu()
    _streaming_case(W.V02_RANK, [0])


@pytest.mark.timeout(600)
def test_v02_whole_performer_every_head():
    """All 40 heads x 920 queries x 61,880 keys of denoise step 0."""
    need_gpu()
    _streaming_case(W.V02_WHOLE, [0])


def _sampled_rows(n_q, n, seed):
    """Seeded rows plus the edges of every 128-row query tile."""
    rng = np.random.default_rng(seed)
    edges = {0, n_q - 1} | {t for t in range(128, n_q, 128)} | {t - 1 for t in range(128, n_q, 128)}
    return sorted(edges | set(rng.choice(n_q, n, replace=False).tolist()))


@pytest.mark.timeout(300)
def test_v02_rank_share_later_steps_sampled_rows():
    """Denoise steps 1-3 (fresh queries and own tokens per step) on sampled
    rows of two heads."""
    need_gpu()
    _streaming_case(W.V02_RANK, [1, 2, 3], heads_sampled=[3, 6],
                    rows_sampled=_sampled_rows(W.V02_RANK.n_q, 64, 1))


@pytest.mark.timeout(300)
def test_v02_whole_performer_later_steps_sampled_rows():
    need_gpu()
    _streaming_case(W.V02_WHOLE, [1, 2, 3], heads_sampled=[7, 30],
                    rows_sampled=_sampled_rows(W.V02_WHOLE.n_q, 64, 2))


@pytest.mark.timeout(600)
def test_audio_long_history_sampled_heads():
    need_gpu()
    _streaming_case(W.AUDIO_LONG, [3], heads_sampled=[0, 5, 10, 13, 20, 27, 33, 39])


@pytest.mark.timeout(600)
def test_audio_long_history_every_head():
    """All 40 heads x 4 queries x 244,772 keys of denoise step 0; the oracle
    takes the heads eight at a time to bound host memory."""
    need_gpu()
    from cached_block_causal_amd import AttnCall
    w = W.AUDIO_LONG
    print(f"attn {w.name} step 0 every head", flush=True)
    cache = poisoned_cache(w.heads, w.head_dim, w.capacity)
    fill_history(cache, w)
    q, ks, vs, _ = G.step_tensors(w, 0)
    out = host_bits(AttnCall(cache, dev_bits(q), dev_bits(ks), dev_bits(vs)).run())
    ids = G.history_unit_ids(w)
    results = []
    for h0 in range(0, w.heads, 8):
        sel = list(range(h0, min(w.heads, h0 + 8)))
        hk, hv = G.history_bits(w, [w.head_begin + h for h in sel])
        k, v, ku = O.streaming_keys(hk, hv, w.cache_len, ids, ks[sel], vs[sel], w.current_unit)
        want = O.attention(q[sel], k, v, np.full(w.n_q, w.current_unit), ku, 1 / np.sqrt(w.head_dim))
        results.append(assert_close(out[sel], want, f"{w.name} heads {sel[0]}-{sel[-1]}"))
    print(results, flush=True)


@pytest.mark.timeout(600)
def test_joint_audio_video_call_every_head():
    """The unit's audio and video queries in one call (audio rows first): on
    every head every row equals the oracle, where the audio rows see the
    cache and the unit's audio tokens and the video rows also the unit's
    video tokens; the audio rows also agree with a call for audio alone."""
    need_gpu()
    from cached_block_causal_amd import AttnCall
    w = W.JOINT_RANK
    print(f"joint {w.name} n_q {w.n_q} n_keys {w.n_keys}", flush=True)
    cache = poisoned_cache(w.heads, w.head_dim, w.capacity)
    fill_history(cache, w)
    assert cache.len == w.cache_len
    q, ks, vs, _ = G.step_tensors(w, 1)
    out = host_bits(AttnCall(cache, dev_bits(q), dev_bits(ks), dev_bits(vs), w.q_unit_begin(),
                             w.unit_kend()).run())
    a = w.audio_tokens
    alone = host_bits(AttnCall(cache, dev_bits(q[:, :a].copy()), dev_bits(ks[:, :a].copy()),
                               dev_bits(vs[:, :a].copy())).run())
    ids = G.history_unit_ids(w)
    u = w.current_unit
    ku = np.concatenate([ids, np.full(a, u), np.full(w.video_tokens, u + 1)])
    qu = np.concatenate([np.full(a, u), np.full(w.video_tokens, u + 1)])
    for h0 in range(0, w.heads, 2):              # every head, two at a time
        sel = [h0, h0 + 1]
        hk, hv = G.history_bits(w, [w.head_begin + h for h in sel])
        k = np.concatenate([O.bf16_to_f64(hk), O.bf16_to_f64(ks[sel])], axis=1)
        v = np.concatenate([O.bf16_to_f64(hv), O.bf16_to_f64(vs[sel])], axis=1)
        want = O.attention(q[sel], k, v, qu, ku, 1 / np.sqrt(w.head_dim))
        print(assert_close(out[sel], want, f"joint call heads {sel}"), flush=True)
        assert_close(alone[sel], want[:, :a], f"audio alone heads {sel}")
        assert_close(out[sel][:, :a], want[:, :a], f"joint audio rows heads {sel}")


def _multi_unit_tiny():
    """The tiny workload in its multi-unit form: all three units' tokens in
    the cache, queries of all three units, unit u seeing units <= u."""
    w = W.TINY
    n_units = w.cached_units + 1
    ks = [G.cache_unit_tokens(w, u, range(w.heads)) for u in range(n_units)]
    ck = np.concatenate([k for k, _ in ks], axis=1)
    cv = np.concatenate([v for _, v in ks], axis=1)
    q = np.concatenate([G.step_tensors(w, 0, unit=u)[0] for u in range(n_units)], axis=1)
    ku = np.repeat(np.arange(n_units), w.unit_tokens)
    qu = np.repeat(np.arange(n_units), w.video_tokens)
    qb = [w.video_tokens * u for u in range(n_units + 1)]
    kend = [w.unit_tokens * (u + 1) for u in range(n_units)]
    return w, ck, cv, q, ku, qu, qb, kend


def _run_multi(w, ck, cv, q, qb, kend, n_splits=0):
    from cached_block_causal_amd import block_causal_attn, kv_append
    cache = poisoned_cache(w.heads, w.head_dim, ck.shape[1] + 40)
    kv_append(cache, dev_bits(ck), dev_bits(cv), layout="head")
    return host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=qb, unit_kend=kend,
                                       n_splits=n_splits))


@pytest.mark.parametrize("n_splits", [0, 1, 4])
def test_tiny_multi_unit_block_causal(n_splits):
    need_gpu()
    w, ck, cv, q, ku, qu, qb, kend = _multi_unit_tiny()
    out = _run_multi(w, ck, cv, q, qb, kend, n_splits)
    want = O.attention(q, ck, cv, qu, ku, 1 / np.sqrt(w.head_dim))
    assert_close(out, want, f"multi-unit splits {n_splits}")


def test_later_unit_changes_leave_earlier_outputs_bit_identical():
    need_gpu()
    w, ck, cv, q, ku, qu, qb, kend = _multi_unit_tiny()
    base = _run_multi(w, ck, cv, q, qb, kend)
    ck2, cv2 = ck.copy(), cv.copy()
    late = ku == 2
    big = G.bf16_rne_bits(np.where(np.arange(w.head_dim) % 2 == 0, 1e4, -1e4).astype(np.float32))
    ck2[:, late] = big
    cv2[:, late] = G.bf16_rne_bits(np.array([123.0], np.float32))[0]
    pert = _run_multi(w, ck2, cv2, q, qb, kend)
    early = qu < 2
    assert np.array_equal(base[:, early], pert[:, early])
    assert not np.array_equal(base[:, ~early], pert[:, ~early])


@pytest.mark.parametrize("n_splits", [1, 2, 7, 33])
def test_split_counts_agree_with_oracle(n_splits):
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    w = W.V01_UNIT
    cache = poisoned_cache(w.heads, w.head_dim, w.capacity)
    fill_history(cache, w)
    q, ks, vs, _ = G.step_tensors(w, 1)
    out = host_bits(block_causal_attn(cache, dev_bits(q), dev_bits(ks), dev_bits(vs),
                                      n_splits=n_splits))
    hk, hv = G.history_bits(w, [0, 23])
    k, v, ku = O.streaming_keys(hk, hv, w.cache_len, G.history_unit_ids(w), ks[[0, 23]],
                                vs[[0, 23]], w.current_unit)
    want = O.attention(q[[0, 23]], k, v, np.full(w.n_q, w.current_unit), ku, 1 / np.sqrt(128))
    assert_close(out[[0, 23]], want, f"splits {n_splits}")


def test_repeated_runs_are_bit_identical():
    need_gpu()
    from cached_block_causal_amd import block_causal_attn
    w = W.V01_UNIT
    cache = poisoned_cache(w.heads, w.head_dim, w.capacity)
    fill_history(cache, w)
    q, ks, vs, _ = G.step_tensors(w, 2)
    a = host_bits(block_causal_attn(cache, dev_bits(q), dev_bits(ks), dev_bits(vs)))
    b = host_bits(block_causal_attn(cache, dev_bits(q), dev_bits(ks), dev_bits(vs)))
    assert np.array_equal(a, b)
