"""Consecutive streaming units with overlapped slice appends (run_units)
against the oracle: each unit's slice lands behind the previous unit's
committed latents, each unit's attention sees exactly the units before it,
its slice and its own tokens, and the two-stream schedule gives the same
bits as one stream."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from workloads import gen as G
from tests.gpu_common import POISON_BITS, assert_close, dev_bits, host_bits, need_gpu

pytestmark = pytest.mark.gpu


def _inputs(w, n_units):
    """Host bits of the units after the workload's history."""
    heads = list(range(w.head_begin, w.head_begin + w.heads))
    units = []
    for i in range(n_units):
        u = w.cached_units + i
        sk, sv = G.cache_unit_tokens(w, u, range(w.heads_total), w.slice_tokens)
        steps = [G.step_tensors(w, s, unit=u) for s in range(w.steps)]
        x0 = G.normal_heads(w.seed, G.TAG_X0, u, 0, heads, w.n_q, w.head_dim)
        units.append((G.token_major(sk), G.token_major(sv), steps, x0))
    return units


def _run(w, units, overlap):
    from cached_block_causal_amd import KVCache, UnitInputs, kv_append, run_units
    heads = list(range(w.head_begin, w.head_begin + w.heads))
    cap = w.history_len + len(units) * w.unit_tokens + 13
    cache = KVCache(w.heads, w.head_dim, cap)
    cache.k.view(torch.int16).fill_(POISON_BITS)
    cache.v.view(torch.int16).fill_(POISON_BITS)
    for u in range(w.cached_units):
        k, v = G.cache_unit_tokens(w, u, heads)
        kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    ins = []
    for sk, sv, steps, x0 in units:
        dsteps = [tuple(dev_bits(t) for t in st) for st in steps]
        outs = [torch.empty((w.heads, w.n_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
                for _ in steps]
        ins.append(UnitInputs(dev_bits(sk), dev_bits(sv), dsteps, torch.from_numpy(x0).to("cuda"),
                              dsteps[-1][1], dsteps[-1][2], w.head_begin, outs))
    run_units(cache, ins, w.dt, overlap=overlap)
    torch.cuda.synchronize()
    return (host_bits(cache.k), host_bits(cache.v), cache.len,
            [[host_bits(o) for o in u.outs] for u in ins], [u.x.cpu().numpy() for u in ins])


@pytest.mark.parametrize("w", [W.TINY, W.V01_UNIT], ids=["tiny", "v01_unit"])
def test_units_against_oracle_and_one_stream(w):
    need_gpu()
    n_units = 3
    print(f"pipeline {w.name} units {n_units}", flush=True)
    units = _inputs(w, n_units)
    ck, cv, length, outs, xs = _run(w, units, overlap=True)
    # the cache: history, then per unit its slice and its committed latents
    heads = list(range(w.head_begin, w.head_begin + w.heads))
    cap = ck.shape[1]
    ek = np.full((w.heads, cap, w.head_dim), POISON_BITS, np.uint16)
    ev = ek.copy()
    el, ids = 0, []
    for u in range(w.cached_units):
        k, v = G.cache_unit_tokens(w, u, heads)
        ek, ev, el = O.kv_append(ek, ev, el, k, v, 0, O.HEAD_MAJOR)
        ids += [u] * k.shape[1]
    scale = 1 / np.sqrt(w.head_dim)
    for i, (sk, sv, steps, x0) in enumerate(units):
        u = w.cached_units + i
        ek, ev, el = O.kv_append(ek, ev, el, sk, sv, w.head_begin, O.TOKEN_MAJOR)
        ids += [u] * sk.shape[0]
        for s, (q, ks, vs, _) in enumerate(steps):
            k, v, ku = O.streaming_keys(ek, ev, el, np.array(ids), ks, vs, u)
            want = O.attention(q, k, v, np.full(w.n_q, u), ku, scale)
            assert_close(outs[i][s], want, f"unit {i} step {s}")
        want_x = O.fm_euler_unit(x0, [st[3] for st in steps], w.dt)
        assert np.array_equal(xs[i], want_x), f"unit {i} Euler state"
        ek, ev, el = O.kv_append(ek, ev, el, steps[-1][1], steps[-1][2], 0, O.HEAD_MAJOR)
        ids += [u] * w.n_self
    assert length == el
    assert np.array_equal(ck, ek) and np.array_equal(cv, ev)
    # one stream: the same bits
    ck1, cv1, length1, outs1, xs1 = _run(w, units, overlap=False)
    assert length1 == length and np.array_equal(ck1, ck) and np.array_equal(cv1, cv)
    for i in range(n_units):
        assert np.array_equal(xs1[i], xs[i])
        for s in range(w.steps):
            assert np.array_equal(outs1[i][s], outs[i][s])


def test_rank_share_two_units_sampled_against_oracle_and_one_stream():
    """The benched shape (v02_rank_share, 10 heads, 920 queries over ~62k keys):
    two consecutive units with the unit-end append beside the last denoise
    step; every step's output on two heads at sampled rows (query-tile edges
    and random rows) against the oracle, the Euler states and the final cache
    bit-exact, and every output bit-identical to the one-stream schedule."""
    need_gpu()
    w = W.V02_RANK
    n_units = 2
    print(f"pipeline {w.name} units {n_units}", flush=True)
    units = _inputs(w, n_units)
    ck, cv, length, outs, xs = _run(w, units, overlap=True)
    sample_heads = [0, 9]
    rng = np.random.default_rng(11)
    rows = np.array(sorted(set([0, 1, 127, 128, 895, 896, 919] + rng.integers(0, w.n_q, 40).tolist())))
    hk, hv = G.history_bits(w, [w.head_begin + h for h in sample_heads])
    ids = list(G.history_unit_ids(w)[:w.history_len])
    ek, ev, el = hk[:, :w.history_len], hv[:, :w.history_len], w.history_len
    scale = 1 / np.sqrt(w.head_dim)
    for i, (sk, sv, steps, x0) in enumerate(units):
        u = w.cached_units + i
        # the slice (this GPU's heads of the all-heads token-major source)
        sl_k = sk[:, [w.head_begin + h for h in sample_heads]].transpose(1, 0, 2)
        sl_v = sv[:, [w.head_begin + h for h in sample_heads]].transpose(1, 0, 2)
        ek, ev = np.concatenate([ek, sl_k], 1), np.concatenate([ev, sl_v], 1)
        el += sk.shape[0]
        ids += [u] * sk.shape[0]
        for s, (q, ks, vs, _) in enumerate(steps):
            k, v, ku = O.streaming_keys(ek, ev, el, np.array(ids), ks[sample_heads],
                                        vs[sample_heads], u)
            want = O.attention(q[sample_heads][:, rows], k, v, np.full(len(rows), u), ku, scale)
            assert_close(outs[i][s][sample_heads][:, rows], want, f"unit {i} step {s}")
        want_x = O.fm_euler_unit(x0, [st[3] for st in steps], w.dt)
        assert np.array_equal(xs[i], want_x), f"unit {i} Euler state"
        ek = np.concatenate([ek, steps[-1][1][sample_heads]], 1)
        ev = np.concatenate([ev, steps[-1][2][sample_heads]], 1)
        el += w.n_self
        ids += [u] * w.n_self
    assert length == w.history_len + n_units * w.unit_tokens
    assert np.array_equal(ck[sample_heads][:, :length], ek)
    assert np.array_equal(cv[sample_heads][:, :length], ev)
    ck1, cv1, length1, outs1, xs1 = _run(w, units, overlap=False)
    assert length1 == length and np.array_equal(ck1, ck) and np.array_equal(cv1, cv)
    for i in range(n_units):
        assert np.array_equal(xs1[i], xs[i])
        for s in range(w.steps):
            assert np.array_equal(outs1[i][s], outs[i][s])
