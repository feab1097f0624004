"""A whole streaming unit captured once into a HIP graph and replayed.

The library only enqueues kernels on the caller's stream (it allocates,
clears and synchronises nothing), so a caller may capture a unit (the slice
append, 4 x (attention partial + merge + Euler update), the commit of the
unit's latents) and replay it. Each replay must give the bits of the same
unit run eagerly. The replays are separated by unrelated eager work and
synchronisations, and every replay is checked. The same holds for a unit
built from the one-launch unit-end append and the allocation-free attention
(whose partials live in the library's scratch), and for a call whose unit
table a kernel copies into the workspace or the scratch.
"""
import numpy as np
import pytest
import torch

import workloads as W
from workloads import gen as G
from tests.gpu_common import dev_bits, host_bits, need_gpu, poisoned_cache

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w", [W.V01_UNIT, W.AUDIO_LONG], ids=["v01_unit", "audio_long_history"])
def test_unit_graph_replays_match_eager(w):
    need_gpu()
    from cached_block_causal_amd import AttnCall, fm_euler_step, kv_append
    from tests.gpu_common import fill_history
    print(f"graph {w.name}", flush=True)
    cache = poisoned_cache(w.heads, w.head_dim, w.capacity)
    fill_history(cache, w)                      # history and the current slice
    slice_k, slice_v = G.cache_unit_tokens(w, w.current_unit, range(w.heads_total),
                                           w.slice_tokens)
    slice_k, slice_v = dev_bits(G.token_major(slice_k)), dev_bits(G.token_major(slice_v))
    history_len = cache.len - w.slice_tokens
    steps = [tuple(dev_bits(t) for t in G.step_tensors(w, s)) for s in range(w.steps)]
    calls = [AttnCall(cache, q, ks, vs) for q, ks, vs, _ in steps]   # buffers made before capture
    x0 = torch.from_numpy(G.x0(w)).to("cuda")

    def unit(x):
        cache.rewind(history_len)
        kv_append(cache, slice_k, slice_v, head_begin=w.head_begin)
        for c, (_, _, _, vel) in zip(calls, steps):
            c.partial()
            c.merge()
            fm_euler_step(x, vel, w.dt)
        kv_append(cache, steps[-1][1], steps[-1][2], layout="head")

    # eager: the outputs of every step (the same each unit) and x after each unit
    x_eager = x0.clone()
    want_x = []
    for _ in range(3):
        unit(x_eager)
        torch.cuda.synchronize()
        want_x.append(x_eager.cpu().numpy().copy())
    want_out = [host_bits(c.out) for c in calls]
    # the rows a unit writes (slice, then commit), with 8 untouched rows on
    # either side
    lo, hi = history_len - 8, min(cache.capacity, cache.len + 8)

    def written():
        return (host_bits(cache.k[:, lo:hi].contiguous()), host_bits(cache.v[:, lo:hi].contiguous()))

    want_k, want_v = written()

    x = x0.clone()
    for c in calls:
        c.out.view(torch.int16).fill_(0x7FC0)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            unit(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    junk = torch.arange(1 << 20, device="cuda", dtype=torch.float32)
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        for c, want in zip(calls, want_out):
            assert np.array_equal(host_bits(c.out), want), f"replay {r}: attention output"
        assert np.array_equal(x.cpu().numpy(), want_x[r]), f"replay {r}: latent"
        got_k, got_v = written()
        assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v), \
            f"replay {r}: cache"
        junk.mul_(1.0001).add_(r)              # unrelated eager work between replays
        torch.cuda.synchronize()


def _replay_and_check(fn, check, reps=3):
    """Capture fn() once, then replay it `reps` times with unrelated eager
    work and synchronisations in between, calling check(r) after each."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    junk = torch.arange(1 << 20, device="cuda", dtype=torch.float32)
    for r in range(reps):
        g.replay()
        torch.cuda.synchronize()
        check(r)
        junk.mul_(1.0001).add_(r)
        torch.cuda.synchronize()


def test_noalloc_unit_with_one_launch_unit_end_in_graph():
    """The callers the allocation-free entry point is for: a unit whose end
    (committed latents head-major, then the next slice token-major) is one
    ws_kv_append_segments launch and whose attention runs through
    ws_block_causal_attn_noalloc (partials in the library's scratch), all
    captured once; every replay equals the eager unit bit for bit."""
    need_gpu()
    from cached_block_causal_amd import block_causal_attn_noalloc, fm_euler_step, kv_append_segments
    from tests.gpu_common import fill_history
    w = W.V01_UNIT
    print(f"graph noalloc {w.name}", flush=True)
    cache = poisoned_cache(w.heads, w.head_dim, w.capacity)
    fill_history(cache, w)
    slice_k, slice_v = G.cache_unit_tokens(w, w.current_unit, range(w.heads_total),
                                           w.slice_tokens)
    slice_k, slice_v = dev_bits(G.token_major(slice_k)), dev_bits(G.token_major(slice_v))
    start = cache.len - w.slice_tokens
    steps = [tuple(dev_bits(t) for t in G.step_tensors(w, s)) for s in range(w.steps)]
    commit_k, commit_v = steps[0][1], steps[0][2]            # head-major [H][n][D]
    outs = [torch.empty_like(q) for q, _, _, _ in steps]
    x0 = torch.from_numpy(G.x0(w)).to("cuda")

    def unit(x):
        cache.rewind(start)
        kv_append_segments(cache, [(commit_k, commit_v, "head", 0),
                                   (slice_k, slice_v, "token", w.head_begin)])
        for (q, ks, vs, vel), o in zip(steps, outs):
            block_causal_attn_noalloc(cache, q, ks, vs, out=o)
            fm_euler_step(x, vel, w.dt)

    x_eager = x0.clone()
    want_x = []
    for _ in range(3):
        unit(x_eager)
        torch.cuda.synchronize()
        want_x.append(x_eager.cpu().numpy().copy())
    want_out = [host_bits(o) for o in outs]
    lo, hi = start - 8, min(cache.capacity, cache.len + 8)
    want_k = host_bits(cache.k[:, lo:hi].contiguous())
    want_v = host_bits(cache.v[:, lo:hi].contiguous())
    x = x0.clone()
    for o in outs:
        o.view(torch.int16).fill_(0x7FC0)

    def check(r):
        for o, want in zip(outs, want_out):
            assert np.array_equal(host_bits(o), want), f"replay {r}: attention output"
        assert np.array_equal(x.cpu().numpy(), want_x[r]), f"replay {r}: latent"
        assert np.array_equal(host_bits(cache.k[:, lo:hi].contiguous()), want_k), f"replay {r}: K"
        assert np.array_equal(host_bits(cache.v[:, lo:hi].contiguous()), want_v), f"replay {r}: V"

    _replay_and_check(lambda: unit(x), check)


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_unit_table_upload_in_graph(entry):
    """A call with 90 units holding queries (unit table copied into the
    workspace, or the scratch, by a kernel on the call's stream) captured
    once; every replay equals the eager call bit for bit."""
    need_gpu()
    from cached_block_causal_amd import AttnCall, block_causal_attn_noalloc, kv_append
    rng = np.random.default_rng(13)
    unit_keys = rng.integers(8, 60, 90).tolist()
    unit_queries = rng.integers(1, 5, 90).tolist()
    heads, d = 3, 128
    n_k, n_q = sum(unit_keys), sum(unit_queries)
    print(f"graph unit table {entry}: 90 units n_q {n_q} n_keys {n_k}", flush=True)
    k = G.bf16_heads(53, G.TAG_CACHE_K, 0, 0, range(heads), n_k, d)
    v = G.bf16_heads(53, G.TAG_CACHE_V, 0, 0, range(heads), n_k, d)
    q = dev_bits(G.bf16_heads(53, G.TAG_Q, 0, 0, range(heads), n_q, d))
    cache = poisoned_cache(heads, d, n_k + 3)
    kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    qb = np.concatenate([[0], np.cumsum(unit_queries)]).tolist()
    ke = np.cumsum(unit_keys).tolist()
    out = torch.empty_like(q)
    if entry == "workspace":
        call = AttnCall(cache, q, q_unit_begin=qb, unit_kend=ke, n_splits=2, out=out)

        def fn():
            call.run()
    else:
        def fn():
            block_causal_attn_noalloc(cache, q, q_unit_begin=qb, unit_kend=ke, n_splits=2, out=out)
    fn()
    torch.cuda.synchronize()
    want = host_bits(out)
    out.view(torch.int16).fill_(0x7FC0)

    def check(r):
        assert np.array_equal(host_bits(out), want), f"replay {r}"

    _replay_and_check(fn, check)
