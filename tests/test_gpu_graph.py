"""A whole streaming unit captured once into a HIP graph and replayed.

The library only enqueues kernels on the caller's stream (it allocates,
clears and synchronises nothing), so a caller may capture a unit (the slice
append, 4 x (attention partial + merge + Euler update), the commit of the
unit's latents) and replay it. Each replay must give the bits of the same
unit run eagerly. The replays are separated by unrelated eager work and
synchronisations, and every replay is checked.
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
