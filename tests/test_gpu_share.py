"""Properties a multi-GPU deployment relies on, checked on one GPU.

* Rank-share consistency: the whole performer's attention (40 heads) and
  the four rank shares of 10 heads each (what four Ulysses ranks would
  compute, each over its own head-sharded cache built with its head_begin)
  give the same bits head for head, at the same split count: every (head,
  query tile, split) item is computed independently of the others.
* Guard bands: the output and the split workspace are written only inside
  their ranges (poisoned bands before and after them stay untouched), for
  the 128-row and the narrow kernel.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from workloads import gen as G
from tests.gpu_common import (POISON_BITS, assert_close, dev_bits, fill_history, host_bits,
                              need_gpu, poisoned_cache)

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(300)
def test_rank_shares_equal_the_whole_performer_bitwise():
    need_gpu()
    from cached_block_causal_amd import AttnCall
    whole = W.V02_WHOLE
    print("share consistency", flush=True)
    cache = poisoned_cache(whole.heads, whole.head_dim, whole.capacity)
    fill_history(cache, whole)
    q, ks, vs, _ = G.step_tensors(whole, 0)
    splits = 6
    out_whole = host_bits(AttnCall(cache, dev_bits(q), dev_bits(ks), dev_bits(vs),
                                   n_splits=splits).run())
    del cache
    torch.cuda.empty_cache()
    share = W.V02_RANK
    assert whole.heads == 4 * share.heads
    for r in range(4):
        w_r = dataclasses.replace(share, head_begin=share.heads * r)
        c_r = poisoned_cache(w_r.heads, w_r.head_dim, w_r.capacity)
        fill_history(c_r, w_r)                  # this rank's heads of the same history
        hs = slice(share.heads * r, share.heads * (r + 1))
        out_r = host_bits(AttnCall(c_r, dev_bits(np.ascontiguousarray(q[hs])),
                                   dev_bits(np.ascontiguousarray(ks[hs])),
                                   dev_bits(np.ascontiguousarray(vs[hs])),
                                   n_splits=splits).run())
        assert np.array_equal(out_r, out_whole[hs]), f"rank {r}"
        del c_r
        torch.cuda.empty_cache()


def _bits(rng, shape):
    return G.bf16_rne_bits(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("n_q", [300, 7], ids=["128-row kernel", "narrow kernel"])
def test_outputs_and_workspace_stay_inside_their_ranges(n_q):
    need_gpu()
    import oracle as O
    from cached_block_causal_amd import AttnCall, attn_workspace_bytes, kv_append
    rng = np.random.default_rng(n_q)
    h, d, nc, ns = 3, 128, 2000, 11
    ck, cv = _bits(rng, (h, nc, d)), _bits(rng, (h, nc, d))
    sk, sv = _bits(rng, (h, ns, d)), _bits(rng, (h, ns, d))
    q = _bits(rng, (h, n_q, d))
    cache = poisoned_cache(h, d, nc + 64)
    kv_append(cache, dev_bits(ck), dev_bits(cv), layout="head")
    splits = 5
    out_all = torch.full((3, h, n_q, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    out_all.view(torch.int16).fill_(POISON_BITS)
    need = attn_workspace_bytes(h, n_q, d, splits)
    guard = 4096
    ws_all = torch.full((need + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    call = AttnCall(cache, dev_bits(q), dev_bits(sk), dev_bits(sv), n_splits=splits,
                    out=out_all[1], workspace=ws_all[guard:guard + need])
    call.run()
    torch.cuda.synchronize()
    bands = host_bits(out_all)
    assert np.all(bands[0] == POISON_BITS) and np.all(bands[2] == POISON_BITS), "output guard"
    ws = ws_all.cpu().numpy()
    assert np.all(ws[:guard] == 0xA5) and np.all(ws[guard + need:] == 0xA5), "workspace guard"
    k = np.concatenate([ck, sk], axis=1)
    v = np.concatenate([cv, sv], axis=1)
    want = O.attention(q, k, v, np.zeros(n_q), np.zeros(nc + ns), 1 / np.sqrt(d))
    assert_close(bands[1], want, f"guarded call n_q {n_q}")
