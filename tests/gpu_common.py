"""Helpers of the GPU parity tests (device <-> host bits, cache building,
tolerance checks). The oracle side never sees a value produced on the GPU."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import gen as G
from workloads.device import dev_bits, host_bits  # noqa: F401

# bf16 quiet NaN used to poison unused cache capacity and guard bands
POISON_BITS = 0x7FC0
# parity bar for attention and Euler outputs: bf16 inputs, fp32 accumulation
MAX_ABS = 2e-2
REL_FRO = 5e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def poisoned_cache(heads, head_dim, capacity):
    from cached_block_causal_amd import KVCache
    c = KVCache(heads, head_dim, capacity)
    c.k.view(torch.int16).fill_(POISON_BITS)
    c.v.view(torch.int16).fill_(POISON_BITS)
    return c


def fill_history(cache, w, slice_heads_all=True):
    """Append the workload's prior units (head-major commits of this GPU's
    heads) and then, for the streaming step, the current unit's slice
    (token-major, all w.heads_total heads, keeping this GPU's block) through
    ws_kv_append."""
    from cached_block_causal_amd import kv_append
    heads = list(range(w.head_begin, w.head_begin + w.heads))
    for u in range(w.cached_units):
        k, v = G.cache_unit_tokens(w, u, heads)
        kv_append(cache, dev_bits(k), dev_bits(v), head_begin=0, layout="head")
    if w.prefill:
        return
    src_heads = range(w.heads_total) if slice_heads_all else heads
    k, v = G.cache_unit_tokens(w, w.current_unit, src_heads, w.slice_tokens)
    kv_append(cache, dev_bits(G.token_major(k)), dev_bits(G.token_major(v)),
              head_begin=w.head_begin if slice_heads_all else 0, layout="token")


def all_finite_bits(bits) -> bool:
    """No bf16 NaN or infinity (exponent field all ones) among the bits."""
    return not np.any((np.asarray(bits, dtype=np.uint16) & 0x7F80) == 0x7F80)


def errors(got_bits: np.ndarray, want: np.ndarray):
    got = O.bf16_to_f64(got_bits)
    diff = got - want
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-300))
    return max_abs, rel


def assert_close(got_bits, want, what=""):
    max_abs, rel = errors(got_bits, want)
    assert np.all(np.isfinite(O.bf16_to_f64(got_bits))), f"{what}: non-finite output"
    assert max_abs <= MAX_ABS and rel <= REL_FRO, f"{what}: max_abs {max_abs:.3e} rel_fro {rel:.3e}"
    return max_abs, rel
