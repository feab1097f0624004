"""Hand-derived fixtures (tests/golden/): each holds a tiny case whose expected
values follow from the definition the pages state by exact arithmetic (the
derivation is written in the file). The CPU tests pin the oracle to them; the
GPU tests run the same cases through the C ABI, with head_dim padded to 64 by
zeros (which changes no dot product and no copied value)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def bf16_bits(values) -> np.ndarray:
    """bf16 bits of values that bf16 represents exactly (checked)."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "fixture value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def fraction_array(rows) -> np.ndarray:
    return np.array([[float(Fraction(x)) for x in r] for r in rows], dtype=np.float64)


def scale_of(fx) -> float:
    return math.log(3.0) if fx["scale"] == "ln3" else float(fx["scale"])


def pad(a, d, axis=-1, value=0.0):
    a = np.asarray(a, dtype=np.float32)
    widths = [(0, 0)] * a.ndim
    widths[axis] = (0, d - a.shape[axis])
    return np.pad(a, widths, constant_values=value)


def test_fixture_inputs_are_bf16_exact():
    for name in ("attention_two_units.json", "append_head_block.json", "euler_unit.json"):
        fx = load(name)
        for key in ("q", "k", "v", "k_slice", "v_slice", "x0"):
            if key in fx:
                bf16_bits(fx[key])
        assert "citation" in fx and "derivation" in fx


def test_oracle_attention_matches_hand_derived_weights():
    fx = load("attention_two_units.json")
    q = bf16_bits(fx["q"])[None]
    k = bf16_bits(fx["k"])[None]
    v = bf16_bits(fx["v"])[None]
    out = O.attention(q, k, v, fx["q_unit"], fx["k_unit"], scale_of(fx))
    np.testing.assert_allclose(out[0], fraction_array(fx["expected"]), rtol=0, atol=1e-12)


def test_oracle_append_matches_hand_derived_cache():
    fx = load("append_head_block.json")
    hr, cap, d = 2, fx["capacity"], 2
    cache_k = bf16_bits(np.full((hr, cap, d), fx["sentinel"]))
    cache_v = cache_k.copy()
    nk, nv, length = O.kv_append(cache_k, cache_v, fx["length"], bf16_bits(fx["k_slice"]),
                                 bf16_bits(fx["v_slice"]), fx["head_begin"], O.TOKEN_MAJOR)
    assert length == fx["expected_length"]
    assert np.array_equal(nk, bf16_bits(fx["expected_k"]))
    assert np.array_equal(nv, bf16_bits(fx["expected_v"]))


def test_oracle_euler_matches_exact_dyadic_states():
    fx = load("euler_unit.json")
    x = O.fm_euler_unit(np.array(fx["x0"], np.float32), [bf16_bits(v) for v in fx["v"]], fx["dt"])
    assert np.array_equal(x, np.array(fx["expected_x"], np.float32))


# ------------------------------------------------------------------ GPU side

@pytest.mark.gpu
def test_gpu_attention_fixture():
    from tests.gpu_common import assert_close, dev_bits, host_bits, need_gpu
    need_gpu()
    from cached_block_causal_amd import KVCache, block_causal_attn, kv_append
    fx = load("attention_two_units.json")
    d = 64
    q = bf16_bits(pad(fx["q"], d))[None]
    k = bf16_bits(pad(fx["k"], d))[None]
    v = bf16_bits(pad(fx["v"], d))[None]
    cache = KVCache(1, d, 8, fill=float("nan"))
    kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    # units as the C ABI takes them: query rows [0, 1) and [1, 3); unit 0 sees
    # the first 2 keys, unit 1 all 3
    want = pad(fraction_array(fx["expected"]), d).astype(np.float64)[None]
    for n_splits in (0, 1, 2):
        out = host_bits(block_causal_attn(cache, dev_bits(q), q_unit_begin=[0, 1, 3],
                                          unit_kend=[2, 3], scale=scale_of(fx),
                                          n_splits=n_splits))
        assert_close(out, want, f"golden attention splits {n_splits}")


@pytest.mark.gpu
def test_gpu_append_fixture_bit_exact():
    from tests.gpu_common import dev_bits, need_gpu
    need_gpu()
    import torch

    from cached_block_causal_amd import KVCache, kv_append
    fx = load("append_head_block.json")
    d, sentinel = 64, fx["sentinel"]
    cache = KVCache(2, d, fx["capacity"], fill=sentinel)
    # length 1 first: a one-token slice of sentinel rows
    pre = bf16_bits(np.full((1, 2, d), sentinel))
    kv_append(cache, dev_bits(pre), dev_bits(pre), layout="token")
    assert cache.len == fx["length"]
    kv_append(cache, dev_bits(bf16_bits(pad(fx["k_slice"], d))),
              dev_bits(bf16_bits(pad(fx["v_slice"], d))), head_begin=fx["head_begin"],
              layout="token")
    torch.cuda.synchronize()
    assert cache.len == fx["expected_length"]
    for got, key in ((cache.k, "expected_k"), (cache.v, "expected_v")):
        want = pad(fx[key], d)
        want[:, [0, cap_last(fx)], 2:] = sentinel  # untouched rows keep the fill everywhere
        bits = got.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(bits, bf16_bits(want)), key


def cap_last(fx):
    return fx["capacity"] - 1


@pytest.mark.gpu
def test_gpu_euler_fixture_bit_exact():
    from tests.gpu_common import dev_bits, need_gpu
    need_gpu()
    import torch

    from cached_block_causal_amd import fm_euler_step
    fx = load("euler_unit.json")
    x = torch.tensor(fx["x0"], dtype=torch.float32, device="cuda")
    for v in fx["v"]:
        fm_euler_step(x, dev_bits(bf16_bits(v)), fx["dt"])
    assert np.array_equal(x.cpu().numpy(), np.array(fx["expected_x"], np.float32))
