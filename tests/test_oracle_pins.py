"""Pins of the fp64 oracle against facts other than itself.

Each test fixes the oracle to brute force, a closed form, a library special
case or an invariant of the definition, chosen so that a plausible mistake
(a dropped scale, a wrong sign, a transposed operand, '<' for '<=' in the
mask, a wrong head offset, double rounding in the Euler step) fails one.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from tests import brute
from workloads import gen as G


def _rand_bits(rng, shape, scale=1.0):
    return G.bf16_rne_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


# ------------------------------------------------------------------ bf16

def test_bf16_decode_known_patterns():
    pats = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x3FC0: 1.5,
            0x4049: 3.140625, 0x7F80: math.inf, 0xFF80: -math.inf,
            0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127}
    got = O.bf16_to_f64(np.array(list(pats), dtype=np.uint16))
    assert list(got) == list(pats.values())
    assert math.copysign(1.0, O.bf16_to_f64(np.uint16(0x8000))) == -1.0


def test_bf16_decode_matches_field_decoding_exhaustive():
    finite = np.array([b for b in range(1 << 16) if ((b >> 7) & 0xFF) != 0xFF],
                      dtype=np.uint16)
    got = O.bf16_to_f64(finite)
    for i in range(0, len(finite), 97):
        assert got[i] == brute.bf16_value(int(finite[i]))


# ------------------------------------------------------------- attention

def _tiny_case(seed, h=2, d=8, unit_sizes=(5, 3, 6), nq_per_unit=(2, 4, 3)):
    rng = np.random.default_rng(seed)
    nk = sum(unit_sizes)
    k_unit = np.repeat(np.arange(len(unit_sizes)), unit_sizes)
    q_unit = np.repeat(np.arange(len(nq_per_unit)), nq_per_unit)
    q = O.bf16_to_f64(_rand_bits(rng, (h, len(q_unit), d)))
    k = O.bf16_to_f64(_rand_bits(rng, (h, nk, d)))
    v = O.bf16_to_f64(_rand_bits(rng, (h, nk, d)))
    return q, k, v, q_unit, k_unit


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_attention_equals_brute_force(seed):
    q, k, v, qu, ku = _tiny_case(seed)
    scale = [0.35, 1.0, 1 / math.sqrt(8), 2.5][seed]
    got = O.attention(q, k, v, qu, ku, scale)
    want = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(),
                                    qu.tolist(), ku.tolist(), scale))
    assert np.max(np.abs(got - want)) <= 1e-12


def test_attention_brute_force_shuffled_units():
    # keys of different units interleaved: visibility depends on the log, not order
    rng = np.random.default_rng(7)
    h, d, nk, nq = 2, 4, 11, 6
    ku = rng.integers(0, 3, nk)
    qu = np.sort(rng.integers(0, 3, nq))
    qu[-1] = 2
    ku[0] = 0
    q = O.bf16_to_f64(_rand_bits(rng, (h, nq, d)))
    k = O.bf16_to_f64(_rand_bits(rng, (h, nk, d)))
    v = O.bf16_to_f64(_rand_bits(rng, (h, nk, d)))
    got = O.attention(q, k, v, qu, ku, 0.7)
    want = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(),
                                    qu.tolist(), ku.tolist(), 0.7))
    assert np.max(np.abs(got - want)) <= 1e-12


def test_softmax_rows_sum_to_one_and_masked_are_zero():
    q, k, v, qu, ku = _tiny_case(11)
    p = O.attention_probs_head(q[0], k[0], qu, ku, 0.5)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
    mask = ku[None, :] <= qu[:, None]
    assert np.all(p[~mask] == 0.0)
    assert np.all(p[mask] > 0.0)


def test_single_visible_key_returns_v_exactly():
    rng = np.random.default_rng(3)
    d = 16
    k = O.bf16_to_f64(_rand_bits(rng, (1, 4, d)))
    v = O.bf16_to_f64(_rand_bits(rng, (1, 4, d)))
    q = O.bf16_to_f64(_rand_bits(rng, (1, 2, d)))
    ku = np.array([0, 1, 1, 1])
    qu = np.array([0, 0])           # only key 0 is visible
    o = O.attention(q, k, v, qu, ku, 0.25)
    assert np.array_equal(o[0, 0], v[0, 0]) and np.array_equal(o[0, 1], v[0, 0])


def test_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(4)
    d, nk = 8, 9
    row = O.bf16_to_f64(_rand_bits(rng, (d,)))
    k = np.broadcast_to(row, (1, nk, d)).copy()
    v = O.bf16_to_f64(_rand_bits(rng, (1, nk, d)))
    q = O.bf16_to_f64(_rand_bits(rng, (1, 3, d)))
    ku = np.array([0, 0, 0, 1, 1, 2, 2, 2, 2])
    qu = np.array([0, 1, 2])
    o = O.attention(q, k, v, qu, ku, 1.3)
    for i, u in enumerate(qu):
        want = v[0, ku <= u].mean(axis=0)
        assert np.max(np.abs(o[0, i] - want)) <= 1e-14


def test_two_key_closed_form():
    # softmax of two logits is a logistic: o = v2 + sigmoid(s1 - s2) (v1 - v2)
    rng = np.random.default_rng(5)
    d = 12
    q = O.bf16_to_f64(_rand_bits(rng, (1, 1, d)))
    k = O.bf16_to_f64(_rand_bits(rng, (1, 2, d)))
    v = O.bf16_to_f64(_rand_bits(rng, (1, 2, d)))
    scale = 0.6
    s1 = scale * math.fsum(q[0, 0] * k[0, 0])
    s2 = scale * math.fsum(q[0, 0] * k[0, 1])
    sig = 1.0 / (1.0 + math.exp(-(s1 - s2)))
    want = v[0, 1] + sig * (v[0, 0] - v[0, 1])
    o = O.attention(q, k, v, [0], [0, 0], scale)
    assert np.max(np.abs(o[0, 0] - want)) <= 1e-14


def test_later_units_do_not_change_earlier_outputs():
    q, k, v, qu, ku = _tiny_case(21)
    base = O.attention(q, k, v, qu, ku, 0.5)
    k2, v2 = k.copy(), v.copy()
    late = ku == 2
    k2[:, late] = np.where(np.arange(k.shape[2]) % 2 == 0, 1e4, -1e4)
    v2[:, late] = 123.0
    pert = O.attention(q, k2, v2, qu, ku, 0.5)
    early = qu < 2
    assert np.array_equal(base[:, early], pert[:, early])
    assert not np.allclose(base[:, ~early], pert[:, ~early])


def test_streaming_step_equals_sdpa_without_mask():
    rng = np.random.default_rng(8)
    h, d, nq, nk = 3, 16, 7, 40
    q = O.bf16_to_f64(_rand_bits(rng, (h, nq, d)))
    k = O.bf16_to_f64(_rand_bits(rng, (h, nk, d)))
    v = O.bf16_to_f64(_rand_bits(rng, (h, nk, d)))
    scale = 1 / math.sqrt(d)
    got = O.attention(q, k, v, np.full(nq, 5), np.repeat([0, 1, 2, 3, 4, 5], [8, 8, 8, 8, 4, 4]), scale)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()
    assert np.max(np.abs(got - want)) <= 1e-12


def test_multi_unit_equals_sdpa_with_block_causal_mask():
    q, k, v, qu, ku = _tiny_case(9, h=3, d=16, unit_sizes=(6, 6, 6), nq_per_unit=(6, 6, 6))
    scale = 0.21
    got = O.attention(q, k, v, qu, ku, scale)
    mask = torch.from_numpy(ku[None, :] <= qu[:, None])
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=mask, scale=scale).numpy()
    assert np.max(np.abs(got - want)) <= 1e-12


def test_attention_row_chunking_does_not_change_rows():
    q, k, v, qu, ku = _tiny_case(13)
    # chunks only bound memory; BLAS may pick another kernel per chunk shape,
    # so rows agree to rounding order, not bit for bit
    a = O.attention(q, k, v, qu, ku, 0.4)
    b = O.attention(q, k, v, qu, ku, 0.4, row_chunk_elems=1)
    assert np.max(np.abs(a - b)) <= 1e-14


def test_attention_rejects_empty_rows_and_nonfinite():
    q, k, v, qu, ku = _tiny_case(1)
    with pytest.raises(ValueError):
        O.attention(q, k, v, qu - 1, ku, 1.0)      # unit -1 sees nothing
    k2 = k.copy()
    k2[0, 0, 0] = np.nan
    with pytest.raises(ValueError):
        O.attention(q, k2, v, qu, ku, 1.0)


def test_streaming_keys_concatenate_cache_then_self():
    rng = np.random.default_rng(2)
    ck = _rand_bits(rng, (2, 10, 4))
    cv = _rand_bits(rng, (2, 10, 4))
    sk = _rand_bits(rng, (2, 3, 4))
    sv = _rand_bits(rng, (2, 3, 4))
    k, v, ku = O.streaming_keys(ck, cv, 6, [0, 0, 1, 1, 2, 2, 9, 9, 9, 9], sk, sv, 2)
    assert k.shape == (2, 9, 4)
    assert np.array_equal(k[:, :6], O.bf16_to_f64(ck[:, :6]))
    assert np.array_equal(v[:, 6:], O.bf16_to_f64(sv))
    assert list(ku) == [0, 0, 1, 1, 2, 2, 2, 2, 2]


# ---------------------------------------------------------------- append

@pytest.mark.parametrize("token_major", [True, False])
def test_append_equals_brute_force_copy(token_major):
    rng = np.random.default_rng(17)
    hr, cap, d, h_src, n, hb, length = 3, 12, 4, 5, 4, 2, 5
    sentinel = 0x7FC0
    ck = np.full((hr, cap, d), sentinel, dtype=np.uint16)
    cv = np.full((hr, cap, d), sentinel, dtype=np.uint16)
    ck[:, :length] = _rand_bits(rng, (hr, length, d))
    shape = (n, h_src, d) if token_major else (h_src, n, d)
    sk = _rand_bits(rng, shape)
    sv = _rand_bits(rng, shape)
    layout = O.TOKEN_MAJOR if token_major else O.HEAD_MAJOR
    nk, nv, nl = O.kv_append(ck, cv, length, sk, sv, hb, layout)
    wk, wl = brute.append(ck.tolist(), length, sk.tolist(), hb, token_major)
    wv, _ = brute.append(cv.tolist(), length, sv.tolist(), hb, token_major)
    assert nl == wl == length + n
    assert nk.tolist() == wk and nv.tolist() == wv
    assert np.all(nk[:, length + n:] == sentinel)
    assert np.array_equal(nk[:, :length], ck[:, :length])


def test_append_layouts_agree():
    rng = np.random.default_rng(18)
    src = _rand_bits(rng, (6, 4, 8))                     # token-major [n][H][D]
    ck = np.zeros((2, 10, 8), dtype=np.uint16)
    a = O.kv_append(ck, ck, 1, src, src, 1, O.TOKEN_MAJOR)
    b = O.kv_append(ck, ck, 1, src.transpose(1, 0, 2).copy(), src.transpose(1, 0, 2).copy(),
                    1, O.HEAD_MAJOR)
    assert np.array_equal(a[0], b[0]) and a[2] == b[2] == 7
    assert np.array_equal(a[0][1, 1:7], src[:, 2, :])     # cache head 1 = source head 2


def test_append_rejects_overflow_and_bad_heads():
    ck = np.zeros((2, 5, 4), dtype=np.uint16)
    src = np.zeros((3, 2, 4), dtype=np.uint16)
    with pytest.raises(ValueError):
        O.kv_append(ck, ck, 3, src, src, 0)
    with pytest.raises(ValueError):
        O.kv_append(ck, ck, 0, src, src, 1)


# ----------------------------------------------------------------- Euler

def _round_to_f32(fr: Fraction) -> float:
    """Round a rational to the nearest binary32 (ties to even), from the
    definition: pick the binade, scale to a 24-bit significand, round."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                               # subnormal spacing floor
    scaled = a / Fraction(2) ** (e - 23)           # significand in units of the ulp
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * math.ldexp(n, e - 23)


def test_euler_state_is_correctly_rounded_sum():
    rng = np.random.default_rng(23)
    n = 3000
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    v = _rand_bits(rng, (n,), 1.0)
    v[:50] = G.bf16_rne_bits((rng.standard_normal(50) * 2.0 ** 30).astype(np.float32))
    for dt in (0.25, 0.1, -0.37):
        got = O.fm_euler_state(x, v, dt)
        dtf = Fraction(float(np.float32(dt)))
        for i in range(0, n, 7):
            exact = Fraction(float(x[i])) + dtf * Fraction(brute.bf16_value(int(v[i])))
            assert float(got[i]) == _round_to_f32(exact), (i, dt)


def test_euler_closed_forms():
    rng = np.random.default_rng(24)
    x0 = rng.standard_normal(500).astype(np.float32)
    vs = [_rand_bits(rng, (500,)) for _ in range(4)]
    assert np.array_equal(O.fm_euler_unit(x0, vs, 0.0), x0)          # dt = 0
    same = [vs[0]] * 4
    zero = np.zeros(500, dtype=np.float32)
    # from 0, four steps of 1/4 with a constant bf16 v land exactly on v
    assert np.array_equal(O.fm_euler_unit(zero, same, 0.25), O.bf16_to_f64(vs[0]).astype(np.float32))
    x4 = O.fm_euler_unit(x0, vs, 0.25).astype(np.float64)
    lin = x0.astype(np.float64) + 0.25 * sum(O.bf16_to_f64(v) for v in vs)
    assert np.max(np.abs(x4 - lin) / np.maximum(np.abs(lin), 1e-3)) <= 4 * 2.0 ** -24 * 8
