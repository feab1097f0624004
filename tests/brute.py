"""Pure-Python brute force for tiny shapes (pins the NumPy oracle).

Triple loops over Python floats with math.exp / math.fsum; no NumPy
arithmetic, so a mistake in the oracle's vectorised code cannot hide here.
"""
import math


def bf16_value(bits: int) -> float:
    """Value of a bf16 bit pattern from its fields (sign, exponent, fraction)."""
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:
        return sign * math.ldexp(frac, -126 - 7)
    return sign * math.ldexp(128 + frac, exp - 127 - 7)


def attention(q, k, v, q_unit, k_unit, scale):
    """q: [H][Nq][D], k/v: [H][Nk][D] nested lists of floats."""
    out = []
    for h in range(len(q)):
        rows = []
        for i in range(len(q[h])):
            vis = [j for j in range(len(k[h])) if k_unit[j] <= q_unit[i]]
            s = [scale * math.fsum(q[h][i][d] * k[h][j][d] for d in range(len(q[h][i])))
                 for j in vis]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            rows.append([math.fsum(e[t] * v[h][vis[t]][d] for t in range(len(vis))) / z
                         for d in range(len(v[h][0]))])
        out.append(rows)
    return out


def append(cache, length, src, head_begin, token_major=True):
    """cache: [Hr][cap][D] nested lists of ints (copied); src token-major
    [n][H][D] or head-major [H][n][D]."""
    new = [[list(row) for row in head] for head in cache]
    n = len(src) if token_major else len(src[0])
    for h in range(len(cache)):
        for t in range(n):
            row = src[t][head_begin + h] if token_major else src[head_begin + h][t]
            new[h][length + t] = list(row)
    return new, length + n
