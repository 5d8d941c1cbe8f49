"""Pins of the oracle's FP8 KV cache (reading R19: E4M3 codes with one
float32 scale per KV head for K and one for V) against facts that do not
come from the oracle itself: exact round trips of representable values,
ties-to-even and saturation, a brute-force nearest-value search, the
invariances of attention under the scales, a closed form for a constant V,
and an explicit loop version of a tiny case.  [OV §2.3.2: FP8 in the fastest
configuration; OCP OFP8 E4M3]"""
import math

import numpy as np
import pytest

import oracle



def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]                     # drop the two NaN codes


def _e4m3_value(code: int) -> float:
    """E4M3 value from the bit fields, written out for the pins."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 0:
        return sign * m * 2.0 ** -9                  # subnormal: m/8 * 2^-6
    return sign * (1 + m / 8) * 2.0 ** (e - 7)


def test_quant_round_trip_is_exact_for_representable_values():
    codes = _finite_codes()
    for k, scale in enumerate([1.0, 2.0 ** -7, 2.0 ** 3]):
        vals = np.array([_e4m3_value(int(c)) * scale for c in codes], dtype=np.float32)
        x = np.stack([vals, vals[::-1]], axis=1)[:, :, None]      # [n][Hkv=2][dh=1]
        sc = np.full(2, scale, np.float32)
        got = oracle.kv_quant_fp8(x, sc)
        assert np.array_equal(got[:, 0, 0], codes), k
        assert np.array_equal(got[:, 1, 0], codes[::-1]), k


def test_quant_ties_to_even_and_saturation():
    # 1.0625 lies halfway between 1.0 (code 0x38) and 1.125 (0x39): even code
    # 0x38; 1.1875 between 1.125 (0x39) and 1.25 (0x3A): even 0x3A.
    x = np.array([1.0625, 1.1875, -1.0625, 500.0, -1e6, 448.0, 2.0 ** -10, -(2.0 ** -11)],
                 np.float32)[:, None, None]
    got = oracle.kv_quant_fp8(x, np.ones(1, np.float32))[:, 0, 0]
    assert list(got) == [0x38, 0x3A, 0xB8, 0x7E, 0xFE, 0x7E, 0x00, 0x80]


def test_quant_matches_brute_force_nearest_value():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((40, 3, 8)) * 3).astype(np.float32)
    scale = np.array([0.0123, 0.5, 3.7], np.float32)
    got = oracle.kv_quant_fp8(x, scale)
    table = [(c, _e4m3_value(c)) for c in range(0x7F)]           # non-negative finite
    for idx in np.ndindex(x.shape):
        inv = np.float32(1) / scale[idx[1]]
        y = float(np.float32(x[idx] * inv))
        y = max(-448.0, min(448.0, y))
        a = abs(y)
        best = min(table, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))   # nearest, then even
        want = best[0] | (0x80 if math.copysign(1.0, y) < 0 else 0)
        assert got[idx] == want, (idx, y)


def _case(seed=0, Bq=3, P=11, Hq=4, Hkv=2, dh=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Bq, Hq, dh))
    kc = rng.integers(0, 256, (Hkv, P + Bq, dh)).astype(np.uint8)
    vc = rng.integers(0, 256, (Hkv, P + Bq, dh)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x11                   # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x22
    ks = np.array([0.01, 0.02], np.float32)[:Hkv]
    vs = np.array([0.5, 0.125], np.float32)[:Hkv]
    intra = np.tril(np.ones((Bq, Bq), bool))
    return q, kc, vc, ks, vs, P, intra


def test_k_scale_moves_into_the_queries():
    q, kc, vc, ks, vs, P, intra = _case()
    base = oracle.block_attn_fp8kv(q, kc, vc, ks, vs, P, intra)
    c = 4.0
    q2 = q / c                                       # both KV heads scaled by c
    got = oracle.block_attn_fp8kv(q2, kc, vc, (ks * c).astype(np.float32), vs, P, intra)
    assert np.abs(got - base).max() <= 1e-12 * max(1.0, np.abs(base).max())


def test_v_scale_scales_the_output_of_its_heads_only():
    q, kc, vc, ks, vs, P, intra = _case(seed=1)
    base = oracle.block_attn_fp8kv(q, kc, vc, ks, vs, P, intra)
    vs2 = vs.copy()
    vs2[1] *= 8
    got = oracle.block_attn_fp8kv(q, kc, vc, ks, vs2, P, intra)
    group = q.shape[1] // kc.shape[0]
    assert np.allclose(got[:, :group], base[:, :group], rtol=0, atol=1e-14)
    assert np.allclose(got[:, group:], 8 * base[:, group:], rtol=1e-13, atol=0)


def test_constant_v_gives_its_value():
    q, kc, vc, ks, vs, P, intra = _case(seed=2)
    vc[:] = 0x4C                                     # 1.5 * 2^2 = 6.0 everywhere
    got = oracle.block_attn_fp8kv(q, kc, vc, ks, vs, P, intra)
    group = q.shape[1] // kc.shape[0]
    for g in range(kc.shape[0]):
        assert np.allclose(got[:, g * group:(g + 1) * group], 6.0 * float(vs[g]), rtol=1e-13)


def test_tiny_case_against_explicit_loops():
    q, kc, vc, ks, vs, P, intra = _case(seed=5, Bq=2, P=3, Hq=2, Hkv=1, dh=4)
    got = oracle.block_attn_fp8kv(q, kc, vc, ks, vs, P, intra)
    Bq, Hq, dh = q.shape
    for i in range(Bq):
        for h in range(Hq):
            keys = [j for j in range(P + Bq) if j < P or intra[i, j - P]]
            s = []
            for j in keys:
                dot = sum(q[i, h, d] * _e4m3_value(int(kc[0, j, d])) * float(ks[0])
                          for d in range(dh))
                s.append(dot / math.sqrt(dh))
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            for d in range(dh):
                o = sum(wj * _e4m3_value(int(vc[0, j, d])) * float(vs[0])
                        for wj, j in zip(w, keys)) / sum(w)
                assert abs(got[i, h, d] - o) <= 1e-12 * max(1.0, abs(o))
