"""Pins of the oracle's FP8 (W8A8) LM head.

The number format is OCP E4M3 (OFP8 specification): its decoding and its
round-to-nearest-even encoding are pinned to torch's float8_e4m3fn type and to
the format's published constants; the per-row activation quantizer to torch's
float32 arithmetic and to scaling invariants; the W8A8 logits to exact
rational arithmetic on inputs where every quantization step is exact.
[Fast-dVLM overview §2.3.2: FP8 SmoothQuant W8A8]
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
from block_diffusion_vlm_amd import synth
from oracle.guards import lmhead_margins


def torch_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(y32):
    return torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


FINITE = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)


# ---------------------------------------------------------------------------
# E4M3 decode / encode
# ---------------------------------------------------------------------------

def test_decode_matches_library_on_every_code():
    c = np.arange(256, dtype=np.uint8)
    a, b = oracle.e4m3_decode(c), torch_decode(c)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok])
    assert np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))


def test_decode_format_constants():
    d = lambda c: float(oracle.e4m3_decode(np.uint8(c)))  # noqa: E731
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0          # largest finite, S.1111.110
    assert d(0x08) == 2.0 ** -6                            # smallest normal
    assert d(0x07) == 7 * 2.0 ** -9 and d(0x01) == 2.0 ** -9   # subnormals m 2^-9
    assert d(0x38) == 1.0 and d(0x39) == 1.125 and d(0x40) == 2.0
    assert d(0x00) == 0.0 and not np.signbit(d(0x00)) and np.signbit(d(0x80))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))        # S.1111.111, no infinities
    v = oracle.e4m3_decode(np.arange(256))
    assert np.isfinite(v).sum() == 254 and not np.isinf(v).any()
    pos = oracle.e4m3_decode(np.arange(0x7F))
    assert (np.diff(pos) > 0).all()
    assert np.array_equal(oracle.e4m3_decode(np.arange(0x7F) | 0x80), -pos)


def test_encode_round_trips_every_finite_code():
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(FINITE)), FINITE)


def test_encode_matches_library_rounding_including_ties():
    rng = np.random.default_rng(11)
    pos = oracle.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2                       # exact in float32 (5 bits)
    ulp = np.spacing(mids.astype(np.float32))
    y = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000),          # subnormal range
        np.exp2(rng.uniform(-12, 8.8, 20000)) * rng.choice([-1, 1], 20000),
        mids, -mids, mids - ulp, mids + ulp, -(mids + ulp),
        [0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -11, 448.0, -448.0],
    ]).astype(np.float32)
    y = np.clip(y, -448, 448)
    assert np.array_equal(oracle.e4m3_encode(y.astype(np.float64)), torch_encode(y))


def test_encode_ties_go_to_even_code():
    pos = oracle.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    got = oracle.e4m3_encode(mids).astype(int)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))


# ---------------------------------------------------------------------------
# Per-row activation quantizer
# ---------------------------------------------------------------------------

def _rows(rng):
    x = rng.standard_normal((12, 300)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, 12)).astype(np.float32)[:, None]
    x[3] = 0.0                                           # all-zero row
    x[4] = 0.0
    x[4, 17] = -3.5                                      # one non-zero element
    x[5, :] = np.float32(1e-3)                           # constant row
    return synth.bf16_bits(x)


def test_quant_rows_match_library_float32_steps():
    xb = _rows(np.random.default_rng(3))
    codes, s = oracle.quant_fp8_rows(xb)
    x = torch.from_numpy(oracle.widen(xb).astype(np.float32))
    amax = x.abs().amax(dim=1)
    nz = amax > 0
    r = torch.where(nz, torch.tensor(448.0) / torch.where(nz, amax, torch.ones(())),
                    torch.ones(()))
    y = (x * r[:, None]).clamp(-448, 448)
    assert np.array_equal(codes, y.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    s_ref = torch.where(nz, amax / torch.tensor(448.0), torch.ones(())).numpy()
    assert np.array_equal(s, s_ref)


def test_quant_rows_invariants():
    xb = _rows(np.random.default_rng(4))
    x = oracle.widen(xb)
    codes, s = oracle.quant_fp8_rows(xb)
    dec = oracle.e4m3_decode(codes)
    for i in range(x.shape[0]):
        amax = np.abs(x[i]).max()
        if amax == 0:
            assert s[i] == 1.0 and (codes[i] & 0x7F == 0).all()
            continue
        k = np.argmax(np.abs(x[i]))
        assert abs(dec[i, k]) == 448.0 and np.sign(dec[i, k]) == np.sign(x[i, k])
        assert abs(float(s[i]) * 448.0 / amax - 1) <= 2.0 ** -23
        # round to nearest: within half a step of E4M3 (relative 2^-4 for
        # normals, absolute 2^-10 for subnormals), plus float32 rounding
        y = x[i] / float(s[i])
        err = np.abs(dec[i] - np.clip(y, -448, 448))
        assert (err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + np.abs(y) * 2.0 ** -21).all()


def test_quant_rows_power_of_two_equivariance():
    # scaling a row by 2^k scales amax, r and s exactly, so the codes repeat
    xb = _rows(np.random.default_rng(5))
    codes, s = oracle.quant_fp8_rows(xb)
    for k in (-7, 1, 5):
        x2 = oracle.widen(xb).astype(np.float32) * np.float32(2.0 ** k)
        c2, s2 = oracle.quant_fp8_rows(x2)
        assert np.array_equal(c2, codes)
        nz = np.abs(oracle.widen(xb)).max(axis=1) > 0
        assert np.array_equal(s2[nz], (s * np.float32(2.0 ** k))[nz])


# ---------------------------------------------------------------------------
# W8A8 logits
# ---------------------------------------------------------------------------

def test_fp8_logits_exact_rational_brute_force():
    # Each h row is E4M3 values times 2^k with one element of magnitude
    # exactly 448 * 2^k, so r = 2^-k and s = 2^k exactly and the codes are
    # the values themselves: every logit is then an exact rational.
    rng = np.random.default_rng(21)
    B, d, V = 4, 24, 40
    ks = [-3, 0, 2, 5]
    hc = rng.choice(FINITE, size=(B, d))
    hc[:, 5] = np.where(rng.random(B) < 0.5, 0x7E, 0xFE)     # +-448 in every row
    hc[hc & 0x7F == 0x7E] = 0x7E | (hc[hc & 0x7F == 0x7E] & 0x80)
    hv = torch_decode(hc) * np.exp2(ks)[:, None]
    Wq = rng.choice(FINITE, size=(V, d))
    ws = (np.exp2(rng.integers(-9, -3, V)) * rng.choice([1.0, 0.75, 1.25], V)).astype(np.float32)
    h32 = hv.astype(np.float32)
    qh, sh = oracle.quant_fp8_rows(h32)
    assert np.array_equal(torch_decode(qh), torch_decode(hc))
    assert np.array_equal(sh, np.exp2(ks).astype(np.float32))

    Wv = torch_decode(Wq)
    exact = [[sum(Fraction(float(hv[b, k])) * Fraction(float(Wv[v, k])) for k in range(d))
              * Fraction(float(ws[v])) for v in range(V)] for b in range(B)]
    conf, a = oracle.lmhead_conf_fp8(h32, Wq, ws)
    for b in range(B):
        m = max(exact[b])
        assert a[b] == exact[b].index(m)
        ref = 1.0 / sum(np.exp(float(l - m)) for l in exact[b])
        assert abs(conf[b] / ref - 1) <= 1e-14


def test_fp8_planted_targets_recovered_and_guards_hold():
    r = synth.qwen_decode_fp8(V=5000, d=256, B=16)
    conf, a = oracle.lmhead_conf_fp8(r["h"], r["W"], r["w_scale"])
    assert np.array_equal(a, r["targets"])
    gap, dist = lmhead_margins(r["h"], r["W"], r["tau"], w_scale=r["w_scale"])
    assert (gap > 1e-2).all() and (dist >= 1e-3).all()
    assert np.array_equal(conf > r["tau"], r["planted_commit"])
