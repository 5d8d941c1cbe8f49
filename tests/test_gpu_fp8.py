"""GPU-vs-oracle parity of the FP8 (OCP E4M3, W8A8) LM head and of the
per-row quantizer it applies to the hidden states, through the C ABI (run on
an MI355X).

E4M3 codes and scales: bit-exact (both sides take the rounding decisions in
float32, to nearest even).  argmax and commits: bit-exact (the inputs keep
the top-2 logit gap above 1e-2 and every confidence 1e-3 away from tau).
Confidence: within 1e-4 relative.  [Fast-dVLM overview §2.3.2, FP8
SmoothQuant W8A8]
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth
from oracle.guards import lmhead_margins, row_guard

pytestmark = pytest.mark.gpu

TAU32 = float(np.float32(0.9))


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def quant_gpu(xb):
    R, d = xb.shape
    x = runner.to_dev(xb)
    q = torch.full((max(R, 1), d), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((max(R, 1),), -1.0, dtype=torch.float32, device="cuda")
    bd.bd_quant_fp8_rows(x, R, d, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy()[:R], s.cpu().numpy()[:R]


def crafted_rows(d=512):
    """Rows whose maximum is 448 (so r = 1 and the products are the inputs):
    they test the rounding itself.  Every midpoint between neighbouring E4M3
    values (ties go to the even code) and its negative, the bfloat16
    neighbours of each midpoint, subnormal ties, magnitudes below half the
    smallest subnormal, and negative values that round to zero (0x80)."""
    pos = oracle.e4m3_decode(np.arange(0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    mb = synth.bf16_bits(mids)
    up = oracle.widen(mb + np.uint16(1))
    down = oracle.widen(mb - np.uint16(1))
    tiny = np.array([2.0 ** -10, 3 * 2.0 ** -10, 5 * 2.0 ** -10, 2.0 ** -11, 2.0 ** -16,
                     -(2.0 ** -10), -(2.0 ** -11), -(3 * 2.0 ** -10), -(2.0 ** -20), 0.0])
    rows = []
    for body in (np.concatenate([mids, -mids]), np.concatenate([up, -down]),
                 np.concatenate([down, -up]), tiny):
        r = np.zeros(d)
        r[0] = 448.0 if len(rows) % 2 == 0 else -448.0
        r[1:1 + body.size] = body
        rows.append(r)
    return synth.bf16_bits(np.array(rows, np.float32))


def test_quant_rows_rounding_is_bit_exact():
    xb = crafted_rows()
    q, s = quant_gpu(xb)
    oq, os_ = oracle.quant_fp8_rows(xb)
    assert np.array_equal(s, os_) and (s == 1.0).all()
    bad = np.argwhere(q != oq)
    assert bad.size == 0, [(int(i), int(j), float(oracle.widen(xb[i, j])), int(q[i, j]),
                            int(oq[i, j])) for i, j in bad[:10]]


@pytest.mark.parametrize("R,d", [(1, 8), (5, 136), (37, 2048), (3, 16384), (300, 256)])
def test_quant_rows_random_bit_exact(R, d):
    rng = np.random.default_rng(R * 1000 + d)
    x = rng.standard_normal((R, d)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, R)).astype(np.float32)[:, None]
    if R > 2:
        x[1] = 0.0                       # all-zero row: scale 1, zero codes
        x[2, :] = 0.0
        x[2, d // 2] = -7.0              # one non-zero element
    xb = synth.bf16_bits(x)
    q, s = quant_gpu(xb)
    oq, os_ = oracle.quant_fp8_rows(xb)
    assert np.array_equal(s, os_)
    assert np.array_equal(q, oq)


def test_quant_rows_empty_is_a_no_op():
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.full((1, 64), 7, dtype=torch.uint8, device="cuda")
    s = torch.full((1,), 3.0, device="cuda")
    assert bd.bd_quant_fp8_rows(x, 0, 64, q, s) == bd.BD_OK
    torch.cuda.synchronize()
    assert (q == 7).all() and (s == 3.0).all()


# ---------------------------------------------------------------------------
# LM head
# ---------------------------------------------------------------------------

def _case(B, d, V, seed, tau=None):
    """An input whose every decision is off the floating-point boundary (top-2
    gap > 1e-2; with tau, confidences at least 1e-3 from it): rows that fail
    are re-drawn by the generator."""
    r = synth.qwen_decode_fp8(seed=seed, B=B, d=d, V=V, n_vis=4, n_prompt=4, Hq=2, Hkv=1,
                              guard=row_guard(tau))
    gap, dist = lmhead_margins(r["h"], r["W"], tau, w_scale=r["w_scale"])
    assert gap.min() > 1e-2 and (dist is None or dist.min() >= 1e-3)
    return r


SHAPES = [
    (1, 128, 17), (4, 256, 1000), (16, 512, 4099), (16, 640, 777), (16, 1024, 5000),
    (17, 1024, 3001), (32, 2048, 20011), (33, 384, 999), (64, 2048, 3001),
    (16, 2048, 151936),
    # shapes outside the streaming kernel's register/LDS plan (generic path)
    (16, 8192, 3000), (48, 4096, 2001), (2, 16384, 333),
]


@pytest.mark.parametrize("B,d,V", SHAPES)
def test_lmhead_fp8_matches_oracle(B, d, V):
    print(f"fp8 lmhead B={B} d={d} V={V}", flush=True)
    r = _case(B, d, V, seed=B * 7 + d + V)
    h, W, ws = runner.to_dev(r["h"]), runner.to_dev(r["W"]), runner.to_dev(r["w_scale"])
    lm = runner.LMHeadFP8(W, ws, B, d, V)
    lm(h)
    torch.cuda.synchronize()
    conf0, a0 = lm.conf.cpu().numpy().copy(), lm.argmax.cpu().numpy().copy()
    oc, oa = oracle.lmhead_conf_fp8(r["h"], r["W"], r["w_scale"])
    assert np.array_equal(a0, oa)
    assert np.abs(conf0 / oc - 1).max() <= 1e-4
    # deterministic on a dirty workspace
    lm(h)
    torch.cuda.synchronize()
    assert np.array_equal(lm.conf.cpu().numpy(), conf0)
    assert np.array_equal(lm.argmax.cpu().numpy(), a0)


@pytest.mark.parametrize("B,d,V", [(1, 128, 1000), (16, 2048, 30011), (32, 2048, 3001),
                                   (33, 384, 999), (20, 8192, 700)])
def test_lmhead_fp8_conf_commit_equals_separate_calls(B, d, V):
    r = _case(B, d, V, seed=B + V, tau=TAU32)
    h, W, ws = runner.to_dev(r["h"]), runner.to_dev(r["W"]), runner.to_dev(r["w_scale"])
    masked0 = (np.random.default_rng(B).random(B) < 0.8).astype(np.uint8)
    tokens0 = np.arange(B, dtype=np.int32) + 7
    out = {}
    for fused in (False, True):
        lm = runner.LMHeadFP8(W, ws, B, d, V)
        masked, tokens = runner.to_dev(masked0), runner.to_dev(tokens0)
        n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        if fused:
            lm.conf_commit(h, TAU32, masked, tokens, n)
        else:
            lm(h)
            bd.bd_commit(lm.conf, lm.argmax, B, TAU32, masked, tokens, n)
        torch.cuda.synchronize()
        out[fused] = (lm.conf.cpu().numpy(), lm.argmax.cpu().numpy(), runner.to_host(masked),
                      runner.to_host(tokens), int(n.item()))
    for a, b in zip(out[False], out[True]):
        assert np.array_equal(a, b)
    oc, oa = oracle.lmhead_conf_fp8(r["h"], r["W"], r["w_scale"])
    m2, t2, nc = oracle.commit(oc, oa, masked0, tokens0, TAU32)
    assert np.array_equal(out[True][1], oa)
    assert np.array_equal(out[True][2], m2) and np.array_equal(out[True][3], t2)
    assert out[True][4] == nc


def test_decode_step_fp8_full_size():
    r = synth.qwen_decode_fp8(guard=row_guard(TAU32))
    gap, dist = lmhead_margins(r["h"], r["W"], TAU32, w_scale=r["w_scale"])
    assert gap.min() > 1e-2 and dist.min() >= 1e-3
    step = runner.DecodeStep(r)
    step.run()
    torch.cuda.synchronize()
    o = oracle.decode_step(r["q"], r["k_cache"], r["v_cache"], r["P"], r["h"], r["W"],
                           r["masked"], r["tokens"], TAU32, w_scale=r["w_scale"])
    assert np.array_equal(step.lm.argmax.cpu().numpy(), o["argmax"])
    assert np.array_equal(runner.to_host(step.masked), o["masked"])
    assert np.array_equal(runner.to_host(step.tokens), o["tokens"])
    assert int(step.n_committed.item()) == o["n_committed"]
    assert np.abs(step.lm.conf.cpu().numpy() / o["conf"] - 1).max() <= 1e-4
    assert np.abs(oracle.widen(runner.to_host(step.attn.out)) - o["attn"]).max() <= 2e-2
