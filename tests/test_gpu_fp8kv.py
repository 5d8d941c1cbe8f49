"""GPU-vs-oracle parity of the FP8 (OCP E4M3) KV cache, through the C ABI
(run on an MI355X): the quantizer that writes new rows into the cache and
block attention over the cache (reading R19: one float32 scale per KV head
for K and one for V).

Codes: bit-exact (both sides take the rounding decision in float32, to
nearest even).  Attention outputs: within 2e-2 absolute, the bf16 bar; with
unit scales, bit-identical to bd_block_attn on the decoded bf16 cache (the
same MFMA path runs on the same values).  [OV §2.3.2; OCP OFP8]"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth

pytestmark = pytest.mark.gpu

KINDS = {"bidir": bd.BD_MASK_BIDIR, "causal": bd.BD_MASK_CAUSAL,
         "spec_fused": bd.BD_MASK_SPEC_FUSED}


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def bf16_host(t):
    return oracle.widen(runner.to_host(t))


def quant_gpu(x_bits, scale, cap, pos, fill=0x5A):
    n, hkv, dh = x_bits.shape
    cache = torch.full((hkv, cap, dh), fill, dtype=torch.uint8, device="cuda")
    st = bd.bd_kv_quant_fp8(runner.to_dev(x_bits), n, hkv, dh, runner.to_dev(scale), cache,
                            cap, pos)
    assert st == bd.BD_OK
    torch.cuda.synchronize()
    return cache.cpu().numpy()


@pytest.mark.parametrize("n,hkv,dh,pos", [(16, 2, 128, 1280), (5, 3, 36, 0), (1, 1, 4, 7),
                                          (33, 2, 128, 100)])
def test_kv_quant_is_bit_exact(n, hkv, dh, pos):
    rng = np.random.default_rng(n * 100 + dh)
    x = rng.standard_normal((n, hkv, dh)).astype(np.float32) * 3
    x[0, 0, :4] = [1e6, -1e6, 0.0, -0.0]             # saturation and signed zero
    xb = synth.bf16_bits(x)
    scale = (rng.uniform(0.5, 2.0, hkv) / 112).astype(np.float32)
    cap = pos + n + 3
    got = quant_gpu(xb, scale, cap, pos)
    want = oracle.kv_quant_fp8(xb, scale)              # [n][hkv][dh]
    for g in range(hkv):
        assert np.array_equal(got[g, pos:pos + n], want[:, g, :]), g
        assert (got[g, :pos] == 0x5A).all() and (got[g, pos + n:] == 0x5A).all()


def test_kv_quant_ties_to_even():
    # With scale 1 the products are the inputs: every midpoint between
    # neighbouring E4M3 values (in bf16) and its negative.
    pos_vals = oracle.e4m3_decode(np.arange(0x7F))
    mids = (pos_vals[:-1] + pos_vals[1:]) / 2
    vals = np.concatenate([mids, -mids]).astype(np.float32)
    xb = synth.bf16_bits(vals)
    keep = oracle.widen(xb) == vals                    # midpoints exact in bf16
    dh = 4 * ((vals.size + 3) // 4)
    row = np.zeros(dh, np.uint16)
    row[:vals.size] = xb
    got = quant_gpu(row[None, None, :], np.ones(1, np.float32), 1, 0)[0, 0, :vals.size]
    want = oracle.kv_quant_fp8(row[None, None, :], np.ones(1, np.float32))[0, 0, :vals.size]
    assert keep.sum() > 200
    assert np.array_equal(got, want)


def test_kv_quant_empty_is_a_no_op():
    cache = torch.full((1, 4, 8), 7, dtype=torch.uint8, device="cuda")
    x = torch.zeros((1, 1, 8), dtype=torch.bfloat16, device="cuda")
    s = torch.ones(1, device="cuda")
    assert bd.bd_kv_quant_fp8(x, 0, 1, 8, s, cache, 4, 4) == bd.BD_OK
    torch.cuda.synchronize()
    assert (cache == 7).all()


def _attn_case(Bq, P, Hq, Hkv, kind, seed):
    rng = np.random.default_rng(seed)
    cap = P + Bq + 5
    q = synth.bf16_bits(rng.standard_normal((Bq, Hq, 128)).astype(np.float32))
    kc = synth.normal_e4m3(rng, (Hkv * cap, 128)).reshape(Hkv, cap, 128)
    vc = synth.normal_e4m3(rng, (Hkv * cap, 128)).reshape(Hkv, cap, 128)
    ks = (rng.uniform(0.9, 1.1, Hkv) / 112).astype(np.float32)
    vs = (rng.uniform(0.9, 1.1, Hkv) / 112).astype(np.float32)
    return q, kc, vc, ks, vs, cap


@pytest.mark.parametrize("Bq,P,Hq,Hkv,kind", [
    (16, 1280, 16, 2, "bidir"), (5, 100, 4, 2, "causal"), (32, 4608, 16, 2, "spec_fused"),
    (1, 0, 2, 1, "bidir"), (7, 63, 8, 8, "causal"), (64, 700, 2, 1, "bidir"),
    (16, 65520, 2, 1, "bidir"),                     # P + Bq = 65536, the largest
])
def test_block_attn_fp8kv_matches_oracle(Bq, P, Hq, Hkv, kind):
    print(f"fp8kv attention Bq={Bq} P={P} Hq={Hq} Hkv={Hkv} {kind}", flush=True)
    q, kc, vc, ks, vs, cap = _attn_case(Bq, P, Hq, Hkv, kind, seed=Bq + P)
    att = runner.BlockAttnFP8KV(KINDS[kind], Bq, P, cap, Hq, Hkv)
    att(runner.to_dev(q), runner.to_dev(kc), runner.to_dev(vc), runner.to_dev(ks),
        runner.to_dev(vs))
    torch.cuda.synchronize()
    ref = oracle.block_attn_fp8kv(q, kc, vc, ks, vs, P, oracle.intra_block_mask(kind, Bq))
    assert np.abs(bf16_host(att.out) - ref).max() <= 2e-2


def test_unit_scales_equal_the_bf16_path_on_decoded_values():
    Bq, P, Hq, Hkv = 16, 1280, 16, 2
    q, kc, vc, _, _, cap = _attn_case(Bq, P, Hq, Hkv, "bidir", seed=3)
    ones = np.ones(Hkv, np.float32)
    a = runner.BlockAttnFP8KV(bd.BD_MASK_BIDIR, Bq, P, cap, Hq, Hkv)
    a(runner.to_dev(q), runner.to_dev(kc), runner.to_dev(vc), runner.to_dev(ones),
      runner.to_dev(ones))
    kb = synth.bf16_bits(oracle.e4m3_decode(kc).astype(np.float32))
    vb = synth.bf16_bits(oracle.e4m3_decode(vc).astype(np.float32))
    b = runner.BlockAttn(bd.BD_BF16, bd.BD_MASK_BIDIR, Bq, P, cap, Hq, Hkv, 128)
    b(runner.to_dev(q), runner.to_dev(kb), runner.to_dev(vb))
    torch.cuda.synchronize()
    assert torch.equal(a.out, b.out)


def test_quantized_block_rows_then_attention():
    r = synth.qwen_decode_fp8kv()
    B, P, cap, Hkv = r["B"], r["P"], r["cap"], r["Hkv"]
    kc = runner.to_dev(r["k_codes"])
    vc = runner.to_dev(r["v_codes"])
    ks, vs = runner.to_dev(r["k_scale"]), runner.to_dev(r["v_scale"])
    # the block's own rows P .. P+B-1 come from the quantizer
    assert bd.bd_kv_quant_fp8(runner.to_dev(r["k_new"]), B, Hkv, 128, ks, kc, cap, P) == bd.BD_OK
    assert bd.bd_kv_quant_fp8(runner.to_dev(r["v_new"]), B, Hkv, 128, vs, vc, cap, P) == bd.BD_OK
    att = runner.BlockAttnFP8KV(bd.BD_MASK_BIDIR, B, P, cap, r["Hq"], Hkv)
    att(runner.to_dev(r["q"]), kc, vc, ks, vs)
    torch.cuda.synchronize()
    kh, vh = r["k_codes"].copy(), r["v_codes"].copy()
    kh[:, P:P + B] = oracle.kv_quant_fp8(r["k_new"], r["k_scale"]).transpose(1, 0, 2)
    vh[:, P:P + B] = oracle.kv_quant_fp8(r["v_new"], r["v_scale"]).transpose(1, 0, 2)
    assert np.array_equal(kc.cpu().numpy(), kh) and np.array_equal(vc.cpu().numpy(), vh)
    ref = oracle.block_attn_fp8kv(r["q"], kh, vh, r["k_scale"], r["v_scale"], P,
                                  oracle.intra_block_mask("bidir", B))
    assert np.abs(bf16_host(att.out) - ref).max() <= 2e-2
