"""Seeded random geometries for the attention entry points, each compared
with the oracle (run on an MI355X).  The fixed-shape tests pick the
interesting corners by hand; this sweep draws sizes, head groupings, block
sizes and segmentations at random so that tile tails, split counts and mask
boundaries fall in places nobody chose.  Tolerances are those of the other
parity tests: 2e-2 absolute on bf16 outputs, 1e-2 of the largest value on
bf16 gradients plus the absolute error that D = rowsum(dO * O), formed from
the bf16 output, can add to dQ and dK (grad_bounds.py).  [OV §1.2, §2.2.1-§2.2.2, §2.3.1-§2.3.2]"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth
from grad_bounds import grad_tolerances, within

pytestmark = pytest.mark.gpu

KINDS = {"bidir": bd.BD_MASK_BIDIR, "causal": bd.BD_MASK_CAUSAL,
         "spec_fused": bd.BD_MASK_SPEC_FUSED}


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def bf16_host(t):
    return oracle.widen(runner.to_host(t))


def _segments(rng, n_txt):
    k = int(rng.integers(1, min(8, n_txt) + 1))
    cuts = sorted(rng.choice(np.arange(1, n_txt), k - 1, replace=False).tolist()) if k > 1 else []
    return [0] + cuts


@pytest.mark.parametrize("case", range(12))
def test_dualstream_forward_random(case):
    rng = np.random.default_rng(7000 + case)
    n_vis = int(rng.integers(0, 300))
    n_txt = int(rng.integers(1, 400))
    block = int(rng.choice([1, 2, 3, 7, 16, 32, 64, 100]))
    H = int(rng.integers(1, 4))
    seg = _segments(rng, n_txt) if case % 2 else None
    print(f"dual-stream n_vis={n_vis} n_txt={n_txt} block={block} H={H} seg={seg}", flush=True)
    r = synth.dualstream(seed=case, n_vis=n_vis, n_txt=n_txt, block=block, H=H)
    if seg is not None:
        r["seg_starts"] = seg
    ds = runner.DualStream(r)
    ds.run()
    torch.cuda.synchronize()
    ref = oracle.dualstream_attn(r["q"], r["k"], r["v"], n_vis, n_txt, block, seg_starts=seg)
    assert np.abs(bf16_host(ds.out) - ref).max() <= 2e-2


@pytest.mark.parametrize("case", range(6))
def test_dualstream_backward_random(case):
    rng = np.random.default_rng(8000 + case)
    n_vis = int(rng.integers(0, 200))
    n_txt = int(rng.integers(1, 250))
    block = int(rng.choice([1, 4, 13, 32, 64]))
    seg = _segments(rng, n_txt) if case % 2 else None
    print(f"backward n_vis={n_vis} n_txt={n_txt} block={block} seg={seg}", flush=True)
    r = synth.dualstream(seed=50 + case, n_vis=n_vis, n_txt=n_txt, block=block, H=2)
    if seg is not None:
        r["seg_starts"] = seg
    tr = runner.DualStreamTrain(r)
    tr.forward()
    tr.backward()
    torch.cuda.synchronize()
    dq, dk, dv = oracle.dualstream_attn_bwd(r["q"], r["k"], r["v"], r["d_out"], n_vis, n_txt,
                                            block, seg_starts=seg)
    extra = grad_tolerances(r, seg)
    for name, got, ref in (("dq", tr.dq, dq), ("dk", tr.dk, dk), ("dv", tr.dv, dv)):
        ok, err, bound = within(bf16_host(got), ref, extra[name])
        assert ok, (name, err, bound)


@pytest.mark.parametrize("case", range(16))
def test_block_attention_random(case):
    rng = np.random.default_rng(9000 + case)
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 3, 8]))
    kind = ["bidir", "causal", "spec_fused"][case % 3]
    Bq = int(rng.integers(1, 33)) * (2 if kind == "spec_fused" else 1)
    # cases 12-15: long prefixes, so that splits take several key tiles
    P = int(rng.integers(0, 3000)) if case < 12 else int(rng.integers(6000, 20000))
    cap = P + Bq + int(rng.integers(0, 40))
    print(f"block attention Bq={Bq} P={P} Hq={Hq} Hkv={Hkv} {kind}", flush=True)
    q = synth.bf16_bits(synth.normal(rng, (Bq, Hq, 128)))
    kc = synth.bf16_bits(synth.normal(rng, (Hkv, cap, 128)))
    vc = synth.bf16_bits(synth.normal(rng, (Hkv, cap, 128), trunc=4.0))
    a = runner.BlockAttn(bd.BD_BF16, KINDS[kind], Bq, P, cap, Hq, Hkv, 128)
    a(runner.to_dev(q), runner.to_dev(kc), runner.to_dev(vc))
    # the same cache as E4M3 codes with per-head scales
    k8 = synth.normal_e4m3(rng, (Hkv * cap, 128)).reshape(Hkv, cap, 128)
    v8 = synth.normal_e4m3(rng, (Hkv * cap, 128)).reshape(Hkv, cap, 128)
    ks = (rng.uniform(0.5, 2.0, Hkv) / 112).astype(np.float32)
    vs = (rng.uniform(0.5, 2.0, Hkv) / 112).astype(np.float32)
    a8 = runner.BlockAttnFP8KV(KINDS[kind], Bq, P, cap, Hq, Hkv)
    a8(runner.to_dev(q), runner.to_dev(k8), runner.to_dev(v8), runner.to_dev(ks),
       runner.to_dev(vs))
    torch.cuda.synchronize()
    intra = oracle.intra_block_mask(kind, Bq)
    assert np.abs(bf16_host(a.out) - oracle.block_attn(q, kc, vc, P, intra)).max() <= 2e-2
    ref8 = oracle.block_attn_fp8kv(q, k8, v8, ks, vs, P, intra)
    assert np.abs(bf16_host(a8.out) - ref8).max() <= 2e-2


@pytest.mark.parametrize("case", range(8))
def test_block_attention_random_masks(case):
    """Arbitrary intra-block masks: every row a random 64-bit word, of which
    bit j < Bq says whether the row's query sees block key j (the higher bits
    are ignored).  Bq up to 64, ragged prefixes, GQA; bf16 and FP8 caches."""
    rng = np.random.default_rng(9500 + case)
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 4, 8]))
    Bq = int(rng.integers(1, 65))
    P = int(rng.integers(0, 2000))
    cap = P + Bq + int(rng.integers(0, 10))
    print(f"block attention, random masks: Bq={Bq} P={P} Hq={Hq} Hkv={Hkv}", flush=True)
    rows = rng.integers(0, 2**63, size=Bq, dtype=np.int64).astype(np.uint64) * np.uint64(2) \
        + rng.integers(0, 2, size=Bq).astype(np.uint64)
    intra = ((rows[:, None] >> np.arange(Bq, dtype=np.uint64)[None]) & np.uint64(1)).astype(bool)
    q = synth.bf16_bits(synth.normal(rng, (Bq, Hq, 128)))
    kc = synth.bf16_bits(synth.normal(rng, (Hkv, cap, 128)))
    vc = synth.bf16_bits(synth.normal(rng, (Hkv, cap, 128), trunc=4.0))
    a = runner.BlockAttn(bd.BD_BF16, bd.BD_MASK_BIDIR, Bq, P, cap, Hq, Hkv, 128)
    a.mask.copy_(runner.to_dev(rows))
    a(runner.to_dev(q), runner.to_dev(kc), runner.to_dev(vc))
    k8 = synth.normal_e4m3(rng, (Hkv * cap, 128)).reshape(Hkv, cap, 128)
    v8 = synth.normal_e4m3(rng, (Hkv * cap, 128)).reshape(Hkv, cap, 128)
    ks = (rng.uniform(0.5, 2.0, Hkv) / 112).astype(np.float32)
    vs = (rng.uniform(0.5, 2.0, Hkv) / 112).astype(np.float32)
    a8 = runner.BlockAttnFP8KV(bd.BD_MASK_BIDIR, Bq, P, cap, Hq, Hkv)
    a8.mask.copy_(runner.to_dev(rows))
    a8(runner.to_dev(q), runner.to_dev(k8), runner.to_dev(v8), runner.to_dev(ks),
       runner.to_dev(vs))
    torch.cuda.synchronize()
    assert np.abs(bf16_host(a.out) - oracle.block_attn(q, kc, vc, P, intra)).max() <= 2e-2
    ref8 = oracle.block_attn_fp8kv(q, k8, v8, ks, vs, P, intra)
    assert np.abs(bf16_host(a8.out) - ref8).max() <= 2e-2
