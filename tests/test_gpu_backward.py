"""GPU-vs-oracle parity of the dual-stream training forward's row
log-sum-exp and of the training backward (dQ, dK, dV), run on an MI355X.

Tolerances (float32 accumulation, bf16 inputs and outputs): the bf16
log-sum-exp is formed from the bf16-rounded probabilities the output uses,
each within 2^-9 relative, so the sum is within 2^-9 and the log within
4e-3 absolute; gradients are stored in bf16 (2^-9 relative) after products
with bf16-rounded P and dS (2^-9 each) and a D formed from the bf16 output, so
every gradient is compared as max |got - ref| <= 1e-2 max |ref|, per tensor
(the three roundings bound the error near 3 * 2^-9 = 6e-3 of the largest
value; about 4e-3 is observed).
float32: 1e-5 relative to the largest reference value (lse: 1e-5 absolute).
[Fast-dVLM overview §2.2.1; Thai article §4.1, §4.3]
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def host(t):
    return oracle.widen(runner.to_host(t))


def rel_max(got, ref):
    return np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)


CASES = [
    # n_vis, n_txt, block, H, segment starts
    (64, 96, 32, 2, None),
    (5, 37, 4, 1, None),
    (0, 70, 8, 1, None),
    (100, 0, 4, 2, None),
    (128, 128, 32, 1, None),
    (130, 250, 7, 1, None),
    (64, 300, 32, 2, [0, 37, 150, 151, 299]),
    (1, 1, 1, 3, None),
]


@pytest.mark.parametrize("n_vis,n_txt,block,H,seg", CASES)
def test_dualstream_backward_bf16_matches_oracle(n_vis, n_txt, block, H, seg):
    print(f"bwd n_vis={n_vis} n_txt={n_txt} block={block} H={H} seg={seg}", flush=True)
    r = synth.dualstream(seed=7 * n_vis + n_txt, n_vis=n_vis, n_txt=n_txt, block=block, H=H)
    r["seg_starts"] = seg
    tr = runner.DualStreamTrain(r)
    tr.forward()
    tr.backward()
    torch.cuda.synchronize()
    lse = oracle.dualstream_lse(r["q"], r["k"], n_vis, n_txt, block, seg_starts=seg)
    assert np.abs(tr.lse.cpu().numpy() - lse).max() <= 4e-3
    assert np.abs(host(tr.out) - oracle.dualstream_attn(
        r["q"], r["k"], r["v"], n_vis, n_txt, block, seg_starts=seg)).max() <= 2e-2
    dq, dk, dv = oracle.dualstream_attn_bwd(r["q"], r["k"], r["v"], r["d_out"], n_vis, n_txt,
                                            block, seg_starts=seg)
    for name, got, ref in (("dq", tr.dq, dq), ("dk", tr.dk, dk), ("dv", tr.dv, dv)):
        err = rel_max(host(got), ref)
        print(f"  {name}: max|ref| {np.abs(ref).max():.3g}  rel err {err:.3g}", flush=True)
        assert err <= 1e-2, name
    # deterministic: a second backward gives the same bits
    ref_bits = [t.clone() for t in (tr.dq, tr.dk, tr.dv)]
    tr.backward()
    torch.cuda.synchronize()
    for a, b in zip(ref_bits, (tr.dq, tr.dk, tr.dv)):
        assert torch.equal(a, b)


def test_dualstream_backward_full_size_sampled_heads():
    r = synth.dualstream()
    tr = runner.DualStreamTrain(r)
    tr.forward()
    tr.backward()
    torch.cuda.synchronize()
    for h in (0, 11):
        sl = (slice(None), [h], slice(None))
        dq, dk, dv = oracle.dualstream_attn_bwd(r["q"][sl], r["k"][sl], r["v"][sl],
                                                r["d_out"][sl], r["n_vis"], r["n_txt"],
                                                r["block"])
        for name, got, ref in (("dq", tr.dq, dq), ("dk", tr.dk, dk), ("dv", tr.dv, dv)):
            err = rel_max(host(got)[sl], ref)
            print(f"  head {h} {name}: rel err {err:.3g}", flush=True)
            assert err <= 1e-2, (h, name)


def test_dualstream_backward_f32_tiny():
    t = synth.tiny()
    rng = np.random.default_rng(3)
    r = {"dtype": "f32", "n_vis": 4, "n_txt": 4, "block": 2, "H": 1, "dh": 16,
         "q": t["ds_q"], "k": t["ds_k"], "v": t["ds_v"],
         "d_out": rng.standard_normal(t["ds_q"].shape).astype(np.float32)}
    for seg in (None, [0, 1]):
        r["seg_starts"] = seg
        tr = runner.DualStreamTrain(r)
        tr.forward()
        tr.backward()
        torch.cuda.synchronize()
        lse = oracle.dualstream_lse(r["q"], r["k"], 4, 4, 2, seg_starts=seg)
        assert np.abs(tr.lse.cpu().numpy() - lse).max() <= 1e-5
        dq, dk, dv = oracle.dualstream_attn_bwd(r["q"], r["k"], r["v"], r["d_out"], 4, 4, 2,
                                                seg_starts=seg)
        for got, ref in ((tr.dq, dq), (tr.dk, dk), (tr.dv, dv)):
            assert rel_max(got.cpu().numpy().astype(np.float64), ref) <= 1e-5


def test_training_forward_without_lse_equals_plain_forward():
    r = synth.dualstream(seed=2, n_vis=64, n_txt=200, block=32, H=2)
    a = runner.DualStream(r)
    a.run()
    tr = runner.DualStreamTrain(r)
    tr.forward()
    torch.cuda.synchronize()
    assert torch.equal(a.out, tr.out)
