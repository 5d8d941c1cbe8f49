"""GPU-vs-oracle parity of the dual-stream training forward's row
log-sum-exp and of the training backward (dQ, dK, dV), run on an MI355X.

Tolerances (float32 accumulation, bf16 inputs and outputs): the bf16
log-sum-exp is formed from the bf16-rounded probabilities the output uses,
each within 2^-9 relative, so the sum is within 2^-9 and the log within
4e-3 absolute; gradients are stored in bf16 (2^-9 relative) after products
with bf16-rounded P and dS (2^-9 each), so each gradient is compared as
max |got - ref| <= 1e-2 max |ref| + extra, per tensor: the three roundings
bound the relative part near 3 * 2^-9 = 6e-3 of the largest value, and
`extra` is the absolute error that D = rowsum(dO * O), formed from the bf16
output, can add to dQ and dK (grad_bounds.py derives it).
The backward alone, fed the oracle's forward (bf16 output, float32 lse),
is compared with the oracle's backward from those same inputs at the
relative 1e-2 alone, since D then comes from the same output on both sides.
float32: 1e-5 relative to the largest reference value (lse: 1e-5 absolute).
[Fast-dVLM overview §2.2.1; Thai article §4.1, §4.3]
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth
from grad_bounds import grad_tolerances, within

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
    extra = grad_tolerances(r, seg)
    for name, got, ref in (("dq", tr.dq, dq), ("dk", tr.dk, dk), ("dv", tr.dv, dv)):
        ok, err, bound = within(host(got), ref, extra[name])
        print(f"  {name}: max|ref| {np.abs(ref).max():.3g}  err {err:.3g}  bound {bound:.3g}",
              flush=True)
        assert ok, name
    # deterministic: a second backward gives the same bits
    ref_bits = [t.clone() for t in (tr.dq, tr.dk, tr.dv)]
    tr.backward()
    torch.cuda.synchronize()
    for a, b in zip(ref_bits, (tr.dq, tr.dk, tr.dv)):
        assert torch.equal(a, b)


@pytest.fixture(scope="module")
def train_full():
    """Training forward and backward at the real size (1024 visual + 2048
    clean + 2048 noisy tokens, block 32, 16 heads x 128), run once."""
    r = synth.dualstream()
    tr = runner.DualStreamTrain(r)
    tr.forward()
    tr.backward()
    torch.cuda.synchronize()
    return r, {"lse": tr.lse.cpu().numpy(), "dq": host(tr.dq), "dk": host(tr.dk),
               "dv": host(tr.dv)}


@pytest.mark.parametrize("h0", [0, 4, 8, 12])
def test_dualstream_backward_full_size(train_full, h0):
    # every gradient row of four heads per case; the four cases cover all 16
    # heads (the tolerance applies per head, over each whole gradient tensor)
    r, got = train_full
    for h in range(h0, h0 + 4):
        sl = (slice(None), [h], slice(None))
        lse = oracle.dualstream_lse(r["q"][sl], r["k"][sl], r["n_vis"], r["n_txt"], r["block"])
        assert np.abs(got["lse"][:, [h]] - lse).max() <= 4e-3, h
        dq, dk, dv = oracle.dualstream_attn_bwd(r["q"][sl], r["k"][sl], r["v"][sl],
                                                r["d_out"][sl], r["n_vis"], r["n_txt"],
                                                r["block"])
        extra = grad_tolerances(r, heads=[h])
        for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
            ok, err, bound = within(got[name][sl], ref, extra[name])
            print(f"  head {h} {name}: err {err:.3g}  bound {bound:.3g}", flush=True)
            assert ok, (h, name)


def _given_forward(r, seg=None):
    """The oracle's forward output rounded to bf16 and its row log-sum-exp in
    float32: what a backward receives from a forward, taken from the oracle."""
    args = (r["n_vis"], r["n_txt"], r["block"])
    out = oracle.dualstream_attn(r["q"], r["k"], r["v"], *args, seg_starts=seg)
    lse = oracle.dualstream_lse(r["q"], r["k"], *args, seg_starts=seg)
    return synth.bf16_bits(out), lse.astype(np.float32)


def _backward_from(r, out_bits, lse32):
    tr = runner.DualStreamTrain(r)
    tr.out.copy_(runner.to_dev(out_bits))
    tr.lse.copy_(torch.from_numpy(lse32))
    tr.backward()
    torch.cuda.synchronize()
    return tr


# The backward alone, fed the oracle's forward: the entry point takes D from
# the output it is given, so the oracle's backward from the same bf16 output
# and float32 lse leaves only the three relative roundings (P, dS, the stored
# gradient) and the comparison keeps 1e-2 of the largest value.
@pytest.mark.parametrize("n_vis,n_txt,block,H,seg", CASES)
def test_dualstream_backward_from_given_forward(n_vis, n_txt, block, H, seg):
    print(f"bwd from the oracle's forward n_vis={n_vis} n_txt={n_txt} block={block} H={H} "
          f"seg={seg}", flush=True)
    r = synth.dualstream(seed=7 * n_vis + n_txt, n_vis=n_vis, n_txt=n_txt, block=block, H=H)
    r["seg_starts"] = seg
    out_bits, lse32 = _given_forward(r, seg)
    tr = _backward_from(r, out_bits, lse32)
    ref = oracle.dualstream_attn_bwd_given(r["q"], r["k"], r["v"], out_bits, lse32, r["d_out"],
                                           n_vis, n_txt, block, seg_starts=seg)
    for name, got, want in zip(("dq", "dk", "dv"), (tr.dq, tr.dk, tr.dv), ref):
        err = rel_max(host(got), want)
        print(f"  {name}: rel err {err:.3g}", flush=True)
        assert err <= 1e-2, name


@pytest.fixture(scope="module")
def given_full():
    """The backward at the real size (1024 visual + 2048 clean + 2048 noisy
    tokens, block 32, 16 heads x 128) from the oracle's forward, run once."""
    r = synth.dualstream()
    out_bits, lse32 = _given_forward(r)
    tr = _backward_from(r, out_bits, lse32)
    return r, out_bits, lse32, {"dq": host(tr.dq), "dk": host(tr.dk), "dv": host(tr.dv)}


@pytest.mark.parametrize("h0", [0, 4, 8, 12])
def test_dualstream_backward_from_given_forward_full_size(given_full, h0):
    r, out_bits, lse32, got = given_full
    for h in range(h0, h0 + 4):
        sl = (slice(None), [h], slice(None))
        ref = oracle.dualstream_attn_bwd_given(r["q"][sl], r["k"][sl], r["v"][sl],
                                               out_bits[sl], lse32[:, [h]], r["d_out"][sl],
                                               r["n_vis"], r["n_txt"], r["block"])
        for name, want in zip(("dq", "dk", "dv"), ref):
            err = rel_max(got[name][sl], want)
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
