"""GPU-vs-oracle parity of the device-resident block loop (bd_block_loop),
run on an MI355X: decode steps on one block until it is committed, every
kernel of every step enqueued up front and the steps that run decided on
the device.

Integer results (steps run, commits per step, final tokens and flags, the
argmax of every step that ran) are bit-exact; the confidences of the steps
that ran within 1e-4 relative; the attention outputs within 2e-2 absolute.
The outputs of the steps that did not run stay untouched.  [Fast-dVLM
overview §1.2, §4.1]
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import runner, synth
from oracle.guards import lmhead_margins, row_guard

pytestmark = pytest.mark.gpu

TAU32 = float(np.float32(0.9))


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    from block_diffusion_vlm_amd import bdiff as bd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def _oracle(r, S=None):
    S = r["q_steps"].shape[0] if S is None else S
    return oracle.block_loop(r["q_steps"][:S], r["k_cache"], r["v_cache"], r["P"],
                             r["h_steps"][:S], r["W"], r["masked"], r["tokens"], TAU32,
                             w_scale=r.get("w_scale"))


def _check(loop, r, o):
    n = o["n_steps"]
    # every executed step's rows are off the floating-point boundaries (one
    # pass over W for all of them)
    d = r["h_steps"].shape[-1]
    gap, dist = lmhead_margins(r["h_steps"][:n].reshape(-1, d), r["W"], TAU32,
                               w_scale=r.get("w_scale"))
    assert gap.min() > 1e-2 and dist.min() >= 1e-3
    assert int(loop.n_steps.item()) == n
    assert np.array_equal(loop.n_committed.cpu().numpy(), o["n_committed"][:loop.S])
    assert np.array_equal(runner.to_host(loop.masked), o["masked"])
    assert np.array_equal(runner.to_host(loop.tokens), o["tokens"])
    conf = loop.conf.cpu().numpy()
    am = loop.argmax.cpu().numpy()
    for s in range(n):
        assert np.array_equal(am[s], o["argmax"][s]), s
        assert np.abs(conf[s] / o["conf"][s] - 1).max() <= 1e-4, s
        out = oracle.widen(runner.to_host(loop.attn_out[s]))
        assert np.abs(out - o["attn"][s]).max() <= 2e-2, s
    # steps after the block completed left their outputs alone
    assert (conf[n:] == -1.0).all() and (am[n:] == -1).all()
    assert not loop.attn_out[n:].any().item()


@pytest.mark.parametrize("fp8", [False, True])
def test_block_loop_matches_oracle(fp8):
    r = synth.qwen_block_loop(V=30011, fp8=fp8, guard=row_guard(TAU32))
    loop = runner.BlockLoop(r)
    loop.run()
    torch.cuda.synchronize()
    o = _oracle(r)
    assert o["n_steps"] == r["T"]
    _check(loop, r, o)


def test_block_loop_stops_at_max_steps():
    r = synth.qwen_block_loop(V=30011, guard=row_guard(TAU32))
    loop = runner.BlockLoop(r, max_steps=3)
    loop.run()
    torch.cuda.synchronize()
    o = _oracle(r, S=3)
    assert o["n_steps"] == 3 and o["masked"].any()
    _check(loop, r, o)


def test_block_loop_complete_block_runs_nothing():
    r = synth.qwen_block_loop(V=30011)
    r["masked"] = np.zeros_like(r["masked"])
    loop = runner.BlockLoop(r)
    loop.run()
    torch.cuda.synchronize()
    assert int(loop.n_steps.item()) == 0
    assert (loop.n_committed == 0).all()
    assert np.array_equal(runner.to_host(loop.tokens), r["tokens"])
    assert (loop.conf == -1.0).all()


def test_block_loop_f32_tiny():
    t = synth.tiny()
    S = 6
    r = {"dtype": "f32", "B": t["B"], "P": t["P"], "cap": t["cap"], "Hq": 1, "Hkv": 1,
         "dh": t["dh"], "d": t["d"], "V": t["V"], "tau": 0.9,
         "q_steps": np.stack([t["q"]] * S), "h_steps": np.stack([t["h"]] * S),
         "k_cache": t["k_cache"], "v_cache": t["v_cache"], "W": t["W"],
         "masked": t["masked"], "tokens": t["tokens"]}
    loop = runner.BlockLoop(r)
    loop.run()
    torch.cuda.synchronize()
    o = _oracle(r)
    n = o["n_steps"]
    assert int(loop.n_steps.item()) == n
    assert np.array_equal(loop.n_committed.cpu().numpy(), o["n_committed"])
    assert np.array_equal(runner.to_host(loop.tokens), o["tokens"])
    for s in range(n):
        assert np.array_equal(loop.argmax[s].cpu().numpy(), o["argmax"][s])
        out = loop.attn_out[s].cpu().numpy().astype(np.float64)
        assert np.abs(out - o["attn"][s]).max() <= 1e-5 * max(np.abs(o["attn"][s]).max(), 1)


def test_block_loop_graph_replays_match_eager():
    r = synth.qwen_block_loop(V=30011)
    loop = runner.BlockLoop(r)
    loop.reset()
    loop.run()
    torch.cuda.synchronize()
    ref = {k: getattr(loop, k).clone() for k in ("tokens", "masked", "n_committed", "n_steps",
                                                 "conf", "argmax", "attn_out")}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        loop.reset()
        loop.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop.reset()
        loop.run()
    torch.cuda.synchronize()
    for rep in range(3):
        loop.tokens.fill_(-3)
        loop.masked.fill_(1)
        loop.n_steps.fill_(99)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(getattr(loop, k), v), (rep, k)


def test_block_loop_full_size():
    r = synth.qwen_block_loop()
    loop = runner.BlockLoop(r)
    loop.run()
    torch.cuda.synchronize()
    o = _oracle(r)
    assert o["n_steps"] == r["T"]
    _check(loop, r, o)
