"""GPU-vs-oracle parity of the multi-block loop (bd_decode_blocks), run on an
MI355X: blocks decoded in order with a device-side kv_len, each seeded by an
AR step, denoised on the device and appended to the KV cache.

Integer results are bit-exact: kv_len, the cache rows, every block's tokens,
masked flags, steps run and commits per step, the argmax of every step that
ran.  Confidences within 1e-4 relative; attention outputs (seed and steps)
within 2e-2 absolute (bf16 outputs, |v| <= 4).  Outputs of steps that did
not run stay untouched.  [Fast-dVLM overview §1.2, §2.2.2, §4.1]
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


def _oracle(r, S):
    return oracle.decode_blocks(r["q_seed"], r["h_seed"], r["q_steps"][:, :S],
                                r["h_steps"][:, :S], r["k_blk"], r["v_blk"], r["k_cache"],
                                r["v_cache"], r["P0"], r["W"], TAU32, w_scale=r.get("w_scale"))


def _run(r, **kw):
    ws = r.get("w_scale")
    run = runner.DecodeBlocks(r, w_scale=None if ws is None else runner.to_dev(ws), **kw)
    run.run()
    torch.cuda.synchronize()
    return run


def _check(run, r, o, guards=True):
    nb, S, B = run.nb, run.S, run.B
    if guards:
        # every LM-head row that decides something is off the float boundaries
        d = r["h_steps"].shape[-1]
        rows = [r["h_seed"]] + [r["h_steps"][b, :o["blocks"][b]["n_steps"]].reshape(-1, d)
                                for b in range(nb)]
        gap, dist = lmhead_margins(np.concatenate(rows), r["W"], TAU32, r.get("w_scale"))
        assert gap.min() > 1e-2 and (dist[nb:].size == 0 or dist[nb:].min() >= 1e-3)
    assert int(run.kv_len.item()) == o["kv_len"] == r["P0"] + nb * B
    assert np.array_equal(runner.to_host(run.k_cache), o["k_cache"])
    assert np.array_equal(runner.to_host(run.v_cache), o["v_cache"])
    tokens, masked = run.tokens.cpu().numpy(), run.masked.cpu().numpy()
    n_steps, ncom = run.n_steps.cpu().numpy(), run.n_committed.cpu().numpy()
    conf, am = run.conf.cpu().numpy(), run.argmax.cpu().numpy()
    seed_conf = run.seed_conf.cpu().numpy()
    for b, blk in enumerate(o["blocks"]):
        assert np.array_equal(tokens[b], blk["tokens"]), b
        assert np.array_equal(masked[b], blk["masked"]), b
        assert n_steps[b] == blk["n_steps"], b
        assert np.array_equal(ncom[b], blk["n_committed"][:S]), b
        assert abs(seed_conf[b] / blk["seed_conf"] - 1) <= 1e-4, b
        got = oracle.widen(runner.to_host(run.seed_attn[b]))
        assert np.abs(got - blk["seed_attn"]).max() <= 2e-2, b
        n = blk["n_steps"]
        for s in range(n):
            assert np.array_equal(am[b, s], blk["argmax"][s]), (b, s)
            assert np.abs(conf[b, s] / blk["conf"][s] - 1).max() <= 1e-4, (b, s)
            got = oracle.widen(runner.to_host(run.attn_out[b, s]))
            assert np.abs(got - blk["attn"][s]).max() <= 2e-2, (b, s)
        assert (conf[b, n:] == -1.0).all() and (am[b, n:] == -1).all()
        assert not run.attn_out[b, n:].any().item()


def test_decode_blocks_matches_oracle():
    r = synth.qwen_decode_blocks(n_blocks=3, V=30011, guard=row_guard(TAU32))
    print("decode_blocks 3 blocks V=30011", flush=True)
    run = runner.DecodeBlocks(r)
    run.run()
    torch.cuda.synchronize()
    o = _oracle(r, run.S)
    for b, blk in enumerate(o["blocks"]):
        assert blk["n_steps"] == r["T"] and blk["seed_token"] == r["seed_targets"][b]
    _check(run, r, o)


def test_decode_blocks_too_few_steps_still_appends():
    r = synth.qwen_decode_blocks(n_blocks=2, V=30011, guard=row_guard(TAU32))
    print("decode_blocks max_steps=3", flush=True)
    run = runner.DecodeBlocks(r, max_steps=3)
    run.run()
    torch.cuda.synchronize()
    o = _oracle(r, 3)
    assert all(blk["masked"].any() for blk in o["blocks"])
    _check(run, r, o)


def test_decode_blocks_device_kv_len_below_the_host_bound():
    # the host bound P_max leaves 100 spare rows; the device kv_len (P0)
    # decides where the blocks go and what they attend
    r = synth.qwen_decode_blocks(n_blocks=2, V=30011, guard=row_guard(TAU32))
    print("decode_blocks kv_len < P_max", flush=True)
    pad = 100
    big = dict(r)
    for k in ("k_cache", "v_cache"):
        a = np.zeros((r["Hkv"], r["cap"] + pad, r["dh"]), np.uint16)
        a[:, :r["cap"]] = r[k]
        big[k] = a
    big["cap"] = r["cap"] + pad
    run = runner.DecodeBlocks(big)
    run.P0 = r["P0"] + pad                  # host bound: larger than the device kv_len
    run.ws_bytes = bd.bd_decode_blocks_ws_bytes(run.P0, run.nb, run.B, run.Hq, run.Hkv, run.dh,
                                                run.d, run.V, False)
    run.ws = runner.workspace(run.ws_bytes)
    run.kv_len.fill_(r["P0"])
    run.run()
    torch.cuda.synchronize()
    o = _oracle(r, run.S)
    assert int(run.kv_len.item()) == o["kv_len"]
    kc = runner.to_host(run.k_cache)
    assert np.array_equal(kc[:, :r["cap"]], o["k_cache"]) and not kc[:, r["cap"]:].any()
    assert np.array_equal(run.tokens.cpu().numpy(), np.stack([b["tokens"] for b in o["blocks"]]))
    for b, blk in enumerate(o["blocks"]):
        got = oracle.widen(runner.to_host(run.seed_attn[b]))
        assert np.abs(got - blk["seed_attn"]).max() <= 2e-2
        for s in range(blk["n_steps"]):
            got = oracle.widen(runner.to_host(run.attn_out[b, s]))
            assert np.abs(got - blk["attn"][s]).max() <= 2e-2


def test_decode_blocks_graph_replays_match_eager():
    r = synth.qwen_decode_blocks(n_blocks=2, V=30011)
    run = runner.DecodeBlocks(r)
    run.reset()
    run.run()
    torch.cuda.synchronize()
    keys = ("tokens", "masked", "n_steps", "n_committed", "conf", "argmax", "attn_out",
            "seed_attn", "seed_conf", "kv_len", "k_cache", "v_cache")
    ref = {k: getattr(run, k).clone() for k in keys}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run.reset()
        run.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.reset()
        run.run()
    torch.cuda.synchronize()
    for rep in range(3):
        run.tokens.fill_(-3)
        run.masked.fill_(1)
        run.kv_len.fill_(7)
        run.k_cache.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(getattr(run, k), ref[k]), (rep, k)


def test_decode_blocks_full_size():
    r = synth.qwen_decode_blocks(n_blocks=2)
    print("decode_blocks full size, 2 blocks", flush=True)
    run = runner.DecodeBlocks(r)
    run.run()
    torch.cuda.synchronize()
    o = _oracle(r, run.S)
    for b, blk in enumerate(o["blocks"]):
        assert blk["n_steps"] == r["T"] and blk["seed_token"] == r["seed_targets"][b]
    _check(run, r, o)


@pytest.mark.parametrize("B,S,T,n_vis,n_prompt,Hq,Hkv,d,V", [
    (5, 4, 3, 37, 11, 4, 1, 256, 3001),       # ragged block, prefix off the tile grid
    (1, 1, 1, 20, 3, 2, 1, 128, 1000),        # the seed is the whole block: no steps run
    (64, 8, 6, 100, 20, 2, 2, 128, 1000),     # the largest block (one mask word)
])
def test_decode_blocks_ragged_shapes(B, S, T, n_vis, n_prompt, Hq, Hkv, d, V):
    r = synth.qwen_decode_blocks(n_blocks=3, B=B, S=S, T=T, n_vis=n_vis, n_prompt=n_prompt,
                                 Hq=Hq, Hkv=Hkv, d=d, V=V, guard=row_guard(TAU32))
    print(f"decode_blocks B={B} S={S} P0={n_vis + n_prompt} Hq={Hq} Hkv={Hkv} d={d} V={V}",
          flush=True)
    run = _run(r)
    o = _oracle(r, run.S)
    for b, blk in enumerate(o["blocks"]):
        assert blk["n_steps"] == (T if B > 1 else 0) and blk["seed_token"] == r["seed_targets"][b]
    _check(run, r, o)


def test_decode_blocks_fp8_lm_head_matches_oracle():
    r = synth.qwen_decode_blocks(n_blocks=3, V=30011, fp8=True, guard=row_guard(TAU32))
    print("decode_blocks FP8 LM head, 3 blocks V=30011", flush=True)
    run = _run(r)
    o = _oracle(r, run.S)
    for b, blk in enumerate(o["blocks"]):
        assert blk["n_steps"] == r["T"] and blk["seed_token"] == r["seed_targets"][b]
    _check(run, r, o)

