"""Pins of the oracle's multi-block decode loop (oracle.decode_blocks): blocks
decoded in order, each started by an AR seed step and appended to the KV
cache before the next.  [Fast-dVLM overview §1.2: blocks one after another
with the KV cache reused; §2.2.2: causal-context decoding, the block's first
token from the AR prediction]

What pins it, independently of the oracle's own helpers:
- the cache: the prefix rows are unchanged and each block's rows sit at
  P0 + b B .. P0 + (b+1) B - 1, exactly the generator's rows; kv_len ends at
  P0 + n_blocks B;
- attention: the seed query of block b and the step queries of block b equal
  torch's scaled_dot_product_attention (float64) over keys concatenated by
  hand from the generator's arrays (the prompt prefix, the earlier blocks'
  rows, and for the steps the block's own rows);
- decisions: on planted trajectories the seed token is the planted one and
  every masked position is committed at its planted step with its planted
  token.
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import synth

TAU = float(np.float32(0.9))


@pytest.fixture(scope="module")
def small():
    r = synth.qwen_decode_blocks(n_blocks=3, V=3000, d=256, n_vis=40, n_prompt=8, Hq=4, Hkv=2,
                                 dh=16)
    o = oracle.decode_blocks(r["q_seed"], r["h_seed"], r["q_steps"], r["h_steps"], r["k_blk"],
                             r["v_blk"], r["k_cache"], r["v_cache"], r["P0"], r["W"], TAU)
    return r, o


def _sdpa(q, k, v):
    """Dense softmax attention, q [Nq][Hq][dh], k/v [Nk][Hkv][dh] (GQA)."""
    q, k, v = (torch.from_numpy(oracle.widen(x)) for x in (q, k, v))
    g = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2), k.permute(1, 0, 2), v.permute(1, 0, 2))
    return o.permute(1, 0, 2).numpy()


def test_cache_grows_by_each_blocks_rows(small):
    r, o = small
    P0, B, nb = r["P0"], r["B"], r["n_blocks"]
    assert o["kv_len"] == P0 + nb * B
    assert np.array_equal(o["k_cache"][:, :P0], r["k_cache"][:, :P0])
    assert np.array_equal(o["v_cache"][:, :P0], r["v_cache"][:, :P0])
    for b in range(nb):
        rows = slice(P0 + b * B, P0 + (b + 1) * B)
        for g in range(r["Hkv"]):
            assert np.array_equal(o["k_cache"][g, rows], r["k_blk"][b][:, g])
            assert np.array_equal(o["v_cache"][g, rows], r["v_blk"][b][:, g])
        assert o["blocks"][b]["P"] == P0 + b * B


def _keys(r, upto_block, own_block=None):
    """[P0 prefix rows; rows of blocks < upto_block; (own block rows)] as
    [N][Hkv][dh], built from the generator's arrays."""
    P0 = r["P0"]
    ks = [np.transpose(r["k_cache"][:, :P0], (1, 0, 2))] + [r["k_blk"][j]
                                                             for j in range(upto_block)]
    vs = [np.transpose(r["v_cache"][:, :P0], (1, 0, 2))] + [r["v_blk"][j]
                                                             for j in range(upto_block)]
    if own_block is not None:
        ks.append(r["k_blk"][own_block])
        vs.append(r["v_blk"][own_block])
    return np.concatenate(ks), np.concatenate(vs)


def test_seed_attends_the_prompt_and_every_earlier_block(small):
    r, o = small
    for b in range(r["n_blocks"]):
        k, v = _keys(r, b)
        ref = _sdpa(r["q_seed"][b][None], k, v)[0]
        assert np.abs(o["blocks"][b]["seed_attn"] - ref).max() <= 1e-12


def test_steps_attend_earlier_blocks_and_their_own_block(small):
    r, o = small
    for b in range(r["n_blocks"]):
        k, v = _keys(r, b, own_block=b)
        for s in range(o["blocks"][b]["n_steps"]):
            ref = _sdpa(r["q_steps"][b][s], k, v)            # bidirectional block
            assert np.abs(o["blocks"][b]["attn"][s] - ref).max() <= 1e-12, (b, s)


def test_planted_blocks_commit_seed_and_positions_at_their_steps(small):
    r, o = small
    T = r["T"]
    for b, blk in enumerate(o["blocks"]):
        assert blk["seed_token"] == r["seed_targets"][b]
        assert blk["tokens"][0] == r["seed_targets"][b]
        assert np.array_equal(blk["tokens"][1:], r["final_tokens"][b][1:])
        assert not blk["masked"].any() and blk["n_steps"] == T
        c = r["commit_step"][b][1:]
        assert np.array_equal(blk["n_committed"][:T], np.bincount(c, minlength=T))
        assert (blk["n_committed"][T:] == 0).all()
        assert blk["seed_conf"] > 0.9


def test_one_block_with_too_few_steps_stays_masked_and_is_still_appended():
    r = synth.qwen_decode_blocks(n_blocks=2, S=3, T=8, V=3000, d=256, n_vis=16, n_prompt=8,
                                 Hq=2, Hkv=1, dh=16)
    o = oracle.decode_blocks(r["q_seed"], r["h_seed"], r["q_steps"], r["h_steps"], r["k_blk"],
                             r["v_blk"], r["k_cache"], r["v_cache"], r["P0"], r["W"], TAU)
    assert o["kv_len"] == r["P0"] + 2 * r["B"]
    for blk in o["blocks"]:
        assert blk["n_steps"] == 3 and blk["masked"].any()
        assert int(blk["masked"].sum()) == r["B"] - 1 - int(blk["n_committed"].sum())


def test_planted_fp8_blocks_commit_seed_and_positions_at_their_steps():
    # the same trajectories with an E4M3 weight matrix (one scale per row):
    # the W8A8 logits recover every planted token at its planted step
    r = synth.qwen_decode_blocks(n_blocks=2, B=6, S=5, T=4, V=2000, d=256, n_vis=24, n_prompt=8,
                                 Hq=2, Hkv=1, dh=16, fp8=True)
    o = oracle.decode_blocks(r["q_seed"], r["h_seed"], r["q_steps"], r["h_steps"], r["k_blk"],
                             r["v_blk"], r["k_cache"], r["v_cache"], r["P0"], r["W"], TAU,
                             w_scale=r["w_scale"])
    T = r["T"]
    for b, blk in enumerate(o["blocks"]):
        assert blk["seed_token"] == r["seed_targets"][b]
        assert np.array_equal(blk["tokens"][1:], r["final_tokens"][b][1:])
        assert not blk["masked"].any() and blk["n_steps"] == T
        assert np.array_equal(blk["n_committed"][:T], np.bincount(r["commit_step"][b][1:],
                                                                  minlength=T))
