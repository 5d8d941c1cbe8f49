"""Pins of the oracle's block loop (decode steps on one block until every
position is committed).  [Fast-dVLM overview §1.2: a block is denoised in
parallel over several steps; §4.1: threshold 0.9]"""
import numpy as np

import oracle
from block_diffusion_vlm_amd import synth

TAU = float(np.float32(0.9))


def _tiny_steps(S, masked=None):
    r = synth.tiny()
    B = r["B"]
    q = np.stack([r["q"]] * S)
    h = np.stack([r["h"]] * S)
    m = np.ones(B, np.uint8) if masked is None else np.asarray(masked, np.uint8)
    return r, q, h, m


def test_fixed_inputs_commit_above_threshold_then_one_per_step():
    # With the same hidden rows at every step the confidences never change:
    # the first step commits every masked position above tau (or, if none is,
    # the most confident one), and each later step commits exactly the most
    # confident position still masked.
    for masked in ([1, 1, 1, 1], [0, 1, 1, 1], [1, 0, 1, 0]):
        r, q, h, m = _tiny_steps(6, masked)
        conf, a = oracle.lmhead_conf(r["h"], r["W"])
        m0 = np.asarray(masked, bool)
        k = int((m0 & (conf > TAU)).sum())
        rest = int(m0.sum()) - k
        expect = ([k] if k else []) + [1] * rest
        o = oracle.block_loop(q, r["k_cache"], r["v_cache"], r["P"], h, r["W"], m,
                              r["tokens"], TAU)
        assert o["n_steps"] == len(expect)
        assert list(o["n_committed"][:len(expect)]) == expect
        assert (o["n_committed"][len(expect):] == 0).all()
        assert not o["masked"].any()
        assert np.array_equal(o["tokens"][m0], a[m0])
        assert np.array_equal(o["tokens"][~m0], r["tokens"][~m0])
        # the positions below tau are committed in descending confidence
        below = [i for i in np.argsort(-conf, kind="stable") if m0[i] and not conf[i] > TAU]
        state = m.copy()
        for s in range(len(expect)):
            st = oracle.decode_step(q[s], r["k_cache"], r["v_cache"], r["P"], h[s], r["W"],
                                    state, r["tokens"], TAU)
            newly = np.nonzero(state.astype(bool) & ~st["masked"].astype(bool))[0]
            if s > 0 or k == 0:
                assert list(newly) == [below.pop(0)]
            state = st["masked"]


def test_max_steps_bounds_the_loop():
    r, q, h, m = _tiny_steps(2)
    conf, _ = oracle.lmhead_conf(r["h"], r["W"])
    o = oracle.block_loop(q, r["k_cache"], r["v_cache"], r["P"], h, r["W"], m, r["tokens"], TAU)
    assert o["n_steps"] == 2
    assert int(o["masked"].sum()) == 4 - int(o["n_committed"].sum())


def test_complete_block_runs_no_step():
    r, q, h, _ = _tiny_steps(3)
    o = oracle.block_loop(q, r["k_cache"], r["v_cache"], r["P"], h, r["W"],
                          np.zeros(4, np.uint8), r["tokens"], TAU)
    assert o["n_steps"] == 0 and (o["n_committed"] == 0).all()
    assert np.array_equal(o["tokens"], r["tokens"])


def test_planted_trajectory_commits_each_position_at_its_step():
    r = synth.qwen_block_loop(V=3000, d=256)
    o = oracle.block_loop(r["q_steps"], r["k_cache"], r["v_cache"], r["P"], r["h_steps"], r["W"],
                          r["masked"], r["tokens"], TAU)
    c = r["commit_step"][1:]
    assert o["n_steps"] == r["T"]
    assert np.array_equal(o["n_committed"][:r["T"]], np.bincount(c, minlength=r["T"]))
    assert np.array_equal(o["tokens"][1:], r["final_tokens"][1:])
    assert o["tokens"][0] == r["tokens"][0] and not o["masked"].any()
    # every step before T commits at least one position by threshold
    assert (o["n_committed"][:r["T"]] >= 1).all()


def test_planted_trajectory_fp8_head():
    r = synth.qwen_block_loop(V=3000, d=256, fp8=True)
    o = oracle.block_loop(r["q_steps"], r["k_cache"], r["v_cache"], r["P"], r["h_steps"], r["W"],
                          r["masked"], r["tokens"], TAU, w_scale=r["w_scale"])
    assert o["n_steps"] == r["T"]
    assert np.array_equal(o["tokens"][1:], r["final_tokens"][1:])
