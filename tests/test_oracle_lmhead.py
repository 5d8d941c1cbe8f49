"""Pins of the oracle's LM-head confidence/argmax.

conf is the largest softmax probability, max_w p(y = w | .) (LOWN article,
'method step details', the anchor confidence); the argmax is the token.
"""
import numpy as np
import scipy.special
import torch

import oracle
from block_diffusion_vlm_amd import synth
from oracle.guards import lmhead_margins


def test_logits_equal_library_matmul():
    rng = np.random.default_rng(0)
    h, W = rng.standard_normal((5, 64)), rng.standard_normal((1000, 64))
    ref = (torch.from_numpy(h) @ torch.from_numpy(W).T).numpy()
    assert np.abs(oracle.lm_logits(h, W, chunk=97) - ref).max() <= 1e-12


def test_conf_equals_library_softmax_max():
    rng = np.random.default_rng(1)
    h, W = rng.standard_normal((7, 32)), rng.standard_normal((500, 32))
    conf, a = oracle.lmhead_conf(h, W)
    p = scipy.special.softmax(h @ W.T, axis=1)
    assert np.abs(conf - p.max(axis=1)).max() <= 1e-14
    assert np.array_equal(a, p.argmax(axis=1))


def test_uniform_logits_give_one_over_v_and_lowest_index():
    V, d = 37, 8
    W = np.ones((V, d))
    h = np.full((3, d), 0.25)
    conf, a = oracle.lmhead_conf(h, W)
    assert np.allclose(conf, 1.0 / V, rtol=0, atol=1e-15)
    assert (a == 0).all()


def test_one_raised_logit_closed_form():
    V, d, t = 50, 4, 17
    for delta in (0.0, 0.5, 3.0, 12.0):
        W = np.zeros((V, d))
        W[:, 0] = 1.0
        W[t, 0] = 1.0 + delta
        h = np.array([[1.0, 0.0, 0.0, 0.0]])
        conf, a = oracle.lmhead_conf(h, W)
        expect = 1.0 / (1.0 + (V - 1) * np.exp(-delta))
        assert abs(conf[0] - expect) <= 1e-15
        assert a[0] == (t if delta > 0 else 0)


def test_ties_resolve_to_lowest_index():
    W = np.zeros((10, 2))
    W[[3, 7], 0] = 2.0
    conf, a = oracle.lmhead_conf(np.array([[1.0, 0.0]]), W)
    assert a[0] == 3
    assert abs(conf[0] - np.exp(2) / (2 * np.exp(2) + 8)) <= 1e-15


def test_shift_invariance_of_conf():
    # adding a constant to every logit leaves the softmax unchanged
    rng = np.random.default_rng(2)
    h, W = rng.standard_normal((4, 16)), rng.standard_normal((300, 16))
    h2 = np.concatenate([h, np.ones((4, 1)) * 7.0], axis=1)
    W2 = np.concatenate([W, np.ones((300, 1))], axis=1)
    c1, a1 = oracle.lmhead_conf(h, W)
    c2, a2 = oracle.lmhead_conf(h2, W2)
    assert np.abs(c1 - c2).max() <= 1e-13 and np.array_equal(a1, a2)


def test_planted_targets_recovered_and_guards_hold_small():
    r = synth.qwen_decode(V=5000, d=256, B=16)
    conf, a = oracle.lmhead_conf(r["h"], r["W"])
    assert np.array_equal(a, r["targets"])
    gap, dist = lmhead_margins(r["h"], r["W"], r["tau"])
    assert (gap > 1e-2).all() and (dist >= 1e-3).all()
    # the band each row was planted in is the side of tau it lands on
    assert np.array_equal(conf > r["tau"], r["planted_commit"])
