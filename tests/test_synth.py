"""The seeded input generators: determinism, number format, shapes, and the
guards the parity tests rely on (checked with the oracle at full size)."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import synth
from oracle.guards import lmhead_margins


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3e38, -2e-39],
                                 np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits(x), ref)


def test_same_seed_same_inputs_and_streams_differ():
    a, b = synth.tiny(), synth.tiny()
    for k in ("ds_q", "W", "h", "k_cache"):
        assert np.array_equal(a[k], b[k])
    c = synth.tiny(seed=5)
    assert not np.array_equal(a["W"], c["W"])
    d1 = synth.dualstream(n_vis=8, n_txt=8, H=2, dh=16)
    d2 = synth.dualstream(n_vis=8, n_txt=8, H=2, dh=16)
    assert np.array_equal(d1["q"], d2["q"])


def test_truncated_values_and_shared_mask_rows():
    r = synth.dualstream(n_vis=16, n_txt=64, H=2, dh=16, dtype="f32")
    assert np.abs(r["v"]).max() <= 4.0
    rows = r["n_vis"] + r["n_txt"] + np.nonzero(r["is_mask"])[0]
    if rows.size > 1:
        assert (r["q"][rows] == r["q"][rows[0]]).all()
        assert (r["v"][rows] == r["v"][rows[0]]).all()


def test_decode_shapes_full_size_metadata():
    r = synth.qwen_decode(V=2000, d=256)
    assert r["q"].shape == (16, 16, 128) and r["q"].dtype == np.uint16
    assert r["k_cache"].shape == (2, 1296, 128) and r["P"] == 1280
    assert r["masked"][0] == 0 and r["masked"][1:].all()


def test_full_size_decode_guards_hold():
    """The Qwen-shaped decode step at its real size: the planted hidden rows
    keep the top-2 logit gap above 1e-2 and every confidence at least 1e-3
    away from tau, so float32 and float64 take the same decisions."""
    r = synth.qwen_decode()
    gap, dist = lmhead_margins(r["h"], r["W"], r["tau"])
    assert gap.min() > 1e-2 and dist.min() >= 1e-3
    conf, a = oracle.lmhead_conf(r["h"], r["W"])
    assert np.array_equal(a, r["targets"])
    assert 0 < (conf[1:] > r["tau"]).sum() < 15


@pytest.mark.parametrize("which", ["linear", "fused"])
def test_full_size_spec_guards_hold(which):
    if which == "linear":
        r = synth.linear_spec()
        hs = [r["h_draft"], r["h_verify"]]
    else:
        r = synth.fused_spec()
        hs = [r["h"]]
    for h in hs:
        gap, _ = lmhead_margins(h, r["W"])
        assert gap.min() > 1e-2


def test_fp8_weights_format_and_determinism():
    a = synth.qwen_decode_fp8(V=3000, d=256)
    b = synth.qwen_decode_fp8(V=3000, d=256)
    assert np.array_equal(a["W"], b["W"]) and np.array_equal(a["h"], b["h"])
    assert a["W"].dtype == np.uint8 and a["W"].shape == (3000, 256)
    assert not ((a["W"] & 0x7F) == 0x7F).any()             # no NaN codes
    assert a["w_scale"].dtype == np.float32 and (a["w_scale"] > 0).all()
    ref = torch.from_numpy(np.array([1.0, -3.3, 447.0, 0.01], np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.e4m3_codes(np.array([1.0, -3.3, 447.0, 0.01])), ref)
    # the stored weights stand for N(0, sigma_w^2) entries
    w = synth.e4m3_row_values(a["W"]) * a["w_scale"][:, None]
    assert abs(w.std() / 0.02 - 1) < 0.05


def test_full_size_fp8_decode_guards_hold():
    r = synth.qwen_decode_fp8()
    gap, dist = lmhead_margins(r["h"], r["W"], r["tau"], w_scale=r["w_scale"])
    assert gap.min() > 1e-2 and dist.min() >= 1e-3
    conf, a = oracle.lmhead_conf_fp8(r["h"], r["W"], r["w_scale"])
    assert np.array_equal(a, r["targets"])
    assert 0 < (conf[1:] > r["tau"]).sum() < 15


def test_guard_redraws_only_failing_rows_from_a_separate_stream():
    """A row the guard rejects is planted again (same target, same side of
    the threshold); every other row and every tensor drawn after the hidden
    rows stay as the unguarded draw has them."""
    from oracle.guards import rows_guarded
    base = synth.qwen_decode(V=3000, d=256)
    calls = [0]

    def reject_row3_once(h, W, w_scale=None):
        calls[0] += 1
        ok = rows_guarded(h, W, 0.9, w_scale)
        if calls[0] == 1:
            ok[3] = False
        return ok

    r = synth.qwen_decode(V=3000, d=256, guard=reject_row3_once)
    changed = np.nonzero((r["h"] != base["h"]).any(axis=1))[0]
    assert changed.tolist() == [3] and calls[0] == 2
    for k in ("q", "k_cache", "v_cache", "W", "targets", "tokens", "masked"):
        assert np.array_equal(r[k], base[k]), k
    conf, a = oracle.lmhead_conf(r["h"], r["W"])
    assert a[3] == r["targets"][3]
    assert (conf[3] > 0.9) == bool(r["planted_commit"][3])
    # a guard that never passes is an error, not a silent pass
    with pytest.raises(RuntimeError):
        synth.qwen_decode(V=3000, d=256, guard=lambda h, W, w=None: np.zeros(len(h), bool))


@pytest.mark.parametrize("fp8", [False, True])
def test_full_size_block_loop_guards_hold(fp8):
    """Every step's planted rows of the full-size block loop keep the top-2
    gap above 1e-2 and every confidence at least 1e-3 from tau as drawn, so
    the unguarded draw (the benchmark's) equals the guarded one."""
    r = synth.qwen_block_loop(fp8=fp8)
    d = r["h_steps"].shape[-1]
    gap, dist = lmhead_margins(r["h_steps"].reshape(-1, d), r["W"], r["tau"],
                               w_scale=r.get("w_scale"))
    assert gap.min() > 1e-2 and dist.min() >= 1e-3
