"""Back-to-back LM-head calls on one workspace, through the C ABI (run on an
MI355X).

The streaming kernel leaves one partial state per workgroup and position in
the workspace, and the merge kernel that follows reads them.  These tests
alternate two inputs on one workspace with no synchronisation between the
calls.  A merge that read a partial left by the previous call would show
here.  Every call's argmax must equal the oracle's, and its confidence must
lie within 1e-4 relative of the oracle's.  [LOWN article, 'method step
details' (1): a position's confidence is its largest softmax probability]
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth
from oracle.guards import lmhead_margins, row_guard

pytestmark = pytest.mark.gpu

CALLS = 24


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def _bf16_case(B, d, V, seed):
    r = synth.qwen_decode(seed=seed, B=B, d=d, V=V, n_vis=4, n_prompt=4, Hq=2, Hkv=1,
                          guard=row_guard())
    gap, _ = lmhead_margins(r["h"], r["W"])
    assert gap.min() > 1e-2
    return r


def _fp8_case(B, d, V, seed):
    r = synth.qwen_decode_fp8(seed=seed, B=B, d=d, V=V, n_vis=4, n_prompt=4, Hq=2, Hkv=1,
                              guard=row_guard())
    gap, _ = lmhead_margins(r["h"], r["W"], w_scale=r["w_scale"])
    assert gap.min() > 1e-2
    return r


def _check_calls(outs, refs):
    for i, (conf, am) in enumerate(outs):
        oc, oa = refs[i % 2]
        assert np.array_equal(am.cpu().numpy(), oa), f"call {i}: argmax"
        assert np.abs(conf.cpu().numpy() / oc - 1).max() <= 1e-4, f"call {i}: confidence"


@pytest.mark.parametrize("B,d,V", [(16, 2048, 30000), (4, 256, 1000), (33, 384, 999)])
def test_lmhead_bf16_alternating_calls(B, d, V):
    print(f"bf16 lmhead x{CALLS} B={B} d={d} V={V}", flush=True)
    cases = [_bf16_case(B, d, V, seed=s) for s in (B + d, B + d + 1)]
    h = [runner.to_dev(r["h"]) for r in cases]
    W = [runner.to_dev(r["W"]) for r in cases]
    refs = [oracle.lmhead_conf(r["h"], r["W"]) for r in cases]
    wsb = bd.bd_lmhead_conf_ws_bytes(B, d, V)
    ws = runner.workspace(wsb)
    outs = [(torch.empty(B, device="cuda"), torch.empty(B, dtype=torch.int32, device="cuda"))
            for _ in range(CALLS)]
    for i, (conf, am) in enumerate(outs):
        st = bd.bd_lmhead_conf(bd.BD_BF16, h[i % 2], W[i % 2], B, d, V, conf, am, ws, wsb)
        assert st == bd.BD_OK
    torch.cuda.synchronize()
    _check_calls(outs, refs)


@pytest.mark.parametrize("B,d,V", [(16, 2048, 30011), (5, 512, 777)])
def test_lmhead_fp8_alternating_calls(B, d, V):
    print(f"fp8 lmhead x{CALLS} B={B} d={d} V={V}", flush=True)
    cases = [_fp8_case(B, d, V, seed=s) for s in (B + d, B + d + 1)]
    h = [runner.to_dev(r["h"]) for r in cases]
    W = [runner.to_dev(r["W"]) for r in cases]
    sc = [runner.to_dev(r["w_scale"]) for r in cases]
    refs = [oracle.lmhead_conf_fp8(r["h"], r["W"], r["w_scale"]) for r in cases]
    wsb = bd.bd_lmhead_conf_fp8_ws_bytes(B, d, V)
    ws = runner.workspace(wsb)
    outs = [(torch.empty(B, device="cuda"), torch.empty(B, dtype=torch.int32, device="cuda"))
            for _ in range(CALLS)]
    for i, (conf, am) in enumerate(outs):
        st = bd.bd_lmhead_conf_fp8(h[i % 2], W[i % 2], sc[i % 2], B, d, V, conf, am, ws, wsb)
        assert st == bd.BD_OK
    torch.cuda.synchronize()
    _check_calls(outs, refs)
