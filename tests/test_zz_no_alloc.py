"""bd_lmhead_conf_noalloc (the LM-head call whose scratch is a static device
array of the library) against bd_lmhead_conf with a caller workspace, through
the C ABI on an MI355X: conf and argmax bit-identical, argmax equal to the
oracle's, on consecutive calls that shrink (the array keeps the previous
call's partials, which must not leak into the next result)."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth
from oracle.guards import row_guard

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def _pair(dt, h, W, B, d, V):
    """(conf, argmax) from the no-alloc call and from bd_lmhead_conf."""
    conf = torch.full((B,), -1.0, dtype=torch.float32, device="cuda")
    arg = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    bd.bd_lmhead_conf_noalloc(dt, h, W, B, d, V, conf, arg)
    lm = runner.LMHead(dt, W, B, d, V)
    lm(h)
    torch.cuda.synchronize()
    return (conf.cpu().numpy(), arg.cpu().numpy()), (lm.conf.cpu().numpy(),
                                                     lm.argmax.cpu().numpy())


def _bf16_case(B, d, V, seed):
    r = synth.qwen_decode(seed=seed, B=B, d=d, V=V, n_vis=4, n_prompt=4, Hq=2, Hkv=1,
                          guard=row_guard())
    return r, runner.to_dev(r["h"]), runner.to_dev(r["W"])


def test_noalloc_matches_workspace_call_on_shrinking_calls():
    # the Qwen-shaped LM head first, then a smaller one on the same array
    for B, d, V, seed in ((16, 2048, 151936, 11), (5, 256, 1000, 12)):
        print(f"noalloc bf16 B={B} d={d} V={V}", flush=True)
        r, h, W = _bf16_case(B, d, V, seed)
        (c0, a0), (c1, a1) = _pair(bd.BD_BF16, h, W, B, d, V)
        assert np.array_equal(a0, a1) and np.array_equal(c0, c1)
        oc, oa = oracle.lmhead_conf(r["h"], r["W"])
        assert np.array_equal(a0, oa)
        assert np.abs(c0 / oc - 1).max() <= 1e-4


def test_noalloc_float32_then_bf16_again():
    print("noalloc f32 tiny, then bf16", flush=True)
    t = synth.tiny()
    h, W = runner.to_dev(t["h"]), runner.to_dev(t["W"])
    (c0, a0), (c1, a1) = _pair(bd.BD_F32, h, W, t["B"], t["d"], t["V"])
    assert np.array_equal(a0, a1) and np.array_equal(c0, c1)
    oc, oa = oracle.lmhead_conf(t["h"], t["W"])
    assert np.array_equal(a0, oa)
    assert np.abs(c0 / oc - 1).max() <= 1e-5
    r, h, W = _bf16_case(33, 384, 999, 13)
    (c0, a0), (c1, a1) = _pair(bd.BD_BF16, h, W, 33, 384, 999)
    assert np.array_equal(a0, a1) and np.array_equal(c0, c1)


def test_noalloc_rejects_oversized_float32_shape():
    h = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    W = torch.zeros((65537, 16), dtype=torch.float32, device="cuda")
    conf = torch.empty(64, dtype=torch.float32, device="cuda")
    arg = torch.empty(64, dtype=torch.int32, device="cuda")
    st = bd.bd_lmhead_conf_noalloc(bd.BD_F32, h, W, 64, 16, 65537, conf, arg, check=False)
    assert st == bd.BD_E_WORKSPACE
