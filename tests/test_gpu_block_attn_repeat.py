"""Block attention called back to back on one workspace (run on an MI355X).

Each call's split kernel writes per-split partial states into the workspace
and its merge kernel reads them back.  These tests alternate inputs and
shapes on one workspace with no synchronisation between the calls, and check
every output against the oracle (bf16: 2e-2 absolute) and repeated inputs for
identical bits: no call may see another's partials.  [Fast-dVLM overview
§1.2]
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth

pytestmark = pytest.mark.gpu

KINDS = {bd.BD_MASK_BIDIR: "bidir", bd.BD_MASK_CAUSAL: "causal",
         bd.BD_MASK_SPEC_FUSED: "spec_fused"}


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def _case(seed, Bq, P, Hq, Hkv, kind):
    r = synth.qwen_decode(seed=seed, B=Bq, n_vis=P - P // 5, n_prompt=P // 5, Hq=Hq, Hkv=Hkv,
                          V=64, d=128)
    ref = oracle.block_attn(r["q"], r["k_cache"], r["v_cache"], r["P"],
                            oracle.intra_block_mask(KINDS[kind], Bq))
    return r, ref


@pytest.mark.parametrize("Bq,P,Hq,Hkv,kind", [(16, 1280, 16, 2, bd.BD_MASK_BIDIR),
                                               (32, 4608, 16, 2, bd.BD_MASK_SPEC_FUSED)])
def test_alternating_inputs_back_to_back(Bq, P, Hq, Hkv, kind):
    print(f"block attention x24 Bq={Bq} P={P}", flush=True)
    cases = [_case(s, Bq, P, Hq, Hkv, kind) for s in (5, 6)]
    dev = [(runner.to_dev(r["q"]), runner.to_dev(r["k_cache"]), runner.to_dev(r["v_cache"]))
           for r, _ in cases]
    mask = runner.mask_dev(kind, Bq)
    wsb = bd.bd_block_attn_ws_bytes(P, Bq, Hq, Hkv, 128)
    ws = runner.workspace(wsb)
    outs = [torch.empty((Bq, Hq, 128), dtype=torch.bfloat16, device="cuda") for _ in range(24)]
    cap = P + Bq
    for i, o in enumerate(outs):
        qd, kd, vd = dev[i % 2]
        bd.bd_block_attn(bd.BD_BF16, qd, kd, vd, P, cap, mask, Bq, Hq, Hkv, 128, 0.0, o, ws, wsb)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        err = np.abs(oracle.widen(runner.to_host(o)) - cases[i % 2][1]).max()
        assert err <= 2e-2, (i, err)
        assert torch.equal(o, outs[i % 2]), i          # deterministic


def test_alternating_shapes_on_one_workspace():
    shapes = [(16, 1280, 16, 2, bd.BD_MASK_BIDIR), (32, 4608, 16, 2, bd.BD_MASK_SPEC_FUSED),
              (5, 300, 6, 3, bd.BD_MASK_CAUSAL), (64, 700, 8, 1, bd.BD_MASK_BIDIR),
              (1, 0, 2, 1, bd.BD_MASK_BIDIR)]
    print("block attention, five shapes on one workspace, twice", flush=True)
    wsb = max(bd.bd_block_attn_ws_bytes(P, Bq, Hq, Hkv, 128) for Bq, P, Hq, Hkv, _ in shapes)
    ws = runner.workspace(wsb)
    runs = []
    for rep in range(2):
        for j, (Bq, P, Hq, Hkv, kind) in enumerate(shapes):
            r, ref = _case(100 + j, Bq, P, Hq, Hkv, kind)
            qd, kd, vd = runner.to_dev(r["q"]), runner.to_dev(r["k_cache"]), \
                runner.to_dev(r["v_cache"])
            o = torch.empty((Bq, Hq, 128), dtype=torch.bfloat16, device="cuda")
            bd.bd_block_attn(bd.BD_BF16, qd, kd, vd, P, r["cap"], runner.mask_dev(kind, Bq), Bq,
                             Hq, Hkv, 128, 0.0, o, ws, wsb)
            runs.append((o, ref, (qd, kd, vd)))
    torch.cuda.synchronize()
    for i, (o, ref, _) in enumerate(runs):
        err = np.abs(oracle.widen(runner.to_host(o)) - ref).max()
        assert err <= 2e-2, (i, err)
