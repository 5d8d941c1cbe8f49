"""The decode step captured as a HIP graph (as the benchmark runs it): every
replay, with eager work and synchronisations between replays, must reproduce
the eager step bit for bit."""
import numpy as np
import pytest
import torch

from block_diffusion_vlm_amd import runner, synth

pytestmark = pytest.mark.gpu


def _snapshot(step):
    return {"tokens": step.tokens.clone(), "masked": step.masked.clone(),
            "n": step.n_committed.clone(), "conf": step.lm.conf.clone(),
            "argmax": step.lm.argmax.clone(), "attn": step.attn.out.clone()}


@pytest.mark.parametrize("workload", ["bf16", "fp8"])
def test_decode_step_graph_replays_match_eager(workload):
    gen = synth.qwen_decode if workload == "bf16" else synth.qwen_decode_fp8
    r = gen(V=30011, B=16)
    step = runner.DecodeStep(r)
    step.reset()
    step.run()
    torch.cuda.synchronize()
    ref = _snapshot(step)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.reset()
        step.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.reset()
        step.run()
    torch.cuda.synchronize()

    other = runner.DecodeStep(gen(seed=7, V=30011, B=16))
    for rep in range(4):
        # eager work between replays that dirties the step's buffers
        step.tokens.fill_(-5)
        step.masked.fill_(1)
        step.lm.conf.zero_()
        other.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(step)
        for k, v in ref.items():
            assert torch.equal(got[k], v), (rep, k)


def test_multi_slot_graph_matches_eager_on_every_slot():
    # One restore of all block-state copies, then one step per copy, as the
    # benchmark captures it: every copy must end as the eager step leaves its
    # state, on every replay.
    r = synth.qwen_decode(V=30011, B=16)
    S = 4
    step = runner.DecodeStep(r, slots=S)
    step.reset()
    step.run(slot=0)
    torch.cuda.synchronize()
    ref_tokens = step.tokens_slots[0].clone()
    ref_masked = step.masked_slots[0].clone()
    ref_n = step.n_committed.clone()
    # the untouched copies still hold the initial state
    for i in range(1, S):
        assert torch.equal(step.masked_slots[i], torch.as_tensor(
            np.asarray(r["masked"], np.uint8), device="cuda"))

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.reset()
        step.run(slot=0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.reset()
        for i in range(S):
            step.run(slot=i)
    torch.cuda.synchronize()
    for rep in range(3):
        step.state.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(S):
            assert torch.equal(step.tokens_slots[i], ref_tokens), (rep, i)
            assert torch.equal(step.masked_slots[i], ref_masked), (rep, i)
        assert torch.equal(step.n_committed, ref_n), rep
