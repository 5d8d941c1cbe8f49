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


def test_decode_step_graph_replays_match_eager():
    r = synth.qwen_decode(V=30011, B=16)
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

    other = runner.DecodeStep(synth.qwen_decode(seed=7, V=30011, B=16))
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
