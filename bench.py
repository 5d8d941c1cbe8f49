"""Benchmark of the block-diffusion decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads LIST]

A step is one threshold (MDM) block-decode step of the Qwen2.5-VL-3B-shaped
workload: bd_block_attn (16 block queries, bidirectional block, over a
1024-visual + 256-prompt KV prefix; 16 query / 2 KV heads, head_dim 128) ->
bd_lmhead_conf (hidden 2048 x vocabulary 151936, bf16) -> bd_commit
(threshold 0.9), plus the restore of the block state so that every step does
the same work.  Inputs are seeded synthetic tensors already resident in HBM;
S consecutive steps (at most 25 by default) are captured as one HIP graph,
which is replayed K/S times between HIP events (S is the largest divisor of
K up to --graph-steps and K/4, so that exactly K steps are timed in at least
a few replays when K allows).  Each of the S
steps of a graph works on its own copy of the block state, and one device
copy at the head of the graph restores all S copies, so that every step
starts from the same state.
One JSON line is printed.  ``--workloads`` selects the secondary workloads
(comma-separated among fp8, loop, train, attn, spec; "all" or "none"), so
that a profiled run can be cut to the kernels it is about.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "block decode steps/s + committed tok/s (B=16, 1280-tok prefix); % peak HBM GB/s"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published peak
PROFILE_DIR = ROOT / "profiles"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=400,
                    help="untimed steps first (~43 ms of work: the clocks settle)")
    ap.add_argument("--graph-steps", type=int, default=25,
                    help="at most this many decode steps per HIP graph (a divisor of --steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workloads", default="all",
                    help="secondary workloads: all, none, or a comma list of " + ",".join(SECTIONS))
    ap.add_argument("--no-secondary", action="store_true", help="same as --workloads none")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="approximate CPU time budget of the oracle baseline samples")
    a = ap.parse_args()
    if a.no_secondary or a.workloads == "none":
        a.sections = set()
    elif a.workloads == "all":
        a.sections = set(SECTIONS)
    else:
        a.sections = {w.strip() for w in a.workloads.split(",") if w.strip()}
        bad = a.sections - set(SECTIONS)
        if bad:
            ap.error(f"unknown workloads {sorted(bad)}")
    return a


SECTIONS = ("fp8", "loop", "train", "attn", "spec")


def graph_divisor(K, cap):
    """Largest divisor of K that is at most cap (steps per captured graph)."""
    for s in range(min(cap, K), 0, -1):
        if K % s == 0:
            return s
    return 1


def headline_steps_per_graph(K, cap):
    """Steps per captured graph of the headline: the largest divisor of K not
    above cap nor K / 4, so that a short run still times several replays.
    The host writes a replay's dispatches while the first of them already
    waits, so with a single timed replay that wait is inside the timed region
    (20 steps on one box: 9,245-9,320 steps/s as 4 replays of 5 against
    9,143-9,277 as one of 20); long runs keep up to cap steps per replay."""
    return graph_divisor(K, max(1, min(cap, K // 4)))


def timed(fn, iters, warmup, stream):
    """Average ms per call of fn() (launching on `stream`), HIP events on it."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def traffic_from_profile(kind: str):
    """HBM bytes per LM-head call (kind "bf16" or "fp8") from the committed
    counter summary, if it was taken on the current kernel source; else None."""
    from block_diffusion_vlm_amd.rocprof_summary import LMHEAD_KINDS, source_sha
    kernel_hash = source_sha(LMHEAD_KINDS[kind][1])
    f = PROFILE_DIR / ("lmhead_qwen_decode_pmc.json" if kind == "bf16"
                       else "lmhead_fp8_qwen_decode_pmc.json")
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
    except ValueError:
        return None
    if d.get("kernel_source_sha") != kernel_hash:
        return None
    return d.get("hbm_bytes_per_call")


def step_bytes(inp):
    """Algorithmic bytes (each byte the step must touch once) of the LM head
    and of the whole decode step.  FP8 weights take one byte per entry plus
    one float32 scale per vocabulary row."""
    B, P, Hq, Hkv, dh, d, V = (inp[k] for k in ("B", "P", "Hq", "Hkv", "dh", "d", "V"))
    b_W = V * d + 4 * V if inp["dtype"] == "fp8" else V * d * 2
    b_lm = b_W + B * d * 2 + B * 8
    b_kv = 2 * Hkv * (P + B) * dh * 2
    b_attn = b_kv + 2 * B * Hq * dh * 2
    b_commit = B * (4 + 4 + 1 + 4) + B * (1 + 4) + 4
    return b_lm, b_lm + b_attn + b_commit


def graph_ms_per_step(step, S, reps, warm, stream):
    """Capture one restore of the S block states + S steps (one per state)
    as one graph, replay it `reps` times between HIP events, check every
    state against an eager step, and return (ms per step, commits per step)."""
    import torch
    step.reset()
    step.run()
    torch.cuda.synchronize()
    n_commit = int(step.n_committed.item())
    tokens_ref = step.tokens.clone()

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step.reset()
        step.run()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.reset()
        for i in range(S):
            step.run(slot=i)
    torch.cuda.synchronize()

    ms = timed(graph.replay, reps, warm, stream) / S
    torch.cuda.synchronize()
    for i in range(S):
        assert torch.equal(step.tokens_slots[i], tokens_ref), "graph replay diverged"
    assert int(step.n_committed.item()) == n_commit
    return ms, n_commit


def _cpu_model():
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _time_reps(fn, budget_s, max_reps=50):
    """(reps, seconds) of back-to-back fn() calls, at least one, until the
    budget is spent."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= max_reps:
            return n, el


def cpu_baseline(inp, others, budget_s):
    """The oracle (float64 NumPy) on the same inputs, timed on the host cores
    of the machine that holds the GPU: the headline decode step with every
    core and with one thread (BLAS threads limited through threadpoolctl;
    the rest of the oracle is single-threaded NumPy), and one bounded sample
    of each other workload with every core.  `others` holds the other
    workloads' inputs where the secondary section already drew them."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    from block_diffusion_vlm_amd import synth
    cores = len(os.sched_getaffinity(0))
    tau = float(np.float32(0.9))

    def decode():
        oracle.decode_step(inp["q"], inp["k_cache"], inp["v_cache"], inp["P"], inp["h"],
                           inp["W"], inp["masked"], inp["tokens"], tau)

    with threadpool_limits(limits=cores):
        n_all, t_all = _time_reps(decode, 0.3 * budget_s)
    with threadpool_limits(limits=1):
        n_one, t_one = _time_reps(decode, 0.25 * budget_s)
    res = {"value": n_all / t_all, "unit": "steps/s", "cores": cores, "kind": "oracle",
           "sample": f"{n_all} full decode steps of the headline workload (block attention, "
                     f"LM head over all 151936 rows, commit) in {t_all:.1f} s with "
                     f"{cores} BLAS threads",
           "cpu_model": _cpu_model(), "host_cores": cores,
           "single_thread": {"value": n_one / t_one, "unit": "steps/s", "cores": 1,
                             "sample": f"{n_one} decode steps in {t_one:.1f} s"}}
    cfg = {}
    with threadpool_limits(limits=cores):
        t = synth.tiny()
        n, el = _time_reps(lambda: (
            oracle.decode_step(t["q"], t["k_cache"], t["v_cache"], t["P"], t["h"], t["W"],
                               t["masked"], t["tokens"], tau),
            oracle.dualstream_attn(t["ds_q"], t["ds_k"], t["ds_v"], 4, 4, 2)), 0.03 * budget_s,
            max_reps=1000)
        cfg["tiny_f32"] = {"value": round(el / n * 1e6, 1), "unit": "us per decode step + "
                           "dual-stream attention", "sample": f"{n} reps"}
        r3 = others.get("linear") or synth.linear_spec()
        n, el = _time_reps(lambda: oracle.linear_spec_step(
            r3["q_draft"], r3["k_draft"], r3["v_draft"], r3["q_verify"], r3["k_verify"],
            r3["v_verify"], r3["P"], r3["h_draft"], r3["h_verify"], r3["W"]), 0.1 * budget_s)
        cfg["linear_spec_step"] = {"value": n / el, "unit": "spec-steps/s",
                                   "sample": f"{n} steps in {el:.1f} s"}
        r4 = others.get("fused") or synth.fused_spec()

        def fused():
            oracle.fused_spec_step(r4["q"], r4["k_cache"], r4["v_cache"], r4["P"], r4["h"],
                                   r4["W"], r4["draft_in"])
            oracle.cert_scan(r4["anchor_conf"], r4["anchor_tok"], r4["text_tok"], r4["k_cert"])
        n, el = _time_reps(fused, 0.1 * budget_s)
        cfg["fused_spec_step"] = {"value": n / el, "unit": "steps/s (with certificate)",
                                  "sample": f"{n} steps in {el:.1f} s"}
        r5 = others.get("dualstream") or synth.dualstream()
        nh = 2
        t0 = time.perf_counter()
        oracle.dualstream_attn(r5["q"][:, :nh], r5["k"][:, :nh], r5["v"][:, :nh],
                               r5["n_vis"], r5["n_txt"], r5["block"])
        el = time.perf_counter() - t0
        flops = dualstream_pairs(r5["n_vis"], r5["n_txt"], r5["block"]) * nh * 4 * r5["dh"]
        cfg["dualstream_fwd"] = {"value": flops / el / 1e12, "unit": "TFLOP/s (algorithmic)",
                                 "ms_per_forward": round(el * 1e3 * r5["H"] / nh, 1),
                                 "sample": f"{nh} of {r5['H']} heads in {el:.1f} s, the "
                                           "forward's time scaled by heads"}
    res["configs"] = cfg
    return res


def graph_ms(run, S, reps, warm, stream):
    """ms per call of run() (a stateless composition of library calls),
    captured S times in one HIP graph and replayed `reps` times between HIP
    events after `warm` untimed replays."""
    import torch
    run()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        run()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(S):
            run()
    torch.cuda.synchronize()
    return timed(g.replay, reps, warm, stream) / S


def stream_read_gbs(stream, n_bytes=2 ** 31, grid=256, reps=20):
    """Achievable-bandwidth reference: GB/s of a plain streaming read of
    n_bytes (bd_probe_stream_read), HIP events around `reps` reads."""
    import torch
    from block_diffusion_vlm_amd import bdiff as bd
    buf = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ms = timed(lambda: bd.bd_probe_stream_read(buf, n_bytes, grid, sink), reps, 3, stream)
    del buf
    return n_bytes / (ms * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_diffusion_vlm_amd import bdiff as bd
    from block_diffusion_vlm_amd import runner, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if bd.bd_device_check(0) != bd.BD_OK:
        raise SystemExit("device 0 is not gfx950")
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    inp = synth.qwen_decode()
    K = max(1, args.steps)
    S = headline_steps_per_graph(K, max(1, args.graph_steps))
    step = runner.DecodeStep(inp, slots=S)
    B, P, Hq, Hkv, dh, d, V = (inp[k] for k in ("B", "P", "Hq", "Hkv", "dh", "d", "V"))

    ms_step, n_commit = graph_ms_per_step(step, S, K // S, -(-max(0, args.warmup) // S), stream)
    print(f"headline: {ms_step * 1e3:.2f} us per decode step", file=sys.stderr, flush=True)

    # Dominant kernel: the LM head (its two dispatches), timed alone.
    ms_lm = timed(lambda: step.lm(step.h), K, args.warmup, stream)
    ms_attn = timed(lambda: step.attn(step.q, step.k_cache, step.v_cache), K, args.warmup,
                    stream)

    b_lm, b_step = step_bytes(inp)
    steps_per_s = 1e3 / ms_step
    achieved = b_lm / (ms_lm * 1e-3) / 1e9

    # The block attention with its KV cache read from HBM: 256 copies of the
    # cache (340 MB, more than the 256 MB MALL) visited in turn.
    n_copies = 256
    kc_rot = step.k_cache.unsqueeze(0).repeat(n_copies, 1, 1, 1)
    vc_rot = step.v_cache.unsqueeze(0).repeat(n_copies, 1, 1, 1)
    rot = [0]

    def attn_cold():
        i = rot[0] % n_copies
        rot[0] += 1
        step.attn(step.q, kc_rot[i], vc_rot[i])

    ms_attn_cold = timed(attn_cold, 2 * n_copies, n_copies, stream)
    del kc_rot, vc_rot

    # Plain device copy of known size (calibrates the HBM byte counters in a
    # profiled run of this same command), and the streaming-read reference.
    cal = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device="cuda")
    cal2 = torch.empty_like(cal)
    ms_copy = timed(lambda: cal2.copy_(cal), 20, 3, stream)
    del cal, cal2
    read_gbs = stream_read_gbs(stream)

    out = {
        "metric": METRIC,
        "value": round(steps_per_s, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen2.5-VL-3B-shaped MDM block-decode step", "block": B,
                   "prefix": P, "prefix_visual": inp["n_vis"], "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": dh, "hidden": d, "vocab": V, "threshold": 0.9,
                   "global_batch": 1, "parallelism": "none (1 GPU)"},
        "committed_tok_per_s": round(steps_per_s * n_commit, 1),
        "committed_per_step": n_commit,
        "step_hbm_gbs": round(b_step / (ms_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(b_step / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "steps_per_graph": S,
        "roofline": {"bound": "hbm", "kernel": "bd_lmhead_conf (contraction + merge)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile("bf16"),
                     "us_per_launch": round(ms_lm * 1e3, 2), "bytes_per_launch": b_lm,
                     "frac_of_stream_read": round(achieved / read_gbs, 4)},
        "stream_read_2GiB_GBs": round(read_gbs, 1),
        "kernels_us": {"bd_block_attn": round(ms_attn * 1e3, 2),
                       "bd_block_attn_kv_from_hbm": round(ms_attn_cold * 1e3, 2),
                       "bd_lmhead_conf": round(ms_lm * 1e3, 2),
                       "copy_256MiB_GBs": round(2 * 256 * 2 ** 20 / (ms_copy * 1e-3) / 1e9, 1)},
    }

    others = {}
    if args.sections:
        out["secondary"] = secondary(args, stream, others)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, others, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def dualstream_pairs(n_vis, n_txt, block):
    """Visible (query, key) pairs of one head under the N2N/N2C/C2C masks, in
    closed form: causal clean stream, then per noisy row every visual key, the
    clean text up to its position and its own (possibly ragged) block."""
    ctx = n_vis + n_txt
    full, rem = divmod(n_txt, block)
    n2n = full * block * block + rem * rem
    return ctx * (ctx + 1) // 2 + n_txt * n_vis + n_txt * (n_txt + 1) // 2 + n2n


def secondary(args, stream, others):
    """The other workloads, each timed on its own (not part of `value`), for
    the sections in args.sections; the inputs the CPU baseline reuses are left
    in `others`."""
    import numpy as np
    import torch
    from block_diffusion_vlm_amd import bdiff as bd
    from block_diffusion_vlm_amd import runner, synth
    res = {}
    # These lines are not the headline: each is timed over at least 100 calls
    # after at least 80 untimed ones whatever --steps and --warmup say, since
    # a few calls after a few untimed ones time warm-up effects rather than
    # the workload (the linear speculation step read 236-242 us over 16 steps
    # after 16 untimed ones, against 216 us over 96 after 72, on one box).
    iters = max(100, args.steps // 5)
    warm = max(80, args.warmup // 5)
    S = graph_divisor(8 * max(1, iters // 8), max(1, args.graph_steps))

    def note(name):
        print(f"secondary: {name}", file=sys.stderr, flush=True)

    if "fp8" in args.sections:
        # The same decode step with the FP8 (E4M3, W8A8) LM head, captured
        # and replayed like the headline step.
        note("decode_step_fp8")
        r6 = synth.qwen_decode_fp8()
        st8 = runner.DecodeStep(r6, slots=S)
        ms8, n8 = graph_ms_per_step(st8, S, max(1, iters // S), max(1, warm // S), stream)
        ms_lm8 = timed(lambda: st8.lm(st8.h), iters, warm, stream)
        b_lm8, b_step8 = step_bytes(r6)
        res["decode_step_fp8"] = {
            "us": round(ms8 * 1e3, 2), "steps_per_s": round(1e3 / ms8, 1),
            "committed_per_step": n8,
            "hbm_frac": round(b_step8 / (ms8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "lmhead_us": round(ms_lm8 * 1e3, 2),
            "lmhead_gbs": round(b_lm8 / (ms_lm8 * 1e-3) / 1e9, 1),
            "lmhead_hbm_frac": round(b_lm8 / (ms_lm8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "lmhead_bytes": b_lm8,
            "lmhead_traffic": traffic_from_profile("fp8"),
            "shape": "the headline step with E4M3 weights (one float32 scale per row) and "
                     "per-position E4M3 activations"}
        del st8, r6

    if "loop" in args.sections:
        # Whole blocks: the device-resident loop (up to 16 steps enqueued, the
        # steps that run decided on the device), bf16 and FP8 LM heads.
        for fp8 in (False, True):
            note("block_loop" + ("_fp8" if fp8 else ""))
            rl = synth.qwen_block_loop(fp8=fp8)
            loop = runner.BlockLoop(rl)
            loop.reset()
            loop.run()
            torch.cuda.synchronize()
            n_steps = int(loop.n_steps.item())
            tok_ref = loop.tokens.clone()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                loop.reset()
                loop.run()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                loop.reset()
                loop.run()
            torch.cuda.synchronize()
            ms = timed(g.replay, max(5, iters // 8), 2, stream)
            torch.cuda.synchronize()
            assert torch.equal(loop.tokens, tok_ref) and int(loop.n_steps.item()) == n_steps
            committed = int(np.asarray(rl["masked"]).sum())
            res["block_loop_fp8" if fp8 else "block_loop"] = {
                "us_per_block": round(ms * 1e3, 2), "steps": n_steps, "max_steps": loop.S,
                "committed_per_block": committed,
                "committed_tok_per_s": round(committed / (ms * 1e-3), 1),
                "us_per_step": round(ms * 1e3 / n_steps, 2),
                "shape": "one 16-position block of the Qwen-shaped decode, planted to finish "
                         "in 8 steps"}
            del loop, rl, g

        # Several blocks in a row (bd_decode_blocks): each block's K/V rows
        # join the cache at a device-side kv_len, an AR seed step gives its
        # first token, and up to B - 1 = 15 denoising steps (enough for any
        # block) are enqueued; one graph per call.  With the bf16 and with
        # the FP8 (E4M3 W8A8) LM head.
        for key, fp8 in (("decode_blocks", False), ("decode_blocks_fp8", True)):
            note(key)
            rb = synth.qwen_decode_blocks(fp8=fp8)
            wsc = runner.to_dev(rb["w_scale"]) if fp8 else None
            run = runner.DecodeBlocks(rb, w_scale=wsc)
            run.reset()
            run.run()
            torch.cuda.synchronize()
            steps_run = run.n_steps.cpu().numpy().tolist()
            tok_ref = run.tokens.clone()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                run.reset()
                run.run()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run.reset()
                run.run()
            torch.cuda.synchronize()
            ms = timed(g.replay, max(3, iters // 32), 1, stream)
            torch.cuda.synchronize()
            assert torch.equal(run.tokens, tok_ref)
            assert int(run.kv_len.item()) == rb["P0"] + rb["n_blocks"] * rb["B"]
            nb = rb["n_blocks"]
            toks = nb * rb["B"]                  # the seed and 15 commits per block
            res[key] = {
                "us_per_call": round(ms * 1e3, 2), "blocks": nb,
                "us_per_block": round(ms * 1e3 / nb, 2), "steps_per_block": steps_run,
                "max_steps": run.S, "tokens": toks,
                "committed_tok_per_s": round(toks / (ms * 1e-3), 1),
                "shape": "4 blocks of 16 after a 1024 + 256 token prefix, each seeded by an AR "
                         "step (one query over the prefix + the LM head) and planted to finish "
                         "in 8 steps; KV rows appended at a device-side kv_len"
                         + ("; E4M3 LM-head weights with one scale per row" if fp8 else "")}
            del run, rb, g, wsc

    if "train" in args.sections:
        # The training attention is compute-bound: its clock settles only
        # after some tens of milliseconds of back-to-back calls, so these two
        # lines warm up for 300 calls and time the steady state.
        warm_train = max(warm, 300)
        note("dualstream_fwd")
        r5 = synth.dualstream()
        others["dualstream"] = r5
        ds = runner.DualStream(r5)
        ms = timed(ds.run, iters, warm_train, stream)
        flops = dualstream_pairs(r5["n_vis"], r5["n_txt"], r5["block"]) * r5["H"] * 4 * r5["dh"]
        res["dualstream_fwd"] = {
            "us": round(ms * 1e3, 2), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "algorithmic_gflop": round(flops / 1e9, 2),
            "shape": "1024 vis + 2048 clean + 2048 noisy, block 32, 16 heads x 128"}
        del ds
        # Training backward on the same input: dQ, dK, dV from the forward's
        # output and row log-sum-exp.  Algorithmic work = 2.5x the forward's
        # (dV, dP, dQ, dK products and one recomputation of S).
        note("dualstream_bwd")
        tr = runner.DualStreamTrain(r5)
        tr.forward()
        ms_b = timed(tr.backward, iters, warm_train, stream)
        bflops = 2.5 * flops
        res["dualstream_bwd"] = {
            "us": round(ms_b * 1e3, 2), "tflops": round(bflops / (ms_b * 1e-3) / 1e12, 1),
            "mfma_frac": round(bflops / (ms_b * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "shape": "the dual-stream forward's input, output gradient N(0,1)"}
        del tr

    if "attn" in args.sections:
        # Block attention of the decode step over a paged KV cache (16-token
        # pages in shuffled order), full prefix and TEXT-ONLY (visual keys
        # left out), beside the contiguous cache.
        note("block_attn_paged")
        rq = synth.qwen_decode(V=64, d=128)
        B, P, Hq, Hkv = rq["B"], rq["P"], rq["Hq"], rq["Hkv"]
        n = P + B
        ps = 16
        n_pages = -(-n // ps) + 8
        rng = np.random.default_rng(0)
        table = rng.permutation(n_pages)[:-(-n // ps)].astype(np.int32)
        pools = []
        for cache in (rq["k_cache"], rq["v_cache"]):
            pool = np.zeros((n_pages, Hkv, ps, 128), np.uint16)
            for j in range(n):
                pool[table[j // ps], :, j % ps] = cache[:, j]
            pools.append(runner.to_dev(pool))
        tab = runner.to_dev(table)
        qd = runner.to_dev(rq["q"])
        mask = runner.mask_dev(bd.BD_MASK_BIDIR, B)
        out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
        pa = {}
        for key_lo in (0, rq["n_vis"]):
            wsb = bd.bd_block_attn_ws_bytes(P - key_lo, B, Hq, Hkv, 128)
            ws = runner.workspace(wsb)
            ms = timed(lambda: bd.bd_block_attn_paged(qd, pools[0], pools[1], tab, ps, n_pages,
                                                      P, key_lo, mask, B, Hq, Hkv, 128, 0.0,
                                                      out, ws, wsb), iters, warm, stream)
            pa["us_full_prefix" if key_lo == 0 else "us_text_only"] = round(ms * 1e3, 2)
        ba = runner.BlockAttn(bd.BD_BF16, bd.BD_MASK_BIDIR, B, P, rq["cap"], Hq, Hkv, 128)
        kc, vc = runner.to_dev(rq["k_cache"]), runner.to_dev(rq["v_cache"])
        ms = timed(lambda: ba(qd, kc, vc), iters, warm, stream)
        pa["us_contiguous"] = round(ms * 1e3, 2)
        pa["shape"] = "the decode step's block attention, 16-token pages in shuffled order"
        res["block_attn_paged"] = pa
        del pools, ba, kc, vc

        # Block attention of the decode step over an FP8 (E4M3) KV cache with
        # per-head scales, and the quantizer writing the block's own K/V rows.
        note("block_attn_fp8kv")
        rf = synth.qwen_decode_fp8kv()
        B, P, cap, Hq, Hkv = rf["B"], rf["P"], rf["cap"], rf["Hq"], rf["Hkv"]
        att8 = runner.BlockAttnFP8KV(bd.BD_MASK_BIDIR, B, P, cap, Hq, Hkv)
        q8 = runner.to_dev(rf["q"])
        kc8, vc8 = runner.to_dev(rf["k_codes"]), runner.to_dev(rf["v_codes"])
        ks8, vs8 = runner.to_dev(rf["k_scale"]), runner.to_dev(rf["v_scale"])
        kn8 = runner.to_dev(rf["k_new"])
        ms = timed(lambda: att8(q8, kc8, vc8, ks8, vs8), iters, warm, stream)
        ms_q = timed(lambda: bd.bd_kv_quant_fp8(kn8, B, Hkv, 128, ks8, kc8, cap, P), iters,
                     warm, stream)
        kv_bytes = 2 * Hkv * (P + B) * 128
        res["block_attn_fp8kv"] = {
            "us": round(ms * 1e3, 2), "kv_bytes": kv_bytes,
            "us_bf16_cache": pa["us_contiguous"], "us_quant_block_rows": round(ms_q * 1e3, 2),
            "shape": "the decode step's block attention, E4M3 K/V (one byte per entry) "
                     "with per-head scales"}
        del att8, kc8, vc8

    if "spec" in args.sections:
        # Both speculation steps are captured S at a time in one HIP graph,
        # as the headline step is.
        note("linear_spec_step")
        r3 = synth.linear_spec()
        others["linear"] = r3
        lin = runner.LinearSpecStep(r3)
        lin.run()
        torch.cuda.synchronize()
        L = int(lin.accepted.item())
        ms = graph_ms(lin.run, S, max(1, iters // S), max(1, warm // S), stream)
        torch.cuda.synchronize()
        assert int(lin.accepted.item()) == L
        b = 2 * (r3["V"] * r3["d"] * 2 + 2 * r3["Hkv"] * r3["cap"] * r3["dh"] * 2)
        ms_attn = timed(lambda: lin.attn_d(lin.t["q_draft"], lin.t["k_draft"], lin.t["v_draft"]),
                        iters, warm, stream)
        res["linear_spec_step"] = {"us": round(ms * 1e3, 2), "accepted": L,
                                   "accepted_tok_per_s": round(L / (ms * 1e-3), 1),
                                   "hbm_frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "attn_us": round(ms_attn * 1e3, 2), "bytes": b}
        del lin

        note("fused_spec_step")
        r4 = synth.fused_spec()
        others["fused"] = r4
        fu = runner.FusedSpecStep(r4)
        fu.run()
        torch.cuda.synchronize()
        acc, cert = int(fu.accepted.item()), int(fu.cert_L.item())
        ms = graph_ms(fu.run, S, max(1, iters // S), max(1, warm // S), stream)
        torch.cuda.synchronize()
        assert int(fu.accepted.item()) == acc and int(fu.cert_L.item()) == cert
        b = r4["V"] * r4["d"] * 2 + 2 * r4["Hkv"] * r4["cap"] * r4["dh"] * 2
        ms_attn = timed(lambda: fu.attn(fu.t["q"], fu.t["k_cache"], fu.t["v_cache"]), iters,
                        warm, stream)
        res["fused_spec_step"] = {"us": round(ms * 1e3, 2), "accepted": acc,
                                  "cert_accepted": cert,
                                  "hbm_frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "attn_us": round(ms_attn * 1e3, 2), "bytes": b}
        del fu
    return res


if __name__ == "__main__":
    main()
