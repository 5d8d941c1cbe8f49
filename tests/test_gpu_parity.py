"""GPU-vs-oracle parity through the C ABI (run on an MI355X).

Integer results (committed tokens and flags, n_committed, argmax, accepted
length, KV length, certificate order/length/flag) must be bit-exact.
Floating point: float32 outputs within 1e-5 relative (max abs error over max
abs reference); bf16 attention outputs within 2e-2 absolute (the output is
stored in bf16; |o| <= 4 because V is truncated at 4); the LM-head confidence
within 1e-4 relative (informational: commits are decided on it, and the
inputs keep every confidence at least 1e-3 from the threshold).
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth
from oracle.guards import lmhead_margins, row_guard

pytestmark = pytest.mark.gpu

TAU32 = float(np.float32(0.9))


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def rel_err(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    return np.abs(g - r).max() / max(np.abs(r).max(), 1e-30)


def bf16_host(t):
    return oracle.widen(runner.to_host(t))


# ---------------------------------------------------------------------------
# commit / accept / certificate
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B", [0, 1, 5, 16, 33, 64])
def test_commit_matches_oracle(B):
    rng = np.random.default_rng(100 + B)
    grid = np.array([0.1, 0.5, 0.899, TAU32, np.nextafter(np.float32(TAU32), np.float32(1)),
                     0.95, 0.95, 1.0], np.float32)
    for trial in range(40):
        conf = rng.choice(grid, B).astype(np.float32) if trial % 2 else \
            rng.random(B, dtype=np.float32)
        argmax = rng.integers(0, 151936, B).astype(np.int32)
        masked = (rng.random(B) < (0.2 if trial % 3 == 0 else 0.8)).astype(np.uint8)
        tokens = rng.integers(0, 1000, B).astype(np.int32)
        d = {k: runner.to_dev(v) if B else torch.zeros(1, dtype=t, device="cuda")
             for (k, v), t in zip(dict(conf=conf, argmax=argmax, masked=masked,
                                       tokens=tokens).items(),
                                  (torch.float32, torch.int32, torch.uint8, torch.int32))}
        n = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        bd.bd_commit(d["conf"], d["argmax"], B, TAU32, d["masked"], d["tokens"], n)
        torch.cuda.synchronize()
        m2, t2, nc = oracle.commit(conf, argmax, masked, tokens, TAU32)
        assert int(n.item()) == nc
        if B:
            assert np.array_equal(runner.to_host(d["masked"]), m2)
            assert np.array_equal(runner.to_host(d["tokens"]), t2)


@pytest.mark.parametrize("bonus", [False, True])
@pytest.mark.parametrize("B", [0, 1, 7, 16, 32, 64])
def test_spec_accept_matches_oracle(B, bonus):
    rng = np.random.default_rng(200 + B)
    call = bd.bd_spec_accept_bonus if bonus else bd.bd_spec_accept
    for trial in range(30):
        draft = rng.integers(0, 5 if trial % 2 else 151936, B).astype(np.int32)
        verify = draft.copy()
        if B and trial % 5:
            cut = int(rng.integers(0, B))
            verify[cut:] = rng.integers(0, 5, B - cut)
        P = int(rng.integers(0, 5000))
        dd = runner.to_dev(draft) if B else torch.zeros(1, dtype=torch.int32, device="cuda")
        vv = runner.to_dev(verify) if B else torch.zeros(1, dtype=torch.int32, device="cuda")
        acc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        kv = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        out = torch.full((max(B, 1),), -99, dtype=torch.int32, device="cuda")
        call(dd, vv, B, P, acc, kv, out)
        torch.cuda.synchronize()
        n, kvl, toks = oracle.spec_accept(draft, verify, P, bonus=bonus)
        assert int(acc.item()) == n and int(kv.item()) == kvl
        o = runner.to_host(out)
        assert np.array_equal(o[:n], toks) and (o[n:] == -99).all()


@pytest.mark.parametrize("n", [0, 1, 7, 64, 200, 1024])
def test_cert_scan_matches_oracle(n):
    rng = np.random.default_rng(300 + n)
    for trial in range(10):
        if trial % 2:
            conf = rng.choice(np.array([0.1, 0.5, 0.5, 0.9], np.float32), n)
        else:
            conf = rng.random(n, dtype=np.float32)
        at = rng.integers(0, 151936, n).astype(np.int32)
        tt = np.where(rng.random(n) < 0.83 + 0.15 * (trial % 3 == 0), at, at + 1).astype(np.int32)
        k = int(rng.integers(0, 10))
        dev = lambda a, t: runner.to_dev(a) if n else torch.zeros(1, dtype=t, device="cuda")
        c, a_, t_ = dev(conf, torch.float32), dev(at, torch.int32), dev(tt, torch.int32)
        order = torch.full((max(n, 1),), -1, dtype=torch.int32, device="cuda")
        L = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        skip = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        bd.bd_cert_scan(c, a_, t_, n, k, order, L, skip)
        torch.cuda.synchronize()
        o_order, o_L, o_skip = oracle.cert_scan(conf, at, tt, k)
        if n:
            assert np.array_equal(runner.to_host(order), o_order)
        assert int(L.item()) == o_L and int(skip.item()) == o_skip


# ---------------------------------------------------------------------------
# LM head
# ---------------------------------------------------------------------------

def _lmhead_case(B, d, V, seed):
    r = synth.qwen_decode(seed=seed, B=B, d=d, V=V, n_vis=4, n_prompt=4, Hq=2, Hkv=1,
                          guard=row_guard())
    gap, _ = lmhead_margins(r["h"], r["W"])
    assert gap.min() > 1e-2
    return r


@pytest.mark.parametrize("B,d,V", [
    (1, 128, 17), (4, 256, 1000), (16, 512, 4099), (16, 640, 777), (16, 1024, 5000),
    (32, 2048, 20011), (33, 384, 999), (48, 2048, 7001), (64, 2048, 3001),
    (16, 2048, 151936),
    # 17 to 32 positions (two position blocks, folded by different waves)
    # with d = 512 .. 2048: one tile per workgroup (V = 1001), one or two
    # (V = 4097), a ragged vocabulary tail
    (17, 512, 1001), (20, 1536, 4097), (25, 1024, 3000), (31, 2048, 151936),
])
def test_lmhead_bf16_matches_oracle(B, d, V):
    r = _lmhead_case(B, d, V, seed=B * 7 + d + V)
    h, W = runner.to_dev(r["h"]), runner.to_dev(r["W"])
    lm = runner.LMHead(bd.BD_BF16, W, B, d, V)
    lm(h)
    torch.cuda.synchronize()
    conf0, a0 = lm.conf.cpu().numpy().copy(), lm.argmax.cpu().numpy().copy()
    oc, oa = oracle.lmhead_conf(r["h"], r["W"])
    assert np.array_equal(a0, oa)
    assert rel_err(conf0, oc) <= 1e-4 or np.abs(conf0 / oc - 1).max() <= 1e-4
    # Deterministic: a second call on a dirty workspace gives identical bits.
    lm(h)
    torch.cuda.synchronize()
    assert np.array_equal(lm.conf.cpu().numpy(), conf0)
    assert np.array_equal(lm.argmax.cpu().numpy(), a0)


def test_lmhead_workspace_reuse_across_shapes():
    big = _lmhead_case(16, 2048, 30000, 1)
    small = _lmhead_case(5, 256, 333, 2)
    ws = runner.workspace(max(bd.bd_lmhead_conf_ws_bytes(16, 2048, 30000),
                              bd.bd_lmhead_conf_ws_bytes(5, 256, 333)))
    for r in (big, small, big):
        B, d, V = r["h"].shape[0], r["h"].shape[1], r["W"].shape[0]
        conf = torch.empty(B, device="cuda")
        am = torch.empty(B, dtype=torch.int32, device="cuda")
        bd.bd_lmhead_conf(bd.BD_BF16, runner.to_dev(r["h"]), runner.to_dev(r["W"]), B, d, V,
                          conf, am, ws, ws.numel())
        torch.cuda.synchronize()
        oc, oa = oracle.lmhead_conf(r["h"], r["W"])
        assert np.array_equal(am.cpu().numpy(), oa)
        assert np.abs(conf.cpu().numpy() / oc - 1).max() <= 1e-4


def test_lmhead_f32_tiny():
    r = synth.tiny()
    h, W = runner.to_dev(r["h"]), runner.to_dev(r["W"])
    lm = runner.LMHead(bd.BD_F32, W, r["B"], r["d"], r["V"])
    lm(h)
    torch.cuda.synchronize()
    oc, oa = oracle.lmhead_conf(r["h"], r["W"])
    assert np.array_equal(lm.argmax.cpu().numpy(), oa)
    assert rel_err(lm.conf.cpu().numpy(), oc) <= 1e-5


@pytest.mark.parametrize("B,d,V", [(3, 40, 1000), (64, 16, 64), (2, 1, 300)])
def test_lmhead_f32_ragged(B, d, V):
    rng = np.random.default_rng(B + d + V)
    h = rng.standard_normal((B, d)).astype(np.float32)
    W = rng.standard_normal((V, d)).astype(np.float32)
    lm = runner.LMHead(bd.BD_F32, runner.to_dev(W), B, d, V)
    lm(runner.to_dev(h))
    torch.cuda.synchronize()
    oc, oa = oracle.lmhead_conf(h, W)
    gap, _ = lmhead_margins(h, W)
    ok = gap > 1e-4
    assert np.array_equal(lm.argmax.cpu().numpy()[ok], oa[ok])
    assert rel_err(lm.conf.cpu().numpy(), oc) <= 1e-5


@pytest.mark.parametrize("B,d,V,B_acc", [(4, 16, 64, 4), (33, 40, 1000, 17), (64, 16, 700, 64)])
def test_lmhead_conf_accept_f32(B, d, V, B_acc):
    """The float32 LM head with the accept in its merge: argmax and the accept
    bit-exact against the oracle on rows whose top-2 gap exceeds 1e-4."""
    rng = np.random.default_rng(B * 5 + V)
    h = rng.standard_normal((B, d)).astype(np.float32)
    W = rng.standard_normal((V, d)).astype(np.float32)
    oc, oa = oracle.lmhead_conf(h, W)
    gap, _ = lmhead_margins(h, W)
    assert (gap[:B_acc] > 1e-4).all()
    draft = oa[:B_acc].astype(np.int32).copy()
    cut = B_acc // 2
    draft[cut] = (draft[cut] + 1) % V
    lm = runner.LMHead(bd.BD_F32, runner.to_dev(W), B, d, V)
    acc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    kv = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    toks = torch.full((B_acc,), -99, dtype=torch.int32, device="cuda")
    lm.conf_accept(runner.to_dev(h), runner.to_dev(draft), B_acc, 77, acc, kv, toks, bonus=True)
    torch.cuda.synchronize()
    ok = gap > 1e-4
    assert np.array_equal(lm.argmax.cpu().numpy()[ok], oa[ok])
    assert rel_err(lm.conf.cpu().numpy(), oc) <= 1e-5
    n, kvl, ref = oracle.spec_accept(draft, oa[:B_acc].astype(np.int32), 77, bonus=True)
    assert (int(acc.item()), int(kv.item())) == (n, kvl) == (cut + 1, 77 + cut)
    t = runner.to_host(toks)
    assert np.array_equal(t[:n], ref) and (t[n:] == -99).all()


# ---------------------------------------------------------------------------
# Block attention
# ---------------------------------------------------------------------------

def _block_attn_case(Bq, P, Hq, Hkv, kind, seed, dt="bf16", dh=128, extra_cap=3):
    rng = np.random.default_rng(seed)
    cap = P + Bq + extra_cap
    conv = synth.bf16_bits if dt == "bf16" else (lambda x: x)
    q = conv(synth.normal(rng, (Bq, Hq, dh)))
    kc = conv(synth.normal(rng, (Hkv, cap, dh)))
    vc = conv(synth.normal(rng, (Hkv, cap, dh), trunc=4.0))
    code = {"bidir": bd.BD_MASK_BIDIR, "causal": bd.BD_MASK_CAUSAL,
            "spec_fused": bd.BD_MASK_SPEC_FUSED}[kind]
    a = runner.BlockAttn(runner.dtype_code(dt), code, Bq, P, cap, Hq, Hkv, dh)
    a(runner.to_dev(q), runner.to_dev(kc), runner.to_dev(vc))
    torch.cuda.synchronize()
    ref = oracle.block_attn(q, kc, vc, P, oracle.intra_block_mask(kind, Bq))
    got = bf16_host(a.out) if dt == "bf16" else a.out.cpu().numpy()
    return got, ref


@pytest.mark.parametrize("Bq,P,Hq,Hkv,kind", [
    (16, 1280, 16, 2, "bidir"), (32, 1280, 16, 2, "causal"), (32, 1280, 16, 2, "bidir"),
    (32, 4608, 16, 2, "spec_fused"), (5, 70, 4, 1, "causal"), (1, 0, 2, 2, "bidir"),
    (64, 100, 8, 2, "bidir"), (3, 63, 6, 3, "causal"), (2, 1, 1, 1, "spec_fused"),
    (64, 0, 4, 4, "causal"),
    # the largest key count the bf16 path takes: P + Bq = 65536 (1024 splits)
    (16, 65520, 2, 1, "causal"),
])
def test_block_attn_bf16_matches_oracle(Bq, P, Hq, Hkv, kind):
    print(f"block attention Bq={Bq} P={P} Hq={Hq} Hkv={Hkv} {kind}", flush=True)
    got, ref = _block_attn_case(Bq, P, Hq, Hkv, kind, seed=Bq * 1000 + P)
    assert np.abs(got - ref).max() <= 2e-2


def test_block_attn_zero_mask_row_outputs_zero():
    # P = 0 and an all-zero mask row: that query sees no key at all.
    Bq, Hq, Hkv, dh = 4, 2, 1, 128
    rng = np.random.default_rng(5)
    q = synth.bf16_bits(synth.normal(rng, (Bq, Hq, dh)))
    kc = synth.bf16_bits(synth.normal(rng, (Hkv, Bq, dh)))
    vc = synth.bf16_bits(synth.normal(rng, (Hkv, Bq, dh), trunc=4.0))
    rows = bd.bd_make_intra_mask(bd.BD_MASK_CAUSAL, Bq)
    rows[2] = 0
    a = runner.BlockAttn(bd.BD_BF16, bd.BD_MASK_CAUSAL, Bq, 0, Bq, Hq, Hkv, dh)
    a.mask.copy_(runner.to_dev(rows))
    a(runner.to_dev(q), runner.to_dev(kc), runner.to_dev(vc))
    torch.cuda.synchronize()
    intra = ((rows[:, None] >> np.arange(Bq, dtype=np.uint64)[None]) & np.uint64(1)).astype(bool)
    ref = oracle.block_attn(q, kc, vc, 0, intra)
    got = bf16_host(a.out)
    assert (got[2] == 0).all() and np.abs(got - ref).max() <= 2e-2


@pytest.mark.parametrize("Bq,P,Hq,Hkv,dh,kind", [
    (4, 32, 1, 1, 16, "bidir"), (7, 100, 4, 2, 16, "causal"), (6, 65, 2, 1, 128, "spec_fused"),
])
def test_block_attn_f32_matches_oracle(Bq, P, Hq, Hkv, dh, kind):
    got, ref = _block_attn_case(Bq, P, Hq, Hkv, kind, seed=P, dt="f32", dh=dh)
    assert rel_err(got, ref) <= 1e-5


# ---------------------------------------------------------------------------
# Dual-stream attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n_vis,n_txt,block,H", [
    (64, 96, 32, 2), (5, 37, 4, 1), (0, 70, 8, 1), (100, 0, 4, 2), (128, 128, 32, 1),
    (130, 250, 7, 1), (1, 1, 1, 3),
])
def test_dualstream_bf16_matches_oracle(n_vis, n_txt, block, H):
    r = synth.dualstream(seed=n_vis + n_txt, n_vis=n_vis, n_txt=n_txt, block=block, H=H)
    ds = runner.DualStream(r)
    ds.run()
    torch.cuda.synchronize()
    ref = oracle.dualstream_attn(r["q"], r["k"], r["v"], n_vis, n_txt, block)
    assert np.abs(bf16_host(ds.out) - ref).max() <= 2e-2


@pytest.fixture(scope="module")
def dualstream_full():
    """The training-attention workload at its real size (1024 visual + 2048
    clean + 2048 noisy tokens, block 32, 16 heads x 128), run once."""
    r = synth.dualstream()
    ds = runner.DualStream(r)
    ds.run()
    torch.cuda.synchronize()
    return r, bf16_host(ds.out)


@pytest.mark.parametrize("h0", [0, 4, 8, 12])
def test_dualstream_bf16_full_size(dualstream_full, h0):
    # every row of four heads per case; the four cases cover all 16 heads
    r, got = dualstream_full
    hs = list(range(h0, h0 + 4))
    print(f"dual-stream full size, heads {hs}", flush=True)
    ref = oracle.dualstream_attn(r["q"][:, hs], r["k"][:, hs], r["v"][:, hs], r["n_vis"],
                                 r["n_txt"], r["block"])
    assert np.abs(got[:, hs] - ref).max() <= 2e-2


SEGMENTED = [
    # n_vis, n_txt, block, H, segment starts
    (64, 300, 32, 2, [0, 37, 150, 151, 299]),
    (0, 256, 16, 1, [0, 100]),
    (128, 130, 7, 1, list(range(0, 130, 13))),
    (32, 512, 32, 1, [0] + sorted(np.random.default_rng(9).choice(
        np.arange(1, 512), 63, replace=False).tolist())),
    (1024, 2048, 32, 1, [0, 300, 301, 1000, 1500, 2047]),
]


@pytest.mark.parametrize("n_vis,n_txt,block,H,seg", SEGMENTED)
def test_dualstream_auto_truncation_bf16_matches_oracle(n_vis, n_txt, block, H, seg):
    r = synth.dualstream(seed=n_vis + 3 * n_txt, n_vis=n_vis, n_txt=n_txt, block=block, H=H)
    r["seg_starts"] = seg
    ds = runner.DualStream(r)
    ds.run()
    torch.cuda.synchronize()
    ref = oracle.dualstream_attn(r["q"], r["k"], r["v"], n_vis, n_txt, block, seg_starts=seg)
    assert np.abs(bf16_host(ds.out) - ref).max() <= 2e-2


def test_dualstream_one_segment_equals_plain_call():
    r = synth.dualstream(seed=4, n_vis=64, n_txt=200, block=32, H=2)
    a = runner.DualStream(r)
    a.run()
    r2 = dict(r, seg_starts=[0])
    b = runner.DualStream(r2)
    b.run()
    torch.cuda.synchronize()
    assert torch.equal(a.out, b.out)


def test_dualstream_auto_truncation_f32_tiny():
    r = synth.tiny()
    d = {"dtype": "f32", "n_vis": 4, "n_txt": 4, "block": 2, "H": 1, "dh": 16,
         "q": r["ds_q"], "k": r["ds_k"], "v": r["ds_v"], "seg_starts": [0, 1]}
    ds = runner.DualStream(d)
    ds.run()
    torch.cuda.synchronize()
    ref = oracle.dualstream_attn(r["ds_q"], r["ds_k"], r["ds_v"], 4, 4, 2, seg_starts=[0, 1])
    assert rel_err(ds.out.cpu().numpy(), ref) <= 1e-5


def test_dualstream_f32_tiny():
    r = synth.tiny()
    d = {"dtype": "f32", "n_vis": 4, "n_txt": 4, "block": 2, "H": 1, "dh": 16,
         "q": r["ds_q"], "k": r["ds_k"], "v": r["ds_v"]}
    ds = runner.DualStream(d)
    ds.run()
    torch.cuda.synchronize()
    ref = oracle.dualstream_attn(r["ds_q"], r["ds_k"], r["ds_v"], 4, 4, 2)
    assert rel_err(ds.out.cpu().numpy(), ref) <= 1e-5


# ---------------------------------------------------------------------------
# Compositions at the real sizes
# ---------------------------------------------------------------------------

def _assert_guards(h, W, tau=None, w_scale=None):
    """Every row off the floating-point boundaries: top-2 logit gap > 1e-2 and,
    where commits are decided, |conf - tau| >= 1e-3."""
    gap, dist = lmhead_margins(h, W, tau, w_scale=w_scale)
    assert gap.min() > 1e-2, gap.min()
    if dist is not None:
        assert dist.min() >= 1e-3, dist.min()


def test_decode_step_full_size():
    r = synth.qwen_decode(guard=row_guard(TAU32))
    _assert_guards(r["h"], r["W"], TAU32)
    step = runner.DecodeStep(r)
    step.run()
    torch.cuda.synchronize()
    o = oracle.decode_step(r["q"], r["k_cache"], r["v_cache"], r["P"], r["h"], r["W"],
                           r["masked"], r["tokens"], TAU32)
    assert np.array_equal(step.lm.argmax.cpu().numpy(), o["argmax"])
    assert np.array_equal(runner.to_host(step.masked), o["masked"])
    assert np.array_equal(runner.to_host(step.tokens), o["tokens"])
    assert int(step.n_committed.item()) == o["n_committed"]
    assert np.abs(bf16_host(step.attn.out) - o["attn"]).max() <= 2e-2
    # repeated steps after reset are identical
    step.reset()
    step.run()
    torch.cuda.synchronize()
    assert np.array_equal(runner.to_host(step.tokens), o["tokens"])


@pytest.mark.parametrize("B,d,V", [(1, 128, 1000), (16, 2048, 30011), (24, 2048, 9001),
                                   (33, 384, 999), (64, 2048, 3001)])
def test_lmhead_conf_commit_equals_separate_calls(B, d, V):
    r = synth.qwen_decode(seed=B + V, B=B, d=d, V=V, n_vis=4, n_prompt=4, Hq=2, Hkv=1,
                          guard=row_guard(TAU32))
    _assert_guards(r["h"], r["W"], TAU32)
    h, W = runner.to_dev(r["h"]), runner.to_dev(r["W"])
    masked0 = (np.random.default_rng(B).random(B) < 0.8).astype(np.uint8)
    tokens0 = np.arange(B, dtype=np.int32) + 7
    out = {}
    for fused in (False, True):
        lm = runner.LMHead(bd.BD_BF16, W, B, d, V)
        masked, tokens = runner.to_dev(masked0), runner.to_dev(tokens0)
        n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        if fused:
            bd.bd_lmhead_conf_commit(bd.BD_BF16, h, W, B, d, V, TAU32, lm.conf, lm.argmax, masked,
                                     tokens, n, lm.ws, lm.ws_bytes)
        else:
            lm(h)
            bd.bd_commit(lm.conf, lm.argmax, B, TAU32, masked, tokens, n)
        torch.cuda.synchronize()
        out[fused] = (lm.conf.cpu().numpy(), lm.argmax.cpu().numpy(), runner.to_host(masked),
                      runner.to_host(tokens), int(n.item()))
    for a, b in zip(out[False], out[True]):
        assert np.array_equal(a, b)
    oc, oa = oracle.lmhead_conf(r["h"], r["W"])
    m2, t2, nc = oracle.commit(oc, oa, masked0, tokens0, TAU32)
    assert np.array_equal(out[True][2], m2) and np.array_equal(out[True][3], t2)
    assert out[True][4] == nc


@pytest.mark.parametrize("B,d,V,B_acc,bonus", [
    (1, 128, 1000, 1, False), (16, 2048, 30011, 16, False), (16, 1024, 5000, 9, True),
    (17, 512, 4097, 17, True), (32, 2048, 30011, 16, False), (32, 2048, 9001, 32, True),
    (33, 384, 999, 20, False), (48, 1024, 3001, 48, True), (64, 2048, 3001, 64, False),
    (32, 2048, 151936, 16, True)])
def test_lmhead_conf_accept_equals_separate_calls_and_oracle(B, d, V, B_acc, bonus):
    """bd_lmhead_conf_accept = bd_lmhead_conf + bd_spec_accept(_bonus) on its
    argmax: argmax and the accept outputs bit-exact (against the separate
    calls and the oracle), conf equal bit for bit up to 16 positions and
    within float32 rounding above (the merge order differs there)."""
    r = _lmhead_case(B, d, V, seed=3 * B + d + V)
    h, W = runner.to_dev(r["h"]), runner.to_dev(r["W"])
    oc, oa = oracle.lmhead_conf(r["h"], r["W"])
    rng = np.random.default_rng(B * 31 + B_acc)
    call = bd.bd_spec_accept_bonus if bonus else bd.bd_spec_accept
    for trial in range(4):
        # drafts that agree with the verify argmax up to a planted cut (or all)
        draft = oa[:B_acc].astype(np.int32).copy()
        if trial:
            cut = int(rng.integers(0, B_acc))
            draft[cut:] = (draft[cut:] + 1 + rng.integers(0, 5, B_acc - cut)) % V
        P = int(rng.integers(0, 5000))
        dd = runner.to_dev(draft)
        out = {}
        for fused in (False, True):
            lm = runner.LMHead(bd.BD_BF16, W, B, d, V)
            acc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            kv = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            toks = torch.full((B_acc,), -99, dtype=torch.int32, device="cuda")
            if fused:
                lm.conf_accept(h, dd, B_acc, P, acc, kv, toks, bonus=bonus)
            else:
                lm(h)
                call(dd, lm.argmax, B_acc, P, acc, kv, toks)
            torch.cuda.synchronize()
            out[fused] = (lm.conf.cpu().numpy(), lm.argmax.cpu().numpy(), int(acc.item()),
                          int(kv.item()), runner.to_host(toks))
        c0, a0, n0, k0, t0 = out[False]
        c1, a1, n1, k1, t1 = out[True]
        assert np.array_equal(a1, a0) and np.array_equal(a1, oa)
        if B <= 16:
            assert np.array_equal(c1, c0)
        else:
            # Two fixed-order merges of at most 256 positive partials, each
            # within about (256 + 32) float32 roundings (the sums and the
            # exp2 rescales on a tree of depth 8) of the exact value.
            assert np.abs(c1 / c0 - 1).max() <= 2 * (256 + 32) * 2.0 ** -24
        assert rel_err(c1, oc) <= 1e-4 or np.abs(c1 / oc - 1).max() <= 1e-4
        assert (n1, k1) == (n0, k0) and np.array_equal(t1, t0)
        n, kvl, ref = oracle.spec_accept(draft, oa[:B_acc].astype(np.int32), P, bonus=bonus)
        assert n1 == n and k1 == kvl
        assert np.array_equal(t1[:n], ref) and (t1[n:] == -99).all()


def test_decode_step_full_size_separate_calls():
    r = synth.qwen_decode(guard=row_guard(TAU32))
    _assert_guards(r["h"], r["W"], TAU32)
    step = runner.DecodeStep(r, fused=False)
    step.run()
    torch.cuda.synchronize()
    o = oracle.decode_step(r["q"], r["k_cache"], r["v_cache"], r["P"], r["h"], r["W"],
                           r["masked"], r["tokens"], TAU32)
    assert np.array_equal(runner.to_host(step.masked), o["masked"])
    assert np.array_equal(runner.to_host(step.tokens), o["tokens"])
    assert int(step.n_committed.item()) == o["n_committed"]


def test_tiny_decode_step_f32():
    r = synth.tiny()
    step = runner.DecodeStep(r)
    step.run()
    torch.cuda.synchronize()
    o = oracle.decode_step(r["q"], r["k_cache"], r["v_cache"], r["P"], r["h"], r["W"],
                           r["masked"], r["tokens"], TAU32)
    gap, dist = lmhead_margins(r["h"], r["W"], TAU32)
    assert gap.min() > 1e-2 and dist.min() >= 1e-3
    assert np.array_equal(runner.to_host(step.tokens), o["tokens"])
    assert np.array_equal(runner.to_host(step.masked), o["masked"])
    assert rel_err(step.attn.out.cpu().numpy(), o["attn"]) <= 1e-5


def test_linear_spec_step_full_size():
    """Both compositions: the verify LM head and the accept as one call
    (bd_lmhead_conf_accept, the default) and as two."""
    r = synth.linear_spec(guard=row_guard())
    _assert_guards(r["h_draft"], r["W"])
    _assert_guards(r["h_verify"], r["W"])
    o = oracle.linear_spec_step(r["q_draft"], r["k_draft"], r["v_draft"], r["q_verify"],
                                r["k_verify"], r["v_verify"], r["P"], r["h_draft"],
                                r["h_verify"], r["W"])
    for fused_accept in (True, False):
        step = runner.LinearSpecStep(r, fused_accept=fused_accept)
        step.run()
        torch.cuda.synchronize()
        assert int(step.accepted.item()) == o["accepted"] == r["L_true"]
        assert int(step.kv_len.item()) == o["kv_len"]
        assert np.array_equal(runner.to_host(step.out_tokens)[:o["accepted"]], o["out_tokens"])
        assert np.abs(bf16_host(step.attn_d.out) - o["attn_draft"]).max() <= 2e-2
        assert np.abs(bf16_host(step.attn_v.out) - o["attn_verify"]).max() <= 2e-2
        del step


def test_fused_spec_step_full_size():
    """Both compositions: the LM head and the accept as one call
    (bd_lmhead_conf_accept, the default) and as two."""
    r = synth.fused_spec(guard=row_guard())
    _assert_guards(r["h"], r["W"])
    o = oracle.fused_spec_step(r["q"], r["k_cache"], r["v_cache"], r["P"], r["h"], r["W"],
                               r["draft_in"])
    order, L, skip = oracle.cert_scan(r["anchor_conf"], r["anchor_tok"], r["text_tok"],
                                      r["k_cert"])
    for fused_accept in (True, False):
        step = runner.FusedSpecStep(r, fused_accept=fused_accept)
        step.run()
        torch.cuda.synchronize()
        assert np.array_equal(step.lm.argmax.cpu().numpy(), o["argmax"])
        assert int(step.accepted.item()) == o["accepted"] == r["L_true"]
        assert int(step.kv_len.item()) == o["kv_len"]
        assert np.abs(bf16_host(step.attn.out) - o["attn"]).max() <= 2e-2
        assert np.array_equal(runner.to_host(step.order), order)
        assert int(step.cert_L.item()) == L and int(step.skip.item()) == skip
        del step
