"""Host-side checks of the C ABI that need no GPU: the library loads and
exports every entry point include/bdiff.h declares, argument validation
returns the documented status before anything is launched, and the host mask
helper agrees with the oracle's masks."""
import re
from pathlib import Path

import numpy as np
import pytest

import oracle
from block_diffusion_vlm_amd import bdiff as bd

HEADERS = sorted((Path(__file__).resolve().parents[1] / "include").glob("*.h"))
FAKE = 0x10000          # a 16-byte-aligned non-null address; never dereferenced
MISALIGNED = 0x10008


def declared_functions():
    text = "\n".join(h.read_text() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const char\*|bd_status|size_t)\s+(bd_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_exactly_the_bound_entry_points():
    assert declared_functions() == sorted(bd.EXPORTS)


def test_library_loads_and_exports_every_symbol():
    L = bd.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for s in range(8):
        assert isinstance(bd.bd_status_str(s), str) and bd.bd_status_str(s)
    assert bd.bd_status_str(99) == "unknown status"


def test_device_check_reports_no_gfx950_here():
    # On a machine without a GPU the check must fail cleanly, not crash.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert bd.bd_device_check(0) == bd.BD_E_DEVICE
    assert bd.bd_device_check(-1) == bd.BD_E_DEVICE


@pytest.mark.parametrize("kind,name", [(bd.BD_MASK_BIDIR, "bidir"), (bd.BD_MASK_CAUSAL, "causal"),
                                       (bd.BD_MASK_SPEC_FUSED, "spec_fused")])
def test_intra_mask_matches_oracle(kind, name):
    for bq in range(1, 65):
        if name == "spec_fused" and bq % 2:
            assert bd.bd_make_intra_mask(kind, bq, check=False).size == bq  # status checked below
            continue
        rows = bd.bd_make_intra_mask(kind, bq)
        bits = ((rows[:, None] >> np.arange(bq, dtype=np.uint64)[None, :]) & np.uint64(1)).astype(bool)
        assert np.array_equal(bits, oracle.intra_block_mask(name, bq)), bq
        if bq < 64:
            assert not (rows >> np.uint64(bq)).any()      # no bits beyond the block


def test_intra_mask_errors():
    L = bd.lib()
    assert L.bd_make_intra_mask(0, 4, None) == bd.BD_E_NULL
    buf = np.zeros(70, np.uint64)
    assert L.bd_make_intra_mask(0, 0, buf.ctypes.data) == bd.BD_E_SHAPE
    assert L.bd_make_intra_mask(0, 65, buf.ctypes.data) == bd.BD_E_SHAPE
    assert L.bd_make_intra_mask(2, 5, buf.ctypes.data) == bd.BD_E_SHAPE
    assert L.bd_make_intra_mask(7, 4, buf.ctypes.data) == bd.BD_E_SHAPE


def test_workspace_queries():
    assert bd.bd_block_attn_ws_bytes(1280, 16, 16, 2, 128) > 0
    assert bd.bd_block_attn_ws_bytes(-1, 16, 16, 2, 128) == 0
    assert bd.bd_lmhead_conf_ws_bytes(16, 2048, 151936) >= 256
    assert bd.bd_lmhead_conf_ws_bytes(0, 2048, 151936) == 0
    assert bd.bd_lmhead_conf_ws_bytes(65, 2048, 151936) == 0


@pytest.mark.parametrize("Bq,Hq,Hkv", [(1, 16, 2), (16, 16, 2), (32, 16, 2), (64, 16, 2),
                                       (33, 32, 4), (8, 64, 64)])
def test_block_attn_workspace_never_shrinks_with_the_prefix(Bq, Hq, Hkv):
    # A workspace sized for one prefix length must serve every shorter one
    # (the multi-block loop sizes it for its last block), and it must hold at
    # least one partial row per query row: 128 bf16 values plus a float32
    # maximum and sum.
    prev = 0
    for P in range(0, 65536 - Bq + 1, 61):
        w = bd.bd_block_attn_ws_bytes(P, Bq, Hq, Hkv, 128)
        assert w >= prev, P
        assert w >= Bq * Hq * (128 * 2 + 2 * 4)
        prev = w


def _attn(**kw):
    a = dict(dt=bd.BD_BF16, q=FAKE, k_cache=FAKE, v_cache=FAKE, P=32, cap=64, intra_mask=FAKE,
             Bq=16, Hq=16, Hkv=2, dh=128, scale=0.0, out=FAKE, ws=FAKE, ws_bytes=1 << 30,
             stream=0, check=False)
    a.update(kw)
    return bd.bd_block_attn(**a)


def test_block_attn_validation():
    assert _attn(q=None) == bd.BD_E_NULL
    assert _attn(intra_mask=None) == bd.BD_E_NULL
    assert _attn(dt=5) == bd.BD_E_DTYPE
    assert _attn(Bq=0) == bd.BD_E_SHAPE
    assert _attn(Bq=65, cap=200) == bd.BD_E_SHAPE
    assert _attn(Hq=15) == bd.BD_E_SHAPE
    assert _attn(Hkv=0) == bd.BD_E_SHAPE
    assert _attn(P=49) == bd.BD_E_SHAPE          # P + Bq > cap
    assert _attn(P=-1) == bd.BD_E_SHAPE
    assert _attn(dh=64) == bd.BD_E_SHAPE         # bf16 needs dh == 128
    assert _attn(dt=bd.BD_F32, dh=130) == bd.BD_E_SHAPE
    assert _attn(scale=float("nan")) == bd.BD_E_SHAPE
    assert _attn(scale=-0.5) == bd.BD_E_SHAPE
    assert _attn(q=MISALIGNED) == bd.BD_E_ALIGN
    assert _attn(out=MISALIGNED) == bd.BD_E_ALIGN
    assert _attn(ws=None) == bd.BD_E_WORKSPACE
    need = bd.bd_block_attn_ws_bytes(32, 16, 16, 2, 128)
    assert _attn(ws_bytes=need - 1) == bd.BD_E_WORKSPACE
    assert _attn(ws=MISALIGNED) == bd.BD_E_ALIGN


def test_block_attn_paged_validation():
    f = lambda **kw: bd.bd_block_attn_paged(**{**dict(  # noqa: E731
        q=FAKE, k_pool=FAKE, v_pool=FAKE, page_table=FAKE, page_size=16, n_pages=100, P=1280,
        key_lo=0, intra_mask=FAKE, Bq=16, Hq=16, Hkv=2, dh=128, scale=0.0, out=FAKE, ws=FAKE,
        ws_bytes=1 << 30, stream=0, check=False), **kw})
    assert f(page_table=None) == bd.BD_E_NULL
    assert f(v_pool=None) == bd.BD_E_NULL
    assert f(page_size=0) == bd.BD_E_SHAPE
    assert f(n_pages=80) == bd.BD_E_SHAPE          # 1296 keys need 81 pages of 16
    assert f(key_lo=-1) == bd.BD_E_SHAPE
    assert f(key_lo=1281) == bd.BD_E_SHAPE
    assert f(dh=64) == bd.BD_E_SHAPE
    assert f(n_pages=1 << 20) == bd.BD_E_SHAPE     # pool of 4 GiB or more
    assert f(Hq=15) == bd.BD_E_SHAPE
    assert f(k_pool=MISALIGNED) == bd.BD_E_ALIGN
    assert f(ws=None) == bd.BD_E_WORKSPACE
    need = bd.bd_block_attn_ws_bytes(1280 - 1024, 16, 16, 2, 128)
    assert f(key_lo=1024, ws_bytes=need - 1) == bd.BD_E_WORKSPACE


def test_block_attn_fp8kv_validation():
    f = lambda **kw: bd.bd_block_attn_fp8kv(**{**dict(  # noqa: E731
        q=FAKE, k_cache=FAKE, v_cache=FAKE, k_scale=FAKE, v_scale=FAKE, P=1280, cap=1296,
        intra_mask=FAKE, Bq=16, Hq=16, Hkv=2, dh=128, scale=0.0, out=FAKE, ws=FAKE,
        ws_bytes=1 << 30, stream=0, check=False), **kw})
    for name in ("q", "k_cache", "v_cache", "k_scale", "v_scale", "intra_mask", "out"):
        assert f(**{name: None}) == bd.BD_E_NULL, name
    assert f(cap=1295) == bd.BD_E_SHAPE            # P + Bq rows must fit the cache
    assert f(dh=64) == bd.BD_E_SHAPE
    assert f(Bq=65) == bd.BD_E_SHAPE
    assert f(Hq=15) == bd.BD_E_SHAPE
    assert f(scale=-1.0) == bd.BD_E_SHAPE
    assert f(v_cache=MISALIGNED) == bd.BD_E_ALIGN
    assert f(k_scale=FAKE + 2) == bd.BD_E_ALIGN
    assert f(ws=None) == bd.BD_E_WORKSPACE
    need = bd.bd_block_attn_ws_bytes(1280, 16, 16, 2, 128)
    assert f(ws_bytes=need - 1) == bd.BD_E_WORKSPACE
    assert f(ws=MISALIGNED) == bd.BD_E_ALIGN


def test_kv_quant_fp8_validation():
    f = lambda **kw: bd.bd_kv_quant_fp8(**{**dict(  # noqa: E731
        x=FAKE, n=16, Hkv=2, dh=128, scale=FAKE, cache=FAKE, cap=1296, pos=1280, stream=0,
        check=False), **kw})
    for name in ("x", "scale", "cache"):
        assert f(**{name: None}) == bd.BD_E_NULL, name
    assert f(pos=1281) == bd.BD_E_SHAPE            # rows past the cache
    assert f(pos=-1) == bd.BD_E_SHAPE
    assert f(n=-1) == bd.BD_E_SHAPE
    assert f(dh=126) == bd.BD_E_SHAPE              # whole groups of four
    assert f(Hkv=0) == bd.BD_E_SHAPE
    assert f(x=FAKE + 4) == bd.BD_E_ALIGN
    assert f(cache=FAKE + 2) == bd.BD_E_ALIGN
    assert f(scale=FAKE + 1) == bd.BD_E_ALIGN


def _lm(**kw):
    a = dict(dt=bd.BD_BF16, h=FAKE, W=FAKE, B=16, d=2048, V=151936, conf=FAKE, argmax=FAKE,
             ws=FAKE, ws_bytes=1 << 30, stream=0, check=False)
    a.update(kw)
    return bd.bd_lmhead_conf(**a)


def test_lmhead_validation():
    assert _lm(W=None) == bd.BD_E_NULL
    assert _lm(conf=None) == bd.BD_E_NULL
    assert _lm(dt=9) == bd.BD_E_DTYPE
    assert _lm(B=0) == bd.BD_E_SHAPE
    assert _lm(B=65) == bd.BD_E_SHAPE
    assert _lm(V=0) == bd.BD_E_SHAPE
    assert _lm(d=2000) == bd.BD_E_SHAPE          # bf16 needs d % 128 == 0
    assert _lm(d=16512) == bd.BD_E_SHAPE
    assert _lm(h=MISALIGNED) == bd.BD_E_ALIGN
    assert _lm(V=2 ** 30 + 1) == bd.BD_E_SHAPE    # vocabulary sizes up to 2^30
    assert bd.bd_lmhead_conf_ws_bytes(16, 2048, 2 ** 30 + 1) == 0
    assert _lm(ws=None) == bd.BD_E_WORKSPACE
    assert _lm(ws_bytes=bd.bd_lmhead_conf_ws_bytes(16, 2048, 151936) - 1) == bd.BD_E_WORKSPACE


def test_lmhead_conf_accept_validation():
    f = lambda **kw: bd.bd_lmhead_conf_accept(**{**dict(  # noqa: E731
        dt=bd.BD_BF16, h=FAKE, W=FAKE, B=32, d=2048, V=151936, conf=FAKE, argmax=FAKE,
        draft=FAKE, B_acc=16, P=4608, bonus=0, accepted=FAKE, kv_len=FAKE, out_tokens=FAKE,
        ws=FAKE, ws_bytes=1 << 30, stream=0, check=False), **kw})
    for name in ("draft", "accepted", "kv_len", "out_tokens", "conf", "argmax", "h", "W"):
        assert f(**{name: None}) == bd.BD_E_NULL, name
    assert f(dt=9) == bd.BD_E_DTYPE
    assert f(B_acc=0) == bd.BD_E_SHAPE
    assert f(B_acc=33) == bd.BD_E_SHAPE            # more verified positions than rows
    assert f(B=65, B_acc=16) == bd.BD_E_SHAPE
    assert f(P=-1) == bd.BD_E_SHAPE
    assert f(P=2 ** 31 - 16) == bd.BD_E_SHAPE      # P + B_acc must fit in int32
    assert f(h=MISALIGNED) == bd.BD_E_ALIGN
    assert f(ws=None) == bd.BD_E_WORKSPACE
    assert f(ws_bytes=bd.bd_lmhead_conf_ws_bytes(32, 2048, 151936) - 1) == bd.BD_E_WORKSPACE


def test_lmhead_conf_commit_validation():
    f = lambda **kw: bd.bd_lmhead_conf_commit(**{**dict(
        dt=bd.BD_BF16, h=FAKE, W=FAKE, B=16, d=2048, V=151936, tau=0.9, conf=FAKE, argmax=FAKE,
        masked=FAKE, tokens=FAKE, n_committed=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=0,
        check=False), **kw})
    assert f(masked=None) == bd.BD_E_NULL
    assert f(n_committed=None) == bd.BD_E_NULL
    assert f(argmax=None) == bd.BD_E_NULL
    assert f(tau=float("nan")) == bd.BD_E_SHAPE
    assert f(B=0) == bd.BD_E_SHAPE
    assert f(d=100) == bd.BD_E_SHAPE
    assert f(W=MISALIGNED) == bd.BD_E_ALIGN
    assert f(ws_bytes=10) == bd.BD_E_WORKSPACE


def _lm8(commit=False, **kw):
    a = dict(h=FAKE, Wq=FAKE, w_scale=FAKE, B=16, d=2048, V=151936, conf=FAKE, argmax=FAKE,
             ws=FAKE, ws_bytes=1 << 30, stream=0, check=False)
    if commit:
        a.update(tau=0.9, masked=FAKE, tokens=FAKE, n_committed=FAKE)
    a.update(kw)
    return (bd.bd_lmhead_conf_commit_fp8 if commit else bd.bd_lmhead_conf_fp8)(**a)


@pytest.mark.parametrize("commit", [False, True])
def test_lmhead_fp8_validation(commit):
    f = lambda **kw: _lm8(commit, **kw)  # noqa: E731
    assert f(h=None) == bd.BD_E_NULL
    assert f(Wq=None) == bd.BD_E_NULL
    assert f(w_scale=None) == bd.BD_E_NULL
    assert f(argmax=None) == bd.BD_E_NULL
    assert f(B=0) == bd.BD_E_SHAPE
    assert f(B=65) == bd.BD_E_SHAPE
    assert f(V=0) == bd.BD_E_SHAPE
    assert f(d=2000) == bd.BD_E_SHAPE            # d % 128 == 0
    assert f(d=0) == bd.BD_E_SHAPE
    assert f(d=16512) == bd.BD_E_SHAPE
    assert f(h=MISALIGNED) == bd.BD_E_ALIGN
    assert f(Wq=MISALIGNED) == bd.BD_E_ALIGN
    assert f(w_scale=MISALIGNED) == bd.BD_E_ALIGN
    assert f(ws=None) == bd.BD_E_WORKSPACE
    need = bd.bd_lmhead_conf_fp8_ws_bytes(16, 2048, 151936)
    assert f(ws_bytes=need - 1) == bd.BD_E_WORKSPACE
    assert f(ws=MISALIGNED) == bd.BD_E_ALIGN
    if commit:
        assert f(masked=None) == bd.BD_E_NULL
        assert f(n_committed=None) == bd.BD_E_NULL
        assert f(tau=float("nan")) == bd.BD_E_SHAPE


def test_lmhead_fp8_workspace_query():
    assert bd.bd_lmhead_conf_fp8_ws_bytes(16, 2048, 151936) >= 256
    # the generic path keeps the quantized hidden rows in the workspace
    assert bd.bd_lmhead_conf_fp8_ws_bytes(64, 16384, 1000) >= 64 * 16384
    for bad in ((0, 2048, 10), (65, 2048, 10), (16, 2000, 10), (16, 16512, 10), (16, 2048, 0)):
        assert bd.bd_lmhead_conf_fp8_ws_bytes(*bad) == 0


def test_quant_fp8_rows_validation():
    q = lambda **kw: bd.bd_quant_fp8_rows(**{**dict(x=FAKE, R=4, d=64, q=FAKE, scale=FAKE,
                                                    stream=0, check=False), **kw})
    assert q(x=None) == bd.BD_E_NULL
    assert q(q=None) == bd.BD_E_NULL
    assert q(scale=None) == bd.BD_E_NULL
    assert q(R=-1) == bd.BD_E_SHAPE
    assert q(d=0) == bd.BD_E_SHAPE
    assert q(d=12) == bd.BD_E_SHAPE
    assert q(x=MISALIGNED) == bd.BD_E_ALIGN
    assert q(q=MISALIGNED) == bd.BD_E_ALIGN


def _loop(**kw):
    a = dict(dt=bd.BD_BF16, q_steps=FAKE, k_cache=FAKE, v_cache=FAKE, P=32, cap=64,
             intra_mask=FAKE, B=16, Hq=16, Hkv=2, dh=128, scale=0.0, h_steps=FAKE, W=FAKE,
             w_scale=None, d=2048, V=151936, tau=0.9, max_steps=16, masked=FAKE, tokens=FAKE,
             attn_out=FAKE, conf=FAKE, argmax=FAKE, n_committed=FAKE, n_steps=FAKE, ws=FAKE,
             ws_bytes=1 << 30, stream=0, check=False)
    a.update(kw)
    return bd.bd_block_loop(**a)


def test_block_loop_validation():
    for name in ("q_steps", "k_cache", "intra_mask", "h_steps", "W", "masked", "tokens",
                 "attn_out", "conf", "argmax", "n_committed", "n_steps"):
        assert _loop(**{name: None}) == bd.BD_E_NULL, name
    assert _loop(dt=4) == bd.BD_E_DTYPE
    assert _loop(dt=bd.BD_F32, w_scale=FAKE, dh=16, d=16) == bd.BD_E_DTYPE   # FP8 head needs bf16
    assert _loop(B=0) == bd.BD_E_SHAPE
    assert _loop(B=65, cap=200) == bd.BD_E_SHAPE
    assert _loop(P=49) == bd.BD_E_SHAPE                 # P + B > cap
    assert _loop(Hq=15) == bd.BD_E_SHAPE
    assert _loop(dh=64) == bd.BD_E_SHAPE
    assert _loop(d=2000) == bd.BD_E_SHAPE
    assert _loop(V=0) == bd.BD_E_SHAPE
    assert _loop(tau=float("nan")) == bd.BD_E_SHAPE
    assert _loop(max_steps=0) == bd.BD_E_SHAPE
    assert _loop(max_steps=1025) == bd.BD_E_SHAPE
    assert _loop(scale=-1.0) == bd.BD_E_SHAPE
    assert _loop(q_steps=MISALIGNED) == bd.BD_E_ALIGN
    assert _loop(w_scale=MISALIGNED) == bd.BD_E_ALIGN
    assert _loop(attn_out=MISALIGNED) == bd.BD_E_ALIGN
    assert _loop(ws=None) == bd.BD_E_WORKSPACE
    need = bd.bd_block_loop_ws_bytes(32, 16, 16, 2, 128, 2048, 151936, 0)
    assert _loop(ws_bytes=need - 1) == bd.BD_E_WORKSPACE
    need8 = bd.bd_block_loop_ws_bytes(32, 16, 16, 2, 128, 2048, 151936, 1)
    assert _loop(w_scale=FAKE, ws_bytes=need8 - 1) == bd.BD_E_WORKSPACE
    assert _loop(ws=MISALIGNED) == bd.BD_E_ALIGN
    assert bd.bd_block_loop_ws_bytes(32, 0, 16, 2, 128, 2048, 1000, 0) == 0
    assert bd.bd_block_loop_ws_bytes(32, 16, 16, 2, 128, 2000, 1000, 1) == 0


def test_small_calls_validation():
    c = lambda **kw: bd.bd_commit(**{**dict(conf=FAKE, argmax=FAKE, B=16, tau=0.9, masked=FAKE,
                                            tokens=FAKE, n_committed=FAKE, stream=0,
                                            check=False), **kw})
    assert c(conf=None) == bd.BD_E_NULL
    assert c(n_committed=None) == bd.BD_E_NULL
    assert c(B=-1) == bd.BD_E_SHAPE
    assert c(B=65) == bd.BD_E_SHAPE
    assert c(tau=float("nan")) == bd.BD_E_SHAPE
    for fn in (bd.bd_spec_accept, bd.bd_spec_accept_bonus):
        a = lambda **kw: fn(**{**dict(draft=FAKE, verify=FAKE, B=16, P=10, accepted=FAKE,
                                      kv_len=FAKE, out_tokens=FAKE, stream=0, check=False),
                               **kw})
        assert a(verify=None) == bd.BD_E_NULL
        assert a(out_tokens=None) == bd.BD_E_NULL
        assert a(B=65) == bd.BD_E_SHAPE
        assert a(B=-1) == bd.BD_E_SHAPE
        assert a(P=-3) == bd.BD_E_SHAPE
        assert a(P=2 ** 31 - 5) == bd.BD_E_SHAPE
    s = lambda **kw: bd.bd_cert_scan(**{**dict(anchor_conf=FAKE, anchor_tok=FAKE, text_tok=FAKE,
                                               n=64, k=4, order=FAKE, accepted=FAKE,
                                               skip_full=FAKE, stream=0, check=False), **kw})
    assert s(order=None) == bd.BD_E_NULL
    assert s(n=-1) == bd.BD_E_SHAPE
    assert s(n=1025) == bd.BD_E_SHAPE


def test_dualstream_validation():
    d = lambda **kw: bd.bd_dualstream_attn(**{**dict(dt=bd.BD_BF16, q=FAKE, k=FAKE, v=FAKE,
                                                     n_vis=16, n_txt=16, block=4, H=2, dh=128,
                                                     scale=0.0, out=FAKE, stream=0,
                                                     check=False), **kw})
    assert d(v=None) == bd.BD_E_NULL
    assert d(dt=3) == bd.BD_E_DTYPE
    assert d(block=0) == bd.BD_E_SHAPE
    assert d(H=0) == bd.BD_E_SHAPE
    assert d(n_vis=0, n_txt=0) == bd.BD_E_SHAPE
    assert d(n_txt=-1) == bd.BD_E_SHAPE
    assert d(dh=16) == bd.BD_E_SHAPE
    assert d(k=MISALIGNED) == bd.BD_E_ALIGN
    assert d(scale=float("inf")) == bd.BD_E_SHAPE
    assert d(scale=-1.0) == bd.BD_E_SHAPE


def test_dualstream_seg_validation():
    d = lambda seg, **kw: bd.bd_dualstream_attn_seg(**{**dict(  # noqa: E731
        dt=bd.BD_BF16, q=FAKE, k=FAKE, v=FAKE, n_vis=16, n_txt=16, block=4, seg_starts=seg,
        H=2, dh=128, scale=0.0, out=FAKE, stream=0, check=False), **kw})
    assert d([]) == bd.BD_E_NULL                        # no segment at all
    assert d([1]) == bd.BD_E_SHAPE                      # must start at 0
    assert d([0, 5, 5]) == bd.BD_E_SHAPE                # strictly increasing
    assert d([0, 9, 4]) == bd.BD_E_SHAPE
    assert d([0, 16]) == bd.BD_E_SHAPE                  # inside the text
    assert d(list(range(65)), n_txt=100) == bd.BD_E_SHAPE   # at most 64 segments
    assert d([0, 3], v=None) == bd.BD_E_NULL
    assert d([0, 3], block=0) == bd.BD_E_SHAPE
    assert d([0, 3], k=MISALIGNED) == bd.BD_E_ALIGN


def test_dualstream_training_validation():
    f = lambda **kw: bd.bd_dualstream_attn_fwd(**{**dict(  # noqa: E731
        dt=bd.BD_BF16, q=FAKE, k=FAKE, v=FAKE, n_vis=16, n_txt=16, block=4, seg_starts=None,
        H=2, dh=128, scale=0.0, out=FAKE, lse=FAKE, stream=0, check=False), **kw})
    assert f(out=None) == bd.BD_E_NULL
    assert f(seg_starts=[1]) == bd.BD_E_SHAPE
    assert f(lse=FAKE + 2) == bd.BD_E_ALIGN
    assert f(dh=64) == bd.BD_E_SHAPE
    b = lambda **kw: bd.bd_dualstream_attn_bwd(**{**dict(  # noqa: E731
        dt=bd.BD_BF16, q=FAKE, k=FAKE, v=FAKE, out=FAKE, d_out=FAKE, lse=FAKE, n_vis=16,
        n_txt=16, block=4, seg_starts=None, H=2, dh=128, scale=0.0, dq=FAKE, dk=FAKE,
        dv=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=0, check=False), **kw})
    for name in ("q", "k", "v", "out", "d_out", "lse", "dq", "dk", "dv"):
        assert b(**{name: None}) == bd.BD_E_NULL, name
    assert b(dt=7) == bd.BD_E_DTYPE
    assert b(block=0) == bd.BD_E_SHAPE
    assert b(seg_starts=[0, 20]) == bd.BD_E_SHAPE
    assert b(dk=MISALIGNED) == bd.BD_E_ALIGN
    assert b(lse=FAKE + 2) == bd.BD_E_ALIGN
    assert b(ws=None) == bd.BD_E_WORKSPACE
    need = bd.bd_dualstream_attn_bwd_ws_bytes(16, 16, 2)
    assert need >= 48 * 2 * 4
    assert b(ws_bytes=need - 1) == bd.BD_E_WORKSPACE
    assert bd.bd_dualstream_attn_bwd_ws_bytes(0, 0, 2) == 0


def test_python_binding_raises_on_error():
    with pytest.raises(bd.BdError) as e:
        bd.bd_commit(FAKE, FAKE, 99, 0.9, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == bd.BD_E_SHAPE


def test_lmhead_noalloc_validation():
    """Argument errors come back before any device is touched, exactly as for
    bd_lmhead_conf; shapes whose partials exceed the library's scratch array
    return BD_E_WORKSPACE."""
    f = lambda **kw: bd.bd_lmhead_conf_noalloc(**{**dict(  # noqa: E731
        dt=bd.BD_BF16, h=FAKE, W=FAKE, B=16, d=2048, V=151936, conf=FAKE, argmax=FAKE,
        stream=0, check=False), **kw})
    assert f(h=None) == bd.BD_E_NULL
    assert f(argmax=None) == bd.BD_E_NULL
    assert f(dt=5) == bd.BD_E_DTYPE
    assert f(B=0) == bd.BD_E_SHAPE
    assert f(B=65) == bd.BD_E_SHAPE
    assert f(d=1000) == bd.BD_E_SHAPE
    assert f(W=MISALIGNED) == bd.BD_E_ALIGN
    # float32 partials: one per 256 vocabulary rows -> V > 65536 does not fit
    assert f(dt=bd.BD_F32, d=16, V=65537, B=64) == bd.BD_E_WORKSPACE
    # every bf16 shape fits (the persistent grid has at most 256 workgroups);
    # these fail only later, at the device lookup, as there is no GPU here
    if not __import__("torch").cuda.is_available():
        assert f(B=64, d=16384, V=2 ** 30) == bd.BD_E_DEVICE
        assert f(dt=bd.BD_F32, d=16, V=65536, B=64) == bd.BD_E_DEVICE
    assert bd.bd_lmhead_conf_ws_bytes(16, 2048, 2 ** 30 + 1) == 0
    assert f(V=2 ** 30 + 1) == bd.BD_E_SHAPE


def test_probe_stream_read_validation():
    f = lambda **kw: bd.bd_probe_stream_read(**{**dict(  # noqa: E731
        src=FAKE, n_bytes=1 << 20, grid=1024, sink=FAKE, stream=0, check=False), **kw})
    assert f(src=None) == bd.BD_E_NULL
    assert f(sink=None) == bd.BD_E_NULL
    assert f(n_bytes=0) == bd.BD_E_SHAPE
    assert f(n_bytes=24) == bd.BD_E_SHAPE
    assert f(grid=0) == bd.BD_E_SHAPE
    assert f(grid=65537) == bd.BD_E_SHAPE
    assert f(src=MISALIGNED) == bd.BD_E_ALIGN


def test_decode_blocks_validation():
    base = dict(q_seed=FAKE, h_seed=FAKE, q_steps=FAKE, h_steps=FAKE, k_blk=FAKE, v_blk=FAKE,
                k_cache=FAKE, v_cache=FAKE, cap=1344, kv_len=FAKE, P_max=1280, intra_mask=FAKE,
                n_blocks=4, B=16, max_steps=15, Hq=16, Hkv=2, dh=128, scale=0.0, W=FAKE,
                w_scale=None, d=2048, V=151936, tau=0.9, tokens=FAKE, masked=FAKE, n_steps=FAKE,
                n_committed=FAKE, seed_attn=FAKE, seed_conf=FAKE, attn_out=FAKE, conf=FAKE,
                argmax=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=0, check=False)
    f = lambda **kw: bd.bd_decode_blocks(**{**base, **kw})  # noqa: E731
    assert f(kv_len=None) == bd.BD_E_NULL
    assert f(seed_attn=None) == bd.BD_E_NULL
    assert f(h_seed=None) == bd.BD_E_NULL
    assert f(cap=1343) == bd.BD_E_SHAPE                 # P_max + n_blocks B > cap
    assert f(n_blocks=0) == bd.BD_E_SHAPE
    assert f(B=65) == bd.BD_E_SHAPE
    assert f(max_steps=0) == bd.BD_E_SHAPE
    assert f(dh=64) == bd.BD_E_SHAPE
    assert f(Hq=15) == bd.BD_E_SHAPE
    assert f(d=1000) == bd.BD_E_SHAPE
    assert f(tau=float("nan")) == bd.BD_E_SHAPE
    assert f(P_max=65536 - 63, cap=1 << 20) == bd.BD_E_SHAPE
    assert f(k_cache=MISALIGNED) == bd.BD_E_ALIGN
    assert f(kv_len=FAKE + 2) == bd.BD_E_ALIGN
    need = bd.bd_decode_blocks_ws_bytes(1280, 4, 16, 16, 2, 128, 2048, 151936, False)
    assert need > bd.bd_block_attn_ws_bytes(1280 + 3 * 16, 16, 16, 2, 128)
    assert f(ws_bytes=need - 1) == bd.BD_E_WORKSPACE
    assert bd.bd_decode_blocks_ws_bytes(1280, 0, 16, 16, 2, 128, 2048, 151936, False) == 0
