"""Python binding of libbdiff (include/bdiff.h): the same entry points under
the same names, with argument marshalling only.

Tensor arguments may be torch tensors (their data pointer is passed) or raw
integer device addresses.  ``stream=None`` means torch's current stream on
the current device.  Each call returns the bd_status code; a non-zero status
raises BdError unless ``check=False``.  The library must be built
(``python -m block_diffusion_vlm_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

# BDIFF_LIB names another build of the same library (the host-only
# sanitizer build, for argument-validation runs without a GPU).
LIB_PATH = Path(os.environ.get("BDIFF_LIB") or Path(__file__).resolve().parent / "libbdiff.so")

BD_OK, BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_ALIGN, BD_E_WORKSPACE, BD_E_DEVICE, BD_E_LAUNCH = range(8)
BD_F32, BD_BF16 = 0, 1
BD_MASK_BIDIR, BD_MASK_CAUSAL, BD_MASK_SPEC_FUSED = 0, 1, 2

# Every symbol include/bdiff.h and include/bdiff_probe.h declare.
EXPORTS = (
    "bd_status_str", "bd_device_check", "bd_make_intra_mask",
    "bd_block_attn_ws_bytes", "bd_block_attn", "bd_block_attn_paged", "bd_block_attn_fp8kv",
    "bd_kv_quant_fp8",
    "bd_lmhead_conf_ws_bytes", "bd_lmhead_conf", "bd_lmhead_conf_commit", "bd_lmhead_conf_accept",
    "bd_lmhead_conf_noalloc",
    "bd_lmhead_conf_fp8_ws_bytes", "bd_lmhead_conf_fp8", "bd_lmhead_conf_commit_fp8",
    "bd_quant_fp8_rows", "bd_block_loop_ws_bytes", "bd_block_loop",
    "bd_decode_blocks_ws_bytes", "bd_decode_blocks",
    "bd_commit", "bd_spec_accept", "bd_spec_accept_bonus", "bd_cert_scan",
    "bd_dualstream_attn", "bd_dualstream_attn_seg", "bd_dualstream_attn_fwd",
    "bd_dualstream_attn_bwd_ws_bytes", "bd_dualstream_attn_bwd",
    "bd_probe_stream_read",
)


class BdError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {bd_status_str(status)} (status {status})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "bd_status_str": ([_I], ctypes.c_char_p),
    "bd_device_check": ([ctypes.c_int], _I),
    "bd_make_intra_mask": ([_I, _I, _P], _I),
    "bd_block_attn_ws_bytes": ([_I, _I, _I, _I, _I], _SZ),
    "bd_block_attn": ([_I, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _F, _P, _P, _SZ, _P], _I),
    "bd_block_attn_paged": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _I, _I, _I, _F, _P, _P,
                             _SZ, _P], _I),
    "bd_lmhead_conf_ws_bytes": ([_I, _I, _I], _SZ),
    "bd_lmhead_conf": ([_I, _P, _P, _I, _I, _I, _P, _P, _P, _SZ, _P], _I),
    "bd_lmhead_conf_commit": ([_I, _P, _P, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "bd_lmhead_conf_accept": ([_I, _P, _P, _I, _I, _I, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P,
                               _SZ, _P], _I),
    "bd_lmhead_conf_noalloc": ([_I, _P, _P, _I, _I, _I, _P, _P, _P], _I),
    "bd_lmhead_conf_fp8_ws_bytes": ([_I, _I, _I], _SZ),
    "bd_lmhead_conf_fp8": ([_P, _P, _P, _I, _I, _I, _P, _P, _P, _SZ, _P], _I),
    "bd_lmhead_conf_commit_fp8": ([_P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _SZ,
                                   _P], _I),
    "bd_quant_fp8_rows": ([_P, _I, _I, _P, _P, _P], _I),
    "bd_block_loop_ws_bytes": ([_I, _I, _I, _I, _I, _I, _I, _I], _SZ),
    "bd_block_loop": ([_I, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _F, _P, _P, _P, _I, _I, _F,
                       _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "bd_decode_blocks_ws_bytes": ([_I] * 9, _SZ),
    "bd_decode_blocks": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I,
                          _I, _F, _P, _P, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                          _SZ, _P], _I),
    "bd_block_attn_fp8kv": ([_P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _F, _P, _P, _SZ,
                             _P], _I),
    "bd_kv_quant_fp8": ([_P, _I, _I, _I, _P, _P, _I, _I, _P], _I),
    "bd_commit": ([_P, _P, _I, _F, _P, _P, _P, _P], _I),
    "bd_spec_accept": ([_P, _P, _I, _I, _P, _P, _P, _P], _I),
    "bd_spec_accept_bonus": ([_P, _P, _I, _I, _P, _P, _P, _P], _I),
    "bd_cert_scan": ([_P, _P, _P, _I, _I, _P, _P, _P, _P], _I),
    "bd_dualstream_attn": ([_I, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P], _I),
    "bd_dualstream_attn_seg": ([_I, _P, _P, _P, _I, _I, _I, _P, _I, _I, _I, _F, _P, _P], _I),
    "bd_dualstream_attn_fwd": ([_I, _P, _P, _P, _I, _I, _I, _P, _I, _I, _I, _F, _P, _P, _P], _I),
    "bd_dualstream_attn_bwd_ws_bytes": ([_I, _I, _I], _SZ),
    "bd_dualstream_attn_bwd": ([_I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _I, _I, _F,
                                _P, _P, _P, _P, _SZ, _P], _I),
    "bd_probe_stream_read": ([_P, _SZ, _I, _P, _P], _I),
}


def lib() -> ctypes.CDLL:
    """Load libbdiff.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_diffusion_vlm_amd.build`")
        L = ctypes.CDLL(str(LIB_PATH))
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"expected a tensor or an integer address, got {type(x)!r}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ret(fn: str, status: int, check: bool) -> int:
    if check and status != BD_OK:
        raise BdError(fn, status)
    return status


def bd_status_str(status: int) -> str:
    return lib().bd_status_str(int(status)).decode()


def bd_device_check(device: int = 0) -> int:
    return int(lib().bd_device_check(int(device)))


def bd_make_intra_mask(kind: int, Bq: int, check: bool = True) -> np.ndarray:
    rows = np.zeros(max(int(Bq), 1), dtype=np.uint64)
    st = lib().bd_make_intra_mask(int(kind), int(Bq), rows.ctypes.data)
    _ret("bd_make_intra_mask", st, check)
    return rows[: max(int(Bq), 0)]


def bd_block_attn_ws_bytes(P, Bq, Hq, Hkv, dh) -> int:
    return int(lib().bd_block_attn_ws_bytes(P, Bq, Hq, Hkv, dh))


def bd_block_attn(dt, q, k_cache, v_cache, P, cap, intra_mask, Bq, Hq, Hkv, dh, scale, out, ws,
                  ws_bytes, stream=None, check=True) -> int:
    st = lib().bd_block_attn(dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), P, cap, _ptr(intra_mask),
                             Bq, Hq, Hkv, dh, scale, _ptr(out), _ptr(ws), ws_bytes,
                             _stream(stream))
    return _ret("bd_block_attn", st, check)


def bd_block_attn_paged(q, k_pool, v_pool, page_table, page_size, n_pages, P, key_lo, intra_mask,
                        Bq, Hq, Hkv, dh, scale, out, ws, ws_bytes, stream=None,
                        check=True) -> int:
    st = lib().bd_block_attn_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                   page_size, n_pages, P, key_lo, _ptr(intra_mask), Bq, Hq, Hkv,
                                   dh, scale, _ptr(out), _ptr(ws), ws_bytes, _stream(stream))
    return _ret("bd_block_attn_paged", st, check)


def bd_lmhead_conf_ws_bytes(B, d, V) -> int:
    return int(lib().bd_lmhead_conf_ws_bytes(B, d, V))


def bd_lmhead_conf(dt, h, W, B, d, V, conf, argmax, ws, ws_bytes, stream=None, check=True) -> int:
    st = lib().bd_lmhead_conf(dt, _ptr(h), _ptr(W), B, d, V, _ptr(conf), _ptr(argmax), _ptr(ws),
                              ws_bytes, _stream(stream))
    return _ret("bd_lmhead_conf", st, check)


def bd_lmhead_conf_commit(dt, h, W, B, d, V, tau, conf, argmax, masked, tokens, n_committed, ws,
                          ws_bytes, stream=None, check=True) -> int:
    st = lib().bd_lmhead_conf_commit(dt, _ptr(h), _ptr(W), B, d, V, tau, _ptr(conf), _ptr(argmax),
                                     _ptr(masked), _ptr(tokens), _ptr(n_committed), _ptr(ws),
                                     ws_bytes, _stream(stream))
    return _ret("bd_lmhead_conf_commit", st, check)


def bd_lmhead_conf_accept(dt, h, W, B, d, V, conf, argmax, draft, B_acc, P, bonus, accepted,
                          kv_len, out_tokens, ws, ws_bytes, stream=None, check=True) -> int:
    st = lib().bd_lmhead_conf_accept(dt, _ptr(h), _ptr(W), B, d, V, _ptr(conf), _ptr(argmax),
                                     _ptr(draft), B_acc, P, int(bonus), _ptr(accepted),
                                     _ptr(kv_len), _ptr(out_tokens), _ptr(ws), ws_bytes,
                                     _stream(stream))
    return _ret("bd_lmhead_conf_accept", st, check)


def bd_lmhead_conf_noalloc(dt, h, W, B, d, V, conf, argmax, stream=None, check=True) -> int:
    st = lib().bd_lmhead_conf_noalloc(dt, _ptr(h), _ptr(W), B, d, V, _ptr(conf), _ptr(argmax),
                                      _stream(stream))
    return _ret("bd_lmhead_conf_noalloc", st, check)


def bd_lmhead_conf_fp8_ws_bytes(B, d, V) -> int:
    return int(lib().bd_lmhead_conf_fp8_ws_bytes(B, d, V))


def bd_lmhead_conf_fp8(h, Wq, w_scale, B, d, V, conf, argmax, ws, ws_bytes, stream=None,
                       check=True) -> int:
    st = lib().bd_lmhead_conf_fp8(_ptr(h), _ptr(Wq), _ptr(w_scale), B, d, V, _ptr(conf),
                                  _ptr(argmax), _ptr(ws), ws_bytes, _stream(stream))
    return _ret("bd_lmhead_conf_fp8", st, check)


def bd_lmhead_conf_commit_fp8(h, Wq, w_scale, B, d, V, tau, conf, argmax, masked, tokens,
                              n_committed, ws, ws_bytes, stream=None, check=True) -> int:
    st = lib().bd_lmhead_conf_commit_fp8(_ptr(h), _ptr(Wq), _ptr(w_scale), B, d, V, tau,
                                         _ptr(conf), _ptr(argmax), _ptr(masked), _ptr(tokens),
                                         _ptr(n_committed), _ptr(ws), ws_bytes, _stream(stream))
    return _ret("bd_lmhead_conf_commit_fp8", st, check)


def bd_quant_fp8_rows(x, R, d, q, scale, stream=None, check=True) -> int:
    st = lib().bd_quant_fp8_rows(_ptr(x), R, d, _ptr(q), _ptr(scale), _stream(stream))
    return _ret("bd_quant_fp8_rows", st, check)


def bd_block_loop_ws_bytes(P, B, Hq, Hkv, dh, d, V, w_fp8) -> int:
    return int(lib().bd_block_loop_ws_bytes(P, B, Hq, Hkv, dh, d, V, int(bool(w_fp8))))


def bd_block_loop(dt, q_steps, k_cache, v_cache, P, cap, intra_mask, B, Hq, Hkv, dh, scale,
                  h_steps, W, w_scale, d, V, tau, max_steps, masked, tokens, attn_out, conf,
                  argmax, n_committed, n_steps, ws, ws_bytes, stream=None, check=True) -> int:
    st = lib().bd_block_loop(dt, _ptr(q_steps), _ptr(k_cache), _ptr(v_cache), P, cap,
                             _ptr(intra_mask), B, Hq, Hkv, dh, scale, _ptr(h_steps), _ptr(W),
                             _ptr(w_scale), d, V, tau, max_steps, _ptr(masked), _ptr(tokens),
                             _ptr(attn_out), _ptr(conf), _ptr(argmax), _ptr(n_committed),
                             _ptr(n_steps), _ptr(ws), ws_bytes, _stream(stream))
    return _ret("bd_block_loop", st, check)


def bd_decode_blocks_ws_bytes(P_max, n_blocks, B, Hq, Hkv, dh, d, V, w_fp8) -> int:
    return int(lib().bd_decode_blocks_ws_bytes(P_max, n_blocks, B, Hq, Hkv, dh, d, V,
                                               int(bool(w_fp8))))


def bd_decode_blocks(q_seed, h_seed, q_steps, h_steps, k_blk, v_blk, k_cache, v_cache, cap,
                     kv_len, P_max, intra_mask, n_blocks, B, max_steps, Hq, Hkv, dh, scale, W,
                     w_scale, d, V, tau, tokens, masked, n_steps, n_committed, seed_attn,
                     seed_conf, attn_out, conf, argmax, ws, ws_bytes, stream=None,
                     check=True) -> int:
    st = lib().bd_decode_blocks(
        _ptr(q_seed), _ptr(h_seed), _ptr(q_steps), _ptr(h_steps), _ptr(k_blk), _ptr(v_blk),
        _ptr(k_cache), _ptr(v_cache), cap, _ptr(kv_len), P_max, _ptr(intra_mask), n_blocks, B,
        max_steps, Hq, Hkv, dh, scale, _ptr(W), _ptr(w_scale), d, V, tau, _ptr(tokens),
        _ptr(masked), _ptr(n_steps), _ptr(n_committed), _ptr(seed_attn), _ptr(seed_conf),
        _ptr(attn_out), _ptr(conf), _ptr(argmax), _ptr(ws), ws_bytes, _stream(stream))
    return _ret("bd_decode_blocks", st, check)


def bd_commit(conf, argmax, B, tau, masked, tokens, n_committed, stream=None, check=True) -> int:
    st = lib().bd_commit(_ptr(conf), _ptr(argmax), B, tau, _ptr(masked), _ptr(tokens),
                         _ptr(n_committed), _stream(stream))
    return _ret("bd_commit", st, check)


def bd_spec_accept(draft, verify, B, P, accepted, kv_len, out_tokens, stream=None,
                   check=True) -> int:
    st = lib().bd_spec_accept(_ptr(draft), _ptr(verify), B, P, _ptr(accepted), _ptr(kv_len),
                              _ptr(out_tokens), _stream(stream))
    return _ret("bd_spec_accept", st, check)


def bd_spec_accept_bonus(draft, verify, B, P, accepted, kv_len, out_tokens, stream=None,
                         check=True) -> int:
    st = lib().bd_spec_accept_bonus(_ptr(draft), _ptr(verify), B, P, _ptr(accepted),
                                    _ptr(kv_len), _ptr(out_tokens), _stream(stream))
    return _ret("bd_spec_accept_bonus", st, check)


def bd_block_attn_fp8kv(q, k_cache, v_cache, k_scale, v_scale, P, cap, intra_mask, Bq, Hq, Hkv,
                        dh, scale, out, ws, ws_bytes, stream=None, check=True) -> int:
    st = lib().bd_block_attn_fp8kv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                   _ptr(v_scale), P, cap, _ptr(intra_mask), Bq, Hq, Hkv, dh,
                                   scale, _ptr(out), _ptr(ws), ws_bytes, _stream(stream))
    return _ret("bd_block_attn_fp8kv", st, check)


def bd_kv_quant_fp8(x, n, Hkv, dh, scale, cache, cap, pos, stream=None, check=True) -> int:
    st = lib().bd_kv_quant_fp8(_ptr(x), n, Hkv, dh, _ptr(scale), _ptr(cache), cap, pos,
                               _stream(stream))
    return _ret("bd_kv_quant_fp8", st, check)


def bd_cert_scan(anchor_conf, anchor_tok, text_tok, n, k, order, accepted, skip_full,
                 stream=None, check=True) -> int:
    st = lib().bd_cert_scan(_ptr(anchor_conf), _ptr(anchor_tok), _ptr(text_tok), n, k,
                            _ptr(order), _ptr(accepted), _ptr(skip_full), _stream(stream))
    return _ret("bd_cert_scan", st, check)


def bd_dualstream_attn(dt, q, k, v, n_vis, n_txt, block, H, dh, scale, out, stream=None,
                       check=True) -> int:
    st = lib().bd_dualstream_attn(dt, _ptr(q), _ptr(k), _ptr(v), n_vis, n_txt, block, H, dh,
                                  scale, _ptr(out), _stream(stream))
    return _ret("bd_dualstream_attn", st, check)


def bd_dualstream_attn_seg(dt, q, k, v, n_vis, n_txt, block, seg_starts, H, dh, scale, out,
                           stream=None, check=True) -> int:
    """``seg_starts``: a host sequence of int32 segment starts (copied)."""
    seg = np.ascontiguousarray(np.asarray(seg_starts, dtype=np.int32))
    st = lib().bd_dualstream_attn_seg(dt, _ptr(q), _ptr(k), _ptr(v), n_vis, n_txt, block,
                                      seg.ctypes.data if seg.size else None, int(seg.size), H,
                                      dh, scale, _ptr(out), _stream(stream))
    return _ret("bd_dualstream_attn_seg", st, check)


def _segments(seg_starts):
    """(pointer, count, keep-alive array) of a host segment list, or (None, 1, None)."""
    if seg_starts is None:
        return None, 1, None
    seg = np.ascontiguousarray(np.asarray(seg_starts, dtype=np.int32))
    return (seg.ctypes.data if seg.size else None), int(seg.size), seg


def bd_dualstream_attn_fwd(dt, q, k, v, n_vis, n_txt, block, seg_starts, H, dh, scale, out, lse,
                           stream=None, check=True) -> int:
    p, n, _keep = _segments(seg_starts)
    st = lib().bd_dualstream_attn_fwd(dt, _ptr(q), _ptr(k), _ptr(v), n_vis, n_txt, block, p, n,
                                      H, dh, scale, _ptr(out), _ptr(lse), _stream(stream))
    return _ret("bd_dualstream_attn_fwd", st, check)


def bd_dualstream_attn_bwd_ws_bytes(n_vis, n_txt, H) -> int:
    return int(lib().bd_dualstream_attn_bwd_ws_bytes(n_vis, n_txt, H))


def bd_dualstream_attn_bwd(dt, q, k, v, out, d_out, lse, n_vis, n_txt, block, seg_starts, H, dh,
                           scale, dq, dk, dv, ws, ws_bytes, stream=None, check=True) -> int:
    p, n, _keep = _segments(seg_starts)
    st = lib().bd_dualstream_attn_bwd(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(d_out),
                                      _ptr(lse), n_vis, n_txt, block, p, n, H, dh, scale,
                                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes,
                                      _stream(stream))
    return _ret("bd_dualstream_attn_bwd", st, check)


def bd_probe_stream_read(src, n_bytes, grid, sink, stream=None, check=True) -> int:
    """Measurement reference (include/bdiff_probe.h): one streaming read of
    n_bytes of src, XOR-folded into the uint32 at sink."""
    st = lib().bd_probe_stream_read(_ptr(src), n_bytes, grid, _ptr(sink), _stream(stream))
    return _ret("bd_probe_stream_read", st, check)
