"""Device-side plumbing around libbdiff: upload seeded inputs into torch
device tensors, allocate outputs and workspaces, and run the compositions the
pages describe (one MDM decode step, the linear and the fused speculative
steps) as sequences of C-ABI calls.  Every arithmetic step runs in libbdiff;
this module only moves buffers and arguments.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import bdiff as bd


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a NumPy array to the GPU; uint16 arrays are bfloat16 bit
    patterns and become bfloat16 tensors, uint64 becomes a bit-identical int64."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint64:
        return torch.from_numpy(a.view(np.int64)).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Inverse of to_dev (bfloat16 -> uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dtype_code(name: str) -> int:
    return {"f32": bd.BD_F32, "bf16": bd.BD_BF16}[name]


def mask_dev(kind: int, bq: int, device="cuda") -> torch.Tensor:
    return to_dev(bd.bd_make_intra_mask(kind, bq), device)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Zero-filled device workspace of at least 256 bytes."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class LMHead:
    """bd_lmhead_conf over fixed device buffers."""

    def __init__(self, dt: int, W: torch.Tensor, B: int, d: int, V: int, device="cuda"):
        self.dt, self.W, self.B, self.d, self.V = dt, W, B, d, V
        self.conf = torch.empty(B, dtype=torch.float32, device=device)
        self.argmax = torch.empty(B, dtype=torch.int32, device=device)
        self.ws_bytes = bd.bd_lmhead_conf_ws_bytes(B, d, V)
        self.ws = workspace(self.ws_bytes, device)

    def __call__(self, h: torch.Tensor, stream=None):
        bd.bd_lmhead_conf(self.dt, h, self.W, self.B, self.d, self.V, self.conf, self.argmax,
                          self.ws, self.ws_bytes, stream)

    def conf_commit(self, h, tau, masked, tokens, n_committed, stream=None):
        bd.bd_lmhead_conf_commit(self.dt, h, self.W, self.B, self.d, self.V, tau, self.conf,
                                 self.argmax, masked, tokens, n_committed, self.ws,
                                 self.ws_bytes, stream)

    def conf_accept(self, h, draft, B_acc, P, accepted, kv_len, out_tokens, bonus=False,
                    stream=None):
        bd.bd_lmhead_conf_accept(self.dt, h, self.W, self.B, self.d, self.V, self.conf,
                                 self.argmax, draft, B_acc, P, int(bonus), accepted, kv_len,
                                 out_tokens, self.ws, self.ws_bytes, stream)


class LMHeadFP8:
    """bd_lmhead_conf_fp8 over fixed device buffers: W holds E4M3 codes
    (uint8 [V][d]) and w_scale one float32 scale per row; h stays bf16."""

    def __init__(self, W: torch.Tensor, w_scale: torch.Tensor, B: int, d: int, V: int,
                 device="cuda"):
        self.W, self.w_scale, self.B, self.d, self.V = W, w_scale, B, d, V
        self.conf = torch.empty(B, dtype=torch.float32, device=device)
        self.argmax = torch.empty(B, dtype=torch.int32, device=device)
        self.ws_bytes = bd.bd_lmhead_conf_fp8_ws_bytes(B, d, V)
        self.ws = workspace(self.ws_bytes, device)

    def __call__(self, h: torch.Tensor, stream=None):
        bd.bd_lmhead_conf_fp8(h, self.W, self.w_scale, self.B, self.d, self.V, self.conf,
                              self.argmax, self.ws, self.ws_bytes, stream)

    def conf_commit(self, h, tau, masked, tokens, n_committed, stream=None):
        bd.bd_lmhead_conf_commit_fp8(h, self.W, self.w_scale, self.B, self.d, self.V, tau,
                                     self.conf, self.argmax, masked, tokens, n_committed,
                                     self.ws, self.ws_bytes, stream)


class BlockAttn:
    """bd_block_attn over fixed device buffers."""

    def __init__(self, dt: int, kind: int, Bq: int, P: int, cap: int, Hq: int, Hkv: int, dh: int,
                 device="cuda"):
        self.dt, self.Bq, self.P, self.cap, self.Hq, self.Hkv, self.dh = dt, Bq, P, cap, Hq, Hkv, dh
        self.mask = mask_dev(kind, Bq, device)
        tdt = torch.float32 if dt == bd.BD_F32 else torch.bfloat16
        self.out = torch.empty((Bq, Hq, dh), dtype=tdt, device=device)
        self.ws_bytes = bd.bd_block_attn_ws_bytes(P, Bq, Hq, Hkv, dh)
        self.ws = workspace(self.ws_bytes, device)

    def __call__(self, q, k_cache, v_cache, stream=None, scale=0.0):
        bd.bd_block_attn(self.dt, q, k_cache, v_cache, self.P, self.cap, self.mask, self.Bq,
                         self.Hq, self.Hkv, self.dh, scale, self.out, self.ws, self.ws_bytes,
                         stream)


class BlockAttnFP8KV:
    """bd_block_attn_fp8kv (bf16 queries, FP8 E4M3 KV cache with per-head
    scales) over fixed device buffers."""

    def __init__(self, kind: int, Bq: int, P: int, cap: int, Hq: int, Hkv: int, dh: int = 128,
                 device="cuda"):
        self.Bq, self.P, self.cap, self.Hq, self.Hkv, self.dh = Bq, P, cap, Hq, Hkv, dh
        self.mask = mask_dev(kind, Bq, device)
        self.out = torch.empty((Bq, Hq, dh), dtype=torch.bfloat16, device=device)
        self.ws_bytes = bd.bd_block_attn_ws_bytes(P, Bq, Hq, Hkv, dh)
        self.ws = workspace(self.ws_bytes, device)

    def __call__(self, q, k_codes, v_codes, k_scale, v_scale, stream=None, scale=0.0):
        bd.bd_block_attn_fp8kv(q, k_codes, v_codes, k_scale, v_scale, self.P, self.cap,
                               self.mask, self.Bq, self.Hq, self.Hkv, self.dh, scale, self.out,
                               self.ws, self.ws_bytes, stream)


class DecodeStep:
    """One threshold (MDM) block-decode step: bd_block_attn (bidirectional
    block) -> bd_lmhead_conf_commit (LM head, then commit).  With
    ``fused=False`` the LM head and the commit are the two separate calls
    bd_lmhead_conf and bd_commit.  Inputs from synth.qwen_decode, synth.tiny
    or synth.qwen_decode_fp8 (bf16 attention, the FP8 LM-head calls).

    The block state (committed tokens, masked flags) exists in ``slots``
    independent copies in one buffer; ``run(slot=i)`` updates copy i and
    ``reset()`` restores every copy with one device copy, so that repeated
    steps do identical work and a sequence of steps on different slots needs
    one restore in all."""

    def __init__(self, inp: dict, device="cuda", fused=True, slots=1):
        self.fused = fused
        self.inp = inp
        fp8 = inp["dtype"] == "fp8"
        dt = bd.BD_BF16 if fp8 else dtype_code(inp["dtype"])
        B = inp["B"]
        self.q = to_dev(inp["q"], device)
        self.k_cache = to_dev(inp["k_cache"], device)
        self.v_cache = to_dev(inp["v_cache"], device)
        self.h = to_dev(inp["h"], device)
        self.W = to_dev(inp["W"], device)
        self.attn = BlockAttn(dt, bd.BD_MASK_BIDIR, B, inp["P"], inp["cap"], inp["Hq"],
                              inp["Hkv"], inp["q"].shape[-1], device)
        if fp8:
            self.w_scale = to_dev(inp["w_scale"], device)
            self.lm = LMHeadFP8(self.W, self.w_scale, B, inp["d"], inp["V"], device)
        else:
            self.lm = LMHead(dt, self.W, B, inp["d"], inp["V"], device)
        # One slot: tokens int32[B], then masked uint8[B]; slots 256 bytes apart.
        used = 5 * B
        stride = (used + 255) // 256 * 256
        one = np.zeros(stride, np.uint8)
        one[:4 * B] = np.asarray(inp["tokens"], np.int32).view(np.uint8)
        one[4 * B:5 * B] = np.asarray(inp["masked"], np.uint8)
        self.state0 = to_dev(np.tile(one, slots), device)
        self.state = self.state0.clone()
        self.tokens_slots = [self.state[i * stride:i * stride + 4 * B].view(torch.int32)
                             for i in range(slots)]
        self.masked_slots = [self.state[i * stride + 4 * B:i * stride + 5 * B]
                             for i in range(slots)]
        self.tokens = self.tokens_slots[0]
        self.masked = self.masked_slots[0]
        self.n_committed = torch.zeros(1, dtype=torch.int32, device=device)
        self.tau = float(inp["tau"])
        self.B = B

    def reset(self):
        self.state.copy_(self.state0)

    def run(self, stream=None, slot=0):
        tokens, masked = self.tokens_slots[slot], self.masked_slots[slot]
        self.attn(self.q, self.k_cache, self.v_cache, stream)
        lm = self.lm
        if self.fused:
            lm.conf_commit(self.h, self.tau, masked, tokens, self.n_committed, stream)
        else:
            lm(self.h, stream)
            bd.bd_commit(lm.conf, lm.argmax, self.B, self.tau, masked, tokens,
                         self.n_committed, stream)


class BlockLoop:
    """bd_block_loop over device buffers: every decode step of one block, on
    the device, until the block is committed.  Inputs from
    synth.qwen_block_loop (bf16, or the FP8 LM head), or any dict with the
    same keys (q_steps, h_steps, ...).  ``reset()`` restores the block state
    with two device copies."""

    def __init__(self, inp: dict, device="cuda", max_steps=None):
        fp8 = inp["dtype"] == "fp8"
        self.dt = bd.BD_BF16 if fp8 else dtype_code(inp["dtype"])
        B, P = inp["B"], inp["P"]
        S = inp["q_steps"].shape[0] if max_steps is None else max_steps
        Hq, Hkv, dh, d, V = (inp[k] for k in ("Hq", "Hkv", "dh", "d", "V"))
        self.inp = inp
        self.B, self.P, self.S, self.Hq, self.Hkv, self.dh, self.d, self.V = (
            B, P, S, Hq, Hkv, dh, d, V)
        self.cap = inp["cap"]
        self.tau = float(inp["tau"])
        self.q = to_dev(inp["q_steps"], device)
        self.h = to_dev(inp["h_steps"], device)
        self.k_cache = to_dev(inp["k_cache"], device)
        self.v_cache = to_dev(inp["v_cache"], device)
        self.W = to_dev(inp["W"], device)
        self.w_scale = to_dev(inp["w_scale"], device) if fp8 else None
        self.mask = mask_dev(bd.BD_MASK_BIDIR, B, device)
        self.masked0 = to_dev(np.asarray(inp["masked"], np.uint8), device)
        self.tokens0 = to_dev(np.asarray(inp["tokens"], np.int32), device)
        self.masked = self.masked0.clone()
        self.tokens = self.tokens0.clone()
        tdt = torch.float32 if self.dt == bd.BD_F32 else torch.bfloat16
        self.attn_out = torch.zeros((S, B, Hq, dh), dtype=tdt, device=device)
        self.conf = torch.full((S, B), -1.0, dtype=torch.float32, device=device)
        self.argmax = torch.full((S, B), -1, dtype=torch.int32, device=device)
        self.n_committed = torch.full((S,), -1, dtype=torch.int32, device=device)
        self.n_steps = torch.full((1,), -1, dtype=torch.int32, device=device)
        self.ws_bytes = bd.bd_block_loop_ws_bytes(P, B, Hq, Hkv, dh, d, V, fp8)
        self.ws = workspace(self.ws_bytes, device)

    def reset(self):
        self.masked.copy_(self.masked0)
        self.tokens.copy_(self.tokens0)

    def run(self, stream=None):
        bd.bd_block_loop(self.dt, self.q, self.k_cache, self.v_cache, self.P, self.cap, self.mask,
                         self.B, self.Hq, self.Hkv, self.dh, 0.0, self.h, self.W, self.w_scale,
                         self.d, self.V, self.tau, self.S, self.masked, self.tokens,
                         self.attn_out, self.conf, self.argmax, self.n_committed, self.n_steps,
                         self.ws, self.ws_bytes, stream)


class DecodeBlocks:
    """bd_decode_blocks over device buffers from synth.qwen_decode_blocks:
    several blocks, each seeded by an AR step, denoised on the device and
    appended to the KV cache, with a device-side kv_len.  ``reset()`` restores
    the cache and kv_len (two device copies and one fill)."""

    def __init__(self, inp: dict, device="cuda", max_steps=None, w_scale=None):
        nb, B, S = inp["n_blocks"], inp["B"], inp["S"]
        self.S = S if max_steps is None else max_steps
        assert self.S <= S
        Hq, Hkv, dh, d, V = (inp[k] for k in ("Hq", "Hkv", "dh", "d", "V"))
        self.inp = inp
        self.nb, self.B, self.Hq, self.Hkv, self.dh, self.d, self.V = nb, B, Hq, Hkv, dh, d, V
        self.cap, self.P0, self.tau = inp["cap"], inp["P0"], float(inp["tau"])
        t = {k: to_dev(inp[k], device) for k in ("q_seed", "h_seed", "k_blk", "v_blk", "W")}
        # the steps' inputs, cut to max_steps per block (contiguous)
        t["q_steps"] = to_dev(np.ascontiguousarray(inp["q_steps"][:, :self.S]), device)
        t["h_steps"] = to_dev(np.ascontiguousarray(inp["h_steps"][:, :self.S]), device)
        self.t = t
        self.w_scale = w_scale
        self.k0 = to_dev(inp["k_cache"], device)
        self.v0 = to_dev(inp["v_cache"], device)
        self.k_cache, self.v_cache = self.k0.clone(), self.v0.clone()
        self.kv_len = torch.full((1,), self.P0, dtype=torch.int32, device=device)
        self.mask = mask_dev(bd.BD_MASK_BIDIR, B, device)
        self.tokens = torch.full((nb, B), -1, dtype=torch.int32, device=device)
        self.masked = torch.full((nb, B), 7, dtype=torch.uint8, device=device)
        self.n_steps = torch.full((nb,), -1, dtype=torch.int32, device=device)
        self.n_committed = torch.full((nb, self.S), -1, dtype=torch.int32, device=device)
        self.seed_attn = torch.zeros((nb, Hq, dh), dtype=torch.bfloat16, device=device)
        self.seed_conf = torch.full((nb,), -1.0, dtype=torch.float32, device=device)
        self.attn_out = torch.zeros((nb, self.S, B, Hq, dh), dtype=torch.bfloat16, device=device)
        self.conf = torch.full((nb, self.S, B), -1.0, dtype=torch.float32, device=device)
        self.argmax = torch.full((nb, self.S, B), -1, dtype=torch.int32, device=device)
        self.ws_bytes = bd.bd_decode_blocks_ws_bytes(self.P0, nb, B, Hq, Hkv, dh, d, V,
                                                     w_scale is not None)
        self.ws = workspace(self.ws_bytes, device)

    def reset(self):
        self.k_cache.copy_(self.k0)
        self.v_cache.copy_(self.v0)
        self.kv_len.fill_(self.P0)

    def run(self, stream=None):
        t = self.t
        bd.bd_decode_blocks(t["q_seed"], t["h_seed"], t["q_steps"], t["h_steps"], t["k_blk"],
                            t["v_blk"], self.k_cache, self.v_cache, self.cap, self.kv_len,
                            self.P0, self.mask, self.nb, self.B, self.S, self.Hq, self.Hkv,
                            self.dh, 0.0, t["W"], self.w_scale, self.d, self.V, self.tau,
                            self.tokens, self.masked, self.n_steps, self.n_committed,
                            self.seed_attn, self.seed_conf, self.attn_out, self.conf,
                            self.argmax, self.ws, self.ws_bytes, stream)


class LinearSpecStep:
    """Linear self-speculative step: draft (bidirectional) and verify (causal)
    passes, each block attention + LM head, then the accept.  With
    ``fused_accept`` (the default) the verify pass's LM head and the accept
    are one call, bd_lmhead_conf_accept; otherwise bd_lmhead_conf and
    bd_spec_accept."""

    def __init__(self, inp: dict, device="cuda", fused_accept=True):
        self.inp = inp
        B, P = inp["B"], inp["P"]
        dh = inp["q_draft"].shape[-1]
        self.t = {k: to_dev(inp[k], device) for k in
                  ("q_draft", "q_verify", "k_draft", "v_draft", "k_verify", "v_verify",
                   "h_draft", "h_verify", "W")}
        self.attn_d = BlockAttn(bd.BD_BF16, bd.BD_MASK_BIDIR, B, P, inp["cap"], inp["Hq"],
                                inp["Hkv"], dh, device)
        self.attn_v = BlockAttn(bd.BD_BF16, bd.BD_MASK_CAUSAL, B, P, inp["cap"], inp["Hq"],
                                inp["Hkv"], dh, device)
        self.lm_d = LMHead(bd.BD_BF16, self.t["W"], B, inp["d"], inp["V"], device)
        self.lm_v = LMHead(bd.BD_BF16, self.t["W"], B, inp["d"], inp["V"], device)
        self.accepted = torch.zeros(1, dtype=torch.int32, device=device)
        self.kv_len = torch.zeros(1, dtype=torch.int32, device=device)
        self.out_tokens = torch.full((B,), -1, dtype=torch.int32, device=device)
        self.B, self.P = B, P
        self.fused_accept = fused_accept

    def run(self, stream=None):
        t = self.t
        self.attn_d(t["q_draft"], t["k_draft"], t["v_draft"], stream)
        self.lm_d(t["h_draft"], stream)
        self.attn_v(t["q_verify"], t["k_verify"], t["v_verify"], stream)
        if self.fused_accept:
            self.lm_v.conf_accept(t["h_verify"], self.lm_d.argmax, self.B, self.P, self.accepted,
                                  self.kv_len, self.out_tokens, stream=stream)
            return
        self.lm_v(t["h_verify"], stream)
        bd.bd_spec_accept(self.lm_d.argmax, self.lm_v.argmax, self.B, self.P, self.accepted,
                          self.kv_len, self.out_tokens, stream)


class FusedSpecStep:
    """Fused (quadratic) speculative step: one block attention over 2B rows
    under the SPEC_FUSED mask, one LM head over the 2B rows, the accept on
    the verify half; plus the LOWN certificate scan.  With ``fused_accept``
    (the default) the LM head and the accept are one call,
    bd_lmhead_conf_accept; otherwise bd_lmhead_conf and bd_spec_accept."""

    def __init__(self, inp: dict, device="cuda", fused_accept=True):
        self.inp = inp
        B, bq, P = inp["B"], inp["Bq"], inp["P"]
        dh = inp["q"].shape[-1]
        self.t = {k: to_dev(inp[k], device) for k in
                  ("q", "k_cache", "v_cache", "h", "W", "draft_in", "anchor_conf",
                   "anchor_tok", "text_tok")}
        self.attn = BlockAttn(bd.BD_BF16, bd.BD_MASK_SPEC_FUSED, bq, P, inp["cap"], inp["Hq"],
                              inp["Hkv"], dh, device)
        self.lm = LMHead(bd.BD_BF16, self.t["W"], bq, inp["d"], inp["V"], device)
        self.accepted = torch.zeros(1, dtype=torch.int32, device=device)
        self.kv_len = torch.zeros(1, dtype=torch.int32, device=device)
        self.out_tokens = torch.full((B,), -1, dtype=torch.int32, device=device)
        n = inp["anchor_conf"].shape[0]
        self.order = torch.full((n,), -1, dtype=torch.int32, device=device)
        self.cert_L = torch.zeros(1, dtype=torch.int32, device=device)
        self.skip = torch.zeros(1, dtype=torch.int32, device=device)
        self.B, self.P, self.n, self.k = B, P, n, int(inp["k_cert"])
        self.fused_accept = fused_accept

    def run(self, stream=None):
        t = self.t
        self.attn(t["q"], t["k_cache"], t["v_cache"], stream)
        if self.fused_accept:
            self.lm.conf_accept(t["h"], t["draft_in"], self.B, self.P, self.accepted,
                                self.kv_len, self.out_tokens, stream=stream)
        else:
            self.lm(t["h"], stream)
            bd.bd_spec_accept(t["draft_in"], self.lm.argmax, self.B, self.P, self.accepted,
                              self.kv_len, self.out_tokens, stream)
        bd.bd_cert_scan(t["anchor_conf"], t["anchor_tok"], t["text_tok"], self.n, self.k,
                        self.order, self.cert_L, self.skip, stream)


class DualStream:
    """bd_dualstream_attn over device buffers from synth.dualstream; with a
    ``seg_starts`` entry (text segment starts), bd_dualstream_attn_seg."""

    def __init__(self, inp: dict, device="cuda"):
        self.inp = inp
        self.dt = dtype_code(inp["dtype"])
        self.q, self.k, self.v = (to_dev(inp[x], device) for x in ("q", "k", "v"))
        self.out = torch.empty_like(self.q)

    def run(self, stream=None):
        i = self.inp
        if i.get("seg_starts") is not None:
            bd.bd_dualstream_attn_seg(self.dt, self.q, self.k, self.v, i["n_vis"], i["n_txt"],
                                      i["block"], i["seg_starts"], i["H"], i["dh"], 0.0,
                                      self.out, stream)
        else:
            bd.bd_dualstream_attn(self.dt, self.q, self.k, self.v, i["n_vis"], i["n_txt"],
                                  i["block"], i["H"], i["dh"], 0.0, self.out, stream)


class DualStreamTrain:
    """Training forward (output + row log-sum-exp) and backward of the
    dual-stream attention over device buffers from synth.dualstream (which
    also draws the output gradient d_out); an optional ``seg_starts`` entry
    applies the auto-truncation mask."""

    def __init__(self, inp: dict, device="cuda"):
        self.inp = inp
        self.dt = dtype_code(inp["dtype"])
        self.q, self.k, self.v, self.d_out = (to_dev(inp[x], device)
                                              for x in ("q", "k", "v", "d_out"))
        N, H = self.q.shape[0], self.q.shape[1]
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((N, H), dtype=torch.float32, device=device)
        self.dq = torch.empty_like(self.q)
        self.dk = torch.empty_like(self.q)
        self.dv = torch.empty_like(self.q)
        self.ws_bytes = bd.bd_dualstream_attn_bwd_ws_bytes(inp["n_vis"], inp["n_txt"], H)
        self.ws = workspace(self.ws_bytes, device)
        self.seg = inp.get("seg_starts")

    def forward(self, stream=None):
        i = self.inp
        bd.bd_dualstream_attn_fwd(self.dt, self.q, self.k, self.v, i["n_vis"], i["n_txt"],
                                  i["block"], self.seg, i["H"], i["dh"], 0.0, self.out, self.lse,
                                  stream)

    def backward(self, stream=None):
        i = self.inp
        bd.bd_dualstream_attn_bwd(self.dt, self.q, self.k, self.v, self.out, self.d_out,
                                  self.lse, i["n_vis"], i["n_txt"], i["block"], self.seg, i["H"],
                                  i["dh"], 0.0, self.dq, self.dk, self.dv, self.ws,
                                  self.ws_bytes, stream)


def default_scale(dh: int) -> float:
    return 1.0 / math.sqrt(dh)
