"""Seeded synthetic inputs for the block-diffusion decode step and the
dual-stream training attention.

This module only draws random numbers and lays them out: it computes no
attention, no logits, no softmax and no commit/accept/certificate decision.
Both the GPU library's tests/benchmark and the CPU oracle's tests read their
inputs from here, so that the two sides see the same values.

Every tensor is returned as a NumPy array: float32 for the float32 workload,
raw bfloat16 bit patterns (uint16, round-to-nearest-even from float32) for the
bfloat16 workloads.

Shapes follow the workloads on the pages: batch 1, a mostly visual prefix
(visual tokens are 89-97 % of the input in the LOWN article, 'research
motivation'), block 16/32 and threshold 0.9 (Fast-dVLM overview, §4.1 and
§2.3.1), Qwen2.5-VL-3B geometry (16 query heads, 2 KV heads, head_dim 128,
hidden 2048, vocabulary 151936).  Synthetic values stand in for the pages'
benchmarks and trained weights, which are not available.
"""

from __future__ import annotations

import numpy as np

BASE_SEED = 20261203
N_CONFIGS = 11


# ---------------------------------------------------------------------------
# Random streams and number formats
# ---------------------------------------------------------------------------

def config_rng(cfg: int, seed: int | None = None) -> np.random.Generator:
    """PCG64 stream for workload ``cfg`` (1..11): child ``cfg-1`` of
    SeedSequence(seed or BASE_SEED) (a child's stream does not depend on how
    many children are spawned)."""
    ss = np.random.SeedSequence(BASE_SEED if seed is None else seed)
    return np.random.Generator(np.random.PCG64(ss.spawn(N_CONFIGS)[cfg - 1]))


def bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even
    (the rounding torch's .to(torch.bfloat16) performs).  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64 (used to plant
    hidden states against the rounded weights)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def normal(rng, shape, std=1.0, trunc=None) -> np.ndarray:
    """float32 N(0, std^2); with ``trunc`` every |x| > trunc is redrawn."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if trunc is not None:
        bad = np.abs(x) > trunc
        while bad.any():
            x[bad] = rng.standard_normal(int(bad.sum()), dtype=np.float32)
            bad = np.abs(x) > trunc
    if std != 1.0:
        x *= np.float32(std)
    return x


def normal_bf16(rng, shape, std=1.0, trunc=None, chunk_rows=8192) -> np.ndarray:
    """bfloat16 bits of N(0, std^2) (optionally truncated to |x| <= trunc
    before scaling), generated in row chunks to bound host memory."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    for s in range(0, rows, chunk_rows):
        e = min(rows, s + chunk_rows)
        out[s:e] = bf16_bits(normal(rng, (e - s,) + shape[1:], std, trunc))
    return out


# ---------------------------------------------------------------------------
# Hidden-state planting for the LM head
# ---------------------------------------------------------------------------

def plant_hidden(rng, W_bits, targets, target_conf, sigma_w, row=None) -> np.ndarray:
    """Hidden rows h_i = e_i + alpha_i * u_i, where u_i is the unit direction
    of the (bf16-rounded) weight row of target token t_i and e_i ~ N(0, I) is
    drawn and then made orthogonal to u_i.  ``row(t)``, when given, returns
    the float64 weight row of token t instead (for weights stored in another
    format; W_bits then only supplies the shape).

    alpha_i comes from a statistical model of the weights, not from the
    logits: with W entries i.i.d. N(0, sigma_w^2), the target logit is
    alpha * |W_t| and every other logit is ~ N(0, sigma_w^2 |h|^2), whose
    exponential has mean exp(sigma_w^2 |h|^2 / 2).  Setting
        alpha |W_t| - log(V-1) - sigma_w^2 (|e|^2 + alpha^2) / 2 = logit(c_i)
    places the top probability near the requested c_i (within about half a
    percent at the sizes used), with t_i ahead of every other token by a
    wide logit gap.  Returns float32 rows (round them to bf16 with
    ``bf16_bits``)."""
    V, d = W_bits.shape
    targets = np.asarray(targets)
    c = np.asarray(target_conf, dtype=np.float64)
    out = np.empty((targets.size, d), dtype=np.float32)
    s2 = float(sigma_w) ** 2
    for i, t in enumerate(targets):
        w = bf16_to_f64(W_bits[int(t)]) if row is None else row(int(t))
        nw = float(np.sqrt(w @ w))
        u = w / nw
        e = rng.standard_normal(d)
        e -= (e @ u) * u
        ee = float(e @ e)
        C = np.log(V - 1.0) + 0.5 * s2 * ee + np.log(c[i] / (1.0 - c[i]))
        disc = nw * nw - 2.0 * s2 * C
        alpha = (nw - np.sqrt(max(disc, 0.0))) / s2 if s2 > 0 else C / nw
        out[i] = (e + alpha * u).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# FP8 weights
# ---------------------------------------------------------------------------

E4M3_CODE_STD = 112.0   # code-domain std of the weights: 4 std = 448, the largest E4M3 value


def e4m3_codes(x) -> np.ndarray:
    """float32 -> OCP E4M3 codes through torch's float8_e4m3fn cast (round to
    nearest even); the inputs stay within +-448."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_row_values(codes) -> np.ndarray:
    """E4M3 codes -> float64 values through torch's float8_e4m3fn type (used
    to plant hidden states against the stored weights)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def normal_e4m3(rng, shape, chunk_rows=8192) -> np.ndarray:
    """E4M3 codes of 112 x N(0, 1) truncated to |x| <= 4 (so that every value
    is within the format's range), generated in row chunks."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.uint8)
    for s in range(0, shape[0], chunk_rows):
        e = min(shape[0], s + chunk_rows)
        x = normal(rng, (e - s,) + shape[1:], 1.0, trunc=4.0) * np.float32(E4M3_CODE_STD)
        out[s:e] = e4m3_codes(x)
    return out


def _commit_band_conf(rng, n, p_commit=0.4, hi=(0.92, 0.999), lo=(0.02, 0.88)):
    """Target top probabilities: with probability p_commit in ``hi`` (above
    the 0.9 threshold with a margin), else in ``lo`` (below it with a margin)."""
    z = rng.random(n) < p_commit
    c = np.where(z, rng.uniform(hi[0], hi[1], n), rng.uniform(lo[0], lo[1], n))
    return c, z


def _band_redraw(z, hi=(0.92, 0.999), lo=(0.02, 0.88)):
    """Re-draw of target probabilities that keeps each row in its band
    (``z`` true: above the threshold)."""
    z = np.asarray(z, dtype=bool)

    def draw(rng, rows):
        n = len(rows)
        return np.where(z[rows], rng.uniform(hi[0], hi[1], n), rng.uniform(lo[0], lo[1], n))
    return draw


def _uniform_redraw(lo, hi):
    return lambda rng, rows: rng.uniform(lo, hi, len(rows))


def _different_token(rng, tok, V):
    """A uniform token id different from ``tok``."""
    x = int(rng.integers(0, V - 1))
    return x + (x >= tok)


def _redraw_stream(rng) -> np.random.Generator:
    """A fresh PCG64 stream spawned from ``rng``'s seed sequence: re-draws
    take their numbers from it, so the main stream (and every tensor drawn
    after the hidden rows) is the same whether or not a row was re-drawn."""
    return np.random.Generator(np.random.PCG64(rng.bit_generator.seed_seq.spawn(1)[0]))


def planted_bits(rng, W, targets, target_conf, sigma_w, row=None, guard=None, w_scale=None,
                 redraw_conf=None):
    """bf16 bits of hidden rows planted as in ``plant_hidden``.

    ``guard``, when given, is a callable ``guard(h_bits, W, w_scale) -> bool
    per row`` (the tests build it from the oracle's top-2-gap and
    distance-from-threshold checks; this module computes no logits).  Every
    row it rejects is planted again, with fresh noise and a fresh target
    probability ``redraw_conf(rng, rows)`` taken from a spawned stream, until
    it passes (at most 64 rounds).  Returns (bits, target probabilities)."""
    targets = np.asarray(targets)
    conf = np.array(target_conf, dtype=np.float64)
    h = bf16_bits(plant_hidden(rng, W, targets, conf, sigma_w, row=row))
    if guard is None:
        return h, conf
    ok = np.asarray(guard(h, W, w_scale), dtype=bool)
    rr = None
    for _ in range(64):
        bad = np.nonzero(~ok)[0]
        if bad.size == 0:
            return h, conf
        rr = _redraw_stream(rng) if rr is None else rr
        if redraw_conf is not None:
            conf[bad] = redraw_conf(rr, bad)
        h[bad] = bf16_bits(plant_hidden(rr, W, targets[bad], conf[bad], sigma_w, row=row))
        ok[bad] = np.asarray(guard(h[bad], W, w_scale), dtype=bool)
    raise RuntimeError("planted rows still fail the guard after 64 re-draws")


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def tiny(seed: int | None = None) -> dict:
    """Tiny float32 case.  Dual-stream attention over 4 visual + 4 clean +
    4 noisy tokens, block 2, one head, head_dim 16; one decode block of B=4
    queries over a 32-token prefix; LM head d=16 x V=64; threshold 0.9; every
    position masked.  Q/K/V, hidden and W ~ N(0, 1); each hidden row gets a
    planted target token pushed along its weight row by a random amount
    (alpha ~ U(0, 6) in units of the row direction)."""
    rng = config_rng(1, seed)
    n_vis, n_txt, blk, dh = 4, 4, 2, 16
    n = n_vis + 2 * n_txt
    B, P, V, d = 4, 32, 64, 16
    r = {
        "dtype": "f32", "n_vis": n_vis, "n_txt": n_txt, "block": blk, "H": 1, "dh": dh,
        "ds_q": normal(rng, (n, 1, dh)), "ds_k": normal(rng, (n, 1, dh)),
        "ds_v": normal(rng, (n, 1, dh)),
        "B": B, "P": P, "Hq": 1, "Hkv": 1, "cap": P + B,
        "q": normal(rng, (B, 1, dh)),
        "k_cache": normal(rng, (1, P + B, dh)), "v_cache": normal(rng, (1, P + B, dh)),
        "V": V, "d": d, "W": normal(rng, (V, d)),
    }
    t = rng.integers(0, V, B)
    alpha = rng.uniform(0.0, 6.0, B)
    h = normal(rng, (B, d))
    for i in range(B):
        w = r["W"][t[i]].astype(np.float64)
        h[i] += (alpha[i] * w / np.sqrt(w @ w)).astype(np.float32)
    r.update(h=h, targets=t.astype(np.int32), tau=0.9,
             masked=np.ones(B, np.uint8), tokens=np.zeros(B, np.int32))
    return r


def qwen_decode(seed: int | None = None, B=16, n_vis=1024, n_prompt=256, Hq=16, Hkv=2,
                dh=128, d=2048, V=151936, p_commit=0.4, sigma_w=0.02, guard=None) -> dict:
    """One MDM block-decode step shaped like Qwen2.5-VL-3B, bf16.  Prefix KV of
    n_vis visual + n_prompt prompt tokens, then the block's B rows; bidirectional
    intra-block mask.  q, K ~ N(0,1); V ~ N(0,1) truncated to |v| <= 4.  W ~
    N(0, sigma_w^2).  Hidden rows planted so that about p_commit of them have top
    probability in [0.92, 0.999] and the rest in [0.02, 0.88].  Position 0 holds
    the block's AR seed token (already unmasked); 1..B-1 are masked.
    ``guard`` (see ``planted_bits``) re-draws rows that fail it, keeping each
    row's target token and its side of the threshold."""
    rng = config_rng(2, seed)
    P = n_vis + n_prompt
    cap = P + B
    W = normal_bf16(rng, (V, d), std=sigma_w)
    t = rng.integers(0, V, B)
    c, z = _commit_band_conf(rng, B, p_commit)
    h, c = planted_bits(rng, W, t, c, sigma_w, guard=guard, redraw_conf=_band_redraw(z))
    masked = np.ones(B, np.uint8)
    masked[0] = 0
    tokens = np.zeros(B, np.int32)
    tokens[0] = int(rng.integers(0, V))
    return {
        "dtype": "bf16", "B": B, "P": P, "n_vis": n_vis, "n_prompt": n_prompt, "cap": cap,
        "Hq": Hq, "Hkv": Hkv, "dh": dh, "d": d, "V": V, "tau": 0.9,
        "q": normal_bf16(rng, (B, Hq, dh)),
        "k_cache": normal_bf16(rng, (Hkv * cap, dh)).reshape(Hkv, cap, dh),
        "v_cache": normal_bf16(rng, (Hkv * cap, dh), trunc=4.0).reshape(Hkv, cap, dh),
        "W": W, "h": h, "targets": t.astype(np.int32), "target_conf": c, "planted_commit": z,
        "masked": masked, "tokens": tokens,
    }


def qwen_decode_fp8kv(seed: int | None = None, B=16, n_vis=1024, n_prompt=256, Hq=16, Hkv=2,
                      dh=128, scale_spread=0.1) -> dict:
    """The block attention of ``qwen_decode`` over an FP8 (E4M3) KV cache.
    K and V are stored as E4M3 codes of 112 x N(0,1) truncated at 4 std, with
    one float32 scale per KV head, k_scale[g], v_scale[g] = U(1 - spread,
    1 + spread) / 112, so that the stored entries stand for ~N(0,1) values
    (V within +-4, as in the bf16 workload).  Queries bf16 N(0,1);
    bidirectional block.  ``k_new``/``v_new`` [B][Hkv][dh] bf16 are fresh
    block rows for the quantizer (K ~ N(0,1), V truncated at 4)."""
    rng = config_rng(9, seed)
    P = n_vis + n_prompt
    cap = P + B
    return {
        "dtype": "bf16", "B": B, "P": P, "n_vis": n_vis, "n_prompt": n_prompt, "cap": cap,
        "Hq": Hq, "Hkv": Hkv, "dh": dh,
        "q": normal_bf16(rng, (B, Hq, dh)),
        "k_codes": normal_e4m3(rng, (Hkv * cap, dh)).reshape(Hkv, cap, dh),
        "v_codes": normal_e4m3(rng, (Hkv * cap, dh)).reshape(Hkv, cap, dh),
        "k_scale": (rng.uniform(1 - scale_spread, 1 + scale_spread, Hkv)
                    / E4M3_CODE_STD).astype(np.float32),
        "v_scale": (rng.uniform(1 - scale_spread, 1 + scale_spread, Hkv)
                    / E4M3_CODE_STD).astype(np.float32),
        "k_new": normal_bf16(rng, (B, Hkv, dh)),
        "v_new": normal_bf16(rng, (B, Hkv, dh), trunc=4.0),
    }


def qwen_decode_fp8(seed: int | None = None, B=16, n_vis=1024, n_prompt=256, Hq=16, Hkv=2,
                    dh=128, d=2048, V=151936, p_commit=0.4, sigma_w=0.02,
                    scale_spread=0.1, guard=None) -> dict:
    """The decode step of ``qwen_decode`` with an FP8 (E4M3, W8A8) LM head.
    W is stored as E4M3 codes of 112 x N(0,1) (truncated at 4 std) with one
    float32 scale per vocabulary row, w_scale[v] = sigma_w / 112 x U(1 -
    spread, 1 + spread), so that the stored weights stand for N(0, sigma_w^2)
    entries with a per-channel spread.  Hidden rows (bf16) are planted
    against the stored (decoded and scaled) weight rows as in qwen_decode;
    the attention inputs and the block state are drawn the same way.
    ``guard`` as in qwen_decode (it receives the codes and w_scale)."""
    rng = config_rng(6, seed)
    P = n_vis + n_prompt
    cap = P + B
    Wq = normal_e4m3(rng, (V, d))
    w_scale = (np.float32(sigma_w / E4M3_CODE_STD)
               * rng.uniform(1 - scale_spread, 1 + scale_spread, V).astype(np.float32))
    t = rng.integers(0, V, B)
    c, z = _commit_band_conf(rng, B, p_commit)
    h, c = planted_bits(rng, Wq, t, c, sigma_w,
                        row=lambda v: e4m3_row_values(Wq[v]) * float(w_scale[v]),
                        guard=guard, w_scale=w_scale, redraw_conf=_band_redraw(z))
    masked = np.ones(B, np.uint8)
    masked[0] = 0
    tokens = np.zeros(B, np.int32)
    tokens[0] = int(rng.integers(0, V))
    return {
        "dtype": "fp8", "B": B, "P": P, "n_vis": n_vis, "n_prompt": n_prompt, "cap": cap,
        "Hq": Hq, "Hkv": Hkv, "dh": dh, "d": d, "V": V, "tau": 0.9,
        "q": normal_bf16(rng, (B, Hq, dh)),
        "k_cache": normal_bf16(rng, (Hkv * cap, dh)).reshape(Hkv, cap, dh),
        "v_cache": normal_bf16(rng, (Hkv * cap, dh), trunc=4.0).reshape(Hkv, cap, dh),
        "W": Wq, "w_scale": w_scale.astype(np.float32), "h": h,
        "targets": t.astype(np.int32), "target_conf": c, "planted_commit": z,
        "masked": masked, "tokens": tokens,
    }


def _plant_trajectory(rng, W, row, w_scale, B, S, T, V, sigma_w, guard):
    """Hidden rows of S denoising steps of one block (position 0 is the AR
    seed): each masked position i gets a commit step c_i in [0, T), the
    positions 1..B-1 being split in random order into T non-empty groups;
    from step c_i on, row i is planted on its final token with top
    probability in [0.92, 0.999], before it on a fresh uniform token with top
    probability in [0.02, 0.88].  Returns (final tokens, c, h [S][B][d])."""
    d = W.shape[1]
    final = rng.integers(0, V, B)
    order = rng.permutation(np.arange(1, B))
    cuts = np.sort(rng.choice(np.arange(1, B - 1), T - 1, replace=False))
    c = np.zeros(B, np.int64)
    for g, part in enumerate(np.split(order, cuts)):
        c[part] = g
    h = np.empty((S, B, d), np.uint16)
    for s in range(S):
        late = c <= s
        tgt = np.where(late, final, rng.integers(0, V, B))
        conf = np.where(late, rng.uniform(0.92, 0.999, B), rng.uniform(0.02, 0.88, B))
        h[s], _ = planted_bits(rng, W, tgt, conf, sigma_w, row=row, guard=guard,
                               w_scale=w_scale, redraw_conf=_band_redraw(late))
    return final, c, h


def qwen_block_loop(seed: int | None = None, B=16, S=16, T=8, n_vis=1024, n_prompt=256,
                    Hq=16, Hkv=2, dh=128, d=2048, V=151936, sigma_w=0.02, fp8=False,
                    guard=None) -> dict:
    """All steps of one block of the Qwen-shaped decode, bf16 (or with the
    FP8 LM head): a denoising trajectory.  Position 0 is the AR seed; each
    masked position i gets a commit step c_i in [0, T), the masked positions
    being split in random order into T non-empty groups, so that every step
    before T commits at least one position by threshold (about two per step
    at B = 16, T = 8, in line with MDM's 1.95 tokens per forward on the
    overview's benchmarks).  Hidden rows per step: from step c_i on, row i is
    planted on its final token with top probability in [0.92, 0.999]; before
    it, on a fresh uniform token with top probability in [0.02, 0.88].
    Block queries are drawn afresh for every step; the KV cache is fixed.
    S >= T steps are provided (the loop must stop at T on its own).
    ``guard`` as in qwen_decode, applied to every step's rows."""
    rng = config_rng(7 if fp8 else 8, seed)
    P = n_vis + n_prompt
    cap = P + B
    if fp8:
        W = normal_e4m3(rng, (V, d))
        w_scale = (np.float32(sigma_w / E4M3_CODE_STD)
                   * rng.uniform(0.9, 1.1, V).astype(np.float32))
        row = lambda v: e4m3_row_values(W[v]) * float(w_scale[v])  # noqa: E731
    else:
        W = normal_bf16(rng, (V, d), std=sigma_w)
        w_scale, row = None, None
    final, c, h = _plant_trajectory(rng, W, row, w_scale, B, S, T, V, sigma_w, guard)
    masked = np.ones(B, np.uint8)
    masked[0] = 0
    tokens = np.zeros(B, np.int32)
    tokens[0] = int(rng.integers(0, V))
    r = {
        "dtype": "fp8" if fp8 else "bf16", "B": B, "S": S, "T": T, "P": P, "n_vis": n_vis,
        "n_prompt": n_prompt, "cap": cap, "Hq": Hq, "Hkv": Hkv, "dh": dh, "d": d, "V": V,
        "tau": 0.9, "q_steps": normal_bf16(rng, (S * B, Hq, dh)).reshape(S, B, Hq, dh),
        "k_cache": normal_bf16(rng, (Hkv * cap, dh)).reshape(Hkv, cap, dh),
        "v_cache": normal_bf16(rng, (Hkv * cap, dh), trunc=4.0).reshape(Hkv, cap, dh),
        "W": W, "h_steps": h, "final_tokens": final.astype(np.int32), "commit_step": c,
        "masked": masked, "tokens": tokens,
    }
    if fp8:
        r["w_scale"] = w_scale
    return r


def qwen_decode_blocks(seed: int | None = None, n_blocks=4, B=16, S=15, T=8, n_vis=1024,
                       n_prompt=256, Hq=16, Hkv=2, dh=128, d=2048, V=151936, sigma_w=0.02,
                       fp8=False, guard=None) -> dict:
    """Several consecutive blocks of the Qwen-shaped decode, bf16, each
    started by an AR seed step and appended to the KV cache before the next
    (causal-context decoding, Fast-dVLM overview §2.2.2; blocks in order,
    §1.2).  The cache holds the n_vis visual + n_prompt prompt rows (P0);
    rows from P0 on are zero and get each block's own K/V rows ([B][Hkv][dh],
    K ~ N(0,1), V truncated at 4) in turn; cap = P0 + n_blocks B.  Per block:
    a seed query [Hq][dh] and a seed hidden row planted on a uniform token
    with top probability in [0.92, 0.999] (the AR prediction of the block's
    first token), and S >= T denoising steps planted as in qwen_block_loop
    (every masked position committed by threshold within T steps; S = B - 1
    steps always suffice, as every step commits at least one position).
    With ``fp8`` the LM head's W is stored as E4M3 codes with one float32
    scale per row, as in qwen_decode_fp8, and the rows are planted against the
    stored weights (its own random stream).
    ``guard`` as in qwen_decode, applied to every planted row."""
    rng = config_rng(11 if fp8 else 10, seed)
    P0 = n_vis + n_prompt
    cap = P0 + n_blocks * B
    if fp8:
        W = normal_e4m3(rng, (V, d))
        w_scale = (np.float32(sigma_w / E4M3_CODE_STD)
                   * rng.uniform(0.9, 1.1, V).astype(np.float32))
        row = lambda v: e4m3_row_values(W[v]) * float(w_scale[v])  # noqa: E731
    else:
        W = normal_bf16(rng, (V, d), std=sigma_w)
        w_scale, row = None, None
    k_cache = np.zeros((Hkv, cap, dh), np.uint16)
    v_cache = np.zeros((Hkv, cap, dh), np.uint16)
    k_cache[:, :P0] = normal_bf16(rng, (Hkv * P0, dh)).reshape(Hkv, P0, dh)
    v_cache[:, :P0] = normal_bf16(rng, (Hkv * P0, dh), trunc=4.0).reshape(Hkv, P0, dh)
    seed_t = rng.integers(0, V, n_blocks)
    seed_c = rng.uniform(0.92, 0.999, n_blocks)
    h_seed, _ = planted_bits(rng, W, seed_t, seed_c, sigma_w, row=row, guard=guard,
                             w_scale=w_scale, redraw_conf=_uniform_redraw(0.92, 0.999))
    h_steps = np.empty((n_blocks, S, B, d), np.uint16)
    final = np.empty((n_blocks, B), np.int32)
    commit_step = np.empty((n_blocks, B), np.int64)
    for b in range(n_blocks):
        f, c, h = _plant_trajectory(rng, W, row, w_scale, B, S, T, V, sigma_w, guard)
        final[b], commit_step[b], h_steps[b] = f, c, h
    r = {
        "dtype": "fp8" if fp8 else "bf16", "n_blocks": n_blocks, "B": B, "S": S, "T": T, "P0": P0, "cap": cap,
        "n_vis": n_vis, "n_prompt": n_prompt, "Hq": Hq, "Hkv": Hkv, "dh": dh, "d": d, "V": V,
        "tau": 0.9, "W": W, "k_cache": k_cache, "v_cache": v_cache,
        "k_blk": normal_bf16(rng, (n_blocks * B * Hkv, dh)).reshape(n_blocks, B, Hkv, dh),
        "v_blk": normal_bf16(rng, (n_blocks * B * Hkv, dh), trunc=4.0).reshape(
            n_blocks, B, Hkv, dh),
        "q_seed": normal_bf16(rng, (n_blocks * Hq, dh)).reshape(n_blocks, Hq, dh),
        "h_seed": h_seed, "seed_targets": seed_t.astype(np.int32),
        "q_steps": normal_bf16(rng, (n_blocks * S * B * Hq, dh)).reshape(n_blocks, S, B, Hq, dh),
        "h_steps": h_steps, "final_tokens": final, "commit_step": commit_step,
    }
    if fp8:
        r["w_scale"] = w_scale
    return r


def linear_spec(seed: int | None = None, B=32, n_vis=1024, n_prompt=256, Hq=16, Hkv=2,
                dh=128, d=2048, V=151936, p_geo=0.15, sigma_w=0.02, guard=None) -> dict:
    """Linear self-speculative step, bf16: a bidirectional draft pass and a
    causal verify pass of the same B queries over the prefix.  Draft targets
    d_i ~ U{V}; verify targets equal d_i for i < L_true, differ at L_true, and
    are uniform after it; L_true = min(Geometric(p_geo), B) (support >= 1, the
    first token being the AR seed).  Each pass has its own q and its own block
    K/V rows (rows P..P+B-1 of its cache).  ``guard`` as in qwen_decode
    (target probabilities re-drawn in U(0.3, 0.999))."""
    rng = config_rng(3, seed)
    P = n_vis + n_prompt
    cap = P + B
    W = normal_bf16(rng, (V, d), std=sigma_w)
    L_true = int(min(rng.geometric(p_geo), B))
    draft_t = rng.integers(0, V, B)
    ver_t = rng.integers(0, V, B)
    ver_t[:L_true] = draft_t[:L_true]
    if L_true < B:
        ver_t[L_true] = _different_token(rng, int(draft_t[L_true]), V)
    c_d = rng.uniform(0.3, 0.999, B)
    c_v = rng.uniform(0.3, 0.999, B)
    h_d, _ = planted_bits(rng, W, draft_t, c_d, sigma_w, guard=guard,
                          redraw_conf=_uniform_redraw(0.3, 0.999))
    h_v, _ = planted_bits(rng, W, ver_t, c_v, sigma_w, guard=guard,
                          redraw_conf=_uniform_redraw(0.3, 0.999))
    kp = normal_bf16(rng, (Hkv * P, dh)).reshape(Hkv, P, dh)
    vp = normal_bf16(rng, (Hkv * P, dh), trunc=4.0).reshape(Hkv, P, dh)

    def cache(kblk, vblk):
        kc = np.concatenate([kp, kblk], axis=1)
        vc = np.concatenate([vp, vblk], axis=1)
        return kc, vc

    kd, vd = cache(normal_bf16(rng, (Hkv * B, dh)).reshape(Hkv, B, dh),
                   normal_bf16(rng, (Hkv * B, dh), trunc=4.0).reshape(Hkv, B, dh))
    kv_, vv_ = cache(normal_bf16(rng, (Hkv * B, dh)).reshape(Hkv, B, dh),
                     normal_bf16(rng, (Hkv * B, dh), trunc=4.0).reshape(Hkv, B, dh))
    return {
        "dtype": "bf16", "B": B, "P": P, "cap": cap, "Hq": Hq, "Hkv": Hkv, "dh": dh,
        "d": d, "V": V, "W": W, "L_true": L_true,
        "draft_targets": draft_t.astype(np.int32), "verify_targets": ver_t.astype(np.int32),
        "q_draft": normal_bf16(rng, (B, Hq, dh)), "q_verify": normal_bf16(rng, (B, Hq, dh)),
        "k_draft": kd, "v_draft": vd, "k_verify": kv_, "v_verify": vv_,
        "h_draft": h_d, "h_verify": h_v,
    }


def fused_spec(seed: int | None = None, B=16, n_vis=4096, n_prompt=512, Hq=16, Hkv=2,
               dh=128, d=2048, V=151936, p_geo=0.15, sigma_w=0.02, n_cert=64,
               k_cert=4, p_agree=0.83, guard=None) -> dict:
    """Fused (quadratic) speculative step, bf16: 2B query rows under the
    SPEC_FUSED mask over a 4096-visual + 512-text prefix, one LM-head pass over
    the 2B rows.  The draft tokens fed to the verify half are uniform; verify
    rows 0..B-1 are planted to agree with them over a Geometric(p_geo) prefix
    (capped at B); draft-half rows B..2B-1 get uniform targets.
    Certificate inputs: n_cert anchor confidences ~ U(0,1) (float32), anchor
    tokens ~ U{V}, text-only tokens equal to the anchor with probability
    p_agree (83.4 % agreement in the LOWN article), else a different uniform
    token; k_cert is the per-step unmask quota k.  ``guard`` as in
    linear_spec."""
    rng = config_rng(4, seed)
    P = n_vis + n_prompt
    bq = 2 * B
    cap = P + bq
    W = normal_bf16(rng, (V, d), std=sigma_w)
    L_true = int(min(rng.geometric(p_geo), B))
    draft_in = rng.integers(0, V, B)
    ver_t = rng.integers(0, V, B)
    ver_t[:L_true] = draft_in[:L_true]
    if L_true < B:
        ver_t[L_true] = _different_token(rng, int(draft_in[L_true]), V)
    next_t = rng.integers(0, V, B)
    tgt = np.concatenate([ver_t, next_t])
    c = rng.uniform(0.3, 0.999, bq)
    h, _ = planted_bits(rng, W, tgt, c, sigma_w, guard=guard,
                        redraw_conf=_uniform_redraw(0.3, 0.999))
    anchor_conf = rng.random(n_cert, dtype=np.float32)
    anchor_tok = rng.integers(0, V, n_cert)
    agree = rng.random(n_cert) < p_agree
    text_tok = anchor_tok.copy()
    for i in np.nonzero(~agree)[0]:
        text_tok[i] = _different_token(rng, int(anchor_tok[i]), V)
    return {
        "dtype": "bf16", "B": B, "Bq": bq, "P": P, "cap": cap, "Hq": Hq, "Hkv": Hkv,
        "dh": dh, "d": d, "V": V, "W": W, "h": h, "L_true": L_true,
        "draft_in": draft_in.astype(np.int32), "targets": tgt.astype(np.int32),
        "q": normal_bf16(rng, (bq, Hq, dh)),
        "k_cache": normal_bf16(rng, (Hkv * cap, dh)).reshape(Hkv, cap, dh),
        "v_cache": normal_bf16(rng, (Hkv * cap, dh), trunc=4.0).reshape(Hkv, cap, dh),
        "anchor_conf": anchor_conf, "anchor_tok": anchor_tok.astype(np.int32),
        "text_tok": text_tok.astype(np.int32), "k_cert": k_cert,
    }


def dualstream(seed: int | None = None, n_vis=1024, n_txt=2048, block=32, H=16, dh=128,
               dtype="bf16") -> dict:
    """Training-time dual-stream attention input, token order
    [visual | clean text | noisy text].  Q, K ~ N(0,1), V ~ N(0,1) truncated
    to |v| <= 4.  A mask probability t ~ U(0,1) is drawn once; each noisy
    position is replaced by [MASK] with probability t, and every [MASK]
    position carries the same Q/K/V row (one shared embedding).  d_out, the
    output gradient for the training backward, is N(0, 1) (drawn last, so the
    other tensors do not depend on it)."""
    rng = config_rng(5, seed)
    n = n_vis + 2 * n_txt
    q = normal(rng, (n, H, dh))
    k = normal(rng, (n, H, dh))
    v = normal(rng, (n, H, dh), trunc=4.0)
    t = float(rng.random())
    is_mask = rng.random(n_txt) < t
    mq, mk, mv = normal(rng, (H, dh)), normal(rng, (H, dh)), normal(rng, (H, dh), trunc=4.0)
    rows = n_vis + n_txt + np.nonzero(is_mask)[0]
    q[rows], k[rows], v[rows] = mq, mk, mv
    d_out = normal(rng, (n, H, dh))
    conv = bf16_bits if dtype == "bf16" else (lambda x: x)
    return {"dtype": dtype, "n_vis": n_vis, "n_txt": n_txt, "block": block, "H": H, "dh": dh,
            "N": n, "t": t, "is_mask": is_mask, "q": conv(q), "k": conv(k), "v": conv(v),
            "d_out": conv(d_out)}
