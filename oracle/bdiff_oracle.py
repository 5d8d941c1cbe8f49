"""Plain CPU oracle for the block-diffusion decode step and the dual-stream
training attention of Fast-dVLM.

TEST INFRASTRUCTURE ONLY.  This module exists so that tests, the smoke check
and the CPU-baseline leg of the benchmark can compute what the method defines,
slowly and in float64, and compare the GPU library against it.  Nothing on the
product path may import it, and it shares no code with the HIP library.

Sources (web pages on the method; cited by page and section):
  [OV]   Fast-dVLM engineering overview, ocdem.com/news/1032714
         - §1.2: blocks decoded left to right, parallel denoising inside a
           block, KV cache reused across blocks.
         - §2.2.1: dual noisy/clean streams and the three attention masks
           N2N / N2C / C2C, with printed 4x4 matrices for block size 2.
         - §2.2.2: visual tokens kept once, in the clean stream, reached from
           the noisy stream only through N2C; causal-context decoding.
         - §2.3.1: self-speculative decoding, longest verified prefix kept and
           the KV cache truncated; linear (two forwards) and quadratic
           (one forward, O(B^2)) variants.
         - §2.3.2: the fastest configuration adds FP8 SmoothQuant W8A8.
         - §4.1: recommended block_size 16 and denoising threshold 0.9.
  [TH]   Fast-dVLM article (itsolotime.com, Thai), §4.1 "Causal context
         attention": noisy tokens attend bidirectionally inside their block and
         to the preceding clean context including visual tokens; the clean
         stream keeps token-level causal attention.
  [LOWN] LOWN article (paper.rainbus.top/paper/2610.36671), section
         "method step details": anchor confidence s = max_w p(y_i = w | .),
         scan of masked positions in descending anchor confidence, longest
         prefix where the text-only top-1 equals the anchor top-1, and the
         branch rule |U_text| >= k.

Readings where the pages are silent (each one is listed with its reason in the
design notes of the repository):
  R1  N2C is token-level and includes the diagonal (clean j <= noisy i), as in
      the printed matrix; every visual key is visible to every noisy query.
  R2  N2N blocks tile the noisy stream from its first token.
  R3  C2C is causal over [visual | clean text], visual tokens included.
  R4  No clean query sees a noisy key.
  R5  Commit rule: masked positions with conf > tau (strict); if none
      qualifies and some position is masked, the single most confident masked
      position is committed (lowest index on ties).
  R6  Argmax ties resolve to the lowest vocabulary index.
  R7  Attention scale is 1/sqrt(dh); queries/keys are taken post-RoPE.
  R8  A query row with no visible key produces a zero output row.
  R9  Speculative accept compares index-aligned draft and verify arrays and
      accepts exactly L tokens (no bonus token) unless asked for R20's.
  R10 SPEC_FUSED (the quadratic variant's one-forward mask, whose layout the
      pages do not print) is the dual-stream mask restricted to one block:
      rows 0..B-1 (verify half, draft tokens as input) are causal among
      themselves; rows B..2B-1 (draft half) see verify row j iff j <= i-B and
      see all of the draft half.  Both halves see the whole prefix.
  R11 Certificate order: stable sort by anchor confidence, descending, lower
      index first on ties.
  R15 FP8 means OCP E4M3 for weights and activations (W8A8), float32
      accumulation, one float32 scale per vocabulary row of W.
  R16 Activations are quantized per position with the scale amax/448 (the
      row maximum maps onto the largest E4M3 value), in float32, rounding to
      nearest with ties to even.
  R17 Auto-truncation: segments (prompts, responses) start at given text
      positions; N2N blocks tile each segment from its start and end at the
      segment's end.  One segment reduces to R2.
  R18 Paged KV: the pool holds pages of page_size token rows per KV head,
      [n_pages][Hkv][page_size][dh]; a page table maps logical pages to
      physical ones.  A TEXT-ONLY forward attends the prefix from key_lo on.
  R19 FP8 KV cache: K and V are cached as E4M3 codes with one float32 scale
      per KV head for K and one for V; a cached entry stands for
      decode(code) * scale.  New rows are quantized as code = E4M3 rounding of
      fl32(x * fl32(1 / scale)), clamped to [-448, 448] first (float32 steps,
      as in R16).
  R20 Bonus token (optional; the pages do not state one): at the first
      disagreement L < B the verify pass's own token verify[L] is taken as
      well, as greedy speculative decoding does (Leviathan et al. 2023, "Fast
      Inference from Transformers via Speculative Decoding", and Chen et al.
      2023, speculative sampling, both with a greedy target); L + 1 tokens
      are appended and kv_len stays P + L (the K/V row of position L was
      computed from the rejected draft token).  With L = B nothing is added.

Every function below takes float64 (or integer) arrays and returns new arrays;
bfloat16 inputs are passed as raw uint16 bit patterns and widened exactly.
The FP8 functions follow the OCP 8-bit floating point specification (OFP8)
for the E4M3 format; their quantization step is taken in float32 (R16).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "widen", "mask_n2n", "mask_n2c", "mask_c2c", "dualstream_mask",
    "intra_block_mask", "masked_attention", "block_attn", "paged_rows", "block_attn_paged",
    "kv_quant_fp8", "kv_dequant_fp8", "block_attn_fp8kv",
    "dualstream_attn",
    "dualstream_lse", "dualstream_attn_bwd", "dualstream_attn_bwd_given",
    "lm_logits", "conf_argmax", "lmhead_conf", "E4M3_MAX", "e4m3_decode", "e4m3_encode",
    "quant_fp8_rows", "lm_logits_fp8", "lmhead_conf_fp8", "commit", "spec_accept", "cert_scan",
    "decode_step", "block_loop", "decode_blocks", "linear_spec_step", "fused_spec_step",
]


# ---------------------------------------------------------------------------
# Input widening
# ---------------------------------------------------------------------------

def widen(x) -> np.ndarray:
    """Return ``x`` as float64.  uint16 arrays are bfloat16 bit patterns: the
    16 bits are the top half of an IEEE float32, so shifting them into place
    gives the exact value, which float64 then holds exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# Masks  [OV §2.2.1, §2.2.2; TH §4.1]
# ---------------------------------------------------------------------------

def mask_n2n(n_txt: int, block: int, seg_starts=None) -> np.ndarray:
    """Noisy -> noisy: bidirectional inside a block of ``block`` tokens, blocks
    tiling the noisy stream from its first token (R2).  [OV §2.2.1 'N2N']

    With ``seg_starts`` (the auto-truncation mask, R17): the text is split
    into segments (the turns' prompts and responses) starting at the given
    text positions; blocks tile every segment from its own start, and a block
    ends at its segment's end, so no block crosses into the next segment.
    [OV §2.2.2 auto-truncation mask; TH §4.3]"""
    starts = [0] if seg_starts is None else [int(x) for x in seg_starts]
    label = []
    for r in range(n_txt):
        s = max(k for k in range(len(starts)) if starts[k] <= r)
        label.append((s, (r - starts[s]) // block))
    m = np.zeros((n_txt, n_txt), dtype=bool)
    for i in range(n_txt):
        for j in range(n_txt):
            m[i, j] = label[i] == label[j]
    return m


def mask_n2c(n_txt: int) -> np.ndarray:
    """Noisy text i -> clean text j, visible iff j <= i (R1).
    [OV §2.2.1 'N2C', printed lower-triangular matrix]"""
    i = np.arange(n_txt)[:, None]
    j = np.arange(n_txt)[None, :]
    return j <= i


def mask_c2c(n: int) -> np.ndarray:
    """Clean -> clean: token-level causal attention.  [OV §2.2.1 'C2C';
    TH §4.1 item 3]"""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return j <= i


def dualstream_mask(n_vis: int, n_txt: int, block: int, seg_starts=None) -> np.ndarray:
    """Full boolean mask over the token order [visual | clean text | noisy
    text] (vision-efficient concatenation: one copy of the visual tokens,
    in the clean stream).  Row = query, column = key.  ``seg_starts`` selects
    the auto-truncated N2N blocks (see mask_n2n).  [OV §2.2.1, §2.2.2]"""
    ctx = n_vis + n_txt
    n = ctx + n_txt
    m = np.zeros((n, n), dtype=bool)
    m[:ctx, :ctx] = mask_c2c(ctx)                 # C2C over [vis | clean] (R3)
    m[ctx:, :n_vis] = True                        # noisy -> every visual key (R1)
    m[ctx:, n_vis:ctx] = mask_n2c(n_txt)          # N2C
    m[ctx:, ctx:] = mask_n2n(n_txt, block, seg_starts)   # N2N
    # clean -> noisy stays False (R4)
    return m


def intra_block_mask(kind: str, bq: int) -> np.ndarray:
    """Visibility among the Bq block queries at decode time.
    'bidir'      - all ones (N2N over one block)          [OV §1.2]
    'causal'     - j <= i (the AR verify pass)             [OV §2.3.1]
    'spec_fused' - reading R10, Bq = 2B                    [OV §2.3.1]"""
    i = np.arange(bq)[:, None]
    j = np.arange(bq)[None, :]
    if kind == "bidir":
        return np.ones((bq, bq), dtype=bool)
    if kind == "causal":
        return j <= i
    if kind == "spec_fused":
        if bq % 2:
            raise ValueError("spec_fused needs an even number of rows")
        b = bq // 2
        m = np.zeros((bq, bq), dtype=bool)
        m[:b, :b] = mask_c2c(b)          # verify half: causal
        m[b:, :b] = mask_n2c(b)          # draft half -> verify half: j <= i - B
        m[b:, b:] = mask_n2n(b, b)       # draft half: one bidirectional block
        return m
    raise ValueError(f"unknown mask kind {kind!r}")


# ---------------------------------------------------------------------------
# Attention (scaled dot-product over the allowed keys; R7, R8)
# ---------------------------------------------------------------------------

def masked_attention(q, k, v, allowed, scale: float) -> np.ndarray:
    """o_i = sum_j softmax_j(scale * q_i . k_j) v_j over the keys j with
    allowed[i, j]; a row with no allowed key is zero (R8).
    q [Nq][dh], k/v [Nk][dh], allowed [Nq][Nk] bool."""
    q = widen(q)
    k = widen(k)
    v = widen(v)
    allowed = np.asarray(allowed, dtype=bool)
    s = scale * (q @ k.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(s - m)                      # exp(-inf) = 0 for hidden keys
    den = w.sum(axis=1, keepdims=True)
    return (w @ v) / np.where(den > 0.0, den, 1.0)


def block_attn(q, k_cache, v_cache, P: int, intra, scale: float | None = None) -> np.ndarray:
    """Block queries over the cached prefix plus the block itself.
    q [Bq][Hq][dh]; k_cache/v_cache [Hkv][cap][dh] with the block's own keys at
    rows P..P+Bq-1.  Prefix keys are always visible; block key j is visible to
    query i iff intra[i, j].  Query head h reads KV head h // (Hq / Hkv).
    [OV §1.2: cached visual+prompt prefix, bidirectional block]"""
    q = widen(q)
    k_cache = widen(k_cache)
    v_cache = widen(v_cache)
    bq, hq, dh = q.shape
    hkv = k_cache.shape[0]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    allowed = np.zeros((bq, P + bq), dtype=bool)
    allowed[:, :P] = True
    allowed[:, P:] = np.asarray(intra, dtype=bool)
    group = hq // hkv
    out = np.zeros((bq, hq, dh))
    for h in range(hq):
        g = h // group
        out[:, h, :] = masked_attention(q[:, h, :], k_cache[g, :P + bq], v_cache[g, :P + bq],
                                        allowed, scale)
    return out


def paged_rows(pool, page_table, page_size: int, n: int) -> np.ndarray:
    """Logical K or V rows 0..n-1 of a paged cache, [Hkv][n][dh]: logical
    position j of KV head g lives at pool[page_table[j // page_size]][g]
    [j % page_size] (pool [n_pages][Hkv][page_size][dh]).  [OV §2.3.2: the
    serving system manages the KV cache in pages]"""
    pool = np.asarray(pool)
    table = np.asarray(page_table)
    hkv = pool.shape[1]
    out = np.empty((hkv, n, pool.shape[3]), dtype=pool.dtype)
    for j in range(n):
        out[:, j, :] = pool[int(table[j // page_size]), :, j % page_size, :]
    return out


def block_attn_paged(q, k_pool, v_pool, page_table, page_size: int, P: int, intra,
                     key_lo: int = 0, scale: float | None = None) -> np.ndarray:
    """bd_block_attn over a paged KV cache, with the prefix keys below key_lo
    left out (key_lo = the number of visual tokens gives LOWN's TEXT-ONLY
    forward, which skips the visual keys [LOWN 'method step details'; R18]):
    the logical rows [key_lo, P + Bq) gathered from the pages, attended as
    block_attn attends a contiguous cache."""
    bq = q.shape[0]
    kl = paged_rows(k_pool, page_table, page_size, P + bq)[:, key_lo:]
    vl = paged_rows(v_pool, page_table, page_size, P + bq)[:, key_lo:]
    return block_attn(q, kl, vl, P - key_lo, intra, scale)


def kv_dequant_fp8(codes, scale) -> np.ndarray:
    """Values of an FP8 KV cache (R19): codes [Hkv][rows][dh] uint8, scale
    [Hkv] float32; entry = decode(code) * scale[head], in float64."""
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return e4m3_decode(codes) * sc[:, None, None]


def kv_quant_fp8(x, scale) -> np.ndarray:
    """E4M3 codes of new K or V rows for an FP8 cache (R19), in float32 steps:
    inv = fl32(1 / scale[g]); y = fl32(x * inv), clamped to [-448, 448];
    code = the E4M3 rounding of y (ties to even).
    x: [n][Hkv][dh] bfloat16 bits (uint16) or float32; scale [Hkv] float32.
    Returns codes [n][Hkv][dh] uint8 (the caller places them in the cache)."""
    x = np.asarray(x)
    x32 = widen(x).astype(np.float32) if x.dtype == np.uint16 else x.astype(np.float32)
    inv = (np.float32(1) / np.asarray(scale, dtype=np.float32)).astype(np.float32)
    y = (x32 * inv[None, :, None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y.astype(np.float64))


def block_attn_fp8kv(q, k_codes, v_codes, k_scale, v_scale, P: int, intra,
                     scale: float | None = None) -> np.ndarray:
    """bd_block_attn over an FP8 KV cache (R19): the cache's values are
    decode(code) * scale of their KV head, attended as block_attn attends a
    bfloat16 cache.  [OV §2.3.2: the fastest configuration runs FP8]"""
    return block_attn(q, kv_dequant_fp8(k_codes, k_scale), kv_dequant_fp8(v_codes, v_scale),
                      P, intra, scale)


def dualstream_attn(q, k, v, n_vis: int, n_txt: int, block: int,
                    scale: float | None = None, rows=None, seg_starts=None) -> np.ndarray:
    """Training-time attention over [visual | clean text | noisy text] with the
    N2N / N2C / C2C masks.  q/k/v [N][H][dh].  If ``rows`` is given, only those
    query rows are computed (returned in that order), for spot checks at large
    N.  ``seg_starts`` applies the auto-truncation mask.  [OV §2.2.1, §2.2.2;
    TH §4.1]"""
    q = widen(q)
    k = widen(k)
    v = widen(v)
    n, nh, dh = q.shape
    if n != n_vis + 2 * n_txt:
        raise ValueError("N must equal n_vis + 2 * n_txt")
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    allowed = dualstream_mask(n_vis, n_txt, block, seg_starts)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    out = np.zeros((rows.size, nh, dh))
    for h in range(nh):
        out[:, h, :] = masked_attention(q[rows, h, :], k[:, h, :], v[:, h, :],
                                        allowed[rows], scale)
    return out


def dualstream_lse(q, k, n_vis: int, n_txt: int, block: int, scale: float | None = None,
                   seg_starts=None) -> np.ndarray:
    """Row log-sum-exp of the masked, scaled scores, natural log, [N][H]:
    lse[i, h] = log sum_{j visible from i} exp(scale q_i . k_j).  It is what a
    training forward keeps for the backward (P = exp(scale S - lse)).
    [OV §2.2.1, §2.2.2]"""
    q = widen(q)
    k = widen(k)
    n, nh, dh = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    allowed = dualstream_mask(n_vis, n_txt, block, seg_starts)
    out = np.empty((n, nh))
    for h in range(nh):
        s = scale * (q[:, h, :] @ k[:, h, :].T)
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1)
        out[:, h] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def dualstream_attn_bwd(q, k, v, d_out, n_vis: int, n_txt: int, block: int,
                        scale: float | None = None, seg_starts=None):
    """Gradients of the dual-stream attention with respect to q, k and v for
    the output gradient d_out, per head, from the definition of masked
    softmax attention O = P V, P = softmax_row(scale Q K^T + mask):
        dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(P * dP)),
        dQ = scale dS K,   dK = scale dS^T Q.
    All [N][H][dh], float64.  Training the dual-stream model needs this pass
    [OV §2.2.1; TH §4.1]."""
    q = widen(q)
    k = widen(k)
    v = widen(v)
    g = widen(d_out)
    n, nh, dh = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    allowed = dualstream_mask(n_vis, n_txt, block, seg_starts)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(nh):
        s = scale * (q[:, h, :] @ k[:, h, :].T)
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.where(allowed, np.exp(s - m), 0.0)
        p = e / e.sum(axis=1, keepdims=True)
        dv[:, h, :] = p.T @ g[:, h, :]
        dp = g[:, h, :] @ v[:, h, :].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[:, h, :] = scale * (ds @ k[:, h, :])
        dk[:, h, :] = scale * (ds.T @ q[:, h, :])
    return dq, dk, dv


def dualstream_attn_bwd_given(q, k, v, out, lse, d_out, n_vis: int, n_txt: int, block: int,
                              scale: float | None = None, seg_starts=None):
    """The training backward as a backward pass computes it from what the
    forward kept: the probabilities from the given row log-sum-exp lse [N][H]
    (natural log), P = exp(scale Q K^T - lse) on visible pairs, and
    D = rowsum(dO * out) from the given forward output out [N][H][dh]:
        dV = P^T dO,   dS = P * (dO V^T - D),   dQ = scale dS K,
        dK = scale dS^T Q.
    With the exact out and lse it equals dualstream_attn_bwd; with a rounded
    out it shows what that rounding does to the gradients.  All float64.
    [OV §2.2.1; TH §4.1]"""
    q = widen(q)
    k = widen(k)
    v = widen(v)
    o = widen(out)
    g = widen(d_out)
    lse = np.asarray(lse, dtype=np.float64)
    n, nh, dh = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    allowed = dualstream_mask(n_vis, n_txt, block, seg_starts)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(nh):
        s = scale * (q[:, h, :] @ k[:, h, :].T)
        p = np.where(allowed, np.exp(np.where(allowed, s, 0.0) - lse[:, h:h + 1]), 0.0)
        dv[:, h, :] = p.T @ g[:, h, :]
        dp = g[:, h, :] @ v[:, h, :].T
        d = (g[:, h, :] * o[:, h, :]).sum(axis=1, keepdims=True)
        ds = p * (dp - d)
        dq[:, h, :] = scale * (ds @ k[:, h, :])
        dk[:, h, :] = scale * (ds.T @ q[:, h, :])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# LM head confidence  [LOWN 'method step details': s = max_w p(y = w | .)]
# ---------------------------------------------------------------------------

def lm_logits(h, W, chunk: int = 16384) -> np.ndarray:
    """logits[b, v] = sum_k h[b, k] W[v, k], in float64 (W widened in row
    chunks to bound memory; the sum over k is not reordered)."""
    h = widen(h)
    W = np.asarray(W)
    V = W.shape[0]
    out = np.empty((h.shape[0], V))
    for s in range(0, V, chunk):
        out[:, s:s + chunk] = h @ widen(W[s:s + chunk]).T
    return out


def conf_argmax(logits):
    """Per row: argmax token (lowest index on ties, R6) and confidence = the
    largest softmax probability = 1 / sum_v exp(l_v - max l)."""
    m = logits.max(axis=1)
    a = np.argmax(logits, axis=1)          # numpy returns the first maximum
    s = np.exp(logits - m[:, None]).sum(axis=1)
    return 1.0 / s, a.astype(np.int64)


def lmhead_conf(h, W):
    """Confidence and argmax of the logits h W^T (see conf_argmax)."""
    return conf_argmax(lm_logits(h, W))


# ---------------------------------------------------------------------------
# FP8 (W8A8) LM head  [OV §2.3.2: FP8 SmoothQuant W8A8 in the fastest
# configuration; OV §4.1 quant_mode fp8]
#
# Number format: OCP 8-bit floating point (OFP8) E4M3.  Bit 7 is the sign,
# bits 6..3 a biased exponent (bias 7), bits 2..0 the mantissa.  Exponent
# field 0 encodes subnormals (m/8) 2^-6; the all-ones pattern S.1111.111 is
# NaN; every other code is (1 + m/8) 2^(e-7).  No infinities; the largest
# finite magnitude is 448.
#
# W8A8 (R15, R16): every vocabulary row of W is stored as E4M3 codes with one
# float32 scale (per-output-channel weight quantization, done offline); the
# hidden states are quantized per position at run time (per-token dynamic
# activation quantization).  SmoothQuant's smoothing factors are folded into
# the weights and the preceding layer offline, so they do not appear here.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Exact value of E4M3 codes as float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


_E4M3_POS = None


def _e4m3_positive_values() -> np.ndarray:
    """Values of codes 0x00..0x7E (every non-negative finite E4M3 value), which
    increase with the code."""
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = e4m3_decode(np.arange(0x7F))
    return _E4M3_POS


def e4m3_encode(y) -> np.ndarray:
    """Round finite values with |y| <= 448 to the nearest E4M3 value, ties to
    the even code (mantissa bit 0 clear).  The sign bit is taken from y, so a
    negative value that rounds to zero (and -0.0) gives 0x80."""
    y = np.asarray(y, dtype=np.float64)
    if not (np.isfinite(y).all() and (np.abs(y) <= E4M3_MAX).all()):
        raise ValueError("e4m3_encode needs finite inputs with |y| <= 448")
    tab = _e4m3_positive_values()
    a = np.abs(y)
    hi = np.minimum(np.searchsorted(tab, a, side="left"), tab.size - 1)   # tab[hi] >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - tab[lo]
    d_hi = tab[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quant_fp8_rows(x):
    """Per-row dynamic quantization to E4M3 (R16).  The steps are taken in
    float32, the precision in which the kernels take the same rounding
    decisions:  amax = max_k |x_k|;  r = 448 / amax and s = amax / 448, each
    rounded to float32 (r = s = 1 for an all-zero row);  code_k = the E4M3
    rounding of fl32(x_k * r), clamped to [-448, 448] first (the product can
    exceed 448 by an ulp).  Then s * decode(code_k) ~ x_k.
    x: [R][d] bfloat16 bits (uint16) or float32.  Returns (codes uint8 [R][d],
    s float32 [R])."""
    x = np.asarray(x)
    x32 = widen(x).astype(np.float32) if x.dtype == np.uint16 else x.astype(np.float32)
    amax = np.abs(x32).max(axis=1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1))
    r = np.where(nz, np.float32(E4M3_MAX) / safe, np.float32(1)).astype(np.float32)
    s = np.where(nz, safe / np.float32(E4M3_MAX), np.float32(1)).astype(np.float32)
    y = (x32 * r[:, None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y.astype(np.float64)), s


def lm_logits_fp8(h, Wq, w_scale, chunk: int = 16384) -> np.ndarray:
    """W8A8 logits in float64: with (qh, sh) = quant_fp8_rows(h),
        logits[b, v] = sh[b] * w_scale[v] * sum_k dec(qh[b, k]) dec(Wq[v, k]).
    Wq: [V][d] E4M3 codes (uint8), w_scale: [V] float32."""
    qh, sh = quant_fp8_rows(h)
    A = e4m3_decode(qh)
    Wq = np.asarray(Wq)
    ws = np.asarray(w_scale, dtype=np.float64)
    V = Wq.shape[0]
    out = np.empty((A.shape[0], V))
    for s in range(0, V, chunk):
        dot = A @ e4m3_decode(Wq[s:s + chunk]).T
        out[:, s:s + chunk] = dot * sh.astype(np.float64)[:, None] * ws[None, s:s + chunk]
    return out


def lmhead_conf_fp8(h, Wq, w_scale):
    """Confidence and argmax of the W8A8 logits (see lm_logits_fp8)."""
    return conf_argmax(lm_logits_fp8(h, Wq, w_scale))


# ---------------------------------------------------------------------------
# Commit, accept, certificate
# ---------------------------------------------------------------------------

def commit(conf, argmax, masked, tokens, tau: float):
    """Threshold unmasking [OV §4.1 threshold 0.9] with the always-one rule
    (R5).  Returns (masked_out, tokens_out, n_committed)."""
    conf = np.asarray(conf, dtype=np.float64)
    masked = np.asarray(masked).astype(np.uint8).copy()
    tokens = np.asarray(tokens).astype(np.int64).copy()
    b = conf.shape[0]
    chosen = [i for i in range(b) if masked[i] and conf[i] > tau]
    if not chosen:
        best = None
        for i in range(b):
            if masked[i] and (best is None or conf[i] > conf[best]):
                best = i
        if best is not None:
            chosen = [best]
    for i in chosen:
        tokens[i] = int(argmax[i])
        masked[i] = 0
    return masked, tokens, len(chosen)


def spec_accept(draft, verify, P: int, bonus: bool = False):
    """Longest prefix where the diffusion draft equals the causal verify pass;
    the KV cache is truncated to P + L and the L accepted tokens are appended.
    [OV §2.3.1]  With bonus (R20), a first disagreement at L < B also appends
    the verify pass's token there.  Returns (number of tokens appended,
    kv_len, appended tokens)."""
    draft = np.asarray(draft).astype(np.int64)
    verify = np.asarray(verify).astype(np.int64)
    L = 0
    while L < draft.shape[0] and draft[L] == verify[L]:
        L += 1
    tokens = draft[:L].copy()
    if bonus and L < draft.shape[0]:
        tokens = np.append(tokens, verify[L])
    return tokens.shape[0], P + L, tokens


def cert_scan(anchor_conf, anchor_tok, text_tok, k: int):
    """LOWN certificate: order the masked positions by anchor confidence
    (descending, R11), walk that order while the text-only top-1 equals the
    anchor top-1; the walk length is |U_text|, and the image forward can be
    skipped iff |U_text| >= k.  [LOWN 'method step details' (2), (3)]
    Returns (order, L, skip_full)."""
    conf = np.asarray(anchor_conf, dtype=np.float64)
    anchor_tok = np.asarray(anchor_tok)
    text_tok = np.asarray(text_tok)
    n = conf.shape[0]
    order = sorted(range(n), key=lambda i: (-conf[i], i))
    L = 0
    while L < n and text_tok[order[L]] == anchor_tok[order[L]]:
        L += 1
    return np.asarray(order, dtype=np.int64), L, int(L >= k)


# ---------------------------------------------------------------------------
# Compositions
# ---------------------------------------------------------------------------

def decode_step(q, k_cache, v_cache, P, h, W, masked, tokens, tau, kind="bidir",
                w_scale=None):
    """One threshold (MDM) block-decode step: block attention over the prefix,
    LM-head confidence, commit.  The attention output and the LM-head input are
    separate tensors because the remaining transformer layers sit between them.
    With ``w_scale`` given, W holds E4M3 codes and the LM head is the W8A8 one.
    [OV §1.2, §4.1]"""
    bq = q.shape[0]
    o = block_attn(q, k_cache, v_cache, P, intra_block_mask(kind, bq))
    conf, a = lmhead_conf(h, W) if w_scale is None else lmhead_conf_fp8(h, W, w_scale)
    m2, t2, n = commit(conf, a, masked, tokens, tau)
    return {"attn": o, "conf": conf, "argmax": a, "masked": m2, "tokens": t2, "n_committed": n}


def block_loop(q_steps, k_cache, v_cache, P, h_steps, W, masked, tokens, tau, kind="bidir",
               w_scale=None):
    """The block loop: decode steps on one block while any position is still
    masked, at most S = len(h_steps) steps; step s takes the block queries
    q_steps[s] and hidden rows h_steps[s] (the inputs the model's other
    layers would produce at that step).  [OV §1.2: a block is denoised in
    parallel over several steps before the next one starts; OV §4.1:
    threshold 0.9]  Returns the final block state, the number of steps run,
    the commits of every step (0 for steps not run) and the outputs of the
    steps that ran."""
    masked = np.asarray(masked).astype(np.uint8).copy()
    tokens = np.asarray(tokens).astype(np.int64).copy()
    S = len(h_steps)
    n_comm = np.zeros(S, dtype=np.int64)
    attn, conf, argmax = [], [], []
    for s in range(S):
        if not masked.any():
            break
        o = decode_step(q_steps[s], k_cache, v_cache, P, h_steps[s], W, masked, tokens, tau,
                        kind, w_scale)
        masked, tokens = o["masked"], o["tokens"]
        n_comm[s] = o["n_committed"]
        attn.append(o["attn"])
        conf.append(o["conf"])
        argmax.append(o["argmax"])
    return {"masked": masked, "tokens": tokens, "n_steps": len(conf), "n_committed": n_comm,
            "attn": attn, "conf": conf, "argmax": argmax}


def decode_blocks(q_seed, h_seed, q_steps, h_steps, k_blk, v_blk, k_cache, v_cache, P0, W, tau,
                  w_scale=None):
    """Several blocks decoded in order, each after the ones before it has
    joined the KV cache.  [OV §1.2: blocks are generated one after another,
    each denoised in parallel over several steps, with the KV cache of the
    earlier ones reused; OV §2.2.2: causal-context decoding, the first token
    of a block comes from the AR (causal) prediction]

    The KV length starts at P0 (the prompt prefix).  For block b:
      1. its own K/V rows k_blk[b], v_blk[b] ([B][Hkv][dh], the rows the
         model's projections give for the block) are written into the cache
         rows kv_len .. kv_len + B - 1;
      2. AR seed: the query q_seed[b] ([Hq][dh]) attends the cached prefix
         [0, kv_len) (the block's own rows are not visible to it), and the
         argmax of the LM head on h_seed[b] ([d]) becomes the block's first
         token; positions 1 .. B-1 start masked;
      3. the block loop (block_loop) over q_steps[b], h_steps[b] with the
         prefix length kv_len and the block's rows as its keys;
      4. kv_len += B: the block becomes part of the prefix.
    Caches are bfloat16 bit patterns ([Hkv][cap][dh]); copies are updated
    and returned.  Returns the final cache, kv_len, and per block the seed's
    attention output, confidence and token and the block loop's results."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    nb = len(h_steps)
    B = np.asarray(k_blk).shape[1]
    kv = int(P0)
    blocks = []
    for b in range(nb):
        kc[:, kv:kv + B, :] = np.transpose(np.asarray(k_blk[b]), (1, 0, 2))
        vc[:, kv:kv + B, :] = np.transpose(np.asarray(v_blk[b]), (1, 0, 2))
        seed_attn = block_attn(np.asarray(q_seed[b])[None], kc, vc, kv,
                               np.zeros((1, 1), dtype=bool))[0]
        h1 = np.asarray(h_seed[b])[None]
        sc, sa = lmhead_conf(h1, W) if w_scale is None else lmhead_conf_fp8(h1, W, w_scale)
        tokens = np.zeros(B, dtype=np.int64)
        tokens[0] = sa[0]
        masked = np.ones(B, dtype=np.uint8)
        masked[0] = 0
        o = block_loop(q_steps[b], kc, vc, kv, h_steps[b], W, masked, tokens, tau,
                       w_scale=w_scale)
        o.update(seed_attn=seed_attn, seed_conf=float(sc[0]), seed_token=int(sa[0]), P=kv)
        blocks.append(o)
        kv += B
    return {"k_cache": kc, "v_cache": vc, "kv_len": kv, "blocks": blocks}


def linear_spec_step(q_draft, kc_draft, vc_draft, q_verify, kc_verify, vc_verify, P,
                     h_draft, h_verify, W):
    """Linear self-speculative step: a bidirectional draft forward, a causal
    verify forward, then longest-prefix accept.  [OV §2.3.1, two forwards]"""
    bq = q_draft.shape[0]
    o_d = block_attn(q_draft, kc_draft, vc_draft, P, intra_block_mask("bidir", bq))
    _, draft = lmhead_conf(h_draft, W)
    o_v = block_attn(q_verify, kc_verify, vc_verify, P, intra_block_mask("causal", bq))
    _, verify = lmhead_conf(h_verify, W)
    L, kv_len, acc = spec_accept(draft, verify, P)
    return {"attn_draft": o_d, "attn_verify": o_v, "draft": draft, "verify": verify,
            "accepted": L, "kv_len": kv_len, "out_tokens": acc}


def fused_spec_step(q, k_cache, v_cache, P, h, W, draft_in):
    """Quadratic (fused) speculative step: one forward of 2B rows under the
    SPEC_FUSED mask (R10), one LM-head pass over the 2B rows; rows 0..B-1 give
    the verify tokens for the draft tokens that were fed in; rows B..2B-1 give
    the next draft.  [OV §2.3.1, one forward]"""
    bq = q.shape[0]
    b = bq // 2
    o = block_attn(q, k_cache, v_cache, P, intra_block_mask("spec_fused", bq))
    conf, a = lmhead_conf(h, W)
    L, kv_len, acc = spec_accept(draft_in, a[:b], P)
    return {"attn": o, "conf": conf, "argmax": a, "accepted": L, "kv_len": kv_len,
            "out_tokens": acc, "next_draft": a[b:]}
