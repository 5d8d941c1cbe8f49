"""Pins of the oracle's attention against library routines, closed forms and
invariants (float64, CPU).

The pages give no attention formula or numeric example, so the oracle's
attention is pinned to torch's scaled_dot_product_attention (a library
routine, run here in float64 on the CPU) in the cases where the two must
agree, plus invariants that any correct masked softmax attention satisfies.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from block_diffusion_vlm_amd import synth


def _sdpa(q, k, v, mask=None, causal=False, gqa=False):
    """q [Nq][H][dh], k/v [Nk][Hk][dh] -> [Nq][H][dh] through torch SDPA."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(np.transpose(x, (1, 0, 2))))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, is_causal=causal,
                                       enable_gqa=gqa)
    return o[0].numpy().transpose(1, 0, 2)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_all_ones_mask_equals_dense_attention():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 9, 1, 16), _rand(rng, 13, 1, 16), _rand(rng, 13, 1, 16)
    o = oracle.masked_attention(q[:, 0], k[:, 0], v[:, 0], np.ones((9, 13), bool), 0.25)
    ref = _sdpa(q, k, v)[:, 0]
    assert np.abs(o - ref).max() <= 1e-12


def test_causal_mask_equals_library_causal():
    rng = np.random.default_rng(2)
    q, k, v = (_rand(rng, 11, 1, 16) for _ in range(3))
    o = oracle.masked_attention(q[:, 0], k[:, 0], v[:, 0], oracle.mask_c2c(11), 0.25)
    assert np.abs(o - _sdpa(q, k, v, causal=True)[:, 0]).max() <= 1e-12


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 4, 8), _rand(rng, 6, 8), _rand(rng, 6, 8)
    allowed = np.zeros((4, 6), bool)
    for i, j in enumerate([5, 0, 3, 3]):
        allowed[i, j] = True
    o = oracle.masked_attention(q, k, v, allowed, 1.0)
    assert np.array_equal(o, v[[5, 0, 3, 3]])


def test_row_without_visible_key_is_zero():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 3, 8), _rand(rng, 5, 8), _rand(rng, 5, 8)
    allowed = np.ones((3, 5), bool)
    allowed[1] = False
    o = oracle.masked_attention(q, k, v, allowed, 1.0)
    assert np.array_equal(o[1], np.zeros(8)) and np.abs(o[0]).sum() > 0


def test_key_permutation_invariance():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 7, 16), _rand(rng, 20, 16), _rand(rng, 20, 16)
    allowed = rng.random((7, 20)) < 0.6
    allowed[:, 0] = True
    perm = rng.permutation(20)
    a = oracle.masked_attention(q, k, v, allowed, 0.3)
    b = oracle.masked_attention(q, k[perm], v[perm], allowed[:, perm], 0.3)
    assert np.abs(a - b).max() <= 1e-12


def test_causal_rows_ignore_future_keys():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 10, 16), _rand(rng, 10, 16), _rand(rng, 10, 16)
    m = oracle.mask_c2c(10)
    a = oracle.masked_attention(q, k, v, m, 0.3)
    k2, v2 = k.copy(), v.copy()
    k2[6:] += 5.0
    v2[6:] -= 3.0
    b = oracle.masked_attention(q, k2, v2, m, 0.3)
    assert np.array_equal(a[:6], b[:6]) and np.abs(a[6:] - b[6:]).max() > 1e-3


@pytest.mark.parametrize("kind", ["bidir", "causal"])
def test_block_attn_gqa_equals_library(kind):
    rng = np.random.default_rng(7)
    bq, hq, hkv, dh, P = 6, 8, 2, 16, 21
    q = _rand(rng, bq, hq, dh)
    kc, vc = _rand(rng, hkv, P + bq + 3, dh), _rand(rng, hkv, P + bq + 3, dh)
    o = oracle.block_attn(q, kc, vc, P, oracle.intra_block_mask(kind, bq))
    k = kc[:, :P + bq].transpose(1, 0, 2)
    v = vc[:, :P + bq].transpose(1, 0, 2)
    mask = None
    if kind == "causal":  # prefix visible, then causal over the block (offset tril)
        mask = torch.ones(bq, P + bq, dtype=torch.bool).tril(diagonal=P).numpy()
    ref = _sdpa(q, k, v, mask=mask, gqa=True)
    assert np.abs(o - ref).max() <= 1e-12


def test_block_attn_spec_fused_equals_gathered_keys():
    # Each fused row equals plain attention over exactly the keys its reading
    # makes visible, gathered by index (no mask matrix involved).
    rng = np.random.default_rng(8)
    b, hq, hkv, dh, P = 3, 4, 2, 16, 10
    bq = 2 * b
    q = _rand(rng, bq, hq, dh)
    kc, vc = _rand(rng, hkv, P + bq, dh), _rand(rng, hkv, P + bq, dh)
    o = oracle.block_attn(q, kc, vc, P, oracle.intra_block_mask("spec_fused", bq))
    for i in range(bq):
        if i < b:
            keys = list(range(P)) + [P + j for j in range(i + 1)]
        else:
            keys = list(range(P)) + [P + j for j in range(i - b + 1)] + [P + b + j for j in range(b)]
        for h in range(hq):
            g = h // (hq // hkv)
            ref = _sdpa(q[i:i + 1, h:h + 1], kc[g, keys][:, None], vc[g, keys][:, None])
            assert np.abs(o[i, h] - ref[0, 0]).max() <= 1e-12


def test_dualstream_clean_rows_equal_causal_attention_over_clean_stream():
    rng = np.random.default_rng(9)
    n_vis, n_txt, b, H, dh = 5, 8, 4, 2, 16
    n = n_vis + 2 * n_txt
    q, k, v = (_rand(rng, n, H, dh) for _ in range(3))
    o = oracle.dualstream_attn(q, k, v, n_vis, n_txt, b)
    ctx = n_vis + n_txt
    ref = _sdpa(q[:ctx], k[:ctx], v[:ctx], causal=True)
    assert np.abs(o[:ctx] - ref).max() <= 1e-12


def test_dualstream_noisy_rows_equal_gathered_keys():
    rng = np.random.default_rng(10)
    n_vis, n_txt, b, H, dh = 5, 9, 4, 2, 16
    n = n_vis + 2 * n_txt
    q, k, v = (_rand(rng, n, H, dh) for _ in range(3))
    o = oracle.dualstream_attn(q, k, v, n_vis, n_txt, b)
    ctx = n_vis + n_txt
    for r in range(n_txt):
        blk0 = (r // b) * b
        keys = (list(range(n_vis)) + [n_vis + c for c in range(r + 1)]
                + [ctx + j for j in range(blk0, min(blk0 + b, n_txt))])
        ref = _sdpa(q[ctx + r:ctx + r + 1], k[keys], v[keys])
        assert np.abs(o[ctx + r] - ref[0]).max() <= 1e-12


def test_dualstream_rows_subset_matches_full():
    r = synth.tiny()
    full = oracle.dualstream_attn(r["ds_q"], r["ds_k"], r["ds_v"], 4, 4, 2)
    rows = np.array([11, 0, 6])
    part = oracle.dualstream_attn(r["ds_q"], r["ds_k"], r["ds_v"], 4, 4, 2, rows=rows)
    assert np.array_equal(part, full[rows])


def test_widen_bf16_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000], np.uint16)
    vals = oracle.widen(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[5] == 0.0
    assert vals[2] == 3.140625                      # 0x4049 = 0 10000000 1001001
    assert vals[3] == 2.0 ** -133                   # smallest bf16 subnormal
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127    # largest finite bf16


# ---------------------------------------------------------------------------
# Paged KV cache and the key-range start  [OV §2.3.2 paged KV; LOWN TEXT-ONLY]
# ---------------------------------------------------------------------------

def _paged_case(seed, P=37, bq=5, hq=4, hkv=2, dh=8, ps=4, extra_pages=3):
    rng = np.random.default_rng(seed)
    n = P + bq
    n_log = -(-n // ps)
    n_phys = n_log + extra_pages
    table = rng.permutation(n_phys)[:n_log]
    k_pool = rng.standard_normal((n_phys, hkv, ps, dh))
    v_pool = rng.standard_normal((n_phys, hkv, ps, dh))
    q = rng.standard_normal((bq, hq, dh))
    intra = rng.random((bq, bq)) < 0.6
    np.fill_diagonal(intra, True)
    return q, k_pool, v_pool, table, ps, P, intra


def test_paged_rows_follow_the_page_table():
    q, kp, vp, table, ps, P, intra = _paged_case(0)
    rows = oracle.paged_rows(kp, table, ps, P + q.shape[0])
    for j in (0, 3, 4, 17, P + 2):
        assert np.array_equal(rows[:, j], kp[table[j // ps], :, j % ps])


def test_paged_attention_equals_attention_on_the_gathered_cache():
    q, kp, vp, table, ps, P, intra = _paged_case(1)
    n = P + q.shape[0]
    # an independent gather: physical row of every logical position by loops
    kc = np.stack([np.stack([kp[table[j // ps], g, j % ps] for j in range(n)])
                   for g in range(kp.shape[1])])
    vc = np.stack([np.stack([vp[table[j // ps], g, j % ps] for j in range(n)])
                   for g in range(vp.shape[1])])
    a = oracle.block_attn_paged(q, kp, vp, table, ps, P, intra)
    b = oracle.block_attn(q, kc, vc, P, intra)
    assert np.abs(a - b).max() <= 1e-14
    # relabelling physical pages leaves the result unchanged
    perm = np.random.default_rng(2).permutation(kp.shape[0])
    inv = np.argsort(perm)
    c = oracle.block_attn_paged(q, kp[perm], vp[perm], inv[table], ps, P, intra)
    assert np.abs(a - c).max() <= 1e-14


def test_key_lo_leaves_out_the_prefix_below_it():
    q, kp, vp, table, ps, P, intra = _paged_case(3)
    for key_lo in (0, 1, 16, P):
        got = oracle.block_attn_paged(q, kp, vp, table, ps, P, intra, key_lo=key_lo)
        n = P + q.shape[0]
        kc = oracle.paged_rows(kp, table, ps, n)
        vc = oracle.paged_rows(vp, table, ps, n)
        allowed = np.zeros((q.shape[0], n), dtype=bool)
        allowed[:, key_lo:P] = True
        allowed[:, P:] = intra
        scale = 1 / np.sqrt(q.shape[2])
        group = q.shape[1] // kp.shape[1]
        for h in range(q.shape[1]):
            ref = oracle.masked_attention(q[:, h], kc[h // group], vc[h // group], allowed, scale)
            assert np.abs(got[:, h] - ref).max() <= 1e-14
