"""GPU-vs-oracle parity of block attention over a paged KV cache with a
key-range start (bd_block_attn_paged), run on an MI355X.  bf16 outputs
within 2e-2 absolute; with key_lo = 0 the paged call must give exactly the
bits of bd_block_attn on the same (contiguous) cache.  [Fast-dVLM overview
§2.3.2 paged KV; LOWN 'method step details', TEXT-ONLY forward]
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_vlm_amd import bdiff as bd
from block_diffusion_vlm_amd import runner, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert bd.bd_device_check(0) == bd.BD_OK, "device 0 is not gfx950"


def paginate(cache, n, page_size, extra, rng):
    """[Hkv][cap][dh] -> pool [n_pages][Hkv][page_size][dh] holding logical rows
    0..n-1 at a random permutation of pages (plus `extra` unused pages)."""
    hkv, _, dh = cache.shape
    n_log = -(-n // page_size)
    n_pages = n_log + extra
    table = rng.permutation(n_pages)[:n_log].astype(np.int32)
    pool = rng.integers(0, 1 << 16, (n_pages, hkv, page_size, dh)).astype(np.uint16) & 0x3FFF
    for j in range(n):
        pool[table[j // page_size], :, j % page_size] = cache[:, j]
    return pool, table, n_pages


CASES = [
    # Bq, n_vis, n_prompt, Hq, Hkv, page_size, key_lo
    (16, 1024, 256, 16, 2, 16, 0),
    (16, 1024, 256, 16, 2, 16, 1024),     # TEXT-ONLY: visual keys left out
    (16, 1024, 256, 16, 2, 64, 0),
    (16, 1024, 256, 16, 2, 128, 700),
    (16, 1024, 256, 16, 2, 1, 0),
    (5, 30, 7, 4, 2, 5, 0),
    (5, 30, 7, 4, 2, 3, 37),              # key_lo = P: the block's own keys only
    (33, 60, 40, 8, 1, 7, 13),
    (64, 100, 28, 2, 2, 32, 64),
    # long prefixes: two key tiles per split (145 and 129 tiles visited)
    (16, 8192, 1024, 16, 2, 16, 0),
    (16, 8192, 1024, 16, 2, 64, 1000),
]


@pytest.mark.parametrize("Bq,n_vis,n_prompt,Hq,Hkv,ps,key_lo", CASES)
def test_paged_block_attn_matches_oracle(Bq, n_vis, n_prompt, Hq, Hkv, ps, key_lo):
    print(f"paged Bq={Bq} P={n_vis + n_prompt} ps={ps} key_lo={key_lo}", flush=True)
    r = synth.qwen_decode(seed=Bq + ps + key_lo, B=Bq, n_vis=n_vis, n_prompt=n_prompt, Hq=Hq,
                          Hkv=Hkv, d=128, V=64)
    P = r["P"]
    n = P + Bq
    rng = np.random.default_rng(ps + key_lo)
    kpool, table, n_pages = paginate(r["k_cache"], n, ps, 3, rng)
    vpool, _, _ = paginate(r["v_cache"], n, ps, 3, np.random.default_rng(ps + key_lo))
    intra = oracle.intra_block_mask("bidir", Bq) if Bq != 33 else (
        np.random.default_rng(1).random((Bq, Bq)) < 0.5) | np.eye(Bq, dtype=bool)
    rows = np.array([int(sum(int(b) << j for j, b in enumerate(row))) for row in intra],
                    dtype=np.uint64)
    q, kp, vp = runner.to_dev(r["q"]), runner.to_dev(kpool), runner.to_dev(vpool)
    tab, mask = runner.to_dev(table), runner.to_dev(rows)
    out = torch.zeros((Bq, Hq, 128), dtype=torch.bfloat16, device="cuda")
    ws_bytes = bd.bd_block_attn_ws_bytes(P - key_lo, Bq, Hq, Hkv, 128)
    ws = runner.workspace(ws_bytes)
    bd.bd_block_attn_paged(q, kp, vp, tab, ps, n_pages, P, key_lo, mask, Bq, Hq, Hkv, 128, 0.0,
                           out, ws, ws_bytes)
    torch.cuda.synchronize()
    ref = oracle.block_attn_paged(r["q"], kpool, vpool, table, ps, P, intra, key_lo=key_lo)
    assert np.abs(oracle.widen(runner.to_host(out)) - ref).max() <= 2e-2
    if key_lo == 0:
        # same bits as the contiguous call on the same cache
        cont = torch.zeros_like(out)
        wsb = bd.bd_block_attn_ws_bytes(P, Bq, Hq, Hkv, 128)
        w2 = runner.workspace(wsb)
        bd.bd_block_attn(bd.BD_BF16, q, runner.to_dev(r["k_cache"]), runner.to_dev(r["v_cache"]),
                         P, r["cap"], mask, Bq, Hq, Hkv, 128, 0.0, cont, w2, wsb)
        torch.cuda.synchronize()
        assert torch.equal(out, cont)
