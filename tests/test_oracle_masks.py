"""Pins of the oracle's mask builders against what the pages print and fix.

The Fast-dVLM overview (ocdem.com/news/1032714) §2.2.1 prints the N2N and N2C
matrices for block size 2; everything else here is a closed form or a
hand-written fixture derived from those pages (see the fixture headers).
"""
import numpy as np
import pytest

import oracle
from tests.golden.load import matrices


def test_n2n_n2c_equal_printed_matrices():
    g = matrices("printed_masks_b2.txt")
    assert np.array_equal(oracle.mask_n2n(4, 2), g["N2N"])
    assert np.array_equal(oracle.mask_n2c(4), g["N2C"])


def test_c2c_is_the_textbook_causal_mask():
    for n in (1, 4, 9):
        assert np.array_equal(oracle.mask_c2c(n), np.tril(np.ones((n, n), dtype=bool)))


@pytest.mark.parametrize("n", [1, 5, 16])
def test_n2n_block_one_is_identity(n):
    assert np.array_equal(oracle.mask_n2n(n, 1), np.eye(n, dtype=bool))


def test_n2n_single_block_is_all_ones():
    assert oracle.mask_n2n(6, 6).all()


def test_n2n_ragged_last_block():
    m = oracle.mask_n2n(5, 2)
    assert m[4, 4] and not m[4, 3] and m[2, 3] and not m[1, 2]


def test_dualstream_mask_tiny_workload_fixture():
    g = matrices("dualstream_mask_v4_t4_b2.txt")["DUALSTREAM"]
    assert np.array_equal(oracle.dualstream_mask(4, 4, 2), g)


def test_dualstream_mask_structure_at_larger_size():
    n_vis, n_txt, b = 7, 10, 4
    m = oracle.dualstream_mask(n_vis, n_txt, b)
    ctx = n_vis + n_txt
    assert not m[:ctx, ctx:].any()               # no clean -> noisy
    assert m[ctx:, :n_vis].all()                 # noisy -> every visual token
    assert np.array_equal(m[:ctx, :ctx], np.tril(np.ones((ctx, ctx), dtype=bool)))
    # every query sees itself (no empty rows)
    assert m.diagonal().all()
    # pair count: sum over rows of visible keys, written as a count per stream
    clean = ctx * (ctx + 1) // 2
    noisy = n_txt * n_vis + n_txt * (n_txt + 1) // 2 + sum(
        min(b, n_txt - (r // b) * b) for r in range(n_txt))
    assert m.sum() == clean + noisy


def test_intra_block_masks():
    assert oracle.intra_block_mask("bidir", 5).all()
    assert np.array_equal(oracle.intra_block_mask("causal", 5),
                          np.tril(np.ones((5, 5), dtype=bool)))
    g = matrices("spec_fused_b2.txt")["SPEC_FUSED"]
    assert np.array_equal(oracle.intra_block_mask("spec_fused", 4), g)


def test_spec_fused_is_dualstream_mask_of_one_block():
    # Reading: the fused mask is the training mask with no visual tokens and a
    # single block covering the draft half.
    for b in (1, 3, 8):
        fused = oracle.intra_block_mask("spec_fused", 2 * b)
        assert np.array_equal(fused, oracle.dualstream_mask(0, b, b))


def test_spec_fused_b1_by_hand():
    # verify row sees itself; draft row sees verify row 0 (j <= i - B = 0) and itself
    assert np.array_equal(oracle.intra_block_mask("spec_fused", 2),
                          np.array([[1, 0], [1, 1]], dtype=bool))


# ---------------------------------------------------------------------------
# Auto-truncation (segment-clamped N2N blocks)  [OV §2.2.2; TH §4.3]
# ---------------------------------------------------------------------------

def test_one_segment_is_the_plain_n2n_mask():
    for n, b in ((12, 2), (37, 5), (64, 64), (9, 1)):
        assert np.array_equal(oracle.mask_n2n(n, b, [0]), oracle.mask_n2n(n, b))


def test_segment_clamp_worked_example():
    # 7 text tokens, block 2, a prompt of 3 tokens then a response of 4:
    # blocks {0,1} {2} | {3,4} {5,6} -- token 2 ends its segment, so its
    # block is cut to one token instead of spilling into the response.
    want = np.array([
        [1, 1, 0, 0, 0, 0, 0],
        [1, 1, 0, 0, 0, 0, 0],
        [0, 0, 1, 0, 0, 0, 0],
        [0, 0, 0, 1, 1, 0, 0],
        [0, 0, 0, 1, 1, 0, 0],
        [0, 0, 0, 0, 0, 1, 1],
        [0, 0, 0, 0, 0, 1, 1],
    ], dtype=bool)
    assert np.array_equal(oracle.mask_n2n(7, 2, [0, 3]), want)


def test_segment_clamped_blocks_tile_each_segment():
    rng = np.random.default_rng(5)
    for _ in range(30):
        n = int(rng.integers(1, 80))
        b = int(rng.integers(1, 9))
        k = int(rng.integers(0, min(n, 10)))
        starts = [0] + sorted(rng.choice(np.arange(1, n), k, replace=False).tolist()) if n > 1 else [0]
        m = oracle.mask_n2n(n, b, starts)
        assert np.array_equal(m, m.T) and m.diagonal().all()
        bounds = starts + [n]
        for s in range(len(starts)):
            lo, hi = bounds[s], bounds[s + 1]
            for r in range(lo, hi):
                blk = np.nonzero(m[r])[0]
                b0 = lo + ((r - lo) // b) * b
                # the block is contiguous, starts on the segment's grid and is
                # cut at the segment's end
                assert blk[0] == b0 and np.array_equal(blk, np.arange(b0, min(b0 + b, hi)))


def test_segments_change_only_the_n2n_quadrant():
    n_vis, n_txt, b = 3, 10, 4
    plain = oracle.dualstream_mask(n_vis, n_txt, b)
    seg = oracle.dualstream_mask(n_vis, n_txt, b, [0, 6])
    ctx = n_vis + n_txt
    diff = plain != seg
    assert not diff[:, :ctx].any() and not diff[:ctx].any()
    assert np.array_equal(seg[ctx:, ctx:], oracle.mask_n2n(n_txt, b, [0, 6]))
