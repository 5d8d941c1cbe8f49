"""Pins of the oracle's dual-stream training backward and row log-sum-exp.

The backward is pinned to torch autograd (float64) through a masked softmax
attention written with torch operations, and to central finite differences
of the oracle's own forward; the log-sum-exp to scipy's logsumexp over the
visible scores.  [Fast-dVLM overview §2.2.1; Thai article §4.1]
"""
import numpy as np
import scipy.special
import torch

import oracle

CASES = [(3, 4, 2, None), (0, 6, 3, None), (2, 7, 2, [0, 3]), (4, 9, 4, [0, 2, 5, 8])]


def _inputs(n_vis, n_txt, H=2, dh=8, seed=0):
    rng = np.random.default_rng(seed)
    n = n_vis + 2 * n_txt
    return [rng.standard_normal((n, H, dh)) for _ in range(4)]


def test_lse_matches_library_logsumexp():
    for n_vis, n_txt, b, seg in CASES:
        q, k, _, _ = _inputs(n_vis, n_txt)
        lse = oracle.dualstream_lse(q, k, n_vis, n_txt, b, seg_starts=seg)
        allowed = oracle.dualstream_mask(n_vis, n_txt, b, seg)
        scale = 1 / np.sqrt(q.shape[2])
        for h in range(q.shape[1]):
            s = scale * q[:, h] @ k[:, h].T
            ref = scipy.special.logsumexp(np.where(allowed, s, -np.inf), axis=1)
            assert np.abs(lse[:, h] - ref).max() <= 1e-12


def test_backward_matches_torch_autograd():
    for n_vis, n_txt, b, seg in CASES:
        q, k, v, g = _inputs(n_vis, n_txt, seed=n_vis + n_txt)
        allowed = torch.from_numpy(oracle.dualstream_mask(n_vis, n_txt, b, seg))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        scale = 1 / np.sqrt(q.shape[2])
        s = torch.einsum("ihd,jhd->hij", tq, tk) * scale
        s = s.masked_fill(~allowed, float("-inf"))
        o = torch.einsum("hij,jhd->ihd", torch.softmax(s, dim=-1), tv)
        o.backward(torch.from_numpy(g))
        dq, dk, dv = oracle.dualstream_attn_bwd(q, k, v, g, n_vis, n_txt, b, seg_starts=seg)
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.abs(got - ref.numpy()).max() <= 1e-12


def test_backward_matches_finite_differences():
    n_vis, n_txt, b, seg = 2, 5, 2, [0, 3]
    q, k, v, g = _inputs(n_vis, n_txt, H=1, dh=4, seed=3)
    dq, dk, dv = oracle.dualstream_attn_bwd(q, k, v, g, n_vis, n_txt, b, seg_starts=seg)

    def loss(q_, k_, v_):
        return float((oracle.dualstream_attn(q_, k_, v_, n_vis, n_txt, b, seg_starts=seg)
                      * g).sum())

    eps = 1e-6
    rng = np.random.default_rng(4)
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in q.shape)
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            down = loss(*args)
            assert abs((up - down) / (2 * eps) - grad[idx]) <= 1e-7


def test_backward_identities():
    # Every row of P sums to 1, so the dV rows sum to the d_out rows; every
    # row of dS sums to 0, so the dK rows sum to 0 (per head); a clean row 0
    # sees only key 0, so its scores (and dQ_0) get no gradient.
    for n_vis, n_txt, b, seg in CASES:
        q, k, v, g = _inputs(n_vis, n_txt, seed=11)
        dq, dk, dv = oracle.dualstream_attn_bwd(q, k, v, g, n_vis, n_txt, b, seg_starts=seg)
        assert np.abs(dv.sum(axis=0) - g.sum(axis=0)).max() <= 1e-12
        assert np.abs(dk.sum(axis=0)).max() <= 1e-12
        assert np.abs(dq[0]).max() == 0.0


# The backward from what the forward kept (dualstream_attn_bwd_given): with
# the exact output and log-sum-exp it is the gradient above; its response to
# a changed output or log-sum-exp follows from the formulas in closed form.

def test_given_exact_forward_equals_the_gradient():
    for n_vis, n_txt, b, seg in CASES:
        q, k, v, g = _inputs(n_vis, n_txt, seed=3 * n_vis + n_txt)
        out = oracle.dualstream_attn(q, k, v, n_vis, n_txt, b, seg_starts=seg)
        lse = oracle.dualstream_lse(q, k, n_vis, n_txt, b, seg_starts=seg)
        ref = oracle.dualstream_attn_bwd(q, k, v, g, n_vis, n_txt, b, seg_starts=seg)
        got = oracle.dualstream_attn_bwd_given(q, k, v, out, lse, g, n_vis, n_txt, b,
                                               seg_starts=seg)
        for a, r in zip(got, ref):
            assert np.abs(a - r).max() <= 1e-12 * max(1.0, np.abs(r).max())


def test_given_output_enters_through_d_only():
    # out + delta moves D_i by e_i = dO_i . delta_i, which moves dQ_i by
    # -scale e_i sum_j P_ij k_j (attention with the keys as values) and dK_j
    # by -scale sum_i P_ij e_i q_i (the dV of output gradient e * q); dV stays
    n_vis, n_txt, b, seg = 2, 7, 2, [0, 3]
    q, k, v, g = _inputs(n_vis, n_txt, seed=11)
    out = oracle.dualstream_attn(q, k, v, n_vis, n_txt, b, seg_starts=seg)
    lse = oracle.dualstream_lse(q, k, n_vis, n_txt, b, seg_starts=seg)
    delta = 1e-3 * np.random.default_rng(12).standard_normal(out.shape)
    base = oracle.dualstream_attn_bwd_given(q, k, v, out, lse, g, n_vis, n_txt, b, seg_starts=seg)
    moved = oracle.dualstream_attn_bwd_given(q, k, v, out + delta, lse, g, n_vis, n_txt, b,
                                             seg_starts=seg)
    e = (g * delta).sum(axis=2)
    scale = 1 / np.sqrt(q.shape[2])
    pk = oracle.dualstream_attn(q, k, k, n_vis, n_txt, b, seg_starts=seg)
    _, _, pq = oracle.dualstream_attn_bwd(q, k, v, e[:, :, None] * q, n_vis, n_txt, b,
                                          seg_starts=seg)
    assert np.abs(moved[0] - base[0] + scale * e[:, :, None] * pk).max() <= 1e-12
    assert np.abs(moved[1] - base[1] + scale * pq).max() <= 1e-12
    assert np.array_equal(moved[2], base[2])


def test_given_lse_shift_scales_its_row():
    # lse_i + c multiplies row i of P by exp(-c): dQ_i scales by exp(-c),
    # every other row of dQ stays
    n_vis, n_txt, b, seg = 3, 4, 2, None
    q, k, v, g = _inputs(n_vis, n_txt, seed=5)
    out = oracle.dualstream_attn(q, k, v, n_vis, n_txt, b)
    lse = oracle.dualstream_lse(q, k, n_vis, n_txt, b)
    base = oracle.dualstream_attn_bwd_given(q, k, v, out, lse, g, n_vis, n_txt, b)
    i, c = 6, 0.37
    lse2 = lse.copy()
    lse2[i] += c
    dq2 = oracle.dualstream_attn_bwd_given(q, k, v, out, lse2, g, n_vis, n_txt, b)[0]
    assert np.abs(dq2[i] - np.exp(-c) * base[0][i]).max() <= 1e-12
    rest = np.arange(q.shape[0]) != i
    assert np.abs(dq2[rest] - base[0][rest]).max() <= 1e-12
