"""Error bounds for the bf16 training backward's gradients, used by the GPU
parity tests.

The backward receives the forward's output O in bf16 and forms
D_i = sum_d dO_id O_id from it (the softmax gradient dS = P * (dP - D)).
Rounding O to bf16 moves each element by at most 2^-9 of itself, so D_i
moves by at most eD_i = 2^-8 sum_d |dO_id| |O_id| (2^-8 also covers a
one-ulp difference in rounding direction when the float32 value sits next
to a rounding boundary).  That error is absolute, not relative to the
gradient: through dQ = scale dS K and dK = scale dS^T Q it adds
    |d dQ_id| <= scale eD_i sum_j P_ij |k_jd|,
    |d dK_jd| <= scale sum_i P_ij eD_i |q_id|,
and nothing to dV = P^T dO.  It matters where the gradient itself is small
next to |dO| |O| |k|, e.g. a row whose visible keys nearly agree.  The
other roundings (of P, of dS and of the stored gradient, 2^-9 each) are
relative and stay within 1e-2 of the largest reference value.
[Fast-dVLM overview §2.2.1: the training attention whose gradient this is]
"""
import numpy as np

import oracle

REL = 1e-2          # the relative part: three 2^-9 roundings with margin


def d_rounding_terms(q, k, v, d_out, n_vis, n_txt, block, seg_starts=None):
    """Largest absolute error (dq_extra, dk_extra) that the bf16 rounding of
    O can add to dQ and dK, over every row, head and column; float64."""
    q, k, v, g = (oracle.widen(x) for x in (q, k, v, d_out))
    n, nh, dh = q.shape
    scale = 1.0 / np.sqrt(dh)
    allowed = oracle.dualstream_mask(n_vis, n_txt, block, seg_starts)
    dq_x = dk_x = 0.0
    for h in range(nh):
        s = np.where(allowed, scale * (q[:, h] @ k[:, h].T), -np.inf)
        p = np.where(allowed, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v[:, h]
        ed = 2.0 ** -8 * (np.abs(g[:, h]) * np.abs(o)).sum(axis=1)
        dq_x = max(dq_x, scale * (ed[:, None] * (p @ np.abs(k[:, h]))).max())
        dk_x = max(dk_x, scale * (p.T @ (ed[:, None] * np.abs(q[:, h]))).max())
    return dq_x, dk_x


def grad_tolerances(r, seg_starts=None, heads=None):
    """{'dq', 'dk', 'dv'} -> the absolute part of each gradient's bound for
    the dual-stream workload r (optionally only the given heads)."""
    sl = (slice(None), slice(None) if heads is None else list(heads), slice(None))
    dq_x, dk_x = d_rounding_terms(r["q"][sl], r["k"][sl], r["v"][sl], r["d_out"][sl],
                                  r["n_vis"], r["n_txt"], r["block"], seg_starts)
    return {"dq": dq_x, "dk": dk_x, "dv": 0.0}


def within(got, ref, extra):
    """max |got - ref| <= REL max |ref| + extra; returns (ok, err, bound)."""
    err = float(np.abs(got - ref).max())
    bound = REL * float(np.abs(ref).max()) + extra
    return err <= bound, err, bound
