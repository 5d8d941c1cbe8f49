"""Checks that a generated LM-head input keeps every integer decision away
from floating-point ties (test infrastructure only).

A commit decision (conf > tau) or an argmax can only be compared bit-exactly
between a float64 oracle and a float32 GPU kernel if no input sits on the
boundary.  The guards used throughout the tests: the top-2 logit gap of every
row exceeds 1e-2, and every confidence is at least 1e-3 away from tau.
"""
from __future__ import annotations

import numpy as np

from .bdiff_oracle import lm_logits, lm_logits_fp8

GAP_MIN = 1e-2
TAU_DIST_MIN = 1e-3


def lmhead_margins(h, W, tau=None, w_scale=None):
    """Return (top-2 logit gap per row, |conf - tau| per row or None).  With
    ``w_scale`` given, W holds E4M3 codes and the logits are the W8A8 ones."""
    logits = lm_logits(h, W) if w_scale is None else lm_logits_fp8(h, W, w_scale)
    top2 = np.sort(logits, axis=1)[:, -2:]
    gap = top2[:, 1] - top2[:, 0]
    if tau is None:
        return gap, None
    conf = 1.0 / np.exp(logits - top2[:, 1:2]).sum(axis=1)
    return gap, np.abs(conf - tau)


def rows_guarded(h, W, tau=None, w_scale=None) -> np.ndarray:
    """Per row: True iff its top-2 gap exceeds GAP_MIN and (with tau) its
    confidence is at least TAU_DIST_MIN away from tau."""
    gap, dist = lmhead_margins(h, W, tau, w_scale)
    ok = gap > GAP_MIN
    if dist is not None:
        ok &= dist >= TAU_DIST_MIN
    return ok


def row_guard(tau=None):
    """The guard the input generators accept (``guard(h, W, w_scale)`` -> bool
    per row): rows_guarded with the given threshold."""
    return lambda h, W, w_scale=None: rows_guarded(h, W, tau, w_scale)


def lmhead_guarded(h, W, tau=None, w_scale=None) -> bool:
    gap, dist = lmhead_margins(h, W, tau, w_scale)
    ok = bool((gap > GAP_MIN).all())
    if dist is not None:
        ok = ok and bool((dist >= TAU_DIST_MIN).all())
    return ok
