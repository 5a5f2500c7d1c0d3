"""Plain float64 merge of partial attention results over disjoint key sets.

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code may
import or call anything here.

If the keys of a query row are split into disjoint parts and part s gives
the normalised partial output O_s and log-sum-exp LSE_s (natural log, over
the scaled scores of its keys), the attention over all keys is

    LSE = M + ln sum_s exp(LSE_s - M),     M = max_s LSE_s,
    O   = sum_s exp(LSE_s - LSE) O_s.

This is the online-softmax recurrence ("3.6 Attention I -- the memory
problem and FlashAttention principles", 3.6.4) applied to whole parts
instead of key tiles: exp(LSE_s) is part s's sum l_s of exp(scaled score),
O_s l_s its unnormalised output, and the recurrence's result does not depend
on how the keys are grouped or in which order the groups come.  LSE is the
row statistic of 3.6.7.  A part with LSE_s = -inf (no key) contributes
nothing.  The max shift M keeps exp finite for any LSE values (3.6.10: never
exponentiate without subtracting the max).
"""
from __future__ import annotations

import numpy as np

__all__ = ["merge_lse_fp64"]


def merge_lse_fp64(o_parts, lse_parts):
    """Merge partial results.

    o_parts   : array [S, ..., d] of normalised partial outputs.
    lse_parts : array [S, ...] of their log-sum-exps (natural log).
    Returns (O [..., d], LSE [...]) in float64.  Rows whose parts all have
    LSE = -inf get O = 0 and LSE = -inf.
    """
    o = np.asarray(o_parts, dtype=np.float64)
    lse = np.asarray(lse_parts, dtype=np.float64)
    if o.shape[:-1] != lse.shape:
        raise ValueError("o_parts must be [S, ..., d] and lse_parts [S, ...]")
    m = lse.max(axis=0)
    shift = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse - shift)                       # exp(-inf) = 0 for empty parts
    total = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse_out = shift + np.log(total)
    safe = np.where(total > 0, total, 1.0)
    o_out = (w[..., None] * o).sum(axis=0) / safe[..., None]
    return o_out, lse_out
