"""Log-sum-exp merge of per-segment attention partials.  (Oracle only.)

The vLLM PR "[ROCm][MLA] Add guarded gfx942 FP8 context prefill" (#51551,
"What this PR does") processes long contexts in segments, reusing one
quantized Q, and keeps a per-chunk output buffer; how partials are combined
is not written on the pages. The reading used here is the standard identity
for softmax over a union of disjoint key sets:

  L = log( sum_s exp(L_s) )          out = sum_s exp(L_s - L) * out_s

A segment with L_s = -inf (no visible key) gets weight 0; if every segment has
L_s = -inf the result is out = 0, L = -inf.
"""

from __future__ import annotations

import numpy as np


def merge_lse(outs, lses):
    """outs: sequence of [T, H, Dv]; lses: sequence of [H, T]. Returns (out f64, lse f64)."""
    outs = [np.asarray(o, dtype=np.float64) for o in outs]
    lses = [np.asarray(l_, dtype=np.float64) for l_ in lses]
    if len(outs) == 0 or len(outs) != len(lses):
        raise ValueError("need one lse per output and at least one segment")
    big = np.stack(lses)  # [S, H, T]
    m = big.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(big), np.exp(big - m_safe[None]), 0.0)  # [S, H, T]
    tot = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    out = np.zeros_like(outs[0])
    for s, o in enumerate(outs):
        ws = np.where(finite, w[s] / np.where(finite, tot, 1.0), 0.0)  # [H, T]
        out += ws.T[:, :, None] * o
    return out, lse
