"""Chunked-context drivers: attend segment by segment, then merge.  (Oracle only.)

The vLLM PR "[ROCm][MLA] Add guarded gfx942 FP8 context prefill" (#51551)
quantizes Q once per context pass and reuses its per-head scale across context
segments ("What this PR does"), and uses the path once the cached context is
long (the commit that fixes the token threshold). The pages do not give the
segmentation; the reading used here, for one sequence with Lq queries that
are the last Lq of Lk keys (off = Lk - Lq):

  * queries are split into chunks of ``seg`` rows;
  * keys [0, off) are cached context, split into segments of ``seg`` keys; every
    query sees all of them (non-causal calls);
  * for query chunk [r0, r1): the own keys [off, off + r0) are split into segments of
    ``seg`` keys seen in full (non-causal), [off + r0, off + r1) is the diagonal
    (causal, Lq = Lk = r1 - r0), and later keys are not visible;
  * the partials of a chunk are merged with the log-sum-exp identity.

With causal = False every query sees every key and the plan is all non-causal
segments. The result equals the unsegmented call (an invariant the tests pin).
"""

from __future__ import annotations

import numpy as np

from .attention import attention_varlen
from .merge import merge_lse


def segment_plan(lq: int, lk: int, seg: int, causal: bool = True):
    """List of (r0, r1, [(k0, k1, causal), ...]) for one sequence."""
    if seg <= 0:
        raise ValueError("segment length must be positive")
    plan = []
    if not causal:
        for r0 in range(0, lq, seg):
            r1 = min(lq, r0 + seg)
            plan.append((r0, r1, [(k0, min(lk, k0 + seg), False) for k0 in range(0, lk, seg)]))
        return plan
    off = lk - lq
    if off < 0:
        raise ValueError("the chunked plan needs Lk >= Lq")
    for r0 in range(0, lq, seg):
        r1 = min(lq, r0 + seg)
        parts = [(k0, min(off, k0 + seg), False) for k0 in range(0, off, seg)]
        parts += [(off + c0, off + min(r0, c0 + seg), False) for c0 in range(0, r0, seg)]
        parts.append((off + r0, off + r1, True))
        plan.append((r0, r1, parts))
    return plan


def chunked_context(q8, k8, v8, dq, dk, dv, softmax_scale: float, seg: int, causal: bool = True):
    """One sequence: q8 [Lq,H,192], k8 [Lk,H,192], v8 [Lk,H,128]. Returns (out, lse) like
    attention_varlen, computed segment by segment and merged."""
    lq, lk = q8.shape[0], k8.shape[0]
    n_heads = q8.shape[1]
    out = np.zeros((lq, n_heads, v8.shape[2]), dtype=np.float64)
    lse = np.full((n_heads, lq), -np.inf, dtype=np.float64)
    for r0, r1, parts in segment_plan(lq, lk, seg, causal):
        outs, lses = [], []
        for k0, k1, c in parts:
            o, l_ = attention_varlen(
                q8[r0:r1], k8[k0:k1], v8[k0:k1],
                np.array([0, r1 - r0], dtype=np.int32), np.array([0, k1 - k0], dtype=np.int32),
                dq, dk, dv, softmax_scale, c)
            outs.append(o)
            lses.append(l_)
        o, l_ = merge_lse(outs, lses)
        out[r0:r1] = o
        lse[:, r0:r1] = l_
    return out, lse
