"""Softmax attention on dequantized FP8 inputs, packed varlen, out + LSE.  (Oracle only.)

Follows the vLLM PR "[ROCm][MLA] Add guarded gfx942 FP8 context prefill"
(#51551): Background (a packed variable-length kernel for the D192 Q/K, D128 V
shape) and "What this PR does" (12 heads, D192 Q/K, D128 V; FP8 inputs with
per-head scales). The close comment distinguishes causal and non-causal
shapes. The plain definition, in float64, for each sequence b and head h:

  Qd = decode(q8) * dq[h],  Kd = decode(k8) * dk[h],  Vd = decode(v8) * dv[h]
  s_ij = softmax_scale * <Qd_i, Kd_j>
  visible(i, j): non-causal -> every j < Lk
                 causal     -> j <= i + (Lk - Lq)     (bottom-right alignment)
  m_i = max_{visible j} s_ij,  l_i = sum_{visible j} exp(s_ij - m_i)
  out_i = sum_{visible j} exp(s_ij - m_i) * Vd_j / l_i,   lse_i = m_i + ln l_i
  a row with no visible key: out_i = 0, lse_i = -inf

Readings (the pages are silent): the softmax scale is a parameter; LSE is the
natural log; causal alignment is bottom-right, which is the plain lower
triangle when Lq = Lk; a zero-length sequence contributes nothing.

The same definition on bf16 inputs (no quantization, Qd/Kd/Vd are the bf16
values) is the BF16 attention that the close comment of the PR names as the
comparator covering D192/V128 (attention_varlen_bf16, attention_rows_bf16).

Query rows are processed in blocks to bound memory; that blocking only splits
independent rows and does not change any row's arithmetic.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_decode

_ROW_BLOCK = 512


def _dequant(codes: np.ndarray, descale: np.ndarray) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(descale, dtype=np.float32).astype(np.float64)


def _rows_one_head(qd, kd, vd, rows_local, lq, lk, scale, causal):
    """qd [n, Dqk] (the selected rows), kd [lk, Dqk], vd [lk, Dv]; rows_local: row indices i."""
    n = qd.shape[0]
    out = np.zeros((n, vd.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if n == 0 or lk == 0:
        return out, lse
    s = scale * (qd @ kd.T)  # [n, lk]
    if causal:
        limit = rows_local + (lk - lq)  # last visible key index per row
        vis = np.arange(lk)[None, :] <= limit[:, None]
    else:
        vis = np.ones((n, lk), dtype=bool)
    s = np.where(vis, s, -np.inf)
    has = vis.any(axis=1)
    m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    p = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    o = p @ vd
    out[has] = o[has] / l[has, None]
    lse[has] = m[has] + np.log(l[has])
    return out, lse


def _bf16_values(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention_varlen(q8, k8, v8, cu_seqlens_q, cu_seqlens_k, dq, dk, dv,
                     softmax_scale: float, causal: bool):
    """q8 [Tq,H,192], k8 [Tk,H,192], v8 [Tk,H,128] uint8 codes; descales float32 [H].

    Returns out float64 [Tq, H, 128] and lse float64 [H, Tq].
    """
    return _varlen(lambda r, h: _dequant(q8[r, h], dq[h]), lambda r, h: _dequant(k8[r, h], dk[h]),
                   lambda r, h: _dequant(v8[r, h], dv[h]), q8.shape[0], q8.shape[1], v8.shape[2],
                   cu_seqlens_q, cu_seqlens_k, softmax_scale, causal)


def attention_varlen_bf16(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale: float, causal: bool):
    """q [Tq,H,192], k [Tk,H,192], v [Tk,H,128] bf16 bit patterns (uint16), no scales.

    Returns out float64 [Tq, H, 128] and lse float64 [H, Tq].
    """
    return _varlen(lambda r, h: _bf16_values(q[r, h]), lambda r, h: _bf16_values(k[r, h]),
                   lambda r, h: _bf16_values(v[r, h]), q.shape[0], q.shape[1], v.shape[2],
                   cu_seqlens_q, cu_seqlens_k, softmax_scale, causal)


def _varlen(q_of, k_of, v_of, tq, n_heads, dv_dim, cu_seqlens_q, cu_seqlens_k, softmax_scale,
            causal):
    """q_of(rows, h), k_of(rows, h), v_of(rows, h): float64 values of the given token rows."""
    out = np.zeros((tq, n_heads, dv_dim), dtype=np.float64)
    lse = np.full((n_heads, tq), -np.inf, dtype=np.float64)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    for b in range(cu_q.shape[0] - 1):
        q0, q1 = cu_q[b], cu_q[b + 1]
        k0, k1 = cu_k[b], cu_k[b + 1]
        lq, lk = int(q1 - q0), int(k1 - k0)
        if lq == 0:
            continue
        for h in range(n_heads):
            kd = k_of(slice(k0, k1), h)
            vd = v_of(slice(k0, k1), h)
            for r0 in range(0, lq, _ROW_BLOCK):
                r1 = min(lq, r0 + _ROW_BLOCK)
                qd = q_of(slice(q0 + r0, q0 + r1), h)
                o, l_ = _rows_one_head(qd, kd, vd, np.arange(r0, r1), lq, lk, softmax_scale, causal)
                out[q0 + r0:q0 + r1, h] = o
                lse[h, q0 + r0:q0 + r1] = l_
    return out, lse


def attention_rows(q8, k8, v8, cu_seqlens_q, cu_seqlens_k, dq, dk, dv,
                   softmax_scale: float, causal: bool, rows):
    """Same definition, only for the packed query tokens listed in ``rows``.

    Rows are independent, so each selected row equals that row of attention_varlen.
    Returns out float64 [len(rows), H, 128] and lse float64 [H, len(rows)].
    """
    return _rows(lambda r, h: _dequant(q8[r, h], dq[h]), lambda r, h: _dequant(k8[r, h], dk[h]),
                 lambda r, h: _dequant(v8[r, h], dv[h]), q8.shape[1], v8.shape[2], cu_seqlens_q,
                 cu_seqlens_k, softmax_scale, causal, rows)


def attention_rows_bf16(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale: float, causal: bool,
                        rows):
    """attention_varlen_bf16 for the packed query tokens listed in ``rows`` only."""
    return _rows(lambda r, h: _bf16_values(q[r, h]), lambda r, h: _bf16_values(k[r, h]),
                 lambda r, h: _bf16_values(v[r, h]), q.shape[1], v.shape[2], cu_seqlens_q,
                 cu_seqlens_k, softmax_scale, causal, rows)


def _rows(q_of, k_of, v_of, n_heads, dv_dim, cu_seqlens_q, cu_seqlens_k, softmax_scale, causal,
          rows):
    rows = np.asarray(rows, dtype=np.int64)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    out = np.zeros((rows.shape[0], n_heads, dv_dim), dtype=np.float64)
    lse = np.full((n_heads, rows.shape[0]), -np.inf, dtype=np.float64)
    seq = np.searchsorted(cu_q, rows, side="right") - 1
    for b in np.unique(seq):
        sel = np.nonzero(seq == b)[0]
        q0, q1 = cu_q[b], cu_q[b + 1]
        k0, k1 = cu_k[b], cu_k[b + 1]
        lq, lk = int(q1 - q0), int(k1 - k0)
        local = rows[sel] - q0
        for h in range(n_heads):
            kd = k_of(slice(k0, k1), h)
            vd = v_of(slice(k0, k1), h)
            for c0 in range(0, sel.shape[0], _ROW_BLOCK):
                idx = sel[c0:c0 + _ROW_BLOCK]
                loc = local[c0:c0 + _ROW_BLOCK]
                qd = q_of(rows[idx], h)
                o, l_ = _rows_one_head(qd, kd, vd, loc, lq, lk, softmax_scale, causal)
                out[idx, h] = o
                lse[h, idx] = l_
    return out, lse
