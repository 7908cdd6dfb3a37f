"""Tolerance gates for attention parity (GPU result vs the fp64 oracle).

Gates (stated for FP8 MLA context prefill: max-abs 2e-2, rel-RMS 1e-2):
  * rel-RMS = ||out_gpu - out_ref||_2 / ||out_ref||_2 over the compared output <= 1e-2.
  * max-abs, in units of each V channel's generating scale
    sigma[h, d] = factor_v[h] * (20 if (h, d) is an outlier channel else 1):
    |out_gpu - out_ref| / sigma <= 2e-2, the stated bound made scale-free. Outputs are
    bf16 and reach |out| of 10+ on heads with large factors and on x20 outlier channels,
    where the bf16 spacing alone exceeds 2e-2; and the weights P are rounded to bf16
    (2^-9 relative each), so on peaked rows the error is about 2^-9 * |v_j - out| with v
    of the channel's scale, whatever |out| is.
  * max-abs, in absolute units: |out_gpu - out_ref| <= max(2e-2, ulp_bf16(|out_ref|))
    element by element (one ulp of the reference value allows the output's own rounding
    plus as much again). Always reported; asserted (absolute=True) on workloads whose V
    channels are of unit scale up to the per-head factors, where this and the sigma gate
    coincide; on x20 outlier channels the P rounding error above exceeds it.
  * LSE, row by row: |lse_gpu - lse_ref| <= 2^-9 + 1e-3 + 2^-12 * R_i, where
    R_i = sum_j p_ij * softmax_scale * sum_d |q_id k_jd| (dequantized values; p the
    oracle's softmax weights) is the softmax-weighted magnitude of row i's logit dot
    products. The FP8 MFMA of gfx950 sums its 64 products to about 2^-16 of
    sum |terms| (measured worst case 2^-14.7 for one 64-deep MFMA), so logit j is off by
    at most ~2^-14.7 of its own magnitude term and, to first order, the LSE by the
    p-weighted mean of those: 2^-12 leaves a 6x margin. The row sum adds the weights as
    rounded to bf16 (each within 2^-9 relative, the weights the output uses), so on rows
    whose weights all round the same way (near-uniform rows) the LSE moves by up to
    ln(1 + 2^-9) < 2^-9; 1e-3 covers fp32 accumulation. Rows without a visible key must
    be -inf on both sides (and out = 0).

``record`` appends each comparison's error figures as one JSON line to the file named
by the environment variable MLA_PARITY_LOG (when it is set).
"""

from __future__ import annotations

import json
import os

import numpy as np

REL_RMS_TOL = 1e-2
MAX_ABS_TOL = 2e-2
MAX_ABS_SIGMA_TOL = 2e-2
LSE_TOL = 2.0 ** -9 + 1e-3
LSE_SCALE_TOL = 2.0 ** -12

_ROW_BLOCK = 256


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^(e - 7) for |x| in [2^e, 2^(e+1)); normal range)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def sigma_v(workload) -> np.ndarray:
    f = workload.factors[2].astype(np.float64)[:, None]
    return f * np.where(workload.outlier_mask[2], 20.0, 1.0)


def _row_lse_scale(q_of, k_of, n_heads, cu_q, cu_k, rows, scale, causal, lse_ref):
    """R_i of the module docstring for the packed query tokens `rows` (float64 [H, n])."""
    rows = np.asarray(rows, dtype=np.int64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    r = np.zeros((n_heads, rows.shape[0]))
    seq = np.searchsorted(cu_q, rows, side="right") - 1
    for b in np.unique(seq):
        sel = np.nonzero(seq == b)[0]
        lq = int(cu_q[b + 1] - cu_q[b])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        lk = k1 - k0
        if lk == 0:
            continue
        local = rows[sel] - cu_q[b]
        for h in range(n_heads):
            kd = k_of(slice(k0, k1), h)
            ka = np.abs(kd)
            for c0 in range(0, sel.shape[0], _ROW_BLOCK):
                idx = sel[c0:c0 + _ROW_BLOCK]
                qd = q_of(rows[idx], h)
                vis = np.ones((idx.shape[0], lk), dtype=bool)
                if causal:
                    lim = local[c0:c0 + _ROW_BLOCK] + (lk - lq)
                    vis = np.arange(lk)[None, :] <= lim[:, None]
                lse = lse_ref[h, idx]
                fin = np.isfinite(lse)
                s = scale * (qd @ kd.T)
                p = np.where(vis & fin[:, None], np.exp(s - np.where(fin, lse, 0.0)[:, None]), 0.0)
                a = scale * (np.abs(qd) @ ka.T)
                r[h, idx] = np.sum(p * a, axis=1)
    return r


def lse_scale_fp8(q8, k8, dq, dk, cu_q, cu_k, rows, softmax_scale, causal, lse_ref):
    """R_i for FP8 codes with per-head descales (the dequantized values)."""
    from oracle import e4m3_decode

    dq = np.asarray(dq, dtype=np.float64)
    dk = np.asarray(dk, dtype=np.float64)
    return _row_lse_scale(lambda r_, h: e4m3_decode(q8[r_, h]) * dq[h],
                          lambda r_, h: e4m3_decode(k8[r_, h]) * dk[h], q8.shape[1], cu_q, cu_k,
                          rows, softmax_scale, causal, lse_ref)


def lse_scale_bf16(q, k, cu_q, cu_k, rows, softmax_scale, causal, lse_ref):
    """R_i for bf16 inputs (bit patterns)."""
    return _row_lse_scale(lambda r_, h: bf16_bits_to_f64(q[r_, h]),
                          lambda r_, h: bf16_bits_to_f64(k[r_, h]), q.shape[1], cu_q, cu_k, rows,
                          softmax_scale, causal, lse_ref)


def attention_errors(out_gpu, out_ref, lse_gpu, lse_ref, sigma, r_rows=None):
    """out_* [n, H, 128] (float64), lse_* [H, n], sigma [H, 128], r_rows [H, n] (R_i)."""
    d = out_gpu - out_ref
    ref_norm = np.sqrt(np.sum(out_ref ** 2))
    rel_rms = float(np.sqrt(np.sum(d ** 2)) / ref_norm) if ref_norm > 0 else float(np.sqrt(np.sum(d ** 2)))
    ad = np.abs(d)
    max_abs_sigma = float(np.max(ad / sigma[None])) if d.size else 0.0
    max_abs_raw = float(np.max(ad)) if d.size else 0.0
    abs_gate = np.maximum(MAX_ABS_TOL, ulp_bf16(out_ref))
    max_abs_ratio = float(np.max(ad / abs_gate)) if d.size else 0.0
    fin_ref = np.isfinite(lse_ref)
    fin_gpu = np.isfinite(lse_gpu)
    lse_pattern_ok = bool(np.array_equal(fin_ref, fin_gpu))
    both = fin_ref & fin_gpu
    dl = np.abs(np.where(both, lse_gpu, 0.0) - np.where(both, lse_ref, 0.0))
    lse_max = float(np.max(dl)) if np.any(both) else 0.0
    if r_rows is None:
        r_rows = np.zeros(lse_ref.shape)
    tol = LSE_TOL + LSE_SCALE_TOL * np.asarray(r_rows, dtype=np.float64)
    lse_ratio = float(np.max(dl / tol)) if np.any(both) else 0.0
    return dict(rel_rms=rel_rms, max_abs_raw=max_abs_raw, max_abs_ratio=max_abs_ratio,
                max_abs_sigma=max_abs_sigma, lse_max=lse_max, lse_ratio=lse_ratio,
                lse_pattern_ok=lse_pattern_ok, rows=int(out_ref.shape[0]))


def assert_attention_parity(errs, label="", max_abs=True, absolute=False):
    assert errs["rel_rms"] <= REL_RMS_TOL, (label, errs)
    if max_abs:
        assert errs["max_abs_sigma"] <= MAX_ABS_SIGMA_TOL, (label, errs)
    if absolute:
        assert errs["max_abs_ratio"] <= 1.0, (label, errs)
    assert errs["lse_pattern_ok"], (label, errs)
    assert errs["lse_ratio"] <= 1.0, (label, errs)


def record(label: str, errs: dict, **extra):
    """Append one JSON line with the comparison's figures to $MLA_PARITY_LOG, if set."""
    path = os.environ.get("MLA_PARITY_LOG")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as f:
        f.write(json.dumps(dict(label=label, **errs, **extra)) + "\n")


def stratified_rows(n_rows: int, seed: int, block: int = 32, extra=()):
    """One row per `block`-row block of [0, n_rows) (every 32-row wave block of a query
    tile), the row within each block drawn so that all in-block positions (lanes) occur
    equally often, plus the given extra rows."""
    rng = np.random.default_rng(seed)
    n_blk = (n_rows + block - 1) // block
    lanes = np.concatenate([rng.permutation(block) for _ in range((n_blk + block - 1) // block)])
    rows = np.arange(n_blk) * block + lanes[:n_blk]
    rows = rows[rows < n_rows]
    return np.unique(np.concatenate([rows, np.asarray(extra, dtype=np.int64)]).astype(np.int64))
