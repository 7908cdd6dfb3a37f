"""Tolerance gates for attention parity (GPU result vs the fp64 oracle).

Gates (stated for FP8 MLA context prefill):
  * rel-RMS = ||out_gpu - out_ref||_2 / ||out_ref||_2 over the whole output <= 1e-2
  * max-abs <= 2e-2, measured in units of each V channel's generating scale
    sigma[h, d] = factor_v[h] * (20 if (h, d) is an outlier channel else 1).
    Outputs are bf16 and reach |out| of 10+ on heads with large factors, where
    bf16 spacing alone is 2^-4; in sigma units bf16 rounding stays below 0.016.
    The raw max-abs is reported alongside.
  * |lse_gpu - lse_ref| <= 2^-9 + 1e-3 + 2^-12 * R_h on rows with a visible key, where
    R_h = softmax_scale * dq[h] * dk[h] * max_i |q_i|_2 * max_j |k_j|_2 (codes) bounds
    sum_d |q_id k_jd|, the magnitude scale of head h's logit dot products. The FP8 MFMA
    of gfx950 sums its 64 products to about 2^-16 of sum|terms| (measured worst case
    2^-14.7 for one 64-deep MFMA), so a logit, and hence the LSE, can be off by that
    much of R_h; 2^-12 leaves a 6x margin. The row sum adds the weights as rounded to
    bf16 (each within 2^-9 relative, the same weights the output uses), so on rows whose
    weights all round the same way (near-uniform rows) the LSE moves by up to
    ln(1 + 2^-9) < 2^-9; 1e-3 covers fp32 accumulation. Rows without a visible key must
    be -inf on both sides (and out = 0).
"""

from __future__ import annotations

import numpy as np

REL_RMS_TOL = 1e-2
MAX_ABS_SIGMA_TOL = 2e-2
LSE_TOL = 2.0 ** -9 + 1e-3


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sigma_v(workload) -> np.ndarray:
    f = workload.factors[2].astype(np.float64)[:, None]
    return f * np.where(workload.outlier_mask[2], 20.0, 1.0)


def logit_scale(q8, k8, dq, dk, softmax_scale):
    """R_h (see the module docstring) from the FP8 codes: float64 [H]."""
    from oracle import e4m3_decode

    qn = np.sqrt(np.sum(e4m3_decode(q8) ** 2, axis=2)).max(axis=0) if q8.shape[0] else 0.0
    kn = np.sqrt(np.sum(e4m3_decode(k8) ** 2, axis=2)).max(axis=0) if k8.shape[0] else 0.0
    return softmax_scale * dq.astype(np.float64) * dk.astype(np.float64) * qn * kn


def attention_errors(out_gpu, out_ref, lse_gpu, lse_ref, sigma, r_h=None):
    """out_* [T, H, 128] (float64), lse_* [H, T], sigma [H, 128], r_h [H] logit scale."""
    d = out_gpu - out_ref
    ref_norm = np.sqrt(np.sum(out_ref ** 2))
    rel_rms = float(np.sqrt(np.sum(d ** 2)) / ref_norm) if ref_norm > 0 else float(np.sqrt(np.sum(d ** 2)))
    max_abs_sigma = float(np.max(np.abs(d) / sigma[None])) if d.size else 0.0
    max_abs_raw = float(np.max(np.abs(d))) if d.size else 0.0
    fin_ref = np.isfinite(lse_ref)
    fin_gpu = np.isfinite(lse_gpu)
    lse_pattern_ok = bool(np.array_equal(fin_ref, fin_gpu))
    both = fin_ref & fin_gpu
    dl = np.abs(np.where(both, lse_gpu, 0.0) - np.where(both, lse_ref, 0.0))
    lse_max = float(np.max(dl)) if np.any(both) else 0.0
    if r_h is None:
        r_h = np.zeros(lse_ref.shape[0])
    tol = LSE_TOL + 2.0 ** -12 * np.asarray(r_h, dtype=np.float64)[:, None]
    lse_ratio = float(np.max(dl / tol)) if np.any(both) else 0.0
    return dict(rel_rms=rel_rms, max_abs_sigma=max_abs_sigma, max_abs_raw=max_abs_raw,
                lse_max=lse_max, lse_ratio=lse_ratio, lse_pattern_ok=lse_pattern_ok)


def assert_attention_parity(errs, label=""):
    assert errs["rel_rms"] <= REL_RMS_TOL, (label, errs)
    assert errs["max_abs_sigma"] <= MAX_ABS_SIGMA_TOL, (label, errs)
    assert errs["lse_pattern_ok"], (label, errs)
    assert errs["lse_ratio"] <= 1.0, (label, errs)
