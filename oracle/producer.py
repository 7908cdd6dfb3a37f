"""Un-absorbed MLA K/V producer followed by the static quantizer.  (Oracle only.)

Follows vLLM #60110, Purpose: decode folds W_UK into the query projection, while prefill
keeps the un-absorbed form, where keys and values are expanded from the latent
cache per head. Dimensions from the same page: latent rank 512 (the absorbed
query ql_nope[.., 12, 512]), a 192-wide query head of which 64 dims are the
rope part (W_fold rows 512 + 64), 12 heads per rank. Value head dim 128 and the
quantizer follow "[ROCm][MLA] Add guarded gfx942 FP8 context prefill" (#51551).

For token t and head h, with the latent row c_t (512) and the rope key p_t (64):
  k_nope[t, h] = RN_bf16( W_UK[h] . c_t )        (128 values)
  v[t, h]      = RN_bf16( W_UV[h] . c_t )        (128 values)
  K[t, h]      = [ k_nope[t, h] | p_t ]           (192 values; p_t shared by every head)
  k8 = quant_static(K, dk),  v8 = quant_static(V, dv)

Readings (the pages give the shapes, not the layout): the expansion weight is
one bf16 matrix W [H * 256, 512], rows h*256 .. h*256+127 = W_UK[h] and
h*256+128 .. h*256+255 = W_UV[h]; the products are summed exactly (float64,
whose rounding of 512 products of two bf16 values is far below one bf16 ulp)
and rounded once to bf16, nearest even, as the model's bf16 projection output
would be before the quantizer reads it.
"""

from __future__ import annotations

import numpy as np

from .quant import _bf16_to_f64, quant_static

LATENT = 512
ROPE = 64
NOPE = 128
DV = 128


def rn_bf16_bits(y: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest even, directly (no float32 step).

    Finite inputs only; magnitudes below the bf16 normal range round on the fixed
    2^-133 subnormal grid, magnitudes past the largest finite bf16 give infinity.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("finite inputs only")
    a = np.abs(y)
    _, e = np.frexp(a)  # a = m * 2^e, m in [0.5, 1)
    e = np.maximum(e, -125)  # bf16 normal exponents: a >= 2^-126 <=> e >= -125
    ulp = np.ldexp(1.0, e - 8)  # 8 significant bits
    r = np.round(a / ulp) * ulp  # a / ulp < 2^8 exactly representable; np.round is half-even
    r = np.where(r > 3.3895313892515355e38, np.inf, r)  # past bf16 max -> inf
    f32 = np.copysign(r, y).astype(np.float32)  # exact: r has at most 8 significant bits
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def kv_project_bf16(c_kv_bits, w_bits, n_heads: int):
    """bf16 k_nope [T, H, 128] and v [T, H, 128] (bit patterns) from the latent rows."""
    c = _bf16_to_f64(c_kv_bits)  # [T, 512]
    w = _bf16_to_f64(w_bits).reshape(n_heads, NOPE + DV, LATENT)
    y = np.einsum("tk,hfk->thf", c, w)  # exact products, float64 sums
    bits = rn_bf16_bits(y)
    return bits[:, :, :NOPE], bits[:, :, NOPE:]


def kv_produce(c_kv_bits, k_pe_bits, w_bits, dk, dv):
    """Codes k8 [T, H, 192], v8 [T, H, 128] and the bf16 K [T, H, 192], V [T, H, 128]."""
    dk = np.asarray(dk, dtype=np.float32)
    n_heads = dk.shape[0]
    k_nope, v = kv_project_bf16(c_kv_bits, w_bits, n_heads)
    t = k_nope.shape[0]
    pe = np.broadcast_to(np.asarray(k_pe_bits, dtype=np.uint16)[:, None, :], (t, n_heads, ROPE))
    k = np.concatenate([k_nope, pe], axis=2)
    return quant_static(k, dk), quant_static(v, dv), k, v
