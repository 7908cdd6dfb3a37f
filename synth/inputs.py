"""Seeded synthetic inputs with the shapes of FP8 MLA context prefill.

Shapes and structure follow the vLLM PR "[ROCm][MLA] Add guarded gfx942 FP8
context prefill" (section "What this PR does"): 12 heads per rank, Q/K head
dim 192, V head dim 128, BF16 model activations, packed variable-length
sequences, and long contexts processed in segments with Q quantized once.

Recipe (identical bytes reach the oracle and the GPU):
  * workload Ci uses base seed S = 1000 * i;
  * data draw: ``np.random.default_rng(S)``, float32 standard normal, drawn in
    the order Q, K, V, each as one call of shape [tokens, heads, dim];
  * calibration draw: ``default_rng(S + 1)``, same shapes and order;
  * structure draw: ``default_rng(S + 2)``: varlen lengths first (if any), then
    per-(tensor, head) factors f = 2**U(-2, 2) (if the workload has factors),
    then outlier channels (if any): per tensor, max(1, round(0.001 * H * D))
    distinct (head, dim) columns, scaled by 20;
  * values: x = bf16_RNE(z * g) with g = float32(f[h] * (20 or 1)), the product
    taken in float32 and rounded to bf16 once.

Nothing here encodes FP8, derives scales or computes attention.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

N_HEADS = 12
D_QK = 192
D_V = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    NaN inputs keep a quiet-NaN pattern. Used only to turn random draws into input bytes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((b >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One synthetic workload: bf16 inputs as uint16 bit patterns plus structure.

    q: [total_q, H, 192], k: [total_k, H, 192], v: [total_k, H, 128] (uint16 bf16 bits)
    cu_seqlens_q / cu_seqlens_k: int32 [batch + 1]
    factors: float32 [3, H] per-(tensor, head) factors (Q, K, V); ones if none
    outlier_mask: list of 3 bool arrays [H, D] marking the x20 channels
    segment_len: context segment length for chunked processing (0: one segment)
    """

    name: str
    seed: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    causal: bool
    softmax_scale: float
    factors: np.ndarray
    outlier_mask: list
    segment_len: int
    description: str
    _calib: Optional[tuple] = None

    @property
    def batch(self) -> int:
        return int(self.cu_seqlens_q.shape[0] - 1)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_seqlens_k[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens_q))) if self.batch else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens_k))) if self.batch else 0

    def calib(self):
        """Calibration draw (seed + 1), same shapes and structure; cached after first use."""
        if self._calib is None:
            rng = np.random.default_rng(self.seed + 1)
            self._calib = tuple(
                _draw(rng, x.shape, self.factors[t], self.outlier_mask[t])
                for t, x in enumerate((self.q, self.k, self.v))
            )
        return self._calib

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs that attention reads, summed over sequences (one head)."""
        n = 0
        for b in range(self.batch):
            lq = int(self.cu_seqlens_q[b + 1] - self.cu_seqlens_q[b])
            lk = int(self.cu_seqlens_k[b + 1] - self.cu_seqlens_k[b])
            n += _pairs(lq, lk, self.causal)
        return n


def _pairs(lq: int, lk: int, causal: bool) -> int:
    if not causal:
        return lq * lk
    off = lk - lq  # query i sees keys j <= i + off (bottom-right alignment)
    total = 0
    # rows with i + off >= lk - 1 see all keys; rows with i + off < 0 see none
    i_full = max(0, min(lq, lk - 1 - off))  # first row that sees all lk keys
    # rows 0 .. i_full-1 see max(0, i + off + 1) keys
    lo = max(0, -off)  # first row with at least one key
    if i_full > lo:
        a = lo + off + 1
        b = i_full - 1 + off + 1
        total += (a + b) * (i_full - lo) // 2
    total += (lq - i_full) * lk
    return total


def _draw(rng, shape, factors, outlier_mask) -> np.ndarray:
    z = rng.standard_normal(size=shape, dtype=np.float32)
    g = np.where(outlier_mask, np.float32(20.0), np.float32(1.0)).astype(np.float32)
    g = (g * factors[:, None].astype(np.float32)).astype(np.float32)  # [H, D]
    z *= g[None, :, :]
    return f32_to_bf16_bits(z)


def random_varlen(rng, batch: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths uniform on the integers lo..hi inclusive."""
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def _structure(seed: int, lens_spec, use_factors: bool, use_outliers: bool):
    rng = np.random.default_rng(seed + 2)
    lens = lens_spec(rng) if callable(lens_spec) else np.asarray(lens_spec, dtype=np.int64)
    if use_factors:
        factors = np.exp2(rng.uniform(-2.0, 2.0, size=(3, N_HEADS))).astype(np.float32)
    else:
        factors = np.ones((3, N_HEADS), dtype=np.float32)
    masks = []
    for d in (D_QK, D_QK, D_V):
        m = np.zeros((N_HEADS, d), dtype=bool)
        if use_outliers:
            n = max(1, int(round(0.001 * N_HEADS * d)))
            pos = rng.choice(N_HEADS * d, size=n, replace=False)
            m.reshape(-1)[pos] = True
        masks.append(m)
    return lens, factors, masks


# name -> (index, description, q lengths, k lengths (None: same as q), causal,
#          factors, outliers, segment_len). NC is the non-causal chunk of 4K queries over
#          65K context keys that the pull request's close comment times.
CONFIGS = {
    "C1": dict(index=1, desc="1 sequence x 128 tokens, causal, per-head factors",
               lens=[128], k_lens=None, causal=True, factors=True, outliers=False, segment=0),
    "C2": dict(index=2, desc="8 packed sequences, lengths U{256..4096}, causal, factors + outliers",
               lens=lambda rng: random_varlen(rng, 8, 256, 4096), k_lens=None, causal=True,
               factors=True, outliers=True, segment=0),
    "C3": dict(index=3, desc="1 sequence x 32768 tokens, causal, per-head factors",
               lens=[32768], k_lens=None, causal=True, factors=True, outliers=False, segment=0),
    "C4": dict(index=4, desc="4096 new queries over 65536 cached + 4096 new keys, causal "
                             "bottom-right; context in 4 segments of 16384; N(0,1)",
               lens=[4096], k_lens=[65536 + 4096], causal=True, factors=False, outliers=False,
               segment=16384),
    "C5": dict(index=5, desc="1 sequence x 131072 tokens, causal, factors + outliers; "
                             "8 segments of 16384",
               lens=[131072], k_lens=None, causal=True, factors=True, outliers=True,
               segment=16384),
    "NC": dict(index=6, desc="4096 queries x 65536 context keys, non-causal (one context "
                             "chunk); N(0,1)",
               lens=[4096], k_lens=[65536], causal=False, factors=False, outliers=False,
               segment=0),
}


def make_workload(name: str, scale_tokens: Optional[int] = None) -> Workload:
    """Build a named workload. ``scale_tokens`` (tests only) replaces every length by
    that value with the same structure draw, to get small variants of a config."""
    spec = CONFIGS[name]
    seed = 1000 * spec["index"]
    lens, factors, masks = _structure(seed, spec["lens"], spec["factors"], spec["outliers"])
    k_lens = np.asarray(spec["k_lens"], dtype=np.int64) if spec["k_lens"] is not None else lens
    if scale_tokens is not None:
        lens = np.full_like(lens, scale_tokens)
        k_lens = np.full_like(k_lens, scale_tokens)
    cu_q = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = _draw(rng, (tq, N_HEADS, D_QK), factors[0], masks[0])
    k = _draw(rng, (tk, N_HEADS, D_QK), factors[1], masks[1])
    v = _draw(rng, (tk, N_HEADS, D_V), factors[2], masks[2])
    return Workload(
        name=name, seed=seed, q=q, k=k, v=v, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
        causal=spec["causal"], softmax_scale=1.0 / math.sqrt(D_QK), factors=factors,
        outlier_mask=masks, segment_len=spec["segment"], description=spec["desc"],
    )


def make_random(seed: int, lens_q, lens_k=None, causal: bool = True, heads: int = N_HEADS,
                factor_range: float = 2.0, outliers: bool = False) -> Workload:
    """A small custom workload for tests (ragged lengths, Lq != Lk, fewer heads)."""
    rng_s = np.random.default_rng(seed + 2)
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = lens_q if lens_k is None else np.asarray(lens_k, dtype=np.int64)
    factors = np.exp2(rng_s.uniform(-factor_range, factor_range, size=(3, heads))).astype(np.float32)
    masks = []
    for d in (D_QK, D_QK, D_V):
        m = np.zeros((heads, d), dtype=bool)
        if outliers:
            pos = rng_s.choice(heads * d, size=max(1, int(round(0.001 * heads * d))), replace=False)
            m.reshape(-1)[pos] = True
        masks.append(m)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    q = _draw(rng, (int(cu_q[-1]), heads, D_QK), factors[0], masks[0])
    k = _draw(rng, (int(cu_k[-1]), heads, D_QK), factors[1], masks[1])
    v = _draw(rng, (int(cu_k[-1]), heads, D_V), factors[2], masks[2])
    return Workload(
        name=f"random{seed}", seed=seed, q=q, k=k, v=v, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
        causal=causal, softmax_scale=1.0 / math.sqrt(D_QK), factors=factors, outlier_mask=masks,
        segment_len=0, description="custom test workload",
    )


LATENT = 512
ROPE = 64


def make_latent(seed: int, n_tokens: int, heads: int = N_HEADS):
    """Latent-cache rows and an expansion weight for the un-absorbed K/V producer.

    Recipe: ``default_rng(seed)``; cache = bf16_RNE(standard normal [n_tokens, 576]) (the
    512 latent values of a token followed by its 64 rope-key values, one row per token,
    as a normalised latent and a rotated rope key would be); then
    w = bf16_RNE(standard normal [heads * 256, 512] / sqrt(512)), so that every expanded
    value is about unit-variance. Returns (cache bits [T, 576], w bits [heads * 256, 512]).
    """
    rng = np.random.default_rng(seed)
    cache = f32_to_bf16_bits(rng.standard_normal((n_tokens, LATENT + ROPE), dtype=np.float32))
    w = rng.standard_normal((heads * 256, LATENT), dtype=np.float32) * np.float32(1 / math.sqrt(LATENT))
    return cache, f32_to_bf16_bits(w)


def make_codes(seed: int, n_q: int, n_k: int, heads: int = N_HEADS, lo: int = 0x20,
               hi: int = 0x50):
    """E4M3 code bytes drawn directly, for contexts too long for a bf16 draw on the host.

    Recipe: ``default_rng(seed).bytes`` gives one random byte per element, Q [n_q, H, 192]
    first, then K [n_k, H, 192], then V [n_k, H, 128]; bit 7 is the sign and the low 7
    bits pick a magnitude code on lo..hi (0x20..0x50: values 2^-3 .. 2^3 spread evenly in
    the exponent) through a fixed 128-entry table. No NaN code can occur. Returns
    (q8, k8, v8) as uint8 arrays.
    """
    rng = np.random.default_rng(seed)
    table = (lo + (np.arange(128) * (hi - lo + 1)) // 128).astype(np.uint8)
    table = np.concatenate([table, table | np.uint8(0x80)])

    def draw(shape):
        n = int(np.prod(shape))
        raw = np.frombuffer(rng.bytes(n), dtype=np.uint8)
        return table[raw].reshape(shape)

    return draw((n_q, heads, D_QK)), draw((n_k, heads, D_QK)), draw((n_k, heads, D_V))
