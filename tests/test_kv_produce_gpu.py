"""GPU parity of the fused un-absorbed K/V producer (mla_fp8_kv_produce) against the oracle.

The projection sums 512 products in fp32 on the matrix cores, the oracle exactly,
so the bar is: every bf16 K/V value the kernel produces is the nearest-even bf16 of
some value within E = 2^-16 * sum_j |c_j w_j| of the exact sum (in practice all
but a handful equal the oracle's), and every code is bit-exact for the bf16 value
the kernel produced (the quantizer decision taken on the same bf16 value on both
sides). End to end, the codes are also compared with the oracle's own producer (its
exactly rounded bf16 values, then its quantizer): the fraction of codes that differ is
reported and must stay below 1e-3, and every differing code must be at most one E4M3
step from the oracle's, at an element whose bf16 value differs. The rope part involves
no arithmetic before the quantizer and is bit-exact outright. Cases: ragged token counts around the 128-token tile, a row
stride (latent and rope key sharing one cache row), fewer heads, the optional
bf16 outputs on or off, and sampled tokens of a 32K-token call.
"""

import numpy as np
import pytest

import oracle
from synth import make_latent
from tests.gpu_helpers import dev, dev_bf16, host
from tests.parity import bf16_bits_to_f64, record

pytestmark = pytest.mark.gpu


def _descales(cache, w, heads):
    _, _, k, v = oracle.kv_produce(cache[:, :512], cache[:, 512:], w, np.ones(heads, np.float32),
                                   np.ones(heads, np.float32))
    return (oracle.descale_from_amax(oracle.amax_per_head(k)),
            oracle.descale_from_amax(oracle.amax_per_head(v)))


def _run(B, cache, w, dk, dv, out_bf16=True):
    d_cache = dev_bf16(cache)
    res = B.kv_produce(d_cache[:, :512], d_cache[:, 512:], dev_bf16(w), dev(dk), dev(dv),
                       out_bf16=out_bf16)
    return [host(t) for t in res]


def _allowed(c_bits, w_bits, heads, rows):
    """Exact projection y and the accumulation slack E for the given token rows."""
    c = bf16_bits_to_f64(c_bits[rows, :512])
    wv = bf16_bits_to_f64(w_bits).reshape(heads, 256, 512)
    y = np.einsum("tk,hfk->thf", c, wv)
    e = 2.0 ** -16 * np.einsum("tk,hfk->thf", np.abs(c), np.abs(wv))
    return y, e


def _check(B, n_tokens, heads, seed, sample=None):
    cache, w = make_latent(seed, n_tokens, heads)
    dk, dv = _descales(cache, w, heads) if sample is None else (
        np.full(heads, 4.5 / 448, np.float32), np.full(heads, 4.5 / 448, np.float32))
    k8, v8, kb, vb = _run(B, cache, w, dk, dv, out_bf16=True)
    rows = np.arange(n_tokens) if sample is None else sample
    k8, v8, kb, vb = k8[rows], v8[rows], kb[rows], vb[rows]
    pe = cache[rows, 512:]
    # rope part: the bf16 values are the cache's, the codes the oracle quantizer's
    for h in range(heads):
        assert np.array_equal(kb[:, h, 128:], pe)
    assert np.array_equal(k8, oracle.quant_static(kb, dk))  # codes exact for the kernel's bf16
    assert np.array_equal(v8, oracle.quant_static(vb, dv))
    y, e = _allowed(cache, w, heads, rows)
    got = np.concatenate([kb[:, :, :128], vb], axis=2)
    got_v = bf16_bits_to_f64(got)
    lo = bf16_bits_to_f64(oracle.rn_bf16_bits(y - e))
    hi = bf16_bits_to_f64(oracle.rn_bf16_bits(y + e))
    assert np.all((got_v >= lo) & (got_v <= hi))
    exact = oracle.rn_bf16_bits(y)
    agree = np.mean(got == exact)
    print(f"T={n_tokens} H={heads}: bf16 values equal to the exact rounding: {agree:.6f}", flush=True)
    assert agree >= 0.999
    # end to end against the oracle's producer on the same token rows
    rk8, rv8, _, _ = oracle.kv_produce(cache[rows, :512], cache[rows, 512:], w, dk, dv)
    codes = np.concatenate([k8[:, :, :128], v8], axis=2)
    rcodes = np.concatenate([rk8[:, :, :128], rv8], axis=2)
    assert np.array_equal(k8[:, :, 128:], rk8[:, :, 128:])  # rope part
    diff = codes != rcodes
    frac = float(np.mean(diff))

    def ordinal(c):  # E4M3 codes in value order (+0 and -0 both 0)
        c = c.astype(np.int64)
        return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)

    step = np.abs(ordinal(codes) - ordinal(rcodes))
    steps_ok = bool(np.all(step[diff] <= 1)) and bool(np.all(got[diff] != exact[diff]))
    print(f"T={n_tokens} H={heads}: codes differing from the oracle producer: {int(diff.sum())} of "
          f"{diff.size} ({frac:.2e}), all one step at a differing bf16 value: {steps_ok}", flush=True)
    record(f"kv_produce T={n_tokens} H={heads}", dict(code_mismatch_frac=frac,
                                                     code_mismatch=int(diff.sum()),
                                                     codes=int(diff.size),
                                                     bf16_exact_frac=float(agree),
                                                     one_step=steps_ok))
    assert frac <= 1e-3 and steps_ok
    return k8, v8


@pytest.mark.parametrize("n_tokens", [1, 127, 128, 129, 300, 1000])
def test_kv_produce_ragged(gpu_lib, n_tokens):
    # 1..129 tokens: one 256-token tile (work items in grid order); 300: two tiles, 24
    # items (each XCD a contiguous range); 1000: four tiles, the last of 232 tokens (each
    # XCD half of the heads over a quarter of the tiles)
    _check(gpu_lib, n_tokens, 12, 40 + n_tokens)


def test_kv_produce_few_heads_and_no_bf16_outputs(gpu_lib):
    B = gpu_lib
    cache, w = make_latent(7, 200, 3)
    dk, dv = _descales(cache, w, 3)
    k8a, v8a, _, _ = _run(B, cache, w, dk, dv, out_bf16=True)
    k8b, v8b = _run(B, cache, w, dk, dv, out_bf16=False)
    assert np.array_equal(k8a, k8b) and np.array_equal(v8a, v8b)
    _check(B, 200, 3, 7)


def test_kv_produce_32k_sampled(gpu_lib):
    rng = np.random.default_rng(8)
    n = 32768
    rows = np.unique(np.concatenate([[0, 1, 127, 128, n - 129, n - 1], rng.integers(0, n, 250)]))
    _check(gpu_lib, n, 12, 9, sample=rows)


def test_kv_produce_descales_across_the_contract(gpu_lib):
    """One descale per head across the contract [2^-126, 2^126]: its edges (where the code
    table's window starts below binade 0 or ends above binade 255), scales that put most
    codes among the E4M3 subnormals (64) or saturate them (2^-6), and ordinary ones. Every
    code equals the oracle quantizer's on the kernel's own bf16 value."""
    B = gpu_lib
    heads = 12
    cache, w = make_latent(21, 300, heads)
    d = np.array([2.0 ** -126, 2.0 ** 126, 64.0, 2.0 ** -6, 1.0, 0.0123, 3.0, 1.0 / 448,
                  2.0 ** -120, 2.0 ** 120, 0.7, 5.0], dtype=np.float32)
    dk, dv = d, d[::-1].copy()
    k8, v8, kb, vb = _run(B, cache, w, dk, dv, out_bf16=True)
    assert np.array_equal(k8, oracle.quant_static(kb, dk))
    assert np.array_equal(v8, oracle.quant_static(vb, dv))
