"""GPU parity of the LSE merge against the oracle merge applied to the same
(bf16) partials: 1..8 segments, rows where some or all segments are empty
(-inf), in-place output, and LSE strides."""

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import dev, host
from tests.parity import bf16_bits_to_f64

pytestmark = pytest.mark.gpu


def _partials(rng, n, T, H):
    outs = (rng.standard_normal((n, T, H, 128)) * rng.uniform(0.1, 5, (n, 1, H, 1))).astype(np.float32)
    bits = ((outs.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    lses = (rng.standard_normal((n, H, T)) * 4).astype(np.float32)
    lses[rng.random((n, H, T)) < 0.2] = -np.inf
    lses[:, 0, :5] = -np.inf  # rows where every segment is empty
    return bits, lses


def _compare(got_out, got_lse, bits, lses):
    ref_o, ref_l = oracle.merge_lse([bf16_bits_to_f64(b) for b in bits], [l.astype(np.float64) for l in lses])
    o = bf16_bits_to_f64(host(got_out))
    scale = max(1e-30, float(np.max(np.abs(bf16_bits_to_f64(bits)))))
    assert np.all(np.abs(o - ref_o) <= 2.0 ** -8 * np.abs(ref_o) + 1e-5 * scale)
    gl = host(got_lse).astype(np.float64)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(gl))
    assert np.max(np.abs(gl[fin] - ref_l[fin])) <= 1e-5 * max(1.0, np.max(np.abs(ref_l[fin])))
    assert np.all(o[~fin.T] == 0.0)


@pytest.mark.parametrize("n", [1, 2, 5, 8, 64])  # 64: the most segments one merge takes
def test_merge_matches_oracle(gpu_lib, n):
    import torch

    B = gpu_lib
    rng = np.random.default_rng(n)
    T, H = 517, 12
    bits, lses = _partials(rng, n, T, H)
    outs = [dev(b.view(np.int16)).view(torch.bfloat16) for b in bits]
    ls = [dev(l) for l in lses]
    out, lse = B.merge_lse(outs, ls)
    _compare(out, lse, bits, lses)


def test_merge_in_place_and_strides(gpu_lib):
    import torch

    B = gpu_lib
    rng = np.random.default_rng(77)
    T, H, n = 300, 12, 3
    bits, lses = _partials(rng, n, T, H)
    outs = [dev(b.view(np.int16)).view(torch.bfloat16) for b in bits]
    # LSE partials live in wider buffers (ld = 512); merged LSE written into a slice of ld = 1000
    wide = [torch.full((H, 512), float("nan"), device="cuda") for _ in range(n)]
    for w, l in zip(wide, lses):
        w[:, :T] = dev(l)
    ls = [w[:, :T] for w in wide]
    final = torch.full((H, 1000), 7.0, device="cuda")
    out, lse = B.merge_lse(outs, ls, out=outs[0], lse_out=final[:, 100:100 + T])
    assert out.data_ptr() == outs[0].data_ptr()
    _compare(out, final[:, 100:100 + T], bits, lses)
    assert torch.all(final[:, :100] == 7.0) and torch.all(final[:, 100 + T:] == 7.0)
    # in place on the LSE too (equal strides)
    bits2, lses2 = _partials(np.random.default_rng(5), 2, T, H)
    outs2 = [dev(b.view(np.int16)).view(torch.bfloat16) for b in bits2]
    ls2 = [dev(l) for l in lses2]
    out2, lse2 = B.merge_lse(outs2, ls2, out=outs2[1], lse_out=ls2[1])
    _compare(out2, lse2, bits2, lses2)
