"""GPU parity of the dynamic per-head quantizer (mla_fp8_quant_dynamic): bit-exact E4M3
bytes and descales against oracle.quant_dynamic, which is pinned in
tests/test_oracle_quant_dynamic.py."""

import numpy as np
import pytest

import oracle
from synth import make_workload
from tests.gpu_helpers import dev_bf16, host
from tests.quant_cases import all_bf16_patterns

pytestmark = pytest.mark.gpu


def _check(B, xs_np, xs_dev=None):
    xs_dev = xs_dev if xs_dev is not None else [dev_bf16(x) for x in xs_np]
    codes, d = B.quant_dynamic(xs_dev)
    d = host(d)
    for j, x in enumerate(xs_np):
        ref_c, ref_d = oracle.quant_dynamic(x)
        assert np.array_equal(d[j].view(np.uint32), ref_d.view(np.uint32)), (j, d[j], ref_d)
        got = host(codes[j])
        bad = np.argwhere(got != ref_c)
        assert bad.size == 0, (j, [(tuple(i), hex(int(x[tuple(i)])), int(got[tuple(i)]),
                                    int(ref_c[tuple(i)])) for i in bad[:6]])


def test_three_tensors_with_outliers(gpu_lib):
    wl = make_workload("C2")
    _check(gpu_lib, [wl.q, wl.k, wl.v])


def test_special_heads(gpu_lib):
    rng = np.random.default_rng(11)
    z = rng.standard_normal((300, 6, 192)).astype(np.float32)
    z *= np.array([1.0, 1e-3, 3e4, 2.0 ** -125, 1.0, 7.0], dtype=np.float32)[None, :, None]
    x = (z.view(np.uint32) >> 16).astype(np.uint16)
    x[:, 4, :] = 0          # an all-zero head (with some -0)
    x[::3, 4, ::5] = 0x8000
    x[17, 5, 40] = 0x7F7F   # the largest finite bf16 in one head
    _check(gpu_lib, [x])


@pytest.mark.parametrize("head_dim", [128, 192])
def test_every_finite_bf16_pattern(gpu_lib, head_dim):
    pats = all_bf16_patterns()
    finite = pats[(pats & 0x7F80) != 0x7F80]
    tokens = -(-finite.size // head_dim)
    buf = np.zeros(tokens * head_dim, dtype=np.uint16)
    heads = 3
    x = np.zeros((tokens, heads, head_dim), dtype=np.uint16)
    for h in range(heads):
        buf[:finite.size] = np.roll(finite, 1009 * h)
        x[:, h, :] = buf.reshape(tokens, head_dim)
    # a second tensor whose heads only hold small values, so its descales are small
    small = np.where(np.abs((x.astype(np.uint32) << 16).view(np.float32)) < 1e-3, x, 0).astype(np.uint16)
    _check(gpu_lib, [x, small])


def test_strided_views(gpu_lib):
    import torch

    rng = np.random.default_rng(5)
    big = rng.standard_normal((64, 12, 2 * 192)).astype(np.float32)
    bits = (big.view(np.uint32) >> 16).astype(np.uint16)
    t = dev_bf16(bits)
    view_vec = t[:, :, 192:]           # strides multiple of 8: 16-byte path
    view_odd = t[:, :, 1:193]          # odd offset: element-wise path
    xs_np = [np.ascontiguousarray(bits[:, :, 192:]), np.ascontiguousarray(bits[:, :, 1:193])]
    _check(gpu_lib, xs_np, [view_vec, view_odd])
    assert torch.cuda.is_available()


def test_empty_input_gives_unit_descales(gpu_lib):
    import torch

    x = torch.empty((0, 12, 128), dtype=torch.bfloat16, device="cuda")
    codes, d = gpu_lib.quant_dynamic([x])
    assert codes[0].numel() == 0
    assert np.all(host(d) == 1.0)
