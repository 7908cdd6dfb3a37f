"""GPU parity of the static quantizer and the calibration path: bit-exact E4M3
bytes and descales against the oracle (itself pinned to an exact-rational
rounder), over every bf16 pattern, for ordinary and adversarial descales,
contiguous and strided inputs, and the one-launch Q+K+V form."""

import numpy as np
import pytest

import oracle
from synth import make_workload
from tests.gpu_helpers import dev, dev_bf16, gpu_descales, gpu_quant, host, oracle_codes, oracle_descales
from tests.quant_cases import adversarial_descales, all_bf16_patterns, standard_descales

pytestmark = pytest.mark.gpu


def _exhaustive_tensor(n_heads, head_dim):
    # every head holds all 65536 bf16 patterns once (in a rotated order per head)
    pats = all_bf16_patterns()
    tokens = 65536 // head_dim + (1 if 65536 % head_dim else 0)
    x = np.zeros((tokens, n_heads, head_dim), dtype=np.uint16)
    for h in range(n_heads):
        flat = np.roll(pats, 977 * h)
        buf = np.zeros(tokens * head_dim, dtype=np.uint16)
        buf[:65536] = flat
        x[:, h, :] = buf.reshape(tokens, head_dim)
    return x


@pytest.mark.parametrize("head_dim", [128, 192])
def test_all_bf16_patterns_bit_exact(gpu_lib, head_dim):
    B = gpu_lib
    desc = np.array(list(standard_descales()) + list(adversarial_descales()[:4]), dtype=np.float32)
    x = _exhaustive_tensor(desc.shape[0], head_dim)
    (y,) = B.quant_static([dev_bf16(x)], [dev(desc)])
    got = host(y)
    exp = oracle.quant_static(x, desc)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, [(tuple(i), hex(int(x[tuple(i)])), int(got[tuple(i)]), int(exp[tuple(i)]))
                           for i in bad[:8]]


def test_three_jobs_one_launch_workload_c2(gpu_lib):
    B = gpu_lib
    wl = make_workload("C2")
    d_gpu = gpu_descales(B, wl)
    d_ref = oracle_descales(wl)
    for a, b in zip(d_gpu, d_ref):
        assert np.array_equal(a, b)
    codes, _ = gpu_quant(B, wl, d_gpu)
    ref = oracle_codes(wl, d_ref)
    for c, r in zip(codes, ref):
        assert np.array_equal(host(c), r)


def test_strided_views_vector_and_scalar_paths(gpu_lib):
    import torch

    B = gpu_lib
    rng = np.random.default_rng(42)
    T, H = 333, 12
    d = (np.exp2(rng.uniform(-8, 0, H))).astype(np.float32)
    for pad in (64, 4):  # 192+64: 16-byte aligned strides; 192+4: element-wise path
        full = (rng.standard_normal((T, H, 192 + pad)) * 3).astype(np.float32)
        bits = ((full.view(np.uint32) + 0x7FFF + ((full.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
        xd = dev_bf16(bits)[:, :, :192]
        assert xd.stride(1) == 192 + pad
        (y,) = B.quant_static([xd], [dev(d)])
        exp = oracle.quant_static(np.ascontiguousarray(bits[:, :, :192]), d)
        assert np.array_equal(host(y), exp)
    # token-major slice of a [T, 2H, D] tensor: head stride D, token stride 2*H*D
    big = (rng.standard_normal((T, 2 * H, 128)) * 5).astype(np.float32)
    bits = ((big.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    xd = dev_bf16(bits)[:, H:, :]
    (y,) = B.quant_static([xd], [dev(d)])
    assert np.array_equal(host(y), oracle.quant_static(np.ascontiguousarray(bits[:, H:, :]), d))


def test_amax_bit_exact(gpu_lib):
    B = gpu_lib
    wl = make_workload("C1")
    for c in wl.calib():
        got = host(B.amax_per_head(dev_bf16(c)))
        assert np.array_equal(got, oracle.amax_per_head(c))


def test_zero_tokens_is_noop(gpu_lib):
    import torch

    B = gpu_lib
    x = torch.empty((0, 12, 192), dtype=torch.bfloat16, device="cuda")
    (y,) = B.quant_static([x], [torch.ones(12, dtype=torch.float32, device="cuda")])
    assert y.shape == (0, 12, 192)
    a = B.amax_per_head(x)
    assert np.array_equal(host(a), np.zeros(12, np.float32))


def test_many_heads_scale_lookup_without_lds_table(gpu_lib):
    """Many (tensor, head) pairs (3 x 1100) of a few tokens each: one workgroup, one code
    table and one amax reduction per pair; codes and descales stay bit-exact, for the
    static and the dynamic path."""
    B = gpu_lib
    rng = np.random.default_rng(7)
    T, H = 5, 1100
    xs, ds = [], []
    for dim in (192, 192, 128):
        z = (rng.standard_normal((T, H, dim)) * 4).astype(np.float32)
        xs.append(((z.view(np.uint32) + 0x8000) >> 16).astype(np.uint16))
        ds.append(np.exp2(rng.uniform(-9, 1, H)).astype(np.float32))
    got = B.quant_static([dev_bf16(x) for x in xs], [dev(d) for d in ds])
    for g, x, d in zip(got, xs, ds):
        assert np.array_equal(host(g), oracle.quant_static(x, d))
    codes, d_gpu = B.quant_dynamic([dev_bf16(x) for x in xs])
    for i, (g, x) in enumerate(zip(codes, xs)):
        c_ref, d_ref = oracle.quant_dynamic(x)
        assert np.array_equal(host(d_gpu[i]), d_ref)
        assert np.array_equal(host(g), c_ref)


def test_descales_at_the_contract_edges(gpu_lib):
    """Every bf16 pattern at descales 2^-126 and 2^126 and next to them: the code table's
    window then starts below binade 0 or ends above binade 255 (entries that no bf16
    magnitude reaches); codes stay those of the exact quotient."""
    B = gpu_lib
    desc = np.array([2.0 ** -126, 1.5 * 2.0 ** -126, 1.999 * 2.0 ** -120, 2.0 ** 126,
                     1.75 * 2.0 ** 125, 2.0 ** 120], dtype=np.float32)
    x = _exhaustive_tensor(desc.shape[0], 128)
    (y,) = B.quant_static([dev_bf16(x)], [dev(desc)])
    got = host(y)
    exp = oracle.quant_static(x, desc)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, [(tuple(i), hex(int(x[tuple(i)])), int(got[tuple(i)]), int(exp[tuple(i)]))
                           for i in bad[:8]]


def test_jobs_of_different_lengths_with_an_empty_one(gpu_lib):
    """Three jobs in one launch, the middle one empty: each job's workgroups cover exactly
    its own tokens (257, 0 and 700 tokens; ragged last tiles)."""
    B = gpu_lib
    rng = np.random.default_rng(11)
    H = 12
    shapes = [(257, H, 192), (0, H, 192), (700, H, 128)]
    xs, ds = [], []
    for shp in shapes:
        z = (rng.standard_normal(shp) * 3).astype(np.float32)
        xs.append(((z.view(np.uint32) + 0x8000) >> 16).astype(np.uint16))
        ds.append(np.exp2(rng.uniform(-8, 0, H)).astype(np.float32))
    got = B.quant_static([dev_bf16(x) for x in xs], [dev(d) for d in ds])
    for g, x, d in zip(got, xs, ds):
        assert tuple(g.shape) == x.shape
        if x.shape[0]:
            assert np.array_equal(host(g), oracle.quant_static(x, d))
