"""CPU checks of the Python binding's argument validation.

Every tensor argument is checked (dtype, shape, layout, then device) before the
library is called, so a mis-shaped operand or a host tensor never reaches a
kernel as a pointer. Shape errors are raised for CPU tensors too; correctly
shaped CPU tensors fail the device check.
"""

import pytest
import torch

from fp8_mla_context_amd import binding as B

H, TQ, TK = 3, 10, 14


def _u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def _f32(*shape):
    return torch.ones(shape, dtype=torch.float32)


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _cu(n=2):
    return torch.zeros(n, dtype=torch.int32)


def _prefill(**kw):
    args = dict(q8=_u8(TQ, H, 192), k8=_u8(TK, H, 192), v8=_u8(TK, H, 128), cu_seqlens_q=_cu(),
                cu_seqlens_k=_cu(), max_seqlen_q=TQ, max_seqlen_k=TK, descale_q=_f32(H),
                descale_k=_f32(H), descale_v=_f32(H), softmax_scale=0.1, causal=True)
    args.update(kw)
    return B.prefill_varlen(**args)


@pytest.mark.parametrize("kw,msg", [
    (dict(q8=_u8(TQ, H, 128)), "q must have shape"),
    (dict(q8=_bf(TQ, H, 192)), "q must be torch.uint8"),
    (dict(k8=_u8(TK, H + 1, 192)), "k must have shape"),
    (dict(v8=_u8(TK, H, 192)), "v must have shape"),
    (dict(v8=_u8(TK + 1, H, 128)), "v must have shape"),
    (dict(k8=_u8(TK, 192, H).transpose(1, 2)), "k must be contiguous"),
    (dict(cu_seqlens_q=torch.zeros(2, dtype=torch.int64)), "cu_seqlens_q must be torch.int32"),
    (dict(cu_seqlens_k=_cu(3)), "cu_seqlens_k must have shape"),
    (dict(descale_k=_f32(H + 1)), "descale_k must have shape"),
    (dict(descale_v=torch.ones(H, dtype=torch.float64)), "descale_v must be torch.float32"),
    (dict(out=_bf(TQ, H, 192)), "out must have shape"),
    (dict(out=_f32(TQ, H, 128)), "out must be torch.bfloat16"),
    (dict(lse=_f32(TQ, H).t()), "unit column stride"),
    (dict(lse=_f32(H, TQ - 1)), "lse must be fp32"),
    (dict(lse=_f32(H + 1, TQ)), "lse must be fp32"),
    (dict(), "must be a CUDA tensor"),
])
def test_prefill_varlen_rejects(kw, msg):
    with pytest.raises(ValueError, match=msg):
        _prefill(**kw)


def test_prefill_varlen_bf16_rejects():
    with pytest.raises(ValueError, match="q must be torch.bfloat16"):
        B.prefill_varlen_bf16(_u8(TQ, H, 192), _bf(TK, H, 192), _bf(TK, H, 128), _cu(), _cu(), TQ,
                              TK, 0.1, True)
    with pytest.raises(ValueError, match="v must have shape"):
        B.prefill_varlen_bf16(_bf(TQ, H, 192), _bf(TK, H, 192), _bf(TK, H, 64), _cu(), _cu(), TQ,
                              TK, 0.1, True)
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        B.prefill_varlen_bf16(_bf(TQ, H, 192), _bf(TK, H, 192), _bf(TK, H, 128), _cu(), _cu(), TQ,
                              TK, 0.1, True)


def _chunked(**kw):
    args = dict(q8=_u8(TQ, H, 192), k8=_u8(TK, H, 192), v8=_u8(TK, H, 128), descale_q=_f32(H),
                descale_k=_f32(H), descale_v=_f32(H), softmax_scale=0.1, seg_len=4, causal=True)
    args.update(kw)
    return B.prefill_chunked(**args)


@pytest.mark.parametrize("kw,msg", [
    (dict(k8=_u8(TK, H, 128)), "k8 must have shape"),
    (dict(v8=_u8(TK - 1, H, 128)), "v8 must have shape"),
    (dict(descale_q=_f32(1)), "descale_q must have shape"),
    (dict(out=_bf(TQ + 1, H, 128)), "out must have shape"),
    (dict(lse=_f32(H, TQ)[:, ::2]), "lse must be fp32|unit column stride"),
    (dict(workspace=_f32(16)), "workspace must be torch.uint8"),
    (dict(), "must be a CUDA tensor"),
])
def test_prefill_chunked_rejects(kw, msg):
    with pytest.raises(ValueError, match=msg):
        _chunked(**kw)


def test_merge_rejects():
    outs = [_bf(TQ, H, 128), _bf(TQ, H, 128)]
    lses = [_f32(H, TQ), _f32(H, TQ)]
    with pytest.raises(ValueError, match="outs\\[1\\] must have shape"):
        B.merge_lse([outs[0], _bf(TQ + 1, H, 128)], lses)
    with pytest.raises(ValueError, match="share one row stride"):
        B.merge_lse(outs, [lses[0], _f32(H, TQ + 4)])
    with pytest.raises(ValueError, match="lses\\[0\\] must be fp32"):
        B.merge_lse(outs, [_f32(H + 1, TQ), lses[1]])
    with pytest.raises(ValueError, match="out must have shape"):
        B.merge_lse(outs, lses, out=_bf(TQ, H, 64))
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        B.merge_lse(outs, lses)


def test_quant_rejects():
    x = _bf(TQ, H, 192)
    with pytest.raises(ValueError, match="descale\\[0\\] must have shape"):
        B.quant_static([x], [_f32(H + 2)])
    with pytest.raises(ValueError, match="out\\[0\\] must have shape"):
        B.quant_static([x], [_f32(H)], outs=[_u8(TQ, H, 128)])
    with pytest.raises(ValueError, match="x\\[1\\] must have shape"):
        B.quant_static([x, _bf(TQ, H + 1, 128)], [_f32(H), _f32(H)])
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        B.quant_static([x], [_f32(H)])
    with pytest.raises(ValueError, match="descale_out must have shape"):
        B.quant_dynamic([x], descale_out=_f32(2, H))
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        B.amax_per_head(x)


def test_kv_produce_rejects():
    c = _bf(TK, 576)
    w = _bf(H * 256, 512)
    with pytest.raises(ValueError, match="descale_k must have shape"):
        B.kv_produce(c[:, :512], c[:, 512:], w, _f32(H + 1), _f32(H))
    with pytest.raises(ValueError, match="k8 must have shape"):
        B.kv_produce(c[:, :512], c[:, 512:], w, _f32(H), _f32(H), k8=_u8(TK, H, 128))
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        B.kv_produce(c[:, :512], c[:, 512:], w, _f32(H), _f32(H))


def test_prepare_checks_like_the_call():
    """prepare=True runs the same checks before it returns a callable, so a bad argument
    raises at preparation, never at a later launch."""
    with pytest.raises(ValueError, match="q must have shape"):
        _prefill(q8=_u8(TQ, H, 128), prepare=True)
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        _prefill(prepare=True)
    with pytest.raises(ValueError, match="v8 must have shape"):
        _chunked(v8=_u8(TK - 1, H, 128), prepare=True)
    with pytest.raises(ValueError, match="out\\[0\\] must have shape"):
        B.quant_static([_bf(TQ, H, 192)], [_f32(H)], outs=[_u8(TQ, H, 128)], prepare=True)
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        B.merge_lse([_bf(TQ, H, 128)], [_f32(H, TQ)], prepare=True)
    c = _bf(TK, 576)
    with pytest.raises(ValueError, match="descale_k must have shape"):
        B.kv_produce(c[:, :512], c[:, 512:], _bf(H * 256, 512), _f32(H + 1), _f32(H), prepare=True)
