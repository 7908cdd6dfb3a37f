"""Thin Python binding of libmla_fp8.so (ctypes).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream. If the library is not
built this module raises on first use; there is no fallback path.

Names mirror the C ABI in ``include/mla_fp8.h``.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from .build import LIB_PATH, variant_path

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_HIP = 3

D_QK = 192
D_V = 128

_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_vp = ctypes.c_void_p
_c_fp = ctypes.POINTER(ctypes.c_float)


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)}: {last_error()}")
        self.status = status


class QuantJob(ctypes.Structure):
    _fields_ = [
        ("x", _c_vp),
        ("stride_token", _c_i64),
        ("stride_head", _c_i64),
        ("n_tokens", _c_i64),
        ("head_dim", _c_i32),
        ("descale", _c_vp),
        ("y", _c_vp),
    ]


_LIB = None

# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "mla_abi_version": (ctypes.c_int, []),
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_fp8_quant_static": (ctypes.c_int, [ctypes.POINTER(QuantJob), _c_i32, _c_i32, _c_vp]),
    "mla_fp8_quant_dynamic": (ctypes.c_int, [ctypes.POINTER(QuantJob), _c_i32, _c_i32, _c_vp,
                                             _c_vp]),
    "mla_fp8_amax_per_head": (ctypes.c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_vp,
                                             _c_vp]),
    "mla_fp8_kv_produce": (ctypes.c_int, [
        _c_vp, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp,
        _c_vp, _c_vp, _c_vp, _c_vp]),
    "mla_fp8_prefill_varlen": (ctypes.c_int, [
        _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i64, _c_i64, _c_i32, _c_i32,
        _c_i32, _c_vp, _c_vp, _c_vp, ctypes.c_float, _c_i32, _c_vp, _c_vp, _c_i64, _c_vp]),
    "mla_bf16_prefill_varlen": (ctypes.c_int, [
        _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i64, _c_i64, _c_i32, _c_i32,
        _c_i32, ctypes.c_float, _c_i32, _c_vp, _c_vp, _c_i64, _c_vp]),
    "mla_merge_lse": (ctypes.c_int, [
        _c_i32, ctypes.POINTER(_c_vp), ctypes.POINTER(_c_vp), _c_i64, _c_i64, _c_i32, _c_i32, _c_vp,
        _c_vp, _c_i64, _c_vp]),
    "mla_fp8_prefill_chunked": (ctypes.c_int, [
        _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, ctypes.c_float, _c_i32,
        _c_i32, _c_vp, _c_vp, _c_i64, _c_vp, ctypes.c_uint64, _c_vp]),
    "mla_fp8_chunked_workspace_size": (ctypes.c_int, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                                      ctypes.POINTER(ctypes.c_uint64)]),
    "mla_fp8_prefill_chunked_noalloc": (ctypes.c_int, [
        _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, ctypes.c_float, _c_i32,
        _c_i32, _c_vp, _c_vp, _c_i64, _c_vp]),
    "mla_check_descales_host": (ctypes.c_int, [_c_fp, _c_i32]),
    "mla_descale_from_amax_host": (ctypes.c_int, [_c_fp, _c_i32, _c_fp]),
}


def lib_path() -> str:
    """The in-tree library, or the file named by MLA_FP8_LIB (for comparing builds)."""
    return os.environ.get("MLA_FP8_LIB", LIB_PATH)


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m fp8_mla_context_amd.build`")
    handle = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        _LIB = _load(lib_path())
    return _LIB


def pv_variant_path(mode: int) -> str:
    """The build variant of the FP8 prefill's PV arithmetic: 0 the default library (P and
    V in bf16 on the bf16 MFMA), 1 one E4M3 term of P, 2 two E4M3 terms (FP8 MFMA)."""
    return variant_path({0: "", 1: "_pv1", 2: "_pv2"}[mode], lib_path())


@contextlib.contextmanager
def use_library(path: str):
    """Route this module's calls to another build of the library (same exports) inside
    the block, e.g. a PV variant; the default library is restored afterwards."""
    global _LIB
    saved = _LIB
    _LIB = _load(path)
    try:
        yield _LIB
    finally:
        _LIB = saved


def status_string(status: int) -> str:
    return lib().mla_status_string(status).decode()


def last_error() -> str:
    return lib().mla_last_error().decode()


def _check(status: int, what: str):
    if status != MLA_OK:
        raise MlaError(status, what)


def _launch(name: str, args: tuple, keep: tuple, prepare: bool, result):
    """Call library entry point `name` with the marshalled args and return `result`; with
    prepare, make no call and return a zero-argument callable that makes exactly this call
    (same pointers, sizes and stream; `keep` holds the tensors the pointers refer to), so
    that timing loops measure the launch without the argument checks."""
    f = getattr(lib(), name)
    if prepare:
        def call(_f=f, _args=args, _keep=keep):
            _check(_f(*_args), name)
        return call
    _check(f(*args), name)
    return result


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# --------------------------------------------------------------------------- argument checks
#
# Every tensor argument is checked for dtype, shape and layout first and for its device
# last, all before the library is called: a host pointer or a mis-shaped operand handed
# to a kernel would make it read or write outside the caller's buffers.

def _tensor(name: str, t, dtype, shape=None, contiguous: bool = True):
    """t must be a tensor of `dtype` whose shape matches `shape` (None entries match any
    size); contiguous unless told otherwise. Returns t."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, not {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and w != g for w, g in zip(shape, t.shape)):
            want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
            raise ValueError(f"{name} must have shape {want}, not {list(t.shape)}")
    if contiguous and t.numel() > 0 and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _lse_view(name: str, t, heads: int, rows: int):
    """fp32 [heads, >= rows] with unit column stride; returns its row stride."""
    import torch

    _tensor(name, t, torch.float32, contiguous=False)
    if t.dim() != 2 or t.shape[0] != heads or t.shape[1] < rows:
        raise ValueError(f"{name} must be fp32 [{heads}, >= {rows}], not {list(t.shape)}")
    if t.numel() > 0 and (t.stride(1) != 1 or (heads > 1 and t.stride(0) < rows)):
        raise ValueError(f"{name} must have unit column stride and a row stride >= {rows}")
    return t.stride(0) if heads > 1 else max(rows, t.shape[1])


def _on_one_gpu(**named):
    """Every given tensor (None entries skipped) lives on one CUDA device."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA tensor (it is on {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


# --------------------------------------------------------------------------- host helpers

def check_descales_host(descale: np.ndarray) -> None:
    d = np.ascontiguousarray(descale, dtype=np.float32)
    _check(lib().mla_check_descales_host(d.ctypes.data_as(_c_fp), d.shape[0]),
           "mla_check_descales_host")


def descale_from_amax_host(amax: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty_like(a)
    _check(lib().mla_descale_from_amax_host(a.ctypes.data_as(_c_fp), a.shape[0],
                                            out.ctypes.data_as(_c_fp)),
           "mla_descale_from_amax_host")
    return out


# --------------------------------------------------------------------------- device ops

def amax_per_head(x, stream=None):
    """x: bf16 [T, H, D] (last dim contiguous). Returns fp32 [H] on x's device."""
    import torch

    _tensor("x", x, torch.bfloat16, (None, None, None), contiguous=False)
    if x.numel() > 0 and x.stride(2) != 1:
        raise ValueError("x must have a contiguous last dim")
    _on_one_gpu(x=x)
    amax = torch.empty(x.shape[1], dtype=torch.float32, device=x.device)
    _check(lib().mla_fp8_amax_per_head(_ptr(x), x.stride(0), x.stride(1), x.shape[0], x.shape[1],
                                       x.shape[2], _ptr(amax), _stream(stream)),
           "mla_fp8_amax_per_head")
    return amax


def quant_static(xs: Sequence, descales: Sequence, outs: Optional[Sequence] = None, stream=None,
                 prepare: bool = False):
    """Quantize 1..3 bf16 tensors [T, H, D] (token/head strides allowed, last dim contiguous)
    with fp32 [H] descales in ONE launch. Returns uint8 E4M3 code tensors [T, H, D] (with
    prepare: a callable that repeats the checked launch, see _launch)."""
    if len(xs) != len(descales) or not 1 <= len(xs) <= 3:
        raise ValueError("need 1..3 tensors and one descale vector each")
    jobs, ys, heads = _quant_jobs(xs, descales, outs)
    return _launch("mla_fp8_quant_static", (jobs, len(xs), heads, _stream(stream)),
                   (tuple(xs), tuple(descales), tuple(ys)), prepare, ys)


def _quant_jobs(xs, descales, outs):
    import torch

    if outs is not None and len(outs) != len(xs):
        raise ValueError("need one output per input tensor")
    heads = None
    for i, x in enumerate(xs):
        _tensor(f"x[{i}]", x, torch.bfloat16, (None, heads, None), contiguous=False)
        heads = x.shape[1]
        if x.numel() > 0 and x.stride(2) != 1:
            raise ValueError(f"x[{i}] must have a contiguous last dim")
        if descales is not None:
            _tensor(f"descale[{i}]", descales[i], torch.float32, (heads,))
        if outs is not None:
            _tensor(f"out[{i}]", outs[i], torch.uint8, tuple(x.shape))
    named = {f"x[{i}]": x for i, x in enumerate(xs)}
    if descales is not None:
        named.update({f"descale[{i}]": d for i, d in enumerate(descales)})
    if outs is not None:
        named.update({f"out[{i}]": y for i, y in enumerate(outs)})
    _on_one_gpu(**named)
    jobs = (QuantJob * len(xs))()
    ys = []
    for i, x in enumerate(xs):
        d = descales[i] if descales is not None else None
        y = outs[i] if outs is not None else torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        jobs[i] = QuantJob(_ptr(x), x.stride(0), x.stride(1), x.shape[0], x.shape[2],
                           _ptr(d) if d is not None else None, _ptr(y))
        ys.append(y)
    return jobs, ys, heads


def quant_dynamic(xs: Sequence, outs: Optional[Sequence] = None, descale_out=None, stream=None):
    """Dynamic per-head quantization of 1..3 bf16 tensors [T, H, D]: descales from the
    data's own per-head amax. Returns (codes list, fp32 descales [len(xs), H])."""
    import torch

    if not 1 <= len(xs) <= 3:
        raise ValueError("need 1..3 tensors")
    if descale_out is not None:
        _tensor("descale_out", descale_out, torch.float32, (len(xs), xs[0].shape[1]))
        _on_one_gpu(x=xs[0], descale_out=descale_out)
    jobs, ys, heads = _quant_jobs(xs, None, outs)
    if descale_out is None:
        descale_out = torch.empty((len(xs), heads), dtype=torch.float32, device=xs[0].device)
    _check(lib().mla_fp8_quant_dynamic(jobs, len(xs), heads, _ptr(descale_out), _stream(stream)),
           "mla_fp8_quant_dynamic")
    return ys, descale_out


def kv_produce(c_kv, k_pe, w_kv_b, descale_k, descale_v, out_bf16: bool = False, k8=None,
               v8=None, stream=None, prepare: bool = False):
    """Un-absorbed K/V expansion + static quantization. c_kv [T, >=512] and k_pe [T, >=64] bf16
    (row-strided views allowed), w_kv_b bf16 [H*256, 512]. Returns (k8 [T,H,192], v8 [T,H,128]
    uint8 codes) and, with out_bf16, also the bf16 K and V."""
    import torch

    for name, t in (("c_kv", c_kv), ("k_pe", k_pe), ("w_kv_b", w_kv_b)):
        _tensor(name, t, torch.bfloat16, (None, None), contiguous=False)
        if t.numel() > 0 and t.stride(1) != 1:
            raise ValueError(f"{name} must have unit column stride")
    n = c_kv.shape[0]
    if k_pe.shape[0] != n:
        raise ValueError("c_kv and k_pe must have the same number of rows")
    heads = w_kv_b.shape[0] // 256
    if heads < 1 or w_kv_b.shape[0] != heads * 256 or not w_kv_b.is_contiguous():
        raise ValueError("w_kv_b must be contiguous [n_heads * 256, 512]")
    _tensor("descale_k", descale_k, torch.float32, (heads,))
    _tensor("descale_v", descale_v, torch.float32, (heads,))
    if k8 is not None:
        _tensor("k8", k8, torch.uint8, (n, heads, D_QK))
    if v8 is not None:
        _tensor("v8", v8, torch.uint8, (n, heads, D_V))
    _on_one_gpu(c_kv=c_kv, k_pe=k_pe, w_kv_b=w_kv_b, descale_k=descale_k, descale_v=descale_v,
                k8=k8, v8=v8)
    dev = c_kv.device
    if k8 is None:
        k8 = torch.empty((n, heads, D_QK), dtype=torch.uint8, device=dev)
    if v8 is None:
        v8 = torch.empty((n, heads, D_V), dtype=torch.uint8, device=dev)
    kb = vb = None
    if out_bf16:
        kb = torch.empty((n, heads, D_QK), dtype=torch.bfloat16, device=dev)
        vb = torch.empty((n, heads, D_V), dtype=torch.bfloat16, device=dev)
    return _launch("mla_fp8_kv_produce", (
        _ptr(c_kv), c_kv.stride(0), _ptr(k_pe), k_pe.stride(0), _ptr(w_kv_b), n, heads,
        w_kv_b.shape[1], k_pe.shape[1], _ptr(descale_k), _ptr(descale_v), _ptr(k8), _ptr(v8),
        _ptr(kb), _ptr(vb), _stream(stream)),
        (c_kv, k_pe, w_kv_b, descale_k, descale_v, k8, v8, kb, vb), prepare,
        (k8, v8, kb, vb) if out_bf16 else (k8, v8))


def _attention_args(dtype, q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, lse_stride, descales):
    """Checks shared by the FP8 and BF16 varlen entry points; returns (out, lse, lse_stride)."""
    import torch

    _tensor("q", q, dtype, (None, None, D_QK))
    tq, heads = q.shape[0], q.shape[1]
    _tensor("k", k, dtype, (None, heads, D_QK))
    tk = k.shape[0]
    _tensor("v", v, dtype, (tk, heads, D_V))
    _tensor("cu_seqlens_q", cu_seqlens_q, torch.int32, (None,))
    _tensor("cu_seqlens_k", cu_seqlens_k, torch.int32, (cu_seqlens_q.shape[0],))
    if cu_seqlens_q.shape[0] < 1:
        raise ValueError("cu_seqlens must hold batch + 1 >= 1 entries")
    for name, d in descales.items():
        _tensor(name, d, torch.float32, (heads,))
    if out is not None:
        _tensor("out", out, torch.bfloat16, (tq, heads, D_V))
    if lse is not None:
        stride = _lse_view("lse", lse, heads, tq)
        if lse_stride is not None and lse_stride != stride:
            raise ValueError(f"lse_stride {lse_stride} differs from lse's row stride {stride}")
        lse_stride = stride
    _on_one_gpu(q=q, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, out=out,
                lse=lse, **descales)
    if out is None:
        out = torch.empty((tq, heads, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse_stride = tq if lse_stride is None else int(lse_stride)
        if lse_stride < tq:
            raise ValueError("lse_stride < total_q")
        lse = torch.empty((heads, lse_stride), dtype=torch.float32, device=q.device)
    return out, lse, lse_stride


def prefill_varlen(q8, k8, v8, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                   descale_q, descale_k, descale_v, softmax_scale: float, causal: bool,
                   out=None, lse=None, lse_stride: Optional[int] = None, stream=None,
                   prepare: bool = False):
    """FP8 varlen attention. q8 [Tq,H,192], k8 [Tk,H,192], v8 [Tk,H,128] uint8 codes (contiguous);
    cu_seqlens int32 [B+1] on device. Returns (out bf16 [Tq,H,128], lse fp32 [H, lse_stride])
    (with prepare: a callable that repeats the checked launch, see _launch)."""
    import torch

    out, lse, lse_stride = _attention_args(
        torch.uint8, q8, k8, v8, cu_seqlens_q, cu_seqlens_k, out, lse, lse_stride,
        {"descale_q": descale_q, "descale_k": descale_k, "descale_v": descale_v})
    tq, heads, tk = q8.shape[0], q8.shape[1], k8.shape[0]
    batch = cu_seqlens_q.shape[0] - 1
    return _launch("mla_fp8_prefill_varlen", (
        _ptr(q8), _ptr(k8), _ptr(v8), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch,
        int(max_seqlen_q), int(max_seqlen_k), tq, tk, heads, q8.shape[2], v8.shape[2],
        _ptr(descale_q), _ptr(descale_k), _ptr(descale_v), float(softmax_scale), int(bool(causal)),
        _ptr(out), _ptr(lse), int(lse_stride), _stream(stream)),
        (q8, k8, v8, cu_seqlens_q, cu_seqlens_k, descale_q, descale_k, descale_v, out, lse),
        prepare, (out, lse))


def prefill_varlen_bf16(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                        softmax_scale: float, causal: bool, out=None, lse=None,
                        lse_stride: Optional[int] = None, stream=None):
    """BF16 varlen attention (the comparator). q [Tq,H,192], k [Tk,H,192], v [Tk,H,128] bf16
    (contiguous). Returns (out bf16 [Tq,H,128], lse fp32 [H, lse_stride])."""
    import torch

    out, lse, lse_stride = _attention_args(torch.bfloat16, q, k, v, cu_seqlens_q, cu_seqlens_k, out,
                                           lse, lse_stride, {})
    tq, heads, tk = q.shape[0], q.shape[1], k.shape[0]
    batch = cu_seqlens_q.shape[0] - 1
    _check(lib().mla_bf16_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch,
        int(max_seqlen_q), int(max_seqlen_k), tq, tk, heads, q.shape[2], v.shape[2],
        float(softmax_scale), int(bool(causal)), _ptr(out), _ptr(lse), int(lse_stride),
        _stream(stream)), "mla_bf16_prefill_varlen")
    return out, lse


def merge_lse(outs: Sequence, lses: Sequence, out=None, lse_out=None, stream=None,
              prepare: bool = False):
    """Merge partials: outs bf16 [T,H,128] each, lses fp32 [H, ld] each (same ld). Returns
    (out, lse_out) (with prepare: a callable that repeats the checked launch, see _launch)."""
    import torch

    n = len(outs)
    if n != len(lses) or n < 1:
        raise ValueError("need one lse per output")
    _tensor("outs[0]", outs[0], torch.bfloat16, (None, None, D_V))
    tq, heads = outs[0].shape[0], outs[0].shape[1]
    ld_in = None
    for i, (o, l_) in enumerate(zip(outs, lses)):
        _tensor(f"outs[{i}]", o, torch.bfloat16, (tq, heads, D_V))
        ld = _lse_view(f"lses[{i}]", l_, heads, tq)
        if ld_in is None:
            ld_in = ld
        elif ld != ld_in:
            raise ValueError("lses must share one row stride")
    if out is not None:
        _tensor("out", out, torch.bfloat16, (tq, heads, D_V))
    ld_out = None
    if lse_out is not None:
        ld_out = _lse_view("lse_out", lse_out, heads, tq)
    named = {f"outs[{i}]": o for i, o in enumerate(outs)}
    named.update({f"lses[{i}]": l_ for i, l_ in enumerate(lses)})
    _on_one_gpu(out=out, lse_out=lse_out, **named)
    if out is None:
        out = torch.empty_like(outs[0])
    if lse_out is None:
        lse_out = torch.empty((heads, tq), dtype=torch.float32, device=outs[0].device)
        ld_out = tq
    op = (_c_vp * n)(*[_ptr(o) for o in outs])
    lp = (_c_vp * n)(*[_ptr(l_) for l_ in lses])
    return _launch("mla_merge_lse", (n, op, lp, ld_in, tq, heads, D_V, _ptr(out), _ptr(lse_out),
                                     ld_out, _stream(stream)),
                   (tuple(outs), tuple(lses), out, lse_out), prepare, (out, lse_out))


def chunked_workspace_size(lq: int, lk: int, n_heads: int, seg_len: int, causal: bool = True) -> int:
    n = ctypes.c_uint64(0)
    _check(lib().mla_fp8_chunked_workspace_size(lq, lk, n_heads, seg_len, int(bool(causal)),
                                                ctypes.byref(n)), "mla_fp8_chunked_workspace_size")
    return int(n.value)


def prefill_chunked_noalloc(q8, k8, v8, descale_q, descale_k, descale_v, softmax_scale: float,
                            seg_len: int, causal: bool = True, out=None, lse=None, stream=None):
    """prefill_chunked with the library's own device scratch instead of a workspace: the call
    itself allocates nothing (pass out and lse to keep this wrapper from allocating them)."""
    import torch

    _tensor("q8", q8, torch.uint8, (None, None, D_QK))
    lq, heads = q8.shape[0], q8.shape[1]
    _tensor("k8", k8, torch.uint8, (None, heads, D_QK))
    lk = k8.shape[0]
    _tensor("v8", v8, torch.uint8, (lk, heads, D_V))
    for name, d in (("descale_q", descale_q), ("descale_k", descale_k), ("descale_v", descale_v)):
        _tensor(name, d, torch.float32, (heads,))
    if out is not None:
        _tensor("out", out, torch.bfloat16, (lq, heads, D_V))
    lse_stride = lq
    if lse is not None:
        lse_stride = _lse_view("lse", lse, heads, lq)
    _on_one_gpu(q8=q8, k8=k8, v8=v8, descale_q=descale_q, descale_k=descale_k,
                descale_v=descale_v, out=out, lse=lse)
    if out is None:
        out = torch.empty((lq, heads, D_V), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((heads, lq), dtype=torch.float32, device=q8.device)
    _check(lib().mla_fp8_prefill_chunked_noalloc(
        _ptr(q8), _ptr(k8), _ptr(v8), lq, lk, heads, _ptr(descale_q), _ptr(descale_k),
        _ptr(descale_v), float(softmax_scale), int(seg_len), int(bool(causal)), _ptr(out), _ptr(lse),
        lse_stride, _stream(stream)), "mla_fp8_prefill_chunked_noalloc")
    return out, lse


def prefill_chunked(q8, k8, v8, descale_q, descale_k, descale_v, softmax_scale: float, seg_len: int,
                    causal: bool = True, out=None, lse=None, workspace=None, stream=None,
                    prepare: bool = False):
    """One sequence of Lq queries (the last Lq of Lk tokens) over context segments of seg_len
    keys with one quantized Q; partials merged in the library. Returns (out, lse) (with
    prepare: a callable that repeats the checked launch, see _launch)."""
    import torch

    _tensor("q8", q8, torch.uint8, (None, None, D_QK))
    lq, heads = q8.shape[0], q8.shape[1]
    _tensor("k8", k8, torch.uint8, (None, heads, D_QK))
    lk = k8.shape[0]
    _tensor("v8", v8, torch.uint8, (lk, heads, D_V))
    for name, d in (("descale_q", descale_q), ("descale_k", descale_k), ("descale_v", descale_v)):
        _tensor(name, d, torch.float32, (heads,))
    if out is not None:
        _tensor("out", out, torch.bfloat16, (lq, heads, D_V))
    lse_stride = lq
    if lse is not None:
        lse_stride = _lse_view("lse", lse, heads, lq)
    if workspace is not None:
        _tensor("workspace", workspace, torch.uint8, (None,))
    _on_one_gpu(q8=q8, k8=k8, v8=v8, descale_q=descale_q, descale_k=descale_k,
                descale_v=descale_v, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty((lq, heads, D_V), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((heads, lq), dtype=torch.float32, device=q8.device)
    need = chunked_workspace_size(lq, lk, heads, seg_len, causal)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q8.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    return _launch("mla_fp8_prefill_chunked", (
        _ptr(q8), _ptr(k8), _ptr(v8), lq, lk, heads, _ptr(descale_q), _ptr(descale_k),
        _ptr(descale_v), float(softmax_scale), int(seg_len), int(bool(causal)), _ptr(out), _ptr(lse),
        lse_stride, _ptr(workspace), ws_bytes, _stream(stream)),
        (q8, k8, v8, descale_q, descale_k, descale_v, out, lse, workspace), prepare, (out, lse))
