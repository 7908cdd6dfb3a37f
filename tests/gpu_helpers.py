"""Shared plumbing for the GPU parity tests: moving synthetic inputs to the device,
running the library path (calibration, quantization, prefill), and the oracle side."""

from __future__ import annotations

import numpy as np

import oracle


def dev_bf16(bits: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(arr: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


# ----------------------------------------------------------------- library (GPU) side

def gpu_descales(B, wl):
    """Calibration through the library: device amax kernel, then host amax/448."""
    out = []
    for c in wl.calib():
        if c.shape[0] == 0:
            out.append(None)
            continue
        amax = host(B.amax_per_head(dev_bf16(c)))
        d = B.descale_from_amax_host(amax)
        B.check_descales_host(d)
        out.append(d)
    return out


def gpu_quant(B, wl, descales):
    """One launch for Q, K, V. Returns device code tensors."""
    xs = [dev_bf16(wl.q), dev_bf16(wl.k), dev_bf16(wl.v)]
    ds = [dev(d) for d in descales]
    return B.quant_static(xs, ds), ds


def gpu_prefill(B, wl, codes, ds, causal=None):
    cu_q = dev(wl.cu_seqlens_q)
    cu_k = dev(wl.cu_seqlens_k)
    causal = wl.causal if causal is None else causal
    out, lse = B.prefill_varlen(codes[0], codes[1], codes[2], cu_q, cu_k, wl.max_seqlen_q,
                                wl.max_seqlen_k, ds[0], ds[1], ds[2], wl.softmax_scale, causal)
    return out, lse


# ----------------------------------------------------------------- oracle side

def oracle_descales(wl):
    return [oracle.descale_from_amax(oracle.amax_per_head(c)) for c in wl.calib()]


def oracle_codes(wl, descales):
    return [oracle.quant_static(x, d) for x, d in zip((wl.q, wl.k, wl.v), descales)]


def oracle_attention(wl, codes, descales, causal=None):
    causal = wl.causal if causal is None else causal
    return oracle.attention_varlen(codes[0], codes[1], codes[2], wl.cu_seqlens_q, wl.cu_seqlens_k,
                                   descales[0], descales[1], descales[2], wl.softmax_scale, causal)
