"""Binding of the debug build's per-tile softmax trace (libattn_debug.so).

The debug library is the release library compiled with ATTN_DEBUG_TRACE; it
exports every entry point of attn.h plus ``attn_debug_trace``
(include/attn_debug.h).  ``trace_prefill`` runs one prefill through it and
returns the traced row's state after every key tile: the per-iteration
m_i / l_i comparison that the attention-fusion page (section 6.3) uses to
find where a fused kernel departs from the reference.  Argument marshalling
only, like ``attn``; a missing library is an error.
"""

import ctypes
import math
import os

import numpy as np
import torch

from . import attn

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                         "libattn_debug.so")
_lib = None

_PREFILL = {torch.bfloat16: "attn_prefill", torch.float16: "attn_prefill_f16",
            torch.float32: "attn_prefill_f32"}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m causal_attention_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        for n in _PREFILL.values():
            fn = getattr(L, n)
            fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
            fn.restype = i
        L.attn_prefill_select.argtypes = [i]
        L.attn_prefill_select.restype = i
        L.attn_debug_trace.argtypes = [i, i, i, vp, i]
        L.attn_debug_trace.restype = i
        _lib = L
    return _lib


def trace_prefill(q, k, v, b, h, row, causal=True, scale=None,
                  capacity=1024):
    """One prefill through the debug library with query row ``row`` of
    (batch ``b``, query head ``h``) traced.  16-bit inputs run on the 4-wave
    kernel (the traced one), fp32 on the fp32 kernel.

    Returns (o, lse, records): records is a float64 array [n, 3] of
    (keys covered, m, l) for the tiles that wrote one, in tile order.
    """
    dtype = q.dtype
    if dtype not in _PREFILL:
        raise ValueError("q must be bfloat16, float16 or float32")
    B, Hq, Hkv, S, D = attn._prefill_shapes(q, k, v, dtype)
    if not (0 <= b < B and 0 <= h < Hq and 0 <= row < S):
        raise ValueError(f"trace target ({b}, {h}, {row}) outside "
                         f"B={B}, Hq={Hq}, S={S}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    attn._on_gpu(q=q, k=k, v=v)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    buf = torch.full((capacity, 3), float("nan"), dtype=torch.float32,
                     device=q.device)
    L = lib()
    torch.cuda.synchronize(q.device)
    st = L.attn_debug_trace(b, h, row, attn._ptr(buf), capacity)
    if st != 0:
        raise attn.AttnError(st, "attn_debug_trace")
    prev = L.attn_prefill_select(1)              # ATTN_PREFILL_W4
    try:
        name = _PREFILL[dtype]
        st = getattr(L, name)(attn._ptr(q), attn._ptr(k), attn._ptr(v),
                              attn._ptr(out), attn._ptr(lse), B, Hq, Hkv, S,
                              D, float(scale), int(bool(causal)),
                              attn._stream())
        if st != 0:
            raise attn.AttnError(st, name)
        torch.cuda.synchronize(q.device)
    finally:
        L.attn_prefill_select(prev)
        L.attn_debug_trace(0, 0, 0, None, 0)
    rec = buf.cpu().numpy().astype(np.float64)
    return out, lse, rec[~np.isnan(rec[:, 0])]
