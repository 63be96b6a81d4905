"""Python binding of libattn.so: argument marshalling only.

Each function checks tensor devices, dtypes, shapes and contiguity, allocates
outputs with torch, and calls the C entry point of the same name on torch's
current HIP stream.  Every step of the computation runs in the library's
kernels; there is no host fallback, and a missing library is an error.
"""

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                         "libattn.so")
_lib = None

STATUS = {
    0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE",
    -3: "ATTN_ERR_GQA", -4: "ATTN_ERR_HEAD_DIM", -5: "ATTN_ERR_ALIGN",
    -6: "ATTN_ERR_WORKSPACE", -7: "ATTN_ERR_SPLITS", -8: "ATTN_ERR_LAUNCH",
    -9: "ATTN_ERR_SCALE",
}
MAX_SPLITS = 4096
NOALLOC_SCRATCH_BYTES = 8 << 20


class AttnError(ValueError):
    def __init__(self, status, fn):
        self.status = status
        super().__init__(f"{fn} returned {status} "
                         f"({status_string(status)})")


def lib():
    """The loaded library (built by ``causal_attention_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m causal_attention_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, \
            ctypes.c_size_t
        L.attn_prefill.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.attn_prefill.restype = i
        L.attn_prefill_f16.argtypes = L.attn_prefill.argtypes
        L.attn_prefill_f16.restype = i
        L.attn_prefill_f32.argtypes = L.attn_prefill.argtypes
        L.attn_prefill_f32.restype = i
        L.attn_prefill_ws.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f,
                                      i, vp, sz, vp]
        L.attn_prefill_ws.restype = i
        L.attn_prefill_ws_f16.argtypes = L.attn_prefill_ws.argtypes
        L.attn_prefill_ws_f16.restype = i
        L.attn_prefill_workspace_size.argtypes = [i, i, i, i, i, i]
        L.attn_prefill_workspace_size.restype = sz
        L.attn_prefill_schedule.argtypes = [i, i, i, i, i, i]
        L.attn_prefill_schedule.restype = i
        L.attn_prefill_split_wait.argtypes = [i]
        L.attn_prefill_split_wait.restype = i
        L.attn_decode_workspace_size.argtypes = [i, i, i, i, i]
        L.attn_decode_workspace_size.restype = sz
        L.attn_decode_auto_splits.argtypes = [i, i]
        L.attn_decode_auto_splits.restype = i
        L.attn_prefill_select.argtypes = [i]
        L.attn_prefill_select.restype = i
        L.attn_prefill_kernel_for.argtypes = [i, i, i, i, i]
        L.attn_prefill_kernel_for.restype = i
        L.attn_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp,
                                  vp, sz, vp]
        L.attn_decode.restype = i
        L.attn_decode_f16.argtypes = L.attn_decode.argtypes
        L.attn_decode_f16.restype = i
        L.attn_decode_padded.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i,
                                         f, i, vp, f, vp, sz, vp]
        L.attn_decode_padded.restype = i
        L.attn_kv_append.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp]
        L.attn_kv_append.restype = i
        L.attn_prefill_rope.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i,
                                        i, f, i, f, vp]
        L.attn_prefill_rope.restype = i
        L.attn_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i,
                                          i, f, i, vp]
        L.attn_prefill_varlen.restype = i
        L.attn_prefill_padded.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i,
                                          i, f, i, vp]
        L.attn_prefill_padded.restype = i
        L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f,
                                          i, vp, vp]
        L.attn_decode_noalloc.restype = i
        L.attn_prefill_residual_rmsnorm.argtypes = [vp, vp, vp, vp, vp, vp,
                                                    vp, i, i, i, i, i, f, i,
                                                    f, vp]
        L.attn_prefill_residual_rmsnorm.restype = i
        for n in ("attn_prefill_rope_f16", "attn_prefill_varlen_f16",
                  "attn_prefill_padded_f16", "attn_kv_append_f16",
                  "attn_decode_padded_f16",
                  "attn_prefill_residual_rmsnorm_f16"):
            fn, base = getattr(L, n), getattr(L, n[:-4])
            fn.argtypes, fn.restype = base.argtypes, base.restype
        L.attn_status_string.argtypes = [i]
        L.attn_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status):
    return lib().attn_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t, name, dtype, ndim):
    """Type, dtype, rank and contiguity of one tensor argument (the device
    is checked by ``_on_gpu`` once every shape has been checked)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t, name, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, "
                         f"got {tuple(t.shape)}")


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def _fn(base, dtype):
    """The C entry point for a 16-bit storage type: ``base`` for bf16,
    ``base_f16`` for fp16."""
    if dtype == torch.bfloat16:
        return base
    if dtype == torch.float16:
        return base + "_f16"
    raise ValueError(f"{base}: tensors must be bfloat16 or float16, "
                     f"got {dtype}")


_PREFILL_FN = {torch.bfloat16: "attn_prefill", torch.float16: "attn_prefill_f16",
               torch.float32: "attn_prefill_f32"}
_DECODE_FN = {torch.bfloat16: "attn_decode", torch.float16: "attn_decode_f16"}


def _prefill_shapes(q, k, v, dtype):
    _check(q, "q", dtype, 4)
    _check(k, "k", dtype, 4)
    _check(v, "v", dtype, 4)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape:
        raise ValueError(f"k, v must be [B,Hkv,S,D] = [{B},{Hkv},{S},{D}]")
    return B, Hq, Hkv, S, D


def _lse_arg(lse, with_lse, shape, like):
    if with_lse and lse is None:
        lse = torch.empty(shape, dtype=torch.float32, device=like.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, len(shape))
        _shape(lse, "lse", shape)
    return lse


_PREFILL_WS_FN = {torch.bfloat16: "attn_prefill_ws",
                  torch.float16: "attn_prefill_ws_f16"}
_prefill_ws_on = True
_prefill_ws_cache = {}


def attn_prefill_workspace_size(B, Hq, Hkv, S, D, causal=True):
    """Bytes of workspace that enable the balanced causal schedule or the
    tile queue of a 16-bit prefill of these sizes on the current device (0:
    neither applies)."""
    return int(lib().attn_prefill_workspace_size(
        int(B), int(Hq), int(Hkv), int(S), int(D), int(bool(causal))))


SCHEDULE_STATIC, SCHEDULE_BALANCED, SCHEDULE_QUEUE = 0, 1, 2
SCHEDULE_NAMES = {SCHEDULE_STATIC: "static", SCHEDULE_BALANCED: "balanced",
                  SCHEDULE_QUEUE: "tile queue"}


def prefill_schedule(B, Hq, Hkv, S, D, causal=True):
    """SCHEDULE_STATIC, SCHEDULE_BALANCED or SCHEDULE_QUEUE: the schedule of
    a 16-bit ``attn_prefill`` of these sizes under the current kernel and
    workspace settings (a workspace is passed unless
    ``prefill_workspace_policy(False)`` is set)."""
    if not _prefill_ws_on:
        return SCHEDULE_STATIC
    return int(lib().attn_prefill_schedule(
        int(B), int(Hq), int(Hkv), int(S), int(D), int(bool(causal))))


def prefill_workspace_policy(on):
    """Whether ``attn_prefill`` and ``prepare_prefill`` pass a workspace to
    16-bit launches (the default) or call the plain entry points; returns
    the previous setting."""
    global _prefill_ws_on
    prev, _prefill_ws_on = _prefill_ws_on, bool(on)
    return prev


def prefill_split_wait(ticks):
    """Bound of the balanced schedule's wait for a partner's part, in ticks
    of the 100 MHz GPU real-time counter (-1: the kernel's own rule, 0: give
    up at once); returns the previous setting."""
    prev = int(lib().attn_prefill_split_wait(int(ticks)))
    if prev < -1:
        raise ValueError(f"attn_prefill_split_wait({ticks}): "
                         f"{status_string(prev)}")
    return prev


def new_prefill_workspace(B, Hq, Hkv, S, D, causal=True, device="cuda"):
    """A zeroed workspace for ``attn_prefill(..., workspace=)`` (uint8; at
    least one byte, so that it can be passed where none is needed)."""
    n = max(1, attn_prefill_workspace_size(B, Hq, Hkv, S, D, causal))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _prefill_workspace(q, B, Hq, Hkv, S, D, causal, workspace=None):
    """The workspace for one 16-bit prefill, or None: the caller's, else one
    zero-filled once and kept per (device, stream), so that calls sharing
    one never overlap (the library leaves its flag words and queue counter
    zero after every call)."""
    if q.dtype not in _PREFILL_WS_FN:
        return None
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, 1)
        return workspace
    if not _prefill_ws_on:
        return None
    nbytes = attn_prefill_workspace_size(B, Hq, Hkv, S, D, causal)
    if nbytes == 0:
        return None
    key = (q.device.index, torch.cuda.current_stream(q.device).cuda_stream)
    ws = _prefill_ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=q.device)
        _prefill_ws_cache[key] = ws
    return ws


def attn_prefill(q, k, v, causal=True, scale=None, out=None, lse=None,
                 with_lse=True, workspace=None):
    """Fused prefill attention.

    q [B,Hq,S,D]; k, v [B,Hkv,S,D]; bf16 (calls ``attn_prefill_ws`` or
    ``attn_prefill``), fp16 (``attn_prefill_ws_f16`` or
    ``attn_prefill_f16``) or fp32 (``attn_prefill_f32``).  Returns (o, lse)
    with o like q and lse fp32 [B,Hq,S] (None when ``with_lse`` is False).
    ``scale`` defaults to 1/sqrt(D).  16-bit launches get a workspace:
    ``workspace`` (uint8, from ``new_prefill_workspace``) if given, else one
    kept per stream unless ``prefill_workspace_policy(False)`` is set.
    """
    dtype = q.dtype
    if dtype not in _PREFILL_FN:
        raise ValueError("q must be bfloat16, float16 or float32")
    B, Hq, Hkv, S, D = _prefill_shapes(q, k, v, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dtype, 4)
    _shape(out, "out", q.shape)
    lse = _lse_arg(lse, with_lse, (B, Hq, S), q)
    _on_gpu(q=q, k=k, v=v, out=out, lse=lse, workspace=workspace)
    ws = _prefill_workspace(q, B, Hq, Hkv, S, D, causal, workspace)
    if ws is not None:
        name = _PREFILL_WS_FN[dtype]
        st = getattr(lib(), name)(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, S,
            D, float(scale), int(bool(causal)), _ptr(ws), ws.numel(),
            _stream())
    else:
        name = _PREFILL_FN[dtype]
        st = getattr(lib(), name)(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, S,
            D, float(scale), int(bool(causal)), _stream())
    if st != 0:
        raise AttnError(st, name)
    return out, lse


def attn_decode_auto_splits(B, Hkv):
    return int(lib().attn_decode_auto_splits(int(B), int(Hkv)))


def attn_decode_workspace_size(B, Hq, Hkv, D, num_splits=0):
    n = int(lib().attn_decode_workspace_size(B, Hq, Hkv, D, num_splits))
    if n == 0 and B > 0:
        raise ValueError("invalid decode sizes")
    return n


def new_decode_workspace(B, Hq, Hkv, D, num_splits=0, device="cuda"):
    """A workspace for attn_decode (reusable by calls on one stream)."""
    need = attn_decode_workspace_size(B, Hq, Hkv, D, num_splits) if B else 0
    return torch.zeros(max(need, 16), dtype=torch.uint8, device=device)


def _decode_outputs(q, out, lse, with_lse, workspace, Hkv, num_splits):
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.dtype, 3)
    _shape(out, "out", q.shape)
    lse = _lse_arg(lse, with_lse, (B, Hq), q)
    if workspace is None:
        workspace = new_decode_workspace(B, Hq, Hkv, D, num_splits, q.device)
    _check(workspace, "workspace", torch.uint8, 1)
    return out, lse, workspace


def attn_decode(q, kcache, vcache, seqlens, Hkv, num_splits=0, scale=None,
                out=None, with_lse=False, lse=None, workspace=None):
    """Split-K decode attention over a packed per-sequence KV cache.

    q [B,Hq,D] bf16 (calls ``attn_decode``) or fp16 (``attn_decode_f16``);
    kcache, vcache flat caches of q's dtype where sequence b is a
    [Hkv, L_b, D] block; seqlens int32 [B] on the GPU.  Returns (o, lse);
    lse is fp32 [B,Hq] or None.  ``workspace`` (uint8 GPU tensor, see
    ``new_decode_workspace``) is allocated when not given.
    """
    dtype = q.dtype
    if dtype not in _DECODE_FN:
        raise ValueError("q must be bfloat16 or float16")
    _check(q, "q", dtype, 3)
    _check(kcache, "kcache", dtype, None)
    _check(vcache, "vcache", dtype, None)
    _check(seqlens, "seqlens", torch.int32, 1)
    B, Hq, D = q.shape
    _shape(seqlens, "seqlens", (B,))
    if kcache.numel() != vcache.numel():
        raise ValueError("kcache and vcache must have the same size")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse, workspace = _decode_outputs(q, out, lse, with_lse, workspace,
                                          Hkv, num_splits)
    _on_gpu(q=q, kcache=kcache, vcache=vcache, seqlens=seqlens, out=out,
            lse=lse, workspace=workspace)
    fn = getattr(lib(), _DECODE_FN[dtype])
    st = fn(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(seqlens), _ptr(out), B,
            Hq, Hkv, D, float(scale), int(num_splits), _ptr(lse),
            _ptr(workspace), workspace.numel(), _stream())
    if st != 0:
        raise AttnError(st, _DECODE_FN[dtype])
    return out, lse


def attn_decode_noalloc(q, kcache, vcache, seqlens, Hkv, out, num_splits=0,
                        scale=None, lse=None):
    """``attn_decode`` (bf16) without a workspace argument: the library's
    fixed device-resident workspace is used (see ``attn_decode_noalloc`` in
    attn.h).  ``out`` (and ``lse`` if wanted) are required, so the call
    allocates nothing.  Returns (out, lse)."""
    _check(q, "q", torch.bfloat16, 3)
    _check(kcache, "kcache", torch.bfloat16, None)
    _check(vcache, "vcache", torch.bfloat16, None)
    _check(seqlens, "seqlens", torch.int32, 1)
    B, Hq, D = q.shape
    _shape(seqlens, "seqlens", (B,))
    if kcache.numel() != vcache.numel():
        raise ValueError("kcache and vcache must have the same size")
    _check(out, "out", torch.bfloat16, 3)
    _shape(out, "out", q.shape)
    if lse is not None:
        _check(lse, "lse", torch.float32, 2)
        _shape(lse, "lse", (B, Hq))
    _on_gpu(q=q, kcache=kcache, vcache=vcache, seqlens=seqlens, out=out,
            lse=lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = lib().attn_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache),
                                   _ptr(seqlens), _ptr(out), B, Hq, Hkv, D,
                                   float(scale), int(num_splits), _ptr(lse),
                                   _stream())
    if st != 0:
        raise AttnError(st, "attn_decode_noalloc")
    return out, lse


def attn_prefill_rope(q, k, v, rope_base, causal=True, scale=None, out=None,
                      lse=None, with_lse=True, k_rot=None):
    """Prefill attention of RoPE(q), RoPE(k), v at positions 0..S-1, bf16
    (``attn_prefill_rope``) or fp16 (``attn_prefill_rope_f16``).

    Returns (o, lse, k_rot) where k_rot [B,Hkv,S,D] holds the rotated keys
    (allocated when not given).  See ``attn_prefill_rope`` in attn.h.
    """
    name = _fn("attn_prefill_rope", q.dtype)
    B, Hq, Hkv, S, D = _prefill_shapes(q, k, v, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.dtype, 4)
    _shape(out, "out", q.shape)
    if k_rot is None:
        k_rot = torch.empty_like(k)
    _check(k_rot, "k_rot", q.dtype, 4)
    _shape(k_rot, "k_rot", k.shape)
    lse = _lse_arg(lse, with_lse, (B, Hq, S), q)
    _on_gpu(q=q, k=k, v=v, out=out, k_rot=k_rot, lse=lse)
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                              _ptr(lse), _ptr(k_rot), B, Hq, Hkv, S, D,
                              float(scale), int(bool(causal)),
                              float(rope_base), _stream())
    if st != 0:
        raise AttnError(st, name)
    return out, lse, k_rot


def attn_prefill_varlen(q, k, v, cu_seqlens, max_seqlen, Hq, Hkv, D,
                        causal=True, scale=None, out=None, lse=None,
                        with_lse=True):
    """Prefill of a ragged batch (bf16 or fp16), each sequence attended on
    its own.

    cu_seqlens int32 [B+1] on the GPU (cu[0] = 0, S_b = cu[b+1] - cu[b]);
    q (and o) hold [Hq, S_b, D] blocks at element offset Hq*D*cu[b], k and v
    [Hkv, S_b, D] blocks at Hkv*D*cu[b] (any contiguous shape with that many
    elements); lse [Hq*cu[B]] holds [Hq, S_b] blocks at offset Hq*cu[b].
    ``max_seqlen`` bounds every S_b.  Returns (o, lse).
    """
    name = _fn("attn_prefill_varlen", q.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, None)
    _check(cu_seqlens, "cu_seqlens", torch.int32, 1)
    B = cu_seqlens.shape[0] - 1
    if B < 0:
        raise ValueError("cu_seqlens needs B + 1 entries")
    if q.numel() % (Hq * D) or k.numel() % (Hkv * D) or \
            q.numel() // (Hq * D) != k.numel() // (Hkv * D) or \
            v.numel() != k.numel():
        raise ValueError("q, k, v sizes do not match Hq, Hkv and D")
    N = q.numel() // (Hq * D)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.dtype, None)
    if out.numel() != q.numel():
        raise ValueError("out must have q's size")
    if with_lse and lse is None:
        lse = torch.empty(Hq * N, dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, None)
        if lse.numel() != Hq * N:
            raise ValueError("lse must have Hq * cu[B] entries")
    _on_gpu(q=q, k=k, v=v, cu_seqlens=cu_seqlens, out=out, lse=lse)
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                              _ptr(lse), _ptr(cu_seqlens), B,
                              int(max_seqlen), Hq, Hkv, D, float(scale),
                              int(bool(causal)), _stream())
    if st != 0:
        raise AttnError(st, name)
    return out, lse


def attn_prefill_padded(q, k, v, seqlens, causal=True, scale=None, out=None,
                        lse=None, with_lse=True):
    """Prefill of a padded batch (bf16 or fp16): q [B,Hq,S,D], k, v
    [B,Hkv,S,D] as for ``attn_prefill``, with seqlens int32 [B] on the GPU
    giving the valid rows L_b of each sequence (clamped to [0, S]).  Rows
    i < L_b attend keys j < L_b only; padding rows get o = 0 and
    lse = -inf.  Returns (o, lse).
    """
    name = _fn("attn_prefill_padded", q.dtype)
    B, Hq, Hkv, S, D = _prefill_shapes(q, k, v, q.dtype)
    _check(seqlens, "seqlens", torch.int32, 1)
    _shape(seqlens, "seqlens", (B,))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.dtype, 4)
    _shape(out, "out", q.shape)
    lse = _lse_arg(lse, with_lse, (B, Hq, S), q)
    _on_gpu(q=q, k=k, v=v, seqlens=seqlens, out=out, lse=lse)
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                              _ptr(lse), _ptr(seqlens), B, Hq, Hkv, S, D,
                              float(scale), int(bool(causal)), _stream())
    if st != 0:
        raise AttnError(st, name)
    return out, lse


def attn_prefill_residual_rmsnorm(q, k, v, residual, weight, eps=1e-6,
                                  causal=True, scale=None, out=None,
                                  lse=None, with_lse=True):
    """Prefill with the fused residual add + RMSNorm epilogue (bf16 or fp16).

    q, residual [B,Hq,S,D]; k, v [B,Hkv,S,D]; weight [D]; all of q's dtype.
    For each head row: x = attention output + residual, out = x /
    sqrt(mean(x^2) + eps) * weight.  ``residual`` is overwritten with x.
    Returns (out, lse).
    """
    name = _fn("attn_prefill_residual_rmsnorm", q.dtype)
    B, Hq, Hkv, S, D = _prefill_shapes(q, k, v, q.dtype)
    _check(residual, "residual", q.dtype, 4)
    _shape(residual, "residual", q.shape)
    _check(weight, "weight", q.dtype, 1)
    _shape(weight, "weight", (D,))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.dtype, 4)
    _shape(out, "out", q.shape)
    lse = _lse_arg(lse, with_lse, (B, Hq, S), q)
    _on_gpu(q=q, k=k, v=v, residual=residual, weight=weight, out=out,
            lse=lse)
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(residual),
                              _ptr(weight), _ptr(out), _ptr(lse), B, Hq, Hkv,
                              S, D, float(scale), int(bool(causal)),
                              float(eps), _stream())
    if st != 0:
        raise AttnError(st, name)
    return out, lse


def attn_kv_append(k_new, v_new, kcache, vcache, seqlens, rope_base=0.0):
    """Append one token per sequence to a padded KV cache (in place).

    k_new, v_new [B,Hkv,D]; kcache, vcache [B,Hkv,cap,D], all bf16 (calls
    ``attn_kv_append``) or all fp16 (``attn_kv_append_f16``); seqlens int32
    [B] on the GPU, advanced by one for every sequence that is not full.
    ``rope_base`` > 0 stores k rotated to its position.  Launches on the
    current stream (graph-capturable).
    """
    dtype = k_new.dtype
    name = _fn("attn_kv_append", dtype)
    _check(k_new, "k_new", dtype, 3)
    _check(v_new, "v_new", dtype, 3)
    _check(kcache, "kcache", dtype, 4)
    _check(vcache, "vcache", dtype, 4)
    _check(seqlens, "seqlens", torch.int32, 1)
    B, Hkv, cap, D = kcache.shape
    _shape(k_new, "k_new", (B, Hkv, D))
    _shape(v_new, "v_new", (B, Hkv, D))
    _shape(vcache, "vcache", kcache.shape)
    _shape(seqlens, "seqlens", (B,))
    _on_gpu(k_new=k_new, v_new=v_new, kcache=kcache, vcache=vcache,
            seqlens=seqlens)
    st = getattr(lib(), name)(_ptr(k_new), _ptr(v_new), _ptr(kcache),
                              _ptr(vcache), _ptr(seqlens), B, Hkv, D, cap,
                              float(rope_base), _stream())
    if st != 0:
        raise AttnError(st, name)


def attn_decode_padded(q, kcache, vcache, seqlens, num_splits=0, scale=None,
                       out=None, with_lse=False, lse=None, workspace=None,
                       rope_base=0.0):
    """Decode attention over a padded cache [B,Hkv,cap,D] (bf16, or fp16
    through ``attn_decode_padded_f16``), with L_b = min(seqlens[b], cap);
    otherwise as ``attn_decode``.  ``rope_base`` > 0 rotates each query to
    its position L_b - 1 in the kernel."""
    name = _fn("attn_decode_padded", q.dtype)
    _check(q, "q", q.dtype, 3)
    _check(kcache, "kcache", q.dtype, 4)
    _check(vcache, "vcache", q.dtype, 4)
    _check(seqlens, "seqlens", torch.int32, 1)
    B, Hq, D = q.shape
    Hkv, cap = kcache.shape[1], kcache.shape[2]
    _shape(kcache, "kcache", (B, Hkv, cap, D))
    _shape(vcache, "vcache", kcache.shape)
    _shape(seqlens, "seqlens", (B,))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse, workspace = _decode_outputs(q, out, lse, with_lse, workspace,
                                          Hkv, num_splits)
    _on_gpu(q=q, kcache=kcache, vcache=vcache, seqlens=seqlens, out=out,
            lse=lse, workspace=workspace)
    st = getattr(lib(), name)(
        _ptr(q), _ptr(kcache), _ptr(vcache), _ptr(seqlens), _ptr(out), B, Hq,
        Hkv, D, cap, float(scale), int(num_splits), _ptr(lse),
        float(rope_base), _ptr(workspace), workspace.numel(), _stream())
    if st != 0:
        raise AttnError(st, name)
    return out, lse


class PreparedCall:
    """One C-ABI call with its arguments validated and converted once.

    Calling the object issues a single ctypes call: no checks, no
    allocation, no stream lookup.  It keeps its tensors alive; the caller
    must not resize or free them while the object is in use.  Meant for
    timing loops and serving loops where per-call Python work would
    otherwise outlast the kernels.
    """

    def __init__(self, fn, name, args, keep):
        self._fn, self._name, self._args, self._keep = fn, name, args, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise AttnError(st, self._name)


def prepare_prefill(q, k, v, out, lse=None, causal=True, scale=None):
    """A PreparedCall of attn_prefill / _f16 / _f32 on the current stream
    (arguments as for ``attn_prefill``; ``out`` is required)."""
    dtype = q.dtype
    if dtype not in _PREFILL_FN:
        raise ValueError("q must be bfloat16, float16 or float32")
    B, Hq, Hkv, S, D = _prefill_shapes(q, k, v, dtype)
    _check(out, "out", dtype, 4)
    _shape(out, "out", q.shape)
    lse = _lse_arg(lse, False, (B, Hq, S), q)
    _on_gpu(q=q, k=k, v=v, out=out, lse=lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ws = _prefill_workspace(q, B, Hq, Hkv, S, D, causal)
    if ws is not None:
        name = _PREFILL_WS_FN[dtype]
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv,
                S, D, ctypes.c_float(scale), int(bool(causal)), _ptr(ws),
                ws.numel(), _stream())
    else:
        name = _PREFILL_FN[dtype]
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv,
                S, D, ctypes.c_float(scale), int(bool(causal)), _stream())
    return PreparedCall(getattr(lib(), name), name, args,
                        (q, k, v, out, lse, ws))


def prepare_decode(q, kcache, vcache, seqlens, out, Hkv, workspace,
                   num_splits=0, lse=None, scale=None):
    """A PreparedCall of attn_decode / attn_decode_f16 on the current stream
    (arguments as for ``attn_decode``; ``out`` and ``workspace`` are
    required)."""
    dtype = q.dtype
    if dtype not in _DECODE_FN:
        raise ValueError("q must be bfloat16 or float16")
    _check(q, "q", dtype, 3)
    _check(kcache, "kcache", dtype, None)
    _check(vcache, "vcache", dtype, None)
    _check(seqlens, "seqlens", torch.int32, 1)
    B, Hq, D = q.shape
    _shape(seqlens, "seqlens", (B,))
    if kcache.numel() != vcache.numel():
        raise ValueError("kcache and vcache must have the same size")
    _check(out, "out", dtype, 3)
    _shape(out, "out", q.shape)
    _check(workspace, "workspace", torch.uint8, 1)
    lse = _lse_arg(lse, False, (B, Hq), q)
    _on_gpu(q=q, kcache=kcache, vcache=vcache, seqlens=seqlens, out=out,
            lse=lse, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    args = (_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(seqlens), _ptr(out), B,
            Hq, Hkv, D, ctypes.c_float(scale), int(num_splits), _ptr(lse),
            _ptr(workspace), workspace.numel(), _stream())
    return PreparedCall(getattr(lib(), _DECODE_FN[dtype]), _DECODE_FN[dtype],
                        args, (q, kcache, vcache, seqlens, out, workspace,
                               lse))


PREFILL_AUTO, PREFILL_W4, PREFILL_RB, PREFILL_KS = 0, 1, 2, 3
PREFILL_KERNEL_NAMES = {PREFILL_W4: "attn_prefill_kernel",
                        PREFILL_RB: "attn_prefill_rb_kernel",
                        PREFILL_KS: "attn_prefill_ks_kernel"}


def prefill_select(kernel):
    """Process-wide choice of the 16-bit prefill kernel (PREFILL_AUTO,
    PREFILL_W4, PREFILL_RB or PREFILL_KS); returns the previous one."""
    prev = int(lib().attn_prefill_select(int(kernel)))
    if prev < 0:
        raise ValueError(f"attn_prefill_select({kernel}): "
                         f"{status_string(prev)}")
    return prev


def prefill_kernel_for(B, Hq, S, D, causal=True):
    """PREFILL_W4, PREFILL_RB or PREFILL_KS: the kernel a dense 16-bit
    prefill launch of these sizes uses under the current setting."""
    return int(lib().attn_prefill_kernel_for(int(B), int(Hq), int(S), int(D),
                                             int(bool(causal))))


def prefill_balanced(B, Hq, Hkv, S, D, causal=True):
    """Whether a 16-bit ``attn_prefill`` of these sizes runs the balanced
    causal schedule (a workspace is passed and the schedule applies)."""
    return prefill_schedule(B, Hq, Hkv, S, D, causal) == SCHEDULE_BALANCED


def prefill_workgroups(B, Hq, Hkv, S, D, causal=True):
    """(kernel, workgroups, threads per workgroup) of one 16-bit prefill
    launch of these sizes through ``attn_prefill``."""
    if prefill_balanced(B, Hq, Hkv, S, D, causal):
        return PREFILL_RB, B * (Hq // 4) * -(-S // 64), 256
    kern = prefill_kernel_for(B, Hq, S, D, causal)
    if kern == PREFILL_KS:
        return kern, B * Hq * -(-S // 32), 256
    if kern == PREFILL_RB and (Hq // Hkv) % 4 == 0:
        return kern, B * (Hq // 4) * -(-S // 64), 256
    if kern == PREFILL_RB:
        return kern, B * Hq * -(-S // 128), 128
    return kern, B * Hq * -(-S // 128), 256
