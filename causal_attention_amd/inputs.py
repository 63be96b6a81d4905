"""Seeded synthetic inputs for the attention workloads.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic, so both the HIP path's tests and the fp64 oracle can
consume the same bytes.  Every workload draws from
``numpy.random.default_rng(seed)`` in a fixed order (decode: sequence lengths
first, then q, k, v; prefill: q, k, v), standard normal scaled by ``sigma``,
then rounds to the storage dtype (bf16 or fp16 with round-to-nearest-even via
torch).

Shapes follow the pages' setups: the single-head and 12-head MHA prefill runs
of "Attention三算子融合实战：从Triton到CUDA的推理加速优化" (section 5.1: batch
1, 12 heads, head_dim 64, sequence 128 to 2048) and the GQA decoder layer of
"手写Triton kernel重构Qwen3.5-0.8B" (section 2.1: 8 query heads sharing 2 KV
heads, head_dim 128, context up to 32768).
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str           # "f32", "bf16" or "f16"
    sigma: float
    seed: int = 0
    S: int = 0           # prefill sequence length
    causal: bool = True
    lmin: int = 0        # decode: per-sequence cache length ~ U[lmin, lmax]
    lmax: int = 0
    sampled_rows: int = 0  # >0: parity on this many seeded rows per head
    notes: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self):
        return _STORAGE[self.dtype]


WORKLOADS = {
    "c1_f32_s128": Workload("c1_f32_s128", "prefill", B=1, Hq=1, Hkv=1, D=64,
                            dtype="f32", sigma=1.0, S=128),
    "c2_mha12_s512": Workload("c2_mha12_s512", "prefill", B=1, Hq=12, Hkv=12,
                              D=64, dtype="bf16", sigma=1.0, S=512),
    "c3_gqa_b4_s2048": Workload("c3_gqa_b4_s2048", "prefill", B=4, Hq=8,
                                Hkv=2, D=128, dtype="bf16", sigma=1.0, S=2048),
    "c4_decode_b32": Workload("c4_decode_b32", "decode", B=32, Hq=8, Hkv=2,
                              D=128, dtype="bf16", sigma=1.0, lmin=256,
                              lmax=4096),
    "c5_gqa_s32768": Workload("c5_gqa_s32768", "prefill", B=1, Hq=8, Hkv=2,
                              D=128, dtype="bf16", sigma=0.5, S=32768,
                              sampled_rows=256),
}


_STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t if dtype == "f32" else t.to(_STORAGE[dtype])


def prefill_inputs(B, Hq, Hkv, S, D, dtype="bf16", sigma=1.0, seed=0):
    """q [B,Hq,S,D], k and v [B,Hkv,S,D] as CPU torch tensors of ``dtype``."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D), dtype=np.float32) * np.float32(sigma)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32) * np.float32(sigma)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32) * np.float32(sigma)
    return _round(q, dtype), _round(k, dtype), _round(v, dtype)


def residual_inputs(B, Hq, S, D, dtype="bf16", sigma=1.0, seed=0):
    """The residual-add + RMSNorm epilogue's extra inputs: a residual
    [B,Hq,S,D] ~ N(0, sigma^2) and a weight [D] = 1 + N(0, 0.25^2), drawn
    from ``default_rng([2, seed])`` (apart from the q, k, v stream)."""
    rng = np.random.default_rng([2, seed])
    r = rng.standard_normal((B, Hq, S, D), dtype=np.float32) * np.float32(sigma)
    w = 1.0 + 0.25 * rng.standard_normal(D, dtype=np.float32)
    return _round(r, dtype), _round(w, dtype)


def decode_seqlens(B, lmin, lmax, seed=0):
    """Per-sequence cache lengths, uniform on [lmin, lmax] inclusive."""
    rng = np.random.default_rng(seed)
    return rng.integers(lmin, lmax + 1, size=B).astype(np.int32)


def decode_inputs(B, Hq, Hkv, D, seqlens=None, lmin=256, lmax=4096,
                  dtype="bf16", sigma=1.0, seed=0):
    """One query row per sequence plus a packed KV cache.

    Returns (seqlens int32 [B], q [B,Hq,D], kcache, vcache) where each cache is
    a flat tensor holding, for sequence b in order, a [Hkv, L_b, D] block.
    With ``seqlens`` given, the lengths are not drawn.
    """
    rng = np.random.default_rng(seed)
    if seqlens is None:
        seqlens = rng.integers(lmin, lmax + 1, size=B)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    n = Hkv * D * int(seqlens.astype(np.int64).sum())
    q = rng.standard_normal((B, Hq, D), dtype=np.float32) * np.float32(sigma)
    k = rng.standard_normal((n,), dtype=np.float32) * np.float32(sigma)
    v = rng.standard_normal((n,), dtype=np.float32) * np.float32(sigma)
    return seqlens, _round(q, dtype), _round(k, dtype), _round(v, dtype)


def workload_inputs(w: Workload):
    if w.kind == "prefill":
        return prefill_inputs(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype, w.sigma,
                              w.seed)
    return decode_inputs(w.B, w.Hq, w.Hkv, w.D, lmin=w.lmin, lmax=w.lmax,
                         dtype=w.dtype, sigma=w.sigma, seed=w.seed)


def sampled_rows(Hq, S, n=256):
    """Seeded query rows per head: {0, 127, 128, S-1} plus draws without
    replacement from the rest, from ``default_rng([1, h])`` for head h.
    Returns int64 [Hq, n], each row sorted."""
    forced = sorted({0, min(127, S - 1), min(128, S - 1), S - 1})
    out = np.zeros((Hq, n), dtype=np.int64)
    for h in range(Hq):
        rng = np.random.default_rng([1, h])
        rest = np.setdiff1d(np.arange(S), forced)
        pick = rng.choice(rest, size=n - len(forced), replace=False)
        out[h] = np.sort(np.concatenate([forced, pick]))
    return out


def pack_kv(blocks):
    """Concatenate per-sequence [Hkv, L_b, D] blocks into one flat cache."""
    return torch.cat([b.reshape(-1) for b in blocks]) if blocks else None


def unpack_kv(flat, seqlens, Hkv, D):
    """Split a flat cache back into per-sequence [Hkv, L_b, D] views."""
    out, off = [], 0
    for L in np.asarray(seqlens, dtype=np.int64):
        n = Hkv * int(L) * D
        out.append(flat[off:off + n].reshape(Hkv, int(L), D))
        off += n
    return out
