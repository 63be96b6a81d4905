"""fp64 reference of the residual-add + RMSNorm epilogue on the attention output.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
HIP path.

What it computes.  The "triton-optimization" skill page, section 3.2 (fused
RMSNorm, and its fused extension with a residual add), normalises one row x
of n values as y = x * r * w with r = 1 / sqrt(mean(x^2) + eps) and a
per-column weight w; in the fused form the row is first added to a residual,
x = row + residual, and x is also written back into the residual buffer for
the next layer.  "第 6 讲：核函数与 Triton" section 9.1 states the same
forward (y = x * r * g, computed in fp32, one row per program), and
"让编码智能体写 Triton 算子" fixes eps = 1e-6 as the usual default.
"Attention三算子融合实战" section 6.3 names a residual add and a norm fused into
the attention kernel as the next extension; the pages fix no row for it.

Readings taken here (where the pages leave a step open):
* The row is one query row of one head: the D values o[b, h, i, :].  That is
  the row a workgroup of the attention kernel holds whole; a norm over all
  heads of a token would need the other heads' rows.
* The attention output enters the sum before it is rounded to the storage
  type (the fused kernel never stores it); the residual and the weight enter
  as their stored values, upcast exactly.
* The residual written back is x itself (the caller's storage type rounds it).
"""

import numpy as np

from .attention import prefill


def residual_rmsnorm(o, residual, weight, eps):
    """x = o + residual; y = x / sqrt(mean(x^2 over the last axis) + eps) * w.

    o and residual have the same shape [..., D]; weight has shape [D].
    Returns (y, x) in float64.
    """
    o = np.asarray(o, dtype=np.float64)
    residual = np.asarray(residual, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.float64)
    if o.shape != residual.shape or weight.shape != o.shape[-1:]:
        raise ValueError("o, residual [..., D] and weight [D] must match")
    x = o + residual
    ms = np.mean(x * x, axis=-1, keepdims=True)     # mean of squares per row
    r = 1.0 / np.sqrt(ms + eps)
    return x * r * weight, x


def prefill_residual_rmsnorm(q, k, v, residual, weight, scale, causal, eps):
    """Prefill attention followed by the residual add and RMSNorm per row.

    q, residual [B,Hq,S,D]; k, v [B,Hkv,S,D]; weight [D].  Returns
    (y [B,Hq,S,D], x [B,Hq,S,D], lse [B,Hq,S]): y the normalised output, x
    the new residual, lse the attention's log-sum-exp (unchanged by the
    epilogue).
    """
    o, lse = prefill(q, k, v, scale, causal)
    y, x = residual_rmsnorm(o, residual, weight, eps)
    return y, x, lse
