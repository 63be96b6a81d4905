"""Plain fp64 CPU oracle for fused causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (``causal_attention_amd/``) and imports nothing from it.

What it computes is the plain definition that the fused method reaches up to
rounding order: materialise the score matrix, run a two-pass softmax, multiply
by V, and report the natural-log log-sum-exp of each score row.  Sources, cited
by page title and section:

* "Attention三算子融合实战：从Triton到CUDA的推理加速优化" (xdnf.cn/news/349386):
  section 1.1 (the chain S = Q K^T scaled, P = row softmax of S, O = P V),
  section 4.3 (causal mask: query i sees key j only when j <= i; masked scores
  become -inf; length mask from a valid-key count), section 1.3 (decode: one
  query row against a key/value history that grows).
* "手写Triton kernel重构Qwen3.5-0.8B：21算子全流程优化与CUDA Graph实践"
  (m.nlpx.cn/news/28229): section 2.1 (GQA, two KV heads broadcast to eight
  query heads), section 2.2 op table rows qk_score / causal_mask_softmax /
  pv_matmul.
* "第 6 讲：核函数与 Triton" (CS336 lecture 6 notes), section 6: softmax as
  subtract the row max, exponentiate, sum, divide; masked entries are -inf.
* "triton-optimization" skill page, section 3.5 (fused cross entropy): the
  log-sum-exp of a row is m + log(d) with m the row max and d the sum of
  exp(x - m), natural logarithm.
* "让编码智能体写 Triton 算子" (zmj.net/articles/3605), step 1: the reference is
  computed in float32 or float64, never in half precision.

``residual_rmsnorm`` and ``prefill_residual_rmsnorm`` (``oracle/epilogue.py``)
add a residual to the attention output and RMS-normalise each head row, the
fused epilogue of the "triton-optimization" skill page, section 3.2.

``rope`` (``oracle/rotary.py``) rotates q and k before attention, following the
"triton-optimization" skill page, section 3.4 (fused RoPE: rotate pairs
(x[i], x[i + D/2]) by position-dependent angles).

Pinned by ``tests/test_oracle.py``, ``tests/test_oracle_rope.py`` and
``tests/test_oracle_epilogue.py`` (closed
forms, brute force on tiny inputs, an fp64 library implementation, algebraic
invariants, planted mistakes).  No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    prefill,
    prefill_rows,
    prefill_varlen,
    prefill_padded,
    decode,
    lse_combine,
    softmax_probabilities,
    prefix_softmax_state,
)
from .rotary import rope  # noqa: F401
from .epilogue import residual_rmsnorm, prefill_residual_rmsnorm  # noqa: F401
