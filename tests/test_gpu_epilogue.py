"""GPU parity of the fused residual-add + RMSNorm prefill epilogue.

attn_prefill_residual_rmsnorm (bf16) and its fp16 sibling, through the C
ABI, under each prefill kernel that carries the epilogue (4-wave,
register-blocked, key-split), against the fp64 oracle (oracle.prefill_residual_rmsnorm): the
"triton-optimization" page's fused RMSNorm with residual (section 3.2)
applied to each head row of the attention output, the extension named by
the attention-fusion page, section 6.3.

Tolerance, derived from the arithmetic: the attention row o carries the
prefill's error (at most 2e-2 for bf16, 5e-3 for fp16, unit-variance
inputs); x = o + residual adds it unchanged and is rounded once to the
storage type (half an ulp, 2^-9 |x| for bf16, 2^-12 |x| for fp16); the
normalisation divides by rms(x), which is about 1 here (residual ~ N(0, 1)),
and the weight (about 1) multiplies; y is rounded once more.  So both
outputs are held to |d| <= atol + rtol |ref| with atol the prefill bound and
rtol 2^-8 (bf16) or 2^-11 (fp16), and the LSE to 1e-3.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from causal_attention_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": (2e-2, 2.0 ** -8), "f16": (5e-3, 2.0 ** -11)}


def say(*a):
    print(*a, flush=True)


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(B, Hq, Hkv, S, D, dtype, causal, eps=1e-6, seed=0):
    say(f"[prefill+rmsnorm] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} {dtype} "
        f"causal={causal} eps={eps} seed={seed}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, dtype, 1.0, seed)
    res, w = inputs.residual_inputs(B, Hq, S, D, dtype, 1.0, seed)
    scale = 1.0 / math.sqrt(D)
    res_d = res.to(DEV)
    out, lse = attn.attn_prefill_residual_rmsnorm(
        q.to(DEV), k.to(DEV), v.to(DEV), res_d, w.to(DEV), eps=eps,
        causal=causal, scale=scale)
    torch.cuda.synchronize()
    ry, rx, rl = oracle.prefill_residual_rmsnorm(
        np64(q), np64(k), np64(v), np64(res), np64(w), scale, causal, eps)
    atol, rtol = TOL[dtype]
    gy, gx = np64(out), np64(res_d)
    ey = np.abs(gy - ry) / (atol + rtol * np.abs(ry))
    ex = np.abs(gx - rx) / (atol + rtol * np.abs(rx))
    el = np.abs(lse.cpu().numpy() - rl)
    say(f"   max|dy|={np.abs(gy - ry).max():.3e} "
        f"max|dx|={np.abs(gx - rx).max():.3e} "
        f"worst/bound y {ey.max():.3f} x {ex.max():.3f} "
        f"max|dLSE|={el.max():.3e}")
    assert np.isfinite(gy).all() and np.isfinite(gx).all()
    assert ey.max() <= 1.0
    assert ex.max() <= 1.0
    assert el.max() <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [1, 63, 200, 513])
@pytest.mark.usefixtures("prefill_kernel")
def test_residual_rmsnorm_shapes(dtype, D, causal, S):
    check(2, 8, 2, S, D, dtype, causal, seed=S)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 8)])
def test_residual_rmsnorm_long_rows_sampled(Hq, Hkv):
    """A launch large enough for the register-blocked kernel under the
    automatic choice (four query heads per workgroup with 8/2 heads, one
    with 8/8), checked on 64 seeded rows per head: the oracle's attention
    rows followed by its epilogue on those rows."""
    from causal_attention_amd import attn as A
    B, S, D = 1, 16384, 128
    assert A.prefill_kernel_for(B, Hq, S, D) == A.PREFILL_RB
    say(f"[prefill+rmsnorm sampled] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, "bf16", 1.0, 9)
    res, w = inputs.residual_inputs(B, Hq, S, D, "bf16", 1.0, 9)
    res_d = res.to(DEV)
    out, lse = attn.attn_prefill_residual_rmsnorm(
        q.to(DEV), k.to(DEV), v.to(DEV), res_d, w.to(DEV))
    torch.cuda.synchronize()
    rows = inputs.sampled_rows(Hq, S, 64)
    ro, rl = oracle.prefill_rows(np64(q), np64(k), np64(v),
                                 1 / math.sqrt(D), True, rows)
    rr = np.stack([np64(res[:, h, rows[h]]) for h in range(Hq)], axis=1)
    ry, rx = oracle.residual_rmsnorm(ro, rr, np64(w), 1e-6)
    gy = np.stack([np64(out[:, h, rows[h]]) for h in range(Hq)], axis=1)
    gx = np.stack([np64(res_d[:, h, rows[h]]) for h in range(Hq)], axis=1)
    gl = np.stack([lse[:, h, rows[h]].cpu().numpy() for h in range(Hq)],
                  axis=1)
    atol, rtol = TOL["bf16"]
    ey = (np.abs(gy - ry) / (atol + rtol * np.abs(ry))).max()
    ex = (np.abs(gx - rx) / (atol + rtol * np.abs(rx))).max()
    el = np.abs(gl - rl).max()
    say(f"   worst/bound y {ey:.3f} x {ex:.3f} max|dLSE|={el:.3e}")
    assert ey <= 1.0 and ex <= 1.0 and el <= 1e-3


def test_residual_rmsnorm_c2_shape():
    check(1, 12, 12, 512, 64, "bf16", True)


def test_residual_rmsnorm_c3_shape():
    check(4, 8, 2, 2048, 128, "bf16", True)


@pytest.mark.parametrize("eps", [0.0, 0.5])
def test_residual_rmsnorm_eps(eps):
    check(1, 4, 1, 130, 128, "bf16", True, eps=eps, seed=7)


@pytest.mark.usefixtures("prefill_kernel")
def test_residual_rmsnorm_attention_part_equals_plain_prefill():
    """With a zero residual and unit weight, out is RMSNorm(o) for the
    attention row o; under each kernel, LSE is the plain prefill's (the same
    kernel, no workspace) bit for bit, and the residual buffer receives o
    itself, rounded the same way."""
    B, Hq, Hkv, S, D = 1, 8, 2, 300, 128
    q, k, v = [t.to(DEV) for t in inputs.prefill_inputs(B, Hq, Hkv, S, D,
                                                         "bf16", 1.0, 3)]
    prev_ws = attn.prefill_workspace_policy(False)
    try:
        o, lse = attn.attn_prefill(q, k, v, causal=True)
    finally:
        attn.prefill_workspace_policy(prev_ws)
    res = torch.zeros_like(q)
    w = torch.ones(D, dtype=torch.bfloat16, device=DEV)
    y, lse2 = attn.attn_prefill_residual_rmsnorm(q, k, v, res, w, eps=0.0)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse2)
    assert torch.equal(res, o)         # x = o + 0, rounded the same way
    ms = (np64(res) ** 2).mean(-1)
    np.testing.assert_allclose(ms, (np64(o) ** 2).mean(-1), rtol=1e-6)
    # y has unit mean square up to its own rounding
    np.testing.assert_allclose((np64(y) ** 2).mean(-1), 1.0, atol=1e-2)


def test_residual_rmsnorm_is_repeatable():
    B, Hq, Hkv, S, D = 2, 8, 2, 256, 64
    q, k, v = [t.to(DEV) for t in inputs.prefill_inputs(B, Hq, Hkv, S, D,
                                                         "bf16", 1.0, 4)]
    res0, w = [t.to(DEV) for t in inputs.residual_inputs(B, Hq, S, D, "bf16",
                                                         1.0, 4)]
    outs = []
    for _ in range(3):
        r = res0.clone()
        y, l = attn.attn_prefill_residual_rmsnorm(q, k, v, r, w)
        outs.append((y, r, l))
    torch.cuda.synchronize()
    for y, r, l in outs[1:]:
        assert torch.equal(y, outs[0][0])
        assert torch.equal(r, outs[0][1])
        assert torch.equal(l, outs[0][2])
