"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Tolerances: max abs error on O of 1e-5 for fp32 storage and 2e-2 for bf16
storage (fp32 accumulation inside the kernels), and 1e-3 on the natural-log
LSE.  Inputs are seeded synthetic tensors; the oracle sees exactly the stored
(bf16-rounded) values.

fp16 storage (the mixed-precision rule of the attention-fusion page, section
5.5: fp16 only in storage and MFMA inputs, fp32 accumulation and state) has no
bound in the pages; it is derived from the arithmetic like the sigma sweep:
P is rounded to fp16 before the PV product and O once more on output, each a
relative error of at most 2^-11 on values bounded by max|v| (about 4.5 for
unit-variance inputs at these sizes), so 2 * 4.5 * 2^-11 = 4.4e-3; the test
uses 5e-3 per unit sigma.

The 1e-5 / 2e-2 bounds are for unit-variance inputs.  For the input-scale
sweep (sigma != 1) the bound is derived from the arithmetic, see ``o_tol``:
with bf16 (fp16) storage the error is the relative rounding of P and O, so it
scales with the value magnitude sigma, above and below 1; with fp32 storage
and sigma >= 1 it is the fp32 accumulation error of the scores, which grows
with |q||k| ~ sigma^2 sqrt(D) and moves O in proportion to |v| ~ sigma, so it
scales with sigma^3, and for sigma < 1 the floor is the fp32 rounding of O, a
few ulp of |o| <= 4.5 sigma, so 1e-6 sigma.  Measured max |dO| (both prefill
kernels; sigma 0.01 / 1 / 4): bf16 5.8e-5 / 7.8e-3 / 6.3-7.0e-2 against
2e-4 / 2e-2 / 8e-2; fp32 2.2e-9 / 1.1e-6 / 1.0e-4 against 1e-8 / 1e-5 /
6.4e-4; fp16 8.0e-6 / - / 8.6-9.7e-3 against 5e-5 / 5e-3 / 2e-2; decode bf16
8.0e-6 / 1.1e-3 / 3.1e-2.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from causal_attention_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LSE_TOL = 1e-3


def o_tol(dtype, sigma=1.0):
    if dtype == "f32":
        return 1e-5 * sigma ** 3 if sigma >= 1.0 else 1e-6 * sigma
    return {"bf16": 2e-2, "f16": 5e-3}[dtype] * sigma


def say(*a):
    print(*a, flush=True)


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_prefill(B, Hq, Hkv, S, D, dtype, causal, sigma=1.0, seed=0,
                scale=None):
    say(f"[prefill] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} {dtype} "
        f"causal={causal} sigma={sigma} seed={seed}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, dtype, sigma, seed)
    scale = 1 / math.sqrt(D) if scale is None else scale
    o, lse = attn.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV),
                               causal=causal, scale=scale)
    torch.cuda.synchronize()
    return q, k, v, o, lse, scale


def check_prefill(B, Hq, Hkv, S, D, dtype, causal, sigma=1.0, seed=0):
    q, k, v, o, lse, scale = run_prefill(B, Hq, Hkv, S, D, dtype, causal,
                                         sigma, seed)
    ro, rl = oracle.prefill(np64(q), np64(k), np64(v), scale, causal)
    eo = np.abs(np64(o) - ro)
    el = np.abs(lse.cpu().numpy() - rl)
    worst = np.unravel_index(np.argmax(eo), eo.shape) if eo.size else None
    say(f"   max|dO|={eo.max() if eo.size else 0:.3e} "
        f"mean|dO|={eo.mean() if eo.size else 0:.3e} at {worst} "
        f"max|dLSE|={el.max() if el.size else 0:.3e}")
    assert np.isfinite(np64(o)).all()
    if eo.size:
        assert eo.max() <= o_tol(dtype, sigma)
        assert el.max() <= LSE_TOL


# ------------------------------------------------------------ the workloads

@pytest.mark.usefixtures("prefill_kernel")
def test_c1_single_head_fp32():
    # fp32: the fp32 kernel under w4 / rb / balanced, its key-split sibling
    # under ks
    w = inputs.WORKLOADS["c1_f32_s128"]
    check_prefill(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype, w.causal, w.sigma)


def test_c2_mha12_s512():
    w = inputs.WORKLOADS["c2_mha12_s512"]
    check_prefill(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype, w.causal, w.sigma)


@pytest.mark.usefixtures("prefill_kernel")
def test_c3_gqa_b4_s2048():
    w = inputs.WORKLOADS["c3_gqa_b4_s2048"]
    check_prefill(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype, w.causal, w.sigma)


@pytest.mark.usefixtures("prefill_kernel")
def test_c5_long_context_sampled_rows():
    w = inputs.WORKLOADS["c5_gqa_s32768"]
    q, k, v, o, lse, scale = run_prefill(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype,
                                         w.causal, w.sigma)
    rows = inputs.sampled_rows(w.Hq, w.S, w.sampled_rows)
    ro, rl = oracle.prefill_rows(np64(q), np64(k), np64(v), scale, True, rows)
    o_c, l_c = o.cpu(), lse.cpu()
    go = np.stack([np64(o_c[:, h, rows[h]]) for h in range(w.Hq)], axis=1)
    gl = np.stack([l_c[:, h, rows[h]].numpy() for h in range(w.Hq)], axis=1)
    eo, el = np.abs(go - ro).max(), np.abs(gl - rl).max()
    say(f"   sampled rows: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= 2e-2 and el <= LSE_TOL
    # every row, checked by properties that hold at any size: finite, and
    # |o| bounded by the largest |v| of its KV head (o is a convex
    # combination of value rows)
    vmax = v.float().abs().amax(dim=(2, 3))           # [B, Hkv]
    omax = o.float().abs().amax(dim=(2, 3)).cpu()     # [B, Hq]
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    G = w.Hq // w.Hkv
    for h in range(w.Hq):
        assert omax[0, h] <= vmax[0, h // G] * (1 + 2 ** -8)


def _randn_bf16(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.bfloat16)


@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_offsets_beyond_4gb_sampled():
    """Tensors past 2^31 elements (q, o: 4.4 GB): the last (batch, head)
    pairs, whose rows start beyond element 2^31, are checked row by row
    against the oracle; every row is finite."""
    B, Hq, Hkv, S, D = 64, 32, 8, 8320, 128
    say(f"[prefill > 4 GB] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}")
    q = _randn_bf16((B, Hq, S, D), 31)
    k = _randn_bf16((B, Hkv, S, D), 32)
    v = _randn_bf16((B, Hkv, S, D), 33)
    assert q.numel() > 2 ** 31
    o, lse = attn.attn_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    rows = np.array([0, 1, 4095, 4096, S - 2, S - 1])
    scale = 1 / math.sqrt(D)
    for b, h in ((B - 1, Hq - 1), (B - 1, 0), (B // 2, Hq // 2)):
        g = h // (Hq // Hkv)
        qs = np64(q[b:b + 1, h:h + 1, rows])
        ro, rl = oracle.prefill_rows(
            np64(q[b:b + 1, h:h + 1]), np64(k[b:b + 1, g:g + 1]),
            np64(v[b:b + 1, g:g + 1]), scale, True, rows[None])
        eo = np.abs(np64(o[b:b + 1, h:h + 1, rows]) - ro).max()
        el = np.abs(lse[b:b + 1, h:h + 1, rows].cpu().numpy() - rl).max()
        say(f"   (b={b}, h={h}) rows {rows.tolist()}: max|dO|={eo:.3e} "
            f"max|dLSE|={el:.3e}")
        assert qs.shape[2] == len(rows)
        assert eo <= o_tol("bf16") and el <= LSE_TOL
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_decode_cache_beyond_4gb_sampled():
    """A packed cache past 2^31 elements per tensor (256 sequences x 8 KV
    heads x 8256 keys): the last sequences, at the highest offsets, against
    the oracle."""
    B, Hq, Hkv, D, L = 256, 32, 8, 128, 8256
    say(f"[decode > 4 GB] B={B} Hq={Hq} Hkv={Hkv} L={L} D={D}")
    kc = _randn_bf16((B * Hkv * L * D,), 41)
    vc = _randn_bf16((B * Hkv * L * D,), 42)
    assert kc.numel() > 2 ** 31
    q = _randn_bf16((B, Hq, D), 43)
    sl = torch.full((B,), L, dtype=torch.int32, device=DEV)
    o, lse = attn.attn_decode(q, kc, vc, sl, Hkv, with_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    per = Hkv * L * D
    for b in (B - 1, B - 2, 0):
        seg = slice(b * per, (b + 1) * per)
        ro, rl = oracle.decode(np64(q[b:b + 1]), np64(kc[seg]),
                               np64(vc[seg]), np.array([L]), 1 / math.sqrt(D),
                               Hkv)
        eo = np.abs(np64(o[b:b + 1]) - ro).max()
        el = np.abs(lse[b:b + 1].cpu().numpy() - rl).max()
        say(f"   sequence {b}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= 2e-2 and el <= LSE_TOL
    del kc, vc
    torch.cuda.empty_cache()


# ------------------------------------------------------- edge shapes, masks

@pytest.mark.parametrize("S", [1, 2, 7, 63, 64, 65, 127, 129, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (12, 12), (8, 2), (8, 1)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_edge_shapes_bf16(S, D, Hq, Hkv, causal):
    check_prefill(2 if S < 200 else 1, Hq, Hkv, S, D, "bf16", causal,
                  seed=S + D)


@pytest.mark.parametrize("S", [1, 33, 128, 129, 300])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_edge_shapes_f32(S, D, causal):
    check_prefill(1, 4, 2, S, D, "f32", causal, seed=S)


@pytest.mark.parametrize("sigma", [0.01, 1.0, 4.0])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_value_scale_sweep(sigma, dtype):
    check_prefill(1, 8, 2, 257, 128, dtype, True, sigma=sigma, seed=7)


@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_is_deterministic():
    w = inputs.WORKLOADS["c3_gqa_b4_s2048"]
    q, k, v = (t.to(DEV) for t in
               inputs.prefill_inputs(1, 8, 2, 1031, 128, "bf16", 1.0, 3))
    o1, l1 = attn.attn_prefill(q, k, v)
    o2, l2 = attn.attn_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_without_lse():
    q, k, v = (t.to(DEV) for t in
               inputs.prefill_inputs(1, 8, 2, 100, 128, "bf16", 1.0, 4))
    o1, _ = attn.attn_prefill(q, k, v)
    o2, l2 = attn.attn_prefill(q, k, v, with_lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1, o2)


# -------------------------------------------------------------------- decode

def run_decode(seqlens, Hq, Hkv, D, num_splits=0, sigma=1.0, seed=0,
               dtype="bf16"):
    say(f"[decode] B={len(seqlens)} Hq={Hq} Hkv={Hkv} D={D} {dtype} "
        f"ns={num_splits} sum(L)={int(np.sum(seqlens))} seed={seed}")
    sl, q, kc, vc = inputs.decode_inputs(len(seqlens), Hq, Hkv, D,
                                         seqlens=seqlens, sigma=sigma,
                                         seed=seed, dtype=dtype)
    o, lse = attn.attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV),
                              torch.from_numpy(sl).to(DEV), Hkv=Hkv,
                              num_splits=num_splits, with_lse=True)
    torch.cuda.synchronize()
    return sl, q, kc, vc, o, lse


def check_decode(seqlens, Hq, Hkv, D, num_splits=0, sigma=1.0, seed=0,
                 dtype="bf16"):
    sl, q, kc, vc, o, lse = run_decode(seqlens, Hq, Hkv, D, num_splits,
                                       sigma, seed, dtype)
    ro, rl = oracle.decode(np64(q), np64(kc), np64(vc), sl, 1 / math.sqrt(D),
                           Hkv)
    go, gl = np64(o), lse.cpu().numpy()
    empty = np.asarray(sl) <= 0
    assert (go[empty] == 0).all() and np.isneginf(gl[empty]).all()
    live = ~empty
    if live.any():
        eo = np.abs(go[live] - ro[live]).max()
        el = np.abs(gl[live] - rl[live]).max()
        say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= o_tol(dtype, sigma) and el <= LSE_TOL
    return o, lse


def test_c4_decode_b32():
    w = inputs.WORKLOADS["c4_decode_b32"]
    sl = inputs.decode_seqlens(w.B, w.lmin, w.lmax, w.seed)
    check_decode(sl, w.Hq, w.Hkv, w.D, num_splits=0, sigma=w.sigma,
                 seed=w.seed)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 16, 0])
def test_decode_lengths_and_splits(num_splits):
    check_decode([1, 15, 16, 17, 255, 4096, 64, 65, 129], 8, 2, 128,
                 num_splits=num_splits, seed=11)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (8, 8), (8, 2), (8, 1), (4, 2)])
def test_decode_heads_and_dims(D, Hq, Hkv):
    check_decode([5, 700, 2000], Hq, Hkv, D, seed=D + Hq)


def test_decode_empty_sequences():
    check_decode([0, 10, 0, 300], 8, 2, 128, seed=5)


@pytest.mark.parametrize("num_splits", [0, 37, 1000])
def test_decode_many_sequences(num_splits):
    # more than 64 sequences: the per-sequence lengths are scanned in chunks
    # of 64, with empty sequences and a segment crossing chunk ends
    rng = np.random.default_rng(3)
    lens = rng.integers(0, 400, size=150)
    lens[[0, 63, 64, 65, 149]] = [0, 0, 2000, 0, 33]
    check_decode(lens.tolist(), 8, 2, 128, num_splits=num_splits, seed=17)


@pytest.mark.parametrize("num_splits", [512, attn.MAX_SPLITS])
def test_decode_more_ranges_than_blocks(num_splits):
    # 35 blocks per KV head, 70 in all: most ranges are empty, some of them
    # between two pieces of one sequence
    check_decode([40, 1000, 3], 8, 2, 128, num_splits=num_splits, seed=19)


def test_decode_workspace_contents_do_not_matter():
    sl, q, kc, vc = inputs.decode_inputs(3, 8, 2, 128, seqlens=[900, 0, 77],
                                         seed=23)
    args = (q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(sl).to(DEV))
    ws = attn.new_decode_workspace(3, 8, 2, 128, 64, DEV)
    ws.fill_(0xFF)          # every float in it reads as NaN
    o, lse = attn.attn_decode(*args, Hkv=2, num_splits=64, with_lse=True,
                              workspace=ws)
    o2, l2 = attn.attn_decode(*args, Hkv=2, num_splits=64, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("sigma", [0.01, 4.0])
def test_decode_value_scale(sigma):
    check_decode([100, 1500], 8, 2, 128, sigma=sigma, seed=9)


def test_decode_split_count_changes_only_rounding():
    ref = None
    for ns in [1, 4, 64, 256]:
        o, lse = run_decode([3000, 200], 8, 2, 128, num_splits=ns, seed=2)[4:]
        if ref is None:
            ref = (o.float(), lse)
        else:
            assert (o.float() - ref[0]).abs().max() <= 2e-2
            assert (lse - ref[1]).abs().max() <= 1e-4


@pytest.mark.usefixtures("prefill_kernel")
def test_decode_equals_last_prefill_row():
    Hq, Hkv, D, L = 8, 2, 128, 333
    q, k, v = inputs.prefill_inputs(1, Hq, Hkv, L, D, "bf16", 1.0, 21)
    po, pl = attn.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    qd = q[:, :, L - 1].contiguous()
    kc, vc = k[0].reshape(-1), v[0].reshape(-1)
    o, lse = attn.attn_decode(qd.to(DEV), kc.to(DEV), vc.to(DEV),
                              torch.tensor([L], dtype=torch.int32,
                                           device=DEV),
                              Hkv=Hkv, with_lse=True)
    torch.cuda.synchronize()
    assert (o.float() - po[:, :, L - 1].float()).abs().max() <= 2e-2
    assert (lse - pl[:, :, L - 1]).abs().max() <= 1e-4


def test_decode_workspace_reused_across_calls():
    # one workspace serves many calls with different lengths
    ws = attn.new_decode_workspace(4, 8, 2, 128, 7, DEV)
    for seed, lens in enumerate([[100, 3000, 1, 640], [5, 5, 5, 5],
                                 [4096, 0, 129, 2048]]):
        sl, q, kc, vc = inputs.decode_inputs(4, 8, 2, 128, seqlens=lens,
                                             seed=seed)
        o, lse = attn.attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV),
                                  torch.from_numpy(sl).to(DEV), Hkv=2,
                                  num_splits=7, with_lse=True, workspace=ws)
        ro, rl = oracle.decode(np64(q), np64(kc), np64(vc), sl,
                               1 / math.sqrt(128), 2)
        live = np.asarray(sl) > 0
        assert np.abs(np64(o)[live] - ro[live]).max() <= 2e-2
        assert np.abs(lse.cpu().numpy()[live] - rl[live]).max() <= LSE_TOL
    torch.cuda.synchronize()


def test_decode_is_deterministic():
    sl, q, kc, vc = inputs.decode_inputs(8, 8, 2, 128, lmin=1, lmax=3000,
                                         seed=4)
    args = (q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(sl).to(DEV))
    o1, l1 = attn.attn_decode(*args, Hkv=2, with_lse=True)
    o2, l2 = attn.attn_decode(*args, Hkv=2, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- fp16 path

@pytest.mark.parametrize("S", [1, 65, 129, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (8, 2)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_edge_shapes_f16(S, D, Hq, Hkv, causal):
    check_prefill(1, Hq, Hkv, S, D, "f16", causal)


@pytest.mark.usefixtures("prefill_kernel")
def test_c3_shape_f16():
    check_prefill(4, 8, 2, 2048, 128, "f16", True)


@pytest.mark.parametrize("sigma", [0.01, 4.0])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_value_scale_f16(sigma):
    check_prefill(1, 8, 2, 300, 128, "f16", True, sigma=sigma)


@pytest.mark.parametrize("num_splits", [1, 7, 0])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_f16(num_splits, D):
    check_decode([1, 15, 17, 255, 4096, 64, 0, 129], 8, 2, D, num_splits,
                 dtype="f16")


def test_c4_decode_f16():
    w = inputs.WORKLOADS["c4_decode_b32"]
    sl = inputs.decode_seqlens(w.B, w.lmin, w.lmax, w.seed)
    check_decode(sl, w.Hq, w.Hkv, w.D, dtype="f16")


# --------------------------------------- padded cache, append, graph replay

def bf16_stored(x):
    """x rounded to bf16 (RNE, straight from fp64), as float64: the value a
    bf16 tensor or a bf16 MFMA operand holds.  With RoPE the rotated q and k
    are such operands (and the cache stores rotated keys in bf16), so the
    expected values round the oracle's fp64 rotation at that point."""
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(
        torch.bfloat16).double().numpy()


def padded_to_packed(kc, sl):
    """[B,Hkv,cap,D] padded cache with lengths sl -> the packed layout."""
    return np.concatenate([kc[b, :, :max(int(L), 0)].reshape(-1)
                           for b, L in enumerate(sl)])


def test_kv_append_writes_rows_and_advances_lengths():
    B, Hkv, cap, D = 3, 2, 8, 128
    say(f"[append] B={B} Hkv={Hkv} cap={cap} D={D}")
    g = torch.Generator().manual_seed(5)
    kc = torch.randn(B, Hkv, cap, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, cap, D, generator=g).to(torch.bfloat16)
    kn = torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16)
    sl = torch.tensor([0, 7, 8], dtype=torch.int32)
    kd, vd, sd = kc.to(DEV), vc.to(DEV), sl.to(DEV)
    attn.attn_kv_append(kn.to(DEV), vn.to(DEV), kd, vd, sd)
    torch.cuda.synchronize()
    ek, ev = kc.clone(), vc.clone()
    for b, L in enumerate(sl.tolist()):
        if L < cap:
            ek[b, :, L] = kn[b]
            ev[b, :, L] = vn[b]
    assert torch.equal(kd.cpu(), ek) and torch.equal(vd.cpu(), ev)
    assert sd.cpu().tolist() == [1, 8, 8]


@pytest.mark.parametrize("num_splits", [1, 5, 0])
def test_decode_padded_matches_oracle(num_splits):
    B, Hq, Hkv, D, cap = 5, 8, 2, 128, 300
    lens = np.array([1, 300, 0, 77, 129], dtype=np.int32)
    say(f"[decode padded] B={B} cap={cap} lens={lens.tolist()} ns={num_splits}")
    rng = np.random.default_rng(9)
    q = torch.from_numpy(rng.standard_normal((B, Hq, D), dtype=np.float32)).to(torch.bfloat16)
    kc = torch.from_numpy(rng.standard_normal((B, Hkv, cap, D), dtype=np.float32)).to(torch.bfloat16)
    vc = torch.from_numpy(rng.standard_normal((B, Hkv, cap, D), dtype=np.float32)).to(torch.bfloat16)
    o, lse = attn.attn_decode_padded(q.to(DEV), kc.to(DEV), vc.to(DEV),
                                     torch.from_numpy(lens).to(DEV),
                                     num_splits=num_splits, with_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(np64(q), padded_to_packed(np64(kc), lens),
                           padded_to_packed(np64(vc), lens), lens,
                           1 / math.sqrt(D), Hkv)
    live = lens > 0
    assert (np64(o)[~live] == 0).all()
    eo = np.abs(np64(o)[live] - ro[live]).max()
    el = np.abs(lse.cpu().numpy()[live] - rl[live]).max()
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= 2e-2 and el <= LSE_TOL


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
def test_decode_step_graph_replay(rope_base):
    """append + decode captured once, replayed step after step with new k/v
    copied in between; every replay is checked against an eager decode and
    against the oracle on the cache as it stands (with RoPE: the oracle's
    own rotation of every key at its position and of q at L - 1)."""
    B, Hq, Hkv, D, cap, steps = 4, 8, 2, 128, 600, 5
    say(f"[graph decode step] B={B} cap={cap} steps={steps} rope={rope_base}")
    rng = np.random.default_rng(13)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    lens0 = np.array([0, 31, 256, 500], dtype=np.int32)
    # raw keys of every position; the cache holds them rotated (oracle
    # rotation, rounded to bf16) when RoPE is on
    kraw = rng.standard_normal((B, Hkv, cap, D))
    kstore = kraw if rope_base == 0 else \
        bf16_stored(oracle.rope(kraw, np.arange(cap), rope_base))
    kc = bf(kstore).to(DEV)
    vc = bf(rng.standard_normal((B, Hkv, cap, D))).to(DEV)
    kref = np64(kc)                       # the oracle's view of the cache
    sl = torch.from_numpy(lens0.copy()).to(DEV)
    q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    kn = torch.empty(B, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vn = torch.empty(B, Hkv, D, dtype=torch.bfloat16, device=DEV)
    o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    ws = attn.new_decode_workspace(B, Hq, Hkv, D, 0, DEV)

    def step():
        attn.attn_kv_append(kn, vn, kc, vc, sl, rope_base=rope_base)
        attn.attn_decode_padded(q, kc, vc, sl, out=o, lse=lse, workspace=ws,
                                rope_base=rope_base)

    # warm up on a side stream (capture requirement), then capture one step
    # and undo the warm-up's append on the host copy of the lengths
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.copy_(bf(rng.standard_normal((B, Hq, D))).to(DEV))
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    sl.copy_(torch.from_numpy(lens0.copy()).to(DEV))
    torch.cuda.synchronize()
    for t in range(steps):
        q.copy_(bf(rng.standard_normal((B, Hq, D))).to(DEV))
        kn.copy_(bf(rng.standard_normal((B, Hkv, D))).to(DEV))
        vn.copy_(bf(rng.standard_normal((B, Hkv, D))).to(DEV))
        torch.cuda.synchronize()
        pos = lens0 + t                   # where this step's key lands
        knew = np64(kn)
        for b in range(B):
            kref[b, :, pos[b]] = knew[b] if rope_base == 0 else \
                bf16_stored(oracle.rope(knew[b], pos[b], rope_base))
        g.replay()
        torch.cuda.synchronize()
        lens = sl.cpu().numpy()
        assert (lens == lens0 + t + 1).all()
        eo, el = attn.attn_decode_padded(q, kc, vc, sl, with_lse=True,
                                         rope_base=rope_base)
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el)
        if rope_base:
            # the stored key of this step: the oracle's rotation, up to the
            # bf16 rounding of the stored value
            for b in range(B):
                d = np.abs(np64(kc)[b, :, pos[b]] - kref[b, :, pos[b]])
                assert d.max() <= 2 ** -8 * np.abs(kref[b, :, pos[b]]).max()
        qref = np64(q) if rope_base == 0 else \
            bf16_stored(oracle.rope(np64(q), (lens - 1)[:, None], rope_base))
        ro, rl = oracle.decode(qref, padded_to_packed(kref, lens),
                               padded_to_packed(np64(vc), lens), lens,
                               1 / math.sqrt(D), Hkv)
        err = np.abs(np64(o) - ro).max()
        say(f"   replay {t}: lens={lens.tolist()} max|dO|={err:.3e}")
        assert err <= 2e-2
        assert np.abs(lse.cpu().numpy() - rl).max() <= LSE_TOL


@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_graph_replay():
    """A prefill launch captured once in a graph and replayed with new
    inputs copied in between: every replay equals an eager launch on the
    same inputs bit for bit and matches the oracle."""
    B, Hq, Hkv, S, D = 2, 8, 2, 300, 128
    say(f"[graph prefill] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}")
    q = torch.empty(B, Hq, S, D, dtype=torch.bfloat16, device=DEV)
    k = torch.empty(B, Hkv, S, D, dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, S, dtype=torch.float32, device=DEV)

    def load(seed):
        for dst, src in zip((q, k, v), inputs.prefill_inputs(
                B, Hq, Hkv, S, D, "bf16", 1.0, seed)):
            dst.copy_(src.to(DEV))

    load(20)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        attn.attn_prefill(q, k, v, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn.attn_prefill(q, k, v, out=o, lse=lse)
    torch.cuda.synchronize()
    for t in range(3):
        load(21 + t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo, el = attn.attn_prefill(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el)
        ro, rl = oracle.prefill(np64(q), np64(k), np64(v), 1 / math.sqrt(D),
                                True)
        err = np.abs(np64(o) - ro).max()
        say(f"   replay {t}: max|dO|={err:.3e}")
        assert err <= o_tol("bf16")
        assert np.abs(lse.cpu().numpy() - rl).max() <= LSE_TOL


# ------------------------------------------------------------ padded batch

@pytest.mark.parametrize("B,Hq,Hkv,S,D,lens", [
    (3, 8, 2, 300, 128, [0, 1, 300]),
    (4, 8, 2, 257, 128, [129, 64, 200, 257]),
    (4, 12, 12, 129, 64, [129, 65, 5, 128]),
    (2, 8, 1, 1000, 128, [999, 333]),
])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_padded_matches_oracle(B, Hq, Hkv, S, D, lens, causal):
    say(f"[prefill padded] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} lens={lens} "
        f"causal={causal}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, "bf16", 1.0, 7)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = attn.attn_prefill_padded(q.to(DEV), k.to(DEV), v.to(DEV), sl,
                                      causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_padded(np64(q), np64(k), np64(v), lens,
                                   1 / math.sqrt(D), causal)
    oo, ll = np64(o), lse.cpu().numpy()
    for b, L in enumerate(lens):
        assert (oo[b, :, L:] == 0).all() and (ll[b, :, L:] == -np.inf).all()
        if L:
            eo = np.abs(oo[b, :, :L] - ro[b, :, :L]).max()
            el = np.abs(ll[b, :, :L] - rl[b, :, :L]).max()
            say(f"   b={b} L={L} max|dO|={eo:.3e} max|dLSE|={el:.3e}")
            assert eo <= o_tol("bf16") and el <= LSE_TOL


def dense_one_range(q, k, v):
    """Dense prefill without a workspace and without the key-split kernel:
    every query tile in one workgroup over its whole key range, the launch
    shape the padded and ragged entry points share (the balanced schedule
    and the key-split kernel merge key ranges and so round differently).
    The kernel is the one those entry points take under the current
    setting: under ATTN_PREFILL_KS the 4-wave kernel, under the automatic
    choice its shape table without the key-split rule (the register-blocked
    kernel for head dim 128 from 4e8 score elements on)."""
    prev = attn.prefill_workspace_policy(False)
    sel = attn.prefill_select(attn.PREFILL_AUTO)
    B, Hq, S, D = q.shape
    if sel == attn.PREFILL_KS:
        force = attn.PREFILL_W4
    elif sel == attn.PREFILL_AUTO:
        big = D == 128 and B * Hq * S * (S + 1) / 2 >= 4e8
        force = attn.PREFILL_RB if big else attn.PREFILL_W4
    else:
        force = sel
    attn.prefill_select(force)
    try:
        return attn.attn_prefill(q, k, v)
    finally:
        attn.prefill_select(sel)
        attn.prefill_workspace_policy(prev)


# ------------------------------------------- balanced causal schedule

FLAG_BYTES = 4096      # the workspace's flag words, one per pair of tiles


@pytest.mark.parametrize("B,Hq,Hkv,S", [(4, 8, 2, 2048), (2, 8, 2, 300),
                                        (1, 16, 4, 1000), (3, 8, 1, 129),
                                        (1, 4, 1, 16384)])
@pytest.mark.parametrize("wait", [-1, 0])
def test_prefill_balanced_matches_oracle_and_leaves_flags_zero(B, Hq, Hkv, S,
                                                               wait):
    """The balanced schedule (forced on with the register-blocked kernel,
    so that it also runs at sizes the automatic choice leaves to the 4-wave
    kernel) against the oracle, with the hand-off waiting
    by the kernel's rule (-1) or giving up at once (0: the second workgroup
    of a pair computes the first one's part itself whenever the part is not
    there yet).  The flag words are zero afterwards either way, and what the
    rest of the workspace held does not matter."""
    D = 128
    say(f"[prefill balanced] B={B} Hq={Hq} Hkv={Hkv} S={S} wait={wait}")
    prev_sel = attn.prefill_select(attn.PREFILL_RB)
    prev_wait = attn.prefill_split_wait(wait)
    try:
        assert attn.attn_prefill_workspace_size(B, Hq, Hkv, S, D) > 0
        q, k, v = (t.to(DEV) for t in
                   inputs.prefill_inputs(B, Hq, Hkv, S, D, "bf16", 1.0, 31))
        ws = attn.new_prefill_workspace(B, Hq, Hkv, S, D, device=DEV)
        nf = FLAG_BYTES
        ws[nf:] = 0xFF                 # every float of the parts reads NaN
        for rep in range(2):
            o, lse = attn.attn_prefill(q, k, v, workspace=ws)
            torch.cuda.synchronize()
            assert int(ws[:nf].count_nonzero()) == 0
            if B * Hq * S <= 16 * 2048:
                ro, rl = oracle.prefill(np64(q), np64(k), np64(v),
                                        1 / math.sqrt(D), True)
                eo = np.abs(np64(o) - ro).max()
                el = np.abs(lse.cpu().numpy() - rl).max()
            else:
                rows = inputs.sampled_rows(Hq, S, 64)
                ro, rl = oracle.prefill_rows(np64(q), np64(k), np64(v),
                                             1 / math.sqrt(D), True, rows)
                oo, ll = np64(o), lse.cpu().numpy()
                eo = max(np.abs(oo[b][h][rows[h]] - ro[b, h]).max()
                         for b in range(B) for h in range(Hq))
                el = max(np.abs(ll[b][h][rows[h]] - rl[b, h]).max()
                         for b in range(B) for h in range(Hq))
            say(f"   rep {rep}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
            assert eo <= o_tol("bf16") and el <= LSE_TOL
    finally:
        attn.prefill_split_wait(prev_wait)
        attn.prefill_select(prev_sel)


def test_prefill_balanced_workspace_reused_across_sizes():
    """One workspace serves launches of different sizes in turn (the flag
    words sit in the same place for all): each launch (balanced schedule
    forced on) matches the oracle on sampled rows and leaves the flags
    zero."""
    D = 128
    prev_sel = attn.prefill_select(attn.PREFILL_RB)
    try:
        ws = attn.new_prefill_workspace(4, 8, 2, 2048, D, device=DEV)
        for (B, Hq, Hkv, S) in [(4, 8, 2, 2048), (1, 8, 2, 4096),
                                (2, 8, 2, 300), (4, 8, 2, 2048)]:
            say(f"[prefill balanced reuse] B={B} Hq={Hq} Hkv={Hkv} S={S}")
            assert 0 < attn.attn_prefill_workspace_size(B, Hq, Hkv, S,
                                                        D) <= ws.numel()
            q, k, v = (t.to(DEV) for t in
                       inputs.prefill_inputs(B, Hq, Hkv, S, D, "bf16", 1.0,
                                             S))
            o, lse = attn.attn_prefill(q, k, v, workspace=ws)
            torch.cuda.synchronize()
            assert int(ws[:FLAG_BYTES].count_nonzero()) == 0
            rows = inputs.sampled_rows(Hq, S, min(S, 64))
            ro, rl = oracle.prefill_rows(np64(q), np64(k), np64(v),
                                         1 / math.sqrt(D), True, rows)
            oo, ll = np64(o), lse.cpu().numpy()
            eo = max(np.abs(oo[b][h][rows[h]] - ro[b, h]).max()
                     for b in range(B) for h in range(Hq))
            el = max(np.abs(ll[b][h][rows[h]] - rl[b, h]).max()
                     for b in range(B) for h in range(Hq))
            say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
            assert eo <= o_tol("bf16") and el <= LSE_TOL
    finally:
        attn.prefill_select(prev_sel)


def test_prefill_balanced_is_the_default_and_reproducible():
    """attn_prefill passes its own workspace: a C3-sized causal launch runs
    the balanced schedule, and repeated calls (merging the same parts in
    the same order) agree bit for bit."""
    B, Hq, Hkv, S, D = 4, 8, 2, 2048, 128
    say(f"[prefill balanced default] B={B} Hq={Hq} Hkv={Hkv} S={S}")
    assert attn.prefill_balanced(B, Hq, Hkv, S, D)
    q, k, v = (t.to(DEV) for t in
               inputs.prefill_inputs(B, Hq, Hkv, S, D, "bf16", 1.0, 32))
    o1, l1 = attn.attn_prefill(q, k, v)
    o2, l2 = attn.attn_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_padded_full_lengths_equal_dense_and_ignore_padding():
    # lengths = S: the dense kernel's results bit for bit; and values written
    # into the padding rows change nothing
    B, Hq, Hkv, S, D = 2, 8, 2, 300, 128
    say(f"[prefill padded vs dense] B={B} S={S}")
    q, k, v = (t.to(DEV) for t in
               inputs.prefill_inputs(B, Hq, Hkv, S, D, "bf16", 1.0, 8))
    full = torch.full((B,), S, dtype=torch.int32, device=DEV)
    o1, l1 = attn.attn_prefill_padded(q, k, v, full)
    o2, l2 = dense_one_range(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    lens = torch.tensor([77, 300], dtype=torch.int32, device=DEV)
    o3, l3 = attn.attn_prefill_padded(q, k, v, lens)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for t in (q2, k2, v2):
        t[0, :, 77:] = 1000.0
    o4, l4 = attn.attn_prefill_padded(q2, k2, v2, lens)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


# ------------------------------------------------------------------- RoPE

@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(1, 8, 2, 300, 128),
                                          (2, 12, 12, 129, 64),
                                          (1, 1, 1, 1, 128),
                                          (4, 8, 2, 2048, 128)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_rope_matches_oracle(B, Hq, Hkv, S, D, causal):
    base = 10000.0
    say(f"[prefill rope] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, "bf16", 1.0, 4)
    o, lse, kr = attn.attn_prefill_rope(q.to(DEV), k.to(DEV), v.to(DEV), base,
                                        causal=causal)
    torch.cuda.synchronize()
    pos = np.arange(S)
    qr = bf16_stored(oracle.rope(np64(q), pos, base))
    krr = bf16_stored(oracle.rope(np64(k), pos, base))
    # rotated keys: the oracle's rotation, stored in bf16 (a rotation that
    # lands next to a rounding boundary may round to the neighbouring value)
    assert np.abs(np64(kr) - krr).max() <= 2 ** -8 * np.abs(krr).max()
    ro, rl = oracle.prefill(qr, krr, np64(v), 1 / math.sqrt(D), causal)
    eo, el = np.abs(np64(o) - ro).max(), np.abs(lse.cpu().numpy() - rl).max()
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= 2e-2 and el <= LSE_TOL


@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_rope_long_positions_sampled():
    """Angles at positions up to 8191: reduced in fp64, so late rows are as
    accurate as early ones.  Sampled rows against the oracle."""
    B, Hq, Hkv, S, D, base = 1, 2, 1, 8192, 128, 10000.0
    say(f"[prefill rope long] S={S}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, "bf16", 1.0, 6)
    o, lse, kr = attn.attn_prefill_rope(q.to(DEV), k.to(DEV), v.to(DEV), base)
    torch.cuda.synchronize()
    pos = np.arange(S)
    krr = bf16_stored(oracle.rope(np64(k), pos, base))
    assert np.abs(np64(kr) - krr).max() <= 2 ** -8 * np.abs(krr).max()
    rows = np.array([0, 1, 77, 4095, 8000, 8190, 8191])
    qr = bf16_stored(oracle.rope(np64(q), pos, base))
    ro, rl = oracle.prefill_rows(qr, krr, np64(v), 1 / math.sqrt(D), True,
                                 np.tile(rows, (Hq, 1)))
    go = np64(o)[:, :, rows]
    eo = np.abs(go - ro).max()
    el = np.abs(lse.cpu().numpy()[:, :, rows] - rl).max()
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= 2e-2 and el <= LSE_TOL


def test_kv_append_rope_stores_rotated_keys():
    B, Hkv, cap, D, base = 3, 2, 5000, 128, 10000.0
    say(f"[append rope] B={B} cap={cap}")
    rng = np.random.default_rng(8)
    kc = torch.zeros(B, Hkv, cap, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kn = torch.from_numpy(rng.standard_normal((B, Hkv, D)).astype(np.float32)).to(torch.bfloat16)
    vn = torch.from_numpy(rng.standard_normal((B, Hkv, D)).astype(np.float32)).to(torch.bfloat16)
    lens = np.array([0, 1, 4999], dtype=np.int32)
    sl = torch.from_numpy(lens.copy()).to(DEV)
    attn.attn_kv_append(kn.to(DEV), vn.to(DEV), kc, vc, sl, rope_base=base)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        ref = bf16_stored(oracle.rope(np64(kn)[b], L, base))
        got = np64(kc)[b, :, L]
        assert np.abs(got - ref).max() <= 2 ** -8 * np.abs(ref).max()
        assert torch.equal(vc[b, :, L].cpu(), vn[b])
    assert sl.cpu().tolist() == [1, 2, 5000]


# ------------------------------------------------------- ragged batch prefill

def packed_inputs(lens, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    N = int(np.sum(lens))
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    q = bf(rng.standard_normal(Hq * N * D))
    k = bf(rng.standard_normal(Hkv * N * D))
    v = bf(rng.standard_normal(Hkv * N * D))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, cu


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (1, 1)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_varlen_matches_oracle(D, Hq, Hkv, causal):
    lens = [0, 1, 127, 128, 129, 1000, 257]
    say(f"[prefill varlen] lens={lens} Hq={Hq} Hkv={Hkv} D={D} causal={causal}")
    q, k, v, cu = packed_inputs(lens, Hq, Hkv, D, 31)
    o, lse = attn.attn_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV),
                                      torch.from_numpy(cu).to(DEV),
                                      max(lens), Hq, Hkv, D, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(np64(q), np64(k), np64(v), cu, Hq, Hkv,
                                   1 / math.sqrt(D), causal)
    eo, el = np.abs(np64(o) - ro).max(), np.abs(lse.cpu().numpy() - rl).max()
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= 2e-2 and el <= LSE_TOL


@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_varlen_equal_lengths_is_the_dense_kernel():
    # with equal lengths the packed layout is [B, H, S, D]; every workgroup
    # does the same arithmetic as the dense launch, so the results match
    # bit for bit
    B, Hq, Hkv, S, D = 3, 8, 2, 300, 128
    say(f"[prefill varlen == dense] B={B} S={S}")
    q, k, v = (t.to(DEV) for t in inputs.prefill_inputs(B, Hq, Hkv, S, D,
                                                         "bf16", 1.0, 3))
    cu = torch.arange(B + 1, dtype=torch.int32, device=DEV) * S
    o, lse = attn.attn_prefill_varlen(q, k, v, cu, S, Hq, Hkv, D)
    do, dl = dense_one_range(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o.view(B, Hq, S, D), do)
    assert torch.equal(lse.view(B, Hq, S), dl)


# ------------------------------------------- a late, far larger row maximum

@pytest.mark.parametrize("boost", [8.0, 1.5])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_late_dominant_key(dtype, causal, boost):
    """One late key aligned with every query row of head 0 and `boost` times
    as long.  boost 8: its score exceeds each row's first-tile maximum by
    about 130 log2 units, past any headroom a kernel may keep over a
    reference maximum; boost 1.5: by about 20, above the headroom of fp16
    probabilities but not of bf16 ones.  The result must match the oracle,
    and for boost 8 the rows that see the key take its value."""
    B, Hq, Hkv, S, D = 1, 2, 1, 1100, 128
    say(f"[prefill late dominant key] {dtype} causal={causal} boost={boost}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, dtype, 1.0, 12)
    j = 1000
    q[:, 0] = q[:, 0, :1]
    k[:, 0, j] = (q[:, 0, 0].float() * boost).to(q.dtype)
    o, lse = attn.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(np64(q), np64(k), np64(v), 1 / math.sqrt(D),
                            causal)
    eo, el = np.abs(np64(o) - ro).max(), np.abs(lse.cpu().numpy() - rl).max()
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert np.isfinite(np64(o)).all()
    assert eo <= o_tol(dtype) and el <= LSE_TOL
    if boost == 8.0:
        rows = slice(j, S) if causal else slice(0, S)
        assert np.abs(np64(o)[0, 0, rows] - np64(v)[0, 0, j]).max() \
            <= o_tol(dtype)
