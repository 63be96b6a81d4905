"""fp16 storage on every path of a serving loop, against the fp64 oracle.

fp16 keeps the mixed-precision rule of the attention-fusion page, section 5.5
(fp16 only in storage and in the MFMA inputs, fp32 accumulation and state).
The pages give no bound for it; the bound is derived from the arithmetic as
in test_gpu_parity.py: P is rounded to fp16 before the PV product and O once
more on output, each at most 2^-11 relative on values bounded by max|v|, so
5e-3 for unit-variance inputs; LSE 1e-3 as everywhere.

Where RoPE is on, the rotated q and k enter the products (and the cache) as
fp16 values, so the expected values round the oracle's fp64 rotation to fp16
at that point, exactly as the bf16 tests round it to bf16.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from causal_attention_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_TOL = 5e-3
LSE_TOL = 1e-3
F16 = torch.float16


def say(*a):
    print(*a, flush=True)


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def f16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(F16)


def f16_stored(x):
    """x (fp64) rounded to fp16, as float64: what an fp16 tensor holds."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(
        np.float64)


def padded_to_packed(kc, sl):
    return np.concatenate([kc[b, :, :max(int(L), 0)].reshape(-1)
                           for b, L in enumerate(sl)])


def close_to_rounded(got, ref):
    # a rotation next to a rounding boundary may round to the neighbour
    return np.abs(got - ref).max() <= 2 ** -10 * np.abs(ref).max()


def test_kv_append_f16_copies_rows():
    B, Hkv, cap, D = 3, 2, 8, 64
    say(f"[append f16] B={B} Hkv={Hkv} cap={cap} D={D}")
    g = torch.Generator().manual_seed(5)
    kc = torch.randn(B, Hkv, cap, D, generator=g).to(F16)
    vc = torch.randn(B, Hkv, cap, D, generator=g).to(F16)
    kn = torch.randn(B, Hkv, D, generator=g).to(F16)
    vn = torch.randn(B, Hkv, D, generator=g).to(F16)
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


@pytest.mark.parametrize("D", [64, 128])
def test_kv_append_rope_f16_stores_rotated_keys(D):
    B, Hkv, cap, base = 3, 2, 5000, 10000.0
    say(f"[append rope f16] B={B} cap={cap} D={D}")
    rng = np.random.default_rng(8)
    kc = torch.zeros(B, Hkv, cap, D, dtype=F16, device=DEV)
    vc = torch.zeros_like(kc)
    kn = f16(rng.standard_normal((B, Hkv, D)))
    vn = f16(rng.standard_normal((B, Hkv, D)))
    lens = np.array([0, 1, 4999], dtype=np.int32)
    sl = torch.from_numpy(lens.copy()).to(DEV)
    attn.attn_kv_append(kn.to(DEV), vn.to(DEV), kc, vc, sl, rope_base=base)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        ref = f16_stored(oracle.rope(np64(kn)[b], L, base))
        got = np64(kc)[b, :, L]
        err = np.abs(got - ref).max()
        say(f"   b={b} pos={L} max|dk|={err:.3e}")
        assert close_to_rounded(got, ref)
        assert torch.equal(vc[b, :, L].cpu(), vn[b])
    assert sl.cpu().tolist() == [1, 2, 5000]


@pytest.mark.parametrize("num_splits", [1, 5, 0])
def test_decode_padded_f16_matches_oracle(num_splits):
    B, Hq, Hkv, D, cap = 5, 8, 2, 128, 300
    lens = np.array([1, 300, 0, 77, 129], dtype=np.int32)
    say(f"[decode padded f16] B={B} cap={cap} lens={lens.tolist()} "
        f"ns={num_splits}")
    rng = np.random.default_rng(9)
    q = f16(rng.standard_normal((B, Hq, D)))
    kc = f16(rng.standard_normal((B, Hkv, cap, D)))
    vc = f16(rng.standard_normal((B, Hkv, cap, D)))
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
    assert eo <= O_TOL and el <= LSE_TOL


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
def test_decode_step_graph_replay_f16(rope_base):
    """fp16 append + decode captured once and replayed with new q, k, v each
    step; every replay equals an eager decode bit for bit and matches the
    oracle on the cache as it stands."""
    B, Hq, Hkv, D, cap, steps = 4, 8, 2, 128, 600, 4
    say(f"[graph decode step f16] B={B} cap={cap} steps={steps} "
        f"rope={rope_base}")
    rng = np.random.default_rng(13)
    lens0 = np.array([0, 31, 256, 500], dtype=np.int32)
    kraw = rng.standard_normal((B, Hkv, cap, D))
    kstore = kraw if rope_base == 0 else \
        f16_stored(oracle.rope(kraw, np.arange(cap), rope_base))
    kc = f16(kstore).to(DEV)
    vc = f16(rng.standard_normal((B, Hkv, cap, D))).to(DEV)
    kref = np64(kc)
    sl = torch.from_numpy(lens0.copy()).to(DEV)
    q = torch.empty(B, Hq, D, dtype=F16, device=DEV)
    kn = torch.empty(B, Hkv, D, dtype=F16, device=DEV)
    vn = torch.empty(B, Hkv, D, dtype=F16, device=DEV)
    o = torch.empty(B, Hq, D, dtype=F16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    ws = attn.new_decode_workspace(B, Hq, Hkv, D, 0, DEV)

    def step():
        attn.attn_kv_append(kn, vn, kc, vc, sl, rope_base=rope_base)
        attn.attn_decode_padded(q, kc, vc, sl, out=o, lse=lse, workspace=ws,
                                rope_base=rope_base)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.copy_(f16(rng.standard_normal((B, Hq, D))).to(DEV))
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
        q.copy_(f16(rng.standard_normal((B, Hq, D))).to(DEV))
        kn.copy_(f16(rng.standard_normal((B, Hkv, D))).to(DEV))
        vn.copy_(f16(rng.standard_normal((B, Hkv, D))).to(DEV))
        torch.cuda.synchronize()
        pos = lens0 + t
        knew = np64(kn)
        for b in range(B):
            kref[b, :, pos[b]] = knew[b] if rope_base == 0 else \
                f16_stored(oracle.rope(knew[b], pos[b], rope_base))
        g.replay()
        torch.cuda.synchronize()
        lens = sl.cpu().numpy()
        assert (lens == lens0 + t + 1).all()
        eo, el = attn.attn_decode_padded(q, kc, vc, sl, with_lse=True,
                                         rope_base=rope_base)
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el)
        if rope_base:
            for b in range(B):
                assert close_to_rounded(np64(kc)[b, :, pos[b]],
                                        kref[b, :, pos[b]])
        qref = np64(q) if rope_base == 0 else \
            f16_stored(oracle.rope(np64(q), (lens - 1)[:, None], rope_base))
        ro, rl = oracle.decode(qref, padded_to_packed(kref, lens),
                               padded_to_packed(np64(vc), lens), lens,
                               1 / math.sqrt(D), Hkv)
        err = np.abs(np64(o) - ro).max()
        lerr = np.abs(lse.cpu().numpy() - rl).max()
        say(f"   replay {t}: lens={lens.tolist()} max|dO|={err:.3e} "
            f"max|dLSE|={lerr:.3e}")
        assert err <= O_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(1, 8, 2, 300, 128),
                                          (2, 12, 12, 129, 64)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_rope_f16_matches_oracle(B, Hq, Hkv, S, D, causal):
    base = 10000.0
    say(f"[prefill rope f16] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} "
        f"causal={causal}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, "f16", 1.0, 4)
    o, lse, kr = attn.attn_prefill_rope(q.to(DEV), k.to(DEV), v.to(DEV), base,
                                        causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == F16 and kr.dtype == F16
    pos = np.arange(S)
    qr = f16_stored(oracle.rope(np64(q), pos, base))
    krr = f16_stored(oracle.rope(np64(k), pos, base))
    assert close_to_rounded(np64(kr), krr)
    ro, rl = oracle.prefill(qr, krr, np64(v), 1 / math.sqrt(D), causal)
    eo, el = np.abs(np64(o) - ro).max(), np.abs(lse.cpu().numpy() - rl).max()
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= O_TOL and el <= LSE_TOL


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_varlen_f16_matches_oracle(causal):
    lens, Hq, Hkv, D = [0, 1, 127, 129, 1000, 257], 8, 2, 128
    say(f"[prefill varlen f16] lens={lens} causal={causal}")
    rng = np.random.default_rng(31)
    N = int(np.sum(lens))
    q = f16(rng.standard_normal(Hq * N * D))
    k = f16(rng.standard_normal(Hkv * N * D))
    v = f16(rng.standard_normal(Hkv * N * D))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, lse = attn.attn_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV),
                                      torch.from_numpy(cu).to(DEV),
                                      max(lens), Hq, Hkv, D, causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == F16
    ro, rl = oracle.prefill_varlen(np64(q), np64(k), np64(v), cu, Hq, Hkv,
                                   1 / math.sqrt(D), causal)
    eo, el = np.abs(np64(o) - ro).max(), np.abs(lse.cpu().numpy() - rl).max()
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= O_TOL and el <= LSE_TOL


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.usefixtures("prefill_kernel")
def test_prefill_padded_f16_matches_oracle(causal):
    B, Hq, Hkv, S, D, lens = 4, 8, 2, 257, 128, [129, 0, 200, 257]
    say(f"[prefill padded f16] lens={lens} causal={causal}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, "f16", 1.0, 7)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = attn.attn_prefill_padded(q.to(DEV), k.to(DEV), v.to(DEV), sl,
                                      causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == F16
    ro, rl = oracle.prefill_padded(np64(q), np64(k), np64(v), lens,
                                   1 / math.sqrt(D), causal)
    oo, ll = np64(o), lse.cpu().numpy()
    for b, L in enumerate(lens):
        assert (oo[b, :, L:] == 0).all() and (ll[b, :, L:] == -np.inf).all()
        if L:
            eo = np.abs(oo[b, :, :L] - ro[b, :, :L]).max()
            el = np.abs(ll[b, :, :L] - rl[b, :, :L]).max()
            say(f"   b={b} L={L} max|dO|={eo:.3e} max|dLSE|={el:.3e}")
            assert eo <= O_TOL and el <= LSE_TOL
