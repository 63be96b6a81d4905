"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test checks the oracle against a closed form, an invariant the
mathematics fixes, brute force on tiny inputs written as plain scalar loops,
or an independent library implementation (torch's scaled_dot_product_attention
in float64).  The last group plants plausible mistakes in the oracle (a wrong
GQA index, a dropped diagonal, a wrong log base, a wrong sign) and checks that
some pin catches each one.

Sources (page titles):
* "Attention三算子融合实战：从Triton到CUDA的推理加速优化": section 1.1 (the
  chain), 2.2 (online softmax merge, order-free), 4.3 (causal and length
  masks), 1.3 (decode: one query row against the whole history).
* "手写Triton kernel重构Qwen3.5-0.8B": section 2.1 (GQA 8/2, head_dim 128).
* "triton-optimization" skill page, section 3.5: log-sum-exp = m + log d.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_attention
from causal_attention_amd import inputs

TOL = 1e-12


def rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def prefill_np(B, Hq, Hkv, S, D, seed=0, sigma=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D)) * sigma
    k = rng.standard_normal((B, Hkv, S, D)) * sigma
    v = rng.standard_normal((B, Hkv, S, D)) * sigma
    return q, k, v


# --------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [True, False])
def test_p1_single_key(causal):
    q, k, v = prefill_np(2, 4, 2, 1, 16, seed=1)
    scale = 0.3
    o, lse = oracle.prefill(q, k, v, scale, causal)
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(o[:, h], v[:, g], atol=TOL)
        np.testing.assert_allclose(
            lse[:, h, 0], scale * np.einsum("bd,bd->b", q[:, h, 0], k[:, g, 0]),
            atol=TOL)


def test_p1_single_key_decode():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 4, 8))
    kc = rng.standard_normal((3 * 2 * 1 * 8,))
    vc = rng.standard_normal((3 * 2 * 1 * 8,))
    o, lse = oracle.decode(q, kc, vc, [1, 1, 1], 0.5, Hkv=2)
    K = kc.reshape(3, 2, 8)
    V = vc.reshape(3, 2, 8)
    for b in range(3):
        for h in range(4):
            np.testing.assert_allclose(o[b, h], V[b, h // 2], atol=TOL)
            assert abs(lse[b, h] - 0.5 * q[b, h] @ K[b, h // 2]) < TOL


def test_p2_causal_row0_is_v0():
    q, k, v = prefill_np(1, 2, 1, 37, 8, seed=3)
    o, lse = oracle.prefill(q, k, v, 0.125, True)
    for h in range(2):
        np.testing.assert_allclose(o[0, h, 0], v[0, 0, 0], atol=TOL)
        assert abs(lse[0, h, 0] - 0.125 * q[0, h, 0] @ k[0, 0, 0]) < TOL


@pytest.mark.parametrize("causal", [True, False])
def test_p3_identical_keys_mean_of_v(causal):
    S, D = 23, 8
    q, _, v = prefill_np(1, 1, 1, S, D, seed=4)
    kk = rand((D,), 5)
    k = np.broadcast_to(kk, (1, 1, S, D)).copy()
    scale = 0.7
    o, lse = oracle.prefill(q, k, v, scale, causal)
    for i in range(S):
        n = i + 1 if causal else S
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(0), atol=1e-12)
        assert abs(lse[0, 0, i] - (scale * q[0, 0, i] @ kk + math.log(n))) < 1e-12


def test_p4_zero_query_prefix_mean_natural_log():
    S, D = 19, 4
    _, k, v = prefill_np(1, 1, 1, S, D, seed=6)
    q = np.zeros((1, 1, S, D))
    o, lse = oracle.prefill(q, k, v, 1.0, True)
    for i in range(S):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :i + 1].mean(0), atol=1e-12)
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_p5_probability_rows_sum_to_one_and_mask(causal):
    q, k, _ = prefill_np(2, 4, 2, 17, 8, seed=7)
    P = oracle.softmax_probabilities(q, k, 0.4, causal)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
    assert (P >= 0).all()
    if causal:
        upper = np.triu(np.ones((17, 17), dtype=bool), k=1)
        assert (P[..., upper] == 0).all()
        assert (P[..., ~upper] > 0).all()


def test_p6_constant_and_zero_values():
    q, k, _ = prefill_np(1, 2, 2, 11, 8, seed=8)
    c = rand((8,), 9)
    v = np.broadcast_to(c, (1, 2, 11, 8)).copy()
    o, _ = oracle.prefill(q, k, v, 0.3, True)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-12)
    o0, _ = oracle.prefill(q, k, np.zeros_like(v), 0.3, True)
    assert (o0 == 0).all()


def test_p7_key_shift():
    q, k, v = prefill_np(1, 2, 1, 13, 8, seed=10)
    u = rand((8,), 11)
    scale = 0.25
    o1, l1 = oracle.prefill(q, k, v, scale, True)
    o2, l2 = oracle.prefill(q, k + u, v, scale, True)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, scale * q @ u, atol=1e-12)


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, scale, causal):
    """Scalar loops with math.exp and an explicit running max: no numpy."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    o = [[[[0.0] * D for _ in range(S)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * S for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for i in range(S):
                keys = range(i + 1) if causal else range(S)
                s = {}
                for j in keys:
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[b, h, i, d]) * float(k[b, g, j, d])
                    s[j] = acc * scale
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                tot = sum(e.values())
                for d in range(D):
                    o[b][h][i][d] = sum(e[j] / tot * float(v[b, g, j, d])
                                        for j in keys)
                lse[b][h][i] = m + math.log(tot)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(1, 1, 1, 1, 1), (2, 4, 2, 9, 8),
                                          (1, 4, 1, 7, 5), (2, 2, 2, 5, 3)])
@pytest.mark.parametrize("causal", [True, False])
def test_p8_brute_force(B, Hq, Hkv, S, D, causal):
    q, k, v = prefill_np(B, Hq, Hkv, S, D, seed=12 + S)
    o, lse = oracle.prefill(q, k, v, 0.6, causal)
    ob, lb = brute_force(q, k, v, 0.6, causal)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)


# ------------------------------------------------- independent library routine

def torch_sdpa_f64(q, k, v, scale, causal):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale,
        enable_gqa=q.shape[1] != k.shape[1])
    return out.numpy()


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [
    (1, 1, 1, 128, 64, True),      # single-head fp32 workload's shape
    (1, 12, 12, 96, 64, True),     # 12-head MHA, shortened
    (2, 8, 2, 64, 128, True),      # GQA 8/2, head_dim 128
    (2, 8, 2, 33, 128, False),
])
def test_p9_matches_torch_sdpa_float64(B, Hq, Hkv, S, D, causal):
    q, k, v = prefill_np(B, Hq, Hkv, S, D, seed=20 + S)
    scale = 1 / math.sqrt(D)
    o, _ = oracle.prefill(q, k, v, scale, causal)
    np.testing.assert_allclose(o, torch_sdpa_f64(q, k, v, scale, causal),
                               atol=1e-10)


def test_p10_gqa_equals_mha_on_repeated_kv():
    q, k, v = prefill_np(2, 8, 2, 21, 16, seed=30)
    rep = lambda a: np.repeat(a, 4, axis=1)          # heads 0-3 -> kv 0
    o1, l1 = oracle.prefill(q, k, v, 0.2, True)
    o2, l2 = oracle.prefill(q, rep(k), rep(v), 0.2, True)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


# ------------------------------------------------------- decode and combining

def pack(blocks):
    return np.concatenate([b.reshape(-1) for b in blocks])


def test_p11_split_combine_equals_unsplit():
    rng = np.random.default_rng(40)
    Hq, Hkv, D, L = 4, 2, 8, 50
    q = rng.standard_normal((1, Hq, D))
    K = rng.standard_normal((Hkv, L, D))
    V = rng.standard_normal((Hkv, L, D))
    o_full, l_full = oracle.decode(q, K.reshape(-1), V.reshape(-1), [L], 0.3, Hkv)
    for bounds in ([0, 50], [0, 1, 50], [0, 17, 17, 33, 50], [0, 0, 0, 50],
                   [0, 10, 20, 30, 40, 50, 50]):
        parts_o, parts_l = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            if b == a:    # an empty chunk: weight zero
                parts_o.append(np.zeros((1, Hq, D)))
                parts_l.append(np.full((1, Hq), -np.inf))
                continue
            o, l = oracle.decode(q, K[:, a:b].reshape(-1), V[:, a:b].reshape(-1),
                                 [b - a], 0.3, Hkv)
            parts_o.append(o)
            parts_l.append(l)
        o, l = oracle.lse_combine(np.stack(parts_o), np.stack(parts_l))
        np.testing.assert_allclose(o, o_full, atol=1e-12)
        np.testing.assert_allclose(l, l_full, atol=1e-12)


def test_p11_all_empty_chunks():
    o, l = oracle.lse_combine(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert (o == 0).all() and np.isneginf(l).all()


def test_p12_decode_equals_last_causal_prefill_row():
    Hq, Hkv, D = 8, 2, 16
    lens = [1, 5, 33]
    qs, ks, vs, want_o, want_l = [], [], [], [], []
    for n, L in enumerate(lens):
        q, k, v = prefill_np(1, Hq, Hkv, L, D, seed=50 + n)
        o, l = oracle.prefill(q, k, v, 0.25, True)
        qs.append(q[0, :, L - 1])
        ks.append(k[0])
        vs.append(v[0])
        want_o.append(o[0, :, L - 1])
        want_l.append(l[0, :, L - 1])
    o, l = oracle.decode(np.stack(qs), pack(ks), pack(vs), lens, 0.25, Hkv)
    np.testing.assert_allclose(o, np.stack(want_o), atol=1e-12)
    np.testing.assert_allclose(l, np.stack(want_l), atol=1e-12)


def test_p13_decode_token_permutation():
    rng = np.random.default_rng(60)
    Hq, Hkv, D, L = 4, 1, 8, 29
    q = rng.standard_normal((1, Hq, D))
    K = rng.standard_normal((Hkv, L, D))
    V = rng.standard_normal((Hkv, L, D))
    perm = rng.permutation(L)
    o1, l1 = oracle.decode(q, K.reshape(-1), V.reshape(-1), [L], 0.5, Hkv)
    o2, l2 = oracle.decode(q, K[:, perm].reshape(-1), V[:, perm].reshape(-1),
                           [L], 0.5, Hkv)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_decode_empty_sequence_gives_zero_and_neg_inf():
    q = np.ones((2, 2, 4))
    kc = np.ones(2 * 3 * 4)
    o, l = oracle.decode(q, kc, kc, [0, 3], 1.0, Hkv=2)
    assert (o[0] == 0).all() and np.isneginf(l[0]).all()
    np.testing.assert_allclose(o[1], 1.0, atol=1e-12)


def test_p14_large_scores_stay_finite_and_pick_argmax():
    q, k, v = prefill_np(1, 2, 1, 40, 16, seed=70, sigma=30.0)
    o, lse = oracle.prefill(q, k, v, 0.25, True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    s = 0.25 * q[0, :, :, :] @ k[0, 0].T
    for h in range(2):
        for i in range(40):
            row = np.sort(s[h, i, :i + 1])[::-1]
            if i > 0 and row[0] - row[1] > 40:
                j = int(np.argmax(s[h, i, :i + 1]))
                np.testing.assert_allclose(o[0, h, i], v[0, 0, j], atol=1e-12)


def test_prefill_rows_equal_full_prefill():
    q, k, v = prefill_np(2, 4, 2, 45, 8, seed=80)
    o, l = oracle.prefill(q, k, v, 0.3, True)
    rows = np.array([[0, 3, 44], [1, 2, 40], [44, 0, 7], [5, 6, 9]])
    orr, lr = oracle.prefill_rows(q, k, v, 0.3, True, rows)
    for h in range(4):
        np.testing.assert_allclose(orr[:, h], o[:, h, rows[h]], atol=1e-12)
        np.testing.assert_allclose(lr[:, h], l[:, h, rows[h]], atol=1e-12)


def test_oracle_sees_exact_bf16_values():
    q, k, v = inputs.prefill_inputs(1, 2, 1, 16, 8, "bf16", 1.0, seed=3)
    o, _ = oracle.prefill(q.float().numpy(), k.float().numpy(),
                          v.float().numpy(), 0.3, True)
    want = torch_sdpa_f64(q.double().numpy(), k.double().numpy(),
                          v.double().numpy(), 0.3, True)
    np.testing.assert_allclose(o, want, atol=1e-10)


# -------------------------------------------- planted mistakes must be caught

def _pins_hold():
    """A compact run of the pins above; False if any of them fails."""
    checks = [
        lambda: test_p2_causal_row0_is_v0(),
        lambda: test_p3_identical_keys_mean_of_v(True),
        lambda: test_p4_zero_query_prefix_mean_natural_log(),
        lambda: test_p7_key_shift(),
        lambda: test_p8_brute_force(2, 4, 2, 9, 8, True),
        lambda: test_p9_matches_torch_sdpa_float64(2, 8, 2, 64, 128, True),
        lambda: test_p12_decode_equals_last_causal_prefill_row(),
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_pins_pass_on_unmodified_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("mutation", [
    "interleaved_gqa", "strict_causal", "log10_lse", "shifted_scale_sign",
    "unnormalised",
])
def test_planted_mistake_is_caught(monkeypatch, mutation):
    A = oracle_attention
    if mutation == "interleaved_gqa":
        monkeypatch.setattr(A, "_kv_head", lambda h, Hq, Hkv: h % Hkv)
    elif mutation == "strict_causal":
        orig = A._visible

        def strict(qp, n, causal):
            vis = orig(qp, n, causal)
            if causal:
                vis = vis & (np.arange(n)[None, :] < np.asarray(qp)[:, None])
                vis[:, 0] |= True    # keep rows non-empty
            return vis
        monkeypatch.setattr(A, "_visible", strict)
    else:
        orig_sm = A._two_pass_softmax

        def bad(s, visible):
            P, lse = orig_sm(s, visible)
            if mutation == "log10_lse":
                m = np.where(visible, s, -np.inf).max(-1)
                lse = m + (lse - m) / math.log(10)
            elif mutation == "shifted_scale_sign":
                P2, _ = orig_sm(-s, visible)
                P = P2
            elif mutation == "unnormalised":
                m = np.where(visible, s, -np.inf).max(-1, keepdims=True)
                P = np.where(visible, np.exp(s - m), 0.0)
            return P, lse
        monkeypatch.setattr(A, "_two_pass_softmax", bad)
    assert not _pins_hold(), f"planted mistake {mutation} not caught"


# ------------------------------------------------------- ragged batch prefill

def _pack(blocks):
    return np.concatenate([b.reshape(-1) for b in blocks]) if blocks else \
        np.zeros(0)


def test_varlen_equal_lengths_equals_the_dense_batch():
    # all S_b equal: the packed layout of [B, H, S, D] is the dense layout
    B, Hq, Hkv, S, D = 3, 4, 2, 9, 8
    q, k, v = prefill_np(B, Hq, Hkv, S, D, seed=21)
    cu = np.arange(B + 1) * S
    o, lse = oracle.prefill_varlen(q, k, v, cu, Hq, Hkv, 0.3, True)
    ro, rl = oracle.prefill(q, k, v, 0.3, True)
    assert np.abs(o - ro.reshape(-1)).max() < TOL
    assert np.abs(lse - rl.reshape(-1)).max() < TOL


def test_varlen_sequences_do_not_see_each_other():
    # each block equals the prefill of that sequence alone, and changing
    # one sequence's values leaves the others' results unchanged
    Hq, Hkv, D = 2, 1, 8
    lens = [5, 0, 1, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    rng = np.random.default_rng(22)
    qs = [rng.standard_normal((Hq, L, D)) for L in lens]
    ks = [rng.standard_normal((Hkv, L, D)) for L in lens]
    vs = [rng.standard_normal((Hkv, L, D)) for L in lens]
    o, lse = oracle.prefill_varlen(_pack(qs), _pack(ks), _pack(vs), cu, Hq,
                                   Hkv, 0.5, True)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        ro, rl = oracle.prefill(qs[b][None], ks[b][None], vs[b][None], 0.5,
                                True)
        assert np.abs(o[Hq * D * cu[b]: Hq * D * cu[b + 1]] -
                      ro.reshape(-1)).max() < TOL
        assert np.abs(lse[Hq * cu[b]: Hq * cu[b + 1]] - rl.reshape(-1)).max() \
            < TOL
    ks2 = [x.copy() for x in ks]
    ks2[3] = ks2[3] * 5.0
    o2, _ = oracle.prefill_varlen(_pack(qs), _pack(ks2), _pack(vs), cu, Hq,
                                  Hkv, 0.5, True)
    keep = slice(0, Hq * D * cu[3])
    assert np.abs(o2[keep] - o[keep]).max() == 0.0


def test_varlen_causal_first_row_is_v0_of_its_own_sequence():
    # the first token of every sequence sees only itself: o = its own v0
    Hq, Hkv, D = 1, 1, 4
    lens = [3, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    rng = np.random.default_rng(23)
    q = rng.standard_normal(sum(lens) * D)
    k = rng.standard_normal(sum(lens) * D)
    v = rng.standard_normal(sum(lens) * D)
    o, _ = oracle.prefill_varlen(q, k, v, cu, Hq, Hkv, 1.0, True)
    for b in range(2):
        r = cu[b] * D
        assert np.abs(o[r: r + D] - v[r: r + D]).max() < TOL


# ------------------------------------------------------------ padded batch

def test_padded_full_lengths_equal_the_dense_batch():
    B, Hq, Hkv, S, D = 2, 4, 2, 9, 8
    q, k, v = prefill_np(B, Hq, Hkv, S, D, seed=24)
    for causal in (True, False):
        o, lse = oracle.prefill_padded(q, k, v, [S, S + 3], 0.3, causal)
        ro, rl = oracle.prefill(q, k, v, 0.3, causal)
        assert np.abs(o - ro).max() < TOL and np.abs(lse - rl).max() < TOL


def test_padded_causal_rows_equal_dense_causal_rows():
    # under the causal mask a valid row i < L never sees a key past i, so
    # it already ignores the padding: the dense causal prefill of the whole
    # padded tensors gives the same valid rows (no slicing involved)
    B, Hq, Hkv, S, D = 3, 2, 1, 11, 8
    q, k, v = prefill_np(B, Hq, Hkv, S, D, seed=25)
    lens = [4, 11, 1]
    o, lse = oracle.prefill_padded(q, k, v, lens, 0.4, True)
    ro, rl = oracle.prefill(q, k, v, 0.4, True)
    for b, L in enumerate(lens):
        assert np.abs(o[b, :, :L] - ro[b, :, :L]).max() < TOL
        assert np.abs(lse[b, :, :L] - rl[b, :, :L]).max() < TOL


def test_padded_rows_and_content():
    # padding rows are o = 0, lse = -inf; what the padding holds does not
    # change any valid row (keys past L_b are masked even without causality)
    B, Hq, Hkv, S, D = 3, 2, 2, 7, 4
    q, k, v = prefill_np(B, Hq, Hkv, S, D, seed=26)
    lens = [0, 3, 7]
    for causal in (True, False):
        o, lse = oracle.prefill_padded(q, k, v, lens, 0.5, causal)
        q2, k2, v2 = (x.copy() for x in (q, k, v))
        for b, L in enumerate(lens):
            for t in (q2, k2, v2):
                t[b, :, L:] = 1e3
        o2, lse2 = oracle.prefill_padded(q2, k2, v2, lens, 0.5, causal)
        for b, L in enumerate(lens):
            assert (o[b, :, L:] == 0).all() and (lse[b, :, L:] == -np.inf).all()
            assert np.array_equal(o2[b, :, :L], o[b, :, :L])
            assert np.array_equal(lse2[b, :, :L], lse[b, :, :L])


# ---------------------------------------- per-key-prefix softmax state (trace)

def test_prefix_state_full_prefix_equals_the_row_lse():
    q, k, v = prefill_np(2, 4, 2, 40, 16, seed=21)
    _, lse = oracle.prefill(q, k, v, 0.3, True)
    _, lse_f = oracle.prefill(q, k, v, 0.3, False)
    for b, h, row in [(0, 0, 0), (1, 3, 17), (0, 2, 39)]:
        m, l = oracle.prefix_softmax_state(q, k, 0.3, True, b, h, row,
                                           [row + 1, 40])
        np.testing.assert_allclose(l, lse[b, h, row], atol=TOL)
        _, lf = oracle.prefix_softmax_state(q, k, 0.3, False, b, h, row,
                                            [40])
        np.testing.assert_allclose(lf, lse_f[b, h, row], atol=TOL)


def test_prefix_state_first_key_and_empty_prefix():
    q, k, _ = prefill_np(1, 4, 2, 12, 8, seed=22)
    for h in range(4):
        m, l = oracle.prefix_softmax_state(q, k, 0.5, True, 0, h, 7, [0, 1])
        s0 = 0.5 * q[0, h, 7] @ k[0, h // 2, 0]
        assert m[0] == -np.inf and l[0] == -np.inf
        np.testing.assert_allclose([m[1], l[1]], [s0, s0], atol=TOL)


def test_prefix_state_identical_keys_closed_form():
    q, k, _ = prefill_np(1, 2, 1, 20, 8, seed=23)
    k[:] = k[:, :, :1, :]
    n = np.arange(1, 21)
    for causal in (True, False):
        m, l = oracle.prefix_softmax_state(q, k, 0.2, causal, 0, 1, 9, n)
        s = 0.2 * q[0, 1, 9] @ k[0, 0, 0]
        seen = np.minimum(n, 10) if causal else n
        np.testing.assert_allclose(m, s, atol=TOL)
        np.testing.assert_allclose(l, s + np.log(seen), atol=TOL)


def test_prefix_state_brute_force():
    q, k, _ = prefill_np(1, 2, 2, 9, 4, seed=24)
    row = 6
    m, l = oracle.prefix_softmax_state(q, k, 0.7, True, 0, 1, row,
                                       range(10))
    for n in range(10):
        ss = [0.7 * sum(q[0, 1, row, d] * k[0, 1, j, d] for d in range(4))
              for j in range(min(n, row + 1))]
        if not ss:
            assert m[n] == -np.inf and l[n] == -np.inf
            continue
        mx = max(ss)
        assert abs(m[n] - mx) <= TOL
        assert abs(l[n] - (mx + math.log(sum(math.exp(x - mx)
                                                for x in ss)))) <= TOL
