"""Pins of the residual-add + RMSNorm epilogue oracle (oracle/epilogue.py).

The epilogue follows the "triton-optimization" skill page, section 3.2:
x = row + residual, y = x / sqrt(mean(x^2) + eps) * w, x written back as the
new residual; "第 6 讲：核函数与 Triton" section 9.1 gives the same forward.
Each test checks the oracle against a closed form, an invariant fixed by the
mathematics, pure-Python scalar loops on tiny inputs, or torch's own
rms_norm in float64; the last group plants plausible mistakes in the oracle
(eps outside the root, a sum for the mean, no weight, no residual, the root
not inverted) and checks that some pin catches each one.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import epilogue as E

TOL = 1e-12


def rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def test_two_value_row_closed_form():
    # x = (3, 4): mean of squares 12.5, so y = x / sqrt(12.5 + eps) * w
    o = np.array([[3.0, 4.0]])
    for eps in (0.0, 1e-6, 0.5):
        y, x = E.residual_rmsnorm(o, np.zeros_like(o), np.array([1.0, 2.0]),
                                  eps)
        r = 1.0 / math.sqrt(12.5 + eps)
        np.testing.assert_allclose(y, [[3.0 * r, 8.0 * r]], atol=TOL)
        np.testing.assert_array_equal(x, o)
    y, _ = E.residual_rmsnorm(o, np.zeros_like(o), np.ones(2), 0.0)
    np.testing.assert_allclose(y, [[3.0 * math.sqrt(2) / 5,
                                    4.0 * math.sqrt(2) / 5]], atol=TOL)


@pytest.mark.parametrize("c", [2.5, -0.125, 7.0])
def test_constant_row_gives_sign_times_weight(c):
    D = 16
    w = rand(D, 1)
    y, _ = E.residual_rmsnorm(np.full((3, D), c), np.zeros((3, D)), w, 0.0)
    np.testing.assert_allclose(y, np.sign(c) * np.broadcast_to(w, (3, D)),
                               atol=TOL)


def test_unit_weight_rows_have_unit_mean_square():
    o = rand((2, 3, 5, 64), 2)
    res = rand((2, 3, 5, 64), 3, 0.3)
    y, _ = E.residual_rmsnorm(o, res, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, atol=TOL)
    # with eps: mean(y^2) = ms / (ms + eps) for each row
    eps = 0.7
    y, x = E.residual_rmsnorm(o, res, np.ones(64), eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + eps),
                               atol=TOL)


def test_scale_and_sign_invariance_without_eps():
    o = rand((4, 32), 4)
    w = rand(32, 5)
    z = np.zeros_like(o)
    y, _ = E.residual_rmsnorm(o, z, w, 0.0)
    y3, _ = E.residual_rmsnorm(3.0 * o, z, w, 0.0)
    yn, _ = E.residual_rmsnorm(-o, z, w, 0.0)
    np.testing.assert_allclose(y3, y, atol=TOL)
    np.testing.assert_allclose(yn, -y, atol=TOL)


def test_weight_scales_columns():
    o = rand((6, 8), 6)
    w = rand(8, 7)
    z = np.zeros_like(o)
    y1, _ = E.residual_rmsnorm(o, z, np.ones(8), 1e-6)
    yw, _ = E.residual_rmsnorm(o, z, w, 1e-6)
    np.testing.assert_allclose(yw, y1 * w, atol=TOL)


def test_residual_is_added_and_returned():
    o = rand((3, 16), 8)
    res = rand((3, 16), 9)
    y, x = E.residual_rmsnorm(o, res, np.ones(16), 1e-6)
    np.testing.assert_array_equal(x, o + res)
    # swapping the two addends changes nothing
    y2, x2 = E.residual_rmsnorm(res, o, np.ones(16), 1e-6)
    np.testing.assert_allclose(y2, y, atol=TOL)
    np.testing.assert_allclose(x2, x, atol=TOL)


def brute_force(o, res, w, eps):
    """Pure-Python scalar loops over the rows of 2-D lists."""
    ys, xs = [], []
    for orow, rrow in zip(o, res):
        x = [a + b for a, b in zip(orow, rrow)]
        ms = 0.0
        for t in x:
            ms += t * t
        ms /= len(x)
        inv = 1.0 / math.sqrt(ms + eps)
        ys.append([t * inv * wi for t, wi in zip(x, w)])
        xs.append(x)
    return ys, xs


@pytest.mark.parametrize("R,D,eps", [(1, 1, 0.0), (3, 5, 1e-6), (4, 8, 0.3)])
def test_brute_force(R, D, eps):
    o = rand((R, D), 10 + D)
    res = rand((R, D), 20 + D)
    w = rand(D, 30 + D)
    y, x = E.residual_rmsnorm(o, res, w, eps)
    yb, xb = brute_force(o.tolist(), res.tolist(), w.tolist(), eps)
    np.testing.assert_allclose(y, np.array(yb), atol=TOL)
    np.testing.assert_allclose(x, np.array(xb), atol=TOL)


@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_matches_torch_rms_norm_float64(eps):
    o = rand((2, 4, 33, 128), 11)
    res = rand((2, 4, 33, 128), 12, 2.0)
    w = rand(128, 13)
    y, x = E.residual_rmsnorm(o, res, w, eps)
    want = torch.nn.functional.rms_norm(
        torch.from_numpy(o + res), (128,), weight=torch.from_numpy(w),
        eps=eps).numpy()
    np.testing.assert_allclose(y, want, atol=1e-10)


def test_zero_values_normalise_the_residual_alone():
    # v = 0 makes the attention output 0, so y = RMSNorm(residual)
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 4, 9, 8))
    k = rng.standard_normal((1, 2, 9, 8))
    v = np.zeros((1, 2, 9, 8))
    res = rng.standard_normal((1, 4, 9, 8))
    w = rng.standard_normal(8)
    y, x, _ = oracle.prefill_residual_rmsnorm(q, k, v, res, w, 0.3, True,
                                              1e-6)
    ms = np.mean(res * res, axis=-1, keepdims=True)
    np.testing.assert_allclose(y, res / np.sqrt(ms + 1e-6) * w, atol=TOL)
    np.testing.assert_allclose(x, res, atol=TOL)


def test_causal_row0_normalises_v0():
    # causal row 0 sees only key 0, so o_0 = v_0 and y_0 = RMSNorm(v_0 + r_0)
    rng = np.random.default_rng(15)
    q = rng.standard_normal((2, 4, 7, 16))
    k = rng.standard_normal((2, 2, 7, 16))
    v = rng.standard_normal((2, 2, 7, 16))
    res = rng.standard_normal((2, 4, 7, 16))
    w = rng.standard_normal(16)
    y, x, lse = oracle.prefill_residual_rmsnorm(q, k, v, res, w, 0.25, True,
                                                0.0)
    for b in range(2):
        for h in range(4):
            x0 = v[b, h // 2, 0] + res[b, h, 0]
            want = x0 / math.sqrt(np.mean(x0 * x0)) * w
            np.testing.assert_allclose(y[b, h, 0], want, atol=TOL)
            np.testing.assert_allclose(x[b, h, 0], x0, atol=TOL)
            # the epilogue leaves the LSE alone: row 0's is scale * q0.k0
            np.testing.assert_allclose(
                lse[b, h, 0], 0.25 * q[b, h, 0] @ k[b, h // 2, 0], atol=TOL)


# -------------------------------------------- planted mistakes must be caught

def _pins_hold():
    checks = [
        test_two_value_row_closed_form,
        lambda: test_constant_row_gives_sign_times_weight(-0.125),
        test_unit_weight_rows_have_unit_mean_square,
        test_weight_scales_columns,
        test_residual_is_added_and_returned,
        lambda: test_brute_force(3, 5, 1e-6),
        lambda: test_matches_torch_rms_norm_float64(1e-2),
        test_zero_values_normalise_the_residual_alone,
        test_causal_row0_normalises_v0,
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_pins_pass_on_unmodified_oracle():
    assert _pins_hold()


def _mutant(kind):
    def f(o, residual, weight, eps):
        o = np.asarray(o, dtype=np.float64)
        residual = np.asarray(residual, dtype=np.float64)
        weight = np.asarray(weight, dtype=np.float64)
        x = o if kind == "no_residual" else o + residual
        if kind == "sum_not_mean":
            ms = np.sum(x * x, axis=-1, keepdims=True)
        else:
            ms = np.mean(x * x, axis=-1, keepdims=True)
        if kind == "eps_outside_root":
            r = 1.0 / (np.sqrt(ms) + eps)
        elif kind == "root_not_inverted":
            r = np.sqrt(ms + eps)
        else:
            r = 1.0 / np.sqrt(ms + eps)
        y = x * r if kind == "no_weight" else x * r * weight
        return y, x
    return f


@pytest.mark.parametrize("kind", ["no_residual", "sum_not_mean",
                                  "eps_outside_root", "root_not_inverted",
                                  "no_weight"])
def test_planted_mistake_is_caught(monkeypatch, kind):
    monkeypatch.setattr(E, "residual_rmsnorm", _mutant(kind))
    assert not _pins_hold(), f"planted mistake {kind} not caught"
