"""Pins of the fp64 RoPE oracle against facts that do not come from it.

Closed forms (position 0 is the identity; one pair is a plane rotation by
p radians; a D = 4 example worked by hand fixes which members form a pair
and the 2i/D exponent), invariants of rotations (pair norms kept, rotations
compose by adding positions, scores depend only on the position difference),
and planted mistakes (interleaved pairing, reversed rotation, a wrong
exponent), each of which must fail one of the pins.

Source: "triton-optimization" skill page, section 3.4 (fused RoPE), and the
Qwen3.5-0.8B page, section 1.2 (RoPE applied while q and k are loaded).
"""

import math

import numpy as np
import pytest

import oracle
from oracle import rotary as R

TOL = 1e-12


def test_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((3, 5, 64))
    assert np.abs(oracle.rope(x, 0, 10000.0) - x).max() == 0.0


@pytest.mark.parametrize("p", [1, 2, 7, 1000])
def test_one_pair_is_a_plane_rotation_by_p_radians(p):
    # D = 2: a single pair with rate base^0 = 1, so the angle is p radians
    e1 = oracle.rope(np.array([1.0, 0.0]), p, 10000.0)
    e2 = oracle.rope(np.array([0.0, 1.0]), p, 10000.0)
    assert abs(e1[0] - math.cos(p)) < TOL and abs(e1[1] - math.sin(p)) < TOL
    assert abs(e2[0] + math.sin(p)) < TOL and abs(e2[1] - math.cos(p)) < TOL


def test_d4_worked_example():
    # D = 4, base 100, position 1: pairs (0, 2) and (1, 3); pair 0 turns by
    # 1 radian, pair 1 by 100^(-2/4) = 0.1 radian
    y0 = oracle.rope(np.array([1.0, 0.0, 0.0, 0.0]), 1, 100.0)
    y1 = oracle.rope(np.array([0.0, 1.0, 0.0, 0.0]), 1, 100.0)
    assert np.abs(y0 - [math.cos(1.0), 0.0, math.sin(1.0), 0.0]).max() < TOL
    assert np.abs(y1 - [0.0, math.cos(0.1), 0.0, math.sin(0.1)]).max() < TOL


def test_pair_norms_are_kept():
    x = np.random.default_rng(1).standard_normal((4, 128))
    y = oracle.rope(x, np.arange(4) * 977, 10000.0)
    n = lambda z: z[..., :64] ** 2 + z[..., 64:] ** 2
    assert np.abs(n(y) - n(x)).max() < 1e-10


def test_rotations_compose_by_adding_positions():
    x = np.random.default_rng(2).standard_normal((6, 64))
    a, b = np.arange(6) * 13, np.arange(6) * 101 + 5
    y = oracle.rope(oracle.rope(x, a, 500.0), b, 500.0)
    assert np.abs(y - oracle.rope(x, a + b, 500.0)).max() < 1e-10


def test_scores_depend_only_on_the_position_difference():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    s = lambda m, n: oracle.rope(q, m, 10000.0) @ oracle.rope(k, n, 10000.0)
    for m, n, t in [(5, 2, 100), (0, 0, 31), (700, 9, 4096)]:
        assert abs(s(m, n) - s(m + t, n + t)) < 1e-9


def _pins_hold():
    try:
        for p in [1, 7]:
            test_one_pair_is_a_plane_rotation_by_p_radians(p)
        test_position_zero_is_identity()
        test_d4_worked_example()
        test_pair_norms_are_kept()
        test_rotations_compose_by_adding_positions()
        test_scores_depend_only_on_the_position_difference()
    except AssertionError:
        return False
    return True


def test_pins_hold_for_the_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("mutation", ["interleaved", "reversed", "exponent"])
def test_planted_mistake_is_caught(monkeypatch, mutation):
    if mutation == "interleaved":
        monkeypatch.setattr(R, "_pairs",
                            lambda D: (np.arange(0, D, 2), np.arange(1, D, 2)))
    elif mutation == "reversed":
        monkeypatch.setattr(R, "_rotate",
                            lambda x1, x2, c, s: (x1 * c + x2 * s,
                                                  -x1 * s + x2 * c))
    else:
        def wrong(positions, D, base):
            i = np.arange(D // 2, dtype=np.float64)
            return np.asarray(positions, np.float64)[..., None] * \
                np.float64(base) ** (-i / D)
        monkeypatch.setattr(R, "_angles", wrong)
    assert not _pins_hold(), f"planted mistake {mutation} not caught"
