"""fp64 reference rotary position embedding (RoPE).

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
HIP path.

What it computes ("triton-optimization" skill page, section 3.4, fused RoPE):
each head vector x of length D is split into halves x1 = x[:D/2] and
x2 = x[D/2:], and pair i = (x1[i], x2[i]) is rotated by an angle theta_i:
x1' = x1 cos(theta) - x2 sin(theta), x2' = x1 sin(theta) + x2 cos(theta).
The page reads cos and sin from a table indexed by (position, i); the
Qwen3.5-0.8B page (section 1.2) computes them in fp32 while q and k are
loaded.  Neither page prints the angle itself, so this takes the standard
definition theta_i(p) = p * base^(-2 i / D), with the base from the caller.
"""

import numpy as np


def _angles(positions, D, base):
    """theta[..., i] = p * base^(-2 i / D) for the D/2 pairs."""
    i = np.arange(D // 2, dtype=np.float64)
    rate = np.float64(base) ** (-2.0 * i / D)
    return np.asarray(positions, dtype=np.float64)[..., None] * rate


def _pairs(D):
    """Indices of the two members of each rotated pair: (i, i + D/2)."""
    first = np.arange(D // 2)
    return first, first + D // 2


def _rotate(x1, x2, c, s):
    return x1 * c - x2 * s, x1 * s + x2 * c


def rope(x, positions, base):
    """Rotate the last axis of x (length D, even) at the given positions.

    ``positions`` broadcasts against x.shape[:-1] (e.g. shape [S] for x of
    shape [B, H, S, D]).  Returns a new float64 array.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    theta = _angles(positions, D, base)
    c, s = np.cos(theta), np.sin(theta)
    a, b = _pairs(D)
    y = x.copy()
    y[..., a], y[..., b] = _rotate(x[..., a], x[..., b], c, s)
    return y
