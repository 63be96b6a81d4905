"""The debug build's per-tile softmax trace against the oracle's prefix state.

The attention-fusion page (section 6.3) debugs its fused kernel by printing
the running m_i and l_i after every key block and comparing them with the
reference's values at the same positions.  libattn_debug.so records that
state for one chosen row after every key tile (include/attn_debug.h); here
each record is checked against oracle.prefix_softmax_state at the same key
count: m + ln l must be the log-sum-exp of the scores seen so far (to the
LSE tolerance, 1e-3), and the kernel's reference max m must lie within the
lazy-rescale band below the running max (at most 2^8 in the exp2 domain, so
8 ln 2 in natural-log units).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from causal_attention_amd import debug, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BAND = 8 * math.log(2)


def say(*a):
    print(*a, flush=True)


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def traced(B, Hq, Hkv, S, D, dtype, causal, targets, seed=0, tile=64,
           lse_tol=1e-3):
    say(f"[trace] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} {dtype} "
        f"causal={causal} targets={targets}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, dtype, 1.0, seed)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = 1.0 / math.sqrt(D)
    for b, h, row in targets:
        o, lse, rec = debug.trace_prefill(qd, kd, vd, b, h, row,
                                          causal=causal, scale=scale)
        keys = rec[:, 0].astype(np.int64)
        # one record per tile the kernel ran for this row's workgroup
        t = np.arange(len(rec))
        if dtype != "f32":
            rows_end = min(S, (row // 128 + 1) * 128) if causal else S
            assert len(rec) == -(-rows_end // tile)
        np.testing.assert_array_equal(keys, np.minimum((t + 1) * tile, S)
                                      if dtype != "f32" else keys)
        assert (np.diff(keys) > 0).all()
        rm, rl = oracle.prefix_softmax_state(np64(q), np64(k), scale, causal,
                                             b, h, row, keys)
        m, l = rec[:, 1], rec[:, 2]
        got = m + np.log(l)
        err = np.abs(got - rl).max()
        say(f"   ({b},{h},{row}): {len(rec)} records, "
            f"max|d lse_prefix|={err:.3e}")
        assert err <= lse_tol
        assert (m <= rm + lse_tol).all()
        assert (m >= rm - BAND - lse_tol).all()
        # the last record is the row's final state: the kernel's own LSE
        assert abs(got[-1] - float(lse[b, h, row])) <= 1e-5 * max(
            1.0, abs(got[-1]))


def test_trace_bf16_causal_gqa():
    traced(1, 8, 2, 300, 128, "bf16", True,
           [(0, 0, 0), (0, 5, 63), (0, 5, 64), (0, 2, 200), (0, 7, 299)])


def test_trace_bf16_full_d64():
    traced(2, 4, 4, 200, 64, "bf16", False, [(1, 3, 0), (0, 1, 150)])


def test_trace_f16_causal():
    traced(1, 4, 1, 260, 128, "f16", True, [(0, 2, 259), (0, 0, 130)])


def test_trace_f32_single_head():
    # the fp32 kernel skips the tiles wholly above a wave's rows, so records
    # cover 32-key tiles up to the wave's last row
    traced(1, 1, 1, 128, 64, "f32", True, [(0, 0, 0), (0, 0, 77),
                                           (0, 0, 127)], tile=32,
           lse_tol=1e-5)


def test_trace_locates_a_wrong_mask():
    """The page's use of the trace: compared with a reference that has a
    mistake (here, the causal mask left out, planted in the reference on the
    CPU), the records agree up to the tile before the row's diagonal and
    disagree from the diagonal tile on, which names where the two depart."""
    B, Hq, Hkv, S, D = 1, 2, 1, 256, 64
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, D, "bf16", 1.0, 5)
    row = 150
    _, _, rec = debug.trace_prefill(q.to(DEV), k.to(DEV), v.to(DEV), 0, 1,
                                    row, causal=True)
    keys = rec[:, 0].astype(np.int64)
    _, wrong = oracle.prefix_softmax_state(np64(q), np64(k), 1 / 8, False,
                                           0, 1, row, keys)
    bad = np.abs(rec[:, 1] + np.log(rec[:, 2]) - wrong) > 1e-3
    first = int(np.argmax(bad))
    assert bad.any() and not bad[:first].any()
    assert keys[first] > row and (first == 0 or keys[first - 1] <= row)
