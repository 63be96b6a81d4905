"""Host-side checks of the seeded input generators (no GPU)."""

import numpy as np
import torch

from causal_attention_amd import inputs

# Cache lengths of the 32-sequence decode batch drawn from seed 0
# (uniform on [256, 4096]); the sum is the KV-token count the decode
# throughput is priced on.
SEQLENS_SEED0 = [3523, 2702, 2219, 1292, 1438, 413, 544, 319, 929, 3379, 2750,
                 3761, 2190, 2586, 3984, 3057, 2684, 2344, 2406, 3847, 1321,
                 3389, 2832, 266, 1769, 3549, 2385, 385, 3193, 3058, 3507, 930]


def test_decode_seqlens_seed0():
    w = inputs.WORKLOADS["c4_decode_b32"]
    s = inputs.decode_seqlens(w.B, w.lmin, w.lmax, w.seed)
    assert s.tolist() == SEQLENS_SEED0
    assert int(s.sum()) == 72951
    s2, q, k, v = inputs.workload_inputs(w)
    assert s2.tolist() == SEQLENS_SEED0
    assert k.numel() == 2 * 128 * 72951 and v.numel() == k.numel()
    assert q.shape == (32, 8, 128) and q.dtype == torch.bfloat16


def test_generators_are_deterministic():
    a = inputs.prefill_inputs(1, 2, 1, 33, 64, "bf16", 1.0, seed=5)
    b = inputs.prefill_inputs(1, 2, 1, 33, 64, "bf16", 1.0, seed=5)
    c = inputs.prefill_inputs(1, 2, 1, 33, 64, "bf16", 1.0, seed=6)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])


def _rne_bf16(x):
    """Round fp32 to bf16 by bit manipulation, ties to even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.random.default_rng(1).standard_normal(10000).astype(np.float32)
    # exact ties: low 16 bits == 0x8000
    ties = (np.arange(64, dtype=np.uint32) << 16 | 0x3F800000 | 0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    got = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, _rne_bf16(x))


def test_sigma_and_shapes():
    w = inputs.WORKLOADS["c5_gqa_s32768"]
    assert w.sigma == 0.5 and w.S == 32768 and (w.Hq, w.Hkv, w.D) == (8, 2, 128)
    q, k, v = inputs.prefill_inputs(1, 8, 2, 256, 128, "bf16", 0.5, seed=0)
    assert abs(float(q.float().std()) - 0.5) < 0.01
    assert k.shape == (1, 2, 256, 128)


def test_sampled_rows():
    r = inputs.sampled_rows(8, 32768, 256)
    assert r.shape == (8, 256)
    for h in range(8):
        assert len(set(r[h].tolist())) == 256
        assert {0, 127, 128, 32767} <= set(r[h].tolist())
    assert np.array_equal(r, inputs.sampled_rows(8, 32768, 256))
    assert not np.array_equal(r[0], r[1])


def test_pack_unpack_roundtrip():
    seqlens, q, k, v = inputs.decode_inputs(3, 4, 2, 8, seqlens=[2, 0, 5])
    blocks = inputs.unpack_kv(k, seqlens, 2, 8)
    assert [b.shape[1] for b in blocks] == [2, 0, 5]
    assert torch.equal(inputs.pack_kv(blocks), k)
