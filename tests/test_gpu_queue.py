"""GPU tests of the register-blocked prefill's tile queue (causal launches of
several rounds of workgroups given a workspace; each workgroup takes its
query tile from a counter in the workspace, heaviest first).

The queue changes only which workgroup computes a tile, never the tile's
arithmetic, so its output must equal the launch without a workspace bit for
bit; it is also checked against the fp64 oracle (bounds as in
test_gpu_parity: 2e-2 bf16, 5e-3 fp16, 1e-3 on the LSE), across calls of
different sizes on one workspace (the counter must come back to zero), and
replayed from a captured graph.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from causal_attention_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 2e-2, "f16": 5e-3}
LSE_TOL = 1e-3

# (B, Hq, Hkv, S): more register-blocked workgroups (B (Hq/4) ceil(S/64))
# than the 256 compute units, ragged query tails included
SHAPES = [(9, 8, 2, 1000), (20, 8, 2, 513), (5, 12, 3, 1100)]


def say(*a):
    print(*a, flush=True)


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture
def forced_rb():
    prev = attn.prefill_select(attn.PREFILL_RB)
    prev_ws = attn.prefill_workspace_policy(True)
    yield
    attn.prefill_select(prev)
    attn.prefill_workspace_policy(prev_ws)


def load(B, Hq, Hkv, S, dtype, seed):
    return [t.to(DEV) for t in inputs.prefill_inputs(B, Hq, Hkv, S, 128,
                                                     dtype, 1.0, seed)]


def static_run(q, k, v):
    prev = attn.prefill_workspace_policy(False)
    try:
        return attn.attn_prefill(q, k, v, causal=True)
    finally:
        attn.prefill_workspace_policy(prev)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,Hq,Hkv,S", SHAPES)
@pytest.mark.usefixtures("forced_rb")
def test_queue_matches_oracle_and_static_order(B, Hq, Hkv, S, dtype):
    say(f"[queue] B={B} Hq={Hq} Hkv={Hkv} S={S} D=128 {dtype}")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert B * (Hq // 4) * -(-S // 64) > n_cu
    assert attn.prefill_schedule(B, Hq, Hkv, S, 128) == attn.SCHEDULE_QUEUE
    q, k, v = load(B, Hq, Hkv, S, dtype, 3)
    ws = attn.new_prefill_workspace(B, Hq, Hkv, S, 128, device=DEV)
    assert ws.numel() == 4096
    o, lse = attn.attn_prefill(q, k, v, causal=True, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].count_nonzero()) == 0       # counter back to zero
    so, sl = static_run(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, so) and torch.equal(lse, sl)
    ro, rl = oracle.prefill(np64(q), np64(k), np64(v), 1 / math.sqrt(128),
                            True)
    eo = np.abs(np64(o) - ro).max()
    el = np.abs(lse.cpu().numpy() - rl).max()
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL[dtype] and el <= LSE_TOL


@pytest.mark.usefixtures("forced_rb")
def test_queue_workspace_shared_by_calls_of_different_sizes():
    """One workspace through queue launches of three grid sizes, a balanced
    launch and a launch with no schedule, twice over: every queue result
    equals the static order's, and the first 4 KB end zero each time."""
    ws = attn.new_prefill_workspace(4, 8, 2, 2048, 128, device=DEV)
    runs = [(9, 8, 2, 1000), (4, 8, 2, 2048), (20, 8, 2, 513),
            (2, 8, 2, 300), (5, 12, 3, 1100)]
    for rep in range(2):
        for i, (B, Hq, Hkv, S) in enumerate(runs):
            say(f"[queue shared ws] rep {rep} B={B} Hq={Hq} Hkv={Hkv} S={S} "
                f"schedule={attn.prefill_schedule(B, Hq, Hkv, S, 128)}")
            assert ws.numel() >= attn.attn_prefill_workspace_size(
                B, Hq, Hkv, S, 128)
            q, k, v = load(B, Hq, Hkv, S, "bf16", 10 * rep + i)
            o, lse = attn.attn_prefill(q, k, v, causal=True, workspace=ws)
            torch.cuda.synchronize()
            assert int(ws[:4096].count_nonzero()) == 0
            if attn.prefill_schedule(B, Hq, Hkv, S, 128) == \
                    attn.SCHEDULE_QUEUE:
                so, sl = static_run(q, k, v)
                torch.cuda.synchronize()
                assert torch.equal(o, so) and torch.equal(lse, sl)


def test_queue_under_the_automatic_choice():
    """B2, 8/2 heads, S = 8192: the table picks the register-blocked kernel
    and 512 workgroups, so a workspace brings the queue; sampled rows
    against the oracle and the whole output against the static order."""
    B, Hq, Hkv, S = 2, 8, 2, 8192
    prev = attn.prefill_select(attn.PREFILL_AUTO)
    prev_ws = attn.prefill_workspace_policy(True)
    try:
        say(f"[queue auto] B={B} Hq={Hq} Hkv={Hkv} S={S}")
        assert attn.prefill_schedule(B, Hq, Hkv, S, 128) == \
            attn.SCHEDULE_QUEUE
        q, k, v = load(B, Hq, Hkv, S, "bf16", 7)
        o, lse = attn.attn_prefill(q, k, v, causal=True)
        so, sl = static_run(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, so) and torch.equal(lse, sl)
        rows = inputs.sampled_rows(Hq, S, 8)
        ro, rl = oracle.prefill_rows(np64(q), np64(k), np64(v),
                                     1 / math.sqrt(128), True, rows)
        oc, lc = o.cpu(), lse.cpu()
        go = np.stack([np64(oc[:, h, rows[h]]) for h in range(Hq)], axis=1)
        gl = np.stack([lc[:, h, rows[h]].numpy() for h in range(Hq)], axis=1)
        eo, el = np.abs(go - ro).max(), np.abs(gl - rl).max()
        say(f"   sampled rows: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL["bf16"] and el <= LSE_TOL
    finally:
        attn.prefill_select(prev)
        attn.prefill_workspace_policy(prev_ws)


@pytest.mark.usefixtures("forced_rb")
def test_queue_graph_replay():
    """A queue launch captured in a graph and replayed with new inputs, with
    eager launches in between: each replay equals the static order bit for
    bit and matches the oracle, and the counter is zero after each."""
    B, Hq, Hkv, S = 9, 8, 2, 1000
    say(f"[queue graph] B={B} Hq={Hq} Hkv={Hkv} S={S}")
    q = torch.empty(B, Hq, S, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.empty(B, Hkv, S, 128, dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, S, dtype=torch.float32, device=DEV)
    ws = attn.new_prefill_workspace(B, Hq, Hkv, S, 128, device=DEV)

    def fill(seed):
        for dst, src in zip((q, k, v), load(B, Hq, Hkv, S, "bf16", seed)):
            dst.copy_(src)

    fill(30)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        attn.attn_prefill(q, k, v, out=o, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn.attn_prefill(q, k, v, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for t in range(3):
        fill(31 + t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(ws[:4].count_nonzero()) == 0
        so, sl = static_run(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, so) and torch.equal(lse, sl)
        ro, rl = oracle.prefill(np64(q), np64(k), np64(v),
                                1 / math.sqrt(128), True)
        err = np.abs(np64(o) - ro).max()
        say(f"   replay {t}: max|dO|={err:.3e}")
        assert err <= TOL["bf16"]
        assert np.abs(lse.cpu().numpy() - rl).max() <= LSE_TOL


@pytest.mark.usefixtures("forced_rb")
def test_queue_with_a_counter_left_nonzero():
    """A workspace whose counter was not zeroed (5: below the block count,
    so the reset happens mid-launch; 12345: above it, so it never does)
    still gives every tile to exactly one workgroup: the output equals the
    static order's bit for bit, on two calls in a row."""
    B, Hq, Hkv, S = 9, 8, 2, 1000          # 288 workgroups
    q, k, v = load(B, Hq, Hkv, S, "bf16", 40)
    so, sl = static_run(q, k, v)
    for start in (5, 12345):
        ws = attn.new_prefill_workspace(B, Hq, Hkv, S, 128, device=DEV)
        ws[:8].copy_(torch.tensor([start], dtype=torch.int64).view(
            torch.uint8).to(DEV))
        for rep in range(2):
            say(f"[queue nonzero counter] start={start} rep={rep}")
            o, lse = attn.attn_prefill(q, k, v, causal=True, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(o, so) and torch.equal(lse, sl)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_queue_long_context_sampled(dtype):
    """The long-context shape (B1, 8/2 heads, S = 32768, 1024 workgroups)
    under the automatic choice, which runs the tile queue: sampled rows
    against the oracle, every row finite, and the whole output equal to the
    static order's."""
    B, Hq, Hkv, S = 1, 8, 2, 32768
    prev = attn.prefill_select(attn.PREFILL_AUTO)
    prev_ws = attn.prefill_workspace_policy(True)
    try:
        say(f"[queue long] B={B} Hq={Hq} Hkv={Hkv} S={S} {dtype}")
        assert attn.prefill_schedule(B, Hq, Hkv, S, 128) == \
            attn.SCHEDULE_QUEUE
        q, k, v = load(B, Hq, Hkv, S, dtype, 11)
        o, lse = attn.attn_prefill(q, k, v, causal=True)
        so, sl = static_run(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, so) and torch.equal(lse, sl)
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        rows = inputs.sampled_rows(Hq, S, 32)
        ro, rl = oracle.prefill_rows(np64(q), np64(k), np64(v),
                                     1 / math.sqrt(128), True, rows)
        oc, lc = o.cpu(), lse.cpu()
        go = np.stack([np64(oc[:, h, rows[h]]) for h in range(Hq)], axis=1)
        gl = np.stack([lc[:, h, rows[h]].numpy() for h in range(Hq)], axis=1)
        eo, el = np.abs(go - ro).max(), np.abs(gl - rl).max()
        say(f"   sampled rows: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL[dtype] and el <= LSE_TOL
    finally:
        attn.prefill_select(prev)
        attn.prefill_workspace_policy(prev_ws)
