"""attn_decode_noalloc: the decode entry point that allocates nothing (its
workspace is the library's device-resident array), against attn_decode with
a caller workspace and against the fp64 oracle.  Two calls in a row, the
second with a smaller input, so the second runs over the array as the first
left it."""

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from causal_attention_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def call_noalloc(q, kc, vc, sl, o, lse, Hkv, num_splits):
    """The C entry point directly (ctypes), with preallocated outputs."""
    B, Hq, D = q.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return attn.lib().attn_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
        ctypes.c_void_p(vc.data_ptr()), ctypes.c_void_p(sl.data_ptr()),
        ctypes.c_void_p(o.data_ptr()), B, Hq, Hkv, D, 1 / math.sqrt(D),
        num_splits, ctypes.c_void_p(lse.data_ptr()), stream)


@pytest.mark.parametrize("num_splits", [0, 7])
def test_noalloc_decode_matches_workspace_decode_twice(num_splits):
    cases = [(32, 8, 2, 128, None, 0),                      # the C4 batch
             (5, 8, 2, 128, [1, 300, 0, 77, 129], 3)]       # smaller input
    for B, Hq, Hkv, D, lens, seed in cases:
        print(f"[noalloc] B={B} Hq={Hq} Hkv={Hkv} D={D} lens={lens} "
              f"ns={num_splits}", flush=True)
        sl, q, kc, vc = inputs.decode_inputs(B, Hq, Hkv, D, seqlens=lens,
                                             seed=seed)
        qd, kd, vd = q.to(DEV), kc.to(DEV), vc.to(DEV)
        sd = torch.from_numpy(sl).to(DEV)
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((B, Hq), float("nan"), device=DEV)
        st = call_noalloc(qd, kd, vd, sd, o, lse, Hkv, num_splits)
        assert st == 0, attn.status_string(st)
        ro, rl = attn.attn_decode(qd, kd, vd, sd, Hkv, num_splits=num_splits,
                                  with_lse=True)
        torch.cuda.synchronize()
        # same kernels, same split: the same bits as the workspace entry
        assert torch.equal(o, ro)
        assert torch.equal(lse, rl)
        eo, el = oracle.decode(np64(q), np64(kc), np64(vc), sl,
                               1 / math.sqrt(D), Hkv)
        live = sl > 0
        err = np.abs(np64(o)[live] - eo[live]).max()
        lerr = np.abs(lse.cpu().numpy()[live] - el[live]).max()
        print(f"   max|dO|={err:.3e} max|dLSE|={lerr:.3e}", flush=True)
        assert err <= 2e-2 and lerr <= 1e-3
        assert (np64(o)[~live] == 0).all()


def test_noalloc_rejects_sizes_beyond_the_array():
    # a workspace larger than the array: refused on the host, nothing runs
    B, Hq, Hkv, D = 4096, 8, 8, 128
    need = attn.attn_decode_workspace_size(B, Hq, Hkv, D, attn.MAX_SPLITS)
    assert need > attn.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    st = attn.lib().attn_decode_noalloc(
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()),
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()),
        ctypes.c_void_p(x.data_ptr()), B, Hq, Hkv, D, 0.1, attn.MAX_SPLITS,
        None, None)
    assert st == -6
