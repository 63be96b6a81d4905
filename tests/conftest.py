import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built libattn.so")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; on a machine without one they are skipped
    # rather than failed, so `-m "not gpu"` and plain runs both stay green.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this machine")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(params=["w4", "rb", "balanced", "ks"])
def prefill_kernel(request):
    """Runs a prefill test under each 16-bit prefill kernel and schedule:
    the 4-wave kernel, the register-blocked one without a workspace, the
    register-blocked one with a workspace (the balanced causal schedule
    where it applies, the tile queue for causal launches of several rounds,
    the register-blocked kernel's static order elsewhere), and the
    key-split kernel (dense calls without RoPE; the others take the 4-wave
    kernel).  The register-blocked kernel applies to head dim 128; at D = 64
    the rb runs use the 4-wave kernel.  Restores the automatic choice
    afterwards."""
    from causal_attention_amd import attn
    prev = attn.prefill_select({"w4": attn.PREFILL_W4, "rb": attn.PREFILL_RB,
                                "balanced": attn.PREFILL_RB,
                                "ks": attn.PREFILL_KS}[request.param])
    prev_ws = attn.prefill_workspace_policy(request.param == "balanced")
    yield request.param
    attn.prefill_select(prev)
    attn.prefill_workspace_policy(prev_ws)
