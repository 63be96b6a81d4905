"""Benchmark of the fused attention hot path on one MI355X.

One step = one causal GQA prefill at long context (batch 1, 8 query heads
over 2 KV heads, head_dim 128, seq 32768, bf16) followed by one split-K
decode (batch 32, same heads, per-sequence cache length uniform in
[256, 4096] from seed 0, bf16), each through the C ABI on torch's current
stream, after at least one second of untimed warm-up steps (the GPU's
clock and power settle over that time).  Inputs are seeded synthetic
tensors resident in HBM before timing;
enough input copies are rotated that no launch finds its inputs in the
256 MB last-level cache.

Prints ONE JSON line.  ``value`` is the prefill's algorithmic TFLOP/s (4*D
per visible query/key pair, causal pairs only) over the prefill kernel's
mean duration measured with HIP events around each launch; the decode's
KV-cache GB/s (K and V bytes read once per KV head, plus q and o) is in
``decode``.  Both carry a ``roofline`` object against MI355X's published
peaks (2.5 PFLOP/s dense bf16 MFMA, 8 TB/s HBM3E) with the mean, median
and minimum launch time.  ``side_configs`` times the other prefill workloads
(batch 4 at seq 2048 by default) the same way, each against its own dtype's
peak.  ``cpu_baseline`` times the fp64 CPU oracle on the host on a bounded
sample of the same workload.  With ``--extras`` the line also carries
``extras``: the widened paths (fp16 storage, RoPE, ragged batch, the fused
residual + RMSNorm epilogue) timed on
the shapes of the batch-4 prefill and the decode.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
LLC_BYTES = 256 * 2 ** 20       # MI355X last-level (Infinity) cache


def peak_tflops(dtype):
    return PEAK_FP32_MATRIX_TFLOPS if dtype == "f32" else PEAK_BF16_TFLOPS


def copies_for(nbytes, at_least=2, at_most=64):
    """Input copies to rotate so that a copy is reused only after more than
    the last-level cache's worth of other inputs has been read."""
    return int(min(at_most, max(at_least, -(-int(1.2 * LLC_BYTES) // max(
        1, nbytes)) + 1)))


def launch_stats(ms):
    """mean / median / min of per-launch times (ms) in microseconds."""
    xs = sorted(ms)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"mean_us": round(1e3 * sum(xs) / n, 3),
            "median_us": round(1e3 * med, 3),
            "min_us": round(1e3 * xs[0], 3), "launches": n}


def prefill_flops(B, Hq, S, D, causal=True):
    pairs = S * (S + 1) // 2 if causal else S * S
    return 4 * D * B * Hq * pairs


def prefill_bytes(B, Hq, Hkv, S, D, elt=2):
    """Q, K, V read once, O and the fp32 LSE written once."""
    return (B * Hq * S * D * 2 + B * Hkv * S * D * 2) * elt + B * Hq * S * 4


def decode_bytes(seqlens, Hq, Hkv, D, elt=2):
    kv = int(sum(int(x) for x in seqlens)) * Hkv * D * elt * 2
    return kv + 2 * len(seqlens) * Hq * D * elt


KERNEL_SOURCES = ("causal_attention_amd/csrc/common.hpp",
                  "causal_attention_amd/csrc/prefill.hpp",
                  "causal_attention_amd/csrc/prefill_ks.hpp",
                  "causal_attention_amd/csrc/decode.hpp",
                  "causal_attention_amd/csrc/kvcache.hpp",
                  "causal_attention_amd/csrc/attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def kernel_source_hash():
    """Hash of the kernel sources' code: comments and whitespace are left
    out, so that a comment edit does not retire measurements of unchanged
    kernels (no string literal in these sources holds a comment marker)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    recorded in profiles/hbm_traffic.txt, or {} when that record was taken
    on different kernel sources."""
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE)
                  if ":" in line and not line.startswith("#"))
    except OSError:
        return {}
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_sources_sha256") != kernel_source_hash():
        return {}
    return kv


def traffic_for(tr, workload):
    """HBM bytes per launch recorded for ``workload``, else None."""
    key = workload + "_hbm_bytes_per_launch"
    return int(tr[key]) if key in tr else None


def copy_calibration(mbytes, reps=5):
    """A plain device copy of known size, for scaling the HBM counters."""
    import torch
    n = int(mbytes * 1e6) // 16 * 16
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n,
                      "reps": reps}), flush=True)


def cpu_baseline(wp, wd, prefill_rows=4096, decode_reps=64):
    """Time the fp64 oracle on the host on a bounded sample of the workload
    (about ten seconds of CPU work): for a long-context prefill, the oracle at
    ``prefill_rows`` seeded query rows per head, taken 256 at a time; else the
    whole prefill once; and the whole decode workload ``decode_reps`` times."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from causal_attention_amd import inputs

    q, k, v = inputs.prefill_inputs(wp.B, wp.Hq, wp.Hkv, wp.S, wp.D,
                                    wp.dtype, wp.sigma, wp.seed)
    q, k, v = (t.float().numpy() for t in (q, k, v))
    if wp.sampled_rows:
        n = min(prefill_rows, wp.S)
        rows = inputs.sampled_rows(wp.Hq, wp.S, n)
        chunks = max(1, n // 256)
        t0 = time.perf_counter()
        for c in range(chunks):
            oracle.prefill_rows(q, k, v, wp.scale, True, rows[:, c::chunks])
        tp = time.perf_counter() - t0
        pflops = 4 * wp.D * wp.B * int((rows + 1).sum())
        what = (f"{n} seeded query rows per head of the prefill, "
                f"{n // chunks} at a time ({tp:.2f} s)")
    else:
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, wp.scale, True)
        tp = time.perf_counter() - t0
        pflops = prefill_flops(wp.B, wp.Hq, wp.S, wp.D)
        what = f"whole prefill workload once ({tp:.2f} s)"
    sl, q, kc, vc = inputs.workload_inputs(wd)
    q, kc, vc = (t.float().numpy() for t in (q, kc, vc))
    t0 = time.perf_counter()
    for _ in range(decode_reps):
        oracle.decode(q, kc, vc, sl, wd.scale, wd.Hkv)
    td = (time.perf_counter() - t0) / decode_reps
    what += (f" and the whole decode workload {decode_reps} times "
             f"({td * decode_reps:.2f} s)")
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    blas = sorted({f"{i.get('internal_api', '?')} {i.get('version') or ''}".strip()
                   for i in info if i.get("user_api") == "blas"})
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": pflops / tp / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{what}, numpy fp64",
        "decode_GBps": decode_bytes(sl, wd.Hq, wd.Hkv, wd.D) / td / 1e9,
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model,
        "blas": ", ".join(blas) or "unknown",
    }


def extras(attn, inputs, torch, dev, wp, wd, reps=20):
    """The widened paths on the same shapes, each timed with HIP events over
    ``reps`` back-to-back launches on warm inputs (they fit the last-level
    cache): fp16 storage, RoPE, the ragged batch.  Rates are algorithmic
    (the same FLOP and byte counts as the main line) against the same
    peaks (fp16 dense MFMA peak = bf16's)."""
    def timed(fn):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps          # ms

    def tf(flops, ms):
        t = flops / (ms * 1e-3) / 1e12
        return {"us": round(ms * 1e3, 3), "TFLOP/s": round(t, 1),
                "frac": round(t / PEAK_BF16_TFLOPS, 4)}

    def gb(nbytes, ms):
        g = nbytes / (ms * 1e-3) / 1e9
        return {"us": round(ms * 1e3, 3), "GB/s": round(g, 1),
                "frac": round(g / PEAK_HBM_GBS, 4)}

    out = {}
    flops = prefill_flops(wp.B, wp.Hq, wp.S, wp.D)
    q, k, v = (t.to(dev) for t in inputs.prefill_inputs(
        wp.B, wp.Hq, wp.Hkv, wp.S, wp.D, "f16", wp.sigma, wp.seed))
    o = torch.empty_like(q)
    call = attn.prepare_prefill(q, k, v, o, None, causal=True)
    out["prefill_f16"] = tf(flops, timed(call))
    sl, dq, kc, vc = inputs.decode_inputs(wd.B, wd.Hq, wd.Hkv, wd.D,
                                          lmin=wd.lmin, lmax=wd.lmax,
                                          dtype="f16", sigma=wd.sigma,
                                          seed=wd.seed)
    dq, kc, vc = dq.to(dev), kc.to(dev), vc.to(dev)
    sld = torch.from_numpy(sl).to(dev)
    ws = attn.new_decode_workspace(wd.B, wd.Hq, wd.Hkv, wd.D, 0, dev)
    do = torch.empty_like(dq)
    dcall = attn.prepare_decode(dq, kc, vc, sld, do, wd.Hkv, ws)
    dbytes = decode_bytes(sl, wd.Hq, wd.Hkv, wd.D)
    out["decode_f16"] = gb(dbytes, timed(dcall))

    # the same decode at 8x the batch (B = 256, lengths from the same
    # distribution, about 600 MB of cache): how far the split kernel's
    # stream goes once the launch's fixed cost is spread over more bytes
    slb, dqb8, kcb, vcb = inputs.decode_inputs(8 * wd.B, wd.Hq, wd.Hkv, wd.D,
                                               lmin=wd.lmin, lmax=wd.lmax,
                                               sigma=wd.sigma, seed=wd.seed)
    dqb8, kcb, vcb = dqb8.to(dev), kcb.to(dev), vcb.to(dev)
    sldb = torch.from_numpy(slb).to(dev)
    wsb = attn.new_decode_workspace(8 * wd.B, wd.Hq, wd.Hkv, wd.D, 0, dev)
    dob8 = torch.empty_like(dqb8)
    bcall = attn.prepare_decode(dqb8, kcb, vcb, sldb, dob8, wd.Hkv, wsb)
    out["decode_b256"] = gb(decode_bytes(slb, wd.Hq, wd.Hkv, wd.D),
                            timed(bcall))
    out["decode_b256"]["cache_MB"] = round(
        2 * kcb.numel() * kcb.element_size() / 1e6, 1)
    del kcb, vcb

    # RoPE: prefill with q rotated on load plus the K rotation pass (timed
    # together; the FLOP count is the attention's), and decode over a padded
    # cache with q rotated in the kernel
    qb, kb, vb = (t.to(dev) for t in inputs.prefill_inputs(
        wp.B, wp.Hq, wp.Hkv, wp.S, wp.D, "bf16", wp.sigma, wp.seed))
    ob, kr = torch.empty_like(qb), torch.empty_like(kb)
    out["prefill_rope"] = tf(flops, timed(
        lambda: attn.attn_prefill_rope(qb, kb, vb, 10000.0, out=ob,
                                       with_lse=False, k_rot=kr)))
    cap = wd.lmax
    kp = torch.zeros(wd.B, wd.Hkv, cap, wd.D, dtype=torch.bfloat16,
                     device=dev)
    vp = torch.zeros_like(kp)
    dqb = dq.to(torch.bfloat16)
    dob = torch.empty_like(dqb)
    out["decode_padded_rope"] = gb(dbytes, timed(
        lambda: attn.attn_decode_padded(dqb, kp, vp, sld, out=dob,
                                        workspace=ws, rope_base=10000.0)))

    # ragged batch: B sequences with the decode workload's lengths
    lens = sl.astype("int64")
    N = int(lens.sum())
    g = torch.Generator().manual_seed(1)
    qv = torch.randn(wp.Hq * N * wp.D, generator=g).to(torch.bfloat16).to(dev)
    kv = torch.randn(wp.Hkv * N * wp.D, generator=g).to(torch.bfloat16).to(dev)
    vv = torch.randn(wp.Hkv * N * wp.D, generator=g).to(torch.bfloat16).to(dev)
    cu = torch.tensor([0] + list(lens.cumsum()), dtype=torch.int32,
                      device=dev)
    ov = torch.empty_like(qv)
    vflops = sum(4 * wp.D * wp.Hq * int(L) * (int(L) + 1) // 2 for L in lens)
    out["prefill_varlen"] = tf(vflops, timed(
        lambda: attn.attn_prefill_varlen(qv, kv, vv, cu, int(lens.max()),
                                         wp.Hq, wp.Hkv, wp.D, out=ov,
                                         with_lse=False)))
    out["prefill_varlen"]["sequences"] = f"{len(lens)} lengths of the decode workload, sum {N}"

    # padded batch: the same lengths, each sequence stored with Smax rows
    Smax = int(lens.max())
    B = len(lens)
    qp = torch.randn(B, wp.Hq, Smax, wp.D, generator=g).to(torch.bfloat16).to(dev)
    kp2 = torch.randn(B, wp.Hkv, Smax, wp.D, generator=g).to(torch.bfloat16).to(dev)
    vp2 = torch.randn(B, wp.Hkv, Smax, wp.D, generator=g).to(torch.bfloat16).to(dev)
    slp = torch.from_numpy(sl.astype("int32")).to(dev)
    op = torch.empty_like(qp)
    out["prefill_padded"] = tf(vflops, timed(
        lambda: attn.attn_prefill_padded(qp, kp2, vp2, slp, out=op,
                                         with_lse=False)))
    out["prefill_padded"]["sequences"] = f"the same {B} lengths, padded to {Smax} rows"

    # residual add + RMSNorm fused into the 4-wave kernel's epilogue, beside
    # the plain 4-wave prefill on the same inputs (the fused path adds a read
    # and a write of the residual and a read of the weight)
    res, wgt = (t.to(dev) for t in inputs.residual_inputs(
        wp.B, wp.Hq, wp.S, wp.D, "bf16", 1.0, wp.seed))
    orms = torch.empty_like(qb)
    out["prefill_residual_rmsnorm"] = tf(flops, timed(
        lambda: attn.attn_prefill_residual_rmsnorm(qb, kb, vb, res, wgt,
                                                   out=orms,
                                                   with_lse=False)))
    prev = attn.prefill_select(attn.PREFILL_W4)
    prev_ws = attn.prefill_workspace_policy(False)
    try:
        out["prefill_w4_plain"] = tf(flops, timed(
            lambda: attn.attn_prefill(qb, kb, vb, out=ob, with_lse=False)))
    finally:
        attn.prefill_select(prev)
        attn.prefill_workspace_policy(prev_ws)
    out["prefill_residual_rmsnorm"]["extra_bytes"] = int(
        2 * res.numel() * res.element_size() + wgt.numel() * 2)

    # the same at a size the register-blocked kernel takes (B1, S16384),
    # beside the plain prefill on that kernel (no workspace)
    Sl = 16384
    ql, kl, vl = (t.to(dev) for t in inputs.prefill_inputs(
        1, wp.Hq, wp.Hkv, Sl, wp.D, "bf16", 1.0, wp.seed))
    resl, wgtl = (t.to(dev) for t in inputs.residual_inputs(
        1, wp.Hq, Sl, wp.D, "bf16", 1.0, wp.seed))
    ol, oln = torch.empty_like(ql), torch.empty_like(ql)
    lflops = prefill_flops(1, wp.Hq, Sl, wp.D)
    out["prefill_residual_rmsnorm_s16384"] = tf(lflops, timed(
        lambda: attn.attn_prefill_residual_rmsnorm(ql, kl, vl, resl, wgtl,
                                                   out=ol, with_lse=False)))
    prev_ws = attn.prefill_workspace_policy(False)
    try:
        out["prefill_plain_s16384"] = tf(lflops, timed(
            lambda: attn.attn_prefill(ql, kl, vl, out=oln, with_lse=False)))
    finally:
        attn.prefill_workspace_policy(prev_ws)
    out["prefill_residual_rmsnorm_s16384"]["kernel"] = \
        attn.PREFILL_KERNEL_NAMES[attn.prefill_kernel_for(1, wp.Hq, Sl, wp.D)]
    return out




def warm_up(run, torch, count, seconds):
    """run(i) for at least ``count`` calls and at least ``seconds`` of
    wall time (the GPU's clock and power settle over the first second of
    sustained load); returns the number of calls."""
    i = 0
    t0 = time.perf_counter()
    while i < count or time.perf_counter() - t0 < seconds:
        run(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def time_prefill(attn, inputs, torch, dev, w, steps, warmup, warmup_s=0.2):
    """Event-timed launches of one prefill workload through prepared C-ABI
    calls, rotating input copies; returns (stats, copies)."""
    q, k, v = inputs.prefill_inputs(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype,
                                    w.sigma, w.seed)
    elt = 4 if w.dtype == "f32" else 2
    R = copies_for(prefill_bytes(w.B, w.Hq, w.Hkv, w.S, w.D, elt))
    ins = [tuple(t.to(dev) for t in (q, k, v)) for _ in range(R)]
    outs = [torch.empty_like(ins[0][0]) for _ in range(R)]
    lses = [torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
            for _ in range(R)]
    calls = [attn.prepare_prefill(*ins[r], outs[r], lses[r], causal=w.causal,
                                  scale=w.scale) for r in range(R)]
    warm_up(lambda i: calls[i % R](), torch, warmup, warmup_s)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        calls[i % R]()
        ev[i][1].record()
    torch.cuda.synchronize()
    return launch_stats([e[0].elapsed_time(e[1]) for e in ev]), R


def prefill_launch(attn, w):
    """Kernel name, workgroups and threads per workgroup of one prefill
    launch of workload w."""
    if w.dtype == "f32":
        if attn.prefill_kernel_for(w.B, w.Hq, w.S, w.D,
                                   w.causal) == attn.PREFILL_KS:
            return {"kernel": "attn_prefill_f32_ks_kernel",
                    "workgroups": w.B * w.Hq * -(-w.S // 32), "threads": 256,
                    "schedule": ("key split: 32 query rows per workgroup, "
                                 "its four waves take every fourth key "
                                 "tile and merge in LDS")}
        return {"kernel": "attn_prefill_f32_kernel",
                "workgroups": w.B * w.Hq * -(-w.S // 128), "threads": 256}
    kern, wgs, thr = attn.prefill_workgroups(w.B, w.Hq, w.Hkv, w.S, w.D,
                                             w.causal)
    sched = attn.prefill_schedule(w.B, w.Hq, w.Hkv, w.S, w.D, w.causal)
    if sched == attn.SCHEDULE_BALANCED:
        schedule = ("balanced: query tiles t and n-1-t paired, each pair's "
                    "key tiles cut between two workgroups")
    elif kern == attn.PREFILL_KS:
        schedule = ("key split: 32 query rows per workgroup, its four waves "
                    "take every fourth key tile and merge in LDS")
    elif sched == attn.SCHEDULE_QUEUE:
        schedule = ("tile queue: one workgroup per query tile, each taking "
                    "the next heaviest tile from a counter in the workspace")
    else:
        schedule = "one workgroup per query tile, heaviest first"
    return {"kernel": attn.PREFILL_KERNEL_NAMES[kern], "workgroups": wgs,
            "threads": thr, "schedule": schedule}


def prefill_record(w, st, R, traffic=None):
    """The roofline object of one prefill workload from its launch stats."""
    elt = 4 if w.dtype == "f32" else 2
    flops = prefill_flops(w.B, w.Hq, w.S, w.D, w.causal)
    peak = peak_tflops(w.dtype)
    tf = flops / (st["mean_us"] * 1e-6) / 1e12
    return {
        "bound": "mfma",
        "achieved": round(tf, 3),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(tf / peak, 4),
        "traffic": traffic,
        "traffic_unit": "HBM bytes per launch",
        "algorithmic_bytes": prefill_bytes(w.B, w.Hq, w.Hkv, w.S, w.D, elt),
        "flops_per_launch": flops,
        **st,
        "median_TFLOPs": round(flops / (st["median_us"] * 1e-6) / 1e12, 3),
        "best_TFLOPs": round(flops / (st["min_us"] * 1e-6) / 1e12, 3),
        "input_copies_rotated": R,
        "shape": {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "D": w.D,
                  "dtype": w.dtype, "causal": w.causal, "sigma": w.sigma,
                  "seed": w.seed},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="least wall time of warm-up steps (the GPU's clock "
                         "and power settle over the first second)")
    ap.add_argument("--prefill", default="c5_gqa_s32768",
                    help="prefill workload of the step (value / roofline)")
    ap.add_argument("--decode", default="c4_decode_b32")
    ap.add_argument("--side",
                    default="c3_gqa_b4_s2048,c2_mha12_s512,c1_f32_s128",
                    help="comma-separated prefill workloads timed after the "
                    "step, reported under side_configs ('' for none)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    metavar="MB", help="only run a plain MB-sized device copy "
                    "(to scale rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--extras", action="store_true",
                    help="also time the fp16 / RoPE / ragged-batch paths "
                    "(reported under \"extras\"; off by default so the "
                    "kernel statistics of the default run hold only the "
                    "step's and side configs' launches)")
    args = ap.parse_args()
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): this "
              "path has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch

    from causal_attention_amd import attn, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wp = inputs.WORKLOADS[args.prefill]
    wd = inputs.WORKLOADS[args.decode]
    side = [inputs.WORKLOADS[n] for n in args.side.split(",") if n]

    # ---- the step: prefill + decode, copies rotated separately
    q, k, v = inputs.prefill_inputs(wp.B, wp.Hq, wp.Hkv, wp.S, wp.D,
                                    wp.dtype, wp.sigma, wp.seed)
    sl, dq, kc, vc = inputs.workload_inputs(wd)
    Rp = copies_for(prefill_bytes(wp.B, wp.Hq, wp.Hkv, wp.S, wp.D))
    dbytes = decode_bytes(sl, wd.Hq, wd.Hkv, wd.D)
    Rd = copies_for(dbytes, at_least=5)
    P = [tuple(t.to(dev) for t in (q, k, v)) for _ in range(Rp)]
    Dd = [tuple(t.to(dev) for t in (dq, kc, vc)) for _ in range(Rd)]
    sl_d = torch.from_numpy(sl).to(dev)
    po = [torch.empty_like(P[0][0]) for _ in range(Rp)]
    plse = [torch.empty((wp.B, wp.Hq, wp.S), dtype=torch.float32, device=dev)
            for _ in range(Rp)]
    do = [torch.empty_like(Dd[0][0]) for _ in range(Rd)]
    ws = attn.new_decode_workspace(wd.B, wd.Hq, wd.Hkv, wd.D,
                                   args.num_splits, dev)
    ns = args.num_splits or attn.attn_decode_auto_splits(wd.B, wd.Hkv)

    # Arguments are converted once; each launch is then a single C call, so
    # the host stays ahead of the GPU and the events time the kernels.
    pre = [attn.prepare_prefill(*P[r], po[r], plse[r], causal=True,
                                scale=wp.scale) for r in range(Rp)]
    dec = [attn.prepare_decode(*Dd[r], sl_d, do[r], wd.Hkv, ws,
                               num_splits=ns, scale=wd.scale)
           for r in range(Rd)]

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        pre[i % Rp]()
        if ev is not None:
            ev[1].record()
        dec[i % Rd]()
        if ev is not None:
            ev[2].record()

    warm_steps = warm_up(step, torch, args.warmup, args.warmup_seconds)

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pst = launch_stats([e[0].elapsed_time(e[1]) for e in evs])
    dst = launch_stats([e[1].elapsed_time(e[2]) for e in evs])

    # ---- side configs (other prefill workloads), timed the same way
    side_rec = {}
    for w in side:
        st, R = time_prefill(attn, inputs, torch, dev, w, K, args.warmup,
                             min(0.2, args.warmup_seconds))
        rec = prefill_record(w, st, R, traffic_for(measured_traffic(), w.name))
        rec.update(prefill_launch(attn, w))
        side_rec[w.name] = rec

    # ---- the decode as a serving loop runs it: the Rd rotated decode
    # calls (standing in for Rd layers of one token) captured once in a
    # hipGraph and replayed; reported per decode
    sstream = torch.cuda.Stream()
    sstream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(sstream):
        for r in range(Rd):
            attn.prepare_decode(*Dd[r], sl_d, do[r], wd.Hkv, ws,
                                num_splits=ns, scale=wd.scale)()
    torch.cuda.current_stream().wait_stream(sstream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(Rd):
            attn.prepare_decode(*Dd[r], sl_d, do[r], wd.Hkv, ws,
                                num_splits=ns, scale=wd.scale)()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    KG = max(2, K // Rd)
    gevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
            for _ in range(KG)]
    for i in range(KG):
        gevs[i][0].record()
        graph.replay()
        gevs[i][1].record()
    torch.cuda.synchronize()
    gst = launch_stats([e[0].elapsed_time(e[1]) / Rd for e in gevs])

    tr = measured_traffic()
    prec = prefill_record(wp, pst, Rp, traffic_for(tr, wp.name))
    prec.pop("shape")
    prec.update(prefill_launch(attn, wp))
    d_gbs = dbytes / (dst["mean_us"] * 1e-6) / 1e9
    g_gbs = dbytes / (gst["mean_us"] * 1e-6) / 1e9
    out = {
        "metric": "prefill attention TFLOP/s + decode KV-cache GB/s, "
                  "% of MI355X roofline",
        "value": prec["achieved"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "warmup_seconds": args.warmup_seconds,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wp.name} prefill + {wd.name} decode",
            "prefill": {"B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "S": wp.S,
                        "D": wp.D, "causal": True, "sigma": wp.sigma,
                        "seed": wp.seed},
            "decode": {"B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "D": wd.D,
                       "seqlens": "U[256,4096] seed 0",
                       "sum_seqlens": int(sl.sum()), "num_splits": ns},
            "input_copies_rotated": {"prefill": Rp, "decode": Rd},
            "timing": "HIP events around each launch on the launching "
                      "stream; value and roofline use the mean launch time, "
                      "median and min beside it",
        },
        "roofline": prec,
        "decode": {
            "value": round(d_gbs, 2),
            "unit": "GB/s",
            "roofline": {
                "bound": "hbm",
                "kernel": "attn_decode_split_kernel + "
                          "attn_decode_combine_kernel",
                "achieved": round(d_gbs, 2),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(d_gbs / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(tr, wd.name),
                "traffic_unit": "HBM bytes per launch (split + combine)",
                "bytes_per_launch": dbytes,
                **dst,
                "median_GBps": round(
                    dbytes / (dst["median_us"] * 1e-6) / 1e9, 2),
                "best_GBps": round(dbytes / (dst["min_us"] * 1e-6) / 1e9, 2),
            },
            "graph": {
                "what": f"{Rd} decode calls (one per rotated cache copy) "
                        "captured in one hipGraph and replayed; time per "
                        "decode",
                **gst,
                "GBps": round(g_gbs, 2),
                "frac": round(g_gbs / PEAK_HBM_GBS, 4),
            },
        },
        "side_configs": side_rec,
    }
    if args.extras:
        out["extras"] = extras(attn, inputs, torch, dev,
                               inputs.WORKLOADS["c3_gqa_b4_s2048"], wd)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wp, wd)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
