"""Checks on the gfx950 assembly of this library's own kernels (no GPU).

The kernels issue some MFMAs and memory accesses as inline assembly, which
the compiler schedules around without knowing what they are.  These tests
compile the device code to assembly (about a minute) and check what the
compiler made of it:

- no kernel spills to scratch memory;
- no VALU write to an AGPR that an assembly QK^T MFMA (VGPR result, AGPR
  B operand) reads, within the instructions right after it: the compiler
  adds no wait states after an MFMA it cannot see, and a Q operand staged
  through shared AGPRs this way was once read after being overwritten;
- no write through the scalar data cache (scalar stores, scalar atomics,
  its write-back and discard) anywhere.
"""

import os
import re
import subprocess

import pytest

from causal_attention_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asm")


@pytest.fixture(scope="module")
def asm():
    os.makedirs(OUT, exist_ok=True)
    path = os.path.join(OUT, "attn.s")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I",
           os.path.join(ROOT, "include"), build.SRC, "-o", path]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(path).read()


def kernels(text):
    """{mangled name: (body, metadata that follows it)}."""
    out = {}
    for name in re.findall(r"^(_ZN4attn\w+):", text, re.M):
        a = text.index(name + ":")
        b = text.index(".Lfunc_end", a)
        out[name] = (text[a:b], text[b:b + 8000])
    return out


def test_no_kernel_spills(asm):
    ks = kernels(asm)
    assert ks
    for name, (_, meta) in ks.items():
        m = re.search(r"; ScratchSize: (\d+)", meta)
        assert m is not None, name
        assert int(m.group(1)) == 0, f"{name} uses {m.group(1)} B of scratch"


def test_no_agpr_rewrite_after_assembly_mfma(asm):
    mfma = re.compile(r"v_mfma_f32_32x32x16_(?:bf16|f16) v\[\d+:\d+\], "
                      r"v\[\d+:\d+\], a\[(\d+):(\d+)\]")
    write = re.compile(r"v_accvgpr_(?:write_b32|mov_b32) a(\d+),")
    seen = 0
    for name, (body, _) in kernels(asm).items():
        lines = [x.strip() for x in body.split("\n")]
        lines = [x for x in lines if x and not x.startswith((";", "."))]
        for i, line in enumerate(lines):
            m = mfma.match(line)
            if not m:
                continue
            seen += 1
            lo, hi = int(m.group(1)), int(m.group(2))
            for nxt in lines[i + 1:i + 9]:
                w = write.match(nxt)
                assert not (w and lo <= int(w.group(1)) <= hi), \
                    f"{name}: '{nxt}' right after '{line}'"
    assert seen > 0     # the pattern still finds the QK^T MFMAs


def test_no_scalar_cache_writes(asm):
    bad = re.findall(r"^\s*(s_(?:store|atomic|buffer_store|scratch_store|"
                     r"dcache_wb|dcache_discard)\w*)", asm, re.M)
    assert not bad, sorted(set(bad))
