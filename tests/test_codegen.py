"""Code-generation checks of the DMA-staged kernels (host only: compiles the
library's DMA translation units to gfx950 assembly and reads it).

The DMA loop stages h into LDS with direct buffer->LDS loads and waits for
them with explicit vector-memory counts, which rely on the order the loads are
issued in.  The compiler may move loads of memory it knows to be unchanging
(the W ring) below a wait and a barrier; the prologue's count must then still
cover the first staged chunk.  This test pins that on the code the library
ships: in every DMA kernel the first IPW vector-memory loads are the chunk-0
staging loads, and the wait before the first barrier leaves fewer loads in
flight than were issued after them.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lm_head_exact_amd", "csrc")
DMA_UNITS = ("fs_configs_dma_a.hip", "fs_configs_dma_b.hip", "fs_configs_dma_ntl.hip")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and
                                not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs hipcc")


def _assemble(unit, outdir):
    from lm_head_exact_amd import build
    out = os.path.join(outdir, unit + ".s")
    cmd = [build.HIPCC, *build.FLAGS, "-S", "--cuda-device-only", os.path.join(CSRC, unit),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _demangle(names):
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    return r.stdout.splitlines()


ALL_UNITS = tuple(sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    """gfx950 assembly of every translation unit of the library, by name."""
    outdir = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(4) as ex:
        texts = list(ex.map(lambda u: _assemble(u, outdir), ALL_UNITS))
    return dict(zip(ALL_UNITS, texts))


@pytest.fixture(scope="module")
def dma_kernels(assembly):
    texts = [assembly[u] for u in DMA_UNITS]
    kernels = {}
    for s in texts:
        names = re.findall(r"^(_Z\S*fused_sample_kernel\S*):", s, re.M)
        for n, d in zip(names, _demangle(names)):
            start = s.index(n + ":")
            end = s.index(".Lfunc_end", start)
            kernels[d] = s[start:end].splitlines()
    assert kernels, "no DMA kernels found"
    return kernels


def _ipw(demangled):
    m = re.search(r"DmaLoop<(\d+), (\d+), (\d+), (\d+), (\d+), (\d+)", demangled)
    assert m, demangled
    _, nt, nw, kc = (int(x) for x in m.groups()[:4])
    return nt * 16 * (kc // 8) // (nw * 64)


def test_dma_prologue_waits_for_the_first_staged_chunk(dma_kernels):
    for name, lines in dma_kernels.items():
        ipw = _ipw(name)
        loads, wait = [], None
        for line in lines:
            t = line.strip()
            if t.startswith(("buffer_load", "global_load")):
                loads.append(t)
            m = re.match(r"s_waitcnt vmcnt\((\d+)\)", t)
            if m:
                wait = int(m.group(1))
            if t.startswith("s_barrier"):
                break
        assert all(x.startswith("buffer_load") and x.endswith("lds") for x in loads[:ipw]), (
            f"{name}: the first {ipw} loads are not the chunk-0 staging loads: {loads[:ipw]}")
        assert wait is not None and len(loads) - wait >= ipw, (
            f"{name}: {len(loads)} loads before the first barrier, wait leaves {wait} in flight")


def test_dma_every_barrier_follows_a_vector_memory_wait(dma_kernels):
    """Each barrier of the staging loop (the bare s_barrier between empty asm
    statements) publishes a staged chunk: a vmcnt wait must come between the
    previous barrier (or the kernel start) and it."""
    for name, lines in dma_kernels.items():
        waited, prev, seen = False, "", 0
        for line in lines:
            t = line.strip()
            if not t:
                continue
            if re.match(r"s_waitcnt vmcnt\(\d+\)", t):
                waited = True
            elif t.startswith("s_barrier"):
                if prev == ";;#ASMEND":
                    assert waited, f"{name}: staging barrier without a preceding vmcnt wait"
                    seen += 1
                waited = False
            prev = t
        assert seen >= 2, f"{name}: staging barriers not found ({seen})"


def test_no_scalar_memory_writes(assembly):
    """No device code of the library writes through the scalar data cache
    (scalar stores, scalar atomics, its write-back or discard): every store
    and atomic is a vector-memory instruction."""
    pat = re.compile(r"^\s*s_(store|atomic|buffer_store|buffer_atomic|scratch_store|dcache_wb|"
                     r"dcache_discard)\w*", re.M)
    for unit, s in assembly.items():
        hits = pat.findall(s)
        assert not hits, f"{unit}: scalar memory writes {hits[:4]}"
