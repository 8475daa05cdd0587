"""Checks of the gfx950 code the kernels compile to (CPU only: hipcc cross-compiles).

Every global -> LDS DMA load is issued from inline assembly, which the
compiler's hazard checks do not see into.  The instruction in front of it
must be the s_nop 4 that supplies the wait states an SGPR written by a VALU
instruction (the buffer resource, a reloaded SGPR) and M0 need before the
load reads them; without them the load may use a stale range check or LDS
address.
"""
import os
import re
import shutil
import subprocess

import pytest

from attention_scores_amd import _build

pytestmark = pytest.mark.skipif(not os.path.exists(_build.HIPCC) and not shutil.which("hipcc"),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    """gfx950 assembly of each kernel source, compiled once per test session."""
    cache = {}

    def get(src):
        if src not in cache:
            cache[src] = _asm(src, tmp_path_factory.mktemp("asm"))
        return cache[src]
    return get


def _asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in _build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [_build.HIPCC] + flags + ["--cuda-device-only", "-S", "-I", _build.INCLUDE, "-I", _build.CSRC,
                                    os.path.join(_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


@pytest.mark.parametrize("src", ["gemm.hip", "attn.hip"])
def test_every_lds_dma_load_follows_its_wait_states(src, asm):
    lines = asm(src)
    loads = 0
    for n, line in enumerate(lines):
        if not re.match(r"\s+buffer_load_dword(x4)? .* lds\s*$", line):
            continue
        loads += 1
        k = n - 1
        while k >= 0 and (not lines[k].strip() or lines[k].strip().startswith((";", "."))):
            k -= 1
        assert lines[k].strip() == "s_nop 4", "line %d: %r before %r" % (n, lines[k].strip(), line.strip())
    assert loads > 0


def test_kernels_use_no_scratch_memory(asm):
    for src in ("gemm.hip", "splitk.hip", "attn.hip"):
        text = "\n".join(asm(src))
        sizes = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)]
        spills = [int(v) for v in re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)]
        assert sizes and max(sizes) == 0, src
        assert spills and max(spills) == 0, src
