"""The large-M kernel's 32-row instantiations keep the weights of K tile t + 2
in flight across the barrier that ends tile t: that barrier is preceded by a
hand-counted wait, vmcnt(kW), which is only right if exactly kW vector loads
are issued after the tile's last activation load (LDS DMA).  This compiles the
kernels to gfx950 assembly (CPU only) and checks every such wait against the
loads the compiler actually emitted, for every format, width and dtype."""

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_only_gemm_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["prefill.hip", "prefill_b3.hip", "prefill_b8.hip"]


def _asm(src, out):
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
                    os.path.join(CSRC, src), "-o", out], check=True, capture_output=True)
    return out


def _check(text):
    """(barriers checked, mismatches) over the 32-row kernels of one file."""
    seen, bad = 0, []
    for m in re.finditer(r"^(_ZN5w4a1617wq_prefill_kernelILi\dELi32E\S*):", text, re.M):
        end = text.index(".Lfunc_end", m.end())
        lines = [l.strip() for l in text[m.end():end].split("\n")]
        pend = None                      # vector loads since the last LDS DMA
        for i, t in enumerate(lines):
            if t.startswith("buffer_load") and t.endswith(" lds"):
                pend = 0
            elif t.startswith(("buffer_load", "global_load")) and pend is not None:
                pend += 1
            w = re.match(r"s_waitcnt vmcnt\((\d+)\)$", t)
            if w and i + 1 < len(lines) and lines[i + 1] == "s_barrier":
                seen += 1
                if pend != int(w.group(1)):
                    bad.append((m.group(1), int(w.group(1)), pend))
    return seen, bad


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
def test_deep_prefetch_waits_match_emitted_loads():
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            outs = list(ex.map(lambda s: _asm(s, os.path.join(d, s + ".s")), SOURCES))
        total = 0
        for o in outs:
            seen, bad = _check(open(o).read())
            assert not bad, bad[:4]
            total += seen
    # 3 widths x 2 dtypes x (INT U in {1, 2, 4}; NF4 with 4 bits) x 2 tail forms,
    # three barriers each (the tile loop is unrolled by three)
    assert total >= 3 * 2 * 3 * 2 * 3
