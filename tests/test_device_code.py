"""Properties of the generated gfx950 code that the kernels rely on.

The grouped GEMMs and the fused router issue their direct-to-LDS loads from inline asm
(`s_mov_b32 m0, base` then `global_load_lds_dwordx4`), so that the compiler
adds no waits of its own for them. m0 is a reserved register: the compiler
ignores the asm's clobber of it. That is only safe while the compiler itself
never reads m0 in those kernels; this test compiles them and checks that
every m0 reference is one of the asm's own writes, followed by its load.
"""
import os
import re
import subprocess

import pytest

from fine_grained_mixture_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fine_grained_mixture_amd", "csrc")


@pytest.mark.parametrize("src", ["gemm_big.hip", "fp8.hip", "gemm_bwd.hip", "route_small.hip"])
def test_m0_only_written_by_the_lds_dma_asm(src, tmp_path):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [hipcc, *build.COMMON, *build.DEVICE_FLAGS, "-S", "--cuda-device-only",
           os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    code = []
    for line in out.read_text().splitlines():
        line = line.strip()
        if not line or line.startswith((";", ".", "//")) or line.endswith(":"):
            continue
        code.append(line)
    refs = [i for i, line in enumerate(code) if re.search(r"\bm0\b", line)]
    assert refs, "no direct-to-LDS loads found"
    for i in refs:
        assert code[i].startswith("s_mov_b32 m0,"), code[i]
        assert any(n.startswith("global_load_lds") for n in code[i + 1:i + 3]), code[i:i + 3]
