"""Checks on the gfx950 assembly of the kernels (no GPU needed; hipcc cross-compiles).

The LDS DMA copies are issued from inline assembly that writes M0 (the LDS base address of the
copy).  M0 is a reserved register the compiler cannot be told about, so the library is only
correct if nothing else in these kernels uses M0: every M0 write must be one of those copy
sequences (M0 write, one wait state, the DMA load), and no instruction that reads M0 implicitly
may appear.
"""
import os
import re
import shutil
import subprocess

import pytest

from rational_softmax_tiled_amd import build

HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")

M0_IMPLICIT = re.compile(r"\b(s_movrel|v_movrel|s_set_gpr_idx|s_sendmsg|ds_gws|ds_ordered_count|"
                         r"v_interp|s_ttracedata)")


def device_asm(src, tmp_path):
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    flags = [f for f in build.COMMON_FLAGS if f != "-fPIC"]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return [l.strip() for l in out.read_text().splitlines()
            if l.strip() and not l.strip().startswith((";", "."))]


@pytest.mark.parametrize("src", ["ra_fwd.hip", "ra_bwd.hip"])
def test_m0_only_feeds_lds_dma(src, tmp_path):
    ins = [l for l in device_asm(src, tmp_path) if not l.endswith(":")]
    n_dma = 0
    for i, line in enumerate(ins):
        assert not M0_IMPLICIT.match(line), line
        if re.search(r"\bm0\b", line):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", line), line
            assert ins[i + 1] == "s_nop 0", ins[i + 1]
            assert re.match(r"buffer_load_dword(x4)? v\d+, s\[\d+:\d+\], s\d+ offen lds$", ins[i + 2]), ins[i + 2]
            n_dma += 1
        elif " lds" in line and line.startswith("buffer_load"):
            assert ins[i - 1] == "s_nop 0" and re.search(r"\bm0\b", ins[i - 2]), line
    assert n_dma > 0
