"""Properties of the gfx950 code built from the kernel sources (CPU only:
hipcc cross-compiles, nothing runs).

The bf16 backward kernels stage their tiles with LDS-direct loads.  These are
written with the buffer-load builtin over a per-stage resource: an SGPR base at
the stage's first row (64-bit arithmetic, any sequence length) and a 32-bit
per-lane offset that stays below the 8 KiB a stage spans.  The compiler then
sets M0 itself; no inline assembly touches it.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "complex_valued_attention_amd", "csrc")
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S", src,
                        "-o", str(out), "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text(), r.stderr


def test_no_inline_asm_emits_instructions():
    # inline asm in the kernels is only ever empty: a compiler barrier, or an
    # empty statement that makes a value opaque to the optimiser; it emits no
    # instruction, so the compiler keeps full knowledge of registers, M0 and
    # the memory counters
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".h")):
            continue
        text = open(os.path.join(CSRC, name)).read()
        for m in re.finditer(r"\b(?:__asm__|asm)\s*(?:__volatile__|volatile)?\s*\(\s*(\"[^\"]*\")", text):
            assert m.group(1) == '""', (name, m.group(0))


def test_bf16_backward_lds_direct_loads_use_sgpr_base(tmp_path):
    asm, err = device_asm(os.path.join(CSRC, "kernel_born_bf16_d64_bwd.hip"), tmp_path)
    assert "inline asm" not in err and "clobber" not in err, err[-2000:]
    lds_loads = [l.strip() for l in asm.splitlines() if re.search(r"\bload_lds_dword|\blds$", l.strip())]
    assert lds_loads, "no LDS-direct loads found"
    for l in lds_loads:
        # buffer_load_dword[x4] <voffset>, s[..], <soffset> offen lds: one 32-bit VGPR offset, SGPR
        # base (x4: the 16-byte stage chunks; dword: the per-query scalar pairs of a stage)
        assert re.match(r"buffer_load_dword(x4)? v\d+, s\[\d+:\d+\], \S+ offen lds$", l), l


def test_bf16_backward_stage_offsets_stay_in_one_stage():
    # the per-lane offset of a stage load is (row within the stage) * 128 B +
    # 16 B * chunk with the row clamped to the last valid row: below 8 KiB for
    # any sequence length (the stage base carries the 64-bit part)
    ROWB, REGION = 128, 8192
    for T in (1, 63, 64, 65, 2 ** 24 - 1, 2 ** 24, 2 ** 24 + 37, 2 ** 30):
        for r0 in {0, max(0, T - 64), max(0, (T - 1) // 64 * 64)}:
            if r0 >= T:
                continue
            for row in range(64):
                g = min(row, T - 1 - r0)
                for lc in range(8):
                    off = g * ROWB + 16 * lc
                    assert 0 <= off < REGION
