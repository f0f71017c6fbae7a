"""The bf16 iterate's lo layout (lo_offset in csrc/muon_internal.h), checked on the CPU.

lo_offset places element (row, col) of the padded NS-frame matrix at the position the
update kernel's thread reads it from and writes it to: thread t = 64 w + l (wave
w = 4 wm + wn, lane l) holds register q of 32 x 32 block (i, j) for tile row
128 wm + 32 i + 8 (q / 4) + 4 (l / 32) + q % 4 and column 64 wn + 32 j + l % 32 (the
MFMA 32 x 32 output layout), in 16-byte chunk v = 4 i + 2 j + q / 8 of the tile.  The
test compiles a small host program against the header and checks that lo_offset is a
bijection onto the padded matrix and agrees with that per-thread description.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "matrix_aware_optimizer_amd", "csrc")

PROGRAM = r"""
#include "muon_internal.h"
#include <cstdio>
#include <vector>
int main() {
    const int mp = 512, np = 768;
    std::vector<int> seen((size_t)mp * np, 0);
    for (int r = 0; r < mp; ++r)
        for (int c = 0; c < np; ++c) {
            const size_t o = muon::lo_offset(r, c, np);
            if (o >= seen.size()) { std::printf("out of range\n"); return 1; }
            ++seen[o];
        }
    for (int x : seen)
        if (x != 1) { std::printf("not a bijection\n"); return 1; }
    long bad = 0;
    for (int ti = 0; ti < mp / 256; ++ti)
        for (int tj = 0; tj < np / 256; ++tj)
            for (int t = 0; t < 512; ++t)
                for (int i = 0; i < 4; ++i)
                    for (int j = 0; j < 2; ++j)
                        for (int q = 0; q < 16; ++q) {
                            const int w = t / 64, l = t % 64, wm = w / 4, wn = w % 4;
                            const int row = ti * 256 + 128 * wm + 32 * i + 8 * (q / 4) + 4 * (l / 32) + q % 4;
                            const int col = tj * 256 + 64 * wn + 32 * j + l % 32;
                            const size_t chunk = (size_t)(4 * i + 2 * j + q / 8) * 512 + t;
                            const size_t want = (size_t)(ti * (np / 256) + tj) * 65536 + chunk * 8 + q % 8;
                            if (muon::lo_offset(row, col, np) != want) ++bad;
                        }
    std::printf("mismatches %ld\n", bad);
    return bad != 0;
}
"""


def test_lo_offset_is_the_update_accumulator_layout(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not available")
    src = tmp_path / "lo_layout.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "lo_layout"
    build = subprocess.run([hipcc, "-O1", "-I", CSRC, str(src), "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "mismatches 0" in run.stdout
