"""The bf16 iterate's lo layout (lo_offset in csrc/muon_internal.h, staging in csrc/lo_stage.h), checked on the CPU.

lo_offset places element (row, col) of the padded NS-frame matrix at the position the
update kernel's thread reads it from and writes it to: thread t = 64 w + l (wave
w = 4 wm + wn, lane l) holds register q of 32 x 32 block (i, j) for tile row
128 wm + 32 i + 8 (q / 4) + 4 (l / 32) + q % 4 and column 64 wn + 32 j + l % 32 (the
MFMA 32 x 32 output layout), in 16-byte chunk v = 4 i + 2 j + q / 8 of the tile.  The
test compiles a small host program against the header and checks that lo_offset is a
bijection onto the padded matrix and agrees with that per-thread description.  It also
runs the momentum kernel's LDS staging of lo (lo_stage8, lo_stage_slot, lo_chunk_dst) on
the host over every 64 x 64 elementwise tile and checks that each element reaches its
lo_offset.
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
#include "lo_stage.h"
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
    if (bad) return 1;

    // The momentum kernel's staging: every 64 x 64 elementwise tile of the matrix, its
    // 512 row groups of 8 staged with lo_stage8 (values name their element), then chunk k
    // copied from LDS chunk lo_stage_slot(k) to lo_chunk_dst.  Each element must land at
    // lo_offset, and no two staged chunks may share an LDS chunk.
    long bad_stage = 0;
    std::vector<uint16_t> stage(muon::LO_STAGE_CHUNKS * 8);
    for (int i0 = 0; i0 < mp; i0 += 64)
        for (int j0 = 0; j0 < np; j0 += 64) {
            for (auto& x : stage) x = 0;
            for (int r = 0; r < 64; ++r)
                for (int c0 = 0; c0 < 64; c0 += 8) {
                    unsigned l[4];
                    for (int k = 0; k < 4; ++k)
                        l[k] = (unsigned)(1 + r * 64 + c0 + 2 * k) | ((unsigned)(1 + r * 64 + c0 + 2 * k + 1) << 16);
                    muon::lo_stage8(stage.data(), r, c0, l);
                }
            std::vector<int> slot_seen(muon::LO_STAGE_CHUNKS, 0);
            for (int k = 0; k < 512; ++k) ++slot_seen[muon::lo_stage_slot(k)];
            int used = 0;
            for (int x : slot_seen) {
                if (x > 1) ++bad_stage;
                used += x;
            }
            if (used != 512) ++bad_stage;
            for (int k = 0; k < 512; ++k) {
                const size_t dst = muon::lo_chunk_dst(i0, j0, np, k);
                for (int e = 0; e < 8; ++e) {
                    const int v = stage[muon::lo_stage_slot(k) * 8 + e];
                    if (v == 0) { ++bad_stage; continue; }
                    const int r = (v - 1) / 64, c = (v - 1) % 64;
                    if (muon::lo_offset(i0 + r, j0 + c, np) != dst + e) ++bad_stage;
                }
            }
        }
    std::printf("stage mismatches %ld\n", bad_stage);
    return bad_stage != 0;
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
    assert "stage mismatches 0" in run.stdout

