"""GEMM tiles find their matrix through runs of equal tile counts (run_matrix in
csrc/muon_internal.h), checked on the CPU against the prefix-sum search (find_matrix)
for every tile of 400 seeded lists: sorted runs of a few sizes, as the plan lays them
out, and arbitrary tile counts; lists of at most NS_ARG_RUNS runs also through the
runs passed by value (run_matrix_args).
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "matrix_aware_optimizer_amd", "csrc")

RUNS_PROGRAM = r"""
#include "muon_internal.h"
#include <cstdio>
#include <vector>
#include <random>
// GEMM tiles find their matrix through runs of equal tile counts (run_matrix); every
// tile of a list must land on the matrix and local index the prefix sums give.
int main() {
    std::mt19937 rng(7);
    long bad = 0, lists = 0, by_args = 0;
    for (int trial = 0; trial < 400; ++trial) {
        const int nmat = 1 + static_cast<int>(rng() % 40);
        std::vector<int32_t> tiles(nmat), prefix(nmat + 1, 0);
        const int kinds = 1 + static_cast<int>(rng() % 4);
        for (int k = 0; k < nmat; ++k) {
            // sorted runs of a few sizes, as the plan lays them out, or arbitrary counts
            tiles[k] = trial % 3 ? 1 + static_cast<int>((k * kinds / nmat + 1) * (1 + trial % 7)) : 1 + static_cast<int>(rng() % 9);
            prefix[k + 1] = prefix[k] + tiles[k];
        }
        std::vector<muon::TileRun> runs;
        for (int k = 0; k < nmat; ++k)
            if (runs.empty() || runs.back().tiles != tiles[k]) runs.push_back(muon::TileRun{prefix[k], k, tiles[k]});
        for (int t = 0; t < prefix[nmat]; ++t) {
            int local;
            const int mi = muon::run_matrix(runs.data(), static_cast<int>(runs.size()), t, local);
            const int want = muon::find_matrix(prefix.data(), nmat, t);
            if (mi != want || local != t - prefix[want] || local < 0 || local >= tiles[want]) ++bad;
            if (static_cast<int>(runs.size()) <= muon::NS_ARG_RUNS) {
                muon::TileRun arg[muon::NS_ARG_RUNS];
                for (int i = 0; i < muon::NS_ARG_RUNS; ++i)
                    arg[i] = i < static_cast<int>(runs.size()) ? runs[i] : muon::TileRun{0, 0, 1};
                int local2;
                const int mi2 = muon::run_matrix_args(arg, static_cast<int>(runs.size()), t, local2);
                if (mi2 != want || local2 != local) ++bad;
                ++by_args;
            }
        }
        ++lists;
    }
    std::printf("lists %ld tiles through the argument runs %ld mismatches %ld\n", lists, by_args, bad);
    return bad != 0 || by_args == 0;
}
"""


def test_tile_runs_find_every_tiles_matrix(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not available")
    src = tmp_path / "runs.cpp"
    src.write_text(RUNS_PROGRAM)
    exe = tmp_path / "runs"
    build = subprocess.run([hipcc, "-O1", "-I", CSRC, str(src), "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "mismatches 0" in run.stdout
