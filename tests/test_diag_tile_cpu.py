"""Diagonal tiles of the symmetric products (diag_modes and CStage in csrc/ns_gemm.hip), checked on the CPU.

A diagonal 256 x 256 tile of A = X X^T or of B = b A + c A A needs only its blocks
(R, C) with R <= C (8 x 8 blocks of 32 x 32): the epilogue stores the upper triangle
directly and mirrored.  The kernel forms each strictly upper block once, either in its
own slot or as the lower twin (C, R) = (R, C)^T in the twin's slot, staged transposed.
This test restates the slot rule and the two staging address maps in Python and checks:

- every block with R <= C is formed exactly once, no slot forms a block nobody stores;
- the work per SIMD is 9 blocks when a SIMD runs the waves with equal wn, and at most 10
  when it runs waves 2 s and 2 s + 1 (16 for the full tile);
- every element of the upper blocks is staged exactly once, at the column-major staging
  address of its own (row, column), with the value of that element or of its transpose.
"""
from __future__ import annotations

WAVES_M, WAVES_N = 2, 4
SKIP, NATIVE, SWAP = 0, 1, 2


def csw(c: int) -> int:
    return (c & 31) ^ (((c >> 5) & 1) << 2)


def mode(wm: int, wn: int, i: int, j: int) -> int:
    R, C = 4 * wm + i, 2 * wn + j
    pair = (R >> 1) == (C >> 1)
    if R == C or (R < C and (pair or not (C & 1))):
        return NATIVE
    if R > C and not pair and (R & 1):
        return SWAP
    return SKIP


def staged_addr(r: int, c: int) -> int:
    """Byte address of tile element (r, c) in the column-major staging."""
    return c * 512 + 8 * ((r >> 2) ^ csw(c)) + 2 * (r & 3)


def formed_blocks():
    out = {}
    for wave in range(8):
        wm, wn = wave // WAVES_N, wave % WAVES_N
        for i in range(4):
            for j in range(2):
                R, C = 4 * wm + i, 2 * wn + j
                md = mode(wm, wn, i, j)
                if md == NATIVE:
                    out.setdefault((R, C), []).append(wave)
                elif md == SWAP:
                    out.setdefault((C, R), []).append(wave)
    return out


def test_each_upper_block_formed_once():
    formed = formed_blocks()
    upper = {(R, C) for R in range(8) for C in range(8) if R <= C}
    assert set(formed) == upper
    assert all(len(v) == 1 for v in formed.values())


def test_simd_balance():
    per_wave = [0] * 8
    for waves in formed_blocks().values():
        per_wave[waves[0]] += 1
    assert sum(per_wave) == 36
    # a SIMD runs waves s and s + 4 (equal wn) ...
    assert [per_wave[s] + per_wave[s + 4] for s in range(4)] == [9, 9, 9, 9]
    # ... or waves 2 s and 2 s + 1
    assert max(per_wave[2 * s] + per_wave[2 * s + 1] for s in range(4)) <= 10


def test_staging_addresses():
    """put (native) and put_transposed (swapped) stage each upper element once, in place."""
    staged = {}
    for wave in range(8):
        wm, wn = wave // WAVES_N, wave % WAVES_N
        for lane in range(64):
            h = lane >> 5
            for i in range(4):
                for j in range(2):
                    md = mode(wm, wn, i, j)
                    if md == SKIP:
                        continue
                    R, C = 4 * wm + i, 2 * wn + j
                    for g in range(4):
                        # accumulator register 4 g + e: element (32 R + 8 g + 4 h + e, 32 C + lane % 32)
                        src = [(32 * R + 8 * g + 4 * h + e, 32 * C + (lane & 31)) for e in range(4)]
                        if md == NATIVE:
                            c = 64 * wn + 32 * j + (lane & 31)
                            wbase = c * 512 + 256 * wm + 8 * (h ^ csw(c))
                            base = wbase ^ (64 * i + 16 * g)
                            vals = src
                        else:
                            # quad transpose: lane 4 q + t takes v[p] = element of quad lane p, row t
                            q, t = (lane & 31) >> 2, lane & 3
                            vals = [(32 * R + 8 * g + 4 * h + t, 32 * C + 4 * q + p) for p in range(4)]
                            c = 32 * R + 8 * g + 4 * h + t
                            u = 8 * C + q
                            base = c * 512 + 8 * (u ^ csw(c))
                        for e in range(4):
                            addr = base + 2 * e
                            assert addr not in staged, "two writes to one staging slot"
                            staged[addr] = vals[e]
    count = 0
    for r in range(256):
        for c in range(256):
            if r // 32 > c // 32:
                continue
            a = staged_addr(r, c)
            assert a in staged, (r, c)
            assert staged[a] in ((r, c), (c, r)), (r, c, staged[a])
            count += 1
    assert count == 36 * 1024
    assert len(staged) == count
