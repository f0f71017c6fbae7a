// LDS staging of the bf16 iterate's lo part in the momentum kernel: one 64 x 64
// elementwise tile is put in the order of lo_offset (muon_internal.h) and stored as
// whole 1 KB chunk rows of the update's accumulator layout.  Host-callable, so that a
// CPU test can run the staging over every tile against lo_offset.
#pragma once
#include "muon_internal.h"

namespace muon {

// The momentum kernel produces lo one 64 x 64 elementwise tile at a time and stages it
// in LDS in the order of lo_offset: the tile covers 2 x 2 of the 32 x 32 blocks of one
// update wave, i.e. 8 chunk rows v of 64 lanes, and staged chunk k = 64 piece + lane is
// chunk row v = 4 i_a + piece (i_a: the tile's first block row) of that wave.  Chunk k
// sits at LDS chunk lo_stage_slot(k): the XOR spreads one wave instruction's 2-byte
// writes (k differing in bits 3-7) over 16 banks instead of 4, and keeps each aligned
// group of 16 chunks (one 16-lane read) in place.
__host__ __device__ constexpr int lo_stage_slot(int k) { return k ^ ((k >> 4) & 15); }
constexpr int LO_STAGE_CHUNKS = EW_TILE * EW_TILE / 8;

// Stage the lo of the 8 columns c0 .. c0 + 7 (c0 % 8 == 0) of tile row r, packed two to
// a word (l[k] holds columns 2 k and 2 k + 1).
__host__ __device__ inline void lo_stage8(uint16_t* stage, int r, int c0, const unsigned (&l)[4]) {
    const int rr = r & 31;
    const int q = 4 * (rr >> 3) + (rr & 3);               // accumulator register
    const int lane = (c0 & 31) + 32 * ((rr >> 2) & 1);
    const int piece = 4 * (r >> 5) + 2 * (c0 >> 5) + (q >> 3);
    for (int e = 0; e < 8; ++e)
        stage[lo_stage_slot(piece * 64 + lane + e) * 8 + (q & 7)] = static_cast<uint16_t>(l[e >> 1] >> (16 * (e & 1)));
}

// Index in the lo buffer of the first element of staged chunk k of the elementwise
// tile whose origin is (i0, j0) (multiples of 64), padded width np.
__host__ __device__ inline size_t lo_chunk_dst(int i0, int j0, int np, int k) {
    const int r0 = i0 & 255, c0 = j0 & 255;
    const size_t tile = static_cast<size_t>(i0 >> 8) * (np >> 8) + (j0 >> 8);
    const int w = 4 * (r0 >> 7) + (c0 >> 6), ia = (r0 >> 5) & 3;
    return tile * 65536 + static_cast<size_t>((4 * ia + (k >> 6)) * 512 + w * 64 + (k & 63)) * 8;
}

}  // namespace muon
