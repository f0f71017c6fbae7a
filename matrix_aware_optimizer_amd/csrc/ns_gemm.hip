// Newton-Schulz GEMMs on the gfx950 matrix cores.
//
// One step of the quintic iteration ([Muon优化器] linsight.cn/f25d614e.html,
// zeropower_via_newtonschulz and section "Newton-Schulz 迭代——高效实现与系数
// 优化") on the NS-frame iterate X (m x n, m <= n):
//     A  = X X^T                 (Gram: symmetric, upper half tiles)
//     B  = b A + c A A           (polynomial: A A = A A^T, upper half tiles)
//     X' = a X + B X             (update)
// Products C[i][j] = sum_k P[i][k] Q[k][j].  P is always stored k-contiguous
// (rows of X for the Gram, of A for the polynomial, of B for the update).  Q
// is k-contiguous too for the Gram and the polynomial (Q^T = X and A), and
// k-major for the update, where Q = X is read in its own row-major layout.
//
// Engine: a 256 x 256 (bf16) or 128 x 128 (fp32) block tile per workgroup of
// 8 waves (2 x 4, two waves per SIMD); each wave owns a 128 x 64 (64 x 32)
// sub-tile of 32 x 32 MFMA blocks (v_mfma_f32_32x32x16_bf16 /
// v_mfma_f32_32x32x2_f32, fp32 accumulation).  A k-step stages 128 bytes of
// every k-contiguous operand row (or 64 / 32 k-rows of a k-major operand, one
// 512-byte tile row each) in LDS with direct global->LDS loads
// (global_load_lds_dwordx4, no VGPR staging) into a ring of five slabs (one
// slab = one operand's k-step); the loads of the next Q slab and of the P slab
// after it are spread between the current k-step's MFMA groups, and MFMA
// fragments are double-buffered in registers.  The loop is rotated: the barrier
// that opens a k-step sits before the previous step's last k-slice, whose MFMAs
// then cover the new step's first fragment reads.
//
// LDS layouts.  k-contiguous rows: 16-byte chunks XOR-swizzled with bits 1..3
// of the row, so 32-row ds_read_b128 fragment reads are free of bank
// conflicts.  k-major rows: chunks swizzled with (row & 3) << 2, which moves
// the 64-byte piece a wave reads from each of 8 k-rows into all four 64-byte
// bank windows.  k-major bf16 fragments are read with ds_read_b64_tr_b16:
// within each group of 16 lanes the instruction hands lane l element (l & 3)
// of the 8 bytes addressed by lane 4e + (l >> 2) as its element e, so lanes
// addressing X[k0 + i/4][n0 + 4 (i%4)] receive column n0 + l, rows k0..k0+3:
// two such reads form the 8-element k-slice of an MFMA B operand.
//
// Epilogues.  bf16 outputs of the Gram, the polynomial and the update are
// staged column-major in LDS straight from the accumulator layout (one 8-byte
// write per 4 values) and stored as whole tile rows through transpose reads;
// symmetric outputs are also stored mirrored, through plain reads of the same
// staging.  The bf16 iterate's lo part is kept in the update's accumulator
// layout: the update reads a lo straight into its accumulators before the
// k-loop and writes lo' straight from them (hi' goes through the staging).
// The fp32 epilogues, the last update's W' and the
// c = 0 polynomial work from registers: a 4 x 4 transpose inside each lane
// quad (DPP) turns a lane's 4 rows x 1 column of a 32 x 32 block into 1 row x
// 4 columns, and for bf16 a swap between lanes c and c ^ 4 then gives each lane
// 8 columns (16 bytes).  Buffers are zero-padded to
// the block tile, so there are no edge masks, and k-loops run over the real
// extent rounded up to a k-step.
//
// Grouping: one launch covers every matrix of the call.  The tile space is the
// concatenation of all matrices' tiles (per-matrix prefix sums, largest
// matrices first), one workgroup per tile.  The hardware deals workgroups
// round-robin over the 8 XCDs; block ids are remapped so that each XCD works
// on runs of consecutive tiles (32 for the update, 16 for the symmetric
// products), whose operand blocks then share its L2.
#include <cmath>

#include "muon_internal.h"

namespace muon {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// native 16-byte vector (HIP's uint4 is a wrapper struct that defeats register promotion)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Cfg;
template <> struct Cfg<uint16_t> {      // 16-byte chunk = 8 bf16 along k
    static constexpr int BM = GEMM_TILE_BF16, BN = GEMM_TILE_BF16;
};
template <> struct Cfg<float> {         // 16-byte chunk = 4 fp32 along k
    static constexpr int BM = GEMM_TILE_F32, BN = GEMM_TILE_F32;
};

constexpr int WAVES_M = 2, WAVES_N = 4;
constexpr int NWAVES = WAVES_M * WAVES_N;
static_assert(NWAVES * 64 == GEMM_THREADS, "GEMM_THREADS must match the wave layout");
constexpr int CHUNKS_PER_ROW = 8;            // 8 x 16 B = 128 B of k per row per k-step
constexpr int QROW_CHUNKS = 32;              // k-major rows: 512 B = one tile width
// XCD_RUN: consecutive tiles per XCD, by phase (measured best on the transformer set:
// 32 for the update's grouped 4 x 8 blocks, 16 for the upper-triangle tiles of the Gram
// and the polynomial, 1.3 and 0.6 % faster there than 32)
constexpr int XCD_COUNT = 8, XCD_RUN_UPD = 32, XCD_RUN_SYM = 16;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) char lds_byte_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) float lds_float_t;

// The wave's index in the workgroup as a wave-uniform (scalar) value, so that LDS
// destinations of the direct-to-LDS loads (M0) and per-wave branch conditions are
// formed with scalar instructions instead of one v_readfirstlane per use.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)); }

// One 16-byte chunk per lane of both operands, accumulated into a 32 x 32 block.
__device__ inline void mfma_chunk(f32x16_t& acc, const u32x4& a, const u32x4& b, uint16_t) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
__device__ inline void mfma_chunk(f32x16_t& acc, const u32x4& a, const u32x4& b, float) {
    // lane half h holds k = 4h + e of this chunk pair; MFMA e reduces over both halves
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// Physical position of logical 16-byte chunk c of k-contiguous LDS row `row`.
__device__ __forceinline__ int swz(int row, int c) { return row * CHUNKS_PER_ROW + (c ^ ((row >> 1) & 7)); }
// Physical position of logical 16-byte chunk c of k-major LDS row `kr` (relative to the region).
__device__ __forceinline__ int qswz(int kr, int c) { return kr * QROW_CHUNKS + (c ^ ((kr & 3) << 2)); }

// Runs of XCD_RUN consecutive tiles on one XCD: block b runs on XCD b % 8.
// A bijection on [0, nb); the tail beyond the last full round keeps its ids.
template <int XCD_RUN>
__device__ inline int xcd_run_remap(int b, int nb) {
    const int full = (nb / (XCD_COUNT * XCD_RUN)) * (XCD_COUNT * XCD_RUN);
    if (b >= full) return b;
    const int xcd = b % XCD_COUNT, slot = b / XCD_COUNT;
    return ((slot / XCD_RUN) * XCD_COUNT + xcd) * XCD_RUN + slot % XCD_RUN;
}

// Update-tile decode: tiles are ordered in groups of GROUP_M tile rows, column-
// major inside a group, so a run of 32 consecutive tiles (what one XCD works
// on at a time) is a GROUP_M x (32 / GROUP_M) block that shares GROUP_M row
// blocks of B and 32 / GROUP_M column blocks of X in its L2.
constexpr int GROUP_M = 4;
__device__ inline void grouped_decode(int q, int tm, int tn, int& ti, int& tj) {
    const int per_group = GROUP_M * tn;
    const int g = q / per_group, r = q % per_group;
    const int first = g * GROUP_M;
    const int gsize = min(tm - first, GROUP_M);
    ti = first + r % gsize;
    tj = r / gsize;
}

// Upper-triangle tile decode: local index -> (ti, tj), ti <= tj, row-major.
__device__ inline void sym_decode(int q, int T, int& ti, int& tj) {
    int i = 0, len = T;
    while (q >= len) { q -= len; ++i; --len; }
    ti = i;
    tj = i + q;
}

// Diagonal tiles of a symmetric product (bf16 256 x 256, 8 x 8 blocks of 32 x 32).
// Only the blocks (R, C) with R <= C are stored, and P = Q, so block (C, R) is the
// transpose of block (R, C): a wave may form the lower block (R, C) of its own slot
// and stage it transposed in place of (C, R).  Each strictly upper block is formed
// once, in its own slot or in its twin's, so that the 36 blocks fall 9 to each SIMD
// when a SIMD runs the two waves with the same wn (which own the columns 2 wn,
// 2 wn + 1, and so the twins of the rows 2 wn, 2 wn + 1), and 10 at most when it runs
// waves 2 s and 2 s + 1.
//   R == C, or R < C in one column pair:      native;
//   R < C in different pairs:                 native for even C, else the twin forms it;
//   R > C in different pairs, R odd:          swapped (formed here, staged as (C, R));
//   otherwise:                                skipped.
// Two bits per slot (i, j) at 2 (2 i + j): 0 skip, 1 native, 2 swapped; wave-uniform.
constexpr unsigned DG_SKIP = 0u, DG_NATIVE = 1u, DG_SWAP = 2u;
__host__ __device__ constexpr unsigned diag_modes_of(int wave) {
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    unsigned m = 0;
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 2; ++j) {
            const int R = 4 * wm + i, C = 2 * wn + j;
            const bool pair = (R >> 1) == (C >> 1);
            unsigned md = DG_SKIP;
            if (R == C || (R < C && (pair || !(C & 1)))) md = DG_NATIVE;
            else if (R > C && !pair && (R & 1)) md = DG_SWAP;
            m |= md << (2 * (2 * i + j));
        }
    return m;
}
__host__ __device__ constexpr unsigned dg_mode(unsigned modes, int i, int j) { return (modes >> (2 * (2 * i + j))) & 3u; }
// fragment row i (A) or column block j (B) feeds some slot that is not skipped
__host__ __device__ constexpr bool dg_needs_a(unsigned modes, int i) {
    return dg_mode(modes, i, 0) != DG_SKIP || dg_mode(modes, i, 1) != DG_SKIP;
}
__host__ __device__ constexpr bool dg_needs_b(unsigned modes, int j) {
    return dg_mode(modes, 0, j) != DG_SKIP || dg_mode(modes, 1, j) != DG_SKIP || dg_mode(modes, 2, j) != DG_SKIP ||
           dg_mode(modes, 3, j) != DG_SKIP;
}
__device__ __forceinline__ unsigned diag_modes() {
    return diag_modes_of(wave_id());
}

// QK: Q is k-major (row k holds BN consecutive columns), else k-contiguous.
template <typename T, bool QK>
struct Engine {
    static constexpr int BM = Cfg<T>::BM, BN = Cfg<T>::BN;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int SM = WM / 32, SN = WN / 32;
    static constexpr int KS = CHUNKS_PER_ROW * 16 / static_cast<int>(sizeof(T));   // k per k-step
    static constexpr int SLAB = BM * CHUNKS_PER_ROW;   // 16-byte chunks of one operand's k-step slab
    static constexpr int SLOTS = 5;                    // LDS ring of slabs
    static constexpr int LDS_CHUNKS = SLOTS * SLAB;
    static constexpr int HL = SLAB / 64 / NWAVES;      // loads per wave per slab
    static constexpr int SUB = CHUNKS_PER_ROW / 2;     // MFMA k-slices per k-step
    static constexpr int GROUPS = SUB * SM;            // MFMA groups per k-step
    static_assert(BM == BN, "P and Q slabs have one size");
    static_assert(2 * HL <= GROUPS, "one load per MFMA group at most");
    // loads of P(kt + 2) issued before the barrier that opens step kt + 1 (the last slice's)
    static constexpr int PB = ((SUB - 1) * SM < 2 * HL ? (SUB - 1) * SM : 2 * HL) - HL;
    static_assert(PB >= 0 && PB <= HL, "the loads of Q(kt + 1) precede the last slice");
    static_assert(SM >= SN, "fragment prefetch pairs A row i with B row i");
    static_assert(!QK || BN * static_cast<int>(sizeof(T)) == QROW_CHUNKS * 16, "k-major rows are one tile wide");
    static_assert(!QK || KS * QROW_CHUNKS == SLAB, "k-major slab holds KS rows");

    // Source of DMA load j of this wave for a k-major slab whose first k-row is at Q
    // (pitch ldq bytes): the load fills slab chunks [(wave*HL + j)*64, +64) in lane
    // order, and each lane fetches the logical chunk that the swizzle puts there.
    static __device__ __forceinline__ const char* kmajor_src(const char* Q, size_t ldq, int j) {
        const int chunk = (static_cast<int>(threadIdx.x >> 6) * HL + j) * 64 + static_cast<int>(threadIdx.x & 63);
        const int kr = chunk / QROW_CHUNKS;
        const int lq = (chunk % QROW_CHUNKS) ^ ((kr & 3) << 2);
        return Q + kr * ldq + lq * 16;
    }
    // Issue this wave's share of the DMA of one k-major slab into LDS slot `slot`.
    static __device__ __forceinline__ void load_kmajor_slab(const char* Q, size_t ldq, u32x4* lds, int slot) {
        const int wave = wave_id();
#pragma unroll
        for (int j = 0; j < HL; ++j)
            __builtin_amdgcn_global_load_lds((const void*)kmajor_src(Q, ldq, j),
                                             (lds_ptr_t)(lds + slot * SLAB + (wave * HL + j) * 64), 16, 0, 0);
    }

    // acc[i][j] = init[i][j] + sum_k P[row0 + i][k] * Q(k, col0 + j) over the whole k
    // range, where P points at row row0 (pitch ldp bytes) and Q at row col0
    // (k-contiguous) or at column col0 of k-row 0 (k-major), pitch ldq bytes.
    // init(acc) fills the accumulators once the first slabs' loads are in flight;
    // hook(kt, Q slab of step kt, acc) runs when step kt's slabs are ready.
    //
    // Slabs are numbered 2 kt (P) and 2 kt + 1 (Q) and slab s lives in LDS slot s % 5.
    // A barrier opens step kt once each wave's loads of P(kt) and Q(kt) are done, so
    // only P(kt + 1) stays in flight across it; after it no wave reads the slots of
    // step kt - 1 again, and step kt refills them with Q(kt + 1) and P(kt + 2).
    // The loop is rotated: that barrier sits before the last k-slice of step kt - 1
    // (after the prologue for step 0), whose MFMAs then cover the first fragment reads
    // of step kt; each wave also waits for its LDS reads before it.
    //
    // p_half: only the first BM / 2 rows of P are real (the last tile row of a matrix
    // whose padded size adds at most BM / 2 rows).  The waves owning rows BM / 2 ..
    // BM - 1 (wm = 1, which also load exactly those P rows) then issue no P loads, read
    // no fragments and run no MFMAs: their accumulators keep init's value (zero for
    // every caller that passes p_half), so the padding stays exactly zero.  They still
    // load their share of Q and take part in every barrier, and wait for all their
    // loads wherever the other waves keep P loads in flight.
    template <typename Init, typename Hook>
    static __device__ __attribute__((always_inline)) void run(const char* __restrict__ P, size_t ldp, const char* __restrict__ Q,
                                      size_t ldq, int ksteps, u32x4* lds, f32x16_t (&acc)[SM][SN], Init init,
                                      Hook hook, bool p_half = false) {
        static_assert(HL * 64 / CHUNKS_PER_ROW == BM / NWAVES && 2 * WAVES_N == NWAVES,
                      "wave w loads P rows w BM / 8 ..: the waves with wm = 1 load exactly rows BM / 2 .. BM - 1");
        if (p_half && wave_id() / WAVES_N == 1)
            run_impl<true, false>(P, ldp, Q, ldq, ksteps, lds, acc, init, hook);
        else
            run_impl<false, false>(P, ldp, Q, ldq, ksteps, lds, acc, init, hook);
    }

    // A diagonal tile of a symmetric product (P = Q, k-contiguous): only the P slabs
    // are loaded, the B fragments and the hook read them too, and the slots that
    // diag_modes() skips run no MFMAs (their accumulators keep init's value).
    template <typename Init, typename Hook>
    static __device__ __attribute__((always_inline)) void run_diag(const char* __restrict__ P, size_t ldp, int ksteps,
                                                                   u32x4* lds, f32x16_t (&acc)[SM][SN], Init init,
                                                                   Hook hook) {
        static_assert(!QK && SM == 4 && SN == 2 && BM == 256 && NWAVES == 8, "diag_modes' block geometry");
        // one copy of the loop per wave, so that the skipped MFMAs and fragment reads
        // drop out at compile time (a branch per MFMA costs the loop its LDS-read overlap)
        switch (wave_id()) {
            case 0: run_impl<false, true, diag_modes_of(0)>(P, ldp, P, ldp, ksteps, lds, acc, init, hook); break;
            case 1: run_impl<false, true, diag_modes_of(1)>(P, ldp, P, ldp, ksteps, lds, acc, init, hook); break;
            case 2: run_impl<false, true, diag_modes_of(2)>(P, ldp, P, ldp, ksteps, lds, acc, init, hook); break;
            case 3: run_impl<false, true, diag_modes_of(3)>(P, ldp, P, ldp, ksteps, lds, acc, init, hook); break;
            case 4: run_impl<false, true, diag_modes_of(4)>(P, ldp, P, ldp, ksteps, lds, acc, init, hook); break;
            case 5: run_impl<false, true, diag_modes_of(5)>(P, ldp, P, ldp, ksteps, lds, acc, init, hook); break;
            case 6: run_impl<false, true, diag_modes_of(6)>(P, ldp, P, ldp, ksteps, lds, acc, init, hook); break;
            default: run_impl<false, true, diag_modes_of(7)>(P, ldp, P, ldp, ksteps, lds, acc, init, hook); break;
        }
    }

    template <bool IDLE, bool DIAGM, unsigned MODES = 0u, typename Init, typename Hook>
    static __device__ __attribute__((always_inline)) void run_impl(const char* __restrict__ P, size_t ldp,
                                      const char* __restrict__ Q, size_t ldq, int ksteps, u32x4* lds,
                                      f32x16_t (&acc)[SM][SN], Init init, Hook hook) {
        const int tid = threadIdx.x;
        const int lane = tid & 63, wave = wave_id();
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;

        // Load j of this wave fills slab chunks [(wave*HL + j)*64, +64) in lane order;
        // the source address holds the logical chunk that the swizzle puts there.
        const char* srcp[HL];
        const char* srcq[HL];
#pragma unroll
        for (int j = 0; j < HL; ++j) {
            const int chunk = (wave * HL + j) * 64 + lane;
            const int row = chunk / CHUNKS_PER_ROW;
            const int lc = (chunk % CHUNKS_PER_ROW) ^ ((row >> 1) & 7);
            srcp[j] = P + row * ldp + lc * 16;
            srcq[j] = QK ? kmajor_src(Q, ldq, j) : Q + row * ldq + lc * 16;
        }
        const size_t pstep = CHUNKS_PER_ROW * 16;
        const size_t qstep = QK ? static_cast<size_t>(KS) * ldq : static_cast<size_t>(CHUNKS_PER_ROW * 16);
        auto issue = [&](int kt, bool q, int slot, int j) {
            lds_ptr_t d = (lds_ptr_t)(lds + slot * SLAB + (wave * HL + j) * 64);
            const char* s = q ? srcq[j] + static_cast<size_t>(kt) * qstep : srcp[j] + static_cast<size_t>(kt) * pstep;
            __builtin_amdgcn_global_load_lds((const void*)s, d, 16, 0, 0);
        };
        if constexpr (!IDLE) {
#pragma unroll
            for (int j = 0; j < HL; ++j) issue(0, false, 0, j);
        }
        if constexpr (!DIAGM) {
#pragma unroll
            for (int j = 0; j < HL; ++j) issue(0, true, 1, j);
        }
        if (!IDLE && ksteps > 1) {
#pragma unroll
            for (int j = 0; j < HL; ++j) issue(1, false, 2, j);
        }
        init(acc);

        const int half = lane >> 5;
        const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
        // B operand of k-slice s (16 bf16 or 8 fp32 of k) for 32-column block j of the Q slab at LQ
        auto read_b = [&](const u32x4* LQ, int j, int s) -> u32x4 {
            if (!QK) return LQ[swz(brow + j * 32, 2 * s + half)];
            const lds_byte_t* Lq = (const lds_byte_t*)LQ;
            if (sizeof(T) == 2) {
                const int i16 = lane & 15, g16 = lane >> 4;
                const int col = wn * WN + j * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
                const int kr = 16 * s + 8 * (g16 >> 1) + (i16 >> 2);
                const int cb = (col & 7) * 2;
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4_t*)(Lq + qswz(kr, col >> 3) * 16 + cb));
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4_t*)(Lq + qswz(kr + 4, col >> 3) * 16 + cb));
                const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
                return u32x4{l2.x, l2.y, h2.x, h2.y};
            } else {
                // MFMA e of the chunk pair uses k = 8 s + 4 half + e
                const int col = wn * WN + j * 32 + (lane & 31);
                const int kr = 8 * s + 4 * half;
                const int cb = (col & 3) * 4;
                u32x4 v;
                v.x = __float_as_uint(*(const lds_float_t*)(Lq + qswz(kr + 0, col >> 2) * 16 + cb));
                v.y = __float_as_uint(*(const lds_float_t*)(Lq + qswz(kr + 1, col >> 2) * 16 + cb));
                v.z = __float_as_uint(*(const lds_float_t*)(Lq + qswz(kr + 2, col >> 2) * 16 + cb));
                v.w = __float_as_uint(*(const lds_float_t*)(Lq + qswz(kr + 3, col >> 2) * 16 + cb));
                return v;
            }
        };

        u32x4 fa[2][SM], fb[2][SN];
        // fp32 products sum in two levels: each run of SUM_BLOCK k-steps (1024 values of k)
        // into part, which is then added to acc.  A single running fp32 sum over k carries a
        // rounding error that grows like sqrt(k) (about 1e-4 relative at k = 2^20); two
        // levels bring it to about sqrt(1024) + sqrt(k / 1024).  The fp32 tile's
        // accumulators are 32 registers, so the second set is cheap; bf16 keeps one level.
        constexpr bool TWO_LEVEL = sizeof(T) == 4;
        constexpr int SUM_BLOCK = 32;
        f32x16_t part[TWO_LEVEL ? SM : 1][TWO_LEVEL ? SN : 1];
        if constexpr (TWO_LEVEL) {
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j) part[i][j] = f32x16_t{};
        }
        // step 0's slabs (P(1) may still be in flight), then its first fragments
        if (!IDLE && ksteps > 1)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(HL) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        // a diagonal tile reads its B fragments from the P slab (same rows, same bytes),
        // and only the fragments that its slots use (the conditions fold at compile time)
        auto need_a = [](int i) { return !DIAGM || dg_needs_a(MODES, i); };
        auto need_b = [](int j) { return !DIAGM || dg_needs_b(MODES, j); };
        if constexpr (!IDLE) {
#pragma unroll
            for (int i = 0; i < SM; ++i)
                if (need_a(i)) fa[0][i] = lds[swz(arow + i * 32, half)];
#pragma unroll
            for (int j = 0; j < SN; ++j)
                if (need_b(j)) fb[0][j] = read_b(DIAGM ? lds : lds + SLAB, j, 0);
        }

        int sp = 0;   // slot of P(kt); Q(kt) sits in the next one
        for (int kt = 0; kt < ksteps; ++kt) {
            const int sq = sp + 1 == SLOTS ? 0 : sp + 1;
            const int s3 = sp >= 2 ? sp - 2 : sp + 3;   // slot of Q(kt + 1)
            const int s4 = sp >= 1 ? sp - 1 : sp + 4;   // slot of P(kt + 2)
            const int np = sp >= 3 ? sp - 3 : sp + 2;   // slot of P(kt + 1)
            const u32x4* L = lds + sp * SLAB;
            const u32x4* LQ = DIAGM ? L : lds + sq * SLAB;
            hook(kt, (const lds_byte_t*)LQ, acc);
            const bool more1 = kt + 1 < ksteps, more2 = kt + 2 < ksteps;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < SUB; ++s) {
                if (s == SUB - 1 && more1) {
                    // Open step kt + 1 before this step's last slice, whose MFMAs then
                    // cover the first fragment reads of the next step.  Every read of
                    // step kt's slabs (fragments and hook) has completed; this wave's
                    // loads of Q(kt + 1) and P(kt + 1) are done, only P(kt + 2) may be
                    // in flight.  After the barrier the slots of step kt are free.
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    if (!IDLE && more2)
                        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PB) : "memory");
                    else
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    asm volatile("s_barrier" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int cn = 2 * (s + 1) + half;
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    if constexpr (!IDLE) {
#pragma unroll
                        for (int j = 0; j < SN; ++j) {
                            if (!DIAGM || dg_mode(MODES, i, j) != DG_SKIP) {
                                if constexpr (TWO_LEVEL)
                                    mfma_chunk(part[i][j], fa[s & 1][i], fb[s & 1][j], T{});
                                else
                                    mfma_chunk(acc[i][j], fa[s & 1][i], fb[s & 1][j], T{});
                            }
                        }
                        if (s + 1 < SUB) {
                            if (need_a(i)) fa[(s + 1) & 1][i] = L[swz(arow + i * 32, cn)];
                            if (i < SN && need_b(i)) fb[(s + 1) & 1][i] = read_b(LQ, i, s + 1);
                        } else if (more1) {
                            if (need_a(i)) fa[0][i] = lds[np * SLAB + swz(arow + i * 32, half)];
                            if (i < SN && need_b(i)) fb[0][i] = read_b(lds + (DIAGM ? np : s3) * SLAB, i, 0);
                        }
                    }
                    const int g = s * SM + i;
                    if (!DIAGM && g < HL && more1) issue(kt + 1, true, s3, g);
                    if (!IDLE && g >= HL && g < 2 * HL && more2) issue(kt + 2, false, s4, g - HL);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (TWO_LEVEL) {
                if (kt % SUM_BLOCK == SUM_BLOCK - 1 || kt + 1 == ksteps) {
#pragma unroll
                    for (int i = 0; i < SM; ++i)
#pragma unroll
                        for (int j = 0; j < SN; ++j) {
                            acc[i][j] += part[i][j];
                            part[i][j] = f32x16_t{};
                        }
                }
            }
            sp = np;
        }
    }
};

// 4 consecutive elements along a row: load / store in the operand dtype.
template <typename T> __device__ inline float4 ld_quad(const void* p, size_t i);
template <> __device__ inline float4 ld_quad<float>(const void* p, size_t i) {
    return ld_f4(static_cast<const float*>(p) + i);
}
template <> __device__ inline float4 ld_quad<uint16_t>(const void* p, size_t i) {
    const u32x2_t q = ld_u2(static_cast<const uint16_t*>(p) + i);
    return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u),
                       __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xffff0000u));
}
template <typename T> __device__ inline void st_quad(void* p, size_t i, float4 v);
template <> __device__ inline void st_quad<float>(void* p, size_t i, float4 v) {
    st_f4(static_cast<float*>(p) + i, v);
}
template <> __device__ inline void st_quad<uint16_t>(void* p, size_t i, float4 v) {
    const u32x2_t q = {pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
    st_u2(static_cast<uint16_t*>(p) + i, q);
}
template <typename T> __device__ inline void st_elem(void* p, size_t i, float v);
template <> __device__ inline void st_elem<float>(void* p, size_t i, float v) { G(static_cast<float*>(p))[i] = v; }
template <> __device__ inline void st_elem<uint16_t>(void* p, size_t i, float v) {
    G(static_cast<uint16_t*>(p))[i] = f32_to_bf16(v);
}
__device__ inline float f4get(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
// Elements e with bit e of `mask` set; a whole-quad store when all are.
template <typename T> __device__ inline void st_quad_masked(void* p, size_t i, const float4& v, unsigned mask) {
    if (mask == 0xFu) {
        st_quad<T>(p, i, v);
    } else if (mask) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (mask & (1u << e)) st_elem<T>(p, i + e, f4get(v, e));
    }
}

// PH_POLY_LDS is the polynomial with b A added from the staged operand (c != 0);
// PH_POLY reads A again in the epilogue and serves any c.
// PH_UPDATE_APPLY is the last update of muon_step, writing W' instead of X'.
enum Phase { PH_GRAM = 0, PH_POLY = 1, PH_UPDATE = 2, PH_POLY_LDS = 3, PH_UPDATE_APPLY = 4 };

struct NoHook {
    template <typename A> __device__ __forceinline__ void operator()(int, const lds_byte_t*, A&) const {}
};


struct ZeroInit {
    template <typename A> __device__ __forceinline__ void operator()(A& acc) const {
#pragma unroll
        for (auto& row : acc)
#pragma unroll
            for (auto& blk : row)
#pragma unroll
                for (int r = 0; r < 16; ++r) blk[r] = 0.0f;
    }
};

// The bf16 update starts from a lo: lo is stored in this workgroup's accumulator
// layout (lo_offset), so thread t's 16 chunks of the tile, chunk (i, j, h) at
// ((4 i + 2 j + h) * 512 + t) * 16 bytes, are its registers 8 h .. 8 h + 7 of
// block (i, j); each wave instruction reads 1 KB contiguous.
template <typename E>
struct LoInit {
    const uint16_t* lo;   // the tile's 64 Ki elements
    float a;
    template <typename A> __device__ __forceinline__ void operator()(A& acc) const {
        static_assert(E::SM == 4 && E::SN == 2, "lo_offset's block numbering");
        const u32x4* p = reinterpret_cast<const u32x4*>(lo) + threadIdx.x;
#pragma unroll
        for (int i = 0; i < E::SM; ++i)
#pragma unroll
            for (int j = 0; j < E::SN; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4 v = G(p)[((E::SN * i + j) * 2 + h) * GEMM_THREADS];
                    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[i][j][8 * h + e] = a * __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
                }
    }
};

// ----------------------------------------------------------------------------
// Epilogue helpers.  Accumulator register r of 32 x 32 block (i, j) holds, in
// lane l, element (8 (r >> 2) + 4 (l >> 5) + (r & 3), l & 31) of the block:
// for g = r >> 2 a lane holds 4 consecutive rows of one column.
// ----------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ float qperm(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// 4 x 4 transpose inside each quad of lanes: on entry lane t of the quad holds
// column t (v[p] = M[p][t]), on exit row t (v[p] = M[t][p]).
__device__ __forceinline__ void quad_transpose(float (&v)[4]) {
    const int t = threadIdx.x & 3;
    float s[4], x[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) s[p] = qperm<0xB1>(v[p]);   // from lane t ^ 1
#pragma unroll
    for (int p = 0; p < 4; ++p) x[p] = ((p ^ t) & 1) ? s[p ^ 1] : v[p];
#pragma unroll
    for (int p = 0; p < 4; ++p) s[p] = qperm<0x4E>(x[p]);   // from lane t ^ 2
#pragma unroll
    for (int p = 0; p < 4; ++p) v[p] = ((p ^ t) & 2) ? s[p ^ 2] : x[p];
}

// Lanes c and c ^ 4 of each 32-lane half hold the same rows (8 g + 4 h + t) and
// adjacent column quads after quad_transpose.  Swapping one quad of a pair of g
// values gives each lane 8 consecutive columns of one row: the lane of the even
// quad (bit 2 of the lane clear) takes row g0 = 2 gg, the other row g1 = 2 gg + 1,
// both starting at column (lane & 24) of the 32-column block.  16-byte accesses.
__device__ __forceinline__ unsigned swap_xor4(unsigned v) {
    return static_cast<unsigned>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x101F));   // lane ^ 4
}
__device__ __forceinline__ bool odd_quad() { return (threadIdx.x >> 2) & 1; }
// Lanes l and l ^ 32 hold the same column and rows 4 apart (8 g + 4 h + (0..3)).
__device__ __forceinline__ unsigned swap_xor32(unsigned v) {
    return static_cast<unsigned>(__builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 32) << 2, static_cast<int>(v)));
}

// Per-lane coordinates inside a wave's sub-tile.
template <typename E>
struct Coords {
    int raw_row, raw_col;   // untransposed: rows raw_row + 32 i + 8 g + (0..3), column raw_col + 32 j
    int tr_row, tr_col;     // transposed:   row tr_row + 32 i + 8 g, columns tr_col + 32 j + (0..3)
    __device__ Coords(int row0, int col0) {
        const int lane = threadIdx.x & 63, wave = wave_id();
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        const int c = lane & 31, h = lane >> 5;
        raw_row = row0 + wm * E::WM + 4 * h;
        raw_col = col0 + wn * E::WN + c;
        tr_row = raw_row + (c & 3);
        tr_col = col0 + wn * E::WN + (c & ~3);
    }
};

// Symmetric output (A or B): tile (ti, tj), ti <= tj, stored at (ti, tj) from
// the transposed layout and mirrored at (tj, ti) from the untransposed one.  A
// diagonal tile stores its upper triangle directly and its strictly upper
// triangle mirrored, so the stored matrix is exactly symmetric.
//   Gram:        value = scale * acc
//   polynomial:  value = b * A + c * acc   (A read at the mirrored position,
//                                            equal to the direct one by symmetry)
template <typename E, typename T, bool POLY>
__device__ __attribute__((always_inline)) void sym_epilogue_quad(f32x16_t (&acc)[E::SM][E::SN], int row0, int col0,
                                                            bool diag, void* dst, size_t ld, float scale,
                                                            const void* amat, float b, float c) {
    const Coords<E> q(row0, col0);
    float4 cur[E::SN * 4], nxt[E::SN * 4];
    auto fetch = [&](float4 (&buf)[E::SN * 4], int i) {
#pragma unroll
        for (int j = 0; j < E::SN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                buf[j * 4 + g] = ld_quad<T>(amat, static_cast<size_t>(q.raw_col + 32 * j) * ld + q.raw_row + 32 * i + 8 * g);
    };
    if (POLY) fetch(cur, 0);
#pragma unroll
    for (int i = 0; i < E::SM; ++i) {
        if (POLY && i + 1 < E::SM) fetch(nxt, i + 1);
#pragma unroll
        for (int j = 0; j < E::SN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float x = acc[i][j][4 * g + p];
                    v[p] = POLY ? fmaf(c, x, b * f4get(cur[j * 4 + g], p)) : scale * x;
                }
                // mirrored: elements (rr + p, cc) go to row cc, columns rr .. rr + 3
                const int rr = q.raw_row + 32 * i + 8 * g, cc = q.raw_col + 32 * j;
                unsigned mm = 0xFu;
                if (diag) {
                    mm = 0;
#pragma unroll
                    for (int p = 0; p < 4; ++p) mm |= (rr + p < cc) ? (1u << p) : 0u;
                }
                st_quad_masked<T>(dst, static_cast<size_t>(cc) * ld + rr, make_float4(v[0], v[1], v[2], v[3]), mm);
                // direct: row tr, columns tc .. tc + 3
                quad_transpose(v);
                const int tr = q.tr_row + 32 * i + 8 * g, tc = q.tr_col + 32 * j;
                unsigned md = 0xFu;
                if (diag) {
                    md = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) md |= (tr <= tc + e) ? (1u << e) : 0u;
                }
                st_quad_masked<T>(dst, static_cast<size_t>(tr) * ld + tc, make_float4(v[0], v[1], v[2], v[3]), md);
            }
        if (POLY) {
#pragma unroll
            for (int k = 0; k < E::SN * 4; ++k) cur[k] = nxt[k];
        }
    }
}

// bf16 symmetric output with 16-byte accesses.  For each pair of 8-row groups
// (g0 = 2 gg, g1 = 2 gg + 1) of a 32 x 32 block:
//   mirrored: lanes l and l ^ 32 swap one quad, so lane half h owns rows
//             8 g_h + (0..7) of its column and stores them as 8 consecutive
//             columns of the mirrored row;
//   direct:   after quad_transpose, lanes c and c ^ 4 swap one quad (as in the
//             update epilogue), giving 8 consecutive columns of one row.
// The polynomial's A is read the same way as the mirrored store (A[cc][8 g_h ..])
// and swapped back to the accumulator rows.  Diagonal tiles mask per element,
// exactly as the 4-element version does.
__device__ __forceinline__ void st_bf16x8_masked(uint16_t* p, const float (&v)[8], unsigned mask) {
    if (mask == 0xFFu) {
        G(reinterpret_cast<u32x4*>(p))[0] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    } else if (mask) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (mask & (1u << e)) G(p)[e] = f32_to_bf16(v[e]);
    }
}

template <typename E, bool POLY>
__device__ __attribute__((always_inline)) void sym_epilogue_bf16(f32x16_t (&acc)[E::SM][E::SN], int row0, int col0,
                                                                 bool diag, uint16_t* dst, size_t ld, float scale,
                                                                 const uint16_t* amat, float b, float c) {
    const Coords<E> q(row0, col0);
    const bool hh = (threadIdx.x >> 5) & 1;
    const bool odd = odd_quad();
    const int mbase = q.raw_row - (hh ? 4 : 0);   // first row of the wave's sub-tile
    u32x4 cur[E::SN * 2], nxt[E::SN * 2];
    auto fetch = [&](u32x4 (&buf)[E::SN * 2], int i) {
#pragma unroll
        for (int j = 0; j < E::SN; ++j)
#pragma unroll
            for (int gg = 0; gg < 2; ++gg)
                buf[j * 2 + gg] = G(reinterpret_cast<const u32x4*>(
                    amat + static_cast<size_t>(q.raw_col + 32 * j) * ld + mbase + 32 * i + 8 * (2 * gg + hh)))[0];
    };
    if (POLY) fetch(cur, 0);
#pragma unroll
    for (int i = 0; i < E::SM; ++i) {
        if (POLY && i + 1 < E::SM) fetch(nxt, i + 1);
#pragma unroll
        for (int j = 0; j < E::SN; ++j)
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
                float r0[4], r1[4];   // raw layout: rows 8 g + 4 h + p of column cc
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    r0[p] = acc[i][j][8 * gg + p];
                    r1[p] = acc[i][j][8 * gg + 4 + p];
                }
                if (POLY) {
                    // this lane read rows 8 g_h + (0..7); words 0-1 hold rows +0..3, words 2-3 rows +4..7
                    const u32x4 w = cur[j * 2 + gg];
                    const unsigned k0 = hh ? w.z : w.x, k1 = hh ? w.w : w.y;
                    const unsigned s0 = swap_xor32(hh ? w.x : w.z), s1 = swap_xor32(hh ? w.y : w.w);
                    const unsigned a0w[2] = {hh ? s0 : k0, hh ? s1 : k1};   // rows 8 g0 + 4 h + (0..3)
                    const unsigned a1w[2] = {hh ? k0 : s0, hh ? k1 : s1};   // rows 8 g1 + 4 h + (0..3)
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        r0[2 * p] = fmaf(c, r0[2 * p], b * __uint_as_float(a0w[p] << 16));
                        r0[2 * p + 1] = fmaf(c, r0[2 * p + 1], b * __uint_as_float(a0w[p] & 0xffff0000u));
                        r1[2 * p] = fmaf(c, r1[2 * p], b * __uint_as_float(a1w[p] << 16));
                        r1[2 * p + 1] = fmaf(c, r1[2 * p + 1], b * __uint_as_float(a1w[p] & 0xffff0000u));
                    }
                } else {
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        r0[p] *= scale;
                        r1[p] *= scale;
                    }
                }
                const int cc = q.raw_col + 32 * j;
                // mirrored: h = 0 stores rows 8 g0 + (0..7), h = 1 rows 8 g1 + (0..7), at row cc
                {
                    float m[8];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float rcv = __uint_as_float(swap_xor32(__float_as_uint(hh ? r0[p] : r1[p])));
                        m[p] = hh ? rcv : r0[p];
                        m[4 + p] = hh ? r1[p] : rcv;
                    }
                    const int mc = mbase + 32 * i + 8 * (2 * gg + hh);
                    unsigned mm = 0xFFu;
                    if (diag) {
                        mm = 0;
#pragma unroll
                        for (int e = 0; e < 8; ++e) mm |= (mc + e < cc) ? (1u << e) : 0u;
                    }
                    st_bf16x8_masked(dst + static_cast<size_t>(cc) * ld + mc, m, mm);
                }
                // direct: row tr, columns tc .. tc + 7
                quad_transpose(r0);
                quad_transpose(r1);
                float x[8];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float keep = odd ? r1[p] : r0[p];
                    const float recv = __uint_as_float(swap_xor4(__float_as_uint(odd ? r0[p] : r1[p])));
                    x[p] = odd ? recv : keep;
                    x[4 + p] = odd ? keep : recv;
                }
                const int tr = q.tr_row + 32 * i + 8 * (2 * gg + odd);
                const int tc = q.tr_col + 32 * j - (odd ? 4 : 0);
                unsigned md = 0xFFu;
                if (diag) {
                    md = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) md |= (tr <= tc + e) ? (1u << e) : 0u;
                }
                st_bf16x8_masked(dst + static_cast<size_t>(tr) * ld + tc, x, md);
            }
        if (POLY) {
#pragma unroll
            for (int k = 0; k < E::SN * 2; ++k) cur[k] = nxt[k];
        }
    }
}

template <typename E, typename T, bool POLY>
__device__ __forceinline__ void sym_epilogue(f32x16_t (&acc)[E::SM][E::SN], int row0, int col0, bool diag, void* dst,
                                             size_t ld, float scale, const void* amat, float b, float c) {
    if (sizeof(T) == 2)
        sym_epilogue_bf16<E, POLY>(acc, row0, col0, diag, static_cast<uint16_t*>(dst), ld, scale,
                                   static_cast<const uint16_t*>(amat), b, c);
    else
        sym_epilogue_quad<E, T, POLY>(acc, row0, col0, diag, dst, ld, scale, amat, b, c);
}

// X' = u (a X + B X).  a X enters the accumulators before or during the
// k-loop, so the epilogue only scales and stores.
//   fp32: the iterate is x32[ping] (also the operand); a X is read into the
//         accumulators while the first operand slabs load (UpdateInit), and
//         X' goes to x32[ping ^ 1].
//   bf16: the iterate is the pair hi + lo (hi = xop[ping], the operand copy,
//         lo = xlo in the accumulator layout).  a lo is the accumulators'
//         initial value (LoInit); a hi is added from LDS during the k-steps that
//         stage the tile's own rows of X as operand k-rows (HiAddend).  X' is
//         stored as hi' = bf16(X') to xop[ping ^ 1] and lo' = bf16(X' - hi') to
//         xlo, in place (update_epilogue_native).
template <typename E, typename T>
struct UpdateInit {   // fp32 iterate
    const void* src;    // x32[ping]
    size_t np;
    int row0, col0;
    float a;
    template <typename A> __device__ __forceinline__ void operator()(A& acc) const {
        const Coords<E> q(row0, col0);
#pragma unroll
        for (int i = 0; i < E::SM; ++i)
#pragma unroll
            for (int j = 0; j < E::SN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 x = ld_quad<T>(src, static_cast<size_t>(q.tr_row + 32 * i + 8 * g) * np + q.tr_col + 32 * j);
                    float v[4] = {a * x.x, a * x.y, a * x.z, a * x.w};
                    quad_transpose(v);   // row layout -> accumulator layout (an involution)
#pragma unroll
                    for (int p = 0; p < 4; ++p) acc[i][j][4 * g + p] = v[p];
                }
    }
};

template <typename E>
struct HiAddend {
    int kt0;    // k-step whose k-rows are the tile's first output rows (row0 / KS)
    float a;
    // Stage kt holds X k-rows [kt KS, kt KS + KS) of the tile's columns; when they are
    // output rows of this tile, the waves owning them add a * hi for those rows.  A
    // transpose read per (i, j, g) delivers the accumulator layout directly: lane
    // group g16 addresses rows 8 g + 4 (g16 >> 1) + (0..3) and 16 columns.
    template <typename A> __device__ __forceinline__ void operator()(int kt, const lds_byte_t* Lq, A& acc) const {
        const int rel = kt - kt0;
        const int lane = threadIdx.x & 63, wave = wave_id();
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        if (rel < 0 || rel >= E::BM / E::KS || (rel * E::KS) / E::WM != wm) return;
        const int ifirst = (rel * E::KS - wm * E::WM) / 32;
        // k-row of this lane's first element: 32 (i - ifirst) + 8 g + kl; the swizzle only
        // depends on kl & 3, so each column block needs one per-lane base offset
        const int i16 = lane & 15, g16 = lane >> 4;
        const int kl = 4 * (g16 >> 1) + (i16 >> 2);
        int base[E::SN];
#pragma unroll
        for (int j = 0; j < E::SN; ++j) {
            const int col = wn * E::WN + 32 * j + 16 * (g16 & 1) + 4 * (i16 & 3);
            base[j] = qswz(kl, col >> 3) * 16 + (col & 7) * 2;
        }
        // one 32-row block at a time keeps the reads' registers few
#pragma unroll
        for (int i = 0; i < E::SM; ++i) {
            if (i >= ifirst && i < ifirst + E::KS / 32) {
                const int rowoff = 32 * (i - ifirst) * QROW_CHUNKS * 16;
#pragma unroll
                for (int j = 0; j < E::SN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const i16x4_t h = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4_t*)(Lq + base[j] + rowoff + 8 * g * QROW_CHUNKS * 16));
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][j][4 * g + e] = fmaf(a, bf16_to_f32(static_cast<uint16_t>(h[e])), acc[i][j][4 * g + e]);
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// Polynomial B = b A + c A A with c != 0, accumulated as c (A A + (b / c) A): the
// Q slab of k-step kt holds A[col0 + r][kt KS + (0..KS-1)], which by symmetry is
// A[kt KS + (0..KS-1)][col0 + r]; when those k are output rows of this tile the
// waves owning them add f A = (b / c) A for those rows.  A lane's 4 accumulator
// rows of one column are 4 consecutive k of one slab row: one 8-byte (bf16) or
// 16-byte (fp32) LDS read.
template <typename E, typename T>
struct PolyAddend {
    int kt0;    // row0 / KS
    float f;    // b / c
    template <typename A> __device__ __forceinline__ void operator()(int kt, const lds_byte_t* Lq, A& acc) const {
        const int rel = kt - kt0;
        const int lane = threadIdx.x & 63, wave = wave_id();
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        if (rel < 0 || rel >= E::BM / E::KS || (rel * E::KS) / E::WM != wm) return;
        const int ifirst = (rel * E::KS - wm * E::WM) / 32;
        constexpr int EPC = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte chunk
        const int h = lane >> 5;
#pragma unroll
        for (int i = 0; i < E::SM; ++i) {
            if (i >= ifirst && i < ifirst + E::KS / 32) {
#pragma unroll
                for (int j = 0; j < E::SN; ++j) {
                    const int sr = wn * E::WN + 32 * j + (lane & 31);
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int kk = 32 * (i - ifirst) + 8 * g + 4 * h;
                        const lds_byte_t* a = Lq + swz(sr, kk / EPC) * 16 + (kk % EPC) * static_cast<int>(sizeof(T));
                        float v[4];
                        if (sizeof(T) == 2) {
                            const u32x2_t w = *(const __attribute__((address_space(3))) u32x2_t*)a;
                            v[0] = __uint_as_float(w.x << 16);
                            v[1] = __uint_as_float(w.x & 0xffff0000u);
                            v[2] = __uint_as_float(w.y << 16);
                            v[3] = __uint_as_float(w.y & 0xffff0000u);
                        } else {
                            const u32x4 w = *(const __attribute__((address_space(3))) u32x4*)a;
                            v[0] = __uint_as_float(w.x);
                            v[1] = __uint_as_float(w.y);
                            v[2] = __uint_as_float(w.z);
                            v[3] = __uint_as_float(w.w);
                        }
#pragma unroll
                        for (int p = 0; p < 4; ++p) acc[i][j][4 * g + p] = fmaf(f, v[p], acc[i][j][4 * g + p]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// fp32 update epilogue: X' = u acc to x32[ping ^ 1], one row of 4 columns per lane.
template <typename E>
__device__ __attribute__((always_inline)) void update_epilogue_f32(f32x16_t (&acc)[E::SM][E::SN], int row0, int col0,
                                                                   float* out, size_t np, float u) {
    const Coords<E> q(row0, col0);
#pragma unroll
    for (int i = 0; i < E::SM; ++i)
#pragma unroll
        for (int j = 0; j < E::SN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) v[p] = acc[i][j][4 * g + p];
                quad_transpose(v);
                const size_t idx = static_cast<size_t>(q.tr_row + 32 * i + 8 * g) * np + q.tr_col + 32 * j;
                st_f4(out + idx, make_float4(u * v[0], u * v[1], u * v[2], u * v[3]));
            }
}

// ----------------------------------------------------------------------------
// Column-major staging of a 256 x 256 bf16 output tile in LDS (128 KB), used by
// the bf16 update and symmetric-output epilogues.  Column c occupies the 512
// bytes at c * 512; its 256 rows form 64 eight-byte units of 4 rows, unit u
// stored at position u ^ csw(c).  In the accumulator layout a lane holds 4
// consecutive rows of one column of each 32 x 32 block, i.e. exactly one unit:
// the tile goes to LDS with one 8-byte write per 4 values and no register
// shuffles (the quad transposes and lane swaps a row-major layout needs cost
// more VALU cycles than the rest of the epilogue).  Read back
//   * row-major, for direct stores: ds_read_b64_tr_b16 over units of 16
//     columns gives each lane 4 consecutive columns of one row; two reads make
//     the 16 bytes of one store, and a wave instruction stores 4 rows x 128
//     columns (whole 128-byte lines);
//   * column-major, for the mirrored store of a symmetric output: one 16-byte
//     read is 8 consecutive rows of column c, i.e. 8 consecutive columns of the
//     mirrored row c (the two units trade places when csw(c) is odd).
// The swizzle makes the writes and the transpose reads free of LDS bank
// conflicts and the mirror reads run at two cycles per half-wave (its minimum);
// a CPU model of every lane address checked this and that each element is
// written and read exactly once.
// ----------------------------------------------------------------------------
__device__ __forceinline__ int csw(int c) { return (c & 31) ^ (((c >> 5) & 1) << 2); }
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

template <typename E>
struct CStage {
    static_assert(E::BM == 256 && E::BN == 256 && E::WM == 128 && E::WN == 64, "staging geometry");
    static_assert(E::BM * 512 <= E::LDS_CHUNKS * 16, "a staged tile fits the LDS");
    int wbase[E::SN];   // byte address of this lane's unit for i = g = 0, per column block j
    __device__ CStage() {
        const int lane = threadIdx.x & 63, wave = wave_id();
        const int wm = wave / WAVES_N, wn = wave % WAVES_N, h = lane >> 5;
#pragma unroll
        for (int j = 0; j < E::SN; ++j) {
            const int c = wn * E::WN + 32 * j + (lane & 31);
            wbase[j] = c * 512 + 256 * wm + 8 * (h ^ csw(c));
        }
    }
    // rows 32 i + 8 g + 4 h + (0..3) of block (i, j): unit 32 wm + 8 i + 2 g + h; the
    // block part of the unit index has no bits in common with wbase's, so XOR adds it
    __device__ __forceinline__ void put(lds_byte_t* L, int i, int j, int g, unsigned w0, unsigned w1) const {
        *(lds_u32x2_t*)(L + (wbase[j] ^ (64 * i + 16 * g))) = u32x2_t{w0, w1};
    }
    // Slot (i, j) holds block (R, C) = (4 wm + i, 2 wn + j) of a diagonal tile; stage its
    // transpose as block (C, R) (diag_modes, swapped).  After a quad transpose lane
    // 4 q + t (of its half h) holds rows 4 q .. 4 q + 3 of column 8 g + 4 h + t of the
    // transpose: unit u = 8 C + q of tile column c = 32 R + 8 g + 4 h + t, at byte
    // c 512 + 8 (u ^ csw(c)).  v: the 4 values of group g in accumulator order.
    __device__ __forceinline__ void put_transposed(lds_byte_t* L, int i, int j, int g, float (&v)[4]) const {
        const int lane = threadIdx.x & 63, wave = wave_id();
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        quad_transpose(v);
        const int c = 32 * (E::SM * wm + i) + 8 * g + 4 * (lane >> 5) + (lane & 3);
        const int u = 8 * (E::SN * wn + j) + ((lane & 31) >> 2);
        *(lds_u32x2_t*)(L + (c * 512 + 8 * (u ^ csw(c)))) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
};

// 8 bf16 (packed, in column order) at p: one 16-byte store, or per element where `mask` has bits clear.
template <bool NT>
__device__ __forceinline__ void st_packed8(uint16_t* p, const u32x4& v, unsigned mask) {
    if (mask == 0xFFu) {
        if (NT) __builtin_nontemporal_store(v, G(reinterpret_cast<u32x4*>(p)));
        else G(reinterpret_cast<u32x4*>(p))[0] = v;
    } else if (mask) {
        const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (mask & (1u << e)) G(p)[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
    }
}

// Direct copy-out of a staged tile: tile row r, columns cc .. cc + 7 per lane and
// instruction.  DIAG stores only the elements with r <= c (the upper triangle of a
// diagonal tile of a symmetric output).
template <typename E, bool DIAG, bool NT>
__device__ __forceinline__ void cstage_store_rows(const lds_byte_t* L, uint16_t* dst, int row0, int col0, size_t ld) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int grp = lane >> 4, k = lane & 15;
    // lane k of a 16-lane group addresses column ccA = 32 grp + 8 (k & 3) + (k >> 2) (read A)
    // and ccA + 4 (read B) at the row quad being stored; the transpose hands lane l the
    // row 4 u + (l & 3), columns 32 grp + 8 ((l & 15) >> 2) + (0..3) and (4..7)
    const int ccA = 32 * grp + 8 * (k & 3) + (k >> 2);
    // wave w stores the row quads 8 w .. 8 w + 7; 8 u = 64 w + 8 du shares no bits with
    // the swizzled unit offset's upper part, and +128 columns is +65536 bytes
    const int pA = (ccA * 512 + 8 * csw(ccA)) ^ (64 * wave);
    const int pB = ((ccA + 4) * 512 + 8 * csw(ccA + 4)) ^ (64 * wave);
    const int r = 32 * wave + (lane & 3);
    const int cs = 32 * grp + 8 * (k >> 2);
    // the store address advances by 4 rows per row quad (kept incremental: precomputing
    // all 16 addresses of an unrolled loop costs registers the caller needs)
    uint16_t* out = dst + static_cast<size_t>(row0 + r) * ld + col0 + cs;
    const size_t quad = 4 * ld;
#pragma unroll 2
    for (int du = 0; du < 8; ++du) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(L + ((pA ^ (8 * du)) + 65536 * half)));
            const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(L + ((pB ^ (8 * du)) + 65536 * half)));
            const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), b2 = __builtin_bit_cast(u32x2_t, b);
            unsigned mask = 0xFFu;
            if (DIAG) {
                const int rr = r + 4 * du, cc = cs + 128 * half;
                mask = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) mask |= (rr <= cc + e) ? (1u << e) : 0u;
            }
            st_packed8<NT>(out + 128 * half, u32x4{a2.x, a2.y, b2.x, b2.y}, mask);
        }
        out += quad;
    }
}

// Mirrored copy-out of a staged symmetric-output tile: column c of the tile is row
// col0 + c of the output, from column row0.  Lanes 0-31 take column c, lanes 32-63
// column c + 1, each 8 consecutive rows.  DIAG stores only rows r < c (the strictly
// upper triangle, mirrored).
template <typename E, bool DIAG>
__device__ __forceinline__ void cstage_store_mirror(const lds_byte_t* L, uint16_t* dst, int row0, int col0, size_t ld) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int m = lane & 31, hh = lane >> 5;
    // column c = 32 w + 2 t + hh: csw(c) = (2 t + hh) ^ (4 (w & 1)), odd exactly when hh = 1;
    // the 16-byte slot of units 2m, 2m + 1 is 2m ^ (csw(c) & ~1)
    const int base = (32 * wave + hh) * 512 + ((16 * m) ^ (32 * (wave & 1)));
#pragma unroll 4
    for (int t = 0; t < 16; ++t) {
        const int c = 32 * wave + 2 * t + hh;
        const u32x4 v = *(const lds_u32x4_t*)(L + ((base ^ (16 * t)) + 1024 * t));
        const u32x4 w = hh ? u32x4{v.z, v.w, v.x, v.y} : v;   // rows 8m .. 8m + 7 in order
        unsigned mask = 0xFFu;
        if (DIAG) {
            mask = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) mask |= (8 * m + e < c) ? (1u << e) : 0u;
        }
        st_packed8<true>(dst + static_cast<size_t>(col0 + c) * ld + row0 + 8 * m, w, mask);
    }
}

// bf16 symmetric output (Gram, polynomial with the staged addend): value = scale * acc,
// staged once, stored directly and mirrored (non-temporal: the next reader is the
// next launch, and a batch's outputs do not stay in the caches until then).
// DGM: the tile was formed by Engine::run_diag, its slots hold what diag_modes says;
// only the upper blocks are staged (the stores below read no lower block).
template <typename E, bool DGM = false>
__device__ __attribute__((always_inline)) void sym_epilogue_cstage(f32x16_t (&acc)[E::SM][E::SN], int row0, int col0,
                                                                   bool diag, uint16_t* dst, size_t ld, float scale,
                                                                   u32x4* lds) {
    const CStage<E> st;
    lds_byte_t* L = (lds_byte_t*)lds;
    const unsigned modes = DGM ? diag_modes() : 0u;
    lds_barrier();   // every wave is done reading the operand slabs
#pragma unroll
    for (int i = 0; i < E::SM; ++i)
#pragma unroll
        for (int j = 0; j < E::SN; ++j) {
            const unsigned md = DGM ? dg_mode(modes, i, j) : DG_NATIVE;
            if (md == DG_SKIP) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16_t& a = acc[i][j];
                if (md == DG_NATIVE) {
                    st.put(L, i, j, g, pack_bf16x2(scale * a[4 * g], scale * a[4 * g + 1]),
                           pack_bf16x2(scale * a[4 * g + 2], scale * a[4 * g + 3]));
                } else {
                    float v[4] = {scale * a[4 * g], scale * a[4 * g + 1], scale * a[4 * g + 2], scale * a[4 * g + 3]};
                    st.put_transposed(L, i, j, g, v);
                }
            }
        }
    lds_barrier();
    if (diag) {
        cstage_store_rows<E, true, true>(L, dst, row0, col0, ld);
        cstage_store_mirror<E, true>(L, dst, row0, col0, ld);
    } else {
        cstage_store_rows<E, false, true>(L, dst, row0, col0, ld);
        cstage_store_mirror<E, false>(L, dst, row0, col0, ld);
    }
}

// bf16 update epilogue: X' = u acc as hi' = bf16(X') and lo' = bf16(X' - hi').  hi' is
// staged column-major in LDS (CStage) by every wave and stored as whole tile rows; lo'
// goes straight from the accumulators to its tile in the accumulator layout (lo_offset),
// 1 KB contiguous per wave instruction.  Both non-temporal: the next reader is the next
// launch.
template <typename E, bool SCALE>
__device__ __attribute__((always_inline)) void update_epilogue_native(f32x16_t (&acc)[E::SM][E::SN], int row0,
                                                                      int col0, uint16_t* hi_out, uint16_t* lo_tile,
                                                                      size_t np, float u, u32x4* lds) {
    static_assert(E::SM == 4 && E::SN == 2, "lo_offset's block numbering");
    const CStage<E> st;
    lds_byte_t* L = (lds_byte_t*)lds;
    u32x4* lp = reinterpret_cast<u32x4*>(lo_tile) + threadIdx.x;
    lds_barrier();   // every wave is done reading the operand slabs
#pragma unroll
    for (int i = 0; i < E::SM; ++i)
#pragma unroll
        for (int j = 0; j < E::SN; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                unsigned lw[4];
#pragma unroll
                for (int gg = 0; gg < 2; ++gg) {
                    const int g = 2 * h + gg;
                    float v[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) v[p] = SCALE ? u * acc[i][j][4 * g + p] : acc[i][j][4 * g + p];
                    const unsigned h0 = pack_bf16x2(v[0], v[1]), h1 = pack_bf16x2(v[2], v[3]);
                    lw[2 * gg] = pack_bf16x2(v[0] - __uint_as_float(h0 << 16), v[1] - __uint_as_float(h0 & 0xffff0000u));
                    lw[2 * gg + 1] = pack_bf16x2(v[2] - __uint_as_float(h1 << 16), v[3] - __uint_as_float(h1 & 0xffff0000u));
                    st.put(L, i, j, g, h0, h1);
                }
                __builtin_nontemporal_store(u32x4{lw[0], lw[1], lw[2], lw[3]},
                                            G(lp + ((E::SN * i + j) * 2 + h) * GEMM_THREADS));
            }
    lds_barrier();
    cstage_store_rows<E, false, true>(L, hi_out, row0, col0, np);
}

// Last update of muon_step: W' = decay W - coef X' goes straight from the
// accumulators into the caller's weight (user frame), in place of storing the
// iterate and running the apply kernel.  X' = u acc in fp32, W' rounded once.
//   untransposed matrix: the direct layout after the quad swap gives 8
//     consecutive NS columns of one row = 8 consecutive user columns;
//   tall matrix (NS frame = user transposed): lanes l and l ^ 32 swap one quad
//     so each owns 8 consecutive NS rows of one NS column = 8 consecutive user
//     columns of one user row.
// With the 16-byte flag (cols % 8 == 0, aligned pointers) a group is inside or
// outside the matrix as a whole; otherwise each element is bounds-checked.
template <typename T> struct WeightIO;
template <> struct WeightIO<uint16_t> {
    static __device__ inline void load8(const void* p, float (&v)[8]) {
        const u32x4 q = G(static_cast<const u32x4*>(p))[0];
        const unsigned w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
    static __device__ inline void store8(void* p, const float (&v)[8]) {
        G(static_cast<u32x4*>(p))[0] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                             pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    }
    static __device__ inline float load1(const void* p) { return bf16_to_f32(G(static_cast<const uint16_t*>(p))[0]); }
    static __device__ inline void store1(void* p, float v) { G(static_cast<uint16_t*>(p))[0] = f32_to_bf16(v); }
};
template <> struct WeightIO<float> {
    static __device__ inline void load8(const void* p, float (&v)[8]) {
        const float4 a = ld_f4(static_cast<const float*>(p)), b = ld_f4(static_cast<const float*>(p) + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ inline void store8(void* p, const float (&v)[8]) {
        st_f4(static_cast<float*>(p), make_float4(v[0], v[1], v[2], v[3]));
        st_f4(static_cast<float*>(p) + 4, make_float4(v[4], v[5], v[6], v[7]));
    }
    static __device__ inline float load1(const void* p) { return G(static_cast<const float*>(p))[0]; }
    static __device__ inline void store1(void* p, float v) { G(static_cast<float*>(p))[0] = v; }
};

template <typename E, typename T>
__device__ __attribute__((always_inline)) void apply_epilogue(f32x16_t (&acc)[E::SM][E::SN], int row0, int col0,
                                                              const MatDesc& d, float u) {
    using IO = WeightIO<T>;
    const Coords<E> q(row0, col0);
    const bool hh = (threadIdx.x >> 5) & 1;
    const bool odd = odd_quad();
    const int mbase = q.raw_row - (hh ? 4 : 0);
    // descriptor fields in registers: the weight stores could alias the descriptor table, so
    // reading them through d would reload them after every store
    const float coef = d.apply_coef, decay = d.decay;
    const bool tall = d.tall != 0, vec = d.uvec != 0;
    const int rows = d.rows, cols = d.cols;
    char* const w = static_cast<char*>(d.w);
    // user-frame origin of 8-element group k of row block i
    auto origin = [&](int i, int k, int& r, int& c) {
        const int j = k >> 1, gg = k & 1;
        if (tall) {
            r = q.raw_col + 32 * j;
            c = mbase + 32 * i + 8 * (2 * gg + hh);
        } else {
            r = q.tr_row + 32 * i + 8 * (2 * gg + odd);
            c = q.tr_col + 32 * j - (odd ? 4 : 0);
        }
    };
    // bf16 weights with 16-byte groups: every group's load is issued before the first
    // store (64 VGPRs of packed weights; the k-loop's fragment registers are free here)
    constexpr bool PACKED = sizeof(T) == 2;
    u32x4 wraw[PACKED ? E::SM : 1][E::SN * 2];
    if (PACKED && vec) {
#pragma unroll
        for (int i = 0; i < E::SM; ++i)
#pragma unroll
            for (int k = 0; k < E::SN * 2; ++k) {
                int r, c;
                origin(i, k, r, c);
                if (r < rows && c < cols)
                    wraw[PACKED ? i : 0][k] = G(reinterpret_cast<const u32x4*>(w + (static_cast<size_t>(r) * cols + c) * sizeof(T)))[0];
            }
    }
#pragma unroll
    for (int i = 0; i < E::SM; ++i) {
        // user-frame origin of each 8-element group of this row block
        int ur[E::SN * 2], uc[E::SN * 2];
#pragma unroll
        for (int j = 0; j < E::SN; ++j)
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
                if (tall) {
                    ur[j * 2 + gg] = q.raw_col + 32 * j;
                    uc[j * 2 + gg] = mbase + 32 * i + 8 * (2 * gg + hh);
                } else {
                    ur[j * 2 + gg] = q.tr_row + 32 * i + 8 * (2 * gg + odd);
                    uc[j * 2 + gg] = q.tr_col + 32 * j - (odd ? 4 : 0);
                }
            }
        // read the weight groups of this row block first
        float wv[E::SN * 2][8];
#pragma unroll
        for (int k = 0; k < E::SN * 2; ++k) {
            const bool in = ur[k] < rows && uc[k] < cols;
            const size_t idx = static_cast<size_t>(ur[k]) * cols + uc[k];
            if (vec) {
                if (PACKED) {
                    const u32x4 qw = wraw[PACKED ? i : 0][k];
                    const unsigned wu[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        wv[k][2 * e] = __uint_as_float(wu[e] << 16);
                        wv[k][2 * e + 1] = __uint_as_float(wu[e] & 0xffff0000u);
                    }
                } else if (in) {
                    IO::load8(w + idx * sizeof(T), wv[k]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    wv[k][e] = (in && uc[k] + e < cols) ? IO::load1(w + (idx + e) * sizeof(T)) : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < E::SN; ++j)
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
                const int k = j * 2 + gg;
                float r0[4], r1[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    r0[p] = u * acc[i][j][8 * gg + p];
                    r1[p] = u * acc[i][j][8 * gg + 4 + p];
                }
                float x[8];
                if (tall) {
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float rcv = __uint_as_float(swap_xor32(__float_as_uint(hh ? r0[p] : r1[p])));
                        x[p] = hh ? rcv : r0[p];
                        x[4 + p] = hh ? r1[p] : rcv;
                    }
                } else {
                    quad_transpose(r0);
                    quad_transpose(r1);
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float keep = odd ? r1[p] : r0[p];
                        const float recv = __uint_as_float(swap_xor4(__float_as_uint(odd ? r0[p] : r1[p])));
                        x[p] = odd ? recv : keep;
                        x[4 + p] = odd ? keep : recv;
                    }
                }
                if (ur[k] >= rows || uc[k] >= cols) continue;
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf(-coef, x[e], decay * wv[k][e]);
                const size_t idx = static_cast<size_t>(ur[k]) * cols + uc[k];
                if (vec) {
                    IO::store8(w + idx * sizeof(T), o);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (uc[k] + e < cols) IO::store1(w + (idx + e) * sizeof(T), o[e]);
                }
            }
    }
}

template <typename T, int PHASE>
__device__ __attribute__((always_inline)) void process_tile(const NsArgs& args, int t, u32x4* lds) {
    constexpr bool UPD = PHASE == PH_UPDATE || PHASE == PH_UPDATE_APPLY;
    using E = Engine<T, UPD>;
    int local;
    const int mi = args.nruns <= NS_ARG_RUNS ? run_matrix_args(args.run, args.nruns, t, local)
                                             : run_matrix(args.runs, args.nruns, t, local);
    // The descriptor by value, read at the tile's start.  After the k-loop, whose
    // direct-to-LDS loads count as memory writes, the compiler no longer reads the table
    // through the scalar cache: a field first used in an epilogue cost a vector load and a
    // wait at the end of every tile.  The ping-pong halves are selected here, not indexed.
    const MatDesc d = args.descs[mi];
    const int mp = d.mp, np = d.np;
    const int ping = args.ping;
    const void* const xop_cur = ping ? d.xop[1] : d.xop[0];
    void* const xop_nxt = ping ? d.xop[0] : d.xop[1];
    const float* const x32_cur = ping ? d.x32[1] : d.x32[0];
    float* const x32_nxt = ping ? d.x32[0] : d.x32[1];

    int ti, tj;
    if (UPD) {
        grouped_decode(local, mp / E::BM, np / E::BN, ti, tj);
    } else {
        sym_decode(local, mp / E::BM, ti, tj);
    }
    // When the last tile row holds at most BM / 2 real rows (bf16), its tiles run with
    // half of the waves idle (Engine::run, p_half).  A symmetric output stores every
    // tile both directly and mirrored, so its last tile column is computed as the
    // mirrored tile (tj, ti), whose padding then also falls in the P half.
    const int tlast = mp / E::BM - 1;
    const bool half_last = sizeof(T) == 2 && d.m - tlast * E::BM <= E::BM / 2;
    if (!UPD && half_last && tj == tlast && ti != tj) {
        tj = ti;
        ti = tlast;
    }
    const bool p_half = half_last && ti == tlast;
    const int row0 = ti * E::BM, col0 = tj * E::BN;

    // k runs over the real extent rounded up to a k-step, not the tile padding: the
    // padding of X, A and B is zero, so the skipped k-steps would add nothing
    const int ks_m = (d.m + E::KS - 1) / E::KS, ks_n = (d.n + E::KS - 1) / E::KS;
    f32x16_t acc[E::SM][E::SN];
    if constexpr (PHASE == PH_GRAM) {
        // the first step reads hi0 (the workspace copy, or the caller's buffer holding the same bits)
        const char* X = static_cast<const char*>(args.first ? d.hi0 : xop_cur);
        const size_t ld = static_cast<size_t>(np) * sizeof(T);
        // first step: X0 = s * M' is folded in as A0 = s^2 M' M'^T
        const float scale = args.first ? G(d.scal)[0] * G(d.scal)[0] : 1.0f;
        if constexpr (sizeof(T) == 2) {
            if (ti == tj && !p_half) {
                E::run_diag(X + row0 * ld, ld, ks_n, lds, acc, ZeroInit{}, NoHook{});
                sym_epilogue_cstage<E, true>(acc, row0, col0, true, static_cast<uint16_t*>(d.amat), mp, scale, lds);
            } else {
                E::run(X + row0 * ld, ld, X + col0 * ld, ld, ks_n, lds, acc, ZeroInit{}, NoHook{}, p_half);
                sym_epilogue_cstage<E>(acc, row0, col0, ti == tj, static_cast<uint16_t*>(d.amat), mp, scale, lds);
            }
        } else {
            E::run(X + row0 * ld, ld, X + col0 * ld, ld, ks_n, lds, acc, ZeroInit{}, NoHook{}, p_half);
            sym_epilogue<E, T, false>(acc, row0, col0, ti == tj, d.amat, mp, scale, nullptr, 0.0f, 0.0f);
        }
    } else if constexpr (PHASE == PH_POLY) {
        const char* A = static_cast<const char*>(d.amat);
        const size_t ld = static_cast<size_t>(mp) * sizeof(T);
        E::run(A + row0 * ld, ld, A + col0 * ld, ld, ks_m, lds, acc, ZeroInit{}, NoHook{}, p_half);
        sym_epilogue<E, T, true>(acc, row0, col0, ti == tj, d.bmat, mp, 1.0f, d.amat, args.b, args.c);
    } else if constexpr (PHASE == PH_POLY_LDS) {
        const char* A = static_cast<const char*>(d.amat);
        const size_t ld = static_cast<size_t>(mp) * sizeof(T);
        if constexpr (sizeof(T) == 2) {
            if (ti == tj && !p_half) {
                E::run_diag(A + row0 * ld, ld, ks_m, lds, acc, ZeroInit{},
                            PolyAddend<E, T>{row0 / E::KS, args.b / args.c});
                sym_epilogue_cstage<E, true>(acc, row0, col0, true, static_cast<uint16_t*>(d.bmat), mp, args.c, lds);
            } else {
                E::run(A + row0 * ld, ld, A + col0 * ld, ld, ks_m, lds, acc, ZeroInit{},
                       PolyAddend<E, T>{row0 / E::KS, args.b / args.c}, p_half);
                sym_epilogue_cstage<E>(acc, row0, col0, ti == tj, static_cast<uint16_t*>(d.bmat), mp, args.c, lds);
            }
        } else {
            E::run(A + row0 * ld, ld, A + col0 * ld, ld, ks_m, lds, acc, ZeroInit{},
                   PolyAddend<E, T>{row0 / E::KS, args.b / args.c}, p_half);
            sym_epilogue<E, T, false>(acc, row0, col0, ti == tj, d.bmat, mp, args.c, nullptr, 0.0f, 0.0f);
        }
    } else {
        // first step: X1 = s (a M' + B0 M') with M' unscaled in the iterate and operand copy
        // (read before the k-loop, like the descriptor)
        const float u = args.first ? G(d.scal)[0] : 1.0f;
        const char* B = static_cast<const char*>(d.bmat);
        const char* X = static_cast<const char*>(args.first ? d.hi0 : xop_cur);
        const size_t ldb = static_cast<size_t>(mp) * sizeof(T), ldx = static_cast<size_t>(np) * sizeof(T);
        // bf16: the tile's lo, in the accumulator layout (lo_offset)
        uint16_t* lo_tile = d.xlo + static_cast<size_t>(ti * (np / E::BN) + tj) * (E::BM * E::BN);
        if constexpr (sizeof(T) == 2) {
            E::run(B + row0 * ldb, ldb, X + col0 * sizeof(T), ldx, ks_m, lds, acc, LoInit<E>{lo_tile, args.a},
                   HiAddend<E>{row0 / E::KS, args.a}, p_half);
        } else {
            const UpdateInit<E, T> init{x32_cur, static_cast<size_t>(np), row0, col0, args.a};
            E::run(B + row0 * ldb, ldb, X + col0 * sizeof(T), ldx, ks_m, lds, acc, init, NoHook{});
        }
        if constexpr (PHASE == PH_UPDATE_APPLY)
            apply_epilogue<E, T>(acc, row0, col0, d, u);
        else if constexpr (sizeof(T) == 2) {
            if (u != 1.0f)
                update_epilogue_native<E, true>(acc, row0, col0, static_cast<uint16_t*>(xop_nxt), lo_tile, np, u, lds);
            else
                update_epilogue_native<E, false>(acc, row0, col0, static_cast<uint16_t*>(xop_nxt), lo_tile, np, u, lds);
        }
        else
            update_epilogue_f32<E>(acc, row0, col0, x32_nxt, np, u);
    }
}

template <typename T, int PHASE>
__global__ __launch_bounds__(GEMM_THREADS, 1) void ns_gemm_kernel(NsArgs args) {
    using E = Engine<T, PHASE == PH_UPDATE || PHASE == PH_UPDATE_APPLY>;
    __shared__ u32x4 lds[E::LDS_CHUNKS];
    const int t = xcd_run_remap<PHASE == PH_UPDATE || PHASE == PH_UPDATE_APPLY ? XCD_RUN_UPD : XCD_RUN_SYM>(blockIdx.x,
                                                                                                        gridDim.x);
    if (t < args.total) process_tile<T, PHASE>(args, t, lds);
}

template <int PHASE>
hipError_t launch_phase(int dtype, const NsArgs& args, hipStream_t s) {
    if (args.total <= 0) return hipSuccess;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL((ns_gemm_kernel<uint16_t, PHASE>), dim3(args.total), dim3(GEMM_THREADS), 0, s, args);
    else
        hipLaunchKernelGGL((ns_gemm_kernel<float, PHASE>), dim3(args.total), dim3(GEMM_THREADS), 0, s, args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gram(int dtype, const NsArgs& args, hipStream_t s) { return launch_phase<PH_GRAM>(dtype, args, s); }
hipError_t launch_poly(int dtype, const NsArgs& args, hipStream_t s) {
    // the kernel forms b / c in fp32; it must be finite for the staged-operand form
    const float f = args.b / args.c;
    if (args.c != 0.0f && std::isfinite(f)) return launch_phase<PH_POLY_LDS>(dtype, args, s);
    return launch_phase<PH_POLY>(dtype, args, s);
}
hipError_t launch_update(int dtype, const NsArgs& args, hipStream_t s) {
    if (args.apply) return launch_phase<PH_UPDATE_APPLY>(dtype, args, s);
    return launch_phase<PH_UPDATE>(dtype, args, s);
}

}  // namespace muon
