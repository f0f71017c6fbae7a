// Internal types shared by the host orchestration (muon_api.hip) and the
// gfx950 kernels (momentum_apply.hip, ns_gemm.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Elementwise kernels walk the Newton-Schulz frame in EW_TILE x EW_TILE tiles.
constexpr int EW_TILE = 64;
constexpr int EW_THREADS = 256;

// Block tile of the MFMA GEMM engine, by operand type.  Every Newton-Schulz
// buffer in the workspace is zero-padded to a multiple of it in both
// dimensions, so the GEMM kernels never need edge masks.
constexpr int GEMM_TILE_BF16 = 256;
constexpr int GEMM_TILE_F32 = 128;
constexpr int GEMM_THREADS = 512;   // 8 waves: two per SIMD

// The bf16 iterate's lo part is kept in the update kernel's accumulator layout, so
// that the update reads it straight into its accumulators and writes it straight from
// them, one contiguous kilobyte per wave instruction.  The padded matrix is cut into
// 256 x 256 tiles in row-major tile order, 64 Ki elements each.  Within a tile, 16-byte
// chunk v * 512 + t belongs to thread t = 64 w + l of the update's workgroup (wave
// w = 4 wm + wn, lane l) and holds its accumulator registers 8 h .. 8 h + 7 of 32 x 32
// block (i, j), v = 4 i + 2 j + h.  Register q of that block is tile row
// 128 wm + 32 i + 8 (q / 4) + 4 (l / 32) + q % 4 and tile column 64 wn + 32 j + l % 32
// (the 32 x 32 MFMA output layout).
static_assert(GEMM_TILE_BF16 == 256, "lo_offset is written for 256 x 256 tiles");
__host__ __device__ inline size_t lo_offset(int row, int col, int np) {
    const int r = row & 255, c = col & 255;
    const int wm = r >> 7, wn = c >> 6, i = (r >> 5) & 3, j = (c >> 5) & 1, rr = r & 31;
    const int q = 4 * (rr >> 3) + (rr & 3);            // accumulator register
    const int l = (c & 31) + 32 * ((rr >> 2) & 1);      // lane
    const int v = 4 * i + 2 * j + (q >> 3);
    const int t = 64 * (4 * wm + wn) + l;
    const size_t tile = static_cast<size_t>(row >> 8) * (np >> 8) + (col >> 8);
    return tile * 65536 + (static_cast<size_t>(v) * 512 + t) * 8 + (q & 7);
}

enum Dtype : int32_t { DT_F32 = 0, DT_BF16 = 1 };

// One active matrix.  "User frame" is the caller's rows x cols layout;
// the "NS frame" is m x n with m = min(rows, cols) <= n: tall matrices
// (rows > cols) are stored transposed there, so the Gram matrix is always
// formed on the smaller side.
struct MatDesc {
    // caller buffers (user frame)
    void* w;            // weight (muon_step) or nullptr (muon_ns)
    const void* g;      // gradient (muon_step) or input (muon_ns)
    void* mom;          // momentum state (muon_step) or nullptr
    float* out;         // fp32 output (muon_ns) or nullptr
    int32_t rows, cols;
    int32_t m, n;       // NS frame
    int32_t mp, np;     // NS frame padded to the GEMM tile
    int32_t tall;       // 1 if rows > cols
    int32_t uvec;       // 1 if cols % 8 == 0 and every caller pointer is 16-byte aligned
    // workspace buffers (NS frame, mp x np, zero-padded).  Step k reads index
    // k & 1 and writes index (k & 1) ^ 1.
    //   fp32: the iterate is x32[k & 1], which is also the MFMA operand.
    //   bf16: the iterate is the pair hi + lo with hi = bf16(X) = xop[k & 1]
    //         (the MFMA operand, row-major) and lo = bf16(X - hi) = xlo (about
    //         16 significant bits in all), stored in the update's accumulator
    //         layout (lo_offset); x32 is unused.
    float* x32[2];
    void* xop[2];       // operand copies, ping-pong; equal to x32 for fp32
    // Operand read by the first step (Gram and update): xop[0], or, when
    // hi_alias is set, the caller's buffer that already holds hi = bf16(U)
    // bit for bit (the stored momentum M' = U, or muon_ns's bf16 input), in
    // which case K1 writes only lo.  Set for bf16, no Nesterov, at least one
    // step, untransposed, rows and cols multiples of the GEMM tile, 16-byte
    // aligned pointers.  If the norm shift applies, the rescale kernel writes
    // the shifted hi to xop[0] and points hi0 there.
    const void* hi0;
    int32_t hi_alias;
    int32_t pad_alias;
    uint16_t* xlo;      // bf16 only, updated in place, element (r, c) at lo_offset(r, c, np)
    void* amat;         // mp x mp, A = X X^T (symmetric, stored in full)
    void* bmat;         // mp x mp, B = b A + c A A (symmetric, stored in full)
    // Normalization scalars, NS_SCAL floats per matrix:
    //   [0] s = 1 / (nu' + eps 2^-E), the scale of X0 = s U' with U' = 2^-E U
    //   [1] nu = ||U||_F (fp32, saturating)
    //   [2] E, the exact power-of-two shift applied to the stored iterate (0
    //       unless nu lies outside [2^-NS_SHIFT_LIMIT, 2^NS_SHIFT_LIMIT])
    float* scal;
    float apply_coef;   // lr * scale_rule(rows, cols)
    float decay;        // 1 - lr * weight_decay
    int32_t ew_tile0, ew_tiles;    // elementwise tiles: first global index, count
    int32_t sym_tile0, sym_tiles;  // Gram / polynomial half tiles
    int32_t upd_tile0, upd_tiles;  // update tiles
};

// Scalars kept per matrix for the normalization (see MatDesc::scal), and the
// norm range in which the iterate is stored unshifted.  Inside it the first
// step's Gram products s^2 U U^T stay far from fp32 overflow (nu^2 <= 2^96)
// and their entries far from underflow.
constexpr int NS_SCAL = 4;
constexpr int NS_SHIFT_LIMIT = 48;

struct EwArgs {
    const MatDesc* descs;
    const int32_t* prefix;   // nmat + 1 exclusive prefix sums of ew_tiles
    double* partials;        // one sum of squares per elementwise tile (fp64)
    int32_t nmat;
    int32_t total;
    int32_t tiles_per_block;
    float beta;
    int32_t nesterov;
    int32_t ns_zero;         // 1 when ns_steps == 0 (output is the normalized input)
    int32_t fin;             // index of the last step's iterate (ns_steps & 1)
};

// A GEMM phase's tile space as runs of consecutive matrices with equal tile counts (the
// plan sorts the matrices by size, so equal shapes are adjacent): run r covers tiles
// tile0 .. of matrices mat0 .., `tiles` tiles each.
struct TileRun {
    int32_t tile0, mat0, tiles;
};

constexpr int NS_ARG_RUNS = 4;   // runs passed by value; longer lists use the table
struct NsArgs {
    const MatDesc* descs;
    const TileRun* runs;     // this phase's runs, ordered by tile0 (tile0 of run 0 is 0)
    int32_t nruns;
    int32_t total;
    TileRun run[NS_ARG_RUNS];   // runs[0 .. nruns) when nruns <= NS_ARG_RUNS
    float a, b, c;           // this step's coefficients
    int32_t first;           // first step: fold the normalization scale in
    int32_t apply;           // last step of muon_step: write W' = decay W - coef X' instead of X'
    int32_t ping;            // x32 / xop index read by this step; ping ^ 1 is written
};

// AdamW: one tensor of the list; work is split into ADAMW_CHUNK-element chunks.
constexpr int ADAMW_THREADS = 256;
constexpr int ADAMW_CHUNK = ADAMW_THREADS * 16;
struct AdamWDesc {
    void* p;
    const void* g;
    float* m;
    float* v;
    int64_t numel;
    int32_t vec;        // 1 if p, g are 4-element aligned and m, v 16-byte aligned
    int32_t pad0;
};
struct AdamWArgs {
    const AdamWDesc* descs;
    const int32_t* prefix;   // n + 1 exclusive prefix sums of chunks
    int32_t n;
    int32_t total;           // chunks
    float beta1, beta2, one_m_beta1, one_m_beta2;
    float eps, decay;        // decay = 1 - lr * weight_decay
    float step_size;         // lr / (1 - beta1^t)
    float inv_sqrt_bc2;      // 1 / sqrt(1 - beta2^t)
};

// Muon-Cayley.  Each matrix is handled in its Stiefel frame N x K (N >= K,
// row-major fp32): the caller's matrix when rows >= cols, its transpose
// otherwise.  K x K reductions over N are split into row blocks of CY_RB rows
// whose partials are summed in a fixed order.
constexpr int CAYLEY_MAX_K = 256;
constexpr int CY_T = 64;          // tile edge of the frame transposes
constexpr int CY_GT = 128;        // output tile edge of the N x K and K x K products
constexpr int CY_RB = 512;        // rows per reduction block
constexpr int CY_THREADS = 256;
constexpr int CY_SOLVE_THREADS = 1024;
constexpr int CY_MT = 32;                // tile edge of the K x K sums (middle step, split-solve blocks)
constexpr int CY_LDS_K = 128;            // K up to which the solve is split and inverts in registers
constexpr int CY_SV_T = 64;              // tile edge of the split solve's K x K products
struct CayleyDesc {
    float* w;            // caller's weight (rows x cols)
    const float* g;      // caller's gradient
    float* m;            // caller's momentum
    int32_t rows, cols;
    int32_t N, K;        // Stiefel frame
    int32_t tall;        // 1: frame = caller's layout; 0: frame = transpose (copies below)
    int32_t nrb;         // reduction row blocks
    int32_t tk;          // K tiles per side: ceil(K / CY_T)
    int32_t tn;          // N tiles: ceil(N / CY_T)
    int32_t gk;          // product tiles per K side: ceil(K / CY_GT)
    int32_t gn;          // product tiles along N: ceil(N / CY_GT)
    float* wf;           // frame W (caller's buffer when tall)
    const float* gf;     // frame G
    float* mf;           // frame M, updated in place
    float* v;            // N x K tangent direction
    float* wnew;         // N x K updated W (frame)
    float* part;         // nrb x 3 x K x K partial products
    float* colpart;      // nrb x 2 x K partial column sums (G, W)
    float* small;        // K (mean) + K x K (S) + 2K x K (Y)
    double* cmat;        // 2K x 2K: B U, then the system I + c B U, then its LU factors
    double* rhs;         // 2K x K right-hand side, then the solution Z
    double* bw;          // 2K x K: B W = [W^T W; -V^T W]
};
struct CayleyArgs {
    const CayleyDesc* descs;
    const int32_t* prefix;   // nmat + 1 prefix sums of this phase's tiles
    int32_t nmat;
    int32_t total;
    float beta, c;           // momentum coefficient, c = lr / 2
};

// Kernel launchers (defined next to the kernels).
// CY_SOLVE inverts C11 and forms the right-hand side (K <= 128) or solves the whole
// system (K > 128); the CY_SV_* phases are the rest of the split solve for K <= 128.
enum CayleyPhase : int32_t { CY_TRANSPOSE_IN = 0, CY_REDUCE1 = 1, CY_MID = 2, CY_P2 = 3, CY_REDUCE3 = 4,
                             CY_SOLVE = 5, CY_P4 = 6, CY_OUT = 7, CY_SV_SUM = 8, CY_SV_G1 = 9, CY_SV_G2 = 10,
                             CY_SV_INV2 = 11, CY_SV_G3 = 12, CY_SV_G4 = 13 };
constexpr int CY_PHASES = 14;
hipError_t launch_cayley(int phase, const CayleyArgs& args, hipStream_t s);
hipError_t launch_adamw(int dtype, const AdamWArgs& args, int grid, hipStream_t s);
hipError_t launch_momentum_norm(int dtype, bool ns_only, const EwArgs& args, int grid, hipStream_t s);
hipError_t launch_norm_finalize(const MatDesc* descs, const double* partials, int nmat, float eps,
                                hipStream_t s);
hipError_t launch_rescale(int dtype, const EwArgs& args, int grid, hipStream_t s);
hipError_t launch_apply(int dtype, bool ns_only, const EwArgs& args, int grid, hipStream_t s);
hipError_t launch_gram(int dtype, const NsArgs& args, hipStream_t s);
hipError_t launch_poly(int dtype, const NsArgs& args, hipStream_t s);
hipError_t launch_update(int dtype, const NsArgs& args, hipStream_t s);

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also fences
// global memory, i.e. waits until every store the wave has issued is
// acknowledged.  Here only LDS operations are waited for, so global stores
// stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Index of the matrix that owns global tile t: the largest i with
// prefix[i] <= t (prefix has nmat + 1 entries, prefix[0] = 0).
__host__ __device__ inline int find_matrix(const int32_t* prefix, int nmat, int t) {
    int lo = 0, hi = nmat - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Matrix of GEMM tile t and the tile's index within it: a search over the runs
// (one to three for a model's layer or expert set) and one division, in place of a
// chain of dependent loads over every matrix's prefix sum.
__host__ __device__ inline int run_matrix(const TileRun* runs, int nruns, int t, int& local) {
    int lo = 0, hi = nruns - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (runs[mid].tile0 <= t) lo = mid; else hi = mid - 1;
    }
    const TileRun r = runs[lo];
    const int q = (t - r.tile0) / r.tiles;
    local = t - r.tile0 - q * r.tiles;
    return r.mat0 + q;
}
// The same from the runs passed by value (nruns <= NS_ARG_RUNS): no memory access, so
// the tile's descriptor is the first load that waits.
__host__ __device__ inline int run_matrix_args(const TileRun (&run)[NS_ARG_RUNS], int nruns, int t, int& local) {
    TileRun r = run[0];
#pragma unroll
    for (int i = 1; i < NS_ARG_RUNS; ++i)
        if (i < nruns && run[i].tile0 <= t) r = run[i];
    const int q = (t - r.tile0) / r.tiles;
    local = t - r.tile0 - q * r.tiles;
    return r.mat0 + q;
}

// Pointers reached through the descriptor table are generic; viewing them in
// the global address space lets the compiler emit global_* (not flat_*)
// memory instructions, which only count against vmcnt.
#define MUON_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ MUON_GLOBAL T* G(T* p) { return (MUON_GLOBAL T*)p; }

// Native vectors for global accesses (HIP's float4 / uint2 wrappers cannot be
// assigned across address spaces).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_f4(const float* p) {
    const f32x4_t v = G(reinterpret_cast<const f32x4_t*>(p))[0];
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_f4(float* p, float4 v) {
    const f32x4_t w = {v.x, v.y, v.z, v.w};
    G(reinterpret_cast<f32x4_t*>(p))[0] = w;
}
__device__ __forceinline__ u32x2_t ld_u2(const void* p) { return G(static_cast<const u32x2_t*>(p))[0]; }
__device__ __forceinline__ void st_u2(void* p, u32x2_t v) { G(static_cast<u32x2_t*>(p))[0] = v; }

// bf16 <-> fp32 (bf16 kept as its 16-bit pattern).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round to nearest, ties to even (v_cvt_pk_bf16_f32 on gfx950); NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two values packed into one dword, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

}  // namespace muon
