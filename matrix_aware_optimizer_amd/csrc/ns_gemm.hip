// Newton-Schulz GEMMs on the gfx950 matrix cores.
//
// One step of the quintic iteration ([Muon优化器] linsight.cn/f25d614e.html,
// zeropower_via_newtonschulz and section "Newton-Schulz 迭代——高效实现与系数
// 优化") on the NS-frame iterate X (m x n, m <= n):
//     A  = X X^T                 (gram_kernel: symmetric, upper half tiles)
//     B  = b A + c A A           (poly_kernel: A A = A A^T, upper half tiles)
//     X' = a X + B X             (update_kernel)
// All three are "TN" products C[i][j] = sum_k P[i][k] Q[j][k] with both
// operands stored k-contiguous: P = Q = X for the Gram, P = Q = A for the
// polynomial (A is symmetric), and P = B, Q = X^T for the update (the
// workspace keeps a transposed operand copy of X for that).
//
// Engine: a 256 x 256 (bf16) or 128 x 128 (fp32) block tile per workgroup of
// 8 waves (2 x 4, two waves per SIMD so one can issue MFMAs while the other
// waits on memory); each wave owns a 128 x 64 (64 x 32) sub-tile built from
// 32 x 32 MFMA blocks (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32,
// fp32 accumulation).  Each k-step stages 128 bytes of every operand row in
// LDS with direct global->LDS loads (global_load_lds_dwordx4, no VGPR
// staging), double-buffered; the loads of the next k-step are spread between
// the MFMA groups of the current one.  16-byte chunks are XOR-swizzled with
// bits 1..3 of the row, which keeps ds_read_b128 fragment reads free of bank
// conflicts on gfx950's LDS (measured with SQ_LDS_BANK_CONFLICT).  MFMA
// fragments are double-buffered in registers: the reads for the next k-slice
// are issued between the MFMAs of the current one, at most 8 in flight.
// Buffers are zero-padded to the block tile, so there are no edge masks.
//
// Grouping: one launch covers every matrix of the call.  The tile space is the
// concatenation of all matrices' tiles (per-matrix prefix sums, largest
// matrices first), one workgroup per tile.  The hardware deals workgroups
// round-robin over the 8 XCDs, so tiles that are close in this order run at
// the same time; the update's tile order (grouped_decode) keeps such tiles on
// shared operand blocks.
#include "muon_internal.h"

namespace muon {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// native 16-byte vector (HIP's uint4 is a wrapper struct that defeats register promotion)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

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

// Physical position of logical 16-byte chunk c of LDS row `row`.
__device__ __forceinline__ int swz(int row, int c) { return row * CHUNKS_PER_ROW + (c ^ ((row >> 1) & 7)); }


// Update-tile decode: tiles are ordered in groups of GROUP_M tile rows, column-
// major inside a group, so a run of 32 consecutive tiles (what one XCD works
// on at a time) is a GROUP_M x (32 / GROUP_M) block that shares GROUP_M row
// blocks of B and 32 / GROUP_M row blocks of X^T in its L2.
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

template <typename T>
struct Engine {
    static constexpr int BM = Cfg<T>::BM, BN = Cfg<T>::BN;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int SM = WM / 32, SN = WN / 32;
    static constexpr int ROWS = BM + BN;                              // P rows then Q rows
    static constexpr int STAGE = ROWS * CHUNKS_PER_ROW;               // 16-byte chunks per stage
    static constexpr int ROWS_PER_LOAD = 64 / CHUNKS_PER_ROW;         // one wave load = 1 KB = 8 rows
    static constexpr int LOADS = STAGE / 64 / NWAVES;                 // loads per wave per k-step
    static constexpr int SUB = CHUNKS_PER_ROW / 2;                    // MFMA k-slices per k-step
    static constexpr int GROUPS = SUB * SM;                           // MFMA groups per k-step
    static_assert(LOADS <= GROUPS, "one load per MFMA group at most");
    static_assert(SM >= SN, "fragment prefetch pairs A row i with B row i");

    // acc[i][j] = sum_k P[row0 + i][k] * Q[col0 + j][k] over the whole k range.
    static __device__ __attribute__((always_inline)) void run(const char* __restrict__ P, size_t ldp, const char* __restrict__ Q,
                                      size_t ldq, int ksteps, u32x4* lds, f32x16_t (&acc)[SM][SN]) {
        const int tid = threadIdx.x;
        const int lane = tid & 63, wave = tid >> 6;
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;

        // Load j of this wave fills LDS chunks [(wave*LOADS + j)*64, +64) of a stage in
        // lane order: lane l lands in row r = l / 8 of that 1 KB block at physical chunk
        // l % 8, which holds the row's logical chunk (l % 8) ^ ((r >> 1) & 7).
        const char* src[LOADS];
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int row = (wave * LOADS + j) * ROWS_PER_LOAD + lane / CHUNKS_PER_ROW;
            const int lc = (lane % CHUNKS_PER_ROW) ^ ((row >> 1) & 7);
            src[j] = (row < BM ? P + row * ldp : Q + (row - BM) * ldq) + lc * 16;
        }
        auto issue = [&](int kt, int j) {
            lds_ptr_t d = (lds_ptr_t)(lds + (kt & 1) * STAGE + (wave * LOADS + j) * 64);
            __builtin_amdgcn_global_load_lds((const void*)(src[j] + static_cast<size_t>(kt) * (CHUNKS_PER_ROW * 16)),
                                             d, 16, 0, 0);
        };
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
        for (int j = 0; j < LOADS; ++j) issue(0, j);

        const int half = lane >> 5;
        const int arow = wm * WM + (lane & 31), brow = BM + wn * WN + (lane & 31);
        for (int kt = 0; kt < ksteps; ++kt) {
            // this wave's loads of stage kt are done; the barrier makes every wave's visible
            // and guarantees stage (kt + 1) & 1 is no longer being read
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
            const u32x4* L = lds + (kt & 1) * STAGE;
            const bool more = kt + 1 < ksteps;
            u32x4 fa[2][SM], fb[2][SN];
#pragma unroll
            for (int i = 0; i < SM; ++i) fa[0][i] = L[swz(arow + i * 32, half)];
#pragma unroll
            for (int j = 0; j < SN; ++j) fb[0][j] = L[swz(brow + j * 32, half)];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < SUB; ++s) {
                const int cn = 2 * (s + 1) + half;
#pragma unroll
                for (int i = 0; i < SM; ++i) {
#pragma unroll
                    for (int j = 0; j < SN; ++j) mfma_chunk(acc[i][j], fa[s & 1][i], fb[s & 1][j], T{});
                    if (s + 1 < SUB) {
                        fa[(s + 1) & 1][i] = L[swz(arow + i * 32, cn)];
                        if (i < SN) fb[(s + 1) & 1][i] = L[swz(brow + i * 32, cn)];
                    }
                    const int g = s * SM + i;
                    if (g < LOADS && more) issue(kt + 1, g);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
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

enum Phase { PH_GRAM = 0, PH_POLY = 1, PH_UPDATE = 2 };

// ----------------------------------------------------------------------------
// Epilogue.  The accumulators leave the registers through LDS in SM passes:
// pass i stages the i-th 32-row block of every wave (WAVES_M strips of 32
// rows x BN columns, fp32).  A row pass then finalizes 4 consecutive columns
// per thread (coalesced along the output row) and writes the final values
// back; an optional column pass stores the same values transposed, 4
// consecutive rows per thread, 8 threads per 32-row column segment.
// ----------------------------------------------------------------------------
template <typename E>
struct EpiLayout {
    static constexpr int STRIP_ROWS = 32 * WAVES_M;
    static constexpr int LDW = E::BN + 4;                 // row stride in floats
    static constexpr int FLOATS = STRIP_ROWS * LDW;
    static constexpr int ROW_ITERS = STRIP_ROWS * (E::BN / 4) / GEMM_THREADS;
    static constexpr int COL_ITERS = WAVES_M * E::BN * 8 / GEMM_THREADS;
};

template <typename E, typename Op>
__device__ __attribute__((always_inline)) void epilogue(f32x16_t (&acc)[E::SM][E::SN], float* sbuf, int row0,
                                                        int col0, Op& op) {
    using L = EpiLayout<E>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    auto rq = [&](int i, int it, int& gi, int& sc, int& sr) {   // the row pass's quads
        const int q = tid + GEMM_THREADS * it;
        sr = q / (E::BN / 4);
        sc = (q % (E::BN / 4)) * 4;
        gi = row0 + (sr >> 5) * E::WM + i * 32 + (sr & 31);
    };
    float4 pre[L::ROW_ITERS];
    lds_barrier();   // the k-loop's last LDS reads are done
#pragma unroll
    for (int i = 0; i < E::SM; ++i) {
#pragma unroll
        for (int j = 0; j < E::SN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int sr = wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int sc = wn * E::WN + j * 32 + (lane & 31);
                sbuf[sr * L::LDW + sc] = acc[i][j][r];
            }
        // acc[i] is in LDS now; its registers take this pass's operands from
        // memory, whose latency overlaps the barrier
        if (Op::PREFETCH) {
#pragma unroll
            for (int it = 0; it < L::ROW_ITERS; ++it) {
                int gi, sc, sr;
                rq(i, it, gi, sc, sr);
                pre[it] = op.fetch(gi, col0 + sc);
            }
        }
        lds_barrier();
#pragma unroll
        for (int it = 0; it < L::ROW_ITERS; ++it) {
            int gi, sc, sr;
            rq(i, it, gi, sc, sr);
            float4* cell = reinterpret_cast<float4*>(sbuf + sr * L::LDW + sc);
            float4 v = *cell;
            op.row(gi, col0 + sc, v, pre[it]);
            *cell = v;
        }
        if (op.transposed) {
            lds_barrier();
#pragma unroll
            for (int it = 0; it < L::COL_ITERS; ++it) {
                const int q = tid + GEMM_THREADS * it;
                const int kq = q & 7, rest = q >> 3;
                const int sc = rest % E::BN, strip = rest / E::BN;
                const int sr = strip * 32 + kq * 4;
                const float4 v = make_float4(sbuf[sr * L::LDW + sc], sbuf[(sr + 1) * L::LDW + sc],
                                             sbuf[(sr + 2) * L::LDW + sc], sbuf[(sr + 3) * L::LDW + sc]);
                op.col(col0 + sc, row0 + strip * E::WM + i * 32 + kq * 4, v);
            }
        }
        lds_barrier();
    }
}

// Symmetric outputs (A, B): tile (ti, tj), ti <= tj, is stored at (ti, tj)
// and mirrored at (tj, ti).  A diagonal tile writes its upper triangle's
// values to both positions, so the stored matrix is exactly symmetric.
template <typename T>
struct SymStore {
    void* dst;
    size_t ld;
    bool diag;
    bool transposed = true;
    __device__ inline void put_row(int gi, int gj, const float4& v) const {
        const size_t idx = static_cast<size_t>(gi) * ld + gj;
        if (!diag || gi <= gj) {
            st_quad<T>(dst, idx, v);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (gi <= gj + e) st_elem<T>(dst, idx + e, f4get(v, e));
        }
    }
    // v holds rows gi..gi+3 of column gj; stored as row gj of the mirror
    __device__ inline void col(int gj, int gi, const float4& v) const {
        const size_t idx = static_cast<size_t>(gj) * ld + gi;
        if (!diag || gi + 3 < gj) {
            st_quad<T>(dst, idx, v);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (gi + e < gj) st_elem<T>(dst, idx + e, f4get(v, e));
        }
    }
};

template <typename T>
struct GramOp : SymStore<T> {
    static constexpr bool PREFETCH = false;
    float scale;
    __device__ inline float4 fetch(int, int) const { return make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ inline void row(int gi, int gj, float4& v, const float4&) const {
        v.x *= scale; v.y *= scale; v.z *= scale; v.w *= scale;
        this->put_row(gi, gj, v);
    }
};

template <typename T>
struct PolyOp : SymStore<T> {
    static constexpr bool PREFETCH = true;
    const void* a;
    float b, c;
    __device__ inline float4 fetch(int gi, int gj) const { return ld_quad<T>(a, static_cast<size_t>(gi) * this->ld + gj); }
    __device__ inline void row(int gi, int gj, float4& v, const float4& av) const {
        v.x = fmaf(c, v.x, b * av.x); v.y = fmaf(c, v.y, b * av.y);
        v.z = fmaf(c, v.z, b * av.z); v.w = fmaf(c, v.w, b * av.w);
        this->put_row(gi, gj, v);
    }
};

// X' = u (a X + B X): the epilogue adds a X (fp32 iterate, requested while
// the pass is staged), scales by u and writes the fp32 iterate in place, its
// bf16 operand copy and the transposed operand copy for the next step (both
// skipped after the last step).
template <typename T>
struct UpdateOp {
    static constexpr bool PREFETCH = true;
    float* x32;
    void* xop;
    void* xnT;
    size_t np, mp;
    float a, u;
    bool transposed;
    __device__ inline float4 fetch(int gi, int gj) const { return ld_f4(x32 + static_cast<size_t>(gi) * np + gj); }
    __device__ inline void row(int gi, int gj, float4& v, const float4& x) const {
        const size_t idx = static_cast<size_t>(gi) * np + gj;
        v.x = u * fmaf(a, x.x, v.x); v.y = u * fmaf(a, x.y, v.y);
        v.z = u * fmaf(a, x.z, v.z); v.w = u * fmaf(a, x.w, v.w);
        st_f4(x32 + idx, v);
        if (sizeof(T) == 2 && transposed) st_quad<T>(xop, idx, v);
    }
    __device__ inline void col(int gj, int gi, const float4& v) const {
        st_quad<T>(xnT, static_cast<size_t>(gj) * mp + gi, v);
    }
};

template <typename T, int PHASE>
__device__ __attribute__((always_inline)) void process_tile(const NsArgs& args, int t, u32x4* lds) {
    using E = Engine<T>;
    const int mi = find_matrix(args.prefix, args.nmat, t);
    const MatDesc& d = args.descs[mi];
    const int local = t - args.prefix[mi];
    const int mp = d.mp, np = d.np;

    int ti, tj;
    if (PHASE == PH_UPDATE) {
        grouped_decode(local, mp / E::BM, np / E::BN, ti, tj);
    } else {
        sym_decode(local, mp / E::BM, ti, tj);
    }
    const int row0 = ti * E::BM, col0 = tj * E::BN;
    float* sbuf = reinterpret_cast<float*>(lds);

    f32x16_t acc[E::SM][E::SN];
    if (PHASE == PH_GRAM) {
        const char* X = static_cast<const char*>(d.xop);
        const size_t ld = static_cast<size_t>(np) * sizeof(T);
        E::run(X + row0 * ld, ld, X + col0 * ld, ld, np * (int)sizeof(T) / (CHUNKS_PER_ROW * 16), lds, acc);
        GramOp<T> op;
        op.dst = d.amat; op.ld = mp; op.diag = ti == tj;
        // first step: X0 = s * M' is folded in as A0 = s^2 M' M'^T
        op.scale = args.first ? G(d.scal)[0] * G(d.scal)[0] : 1.0f;
        epilogue<E>(acc, sbuf, row0, col0, op);
    } else if (PHASE == PH_POLY) {
        const char* A = static_cast<const char*>(d.amat);
        const size_t ld = static_cast<size_t>(mp) * sizeof(T);
        E::run(A + row0 * ld, ld, A + col0 * ld, ld, mp * (int)sizeof(T) / (CHUNKS_PER_ROW * 16), lds, acc);
        PolyOp<T> op;
        op.dst = d.bmat; op.ld = mp; op.diag = ti == tj;
        op.a = d.amat; op.b = args.b; op.c = args.c;
        epilogue<E>(acc, sbuf, row0, col0, op);
    } else {
        const char* B = static_cast<const char*>(d.bmat);
        const char* XT = static_cast<const char*>(d.xopT[args.ping]);
        const size_t ld = static_cast<size_t>(mp) * sizeof(T);
        E::run(B + row0 * ld, ld, XT + col0 * ld, ld, mp * (int)sizeof(T) / (CHUNKS_PER_ROW * 16), lds, acc);
        UpdateOp<T> op;
        op.x32 = d.x32; op.xop = d.xop; op.xnT = d.xopT[args.ping ^ 1];
        op.np = np; op.mp = mp; op.a = args.a;
        // first step: X1 = s (a M' + B0 M') with M' unscaled in x32 / xop
        op.u = args.first ? G(d.scal)[0] : 1.0f;
        op.transposed = !args.last;
        epilogue<E>(acc, sbuf, row0, col0, op);
    }
}

template <typename T, int PHASE>
__global__ __launch_bounds__(GEMM_THREADS, 1) void ns_gemm_kernel(NsArgs args) {
    using E = Engine<T>;
    static_assert(EpiLayout<E>::FLOATS * 4 <= 2 * E::STAGE * 16, "epilogue staging exceeds LDS");
    __shared__ u32x4 lds[2 * E::STAGE];
    if (static_cast<int>(blockIdx.x) < args.total) process_tile<T, PHASE>(args, blockIdx.x, lds);
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
hipError_t launch_poly(int dtype, const NsArgs& args, hipStream_t s) { return launch_phase<PH_POLY>(dtype, args, s); }
hipError_t launch_update(int dtype, const NsArgs& args, hipStream_t s) { return launch_phase<PH_UPDATE>(dtype, args, s); }

}  // namespace muon
