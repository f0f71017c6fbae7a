// Muon-Cayley on the Stiefel manifold for gfx950 (fp32, with an fp64 2K x 2K solve).
//
// Method ([Muon在Stiefel流形上的精确闭式更新解析] mlqm.cn/news/1339166, sections
// 1.3, 3.1-3.3 and 6.2), per matrix in its Stiefel frame W (N x K, N >= K,
// W^T W = I):
//   M' = beta M + (1 - beta) (G - 1 mean(G)^T)       (column-centered gradient, EMA)
//   V  = M' - W sym(W^T M')                          (tangent projection)
//   W' = (I + c A)^-1 (I - c A) W,  A = V W^T - W V^T,  c = lr / 2
// The retraction goes through the 2K x 2K form: with U = [V, W], B = [W^T; -V^T]
// (A = U B), C = I + c B U, B W = [W^T W; -V^T W] and Z = C^-1 (B W - c (B U)(B W)),
// W' = W - c U (B W + Z).  Everything N-sized is then four passes:
//   reduce1  W^T G, W^T M (K x K partials per row block) and, in the same launch,
//            column sums of G, W;
//   mid      mean(G), S = sym(beta W^T M + (1 - beta)(W^T G - colsum(W) mean^T))
//            (= sym(W^T M') by linearity, so M' needs no extra pass);
//   p2       M' (in place) and V = M' - W S;
//   reduce3  W^T W, W^T V, V^T V;
//   solve    in fp64, Y = B W + Z.  For K <= 128 by K x K blocks in phases: the
//            products on many workgroups, C11 and the Schur complement S inverted
//            in registers by one workgroup per matrix, without pivoting unless a
//            pivot is small.
//            For larger K one workgroup per matrix LU-factors C with partial pivoting;
//   p4       W' = W - c (V Y1 + W Y2) into the workspace, copied out by `out` (in
//            place for tall matrices with K <= 128, which need no copy).
// Wide matrices (rows < cols) are transposed into frame copies first and back at
// the end.  Reductions over rows are split into row blocks summed in a fixed
// order, so results are deterministic.
#include "muon_internal.h"

namespace muon {

namespace {

__device__ inline const CayleyDesc& cy_locate(const CayleyArgs& a, int t, int& local) {
    const int mi = find_matrix(a.prefix, a.nmat, t);
    local = t - a.prefix[mi];
    return a.descs[mi];
}

// ---------------------------------------------------------------------------
// Frame copies for wide matrices: frame (i, j) = caller (j, i)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(CY_THREADS) void cy_transpose_in(CayleyArgs a) {
    __shared__ float tile[CY_T][CY_T + 1];
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    const int i0 = (local / d.tk) * CY_T, j0 = (local % d.tk) * CY_T;
    const float* src[3] = {d.w, d.g, d.m};
    float* dst[3] = {d.wf, const_cast<float*>(d.gf), d.mf};
    for (int x = 0; x < 3; ++x) {
        for (int q = threadIdx.x; q < CY_T * CY_T; q += CY_THREADS) {
            const int lr = q / CY_T, lc = q % CY_T;             // caller row j0 + lr, column i0 + lc
            const int ur = j0 + lr, uc = i0 + lc;
            tile[lr][lc] = (ur < d.K && uc < d.N) ? G(src[x])[static_cast<size_t>(ur) * d.cols + uc] : 0.0f;
        }
        __syncthreads();
        for (int q = threadIdx.x; q < CY_T * CY_T; q += CY_THREADS) {
            const int fr = q / CY_T, fc = q % CY_T;
            const int i = i0 + fr, j = j0 + fc;
            if (i < d.N && j < d.K) G(dst[x])[static_cast<size_t>(i) * d.K + j] = tile[fc][fr];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// The N x K and K x K fp32 products run on the matrix cores (v_mfma_f32_32x32x2_f32).
// A workgroup forms one 128 x 128 output tile; its 4 waves split it 2 x 2, and each
// wave holds 2 x 2 blocks of 32 x 32 accumulators.  Operands are staged as 16-row
// k-chunks, both k-major: a[k][i] and b[k][j] (row stride MS floats, so that the two
// lane halves, which read rows k and k + 1, fall in opposite halves of the LDS banks).
// The next chunk is loaded into registers while the current one is multiplied.
// Accumulator register r of block (bi, bj) holds row 64 wm + 32 bi + 8 (r / 4) +
// 4 h + r % 4 and column 64 wn + 32 bj + c of the tile (wave = 2 wm + wn, lane =
// 32 h + c).
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int MK = 16;             // k rows per staged chunk
constexpr int MS = CY_GT + 36;     // LDS row stride in floats (640 B: rows k, k + 1 in opposite bank halves)
static_assert(CY_THREADS == 256 && CY_GT == 128, "4 waves, 2 x 2 of 64 x 64");

struct MfmaAcc {
    f32x16_t v[2][2];
    __device__ void zero() {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                for (int r = 0; r < 16; ++r) v[bi][bj][r] = 0.0f;
    }
    // acc += a^T b over one staged chunk (a: MK x CY_GT, b: MK x CY_GT, pitch MS)
    __device__ void chunk(const float* as, const float* bs) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int c = lane & 31, h = lane >> 5;
        const float* pa = as + h * MS + 64 * (wave >> 1) + c;
        const float* pb = bs + h * MS + 64 * (wave & 1) + c;
#pragma unroll
        for (int k = 0; k < MK; k += 2) {
            const float a0 = pa[k * MS], a1 = pa[k * MS + 32], b0 = pb[k * MS], b1 = pb[k * MS + 32];
            v[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, v[0][0], 0, 0, 0);
            v[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, v[0][1], 0, 0, 0);
            v[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, v[1][0], 0, 0, 0);
            v[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, v[1][1], 0, 0, 0);
        }
    }
    // f(row, col, value) for every accumulator, row and col relative to the tile
    template <typename F>
    __device__ void each(F f) const {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int c = lane & 31, h = lane >> 5;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    f(64 * (wave >> 1) + 32 * bi + 8 * (r >> 2) + 4 * h + (r & 3), 64 * (wave & 1) + 32 * bj + c,
                      v[bi][bj][r]);
    }
};

// X[row][col .. col + 3] (row-major, pitch ld floats), zero outside rows < nrow and cols < ncol.
__device__ __forceinline__ float4 ld4_guard(const float* base, size_t ld, int row, int nrow, int col, int ncol, bool vec) {
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (row >= nrow) return v;
    const float* p = base + static_cast<size_t>(row) * ld + col;
    if (vec && col + 3 < ncol) return ld_f4(p);
    if (col < ncol) v.x = G(p)[0];
    if (col + 1 < ncol) v.y = G(p)[1];
    if (col + 2 < ncol) v.z = G(p)[2];
    if (col + 3 < ncol) v.w = G(p)[3];
    return v;
}
__device__ __forceinline__ bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
__device__ __forceinline__ void st4_lds(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

// K x K partial product over rows [rs, re): out[i][j] = sum_r X[r][i] Y[r][j] for the
// tile at (i0, j0).  Both operands are k-major as stored (row r of X and Y).
__device__ __attribute__((always_inline)) void tn_block(const float* X, const float* Y, int K, int rs, int re, int i0, int j0, float* out) {
    constexpr int C4 = CY_GT / 4, NQ = MK * C4 / CY_THREADS;
    static_assert(NQ * CY_THREADS == MK * C4, "whole chunks per thread");
    __shared__ __attribute__((aligned(16))) float xs[MK * MS], ys[MK * MS];
    const int tid = threadIdx.x;
    const bool vec = (K & 3) == 0 && aligned16(X) && aligned16(Y);
    MfmaAcc acc;
    acc.zero();
    float4 xn[NQ], yn[NQ];
    auto fetch = [&](int r) {
#pragma unroll
        for (int e = 0; e < NQ; ++e) {
            const int q = tid + e * CY_THREADS, rr = q / C4, c4 = q % C4;
            xn[e] = ld4_guard(X, K, r + rr, re, i0 + 4 * c4, K, vec);
            yn[e] = ld4_guard(Y, K, r + rr, re, j0 + 4 * c4, K, vec);
        }
    };
    fetch(rs);
    for (int r = rs; r < re; r += MK) {
#pragma unroll
        for (int e = 0; e < NQ; ++e) {
            const int q = tid + e * CY_THREADS;
            st4_lds(xs + (q / C4) * MS + 4 * (q % C4), xn[e]);
            st4_lds(ys + (q / C4) * MS + 4 * (q % C4), yn[e]);
        }
        lds_barrier();
        if (r + MK < re) fetch(r + MK);
        acc.chunk(xs, ys);
        lds_barrier();   // the chunk is read before the next one is stored
    }
    acc.each([&](int ti, int tj, float x) {
        const int i = i0 + ti, j = j0 + tj;
        if (i < K && j < K) G(out)[static_cast<size_t>(i) * K + j] = x;
    });
}

// column sums of G and W over row block rb (thread j owns column j)
__device__ void colsum_block(const CayleyDesc& d, int rb) {
    __shared__ float part[2][CY_THREADS];
    const int K = d.K, tid = threadIdx.x;
    // column j = tid % K; the CY_THREADS / K row subsets of the block are summed
    // separately (rows s, s + S, ...) and combined in a fixed order
    const int S = max(1, CY_THREADS / K), j = tid % K, sub = tid / K;
    const int rs = rb * CY_RB, re = min(d.N, rs + CY_RB);
    float sg = 0.0f, sw = 0.0f;
    if (sub < S) {
#pragma unroll 8
        for (int r = rs + sub; r < re; r += S) {
            const size_t idx = static_cast<size_t>(r) * K + j;
            sg += G(d.gf)[idx];
            sw += G(d.wf)[idx];
        }
    }
    part[0][tid] = sg;
    part[1][tid] = sw;
    __syncthreads();
    if (tid < K) {
        float tg = 0.0f, tw = 0.0f;
        for (int k = 0; k < S; ++k) {
            tg += part[0][k * K + tid];
            tw += part[1][k * K + tid];
        }
        G(d.colpart)[(static_cast<size_t>(rb) * 2 + 0) * K + tid] = tg;
        G(d.colpart)[(static_cast<size_t>(rb) * 2 + 1) * K + tid] = tw;
    }
}

// One K x K product tile of one row block per workgroup.  REDUCE1: W^T G and W^T M, and
// after them the column sums of G and W, one row block per workgroup (they read the same
// inputs and fill workgroup slots the products leave free); REDUCE3: W^T W, W^T V and
// V^T V (the partial slots 0, 1, 2 of the row block).
template <int PHASE>
__global__ __launch_bounds__(CY_THREADS) void cy_reduce(CayleyArgs a) {
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    const int per = d.gk * d.gk;
    if (PHASE == CY_REDUCE1 && local >= 2 * d.nrb * per) {
        colsum_block(d, local - 2 * d.nrb * per);
        return;
    }
    const int t2 = local % per, rest = local / per;
    const int rb = rest % d.nrb, prod = rest / d.nrb;
    const int i0 = (t2 / d.gk) * CY_GT, j0 = (t2 % d.gk) * CY_GT;
    const int rs = rb * CY_RB, re = min(d.N, rs + CY_RB);
    const size_t kk = static_cast<size_t>(d.K) * d.K;
    float* out = d.part + (static_cast<size_t>(rb) * 3 + prod) * kk;
    if (PHASE == CY_REDUCE1) {
        tn_block(d.wf, prod == 0 ? d.gf : d.mf, d.K, rs, re, i0, j0, out);
    } else {
        const float* X = prod == 2 ? d.v : d.wf;
        const float* Y = prod == 0 ? d.wf : d.v;
        tn_block(X, Y, d.K, rs, re, i0, j0, out);
    }
}


// K x K sums by CY_MT x CY_MT tile pairs: a workgroup sums the row-block partials of
// its tile (i0, j0) and of the mirror tile (j0, i0), both read as coalesced rows, and
// gets the transposed entries it needs from the mirror through LDS.  Thread t holds
// entries (r, c) = (q / CY_MT, q % CY_MT), q = t + e CY_THREADS.
constexpr int MID_E = CY_MT * CY_MT / CY_THREADS;
static_assert(MID_E * CY_THREADS == CY_MT * CY_MT, "whole tiles");

// mean(G) and S = sym(H), H = beta W^T M + (1 - beta)(W^T G - colsum(W) mean^T), which
// equals sym(W^T M') by linearity
__global__ __launch_bounds__(CY_THREADS) void cy_mid(CayleyArgs a) {
    __shared__ float hm[CY_MT][CY_MT + 1];
    __shared__ float mean_s[2][CY_MT], colw_s[2][CY_MT];   // [0]: the tile's rows i, [1]: its columns j
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    const int K = d.K, mt = (K + CY_MT - 1) / CY_MT;
    const int i0 = (local / mt) * CY_MT, j0 = (local % mt) * CY_MT;
    const size_t kk = static_cast<size_t>(K) * K;
    for (int e = threadIdx.x; e < 2 * CY_MT; e += CY_THREADS) {
        const int side = e / CY_MT, col = (side ? j0 : i0) + e % CY_MT;
        float sg = 0.0f, sw = 0.0f;
        if (col < K) {
            for (int rb = 0; rb < d.nrb; ++rb) {
                sg += G(d.colpart)[(static_cast<size_t>(rb) * 2 + 0) * K + col];
                sw += G(d.colpart)[(static_cast<size_t>(rb) * 2 + 1) * K + col];
            }
        }
        const float mean = sg / static_cast<float>(d.N);
        mean_s[side][e % CY_MT] = mean;
        colw_s[side][e % CY_MT] = sw;
        if (side == 1 && i0 == 0 && col < K) G(d.small)[col] = mean;
    }
    __syncthreads();
    const float beta = a.beta, omb = 1.0f - a.beta;
    float hd[MID_E];
#pragma unroll
    for (int e = 0; e < MID_E; ++e) {
        const int q = threadIdx.x + e * CY_THREADS, r = q / CY_MT, c = q % CY_MT;
        const int i = i0 + r, j = j0 + c;     // direct entry H[i][j]
        const int im = j0 + r, jm = i0 + c;   // mirror entry H[im][jm]
        const bool dok = i < K && j < K, mok = im < K && jm < K;
        float g = 0.0f, m = 0.0f, gm = 0.0f, mm = 0.0f;
#pragma unroll 4
        for (int rb = 0; rb < d.nrb; ++rb) {
            const float* pr = d.part + static_cast<size_t>(rb) * 3 * kk;
            if (dok) {
                g += G(pr)[static_cast<size_t>(i) * K + j];
                m += G(pr)[kk + static_cast<size_t>(i) * K + j];
            }
            if (mok) {
                gm += G(pr)[static_cast<size_t>(im) * K + jm];
                mm += G(pr)[kk + static_cast<size_t>(im) * K + jm];
            }
        }
        hd[e] = fmaf(beta, m, omb * (g - colw_s[0][r] * mean_s[1][c]));
        hm[r][c] = fmaf(beta, mm, omb * (gm - colw_s[1][r] * mean_s[0][c]));
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < MID_E; ++e) {
        const int q = threadIdx.x + e * CY_THREADS, r = q / CY_MT, c = q % CY_MT;
        const int i = i0 + r, j = j0 + c;
        if (i < K && j < K) G(d.small)[K + static_cast<size_t>(i) * K + j] = 0.5f * (hd[e] + hm[c][r]);   // H[j][i]
    }
}

// acc += A[r0.., 0:Kr] B[0:Kr, c0..] for a 128 x 128 output tile (A row-major N x lda,
// B row-major K wide); A's chunk is staged transposed, as[k][row].
__device__ void nn_accumulate(const float* A, int lda, int N, const float* B, int K, int Kr, int r0, int c0,
                              MfmaAcc& acc) {
    constexpr int C4 = CY_GT / 4, NQ = MK * C4 / CY_THREADS;
    static_assert(NQ * CY_THREADS == MK * C4, "whole chunks per thread");
    __shared__ __attribute__((aligned(16))) float as[MK * MS], bs[MK * MS];
    const int tid = threadIdx.x;
    const bool avec = (lda & 3) == 0 && aligned16(A), bvec = (K & 3) == 0 && aligned16(B);
    float4 an[NQ], bn[NQ];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int e = 0; e < NQ; ++e) {
            const int q = tid + e * CY_THREADS;
            an[e] = ld4_guard(A, lda, r0 + q / 4, N, k0 + 4 * (q % 4), Kr, avec);   // row r0 + q/4, 4 k
            const int kr = q / C4, c4 = q % C4;
            bn[e] = ld4_guard(B, K, k0 + kr, Kr, c0 + 4 * c4, K, bvec);
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < Kr; k0 += MK) {
#pragma unroll
        for (int e = 0; e < NQ; ++e) {
            const int q = tid + e * CY_THREADS, row = q / 4, k4 = q % 4;
            as[(4 * k4 + 0) * MS + row] = an[e].x;
            as[(4 * k4 + 1) * MS + row] = an[e].y;
            as[(4 * k4 + 2) * MS + row] = an[e].z;
            as[(4 * k4 + 3) * MS + row] = an[e].w;
            st4_lds(bs + (q / C4) * MS + 4 * (q % C4), bn[e]);
        }
        lds_barrier();
        if (k0 + MK < Kr) fetch(k0 + MK);
        acc.chunk(as, bs);
        lds_barrier();   // the chunk is read before the next one is stored
    }
}

// M' = beta M + (1 - beta)(G - mean), in place; V = M' - W S
__global__ __launch_bounds__(CY_THREADS, 4) void cy_p2(CayleyArgs a) {
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    const int r0 = (local / d.gk) * CY_GT, c0 = (local % d.gk) * CY_GT;
    MfmaAcc acc;
    acc.zero();
    const float* S = d.small + d.K;
    nn_accumulate(d.wf, d.K, d.N, S, d.K, d.K, r0, c0, acc);
    const float beta = a.beta, omb = 1.0f - a.beta;
    // descriptor fields in registers: the stores below could alias the descriptor table,
    // so reading them through d would reload them after every store
    const int N = d.N, K = d.K;
    float* const mf = d.mf;
    float* const vo = d.v;
    const float* const gf = d.gf;
    const float* const mean = d.small;
    acc.each([&](int tr, int tc, float x) {
        const int r = r0 + tr, j = c0 + tc;
        if (r < N && j < K) {
            const size_t idx = static_cast<size_t>(r) * K + j;
            const float mn = fmaf(beta, G(mf)[idx], omb * (G(gf)[idx] - G(mean)[j]));
            G(mf)[idx] = mn;
            G(vo)[idx] = mn - x;
        }
    });
}

// W' = W - c (V Y1 + W Y2), into the workspace; in place for a tall matrix one tile
// wide, where this workgroup's rows of W are read only here, before they are written
__global__ __launch_bounds__(CY_THREADS, 4) void cy_p4(CayleyArgs a) {
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    const int r0 = (local / d.gk) * CY_GT, c0 = (local % d.gk) * CY_GT;
    const size_t kk = static_cast<size_t>(d.K) * d.K;
    const float* Y = d.small + d.K + kk;
    MfmaAcc acc;
    acc.zero();
    nn_accumulate(d.v, d.K, d.N, Y, d.K, d.K, r0, c0, acc);
    nn_accumulate(d.wf, d.K, d.N, Y + kk, d.K, d.K, r0, c0, acc);
    const int N = d.N, K = d.K;   // in registers, as in p2
    float* const wnew = d.wnew;
    const float* const wf = d.wf;
    const float c = a.c;
    acc.each([&](int tr, int tc, float x) {
        const int r = r0 + tr, j = c0 + tc;
        if (r < N && j < K) {
            const size_t idx = static_cast<size_t>(r) * K + j;
            G(wnew)[idx] = fmaf(-c, x, G(wf)[idx]);
        }
    });
}

// caller's W (and, for wide matrices, M) from the frame
__global__ __launch_bounds__(CY_THREADS) void cy_out(CayleyArgs a) {
    __shared__ float tile[CY_T][CY_T + 1];
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    const int i0 = (local / d.tk) * CY_T, j0 = (local % d.tk) * CY_T;
    if (d.tall) {
        for (int q = threadIdx.x; q < CY_T * CY_T; q += CY_THREADS) {
            const int i = i0 + q / CY_T, j = j0 + q % CY_T;
            if (i < d.N && j < d.K) {
                const size_t idx = static_cast<size_t>(i) * d.K + j;
                G(d.w)[idx] = G(d.wnew)[idx];
            }
        }
        return;
    }
    const float* src[2] = {d.wnew, d.mf};
    float* dst[2] = {d.w, d.m};
    for (int x = 0; x < 2; ++x) {
        for (int q = threadIdx.x; q < CY_T * CY_T; q += CY_THREADS) {
            const int fr = q / CY_T, fc = q % CY_T;
            const int i = i0 + fr, j = j0 + fc;
            tile[fr][fc] = (i < d.N && j < d.K) ? G(src[x])[static_cast<size_t>(i) * d.K + j] : 0.0f;
        }
        __syncthreads();
        for (int q = threadIdx.x; q < CY_T * CY_T; q += CY_THREADS) {
            const int lr = q / CY_T, lc = q % CY_T;    // caller row j0 + lr, column i0 + lc
            const int ur = j0 + lr, uc = i0 + lc;
            if (ur < d.K && uc < d.N) G(dst[x])[static_cast<size_t>(ur) * d.cols + uc] = tile[lc][lr];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// The 2K x 2K solve, one workgroup per matrix, fp64.
// ---------------------------------------------------------------------------
// The 2K x 2K system in global memory: LU with partial pivoting (any K).
__device__ void solve_global(const CayleyDesc& d, double cc, double* arena) {
    int* perm = reinterpret_cast<int*>(arena);                          // 2K
    double* prow = arena + CAYLEY_MAX_K;                                // 3K: pivot row of C and of the right-hand side
    double* lmul = prow + 3 * CAYLEY_MAX_K;                             // 2K: multipliers of the rows below the pivot
    double (*ta)[33] = reinterpret_cast<double (*)[33]>(lmul + 2 * CAYLEY_MAX_K);   // 32 x 33 product tiles
    double (*tb)[33] = ta + 32;
    const int K = d.K, K2 = 2 * K, tid = threadIdx.x;
    const size_t kk = static_cast<size_t>(K) * K;
    const double c = cc;
    double* C = d.cmat;       // 2K x 2K
    double* R = d.rhs;        // 2K x K
    double* BW = d.bw;        // 2K x K
    // 1. K x K products from the partials: W^T W, W^T V, V^T V (fp64 sums in row-block order)
    for (size_t q = tid; q < kk; q += CY_SOLVE_THREADS) {
        const int i = static_cast<int>(q / K), j = static_cast<int>(q % K);
        double ww = 0.0, wv = 0.0, vw = 0.0, vv = 0.0;   // (W^T W)ij, (W^T V)ij, (W^T V)ji, (V^T V)ij
        // row blocks in ascending order; the loads of RB blocks are issued before their sums
        constexpr int RB = 8;
        for (int rb0 = 0; rb0 < d.nrb; rb0 += RB) {
            float t[RB][4];
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                if (rb0 + u < d.nrb) {
                    const float* pr = d.part + static_cast<size_t>(rb0 + u) * 3 * kk;
                    t[u][0] = G(pr)[q];
                    t[u][1] = G(pr)[kk + q];
                    t[u][2] = G(pr)[kk + static_cast<size_t>(j) * K + i];
                    t[u][3] = G(pr)[2 * kk + q];
                }
            }
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                if (rb0 + u < d.nrb) {
                    ww += t[u][0];
                    wv += t[u][1];
                    vw += t[u][2];
                    vv += t[u][3];
                }
            }
        }
        // B U = [[W^T V, W^T W], [-V^T V, -V^T W]], with (V^T W)ij = (W^T V)ji
        C[static_cast<size_t>(i) * K2 + j] = wv;
        C[static_cast<size_t>(i) * K2 + K + j] = ww;
        C[static_cast<size_t>(K + i) * K2 + j] = -vv;
        C[static_cast<size_t>(K + i) * K2 + K + j] = -vw;
        BW[static_cast<size_t>(i) * K + j] = ww;
        BW[static_cast<size_t>(K + i) * K + j] = -vw;
    }
    __syncthreads();
    // 2. right-hand side B W - c (B U)(B W), 32 x 32 output tiles through LDS
    {
        const int ty = tid / 32, tx = tid % 32;
        for (int r0 = 0; r0 < K2; r0 += 32)
            for (int c0 = 0; c0 < K; c0 += 32) {
                double acc = 0.0;
                for (int l0 = 0; l0 < K2; l0 += 32) {
                    const int ar = r0 + ty, al = l0 + tx, bl = l0 + ty, bc = c0 + tx;
                    ta[ty][tx] = (ar < K2 && al < K2) ? C[static_cast<size_t>(ar) * K2 + al] : 0.0;
                    tb[ty][tx] = (bl < K2 && bc < K) ? BW[static_cast<size_t>(bl) * K + bc] : 0.0;
                    __syncthreads();
#pragma unroll 8
                    for (int l = 0; l < 32; ++l) acc = fma(ta[ty][l], tb[l][tx], acc);
                    __syncthreads();
                }
                const int r = r0 + ty, cc = c0 + tx;
                if (r < K2 && cc < K) R[static_cast<size_t>(r) * K + cc] = BW[static_cast<size_t>(r) * K + cc] - c * acc;
            }
    }
    __syncthreads();
    // 3. C = I + c B U
    for (size_t q = tid; q < static_cast<size_t>(K2) * K2; q += CY_SOLVE_THREADS) {
        const int i = static_cast<int>(q / K2), l = static_cast<int>(q % K2);
        C[q] = (i == l ? 1.0 : 0.0) + c * C[q];
    }
    for (int i = tid; i < K2; i += CY_SOLVE_THREADS) perm[i] = i;
    __syncthreads();
    // 4. LU with partial pivoting, applied to the right-hand side.  Rows stay in
    //    place: perm[i] is the stored row that plays the role of row i.  Per
    //    column: one wave finds the pivot; the pivot row and the multipliers go
    //    to LDS; every thread then updates its elements with one load and one store.
    for (int j = 0; j < K2; ++j) {
        if (tid < 64) {
            double best = -1.0;
            int bidx = K2;
            for (int i = j + tid; i < K2; i += 64) {
                const double v = fabs(C[static_cast<size_t>(perm[i]) * K2 + j]);
                if (v > best) { best = v; bidx = i; }
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const double ov = __shfl_xor(best, off, 64);
                const int oi = __shfl_xor(bidx, off, 64);
                if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
            }
            if (tid == 0 && bidx != j) {
                const int t = perm[j];
                perm[j] = perm[bidx];
                perm[bidx] = t;
            }
        }
        __syncthreads();
        const size_t pj = static_cast<size_t>(perm[j]);
        const int wc = K2 - j - 1, width = wc + K, rows = K2 - j - 1;
        for (int col = tid; col < width; col += CY_SOLVE_THREADS)
            prow[col] = col < wc ? C[pj * K2 + j + 1 + col] : R[pj * K + (col - wc)];
        {
            const double piv = C[pj * K2 + j];
            for (int i = tid; i < rows; i += CY_SOLVE_THREADS)
                lmul[i] = C[static_cast<size_t>(perm[j + 1 + i]) * K2 + j] / piv;
        }
        __syncthreads();
        for (size_t q = tid; q < static_cast<size_t>(rows) * width; q += CY_SOLVE_THREADS) {
            const int ii = static_cast<int>(q / width), col = static_cast<int>(q % width);
            const size_t pi = static_cast<size_t>(perm[j + 1 + ii]);
            double* dst = col < wc ? &C[pi * K2 + j + 1 + col] : &R[pi * K + (col - wc)];
            *dst -= lmul[ii] * prow[col];
        }
        __syncthreads();
    }
    // 5. back substitution by columns of U: the solution for row j goes to row perm[j]
    for (int j = K2 - 1; j >= 0; --j) {
        const size_t pj = static_cast<size_t>(perm[j]);
        const double piv = C[pj * K2 + j];
        for (int col = tid; col < K; col += CY_SOLVE_THREADS) {
            const double x = R[pj * K + col] / piv;
            R[pj * K + col] = x;
            prow[col] = x;
        }
        __syncthreads();
        for (size_t q = tid; q < static_cast<size_t>(j) * K; q += CY_SOLVE_THREADS) {
            const int i = static_cast<int>(q / K), col = static_cast<int>(q % K);
            const size_t pi = static_cast<size_t>(perm[i]);
            R[pi * K + col] -= C[pi * K2 + j] * prow[col];
        }
        __syncthreads();
    }
    // 6. Y = B W + Z, fp32 for the final pass
    float* Y = d.small + K + kk;
    for (size_t q = tid; q < static_cast<size_t>(K2) * K; q += CY_SOLVE_THREADS) {
        const int j = static_cast<int>(q / K), col = static_cast<int>(q % K);
        G(Y)[q] = static_cast<float>(BW[q] + R[static_cast<size_t>(perm[j]) * K + col]);
    }
}


// ---------------------------------------------------------------------------
// K <= 128: block elimination.  With WW = W^T W, WV = W^T V, VV = V^T V and
// VW = WV^T, the system C [z1; z2] = [r1; r2] has the K x K blocks
//   C11 = I + c WV,  C12 = c WW,  C21 = -c VV,  C22 = I - c VW,
// and B W = [WW; -VW].  Eliminating z1:
//   X = C11^-1 C12,  y = C11^-1 r1,  S = C22 - C21 X,  r' = r2 - C21 y,
//   z2 = S^-1 r',  z1 = y - X z2.
// C11 and S are inverted by Gauss-Jordan in registers, without pivoting unless a
// pivot is small; the products are K x K GEMMs through LDS tiles.  Every
// block is nonsingular: det C = det(I + c A) != 0 for skew A, C11 = I + c WV
// with WV skew up to rounding, and det C = det C11 det S.
// ---------------------------------------------------------------------------

// out = ((identity ? I : 0) + scale * src)^-1 by Gauss-Jordan with partial pivoting.
// The working matrix, 128 x 128 with the identity beyond K, lives in registers:
// thread t holds row t / 8, columns 16 (t % 8) .. 16 (t % 8) + 15.  Rows are not
// swapped: step j pivots on the unused row p_j with the largest |M[p][j]| (ties to
// the smaller row) and eliminates column j in place, so the final matrix E holds
// the inverse permuted, inv[a][p_b] = E[p_a][b].  Per step only the pivot search
// and the scaled pivot row pass through LDS.  out may be src.
__device__ __attribute__((always_inline)) void kk_gj_inverse(int K, double* out, const double* src, double scale, bool identity,
                                                           double* lds) {
    static_assert(CY_SOLVE_THREADS == 8 * CY_LDS_K, "eight threads per row of the 128 x 128 matrix");
    constexpr int CB = 16;   // columns per thread
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = tid >> 3, cb = tid & 7;
    double* red_abs = lds;                                  // [2][16] per-wave best |M[i][j]|
    double* red_val = lds + 32;                             // [2][16] its signed value
    int* red_row = reinterpret_cast<int*>(lds + 64);        // [2][16] its row
    // scaled pivot row, [2][8][17]: column block cb at 17 cb, so the 8 blocks that
    // one read instruction touches fall in different LDS banks
    constexpr int PSTRIDE = CB + 1, PBUF = 8 * PSTRIDE;
    double* prow = lds + 80;
    int* piv = reinterpret_cast<int*>(lds + 80 + 2 * PBUF);   // [128] pivot row of step j

    double m[CB];
#pragma unroll
    for (int k = 0; k < CB; ++k) {
        const int col = CB * cb + k;
        if (i < K && col < K)
            m[k] = (identity && i == col ? 1.0 : 0.0) + scale * src[static_cast<size_t>(i) * K + col];
        else
            m[k] = i == col ? 1.0 : 0.0;
    }
    bool used = i >= K;   // rows beyond K never pivot
    int my_step = 0;      // the step at which this row pivoted
    for (int jb = 0; jb < CY_LDS_K / CB && CB * jb < K; ++jb) {
#pragma unroll
        for (int e = 0; e < CB; ++e) {
            const int j = CB * jb + e;
            if (j < K) {   // uniform
                const int buf = j & 1;
                // pivot search.  The wave's 8 rows hold column j in lanes 8 r + jb: their
                // best |M[i][j]| on an unused row (ties to the smaller row), and its value
                double cabs = -1.0;
                int crow = CY_LDS_K;
                if (cb == jb && !used) { cabs = fabs(m[e]); crow = i; }
#pragma unroll
                for (int off = 8; off < 64; off <<= 1) {
                    const double oabs = __shfl_xor(cabs, off, 64);
                    const int orow = __shfl_xor(crow, off, 64);
                    if (oabs > cabs || (oabs == cabs && orow < crow)) { cabs = oabs; crow = orow; }
                }
                const double cval = __shfl(m[e], 8 * (crow & 7) + jb, 64);   // row crow is 8 wave + (crow & 7)
                if (lane == jb) {
                    red_abs[buf * 16 + wave] = cabs;
                    red_val[buf * 16 + wave] = cval;
                    red_row[buf * 16 + wave] = crow;
                }
                lds_barrier();
                // best of the 16 waves' candidates: lanes 0..15 of every wave reduce them
                static_assert(CY_SOLVE_THREADS / 64 == 16, "one candidate per wave, 16 waves");
                double babs = red_abs[buf * 16 + (lane & 15)];
                int brow = red_row[buf * 16 + (lane & 15)], bw = lane & 15;
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) {
                    const double oabs = __shfl_xor(babs, off, 64);
                    const int orow = __shfl_xor(brow, off, 64), ow = __shfl_xor(bw, off, 64);
                    if (oabs > babs || (oabs == babs && orow < brow)) { babs = oabs; brow = orow; bw = ow; }
                }
                const int p = __builtin_amdgcn_readfirstlane(brow);
                const double bval = red_val[buf * 16 + __builtin_amdgcn_readfirstlane(bw)];
                const double inv = 1.0 / bval;
                // M[i][j], from the lane of this row that holds column j
                const double colf = __shfl(m[e], (lane & ~7) | jb, 64);
                if (i == p) {
#pragma unroll
                    for (int k = 0; k < CB; ++k) {
                        m[k] = (CB * cb + k == j) ? inv : m[k] * inv;
                        prow[buf * PBUF + PSTRIDE * cb + k] = m[k];
                    }
                    used = true;
                    my_step = j;
                    if (cb == 0) piv[j] = p;
                }
                lds_barrier();
                if (i != p) {
#pragma unroll
                    for (int k = 0; k < CB; ++k) {
                        const int col = CB * cb + k;
                        m[k] = col == j ? -colf * inv : m[k] - colf * prow[buf * PBUF + PSTRIDE * cb + k];
                    }
                }
            }
        }
    }
    lds_barrier();   // every piv[] entry is written
    if (i < K) {
#pragma unroll
        for (int k = 0; k < CB; ++k) {
            const int b = CB * cb + k;
            if (b < K) out[static_cast<size_t>(my_step) * K + piv[b]] = m[k];
        }
    }
    __syncthreads();   // out is complete (global) before the next product reads it
}

// out = ((identity ? I : 0) + scale * src)^-1 by Gauss-Jordan without pivoting, for
// matrices whose symmetric part is positive definite: every pivot is then at least its
// smallest eigenvalue.  C11 = I + c W^T V: W^T V = skew(W^T M') on the manifold, so
// C11's symmetric part is I and every pivot is >= 1.  S, the Schur complement of C11:
// x^T S x = z^T C z for z = [-C11^-1 C12 x; x], so S's symmetric part is at least C's,
// I + (c / 2) [0, I - V^T V; I - V^T V, 0] on the manifold, whose smallest eigenvalue
// is 1 - (c / 2) max |1 - sigma(V)^2|.  Returns false, with out untouched, if a pivot
// fell below 1/2 in magnitude; the caller then pivots.  out may be src.
//
// The 128 x 128 working matrix (identity beyond K) sits in registers as 4 x 4 blocks:
// thread t holds rows 4 (t / 32) + r and columns 4 (t % 32) + e, so the 32 threads of a
// block row form one half-wave.  Step j: the pivot row's threads scale it and put it in
// LDS (one barrier); every thread reads the 4 entries over its columns, and takes M[i][j]
// for its rows from the lane of its half-wave that holds column j (readlane, no LDS).
__device__ __forceinline__ double readlane_f64(double x, int lane) {
    const long long v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(v), lane);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), lane);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
__device__ __attribute__((always_inline)) bool kk_gj_inverse_unpivoted(int K, double* out, const double* src, double scale,
                                                                     bool identity, double* lds) {
    static_assert(CY_SOLVE_THREADS == (CY_LDS_K / 4) * (CY_LDS_K / 4), "one 4 x 4 block per thread");
    constexpr int NB = CY_LDS_K / 4;   // 4 x 4 blocks per side
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rb = tid / NB, cb = tid % NB;
    const int half = lane >> 5;
    double* prow = lds;                                              // [2][CY_LDS_K] scaled pivot row
    int* wbad = reinterpret_cast<int*>(lds + 2 * CY_LDS_K);          // [16] per-wave small-pivot flags
    double m[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * rb + r, col = 4 * cb + e;
            if (i < K && col < K)
                m[r][e] = (identity && i == col ? 1.0 : 0.0) + scale * src[static_cast<size_t>(i) * K + col];
            else
                m[r][e] = i == col ? 1.0 : 0.0;
        }
    int bad = 0;   // a pivot of this wave's block rows fell below 1/2 (uniform in the wave)
    for (int jb = 0; 4 * jb < K; ++jb) {
#pragma unroll
        for (int je = 0; je < 4; ++je) {
            const int j = 4 * jb + je;
            if (j < K) {   // uniform
                const int buf = j & 1;
                // M[4 rb + r][j], from the lane of this half-wave that holds block column jb
                double colf[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const double c0 = readlane_f64(m[r][je], jb), c1 = readlane_f64(m[r][je], 32 + jb);
                    colf[r] = half ? c1 : c0;
                }
                if (wave == jb >> 1) {   // the wave that holds pivot row j
                    const double diag = readlane_f64(m[je][je], 32 * (jb & 1) + jb);
                    bad |= !(fabs(diag) >= 0.5);
                    if (rb == jb) {
                        const double inv = 1.0 / diag;
#pragma unroll
                        for (int e = 0; e < 4; ++e) m[je][e] = (4 * cb + e == j) ? inv : m[je][e] * inv;
                        f32x4_t* dst = reinterpret_cast<f32x4_t*>(prow + buf * CY_LDS_K + 4 * cb);
                        dst[0] = __builtin_bit_cast(f32x4_t, make_double2(m[je][0], m[je][1]));
                        dst[1] = __builtin_bit_cast(f32x4_t, make_double2(m[je][2], m[je][3]));
                    }
                }
                lds_barrier();
                const f32x4_t* srcp = reinterpret_cast<const f32x4_t*>(prow + buf * CY_LDS_K + 4 * cb);
                const double2 p01 = __builtin_bit_cast(double2, srcp[0]), p23 = __builtin_bit_cast(double2, srcp[1]);
                const double pv[4] = {p01.x, p01.y, p23.x, p23.y};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (4 * rb + r != j) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int col = 4 * cb + e;
                            m[r][e] = col == j ? -colf[r] * pv[e] : m[r][e] - colf[r] * pv[e];
                        }
                    }
                }
            }
        }
    }
    if (lane == 0) wbad[wave] = bad;
    __syncthreads();
    bool ok = true;
#pragma unroll
    for (int w = 0; w < CY_SOLVE_THREADS / 64; ++w) ok = ok && !wbad[w];
    if (ok) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * rb + r, col = 4 * cb + e;
                if (i < K && col < K) out[static_cast<size_t>(i) * K + col] = m[r][e];
            }
    }
    __syncthreads();   // out is complete (global), and every thread has left the LDS buffers
    return ok;
}

// ---------------------------------------------------------------------------
// Split solve for K <= CY_LDS_K.  The K x K fp64 blocks live in the workspace
// (pitch K); each phase reads only blocks that earlier phases wrote:
//   SV_SUM   WW, WV, VV and bwb = -VW from the row-block partials;
//   SOLVE    C11^-1 = (I + c WV)^-1 (one workgroup per matrix; unpivoted, pivoting if
//            a pivot is small), and beside it, on more workgroups, the right-hand side
//            r1 = WW - c (WV WW) - c (WW bwb),  r2 = bwb - c (bwb bwb) + c (VV WW);
//   SV_G1    X = c C11^-1 WW,  y = C11^-1 r1 (into WV's block);
//   SV_G2    S = I + c bwb + c VV X (into r1's block),  r' = r2 + c VV y (into C11^-1's);
//   SV_INV2  S^-1 in place (one workgroup per matrix; unpivoted, pivoting if a pivot
//            is small);
//   SV_G3    z2 = S^-1 r' (into VV's block);
//   SV_G4    z1 = y - X z2, and Y = B W + Z in fp32 for the final pass.
// The products run as 64 x 64 tiles on many workgroups, each element summed in
// ascending k as one fma chain.
// ---------------------------------------------------------------------------
constexpr int SV_T = CY_SV_T;
struct SvBlocks {
    double *WV, *VV, *C11i, *Xm, *R1, *R2, *WW, *bwb;
    __device__ explicit SvBlocks(const CayleyDesc& d) {
        const size_t kk = static_cast<size_t>(d.K) * d.K;
        WV = d.cmat; VV = d.cmat + kk; C11i = d.cmat + 2 * kk; Xm = d.cmat + 3 * kk;
        R1 = d.rhs; R2 = d.rhs + kk; WW = d.bw; bwb = d.bw + kk;
    }
};
__device__ __forceinline__ int sv_tiles(int K) { const int g = (K + SV_T - 1) / SV_T; return g * g; }

// acc = A B for the 64 x 64 tile (ti, tj) of a K x K product (pitch K), by 256 threads
// (tid < 256) with SV_LDS doubles of LDS at lds.  Thread t holds rows 4 (t / 16) + u and
// columns t % 16 + 16 v (u, v < 4); the next 16-wide k-chunk is loaded into registers
// while the current one is multiplied.  Its barriers are workgroup-wide: every 256-thread
// group of the workgroup runs the same k-loop.
constexpr int SV_KC = 16;
constexpr int SV_LDS = SV_T * (SV_KC + 1) + SV_KC * (SV_T + 4);
__device__ __attribute__((always_inline)) void sv_product(int K, const double* A, const double* B, int ti, int tj, double (&acc)[4][4], double* lds,
                           int tid) {
    constexpr int KC = SV_KC, NQ = SV_T * KC / CY_THREADS;
    static_assert(NQ * CY_THREADS == SV_T * KC, "whole chunks per thread");
    double* As = lds;                        // [SV_T][KC + 1]
    double* Bs = lds + SV_T * (KC + 1);      // [KC][SV_T + 4]
    const int ty = tid / 16, tx = tid % 16;
    const int r0 = ti * SV_T, c0 = tj * SV_T;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
    double an[NQ], bn[NQ];
    auto fetch = [&](int l0) {
#pragma unroll
        for (int e = 0; e < NQ; ++e) {
            const int q = tid + e * CY_THREADS;
            const int i = q / KC, l = q % KC;
            an[e] = (r0 + i < K && l0 + l < K) ? A[static_cast<size_t>(r0 + i) * K + l0 + l] : 0.0;
            const int bl = q / SV_T, bj = q % SV_T;
            bn[e] = (l0 + bl < K && c0 + bj < K) ? B[static_cast<size_t>(l0 + bl) * K + c0 + bj] : 0.0;
        }
    };
    fetch(0);
    for (int l0 = 0; l0 < K; l0 += KC) {
#pragma unroll
        for (int e = 0; e < NQ; ++e) {
            const int q = tid + e * CY_THREADS;
            As[(q / KC) * (KC + 1) + q % KC] = an[e];
            Bs[(q / SV_T) * (SV_T + 4) + q % SV_T] = bn[e];
        }
        lds_barrier();
        if (l0 + KC < K) fetch(l0 + KC);
#pragma unroll 4
        for (int l = 0; l < KC; ++l) {
            double av[4], bv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) av[u] = As[(4 * ty + u) * (KC + 1) + l];
#pragma unroll
            for (int v = 0; v < 4; ++v) bv[v] = Bs[l * (SV_T + 4) + tx + 16 * v];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] = fma(av[u], bv[v], acc[u][v]);
        }
        lds_barrier();   // the chunk is read before the next one is stored
    }
}

// out = alpha A B + base_scale base (+ I): one tile, each element rounded as
// alpha * acc, then + base_scale * base, then + 1 on the diagonal.
// Called by 256 threads (tid < 256) with SV_LDS doubles at lds; with store false the
// product runs (for the workgroup's barriers) but nothing is read from base or stored.
__device__ __attribute__((always_inline)) void sv_gemm(int K, double* out, const double* A, const double* B, double alpha, const double* base,
                        double base_scale, bool identity, int tile, double* lds, int tid, bool store = true) {
    const int g = (K + SV_T - 1) / SV_T, ti = tile / g, tj = tile % g;
    double acc[4][4];
    sv_product(K, A, B, ti, tj, acc, lds, tid);
    if (!store) return;
    const int ty = tid / 16, tx = tid % 16;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = ti * SV_T + 4 * ty + u, j = tj * SV_T + tx + 16 * v;
            if (i >= K || j >= K) continue;
            const size_t q = static_cast<size_t>(i) * K + j;
            double x = alpha * acc[u][v];
            if (base) x += base_scale * base[q];
            if (identity && i == j) x += 1.0;
            out[q] = x;
        }
}

// SV_SUM: the K x K blocks from the partials (fp64 sums in row-block order), by CY_MT tile
// pairs as in the middle step; bwb = -V^T W = -(W^T V)^T comes from the mirror tile
__global__ __launch_bounds__(CY_THREADS) void cy_sv_sum(CayleyArgs a) {
    __shared__ double tw[CY_MT][CY_MT + 1];
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    const SvBlocks bk(d);
    const int K = d.K, mt = (K + CY_MT - 1) / CY_MT;
    const int i0 = (local / mt) * CY_MT, j0 = (local % mt) * CY_MT;
    const size_t kk = static_cast<size_t>(K) * K;
#pragma unroll
    for (int e = 0; e < MID_E; ++e) {
        const int q = threadIdx.x + e * CY_THREADS, r = q / CY_MT, c = q % CY_MT;
        const int i = i0 + r, j = j0 + c, im = j0 + r, jm = i0 + c;
        const bool dok = i < K && j < K, mok = im < K && jm < K;
        const size_t qd = static_cast<size_t>(i) * K + j, qm = static_cast<size_t>(im) * K + jm;
        double ww = 0.0, wv = 0.0, vv = 0.0, wvm = 0.0;   // (W^T W)ij, (W^T V)ij, (V^T V)ij, (W^T V)[im][jm]
#pragma unroll 4
        for (int rb = 0; rb < d.nrb; ++rb) {
            const float* pr = d.part + static_cast<size_t>(rb) * 3 * kk;
            if (dok) {
                ww += G(pr)[qd];
                wv += G(pr)[kk + qd];
                vv += G(pr)[2 * kk + qd];
            }
            if (mok) wvm += G(pr)[kk + qm];
        }
        if (dok) {
            bk.WV[qd] = wv;
            bk.VV[qd] = vv;
            bk.WW[qd] = ww;
        }
        tw[r][c] = wvm;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < MID_E; ++e) {
        const int q = threadIdx.x + e * CY_THREADS, r = q / CY_MT, c = q % CY_MT;
        const int i = i0 + r, j = j0 + c;
        if (i < K && j < K) bk.bwb[static_cast<size_t>(i) * K + j] = -tw[c][r];   // -(W^T V)[j][i]
    }
}

// The right-hand side r = B W - c (B U)(B W), each block as two products in turn, by the
// extra workgroups of the SOLVE launch (it needs only the block sums, so it runs beside
// the C11 inversion): workgroup w takes tiles 4 w .. 4 w + 3 of the 2 x sv_tiles(K), one
// per 256-thread quarter, each in its own part of the LDS arena.
__device__ __attribute__((noinline)) void sv_rhs(const CayleyDesc& d, double c, int w, double* arena) {
    static_assert(CY_SOLVE_THREADS == 4 * CY_THREADS, "four tile products per workgroup");
    static_assert(4 * SV_LDS <= CY_LDS_K * CY_LDS_K + 3 * CY_LDS_K, "the quarters fit the arena");
    const SvBlocks bk(d);
    const int quarter = threadIdx.x / CY_THREADS, tid = threadIdx.x % CY_THREADS;
    const int nt = sv_tiles(d.K), idx = 4 * w + quarter;
    const bool valid = idx < 2 * nt;                // a spare quarter repeats tile 0 without storing
    const int t = valid ? idx : 0, tile = t % nt;
    double* lds = arena + quarter * SV_LDS;
    if (t < nt) {   // r1 = WW - c WV WW - c WW bwb
        sv_gemm(d.K, bk.R1, bk.WV, bk.WW, -c, bk.WW, 1.0, false, tile, lds, tid, valid);
        sv_gemm(d.K, bk.R1, bk.WW, bk.bwb, -c, bk.R1, 1.0, false, tile, lds, tid, valid);
    } else {        // r2 = bwb - c bwb bwb + c VV WW
        sv_gemm(d.K, bk.R2, bk.bwb, bk.bwb, -c, bk.bwb, 1.0, false, tile, lds, tid, valid);
        sv_gemm(d.K, bk.R2, bk.VV, bk.WW, c, bk.R2, 1.0, false, tile, lds, tid, valid);
    }
}

// SV_G1 .. SV_G4
template <int PHASE>
__global__ __launch_bounds__(CY_THREADS) void cy_sv_gemm(CayleyArgs a) {
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    const SvBlocks bk(d);
    const int K = d.K, nt = sv_tiles(K), tile = local % nt, which = local / nt;
    const double c = a.c;
    __shared__ double lds[SV_LDS];
    const int tid = threadIdx.x;
    double* y = bk.WV;
    double* S = bk.R1;
    double* rp = bk.C11i;
    double* z2 = bk.VV;
    if (PHASE == CY_SV_G1) {
        if (which == 0) sv_gemm(K, bk.Xm, bk.C11i, bk.WW, c, nullptr, 0.0, false, tile, lds, tid);
        else sv_gemm(K, y, bk.C11i, bk.R1, 1.0, nullptr, 0.0, false, tile, lds, tid);
    } else if (PHASE == CY_SV_G2) {
        if (which == 0) sv_gemm(K, S, bk.VV, bk.Xm, c, bk.bwb, c, true, tile, lds, tid);
        else sv_gemm(K, rp, bk.VV, y, c, bk.R2, 1.0, false, tile, lds, tid);
    } else if (PHASE == CY_SV_G3) {
        sv_gemm(K, z2, S, rp, 1.0, nullptr, 0.0, false, tile, lds, tid);
    } else {
        // z1 = y - X z2, then Y = B W + Z in fp32 (rows 0..K-1: top, K..2K-1: bottom), each
        // element by the thread that forms it
        const int g = (K + SV_T - 1) / SV_T, ti = tile / g, tj = tile % g;
        double acc[4][4];
        sv_product(K, bk.Xm, z2, ti, tj, acc, lds, tid);
        const size_t kk = static_cast<size_t>(K) * K;
        float* Y = d.small + K + kk;
        const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = ti * SV_T + 4 * ty + u, j = tj * SV_T + tx + 16 * v;
                if (i >= K || j >= K) continue;
                const size_t q = static_cast<size_t>(i) * K + j;
                double z1 = -1.0 * acc[u][v];
                z1 += 1.0 * y[q];
                G(Y)[q] = static_cast<float>(bk.WW[q] + z1);
                G(Y)[kk + q] = static_cast<float>(bk.bwb[q] + z2[q]);
            }
    }
}

// SOLVE: C11^-1 for K <= CY_LDS_K, the whole 2K x 2K LU solve otherwise; SV_INV2: S^-1
__global__ __launch_bounds__(CY_SOLVE_THREADS) void cy_solve(CayleyArgs a) {
    __shared__ __attribute__((aligned(16))) double arena[CY_LDS_K * CY_LDS_K + 3 * CY_LDS_K];
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    if (local > 0) {   // the right-hand side, beside the inversion
        sv_rhs(d, a.c, local - 1, arena);
        return;
    }
    if (d.K <= CY_LDS_K) {
        const SvBlocks bk(d);
        if (!kk_gj_inverse_unpivoted(d.K, bk.C11i, bk.WV, a.c, true, arena))
            kk_gj_inverse(d.K, bk.C11i, bk.WV, a.c, true, arena);
    } else {
        solve_global(d, a.c, arena);
    }
}
__global__ __launch_bounds__(CY_SOLVE_THREADS) void cy_sv_inv2(CayleyArgs a) {
    __shared__ __attribute__((aligned(16))) double arena[CY_LDS_K * CY_LDS_K + 3 * CY_LDS_K];
    int local;
    const CayleyDesc& d = cy_locate(a, blockIdx.x, local);
    const SvBlocks bk(d);
    if (!kk_gj_inverse_unpivoted(d.K, bk.R1, bk.R1, 1.0, false, arena))
        kk_gj_inverse(d.K, bk.R1, bk.R1, 1.0, false, arena);
}

}  // namespace

hipError_t launch_cayley(int phase, const CayleyArgs& args, hipStream_t s) {
    if (args.total <= 0) return hipSuccess;
    const dim3 grid(args.total), block(CY_THREADS);
    switch (phase) {
        case CY_TRANSPOSE_IN: hipLaunchKernelGGL(cy_transpose_in, grid, block, 0, s, args); break;
        case CY_REDUCE1: hipLaunchKernelGGL(cy_reduce<CY_REDUCE1>, grid, block, 0, s, args); break;
        case CY_MID: hipLaunchKernelGGL(cy_mid, grid, block, 0, s, args); break;
        case CY_P2: hipLaunchKernelGGL(cy_p2, grid, block, 0, s, args); break;
        case CY_REDUCE3: hipLaunchKernelGGL(cy_reduce<CY_REDUCE3>, grid, block, 0, s, args); break;
        case CY_SOLVE: hipLaunchKernelGGL(cy_solve, grid, dim3(CY_SOLVE_THREADS), 0, s, args); break;
        case CY_SV_SUM: hipLaunchKernelGGL(cy_sv_sum, grid, block, 0, s, args); break;
        case CY_SV_G1: hipLaunchKernelGGL(cy_sv_gemm<CY_SV_G1>, grid, block, 0, s, args); break;
        case CY_SV_G2: hipLaunchKernelGGL(cy_sv_gemm<CY_SV_G2>, grid, block, 0, s, args); break;
        case CY_SV_INV2: hipLaunchKernelGGL(cy_sv_inv2, grid, dim3(CY_SOLVE_THREADS), 0, s, args); break;
        case CY_SV_G3: hipLaunchKernelGGL(cy_sv_gemm<CY_SV_G3>, grid, block, 0, s, args); break;
        case CY_SV_G4: hipLaunchKernelGGL(cy_sv_gemm<CY_SV_G4>, grid, block, 0, s, args); break;
        case CY_P4: hipLaunchKernelGGL(cy_p4, grid, block, 0, s, args); break;
        case CY_OUT: hipLaunchKernelGGL(cy_out, grid, block, 0, s, args); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace muon
