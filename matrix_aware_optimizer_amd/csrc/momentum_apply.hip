// HBM-bound elementwise kernels of the Muon step for gfx950:
//   * momentum + Frobenius-norm partials (and the operand copies for the
//     Newton-Schulz GEMMs),
//   * the per-matrix norm finalize,
//   * scale / weight decay / apply.
// Each walks the Newton-Schulz frame of every matrix in 64 x 64 tiles; one
// grouped launch covers all matrices of a call.  A tile is staged through
// LDS so that both the caller's layout and the transposed layout are read
// and written with coalesced accesses.
//
// Method ([Muon优化器] linsight.cn/f25d614e.html, the industrial Muon class
// and zeropower_via_newtonschulz): M' = beta*M + G; U = M' (or beta*M' + G
// for Nesterov); the iteration starts from U / (||U||_F + eps); after it,
// W' = (1 - lr*wd) W - lr*s*X.
#include "muon_internal.h"
#include "lo_stage.h"

namespace muon {

namespace {

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ inline float load(const void* p, size_t i) { return G(static_cast<const float*>(p))[i]; }
    static __device__ inline void store(void* p, size_t i, float v) { G(static_cast<float*>(p))[i] = v; }
};
template <> struct Elem<uint16_t> {
    static __device__ inline float load(const void* p, size_t i) {
        return bf16_to_f32(G(static_cast<const uint16_t*>(p))[i]);
    }
    static __device__ inline void store(void* p, size_t i, float v) {
        G(static_cast<uint16_t*>(p))[i] = f32_to_bf16(v);
    }
};

// 8 consecutive elements of the caller's dtype as fp32 (one 16-byte bf16 or two
// 16-byte fp32 accesses), and the matching store.
template <typename T> __device__ inline void load8(const void* base, size_t idx, float (&v)[8]);
template <> __device__ inline void load8<float>(const void* base, size_t idx, float (&v)[8]) {
    const float4 a = ld_f4(static_cast<const float*>(base) + idx), b = ld_f4(static_cast<const float*>(base) + idx + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <> __device__ inline void load8<uint16_t>(const void* base, size_t idx, float (&v)[8]) {
    const u32x4_t q = G(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + idx))[0];
    const unsigned w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}
template <typename T> __device__ inline void store8(void* base, size_t idx, const float (&v)[8]);
template <> __device__ inline void store8<float>(void* base, size_t idx, const float (&v)[8]) {
    st_f4(static_cast<float*>(base) + idx, make_float4(v[0], v[1], v[2], v[3]));
    st_f4(static_cast<float*>(base) + idx + 4, make_float4(v[4], v[5], v[6], v[7]));
}
template <> __device__ inline void store8<uint16_t>(void* base, size_t idx, const float (&v)[8]) {
    G(reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(base) + idx))[0] =
        u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}

// Element ownership inside a 64 x 64 tile: thread t covers rows (t >> 3) + 32 p,
// p = 0, 1, and 8 consecutive columns starting at (t & 7) * 8.
constexpr int EW_GROUP = 8;
constexpr int EW_PASSES = EW_TILE * EW_TILE / (EW_GROUP * EW_THREADS);
static_assert(EW_PASSES == 2, "two 8-element groups per thread and tile");
__device__ __forceinline__ int ew_row(int p) { return (threadIdx.x >> 3) + (EW_THREADS / 8) * p; }
__device__ __forceinline__ int ew_col() { return (threadIdx.x & 7) * EW_GROUP; }

// Deterministic block sum (fixed shuffle pattern, fixed wave order).
// LDS barriers only: the tile's global stores stay in flight across them.
__device__ inline double block_sum_256(double v, double* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    lds_barrier();
    double total = ((red[0] + red[1]) + (red[2] + red[3]));
    lds_barrier();
    return total;
}

// Decode global elementwise tile t of matrix d into NS-frame tile origin.
__device__ inline void ew_tile_origin(const MatDesc& d, int local, int& i0, int& j0) {
    const int tcols = d.np / EW_TILE;
    i0 = (local / tcols) * EW_TILE;
    j0 = (local % tcols) * EW_TILE;
}

// ----------------------------------------------------------------------------
// Momentum + norm partials + operand copies.
//   Each thread owns two 8-element row groups of an NS-frame tile.  For a
//   matrix stored untransposed the caller's layout is the NS frame and the
//   groups are read and written in place; a tall matrix is read along the
//   caller's rows (coalesced) and turned through LDS.  Then: rows of the
//   iterate (fp32, or the bf16 pair hi + lo whose hi is the MFMA operand) and
//   the sum of squares, taken in NS-frame order so the result does not depend
//   on the caller's orientation.
// ----------------------------------------------------------------------------
template <typename T, bool NS_ONLY>
__device__ __forceinline__ void momentum_group(const MatDesc& d, float beta, int nesterov, int ur, int uc,
                                               float (&u)[EW_GROUP]) {
#pragma unroll
    for (int e = 0; e < EW_GROUP; ++e) u[e] = 0.0f;
    if (ur >= d.rows || uc >= d.cols) return;
    const size_t idx = static_cast<size_t>(ur) * d.cols + uc;
    if (d.uvec) {   // cols % 8 == 0: the whole group is inside the row
        float g[EW_GROUP];
        load8<T>(d.g, idx, g);
        if (NS_ONLY) {
#pragma unroll
            for (int e = 0; e < EW_GROUP; ++e) u[e] = g[e];
        } else {
            float m[EW_GROUP], mn[EW_GROUP];
            load8<T>(d.mom, idx, m);
#pragma unroll
            for (int e = 0; e < EW_GROUP; ++e) {
                mn[e] = fmaf(beta, m[e], g[e]);
                u[e] = nesterov ? fmaf(beta, mn[e], g[e]) : mn[e];
            }
            store8<T>(d.mom, idx, mn);
        }
    } else {
#pragma unroll
        for (int e = 0; e < EW_GROUP; ++e) {
            if (uc + e >= d.cols) break;
            const float g = Elem<T>::load(d.g, idx + e);
            if (NS_ONLY) {
                u[e] = g;
            } else {
                const float m = Elem<T>::load(d.mom, idx + e);
                const float mn = fmaf(beta, m, g);
                Elem<T>::store(d.mom, idx + e, mn);
                u[e] = nesterov ? fmaf(beta, mn, g) : mn;
            }
        }
    }
}

template <typename T, bool NS_ONLY>
__global__ __launch_bounds__(EW_THREADS) __attribute__((amdgpu_waves_per_eu(8))) void momentum_norm_kernel(EwArgs args) {
    // the turned tile and the lo stage share one LDS area (a barrier separates their uses):
    // at 16.7 KB a block, eight blocks of the grid's eight per CU are resident together
    __shared__ union __attribute__((aligned(16))) {
        float tile[EW_TILE][EW_TILE + 1];
        uint16_t lo[LO_STAGE_CHUNKS * 8];
    } stage;
    __shared__ double red[4];
    auto& tile = stage.tile;
    uint16_t* const lo_stage = stage.lo;
    const int t0 = blockIdx.x * args.tiles_per_block;
    const int t1 = min(args.total, t0 + args.tiles_per_block);
    if (t0 >= t1) return;
    int mi = find_matrix(args.prefix, args.nmat, t0);
    const int jl = ew_col();

    for (int t = t0; t < t1; ++t) {
        while (t >= args.prefix[mi + 1]) ++mi;
        // by value: the fields are read once per tile into registers (the stores below could
        // alias the descriptor table, so reads through a reference would follow every store)
        const MatDesc d = args.descs[mi];
        int i0, j0;
        ew_tile_origin(d, t - args.prefix[mi], i0, j0);
        float u[EW_PASSES][EW_GROUP];
        if (!d.tall) {
#pragma unroll
            for (int p = 0; p < EW_PASSES; ++p)
                momentum_group<T, NS_ONLY>(d, args.beta, args.nesterov, i0 + ew_row(p), j0 + jl, u[p]);
        } else {
            // caller rows are NS columns: load caller row (j0 + r), columns i0 + jl + e
#pragma unroll
            for (int p = 0; p < EW_PASSES; ++p) {
                float v[EW_GROUP];
                momentum_group<T, NS_ONLY>(d, args.beta, args.nesterov, j0 + ew_row(p), i0 + jl, v);
#pragma unroll
                for (int e = 0; e < EW_GROUP; ++e) tile[jl + e][ew_row(p)] = v[e];
            }
            lds_barrier();
#pragma unroll
            for (int p = 0; p < EW_PASSES; ++p)
#pragma unroll
                for (int e = 0; e < EW_GROUP; ++e) u[p][e] = tile[ew_row(p)][jl + e];
            if (sizeof(T) == 2) lds_barrier();   // every read of the turned tile precedes the lo stage
        }

        // ---- NS-frame rows: X32 (and the bf16 operand copy).  The squares are
        // summed in fp64: any fp32 value squares without overflow or underflow.
        double sq = 0.0;
#pragma unroll
        for (int p = 0; p < EW_PASSES; ++p) {
#pragma unroll
            for (int e = 0; e < EW_GROUP; ++e) {
                const double v = static_cast<double>(u[p][e]);
                sq = fma(v, v, sq);
            }
            const size_t idx = static_cast<size_t>(i0 + ew_row(p)) * d.np + (j0 + jl);
            if (sizeof(T) == 2) {
                // the iterate as the pair hi + lo: hi = bf16(U), lo = bf16(U - hi)
                unsigned h[4], l[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float a = u[p][2 * k], b = u[p][2 * k + 1];
                    h[k] = pack_bf16x2(a, b);
                    l[k] = pack_bf16x2(a - __uint_as_float(h[k] << 16), b - __uint_as_float(h[k] & 0xffff0000u));
                }
                // with hi_alias the caller's buffer already holds hi (the stored M', or the input)
                if (!d.hi_alias)
                    G(reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(d.xop[0]) + idx))[0] = u32x4_t{h[0], h[1], h[2], h[3]};
                lo_stage8(lo_stage, ew_row(p), jl, l);
            } else {
                store8<float>(d.x32[0], idx, u[p]);
            }
        }
        if (sizeof(T) == 2) {
            // lo in the update's accumulator layout: the staged tile is 8 whole 1 KB chunk
            // rows (v = 4 i_a + piece, lanes of wave 4 wm + wn), two 16-byte chunks a thread
            lds_barrier();
#pragma unroll
            for (int k = static_cast<int>(threadIdx.x); k < EW_TILE * EW_TILE / 8; k += EW_THREADS) {
                const u32x4_t v = reinterpret_cast<const u32x4_t*>(lo_stage)[lo_stage_slot(k)];
                G(reinterpret_cast<u32x4_t*>(d.xlo + lo_chunk_dst(i0, j0, d.np, k)))[0] = v;
            }
        }
        const double total = block_sum_256(sq, red);   // also orders LDS reuse
        if (threadIdx.x == 0) G(args.partials)[t] = total;
    }
}

// ----------------------------------------------------------------------------
// Norm finalize: one block per matrix sums its tile partials in a fixed order
// (fp64) and stores s = 1 / (||U||_F + eps).  When the norm lies outside
// [2^-NS_SHIFT_LIMIT, 2^NS_SHIFT_LIMIT] the stored iterate is shifted by an
// exact power of two E (rescale_kernel) so that its norm is in [1/2, 1):
// X0 = U / (nu + eps) = U' / (nu' + eps 2^-E) with U' = 2^-E U, nu' = 2^-E nu.
// The Newton-Schulz products then neither overflow (huge inputs) nor lose
// their entries to underflow (tiny inputs, or eps = 0).
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void norm_finalize_kernel(const MatDesc* descs, const double* partials,
                                                            float eps) {
    __shared__ double red[256];
    const MatDesc& d = descs[blockIdx.x];
    double acc = 0.0;
    for (int i = threadIdx.x; i < d.ew_tiles; i += 256) acc += partials[d.ew_tile0 + i];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double nrm = sqrt(red[0]);
        int e = 0;
        const double lim = static_cast<double>(1ull << NS_SHIFT_LIMIT);
        if (nrm > lim || (nrm > 0.0 && nrm < 1.0 / lim)) (void)frexp(nrm, &e);   // nrm = f 2^e, f in [1/2, 1)
        const double s = 1.0 / (ldexp(nrm, -e) + ldexp(static_cast<double>(eps), -e));
        G(d.scal)[0] = static_cast<float>(s);
        G(d.scal)[1] = static_cast<float>(nrm);
        G(d.scal)[2] = static_cast<float>(e);
    }
}

// ----------------------------------------------------------------------------
// Rescale: U' = 2^-E U for the matrices whose shift E is not zero (ldexp is
// exact; hi' = 2^-E hi and lo' = 2^-E lo stay the bf16 pair of U').  Blocks
// skip every matrix with E = 0 after one scalar read, so in the common case
// the launch does no memory traffic beyond that.  A matrix whose hi is the
// caller's buffer (hi_alias) gets its shifted hi in the workspace copy xop[0],
// and its first-step operand pointer hi0 is redirected there (every block of
// the matrix stores the same value; the GEMM launches that read it come later).
// ----------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(EW_THREADS) void rescale_kernel(EwArgs args) {
    const int t0 = blockIdx.x * args.tiles_per_block;
    const int t1 = min(args.total, t0 + args.tiles_per_block);
    if (t0 >= t1) return;
    int mi = find_matrix(args.prefix, args.nmat, t0);
    const int jl = ew_col();
    int t = t0;
    while (t < t1) {
        while (t >= args.prefix[mi + 1]) ++mi;
        const MatDesc d = args.descs[mi];
        const int e = static_cast<int>(G(d.scal)[2]);
        if (e == 0) {   // nothing to do for this matrix: jump past its tiles
            t = args.prefix[mi + 1];
            continue;
        }
        // source of hi: the caller's buffer (never written here) or the workspace copy, in place
        const void* hsrc = d.hi_alias ? (d.mom ? static_cast<const void*>(d.mom) : d.g) : d.xop[0];
        if (d.hi_alias && threadIdx.x == 0) const_cast<MatDesc*>(args.descs)[mi].hi0 = d.xop[0];
        const int tend = min(t1, args.prefix[mi + 1]);
        for (; t < tend; ++t) {
            int i0, j0;
            ew_tile_origin(d, t - args.prefix[mi], i0, j0);
#pragma unroll
            for (int p = 0; p < EW_PASSES; ++p) {
                const size_t idx = static_cast<size_t>(i0 + ew_row(p)) * d.np + (j0 + jl);
                if (sizeof(T) == 2) {
                    float h[EW_GROUP], l[EW_GROUP];
                    load8<uint16_t>(hsrc, idx, h);
                    load8<uint16_t>(d.xlo, idx, l);
#pragma unroll
                    for (int k = 0; k < EW_GROUP; ++k) {
                        h[k] = ldexpf(h[k], -e);
                        l[k] = ldexpf(l[k], -e);
                    }
                    store8<uint16_t>(d.xop[0], idx, h);
                    store8<uint16_t>(d.xlo, idx, l);
                } else {
                    float x[EW_GROUP];
                    load8<float>(d.x32[0], idx, x);
#pragma unroll
                    for (int k = 0; k < EW_GROUP; ++k) x[k] = ldexpf(x[k], -e);
                    store8<float>(d.x32[0], idx, x);
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------
// Apply: W' = (1 - lr*wd) W - lr*s_rule*X  (muon_step), or out = X (muon_ns).
// X is read in the NS frame; an untransposed matrix is written in place, a
// tall one is turned through LDS and written along the caller's rows.
// ----------------------------------------------------------------------------
template <typename T, bool NS_ONLY>
__device__ __forceinline__ void apply_group(const MatDesc& d, float coef, float oscale, int ur, int uc,
                                            const float (&o)[EW_GROUP]) {
    if (ur >= d.rows || uc >= d.cols) return;
    const size_t idx = static_cast<size_t>(ur) * d.cols + uc;
    if (d.uvec) {
        float r[EW_GROUP];
        if (NS_ONLY) {
#pragma unroll
            for (int e = 0; e < EW_GROUP; ++e) r[e] = o[e] * oscale;
            store8<float>(d.out, idx, r);
        } else {
            float w[EW_GROUP];
            load8<T>(d.w, idx, w);
#pragma unroll
            for (int e = 0; e < EW_GROUP; ++e) r[e] = fmaf(-coef, o[e], d.decay * w[e]);
            store8<T>(d.w, idx, r);
        }
    } else {
#pragma unroll
        for (int e = 0; e < EW_GROUP; ++e) {
            if (uc + e >= d.cols) break;
            if (NS_ONLY) {
                G(d.out)[idx + e] = o[e] * oscale;
            } else {
                const float w = Elem<T>::load(d.w, idx + e);
                Elem<T>::store(d.w, idx + e, fmaf(-coef, o[e], d.decay * w));
            }
        }
    }
}

template <typename T, bool NS_ONLY>
__global__ __launch_bounds__(EW_THREADS) void apply_kernel(EwArgs args) {
    __shared__ float tile[EW_TILE][EW_TILE + 1];
    const int t0 = blockIdx.x * args.tiles_per_block;
    const int t1 = min(args.total, t0 + args.tiles_per_block);
    if (t0 >= t1) return;
    int mi = find_matrix(args.prefix, args.nmat, t0);
    const int jl = ew_col();

    for (int t = t0; t < t1; ++t) {
        while (t >= args.prefix[mi + 1]) ++mi;
        const MatDesc& d = args.descs[mi];
        int i0, j0;
        ew_tile_origin(d, t - args.prefix[mi], i0, j0);
        float x[EW_PASSES][EW_GROUP];
#pragma unroll
        for (int p = 0; p < EW_PASSES; ++p) {
            const size_t idx = static_cast<size_t>(i0 + ew_row(p)) * d.np + (j0 + jl);
            if (sizeof(T) == 2) {   // X = hi + lo (exact in fp32)
                float h[EW_GROUP];
                load8<uint16_t>(d.xop[args.fin], idx, h);
#pragma unroll
                for (int e = 0; e < EW_GROUP; ++e) {
                    const uint16_t l = G(d.xlo)[lo_offset(i0 + ew_row(p), j0 + jl + e, d.np)];
                    x[p][e] = h[e] + __uint_as_float(static_cast<uint32_t>(l) << 16);
                }
            } else {
                load8<float>(d.x32[args.fin], idx, x[p]);
            }
        }
        // with no Newton-Schulz step the output is the normalized input
        const float oscale = args.ns_zero ? G(d.scal)[0] : 1.0f;
        const float coef = d.apply_coef * oscale;
        if (!d.tall) {
#pragma unroll
            for (int p = 0; p < EW_PASSES; ++p) apply_group<T, NS_ONLY>(d, coef, oscale, i0 + ew_row(p), j0 + jl, x[p]);
        } else {
#pragma unroll
            for (int p = 0; p < EW_PASSES; ++p)
#pragma unroll
                for (int e = 0; e < EW_GROUP; ++e) tile[ew_row(p)][jl + e] = x[p][e];
            lds_barrier();
            // caller row j0 + r holds NS column j0 + r: columns i0 + jl + e are NS rows
#pragma unroll
            for (int p = 0; p < EW_PASSES; ++p) {
                float o[EW_GROUP];
#pragma unroll
                for (int e = 0; e < EW_GROUP; ++e) o[e] = tile[jl + e][ew_row(p)];
                apply_group<T, NS_ONLY>(d, coef, oscale, j0 + ew_row(p), i0 + jl, o);
            }
            lds_barrier();   // the tile is reused; the stores stay in flight
        }
    }
}

}  // namespace

hipError_t launch_momentum_norm(int dtype, bool ns_only, const EwArgs& args, int grid, hipStream_t s) {
    if (dtype == DT_BF16) {
        if (ns_only) hipLaunchKernelGGL((momentum_norm_kernel<uint16_t, true>), dim3(grid), dim3(EW_THREADS), 0, s, args);
        else hipLaunchKernelGGL((momentum_norm_kernel<uint16_t, false>), dim3(grid), dim3(EW_THREADS), 0, s, args);
    } else {
        if (ns_only) hipLaunchKernelGGL((momentum_norm_kernel<float, true>), dim3(grid), dim3(EW_THREADS), 0, s, args);
        else hipLaunchKernelGGL((momentum_norm_kernel<float, false>), dim3(grid), dim3(EW_THREADS), 0, s, args);
    }
    return hipGetLastError();
}

hipError_t launch_norm_finalize(const MatDesc* descs, const double* partials, int nmat, float eps, hipStream_t s) {
    hipLaunchKernelGGL(norm_finalize_kernel, dim3(nmat), dim3(256), 0, s, descs, partials, eps);
    return hipGetLastError();
}

hipError_t launch_rescale(int dtype, const EwArgs& args, int grid, hipStream_t s) {
    if (dtype == DT_BF16) hipLaunchKernelGGL((rescale_kernel<uint16_t>), dim3(grid), dim3(EW_THREADS), 0, s, args);
    else hipLaunchKernelGGL((rescale_kernel<float>), dim3(grid), dim3(EW_THREADS), 0, s, args);
    return hipGetLastError();
}

hipError_t launch_apply(int dtype, bool ns_only, const EwArgs& args, int grid, hipStream_t s) {
    if (dtype == DT_BF16) {
        if (ns_only) hipLaunchKernelGGL((apply_kernel<uint16_t, true>), dim3(grid), dim3(EW_THREADS), 0, s, args);
        else hipLaunchKernelGGL((apply_kernel<uint16_t, false>), dim3(grid), dim3(EW_THREADS), 0, s, args);
    } else {
        if (ns_only) hipLaunchKernelGGL((apply_kernel<float, true>), dim3(grid), dim3(EW_THREADS), 0, s, args);
        else hipLaunchKernelGGL((apply_kernel<float, false>), dim3(grid), dim3(EW_THREADS), 0, s, args);
    }
    return hipGetLastError();
}

}  // namespace muon
