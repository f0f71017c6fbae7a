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

// Store 4 consecutive values of the operand dtype (8-byte or 16-byte store).
template <typename T> __device__ inline void store4(void* base, size_t idx, float v0, float v1, float v2, float v3);
template <> __device__ inline void store4<float>(void* base, size_t idx, float v0, float v1, float v2, float v3) {
    st_f4(static_cast<float*>(base) + idx, make_float4(v0, v1, v2, v3));
}
template <> __device__ inline void store4<uint16_t>(void* base, size_t idx, float v0, float v1, float v2, float v3) {
    const u32x2_t p = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
    st_u2(static_cast<uint16_t*>(base) + idx, p);
}

// 4 consecutive elements of the caller's dtype as fp32 (8-byte or 16-byte load).
template <typename T> __device__ inline float4 load4(const void* base, size_t idx);
template <> __device__ inline float4 load4<float>(const void* base, size_t idx) {
    return ld_f4(static_cast<const float*>(base) + idx);
}
template <> __device__ inline float4 load4<uint16_t>(const void* base, size_t idx) {
    const u32x2_t q = ld_u2(static_cast<const uint16_t*>(base) + idx);
    return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u),
                       __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xffff0000u));
}
__device__ inline float f4at(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// Deterministic block sum (fixed shuffle pattern, fixed wave order).
__device__ inline float block_sum_256(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float total = ((red[0] + red[1]) + (red[2] + red[3]));
    __syncthreads();
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
//   user-frame load (coalesced) -> fp32 M' (state store) -> U into LDS in the
//   NS frame -> rows of the iterate (fp32, or the bf16 pair hi + lo whose hi
//   is the MFMA operand), coalesced, with the sum of squares taken in NS-frame
//   order so the result does not depend on the caller's orientation.
// ----------------------------------------------------------------------------
template <typename T, bool NS_ONLY>
__global__ __launch_bounds__(EW_THREADS) void momentum_norm_kernel(EwArgs args) {
    __shared__ float tile[EW_TILE][EW_TILE + 1];
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * args.tiles_per_block;
    const int t1 = min(args.total, t0 + args.tiles_per_block);
    if (t0 >= t1) return;
    int mi = find_matrix(args.prefix, args.nmat, t0);
    const float beta = args.beta;

    for (int t = t0; t < t1; ++t) {
        while (t >= args.prefix[mi + 1]) ++mi;
        const MatDesc& d = args.descs[mi];
        int i0, j0;
        ew_tile_origin(d, t - args.prefix[mi], i0, j0);
        const int ur0 = d.tall ? j0 : i0;   // user-frame block origin
        const int uc0 = d.tall ? i0 : j0;
        const int rows = d.rows, cols = d.cols;

        // ---- load phase: 4 consecutive user columns per thread, 16 threads per 64-element row
#pragma unroll
        for (int p = 0; p < EW_TILE * EW_TILE / (4 * EW_THREADS); ++p) {
            const int q = tid + EW_THREADS * p;
            const int lr = q >> 4, lc = (q & 15) * 4;
            const int ur = ur0 + lr, uc = uc0 + lc;
            float u[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (ur < rows && uc < cols) {
                const size_t idx = static_cast<size_t>(ur) * cols + uc;
                if (d.uvec) {   // uc + 3 < cols: cols and uc are multiples of 4
                    const float4 g = load4<T>(d.g, idx);
                    if (NS_ONLY) {
                        u[0] = g.x; u[1] = g.y; u[2] = g.z; u[3] = g.w;
                    } else {
                        const float4 m = load4<T>(d.mom, idx);
                        float mn[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            mn[e] = fmaf(beta, f4at(m, e), f4at(g, e));
                            u[e] = args.nesterov ? fmaf(beta, mn[e], f4at(g, e)) : mn[e];
                        }
                        store4<T>(d.mom, idx, mn[0], mn[1], mn[2], mn[3]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (uc + e >= cols) break;
                        const float g = Elem<T>::load(d.g, idx + e);
                        if (NS_ONLY) {
                            u[e] = g;
                        } else {
                            const float m = Elem<T>::load(d.mom, idx + e);
                            const float mn = fmaf(beta, m, g);
                            Elem<T>::store(d.mom, idx + e, mn);
                            u[e] = args.nesterov ? fmaf(beta, mn, g) : mn;
                        }
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (d.tall) tile[lc + e][lr] = u[e]; else tile[lr][lc + e] = u[e];
            }
        }
        __syncthreads();

        // ---- NS-frame rows: X32 (and the bf16 operand copy)
        float sq = 0.0f;
        {
            const int jl = (tid & 15) * 4;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int il = (tid >> 4) + 16 * p;
                const float v0 = tile[il][jl], v1 = tile[il][jl + 1];
                const float v2 = tile[il][jl + 2], v3 = tile[il][jl + 3];
                sq = fmaf(v0, v0, sq); sq = fmaf(v1, v1, sq);
                sq = fmaf(v2, v2, sq); sq = fmaf(v3, v3, sq);
                const size_t idx = static_cast<size_t>(i0 + il) * d.np + (j0 + jl);
                if (sizeof(T) == 2) {
                    // the iterate as the pair hi + lo: hi = bf16(U), lo = bf16(U - hi)
                    const uint32_t h01 = pack_bf16x2(v0, v1), h23 = pack_bf16x2(v2, v3);
                    const float r0 = v0 - __uint_as_float(h01 << 16), r1 = v1 - __uint_as_float(h01 & 0xffff0000u);
                    const float r2 = v2 - __uint_as_float(h23 << 16), r3 = v3 - __uint_as_float(h23 & 0xffff0000u);
                    st_u2(static_cast<uint16_t*>(d.xop[0]) + idx, u32x2_t{h01, h23});
                    store4<T>(d.xlo, idx, r0, r1, r2, r3);
                } else {
                    st_f4(d.x32[0] + idx, make_float4(v0, v1, v2, v3));
                }
            }
        }
        const float total = block_sum_256(sq, red);   // also orders LDS reuse
        if (tid == 0) G(args.partials)[t] = total;
    }
}

// ----------------------------------------------------------------------------
// Norm finalize: one block per matrix sums its tile partials in a fixed order
// (fp64) and stores s = 1 / (||U||_F + eps).
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void norm_finalize_kernel(const MatDesc* descs, const float* partials,
                                                            float eps) {
    __shared__ double red[256];
    const MatDesc& d = descs[blockIdx.x];
    double acc = 0.0;
    for (int i = threadIdx.x; i < d.ew_tiles; i += 256) acc += static_cast<double>(partials[d.ew_tile0 + i]);
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double nrm = sqrt(red[0]);
        G(d.scal)[0] = static_cast<float>(1.0 / (nrm + static_cast<double>(eps)));
        G(d.scal)[1] = static_cast<float>(nrm);
    }
}

// ----------------------------------------------------------------------------
// Apply: W' = (1 - lr*wd) W - lr*s_rule*X  (muon_step), or out = X (muon_ns).
// X is read in the NS frame and written back in the caller's frame.
// ----------------------------------------------------------------------------
template <typename T, bool NS_ONLY>
__global__ __launch_bounds__(EW_THREADS) void apply_kernel(EwArgs args) {
    __shared__ float tile[EW_TILE][EW_TILE + 1];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * args.tiles_per_block;
    const int t1 = min(args.total, t0 + args.tiles_per_block);
    if (t0 >= t1) return;
    int mi = find_matrix(args.prefix, args.nmat, t0);

    for (int t = t0; t < t1; ++t) {
        while (t >= args.prefix[mi + 1]) ++mi;
        const MatDesc& d = args.descs[mi];
        int i0, j0;
        ew_tile_origin(d, t - args.prefix[mi], i0, j0);
        {
            const int jl = (tid & 15) * 4;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int il = (tid >> 4) + 16 * p;
                const size_t idx = static_cast<size_t>(i0 + il) * d.np + (j0 + jl);
                float4 v;
                if (sizeof(T) == 2) {   // X = hi + lo (exact in fp32)
                    const u32x2_t h = ld_u2(static_cast<const uint16_t*>(d.xop[args.fin]) + idx);
                    const u32x2_t l = ld_u2(d.xlo + idx);
                    v = make_float4(__uint_as_float(h.x << 16) + __uint_as_float(l.x << 16),
                                    __uint_as_float(h.x & 0xffff0000u) + __uint_as_float(l.x & 0xffff0000u),
                                    __uint_as_float(h.y << 16) + __uint_as_float(l.y << 16),
                                    __uint_as_float(h.y & 0xffff0000u) + __uint_as_float(l.y & 0xffff0000u));
                } else {
                    v = ld_f4(d.x32[args.fin] + idx);
                }
                tile[il][jl] = v.x; tile[il][jl + 1] = v.y; tile[il][jl + 2] = v.z; tile[il][jl + 3] = v.w;
            }
        }
        __syncthreads();
        // with no Newton-Schulz step the output is the normalized input
        const float oscale = args.ns_zero ? G(d.scal)[0] : 1.0f;
        const int ur0 = d.tall ? j0 : i0;
        const int uc0 = d.tall ? i0 : j0;
        const float coef = d.apply_coef * oscale;
        const float decay = d.decay;
        // one element per thread and pass: a wave writes one 64-element user row
#pragma unroll 4
        for (int p = 0; p < EW_TILE * EW_TILE / EW_THREADS; ++p) {
            const int q = tid + EW_THREADS * p;
            const int lr = q >> 6, lc = q & 63;
            const int ur = ur0 + lr, uc = uc0 + lc;
            if (ur < d.rows && uc < d.cols) {
                const float o = d.tall ? tile[lc][lr] : tile[lr][lc];
                const size_t idx = static_cast<size_t>(ur) * d.cols + uc;
                if (NS_ONLY) {
                    G(d.out)[idx] = o * oscale;
                } else {
                    const float w = Elem<T>::load(d.w, idx);
                    Elem<T>::store(d.w, idx, fmaf(-coef, o, decay * w));
                }
            }
        }
        __syncthreads();
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

hipError_t launch_norm_finalize(const MatDesc* descs, const float* partials, int nmat, float eps, hipStream_t s) {
    hipLaunchKernelGGL(norm_finalize_kernel, dim3(nmat), dim3(256), 0, s, descs, partials, eps);
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
