// Grouped AdamW step for gfx950: one launch covers every tensor of the call.
//
// Method ([Muon优化器] linsight.cn/f25d614e.html, section "AdamW的问题";
// decoupled decay per [DeepSeek V4 summary], section "Adam优化器的机制与AdamW的
// 改进", applied before the step as in [Muon在Stiefel流形上的精确闭式更新解析],
// section 4.3):
//   m' = beta1 m + (1 - beta1) g,  v' = beta2 v + (1 - beta2) g^2
//   p' = (1 - lr wd) p - (lr / (1 - beta1^t)) m' / (sqrt(v') / sqrt(1 - beta2^t) + eps)
// The per-call scalars are formed on the host in fp64; the arithmetic here is
// fp32 and p' is rounded once to the parameter dtype.
//
// HBM-bound: per element it reads p, g (parameter dtype) and m, v (fp32) and
// writes p, m, v.  The work is split into ADAMW_CHUNK-element chunks
// (concatenated over tensors, per-tensor prefix sums); each block walks chunks
// with a grid stride, each thread handles 4 quads of 4 consecutive elements,
// with 8- or 16-byte accesses when the tensor is aligned for them.  In a whole,
// aligned chunk all of a thread's loads are issued before its first store.
#include "muon_internal.h"

namespace muon {

namespace {

template <typename T> struct PElem;
template <> struct PElem<float> {
    static __device__ inline float4 load4(const void* p, int64_t i) { return ld_f4(static_cast<const float*>(p) + i); }
    static __device__ inline void store4(void* p, int64_t i, float4 v) { st_f4(static_cast<float*>(p) + i, v); }
    static __device__ inline float load(const void* p, int64_t i) { return G(static_cast<const float*>(p))[i]; }
    static __device__ inline void store(void* p, int64_t i, float v) { G(static_cast<float*>(p))[i] = v; }
};
template <> struct PElem<uint16_t> {
    static __device__ inline float4 load4(const void* p, int64_t i) {
        const u32x2_t q = ld_u2(static_cast<const uint16_t*>(p) + i);
        return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u),
                           __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xffff0000u));
    }
    static __device__ inline void store4(void* p, int64_t i, float4 v) {
        st_u2(static_cast<uint16_t*>(p) + i, u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)});
    }
    static __device__ inline float load(const void* p, int64_t i) {
        return bf16_to_f32(G(static_cast<const uint16_t*>(p))[i]);
    }
    static __device__ inline void store(void* p, int64_t i, float v) { G(static_cast<uint16_t*>(p))[i] = f32_to_bf16(v); }
};

struct AdamWMath {
    float b1, b2, omb1, omb2, eps, decay, step_size, isb2;
    // one element: updates m and v in place, returns p'
    __device__ __forceinline__ float operator()(float p, float g, float& m, float& v) const {
        m = fmaf(b1, m, omb1 * g);
        v = fmaf(b2, v, omb2 * (g * g));
        const float denom = fmaf(__builtin_sqrtf(v), isb2, eps);
        return fmaf(decay, p, -(step_size * m / denom));
    }
};

template <typename T>
__global__ __launch_bounds__(ADAMW_THREADS) void adamw_kernel(AdamWArgs args) {
    const AdamWMath f{args.beta1, args.beta2, args.one_m_beta1, args.one_m_beta2, args.eps, args.decay,
                      args.step_size, args.inv_sqrt_bc2};
    const int tid = threadIdx.x;
    for (int c = blockIdx.x; c < args.total; c += gridDim.x) {
        const int ti = find_matrix(args.prefix, args.n, c);
        const AdamWDesc& d = args.descs[ti];
        const int64_t base = static_cast<int64_t>(c - args.prefix[ti]) * ADAMW_CHUNK;
        void* __restrict__ pp = d.p;
        const void* __restrict__ gp = d.g;
        float* __restrict__ mp = d.m;
        float* __restrict__ vp = d.v;
        const int64_t numel = d.numel;
        constexpr int QUADS = ADAMW_CHUNK / (4 * ADAMW_THREADS);
        if (d.vec && base + ADAMW_CHUNK <= numel) {
            // whole chunk: every load of the thread's quads is issued before any store
            float4 p[QUADS], g[QUADS], m[QUADS], v[QUADS];
#pragma unroll
            for (int k = 0; k < QUADS; ++k) {
                const int64_t e0 = base + 4 * (tid + k * ADAMW_THREADS);
                p[k] = PElem<T>::load4(pp, e0);
                g[k] = PElem<T>::load4(gp, e0);
                m[k] = ld_f4(mp + e0);
                v[k] = ld_f4(vp + e0);
            }
#pragma unroll
            for (int k = 0; k < QUADS; ++k) {
                const int64_t e0 = base + 4 * (tid + k * ADAMW_THREADS);
                float4 o;
                o.x = f(p[k].x, g[k].x, m[k].x, v[k].x);
                o.y = f(p[k].y, g[k].y, m[k].y, v[k].y);
                o.z = f(p[k].z, g[k].z, m[k].z, v[k].z);
                o.w = f(p[k].w, g[k].w, m[k].w, v[k].w);
                PElem<T>::store4(pp, e0, o);
                st_f4(mp + e0, m[k]);
                st_f4(vp + e0, v[k]);
            }
            continue;
        }
#pragma unroll
        for (int k = 0; k < QUADS; ++k) {
            const int64_t e0 = base + 4 * (tid + k * ADAMW_THREADS);
            if (e0 >= numel) break;
            if (d.vec && e0 + 3 < numel) {
                const float4 p = PElem<T>::load4(pp, e0), g = PElem<T>::load4(gp, e0);
                float4 m = ld_f4(mp + e0), v = ld_f4(vp + e0);
                float4 o;
                o.x = f(p.x, g.x, m.x, v.x);
                o.y = f(p.y, g.y, m.y, v.y);
                o.z = f(p.z, g.z, m.z, v.z);
                o.w = f(p.w, g.w, m.w, v.w);
                PElem<T>::store4(pp, e0, o);
                st_f4(mp + e0, m);
                st_f4(vp + e0, v);
            } else {
                const int cnt = static_cast<int>(min<int64_t>(4, numel - e0));
                for (int e = 0; e < cnt; ++e) {
                    float m = G(mp)[e0 + e], v = G(vp)[e0 + e];
                    const float o = f(PElem<T>::load(pp, e0 + e), PElem<T>::load(gp, e0 + e), m, v);
                    PElem<T>::store(pp, e0 + e, o);
                    G(mp)[e0 + e] = m;
                    G(vp)[e0 + e] = v;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_adamw(int dtype, const AdamWArgs& args, int grid, hipStream_t s) {
    if (args.total <= 0) return hipSuccess;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(adamw_kernel<uint16_t>, dim3(grid), dim3(ADAMW_THREADS), 0, s, args);
    else
        hipLaunchKernelGGL(adamw_kernel<float>, dim3(grid), dim3(ADAMW_THREADS), 0, s, args);
    return hipGetLastError();
}

}  // namespace muon
