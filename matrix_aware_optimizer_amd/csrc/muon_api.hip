// Host side of the C ABI in include/muon.h: argument validation, the
// grouped-batch plan (orientation, padding, tile prefix sums, workspace
// layout), descriptor upload and the launch sequence
//     momentum+norm -> norm finalize -> T x (Gram -> polynomial -> update) -> apply
// on the caller's stream.  No device memory is allocated here: everything
// lives in the caller's workspace.  Descriptor tables are staged through a
// small ring of pinned host buffers so the upload is truly asynchronous.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "muon.h"
#include "muon_internal.h"

using namespace muon;

namespace {

thread_local std::string g_last_error;

muon_status fail(muon_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

muon_status hip_fail(hipError_t e, const char* what) {
    return fail(MUON_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Validation
// ---------------------------------------------------------------------------

muon_status check_hparams(const muon_hparams* hp, bool need_step_scalars) {
    if (!hp) return fail(MUON_ERR_INVALID_ARG, "hp is NULL");
    if (hp->dtype != MUON_F32 && hp->dtype != MUON_BF16)
        return fail(MUON_ERR_INVALID_ARG, "unknown dtype %d", hp->dtype);
    if (hp->ns_steps < 0 || hp->ns_steps > MUON_MAX_NS_STEPS)
        return fail(MUON_ERR_INVALID_ARG, "ns_steps %d outside [0, %d]", hp->ns_steps, MUON_MAX_NS_STEPS);
    if (hp->ns_steps > 0 && !hp->schedule) return fail(MUON_ERR_INVALID_ARG, "schedule is NULL");
    for (int k = 0; k < hp->ns_steps; ++k) {
        const muon_ns_coeffs& c = hp->schedule[k];
        if (!std::isfinite(c.a) || !std::isfinite(c.b) || !std::isfinite(c.c))
            return fail(MUON_ERR_INVALID_ARG, "schedule[%d] is not finite", k);
    }
    if (!std::isfinite(hp->eps) || hp->eps < 0.0f) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (need_step_scalars) {
        if (!std::isfinite(hp->lr)) return fail(MUON_ERR_INVALID_ARG, "lr is not finite");
        if (!std::isfinite(hp->beta)) return fail(MUON_ERR_INVALID_ARG, "beta is not finite");
        if (!std::isfinite(hp->weight_decay)) return fail(MUON_ERR_INVALID_ARG, "weight_decay is not finite");
        if (hp->scale_rule < MUON_SCALE_NAIVE || hp->scale_rule > MUON_SCALE_MOONLIGHT)
            return fail(MUON_ERR_INVALID_ARG, "unknown scale_rule %d", hp->scale_rule);
        if (hp->flags & ~MUON_FLAG_NESTEROV) return fail(MUON_ERR_INVALID_ARG, "unknown flags 0x%x", hp->flags);
    }
    return MUON_OK;
}

struct Interval {
    uintptr_t lo, hi;
    bool readonly;
    int who;
};

muon_status check_overlaps(std::vector<Interval>& iv) {
    std::sort(iv.begin(), iv.end(), [](const Interval& a, const Interval& b) { return a.lo < b.lo; });
    // sweep: keep the furthest-reaching earlier interval of each kind
    uintptr_t max_hi_rw = 0, max_hi_any = 0;
    int who_rw = -1, who_any = -1;
    for (const Interval& x : iv) {
        if (x.lo < max_hi_rw) return fail(MUON_ERR_INVALID_ARG, "buffers of matrices %d and %d overlap", who_rw, x.who);
        if (!x.readonly && x.lo < max_hi_any)
            return fail(MUON_ERR_INVALID_ARG, "buffers of matrices %d and %d overlap", who_any, x.who);
        if (!x.readonly && x.hi > max_hi_rw) { max_hi_rw = x.hi; who_rw = x.who; }
        if (x.hi > max_hi_any) { max_hi_any = x.hi; who_any = x.who; }
    }
    return MUON_OK;
}

// ---------------------------------------------------------------------------
// Plan and workspace layout
// ---------------------------------------------------------------------------

struct Item {            // one active matrix, before sorting
    int user_index;
    const void* g;
    void* w;
    void* mom;
    float* out;
    int64_t rows, cols;
};

struct Plan {
    std::vector<MatDesc> descs;
    std::vector<int32_t> ew_prefix, sym_prefix, upd_prefix;
    std::vector<TileRun> sym_runs, upd_runs;
    size_t off_descs = 0, off_prefix = 0, off_runs = 0, off_scal = 0, off_partials = 0, header_bytes = 0, total_bytes = 0;
    int64_t total_ew = 0, total_sym = 0, total_upd = 0;
};

float scale_rule_value(int rule, int64_t rows, int64_t cols) {
    const double d_out = static_cast<double>(rows), d_in = static_cast<double>(cols);
    switch (rule) {
        case MUON_SCALE_KELLER_JORDAN: return static_cast<float>(std::sqrt(std::max(1.0, d_out / d_in)));
        case MUON_SCALE_MUP: return static_cast<float>(std::sqrt(d_out / d_in));
        case MUON_SCALE_MOONLIGHT: return static_cast<float>(0.2 * std::sqrt(std::max(d_out, d_in)));
        default: return 1.0f;
    }
}

// Builds descriptors with workspace offsets (pointers are offsets until
// `rebase` adds the workspace base).
muon_status build_plan(std::vector<Item>& items, const muon_hparams* hp, bool ns_only, Plan& pl) {
    const int dtype = hp->dtype;
    const size_t es = dtype == MUON_BF16 ? 2 : 4;
    const int64_t pad = dtype == MUON_BF16 ? GEMM_TILE_BF16 : GEMM_TILE_F32;
    const int nmat = static_cast<int>(items.size());

    struct Shape { int64_t m, n, mp, np; };
    std::vector<Shape> sh(nmat);
    for (int i = 0; i < nmat; ++i) {
        Shape& s = sh[i];
        s.m = std::min(items[i].rows, items[i].cols);
        s.n = std::max(items[i].rows, items[i].cols);
        s.mp = round_up(s.m, pad);
        s.np = round_up(s.n, pad);
    }
    // largest Newton-Schulz work first (stable for equal shapes)
    std::vector<int> order(nmat);
    for (int i = 0; i < nmat; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
        const double ca = static_cast<double>(sh[a].mp) * sh[a].mp * sh[a].np;
        const double cb = static_cast<double>(sh[b].mp) * sh[b].mp * sh[b].np;
        return ca > cb;
    });

    pl.descs.assign(nmat, MatDesc{});
    pl.ew_prefix.assign(nmat + 1, 0);
    pl.sym_prefix.assign(nmat + 1, 0);
    pl.upd_prefix.assign(nmat + 1, 0);

    size_t off = 0;
    pl.off_descs = off;
    off = align_up(off + sizeof(MatDesc) * nmat, ALIGN);
    pl.off_prefix = off;
    off = align_up(off + sizeof(int32_t) * (nmat + 1), ALIGN);
    pl.off_runs = off;                           // sym runs, then upd runs: at most nmat each
    off = align_up(off + sizeof(TileRun) * 2 * nmat, ALIGN);
    pl.header_bytes = off;                       // uploaded from the host
    pl.off_scal = off;
    off = align_up(off + sizeof(float) * NS_SCAL * nmat, ALIGN);

    int64_t ew = 0, sym = 0, upd = 0;
    for (int k = 0; k < nmat; ++k) {
        const Item& it = items[order[k]];
        const Shape& s = sh[order[k]];
        MatDesc& d = pl.descs[k];
        d.w = it.w;
        d.g = it.g;
        d.mom = it.mom;
        d.out = it.out;
        d.rows = static_cast<int32_t>(it.rows);
        d.cols = static_cast<int32_t>(it.cols);
        d.m = static_cast<int32_t>(s.m);
        d.n = static_cast<int32_t>(s.n);
        d.mp = static_cast<int32_t>(s.mp);
        d.np = static_cast<int32_t>(s.np);
        d.tall = it.rows > it.cols ? 1 : 0;
        {
            // 8-element groups with 16-byte accesses
            auto ok = [](const void* ptr) { return ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
            d.uvec = (it.cols % 8 == 0 && ok(it.w) && ok(it.g) && ok(it.mom) && ok(it.out)) ? 1 : 0;
        }
        // the first step can read hi straight from the caller's buffer when that buffer
        // holds bf16(U) in the NS frame with the padded pitch and no padding rows
        d.hi_alias = (dtype == MUON_BF16 && hp->ns_steps > 0 && !(hp->flags & MUON_FLAG_NESTEROV && !ns_only) &&
                      !d.tall && d.uvec && it.rows % pad == 0 && it.cols % pad == 0) ? 1 : 0;
        d.hi0 = d.hi_alias ? (ns_only ? it.g : static_cast<const void*>(it.mom)) : nullptr;
        const int64_t ewt = (s.mp / EW_TILE) * (s.np / EW_TILE);
        const int64_t tm = s.mp / pad, tn = s.np / pad;
        const int64_t symt = tm * (tm + 1) / 2, updt = tm * tn;
        d.ew_tile0 = static_cast<int32_t>(ew);
        d.ew_tiles = static_cast<int32_t>(ewt);
        d.sym_tile0 = static_cast<int32_t>(sym);
        d.sym_tiles = static_cast<int32_t>(symt);
        d.upd_tile0 = static_cast<int32_t>(upd);
        d.upd_tiles = static_cast<int32_t>(updt);
        ew += ewt;
        sym += symt;
        upd += updt;
        if (ew > INT32_MAX || sym > INT32_MAX || upd > INT32_MAX)
            return fail(MUON_ERR_UNSUPPORTED, "too many tiles in one call (split the matrix list)");
        pl.ew_prefix[k + 1] = static_cast<int32_t>(ew);
        pl.sym_prefix[k + 1] = static_cast<int32_t>(sym);
        pl.upd_prefix[k + 1] = static_cast<int32_t>(upd);
        if (ns_only) {
            d.apply_coef = 0.0f;
            d.decay = 1.0f;
        } else {
            const double lr = hp->lr, wd = hp->weight_decay;
            d.apply_coef = static_cast<float>(lr * static_cast<double>(scale_rule_value(hp->scale_rule, it.rows, it.cols)));
            d.decay = static_cast<float>(1.0 - lr * wd);
        }
        d.scal = reinterpret_cast<float*>(pl.off_scal + sizeof(float) * NS_SCAL * k);
    }
    pl.total_ew = ew;
    pl.total_sym = sym;
    pl.total_upd = upd;
    // consecutive matrices with equal tile counts form one run
    auto make_runs = [&](const std::vector<int32_t>& prefix, std::vector<TileRun>& runs) {
        runs.clear();
        for (int k = 0; k < nmat; ++k) {
            const int32_t tiles = prefix[k + 1] - prefix[k];
            if (runs.empty() || runs.back().tiles != tiles) runs.push_back(TileRun{prefix[k], k, tiles});
        }
    };
    make_runs(pl.sym_prefix, pl.sym_runs);
    make_runs(pl.upd_prefix, pl.upd_runs);
    pl.off_partials = off;
    off = align_up(off + sizeof(double) * ew, ALIGN);

    for (int k = 0; k < nmat; ++k) {
        MatDesc& d = pl.descs[k];
        const size_t mn = static_cast<size_t>(d.mp) * d.np, mm = static_cast<size_t>(d.mp) * d.mp;
        // bf16: the iterate as hi (two ping-pong operand copies) + lo (in place);
        // fp32: two iterates that are their own operands
        if (dtype == MUON_BF16) {
            d.x32[0] = d.x32[1] = nullptr;
            for (int p = 0; p < 2; ++p) {
                d.xop[p] = reinterpret_cast<void*>(off);
                off = align_up(off + mn * 2, ALIGN);
            }
            // xop[0] stays in the layout when hi is aliased: the rescale kernel may need it
            d.xlo = reinterpret_cast<uint16_t*>(off);
            off = align_up(off + mn * 2, ALIGN);
        } else {
            for (int p = 0; p < 2; ++p) {
                d.x32[p] = reinterpret_cast<float*>(off);
                off = align_up(off + mn * 4, ALIGN);
                d.xop[p] = d.x32[p];
            }
            d.xlo = nullptr;
        }
        d.amat = reinterpret_cast<void*>(off);
        off = align_up(off + mm * es, ALIGN);
        d.bmat = reinterpret_cast<void*>(off);
        off = align_up(off + mm * es, ALIGN);
    }
    pl.total_bytes = off;
    return MUON_OK;
}

void rebase(Plan& pl, char* base) {
    auto fix = [base](auto*& p) {
        using P = std::remove_reference_t<decltype(p)>;
        p = reinterpret_cast<P>(base + reinterpret_cast<uintptr_t>(p));
    };
    for (MatDesc& d : pl.descs) {
        if (d.xlo) {   // bf16
            fix(d.xop[0]);
            fix(d.xop[1]);
            fix(d.xlo);
            if (!d.hi_alias) d.hi0 = d.xop[0];
        } else {
            fix(d.x32[0]);
            fix(d.x32[1]);
            d.xop[0] = d.x32[0];
            d.xop[1] = d.x32[1];
            d.hi0 = d.xop[0];
        }
        fix(d.amat);
        fix(d.bmat);
        fix(d.scal);
    }
}

// ---------------------------------------------------------------------------
// Device checks, pinned staging, profiling
// ---------------------------------------------------------------------------

std::mutex g_mu;

muon_status check_device(int* dev_out, int* cu_count) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    static std::vector<int> ok_cache;   // -1 unknown, 0 no, 1 yes
    static std::vector<int> cus;
    std::lock_guard<std::mutex> lk(g_mu);
    if (static_cast<int>(ok_cache.size()) <= dev) { ok_cache.resize(dev + 1, -1); cus.resize(dev + 1, 0); }
    if (ok_cache[dev] < 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        ok_cache[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
        cus[dev] = prop.multiProcessorCount;
        if (!ok_cache[dev]) {
            g_last_error = std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950";
        }
    }
    if (!ok_cache[dev]) return fail(MUON_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    *dev_out = dev;
    *cu_count = cus[dev];
    return MUON_OK;
}

struct PinnedSlot {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
};
struct PinnedRing {
    PinnedSlot slot[4];
    int next = 0;
};
std::vector<PinnedRing> g_rings;

// Copy `bytes` of host data to device `dst` asynchronously on `s`.
muon_status upload(int dev, void* dst, const void* src, size_t bytes, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (static_cast<int>(g_rings.size()) <= dev) g_rings.resize(dev + 1);
    PinnedRing& ring = g_rings[dev];
    PinnedSlot& sl = ring.slot[ring.next];
    ring.next = (ring.next + 1) % 4;
    hipError_t e;
    if (sl.pending) {
        e = hipEventSynchronize(sl.ev);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(staging)");
        sl.pending = false;
    }
    if (!sl.ev) {
        e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
    if (sl.cap < bytes) {
        if (sl.host) (void)hipHostFree(sl.host);
        sl.host = nullptr;
        sl.cap = 0;
        const size_t cap = std::max<size_t>(align_up(bytes, 65536), 65536);
        e = hipHostMalloc(&sl.host, cap, hipHostMallocDefault);
        if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(staging)");
        sl.cap = cap;
    }
    std::memcpy(sl.host, src, bytes);
    e = hipMemcpyAsync(dst, sl.host, bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(descriptors)");
    e = hipEventRecord(sl.ev, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(staging)");
    sl.pending = true;
    return MUON_OK;
}

struct ProfRec { int cls; hipEvent_t a, b; };
struct ProfState {
    bool on = false;
    std::vector<ProfRec> recs;
    std::vector<hipEvent_t> pool;
} g_prof;

hipEvent_t prof_event() {
    if (!g_prof.pool.empty()) {
        hipEvent_t e = g_prof.pool.back();
        g_prof.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <typename F>
muon_status timed_launch(int cls, hipStream_t s, const char* what, F launch) {
    hipEvent_t a = nullptr, b = nullptr;
    bool prof;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        prof = g_prof.on;
        if (prof) { a = prof_event(); b = prof_event(); }
    }
    if (prof && a) (void)hipEventRecord(a, s);
    hipError_t e = launch();
    if (e != hipSuccess) return hip_fail(e, what);
    if (prof && b) {
        (void)hipEventRecord(b, s);
        std::lock_guard<std::mutex> lk(g_mu);
        g_prof.recs.push_back({cls, a, b});
    }
    return MUON_OK;
}

// ---------------------------------------------------------------------------
// Workspace of muon_step_noalloc: a file-scope device array, one copy per GPU,
// held until the process ends.  In host code the name `scratch` is a host-side
// stand-in, not the device memory: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MUON_NOALLOC_SCRATCH_BYTES];
std::vector<char*> g_scratch_ptr;   // per device; nullptr until set up

muon_status scratch_address(int dev, char** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (static_cast<int>(g_scratch_ptr.size()) <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MUON_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    *out = g_scratch_ptr[dev];
    return MUON_OK;
}

// The descriptor header written by kernels whose arguments carry it, 3 KB per
// launch: no pinned staging buffer (and so no allocation) is needed, and the
// bytes are copied at launch time, so nothing on the host must outlive the call.
constexpr int HDR_CHUNK_WORDS = 768;
struct HeaderChunk {
    uint32_t word0;    // first 4-byte word of the destination
    uint32_t nwords;
    uint32_t w[HDR_CHUNK_WORDS];
};

__global__ __launch_bounds__(256) void header_write_kernel(HeaderChunk c, uint32_t* dst) {
    for (uint32_t i = threadIdx.x; i < c.nwords; i += 256) dst[c.word0 + i] = c.w[i];
}

muon_status upload_by_args(void* dst, const void* src, size_t bytes, hipStream_t s) {
    if (bytes % 4) return fail(MUON_ERR_INVALID_ARG, "header of %zu bytes is not a whole number of words", bytes);
    const uint32_t* words = static_cast<const uint32_t*>(src);
    const size_t nw = bytes / 4;
    HeaderChunk c;
    for (size_t w0 = 0; w0 < nw; w0 += HDR_CHUNK_WORDS) {
        c.word0 = static_cast<uint32_t>(w0);
        c.nwords = static_cast<uint32_t>(std::min<size_t>(HDR_CHUNK_WORDS, nw - w0));
        std::memcpy(c.w, words + w0, 4 * c.nwords);
        hipLaunchKernelGGL(header_write_kernel, dim3(1), dim3(256), 0, s, c, static_cast<uint32_t*>(dst));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "header write kernel");
    }
    return MUON_OK;
}

// ---------------------------------------------------------------------------
// The launch sequence shared by muon_step and muon_ns
// ---------------------------------------------------------------------------

// header_by_args: write the descriptor header with kernel launches instead of a
// copy from the pinned staging ring (muon_step_noalloc, which allocates nothing).
muon_status run(std::vector<Item>& items, const muon_hparams* hp, bool ns_only, void* workspace,
                size_t ws_bytes, hipStream_t stream, bool header_by_args = false) {
    Plan pl;
    muon_status st = build_plan(items, hp, ns_only, pl);
    if (st != MUON_OK) return st;
    if (!workspace) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % ALIGN)
        return fail(MUON_ERR_WORKSPACE, "workspace is not %zu-byte aligned", ALIGN);
    if (ws_bytes < pl.total_bytes)
        return fail(MUON_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, pl.total_bytes);
    {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(workspace), hi = lo + pl.total_bytes;
        for (const Item& it : items) {
            const size_t es = hp->dtype == MUON_BF16 ? 2 : 4;
            const size_t bytes = static_cast<size_t>(it.rows) * it.cols;
            const void* ptrs[4] = {it.w, it.g, it.mom, it.out};
            const size_t sz[4] = {bytes * es, bytes * es, bytes * es, bytes * 4};
            for (int q = 0; q < 4; ++q) {
                const uintptr_t p = reinterpret_cast<uintptr_t>(ptrs[q]);
                if (p && p < hi && p + sz[q] > lo)
                    return fail(MUON_ERR_INVALID_ARG, "matrix %d overlaps the workspace", it.user_index);
            }
        }
    }
    int dev = 0, cu_count = 0;
    st = check_device(&dev, &cu_count);
    if (st != MUON_OK) return st;

    char* base = static_cast<char*>(workspace);
    rebase(pl, base);
    const int nmat = static_cast<int>(pl.descs.size());

    // header: descriptors, the elementwise prefix sums and the GEMM phases' tile runs
    std::vector<char> header(pl.header_bytes, 0);
    std::memcpy(header.data() + pl.off_descs, pl.descs.data(), sizeof(MatDesc) * nmat);
    std::memcpy(header.data() + pl.off_prefix, pl.ew_prefix.data(), sizeof(int32_t) * (nmat + 1));
    TileRun* runs = reinterpret_cast<TileRun*>(header.data() + pl.off_runs);
    std::memcpy(runs, pl.sym_runs.data(), sizeof(TileRun) * pl.sym_runs.size());
    std::memcpy(runs + nmat, pl.upd_runs.data(), sizeof(TileRun) * pl.upd_runs.size());
    st = header_by_args ? upload_by_args(base, header.data(), pl.header_bytes, stream)
                        : upload(dev, base, header.data(), pl.header_bytes, stream);
    if (st != MUON_OK) return st;

    const MatDesc* d_descs = reinterpret_cast<const MatDesc*>(base + pl.off_descs);
    const int32_t* d_pre = reinterpret_cast<const int32_t*>(base + pl.off_prefix);
    const TileRun* d_runs = reinterpret_cast<const TileRun*>(base + pl.off_runs);
    double* d_partials = reinterpret_cast<double*>(base + pl.off_partials);

    EwArgs ew{};
    ew.descs = d_descs;
    ew.prefix = d_pre;
    ew.partials = d_partials;
    ew.nmat = nmat;
    ew.total = static_cast<int32_t>(pl.total_ew);
    const int target_blocks = std::max(cu_count, 1) * 8;
    ew.tiles_per_block = static_cast<int32_t>(std::max<int64_t>(1, (pl.total_ew + target_blocks - 1) / target_blocks));
    ew.beta = ns_only ? 0.0f : hp->beta;
    ew.nesterov = (!ns_only && (hp->flags & MUON_FLAG_NESTEROV)) ? 1 : 0;
    ew.ns_zero = hp->ns_steps == 0 ? 1 : 0;
    ew.fin = hp->ns_steps & 1;
    const int ew_grid = static_cast<int>((pl.total_ew + ew.tiles_per_block - 1) / ew.tiles_per_block);
    const int dtype = hp->dtype;

    st = timed_launch(0, stream, "momentum/norm kernel", [&] { return launch_momentum_norm(dtype, ns_only, ew, ew_grid, stream); });
    if (st != MUON_OK) return st;
    st = timed_launch(1, stream, "norm finalize kernel", [&] { return launch_norm_finalize(d_descs, d_partials, nmat, hp->eps, stream); });
    if (st != MUON_OK) return st;
    // shifts the stored iterate of the (rare) matrices whose norm is outside the plain range;
    // its workgroups leave at once for every other matrix
    st = timed_launch(1, stream, "rescale kernel", [&] { return launch_rescale(dtype, ew, ew_grid, stream); });
    if (st != MUON_OK) return st;

    NsArgs na{};
    na.descs = d_descs;
    // a phase's runs: by value when they fit in the arguments, the uploaded table otherwise
    auto set_runs = [](NsArgs& a, const TileRun* table, const std::vector<TileRun>& runs) {
        a.runs = table;
        a.nruns = static_cast<int32_t>(runs.size());
        for (int i = 0; i < NS_ARG_RUNS; ++i) a.run[i] = i < a.nruns ? runs[i] : TileRun{0, 0, 1};
    };
    for (int k = 0; k < hp->ns_steps; ++k) {
        na.a = hp->schedule[k].a;
        na.b = hp->schedule[k].b;
        na.c = hp->schedule[k].c;
        na.first = k == 0;
        // muon_step's last update writes W' itself (no apply launch)
        na.apply = (!ns_only && k == hp->ns_steps - 1) ? 1 : 0;
        na.ping = k & 1;
        set_runs(na, d_runs, pl.sym_runs);
        na.total = static_cast<int32_t>(pl.total_sym);
        st = timed_launch(2, stream, "Gram kernel", [&] { return launch_gram(dtype, na, stream); });
        if (st != MUON_OK) return st;
        st = timed_launch(3, stream, "polynomial kernel", [&] { return launch_poly(dtype, na, stream); });
        if (st != MUON_OK) return st;
        set_runs(na, d_runs + nmat, pl.upd_runs);
        na.total = static_cast<int32_t>(pl.total_upd);
        st = timed_launch(na.apply ? 8 : 4, stream, "update kernel", [&] { return launch_update(dtype, na, stream); });
        if (st != MUON_OK) return st;
    }
    if (ns_only || hp->ns_steps == 0) {
        st = timed_launch(5, stream, "apply kernel", [&] { return launch_apply(dtype, ns_only, ew, ew_grid, stream); });
        if (st != MUON_OK) return st;
    }
    g_last_error.clear();
    return MUON_OK;
}

muon_status collect_step(const muon_matrix* mats, int32_t n, const muon_hparams* hp, std::vector<Item>& items) {
    if (n < 0 || n > MUON_MAX_MATRICES) return fail(MUON_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, MUON_MAX_MATRICES);
    if (n > 0 && !mats) return fail(MUON_ERR_INVALID_ARG, "mats is NULL");
    muon_status st = check_hparams(hp, true);
    if (st != MUON_OK) return st;
    const size_t es = hp->dtype == MUON_BF16 ? 2 : 4;
    std::vector<Interval> iv;
    for (int i = 0; i < n; ++i) {
        const muon_matrix& m = mats[i];
        if (!m.grad) continue;
        if (m.rows < 1 || m.cols < 1 || m.rows > MUON_MAX_DIM || m.cols > MUON_MAX_DIM)
            return fail(MUON_ERR_INVALID_ARG, "matrix %d has shape %lld x %lld", i, (long long)m.rows, (long long)m.cols);
        if (!m.weight || !m.momentum) return fail(MUON_ERR_INVALID_ARG, "matrix %d: weight or momentum is NULL", i);
        const uintptr_t pw = reinterpret_cast<uintptr_t>(m.weight), pg = reinterpret_cast<uintptr_t>(m.grad),
                        pm = reinterpret_cast<uintptr_t>(m.momentum);
        if (pw % es || pg % es || pm % es) return fail(MUON_ERR_INVALID_ARG, "matrix %d: misaligned pointer", i);
        const size_t bytes = static_cast<size_t>(m.rows) * static_cast<size_t>(m.cols) * es;
        iv.push_back({pw, pw + bytes, false, i});
        iv.push_back({pm, pm + bytes, false, i});
        iv.push_back({pg, pg + bytes, true, i});
        items.push_back({i, m.grad, m.weight, m.momentum, nullptr, m.rows, m.cols});
    }
    return check_overlaps(iv);
}

muon_status collect_ns(const muon_ns_matrix* mats, int32_t n, const muon_hparams* hp, std::vector<Item>& items) {
    if (n < 0 || n > MUON_MAX_MATRICES) return fail(MUON_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, MUON_MAX_MATRICES);
    if (n > 0 && !mats) return fail(MUON_ERR_INVALID_ARG, "mats is NULL");
    muon_status st = check_hparams(hp, false);
    if (st != MUON_OK) return st;
    const size_t es = hp->dtype == MUON_BF16 ? 2 : 4;
    std::vector<Interval> iv;
    for (int i = 0; i < n; ++i) {
        const muon_ns_matrix& m = mats[i];
        if (m.rows < 1 || m.cols < 1 || m.rows > MUON_MAX_DIM || m.cols > MUON_MAX_DIM)
            return fail(MUON_ERR_INVALID_ARG, "matrix %d has shape %lld x %lld", i, (long long)m.rows, (long long)m.cols);
        if (!m.in || !m.out) return fail(MUON_ERR_INVALID_ARG, "matrix %d: in or out is NULL", i);
        const uintptr_t pi = reinterpret_cast<uintptr_t>(m.in), po = reinterpret_cast<uintptr_t>(m.out);
        if (pi % es || po % 4) return fail(MUON_ERR_INVALID_ARG, "matrix %d: misaligned pointer", i);
        const size_t cnt = static_cast<size_t>(m.rows) * static_cast<size_t>(m.cols);
        iv.push_back({pi, pi + cnt * es, true, i});
        iv.push_back({po, po + cnt * 4, false, i});
        items.push_back({i, m.in, nullptr, nullptr, m.out, m.rows, m.cols});
    }
    return check_overlaps(iv);
}

// ---------------------------------------------------------------------------
// AdamW
// ---------------------------------------------------------------------------

muon_status collect_adamw(const muon_adamw_tensor* ts, int32_t n, const muon_adamw_hparams* hp,
                          std::vector<AdamWDesc>& out) {
    if (n < 0 || n > MUON_MAX_ADAMW_TENSORS)
        return fail(MUON_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, MUON_MAX_ADAMW_TENSORS);
    if (n > 0 && !ts) return fail(MUON_ERR_INVALID_ARG, "tensors is NULL");
    if (!hp) return fail(MUON_ERR_INVALID_ARG, "hp is NULL");
    if (hp->dtype != MUON_F32 && hp->dtype != MUON_BF16) return fail(MUON_ERR_INVALID_ARG, "unknown dtype %d", hp->dtype);
    if (!std::isfinite(hp->lr)) return fail(MUON_ERR_INVALID_ARG, "lr is not finite");
    if (!std::isfinite(hp->weight_decay)) return fail(MUON_ERR_INVALID_ARG, "weight_decay is not finite");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(MUON_ERR_INVALID_ARG, "beta1 and beta2 must lie in [0, 1)");
    if (!std::isfinite(hp->eps) || hp->eps < 0.0f) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (hp->step < 1) return fail(MUON_ERR_INVALID_ARG, "step %d must be >= 1", hp->step);
    const size_t es = hp->dtype == MUON_BF16 ? 2 : 4;
    std::vector<Interval> iv;
    for (int i = 0; i < n; ++i) {
        const muon_adamw_tensor& t = ts[i];
        if (!t.grad) continue;
        if (t.numel < 1 || t.numel > MUON_MAX_ADAMW_NUMEL)
            return fail(MUON_ERR_INVALID_ARG, "tensor %d has numel %lld", i, (long long)t.numel);
        if (!t.param || !t.exp_avg || !t.exp_avg_sq) return fail(MUON_ERR_INVALID_ARG, "tensor %d: a buffer is NULL", i);
        const uintptr_t pp = reinterpret_cast<uintptr_t>(t.param), pg = reinterpret_cast<uintptr_t>(t.grad),
                        pm = reinterpret_cast<uintptr_t>(t.exp_avg), pv = reinterpret_cast<uintptr_t>(t.exp_avg_sq);
        if (pp % es || pg % es || pm % 4 || pv % 4) return fail(MUON_ERR_INVALID_ARG, "tensor %d: misaligned pointer", i);
        const size_t cnt = static_cast<size_t>(t.numel);
        iv.push_back({pp, pp + cnt * es, false, i});
        iv.push_back({pg, pg + cnt * es, true, i});
        iv.push_back({pm, pm + cnt * 4, false, i});
        iv.push_back({pv, pv + cnt * 4, false, i});
        AdamWDesc d{};
        d.p = t.param;
        d.g = t.grad;
        d.m = t.exp_avg;
        d.v = t.exp_avg_sq;
        d.numel = t.numel;
        d.vec = (pp % (4 * es) == 0 && pg % (4 * es) == 0 && pm % 16 == 0 && pv % 16 == 0) ? 1 : 0;
        out.push_back(d);
    }
    return check_overlaps(iv);
}

// ---------------------------------------------------------------------------
// Muon-Cayley
// ---------------------------------------------------------------------------


struct CayleyPlan {
    std::vector<CayleyDesc> descs;
    std::vector<int32_t> prefix[CY_PHASES];
    size_t off_prefix = 0, header_bytes = 0, total_bytes = 0;
};

muon_status collect_cayley(const muon_cayley_matrix* mats, int32_t n, const muon_cayley_hparams* hp,
                           std::vector<CayleyDesc>& out) {
    if (n < 0 || n > MUON_MAX_MATRICES) return fail(MUON_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, MUON_MAX_MATRICES);
    if (n > 0 && !mats) return fail(MUON_ERR_INVALID_ARG, "mats is NULL");
    if (!hp) return fail(MUON_ERR_INVALID_ARG, "hp is NULL");
    if (!std::isfinite(hp->lr)) return fail(MUON_ERR_INVALID_ARG, "lr is not finite");
    if (!(hp->beta >= 0.0f && hp->beta < 1.0f)) return fail(MUON_ERR_INVALID_ARG, "beta must lie in [0, 1)");
    std::vector<Interval> iv;
    for (int i = 0; i < n; ++i) {
        const muon_cayley_matrix& m = mats[i];
        if (!m.grad) continue;
        if (m.rows < 1 || m.cols < 1 || m.rows > MUON_MAX_DIM || m.cols > MUON_MAX_DIM)
            return fail(MUON_ERR_INVALID_ARG, "matrix %d has shape %lld x %lld", i, (long long)m.rows, (long long)m.cols);
        if (std::min(m.rows, m.cols) > MUON_CAYLEY_MAX_K)
            return fail(MUON_ERR_UNSUPPORTED, "matrix %d: min(rows, cols) = %lld exceeds %d", i,
                        (long long)std::min(m.rows, m.cols), MUON_CAYLEY_MAX_K);
        if (!m.weight || !m.momentum) return fail(MUON_ERR_INVALID_ARG, "matrix %d: weight or momentum is NULL", i);
        const uintptr_t pw = reinterpret_cast<uintptr_t>(m.weight), pg = reinterpret_cast<uintptr_t>(m.grad),
                        pm = reinterpret_cast<uintptr_t>(m.momentum);
        if (pw % 4 || pg % 4 || pm % 4) return fail(MUON_ERR_INVALID_ARG, "matrix %d: misaligned pointer", i);
        const size_t bytes = static_cast<size_t>(m.rows) * static_cast<size_t>(m.cols) * 4;
        iv.push_back({pw, pw + bytes, false, i});
        iv.push_back({pm, pm + bytes, false, i});
        iv.push_back({pg, pg + bytes, true, i});
        CayleyDesc d{};
        d.w = m.weight;
        d.g = m.grad;
        d.m = m.momentum;
        d.rows = static_cast<int32_t>(m.rows);
        d.cols = static_cast<int32_t>(m.cols);
        d.tall = m.rows >= m.cols ? 1 : 0;
        d.N = static_cast<int32_t>(std::max(m.rows, m.cols));
        d.K = static_cast<int32_t>(std::min(m.rows, m.cols));
        d.nrb = (d.N + CY_RB - 1) / CY_RB;
        d.tk = (d.K + CY_T - 1) / CY_T;
        d.tn = (d.N + CY_T - 1) / CY_T;
        d.gk = (d.K + CY_GT - 1) / CY_GT;
        d.gn = (d.N + CY_GT - 1) / CY_GT;
        out.push_back(d);
    }
    return check_overlaps(iv);
}

// A tall matrix one product tile wide: p4 writes W' in place (each of its workgroups owns
// whole rows of W, which no other workgroup reads), so there is nothing to copy out.
bool cayley_w_in_place(const CayleyDesc& d) { return d.tall && d.gk == 1; }

muon_status build_cayley_plan(std::vector<CayleyDesc>& descs, CayleyPlan& pl) {
    const size_t nmat = descs.size();
    size_t off = align_up(sizeof(CayleyDesc) * nmat, ALIGN);
    pl.off_prefix = off;
    off = align_up(off + sizeof(int32_t) * CY_PHASES * (nmat + 1), ALIGN);
    pl.header_bytes = off;
    for (int ph = 0; ph < CY_PHASES; ++ph) pl.prefix[ph].assign(nmat + 1, 0);
    int64_t tot[CY_PHASES] = {};
    for (size_t k = 0; k < nmat; ++k) {
        CayleyDesc& d = descs[k];
        const int64_t tiles = static_cast<int64_t>(d.tn) * d.tk;          // 64 x 64 transpose tiles
        const int64_t prod = static_cast<int64_t>(d.gn) * d.gk;           // 128 x 128 N x K product tiles
        const int64_t red = static_cast<int64_t>(d.nrb) * d.gk * d.gk;    // K x K tiles over the row blocks, per product
        // split solve (K <= CY_LDS_K): tiles of the K x K blocks; a larger K solves in CY_SOLVE alone
        const int64_t svg = (d.K + CY_SV_T - 1) / CY_SV_T;
        const int64_t sv = d.K <= CY_LDS_K ? svg * svg : 0;
        int64_t per[CY_PHASES] = {};
        per[CY_TRANSPOSE_IN] = d.tall ? 0 : tiles;
        per[CY_REDUCE1] = 2 * red + d.nrb;   // W^T G, W^T M tiles, then one column-sum block per row block
        const int64_t mt = (d.K + CY_MT - 1) / CY_MT;                     // K x K sums in CY_MT tiles
        per[CY_MID] = mt * mt;
        per[CY_P2] = prod;
        per[CY_REDUCE3] = 3 * red;
        per[CY_SV_SUM] = sv ? mt * mt : 0;
        per[CY_SOLVE] = 1 + (2 * sv + 3) / 4;   // the inversion, and the right-hand side's tiles four a workgroup
        per[CY_SV_G1] = 2 * sv;
        per[CY_SV_G2] = 2 * sv;
        per[CY_SV_INV2] = sv ? 1 : 0;
        per[CY_SV_G3] = sv;
        per[CY_SV_G4] = sv;
        per[CY_P4] = prod;
        const bool w_in_place = cayley_w_in_place(d);
        per[CY_OUT] = w_in_place ? 0 : tiles;
        for (int ph = 0; ph < CY_PHASES; ++ph) {
            tot[ph] += per[ph];
            if (tot[ph] > INT32_MAX) return fail(MUON_ERR_UNSUPPORTED, "too many tiles in one call (split the list)");
            pl.prefix[ph][k + 1] = static_cast<int32_t>(tot[ph]);
        }
        const size_t nk = static_cast<size_t>(d.N) * d.K * 4, kk = static_cast<size_t>(d.K) * d.K;
        auto take = [&](size_t bytes) { const size_t at = off; off = align_up(off + bytes, ALIGN); return at; };
        if (d.tall) {
            d.wf = d.w;
            d.gf = d.g;
            d.mf = d.m;
        } else {
            d.wf = reinterpret_cast<float*>(take(nk));
            d.gf = reinterpret_cast<const float*>(take(nk));
            d.mf = reinterpret_cast<float*>(take(nk));
        }
        d.v = reinterpret_cast<float*>(take(nk));
        d.wnew = w_in_place ? d.w : reinterpret_cast<float*>(take(nk));
        d.part = reinterpret_cast<float*>(take(static_cast<size_t>(d.nrb) * 3 * kk * 4));
        d.colpart = reinterpret_cast<float*>(take(static_cast<size_t>(d.nrb) * 2 * d.K * 4));
        d.small = reinterpret_cast<float*>(take((d.K + kk + 2 * kk) * 4));
        d.cmat = reinterpret_cast<double*>(take(4 * kk * 8));
        d.rhs = reinterpret_cast<double*>(take(2 * kk * 8));
        d.bw = reinterpret_cast<double*>(take(2 * kk * 8));
    }
    pl.total_bytes = off;
    pl.descs = descs;
    return MUON_OK;
}

void rebase_cayley(CayleyPlan& pl, char* base) {
    auto fix = [base](auto*& p) {
        using P = std::remove_reference_t<decltype(p)>;
        p = reinterpret_cast<P>(base + reinterpret_cast<uintptr_t>(p));
    };
    for (CayleyDesc& d : pl.descs) {
        if (!d.tall) {
            fix(d.wf);
            fix(d.gf);
            fix(d.mf);
        }
        fix(d.v);
        if (!cayley_w_in_place(d)) fix(d.wnew);
        fix(d.part);
        fix(d.colpart);
        fix(d.small);
        fix(d.cmat);
        fix(d.rhs);
        fix(d.bw);
    }
}

size_t adamw_header_bytes(size_t n) {
    return align_up(align_up(sizeof(AdamWDesc) * n, ALIGN) + sizeof(int32_t) * (n + 1), ALIGN);
}

}  // namespace

extern "C" {

size_t muon_cayley_workspace_bytes(const muon_cayley_matrix* mats, int32_t n, const muon_cayley_hparams* hp) {
    std::vector<CayleyDesc> descs;
    if (collect_cayley(mats, n, hp, descs) != MUON_OK) return 0;
    if (descs.empty()) return ALIGN;
    CayleyPlan pl;
    if (build_cayley_plan(descs, pl) != MUON_OK) return 0;
    return pl.total_bytes;
}

muon_status muon_cayley_step(const muon_cayley_matrix* mats, int32_t n, const muon_cayley_hparams* hp,
                             void* workspace, size_t workspace_bytes, void* stream) {
    std::vector<CayleyDesc> descs;
    muon_status st = collect_cayley(mats, n, hp, descs);
    if (st != MUON_OK) return st;
    if (descs.empty()) { g_last_error.clear(); return MUON_OK; }
    CayleyPlan pl;
    st = build_cayley_plan(descs, pl);
    if (st != MUON_OK) return st;
    if (!workspace) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % ALIGN)
        return fail(MUON_ERR_WORKSPACE, "workspace is not %zu-byte aligned", ALIGN);
    if (workspace_bytes < pl.total_bytes)
        return fail(MUON_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, pl.total_bytes);
    {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(workspace), hi = lo + pl.total_bytes;
        for (const CayleyDesc& d : pl.descs) {
            const size_t bytes = static_cast<size_t>(d.rows) * d.cols * 4;
            const void* ptrs[3] = {d.w, d.g, d.m};
            for (int q = 0; q < 3; ++q) {
                const uintptr_t p = reinterpret_cast<uintptr_t>(ptrs[q]);
                if (p < hi && p + bytes > lo) return fail(MUON_ERR_INVALID_ARG, "a matrix overlaps the workspace");
            }
        }
    }
    int dev = 0, cu_count = 0;
    st = check_device(&dev, &cu_count);
    if (st != MUON_OK) return st;
    char* base = static_cast<char*>(workspace);
    rebase_cayley(pl, base);
    const size_t nmat = pl.descs.size();
    std::vector<char> header(pl.header_bytes, 0);
    std::memcpy(header.data(), pl.descs.data(), sizeof(CayleyDesc) * nmat);
    for (int ph = 0; ph < CY_PHASES; ++ph)
        std::memcpy(header.data() + pl.off_prefix + sizeof(int32_t) * ph * (nmat + 1), pl.prefix[ph].data(),
                    sizeof(int32_t) * (nmat + 1));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = upload(dev, workspace, header.data(), header.size(), s);
    if (st != MUON_OK) return st;
    CayleyArgs a{};
    a.descs = reinterpret_cast<const CayleyDesc*>(base);
    a.nmat = static_cast<int32_t>(nmat);
    a.beta = hp->beta;
    a.c = 0.5f * hp->lr;
    const int order[CY_PHASES] = {CY_TRANSPOSE_IN, CY_REDUCE1, CY_MID,   CY_P2,    CY_REDUCE3, CY_SV_SUM, CY_SOLVE,
                                  CY_SV_G1,        CY_SV_G2,   CY_SV_INV2, CY_SV_G3, CY_SV_G4,   CY_P4,     CY_OUT};
    for (int ph : order) {
        a.prefix = reinterpret_cast<const int32_t*>(base + pl.off_prefix + sizeof(int32_t) * ph * (nmat + 1));
        a.total = pl.prefix[ph][nmat];
        st = timed_launch(7, s, "Muon-Cayley kernel", [&] { return launch_cayley(ph, a, s); });
        if (st != MUON_OK) return st;
    }
    g_last_error.clear();
    return MUON_OK;
}

size_t muon_adamw_workspace_bytes(const muon_adamw_tensor* tensors, int32_t n, const muon_adamw_hparams* hp) {
    std::vector<AdamWDesc> descs;
    if (collect_adamw(tensors, n, hp, descs) != MUON_OK) return 0;
    return std::max(adamw_header_bytes(descs.size()), ALIGN);
}

muon_status muon_adamw_step(const muon_adamw_tensor* tensors, int32_t n, const muon_adamw_hparams* hp,
                            void* workspace, size_t workspace_bytes, void* stream) {
    std::vector<AdamWDesc> descs;
    muon_status st = collect_adamw(tensors, n, hp, descs);
    if (st != MUON_OK) return st;
    if (descs.empty()) { g_last_error.clear(); return MUON_OK; }
    const size_t need = adamw_header_bytes(descs.size());
    if (!workspace) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % ALIGN)
        return fail(MUON_ERR_WORKSPACE, "workspace is not %zu-byte aligned", ALIGN);
    if (workspace_bytes < need) return fail(MUON_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(workspace), hi = lo + need;
        const size_t es = hp->dtype == MUON_BF16 ? 2 : 4;
        for (const AdamWDesc& d : descs) {
            const size_t cnt = static_cast<size_t>(d.numel);
            const void* ptrs[4] = {d.p, d.g, d.m, d.v};
            const size_t sz[4] = {cnt * es, cnt * es, cnt * 4, cnt * 4};
            for (int q = 0; q < 4; ++q) {
                const uintptr_t p = reinterpret_cast<uintptr_t>(ptrs[q]);
                if (p < hi && p + sz[q] > lo) return fail(MUON_ERR_INVALID_ARG, "a tensor overlaps the workspace");
            }
        }
    }
    // chunk prefix sums (int32 chunk indices)
    const size_t nt = descs.size();
    std::vector<int32_t> prefix(nt + 1, 0);
    int64_t total = 0;
    for (size_t i = 0; i < nt; ++i) {
        total += (descs[i].numel + ADAMW_CHUNK - 1) / ADAMW_CHUNK;
        if (total > INT32_MAX) return fail(MUON_ERR_UNSUPPORTED, "too many elements in one call (split the list)");
        prefix[i + 1] = static_cast<int32_t>(total);
    }
    int dev = 0, cu_count = 0;
    st = check_device(&dev, &cu_count);
    if (st != MUON_OK) return st;
    const size_t off_prefix = align_up(sizeof(AdamWDesc) * nt, ALIGN);
    std::vector<char> header(off_prefix + sizeof(int32_t) * (nt + 1), 0);
    std::memcpy(header.data(), descs.data(), sizeof(AdamWDesc) * nt);
    std::memcpy(header.data() + off_prefix, prefix.data(), sizeof(int32_t) * (nt + 1));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = upload(dev, workspace, header.data(), header.size(), s);
    if (st != MUON_OK) return st;

    // per-call scalars in fp64 from the fp32 hyperparameters
    const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, wd = hp->weight_decay;
    const double bc1 = 1.0 - std::pow(b1, static_cast<double>(hp->step));
    const double bc2 = 1.0 - std::pow(b2, static_cast<double>(hp->step));
    AdamWArgs a{};
    a.descs = static_cast<const AdamWDesc*>(workspace);
    a.prefix = reinterpret_cast<const int32_t*>(static_cast<char*>(workspace) + off_prefix);
    a.n = static_cast<int32_t>(nt);
    a.total = static_cast<int32_t>(total);
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.one_m_beta1 = static_cast<float>(1.0 - b1);
    a.one_m_beta2 = static_cast<float>(1.0 - b2);
    a.eps = hp->eps;
    a.decay = static_cast<float>(1.0 - lr * wd);
    a.step_size = static_cast<float>(lr / bc1);
    a.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(bc2));
    const int grid = static_cast<int>(std::min<int64_t>(total, static_cast<int64_t>(std::max(cu_count, 1)) * 8));
    st = timed_launch(6, s, "AdamW kernel", [&] { return launch_adamw(hp->dtype, a, grid, s); });
    if (st != MUON_OK) return st;
    g_last_error.clear();
    return MUON_OK;
}

size_t muon_workspace_bytes(const muon_matrix* mats, int32_t n, const muon_hparams* hp) {
    std::vector<Item> items;
    if (collect_step(mats, n, hp, items) != MUON_OK) return 0;
    if (items.empty()) return ALIGN;
    Plan pl;
    if (build_plan(items, hp, false, pl) != MUON_OK) return 0;
    return pl.total_bytes;
}

muon_status muon_step(const muon_matrix* mats, int32_t n, const muon_hparams* hp, void* workspace,
                      size_t workspace_bytes, void* stream) {
    std::vector<Item> items;
    muon_status st = collect_step(mats, n, hp, items);
    if (st != MUON_OK) return st;
    if (items.empty()) { g_last_error.clear(); return MUON_OK; }
    return run(items, hp, false, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

muon_status muon_step_noalloc(const muon_matrix* mats, int32_t n, const muon_hparams* hp, void* stream) {
    std::vector<Item> items;
    muon_status st = collect_step(mats, n, hp, items);
    if (st != MUON_OK) return st;
    if (items.empty()) { g_last_error.clear(); return MUON_OK; }
    {
        Plan pl;
        st = build_plan(items, hp, false, pl);
        if (st != MUON_OK) return st;
        if (pl.total_bytes > MUON_NOALLOC_SCRATCH_BYTES)
            return fail(MUON_ERR_WORKSPACE, "this list needs %zu bytes of workspace; muon_step_noalloc holds at most %zu "
                        "(use muon_step with a caller workspace, or split the list)",
                        pl.total_bytes, static_cast<size_t>(MUON_NOALLOC_SCRATCH_BYTES));
    }
    int dev = 0, cu_count = 0;
    st = check_device(&dev, &cu_count);
    if (st != MUON_OK) return st;
    char* ws = nullptr;
    st = scratch_address(dev, &ws);
    if (st != MUON_OK) return st;
    return run(items, hp, false, ws, MUON_NOALLOC_SCRATCH_BYTES, static_cast<hipStream_t>(stream), true);
}

size_t muon_ns_workspace_bytes(const muon_ns_matrix* mats, int32_t n, const muon_hparams* hp) {
    std::vector<Item> items;
    if (collect_ns(mats, n, hp, items) != MUON_OK) return 0;
    if (items.empty()) return ALIGN;
    Plan pl;
    if (build_plan(items, hp, true, pl) != MUON_OK) return 0;
    return pl.total_bytes;
}

muon_status muon_ns(const muon_ns_matrix* mats, int32_t n, const muon_hparams* hp, void* workspace,
                    size_t workspace_bytes, void* stream) {
    std::vector<Item> items;
    muon_status st = collect_ns(mats, n, hp, items);
    if (st != MUON_OK) return st;
    if (items.empty()) { g_last_error.clear(); return MUON_OK; }
    return run(items, hp, true, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

const char* muon_status_string(int32_t status) {
    switch (status) {
        case MUON_OK: return "MUON_OK";
        case MUON_ERR_INVALID_ARG: return "MUON_ERR_INVALID_ARG: invalid argument";
        case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED: unsupported device or size";
        case MUON_ERR_WORKSPACE: return "MUON_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case MUON_ERR_HIP: return "MUON_ERR_HIP: HIP runtime error";
        default: return "unknown muon_status";
    }
}

const char* muon_last_error_message(void) { return g_last_error.c_str(); }

muon_status muon_profile_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_prof.on = on != 0;
    return MUON_OK;
}

muon_status muon_profile_read(muon_profile* out) {
    if (!out) return fail(MUON_ERR_INVALID_ARG, "out is NULL");
    std::vector<ProfRec> recs;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        recs.swap(g_prof.recs);
    }
    std::memset(out, 0, sizeof(*out));
    muon_status st = MUON_OK;
    for (const ProfRec& r : recs) {
        hipError_t e = hipEventSynchronize(r.b);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && st == MUON_OK) st = hip_fail(e, "hipEventElapsedTime");
        out->ms[r.cls] += ms;
        out->launches[r.cls] += 1;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    for (const ProfRec& r : recs) { g_prof.pool.push_back(r.a); g_prof.pool.push_back(r.b); }
    return st;
}

int32_t muon_version(void) { return 100; }

}  // extern "C"
