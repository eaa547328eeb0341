// ddm.hip -- host side of the C ABI declared in include/ddm.h: argument
// validation, workspace layout and the stream-ordered launch sequences.
// Every step of every call runs in the kernels of ddm_sweep.hpp / ddm_aux.hpp;
// the host only checks arguments and enqueues.
#include "../../include/ddm.h"
#include "ddm_frm.hpp"
#include "ddm_c2f.hpp"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <array>
#include <atomic>
#include <list>
#include <mutex>
#include <vector>

using namespace ddm;

// Workspace of ddm_frm_match_noalloc: library-held device memory, one copy per device, for the
// life of the process. Host code never passes this name to a kernel (on the host it is only a
// stand-in for the symbol); the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[DDM_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on each device, looked up once per device with that device current.
int scratch_ptr(int dev, void **out) {
    static std::mutex mu;
    static std::vector<void *> ptrs;
    std::lock_guard<std::mutex> g(mu);
    if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
    if (!ptrs[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DDM_ERR_HIP;
        ptrs[dev] = ptr;
    }
    *out = ptrs[dev];
    return DDM_OK;
}

// Sweep shapes. Each wave holds RQ query tiles of 16 rows. A workgroup keeps one
// LDS-resident reference chunk and carries 8 waves (two per SIMD), so that one
// wave's matrix-core work overlaps the other's epilogue; fp32 maps use 4 waves.
constexpr int nw_for(int dt) { return dt == DT_F32 ? 4 : 8; }
// Query tiles per wave: 6 for fp16/bf16 with up to 64 components (two
// accumulator sets of the software pipeline fit in 256 VGPRs), 4 for wider
// rows, 2 for fp32 maps (up to 32 K-blocks of A resident).
constexpr int rq_for(int dt, int nkb) { return dt == DT_F32 ? 2 : (nkb <= 2 ? 6 : 4); }
constexpr size_t LDS_MAX = 160 * 1024;
constexpr long long MIN_WG = 256;          // one workgroup per CU
constexpr size_t LOOP_LDS_MAX = LDS_MAX - 1024;   // the FRM loop kernel keeps a few LDS words of its own
constexpr int MAX_PIX = 1 << 27;
constexpr int OUT_MAX_PIXELS = 1 << 19;     // image-1 pixels of the one-workgroup FRM output (bitmap + ranks: 128 KB)

struct MapFmt {
    int dtype, d;
    int ld;        // stored row stride (elements) seen by the kernels
    int np;        // compile-time pieces per row (0 = runtime, fp32)
    int nkb;       // compile-time K blocks
    int esz;       // bytes per element
    bool repack;   // rows are copied into a prepared [n][ld] buffer first (zero padding or metric rows)
    bool l2;       // Euclidean metric: fp32 rows of d_in, prepared as d = d_in + 2 (query / reference side)
    int d_in;      // elements per input row
    int tile_bytes() const { return dtype == DT_F32 ? ld * 16 * 4 : np * 16 * 16; }
    int group() const { return TILE * group_tiles(dtype); }          // references per index group
    int sb_rows() const { return nw_for(dtype) * rq_for(dtype, nkb) * 16; }
};

bool make_fmt(int dtype, int d, MapFmt *f, int metric = DDM_DOT) {
    if (d < 1 || d > DDM_MAX_D) return false;
    f->l2 = false; f->d_in = d;
    if (metric == DDM_L2) {
        if (dtype != DT_F32 || d + 2 > DDM_MAX_D) return false;
        f->dtype = DT_F32; f->d = d + 2; f->ld = d + 2; f->np = 0; f->nkb = d + 2 <= 32 ? 8 : 32; f->esz = 4;
        f->repack = true; f->l2 = true;
        return true;
    }
    if (metric != DDM_DOT) return false;
    f->dtype = dtype; f->d = d;
    if (dtype == DT_F32) {
        f->ld = d; f->np = 0; f->nkb = d <= 32 ? 8 : 32; f->esz = 4; f->repack = false;
        return true;
    }
    if (dtype != DT_F16 && dtype != DT_BF16) return false;
    static const int supported[] = {1, 2, 3, 4, 6, 8, 12, 16};
    const int need = (d + 7) / 8;
    int np = 16;
    for (int s : supported) if (s >= need) { np = s; break; }
    f->np = np; f->nkb = (np + 3) / 4; f->ld = np * 8; f->esz = 2; f->repack = (f->ld != d);
    return true;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Bump {
    size_t off = 0;
    size_t take(size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; }
};

// LDS of a sweep task past the chunk (and COLMAX's column array): the unit counter
constexpr size_t SWEEP_LDS_EXTRA = 16;

int chunk_limit(const MapFmt &f, bool colmax, size_t lds_max = LDS_MAX) {
    const size_t per_ref = (size_t)f.tile_bytes() / TILE + (colmax ? 4 : 0);
    const int grp = f.group();
    int c = (int)((lds_max - SWEEP_LDS_EXTRA) / per_ref) / grp * grp;
    return std::max(c, grp);
}

size_t sweep_lds(const MapFmt &f, int chunk, bool colmax) {
    return (size_t)(chunk / TILE) * f.tile_bytes() + (colmax ? (size_t)chunk * 4 : 0) + SWEEP_LDS_EXTRA;
}

// ----------------------------------------------------------------- dispatch
// launch == false only raises the instantiation's dynamic-LDS limit (done once,
// before any launch, so that it never happens inside a stream capture).
template <int DT, int NP, int NKB, bool COLMAX>
hipError_t launch_sweep_t(const SweepArgs &a, dim3 grid, size_t lds, hipStream_t s, bool launch) {
    constexpr int rq = rq_for(DT, NKB);
    constexpr int nw = nw_for(DT);
    auto k = sweep_kernel<DT, NP, NKB, rq, nw, COLMAX>;
    if (!launch)
        return hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_MAX);
    hipLaunchKernelGGL(k, grid, dim3(nw * 64), lds, s, a);
    return hipGetLastError();
}

template <int DT, bool COLMAX>
hipError_t launch_sweep_dt(const MapFmt &f, const SweepArgs &a, dim3 grid, size_t lds, hipStream_t s, bool launch) {
    if constexpr (DT == DT_F32) {
        if (f.nkb == 8) return launch_sweep_t<DT_F32, 0, 8, COLMAX>(a, grid, lds, s, launch);
        return launch_sweep_t<DT_F32, 0, 32, COLMAX>(a, grid, lds, s, launch);
    } else {
        switch (f.np) {
        case 1: return launch_sweep_t<DT, 1, 1, COLMAX>(a, grid, lds, s, launch);
        case 2: return launch_sweep_t<DT, 2, 1, COLMAX>(a, grid, lds, s, launch);
        case 3: return launch_sweep_t<DT, 3, 1, COLMAX>(a, grid, lds, s, launch);
        case 4: return launch_sweep_t<DT, 4, 1, COLMAX>(a, grid, lds, s, launch);
        case 6: return launch_sweep_t<DT, 6, 2, COLMAX>(a, grid, lds, s, launch);
        case 8: return launch_sweep_t<DT, 8, 2, COLMAX>(a, grid, lds, s, launch);
        case 12: return launch_sweep_t<DT, 12, 3, COLMAX>(a, grid, lds, s, launch);
        case 16: return launch_sweep_t<DT, 16, 4, COLMAX>(a, grid, lds, s, launch);
        default: return hipErrorInvalidValue;
        }
    }
}

hipError_t sweep_switch(const MapFmt &f, bool colmax, const SweepArgs &a, dim3 grid, size_t lds, hipStream_t s,
                        bool launch) {
    switch (f.dtype) {
    case DT_F16: return colmax ? launch_sweep_dt<DT_F16, true>(f, a, grid, lds, s, launch)
                               : launch_sweep_dt<DT_F16, false>(f, a, grid, lds, s, launch);
    case DT_BF16: return colmax ? launch_sweep_dt<DT_BF16, true>(f, a, grid, lds, s, launch)
                                : launch_sweep_dt<DT_BF16, false>(f, a, grid, lds, s, launch);
    default: return colmax ? launch_sweep_dt<DT_F32, true>(f, a, grid, lds, s, launch)
                           : launch_sweep_dt<DT_F32, false>(f, a, grid, lds, s, launch);
    }
}

// Format dispatch for the loop kernel: fn(dtype, pieces, K blocks) as constants.
template <int DT, class Fn>
hipError_t np_dispatch(const MapFmt &f, Fn &&fn) {
    using std::integral_constant;
    using D = integral_constant<int, DT>;
    if constexpr (DT == DT_F32) {
        if (f.nkb == 8) return fn(D{}, integral_constant<int, 0>{}, integral_constant<int, 8>{});
        return fn(D{}, integral_constant<int, 0>{}, integral_constant<int, 32>{});
    } else {
        switch (f.np) {
        case 1: return fn(D{}, integral_constant<int, 1>{}, integral_constant<int, 1>{});
        case 2: return fn(D{}, integral_constant<int, 2>{}, integral_constant<int, 1>{});
        case 3: return fn(D{}, integral_constant<int, 3>{}, integral_constant<int, 1>{});
        case 4: return fn(D{}, integral_constant<int, 4>{}, integral_constant<int, 1>{});
        case 6: return fn(D{}, integral_constant<int, 6>{}, integral_constant<int, 2>{});
        case 8: return fn(D{}, integral_constant<int, 8>{}, integral_constant<int, 2>{});
        case 12: return fn(D{}, integral_constant<int, 12>{}, integral_constant<int, 3>{});
        case 16: return fn(D{}, integral_constant<int, 16>{}, integral_constant<int, 4>{});
        default: return hipErrorInvalidValue;
        }
    }
}
template <class Fn>
hipError_t fmt_dispatch(const MapFmt &f, Fn &&fn) {
    switch (f.dtype) {
    case DT_F16: return np_dispatch<DT_F16>(f, fn);
    case DT_BF16: return np_dispatch<DT_BF16>(f, fn);
    default: return np_dispatch<DT_F32>(f, fn);
    }
}

// Test aid: upper bound on the grid of the FRM phase kernels, which stride their
// tasks over whatever grid they get (0 = none). Results must not depend on it;
// a bound of 1 runs every task in one workgroup.
std::atomic<int> &frm_grid_cap() { static std::atomic<int> n{0}; return n; }
long long capped_grid(long long g) {
    const int cap = frm_grid_cap().load();
    return cap > 0 ? std::min<long long>(g, cap) : g;
}

// FRM phase kernels of one map format. which = 0: per-half-step sweep of
// half-step h (plain launch), 1: loop kernel from half-step h (cooperative
// launch), 2: tail kernel from half-step h (plain launch). The grid is
// min(ntask, workgroups the device keeps resident).
// launch == false only raises the kernels' dynamic-LDS limit.
template <int DT, int NP, int NKB>
hipError_t launch_frm_t(int which, const FrmArgs *a, int h, size_t lds, long long ntask, hipStream_t s,
                        bool launch) {
    constexpr int rq = rq_for(DT, NKB);
    constexpr int nw = nw_for(DT);
    auto ks = frm_sweep_kernel<DT, NP, NKB, rq, nw>;
    auto kl = frm_loop_kernel<DT, NP, NKB, rq, nw>;
    auto kt = frm_tail_kernel<DT, NP, NKB, rq, nw>;
    if (!launch) {
        for (const void *k : {(const void *)ks, (const void *)kl, (const void *)kt}) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LOOP_LDS_MAX);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const void *kf = which == 0 ? (const void *)ks : which == 1 ? (const void *)kl : (const void *)kt;
    int dev = 0, ncu = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kf, nw * 64, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || ncu < 1) return hipErrorInvalidConfiguration;
    const unsigned grid =
        (unsigned)std::max<long long>(1, capped_grid(std::min<long long>(ntask, (long long)per_cu * ncu)));
    if (which == 0) {
        hipLaunchKernelGGL(ks, dim3(grid), dim3(nw * 64), lds, s, *a, h);
        return hipGetLastError();
    }
    if (which == 2) {
        hipLaunchKernelGGL(kt, dim3(grid), dim3(nw * 64), lds, s, *a, h);
        return hipGetLastError();
    }
    void *args[] = {(void *)a, (void *)&h};
    return hipLaunchCooperativeKernel((const void *)kl, dim3(grid), dim3(nw * 64), args, (unsigned)lds, s);
}

hipError_t frm_switch(const MapFmt &f, int which, const FrmArgs *a, int h, size_t lds, long long ntask,
                      hipStream_t s, bool launch) {
    return fmt_dispatch(f, [&](auto dt, auto np, auto nkb) {
        return launch_frm_t<decltype(dt)::value, decltype(np)::value, decltype(nkb)::value>(which, a, h, lds, ntask,
                                                                                          s, launch);
    });
}

// Raise the dynamic-LDS limit of every sweep instantiation once per process.
hipError_t prepare_kernels() {
    static std::once_flag once;
    static hipError_t status = hipSuccess;
    std::call_once(once, [] {
        const int dts[] = {DT_F32, DT_F16, DT_BF16};
        for (int dt : dts)
            for (int np : {1, 2, 3, 4, 6, 8, 12, 16})
                for (int cm = 0; cm < 2; ++cm) {
                    MapFmt f;
                    if (!make_fmt(dt, dt == DT_F32 ? (np <= 4 ? 8 : 64) : np * 8, &f)) continue;
                    SweepArgs a{};
                    hipError_t e = sweep_switch(f, cm != 0, a, dim3(1), 0, nullptr, false);
                    if (e != hipSuccess) status = e;
                    if (cm == 0) {
                        e = frm_switch(f, 0, nullptr, 0, 0, 0, nullptr, false);
                        if (e != hipSuccess) status = e;
                    }
                }
        hipError_t e = hipFuncSetAttribute((const void *)frm_output_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(OUT_MAX_PIXELS / 4));
        if (e != hipSuccess) status = e;
    });
    return status;
}

// ------------------------------------------------------------ sweep timing
// When enabled, every sweep launch of the selected kinds is bracketed by two
// HIP events on its stream; ddm_profile_read sums their elapsed times.
struct Profiler {
    std::mutex mu;
    int mask = 0;                                   // 1 = mutual sweeps, 2 = NN/FRM sweeps
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pending, pool;
};
Profiler &prof() { static Profiler p; return p; }

// Set while ddm_frm_match_noalloc enqueues: no timing events are created or recorded.
thread_local bool t_no_events = false;

// Enqueue fn(), bracketed by two events on s when timing of `kind` is on.
template <class Fn>
hipError_t with_events(int kind, hipStream_t s, Fn fn) {
    Profiler &P = prof();
    if (t_no_events || !(P.mask & kind)) return fn();
    std::pair<hipEvent_t, hipEvent_t> ev;
    {
        std::lock_guard<std::mutex> g(P.mu);
        if (P.pool.empty()) {
            if (hipEventCreate(&ev.first) != hipSuccess || hipEventCreate(&ev.second) != hipSuccess)
                return hipErrorOutOfMemory;
        } else {
            ev = P.pool.back(); P.pool.pop_back();
        }
    }
    hipError_t e = hipEventRecord(ev.first, s);
    if (e == hipSuccess) e = fn();
    if (e == hipSuccess) e = hipEventRecord(ev.second, s);
    std::lock_guard<std::mutex> g(P.mu);
    P.pending.push_back(ev);
    return e;
}

hipError_t launch_sweep_impl(const MapFmt &f, bool colmax, const SweepArgs &a, dim3 grid, hipStream_t s);

hipError_t launch_sweep(const MapFmt &f, bool colmax, const SweepArgs &a, dim3 grid, hipStream_t s) {
    return with_events(colmax ? 1 : 2, s, [&] { return launch_sweep_impl(f, colmax, a, grid, s); });
}

hipError_t launch_sweep_impl(const MapFmt &f, bool colmax, const SweepArgs &a, dim3 grid, hipStream_t s) {
    return sweep_switch(f, colmax, a, grid, sweep_lds(f, a.chunk, colmax), s, true);
}

#define DDM_DT_SWITCH(dtype, KERNEL, ...)                                                         \
    do {                                                                                          \
        if ((dtype) == DT_F16) hipLaunchKernelGGL(KERNEL<DT_F16>, __VA_ARGS__);                   \
        else if ((dtype) == DT_BF16) hipLaunchKernelGGL(KERNEL<DT_BF16>, __VA_ARGS__);            \
        else hipLaunchKernelGGL(KERNEL<DT_F32>, __VA_ARGS__);                                     \
    } while (0)

// resolve kernels: dtype x queries per block
#define DDM_QB_LAUNCH(DT, qb, KERNEL, ...)                                                        \
    do {                                                                                          \
        if ((qb) == 256) hipLaunchKernelGGL(HIP_KERNEL_NAME(KERNEL<DT, 256>), __VA_ARGS__);       \
        else if ((qb) == 64) hipLaunchKernelGGL(HIP_KERNEL_NAME(KERNEL<DT, 64>), __VA_ARGS__);    \
        else hipLaunchKernelGGL(HIP_KERNEL_NAME(KERNEL<DT, 16>), __VA_ARGS__);                    \
    } while (0)
#define DDM_DT_QB_SWITCH(dtype, qb, KERNEL, ...)                                                  \
    do {                                                                                          \
        if ((dtype) == DT_F16) DDM_QB_LAUNCH(DT_F16, qb, KERNEL, __VA_ARGS__);                    \
        else if ((dtype) == DT_BF16) DDM_QB_LAUNCH(DT_BF16, qb, KERNEL, __VA_ARGS__);             \
        else DDM_QB_LAUNCH(DT_F32, qb, KERNEL, __VA_ARGS__);                                      \
    } while (0)

// Queries per resolve block: large blocks amortise the phase-1 reduction, but
// the launch should still give every CU several blocks.
int resolve_qb(long long nq) {
    for (int qb : {256, 64})
        if (nq / qb >= 2048) return qb;
    return 16;
}

#define DDM_CHECK(expr)                                                                           \
    do {                                                                                          \
        if ((expr) != hipSuccess) return DDM_ERR_HIP;                                             \
    } while (0)
#define DDM_CHECK_LAUNCH() DDM_CHECK(hipGetLastError())

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool map_ok(const void *p, const MapFmt &f) {
    if (!p) return false;
    return aligned(p, f.repack ? 2 : (size_t)(f.dtype == DT_F32 ? 4 : 16));
}

int pix_ok(int H, int W) {
    return H >= 1 && W >= 1 && (long long)H * W <= MAX_PIX;
}

int64_t seed_count(int H, int W, int S) {
    if (S <= 0 || H < 0 || W < 0) return -1;
    const int h0 = S / 2;
    const int64_t ky = H > h0 ? (H - h0 + S - 1) / S : 0;
    const int64_t kx = W > h0 ? (W - h0 + S - 1) / S : 0;
    return ky * kx;
}

// Repack every map of a batch into ld-strided rows when needed.
// ref_side selects the reference-side rows of the Euclidean metric (ignored otherwise).
int maybe_repack(const MapFmt &f, const void *src, long long rows, void *dst, hipStream_t s, const void **use,
                 int ref_side = 0) {
    if (!f.repack) { *use = src; return DDM_OK; }
    if (f.l2) {
        const int blocks = (int)std::min<long long>((rows + 255) / 256, 65535);
        hipLaunchKernelGGL(l2_augment_kernel, dim3(std::max(blocks, 1)), dim3(256), 0, s, (const float *)src, f.d_in,
                           rows, ref_side, (float *)dst);
        DDM_CHECK_LAUNCH();
        *use = dst;
        return DDM_OK;
    }
    const long long total = rows * f.ld;
    const int blocks = (int)std::min<long long>((total + 255) / 256, 65535);
    hipLaunchKernelGGL(repack_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t *)src, f.d, (uint16_t *)dst,
                       f.ld, rows);
    DDM_CHECK_LAUNCH();
    *use = dst;
    return DDM_OK;
}

// ----------------------------------------------------------------- NN plan
struct NnPlan {
    MapFmt f;
    int NQ, M, N, chunk, nchunks, qblocks;
    size_t o_part, o_rq, o_rr, o_rows, total;
};

int nn_plan(int NQ, int M, int N, int d, int dtype, NnPlan *p, int metric = DDM_DOT) {
    if (NQ < 1 || M < 1 || N < 1 || N > MAX_PIX || M > MAX_PIX || NQ > MAX_PIX) return DDM_ERR_INVALID;
    if (dtype != DT_F32 && dtype != DT_F16 && dtype != DT_BF16) return DDM_ERR_UNSUPPORTED;
    if (!make_fmt(dtype, d, &p->f, metric)) return DDM_ERR_UNSUPPORTED;
    p->NQ = NQ; p->M = M; p->N = N;
    const int sbr = p->f.sb_rows();
    p->qblocks = (M + sbr - 1) / sbr;
    int chunk = chunk_limit(p->f, false);
    // largest LDS-resident chunk; shrink only while there is less than one workgroup per CU
    while (chunk > p->f.group() && (long long)p->qblocks * ((N + chunk - 1) / chunk) < MIN_WG) chunk -= p->f.group();
    p->chunk = chunk;
    p->nchunks = (N + chunk - 1) / chunk;
    Bump b;
    p->o_part = b.take((size_t)p->nchunks * M * 8);
    p->o_rq = p->f.repack ? b.take((size_t)NQ * p->f.ld * p->f.esz) : 0;
    p->o_rr = p->f.repack ? b.take((size_t)N * p->f.ld * p->f.esz) : 0;
    p->o_rows = b.take((size_t)M * 4);
    p->total = b.off;
    return DDM_OK;
}

// ----------------------------------------------------------------- FRM plan
struct FrmPlan {
    MapFmt f;
    int B, H1, W1, N1, N2, k, kx, S, max_iter, nhalf;
    int chunk1, chunk2, nch1, nch2, qblocks, nblk;
    long long k_bs, cnt_bs, part_bs;
    size_t o_u, o_v, o_conv, o_score, o_act0, o_act1, o_qr0, o_qr1, o_counts, o_part, o_mj, o_ms, o_bc, o_bo,
        o_r1, o_r2, o_r1b, o_r2b, o_ctl, o_uprev, o_uiter, o_marks, total;
    size_t loop_lds;       // dynamic LDS of the loop kernel
    bool explicit_starts;  // seeds from a caller list (k = its length, an upper bound) instead of the grid
};

// Options of the routine beyond the grid form: explicit start pixels, the pixel
// tolerance of the final selection, and the basin variant.
struct FrmOpts {
    const int32_t *starts = nullptr;   // device int32[n_starts] linear image-1 pixels, or null for the grid
    int n_starts = 0;
    double pixel_tol = 0.0;
    int32_t *basin = nullptr;          // device int32[N1], or null
};

int frm_chunk(const MapFmt &f, int nref, long long wg_other) {
    int chunk = chunk_limit(f, false, LOOP_LDS_MAX);
    while (chunk > f.group() && wg_other * ((nref + chunk - 1) / chunk) < MIN_WG) chunk -= f.group();
    return chunk;
}

// n_starts < 0: seeds on the stride-S grid; n_starts >= 0: that many explicit starts (one pair only).
int frm_plan(int B, int H1, int W1, int H2, int W2, int d, int dtype, int S, int max_iter, FrmPlan *p,
             int n_starts = -1, int metric = DDM_DOT) {
    if (B < 1 || !pix_ok(H1, W1) || !pix_ok(H2, W2)) return DDM_ERR_INVALID;
    if (max_iter < 1 || max_iter > DDM_MAX_ITER) return DDM_ERR_INVALID;
    if (n_starts < 0 && S < 1) return DDM_ERR_INVALID;
    if (n_starts >= 0 && (B != 1 || n_starts > MAX_PIX)) return DDM_ERR_INVALID;
    if (dtype != DT_F32 && dtype != DT_F16 && dtype != DT_BF16) return DDM_ERR_UNSUPPORTED;
    if (!make_fmt(dtype, d, &p->f, metric)) return DDM_ERR_UNSUPPORTED;
    p->B = B; p->H1 = H1; p->W1 = W1; p->N1 = H1 * W1; p->N2 = H2 * W2;
    p->max_iter = max_iter; p->nhalf = 2 * max_iter;
    p->explicit_starts = n_starts >= 0;
    if (p->explicit_starts) {
        p->S = 1; p->k = n_starts; p->kx = 0;
    } else {
        p->S = S;
        p->k = (int)seed_count(H1, W1, S);
        p->kx = W1 > S / 2 ? (W1 - S / 2 + S - 1) / S : 0;
    }
    const int sbr = p->f.sb_rows();
    const int kk = std::max(p->k, 1);
    p->qblocks = (kk + sbr - 1) / sbr;
    p->chunk2 = frm_chunk(p->f, p->N2, (long long)p->qblocks * B);
    p->chunk1 = frm_chunk(p->f, p->N1, (long long)p->qblocks * B);
    p->nch2 = (p->N2 + p->chunk2 - 1) / p->chunk2;
    p->nch1 = (p->N1 + p->chunk1 - 1) / p->chunk1;
    p->nblk = (p->N1 + CB - 1) / CB;
    p->k_bs = kk;
    p->cnt_bs = (long long)align_up((size_t)p->nhalf + 1, 64);
    // partial slots of the runtime split: chunks x sub-chunks x rows per slot <= chunks x all query blocks
    p->part_bs = (long long)std::max(p->nch1, p->nch2) * p->qblocks * sbr;
    Bump b;
    const size_t kb = (size_t)B * kk * 4;
    p->o_u = b.take(kb); p->o_v = b.take(kb); p->o_conv = b.take(kb); p->o_score = b.take(kb);
    p->o_act0 = b.take(kb); p->o_act1 = b.take(kb); p->o_qr0 = b.take(kb); p->o_qr1 = b.take(kb);
    p->o_counts = b.take((size_t)B * p->cnt_bs * 4);
    p->o_part = b.take((size_t)B * p->part_bs * 8);
    p->o_mj = b.take((size_t)B * p->N1 * 4);
    p->o_ms = b.take((size_t)B * p->N1 * 4);
    p->o_bc = b.take((size_t)B * p->nblk * 4);
    p->o_bo = b.take((size_t)B * p->nblk * 4);
    p->o_r1 = p->f.repack ? b.take((size_t)B * p->N1 * p->f.ld * p->f.esz) : 0;
    p->o_r2 = p->f.repack ? b.take((size_t)B * p->N2 * p->f.ld * p->f.esz) : 0;
    // the Euclidean metric needs each map on both sides (query and reference rows differ)
    p->o_r1b = p->f.l2 ? b.take((size_t)B * p->N1 * p->f.ld * p->f.esz) : 0;
    p->o_r2b = p->f.l2 ? b.take((size_t)B * p->N2 * p->f.ld * p->f.esz) : 0;
    p->o_ctl = b.take(1024);    // control words 128 B apart: barrier, error, tail ticket / done / ready
    p->o_uprev = b.take(kb); p->o_uiter = b.take(kb);
    p->o_marks = p->explicit_starts ? b.take((size_t)p->N1 * 4) : 0;
    p->total = b.off;
    p->loop_lds = std::max(sweep_lds(p->f, std::max(p->chunk1, p->chunk2), false),
                           (size_t)nw_for(dtype) * 64 * sizeof(uint64_t));
    return DDM_OK;
}

int compact_run(const int32_t *mj, const float *ms, long long n_bs, int n, int B, int nblk, int32_t *bc, int32_t *bo,
                int32_t *out_i, int32_t *out_j, float *out_s, long long out_bs, int32_t *out_count, hipStream_t s,
                const int32_t *err = nullptr, const int32_t *owner = nullptr) {
    hipLaunchKernelGGL(compact_count_kernel, dim3(nblk, B), dim3(256), 0, s, mj, n_bs, n, bc, nblk, owner);
    DDM_CHECK_LAUNCH();
    hipLaunchKernelGGL(compact_scan_kernel, dim3(B), dim3(256), 0, s, (const int32_t *)bc, bo, nblk, out_count,
                       (int)out_bs, err);
    DDM_CHECK_LAUNCH();
    hipLaunchKernelGGL(compact_scatter_kernel, dim3(nblk, B), dim3(256), 0, s, mj, ms, n_bs, n,
                       (const int32_t *)bo, nblk, out_i, out_j, out_s, out_bs, (int)out_bs, owner);
    DDM_CHECK_LAUNCH();
    return DDM_OK;
}

// Sweep and resolve arguments of one FRM direction (0: image 1 -> 2, 1: back).
// m1q/m2q: the maps as queries, m1r/m2r: as references (the same buffers except
// under the Euclidean metric).
void frm_dir_args(const FrmPlan &P, const void *m1q, const void *m1r, const void *m2q, const void *m2r,
                  uint64_t *part, int dir, SweepArgs *a, ResolveArgs *r) {
    const MapFmt &f = P.f;
    const long long b1 = (long long)P.N1 * f.ld * f.esz, b2 = (long long)P.N2 * f.ld * f.esz;
    *a = SweepArgs{};
    a->Q = (const unsigned char *)(dir == 0 ? m1q : m2q);
    a->R = (const unsigned char *)(dir == 0 ? m2r : m1r);
    a->q_bs = dir == 0 ? b1 : b2;
    a->r_bs = dir == 0 ? b2 : b1;
    a->qrows_bs = P.k_bs;
    a->qcount_bs = P.cnt_bs;
    a->rowpart = part; a->rowpart_bs = P.part_bs;
    a->nq = P.k;
    a->nref = dir == 0 ? P.N2 : P.N1;
    a->ld = f.ld;
    a->chunk = dir == 0 ? P.chunk2 : P.chunk1;
    a->nchunks = dir == 0 ? P.nch2 : P.nch1;
    a->sb_per_wg = 1;
    a->rowcap = (int)P.k_bs;
    const int split = (int)std::max<long long>(1, MIN_WG / P.B);      // fill the device across the batch
    a->split = split; a->qblocks = P.qblocks; a->split_rows = f.sb_rows();
    *r = ResolveArgs{};
    r->rowpart = part; r->rowpart_bs = P.part_bs; r->nchunks = a->nchunks; r->rowcap = (int)P.k_bs;
    r->Q = a->Q; r->q_bs = a->q_bs; r->nq = P.k;
    r->R = a->R; r->r_bs = a->r_bs; r->nref = a->nref; r->ld = f.ld; r->d = f.d;
    r->split = split; r->qblocks = P.qblocks; r->split_rows = f.sb_rows(); r->chunk_groups = a->chunk / f.group();
    r->neg_out = f.l2 ? 1 : 0;
}

// Largest image-1 map (pixels) whose FRM output goes through the one-workgroup
// bitmap kernel; larger maps (or a test aid lowering it) take the collection
// kernel and the multi-workgroup compaction.
std::atomic<int> &output_bitmap_limit() { static std::atomic<int> n{OUT_MAX_PIXELS}; return n; }

// Polls per grid-barrier wait of the loop kernel (a test aid lowers it to force the failure path).
std::atomic<int> &loop_spin_limit() { static std::atomic<int> n{kSpinLimit}; return n; }

// How the half-steps of one FRM call are launched: [0, h_split) as one sweep
// and one update launch each, the rest in one loop kernel (tail = 1,
// cooperative) or one tail kernel (tail = 2); both stop when no seed is active.
struct FrmExec {
    int h_split, tail;
};

// Iterations run per half-step before the tail kernel takes over
// (DDM_FRM_TAIL); -1 chooses by the work of one full sweep.
std::atomic<int> &tail_after() { static std::atomic<int> n{-1}; return n; }

// Launch plan of a call in the effective mode `mode` (the caller has already
// replaced the loop mode where the device has no cooperative launches).
// Automatic split, in half-steps: kernel boundaries cost less than the tail
// kernel's completion counters and waits while a half-step has much work, and
// larger problems keep real work in later half-steps (more seeds, larger maps,
// slower convergence), so the hand-over moves later with w = pairs x seeds x
// image-2 pixels: after 2 half-steps up to 2^24, 3 up to 2^27, 5 up to 2^31,
// else 8 (the best of 2..8 on each of six measured workloads, 64x48 to
// 16 x 512x384 and 512x512x64).
FrmExec frm_exec(int mode, const FrmPlan &P) {
    if (mode == DDM_FRM_LOOP) return {0, 1};
    if (mode == DDM_FRM_TAIL) {
        const int it = tail_after().load();
        if (it >= 0) return {std::min(P.nhalf, 2 * it), 2};
        const long long w = (long long)P.B * P.k * P.N2;
        const int hs = w <= (1LL << 24) ? 2 : w <= (1LL << 27) ? 3 : w <= (1LL << 31) ? 5 : 8;
        return {std::min(P.nhalf, hs), 2};
    }
    return {P.nhalf, 0};
}

// Half-steps per E (all of them per half-step when E.h_split >= nhalf). The
// whole sequence can be captured into a graph.
int frm_run(const FrmPlan &P, const FrmOpts &O, const void *D1, const void *D2, int32_t *out_i, int32_t *out_j,
            float *out_score, int32_t capacity, int32_t *out_count, int32_t *seed_state, int32_t *query_counts,
            void *ws, hipStream_t s, FrmExec E) {
    unsigned char *w = (unsigned char *)ws;
    const MapFmt &f = P.f;
    const void *m1, *m2, *m1r, *m2r;
    int rc = maybe_repack(f, D1, (long long)P.B * P.N1, w + P.o_r1, s, &m1);
    if (rc) return rc;
    rc = maybe_repack(f, D2, (long long)P.B * P.N2, w + P.o_r2, s, &m2);
    if (rc) return rc;
    m1r = m1; m2r = m2;
    if (f.l2) {
        rc = maybe_repack(f, D1, (long long)P.B * P.N1, w + P.o_r1b, s, &m1r, 1);
        if (rc) return rc;
        rc = maybe_repack(f, D2, (long long)P.B * P.N2, w + P.o_r2b, s, &m2r, 1);
        if (rc) return rc;
    }

    FrmState st;
    st.u = (int32_t *)(w + P.o_u); st.v = (int32_t *)(w + P.o_v); st.conv = (int32_t *)(w + P.o_conv);
    st.score = (float *)(w + P.o_score);
    st.act[0] = (int32_t *)(w + P.o_act0); st.act[1] = (int32_t *)(w + P.o_act1);
    st.qrows[0] = (int32_t *)(w + P.o_qr0); st.qrows[1] = (int32_t *)(w + P.o_qr1);
    st.counts = (int32_t *)(w + P.o_counts);
    st.match_j = (int32_t *)(w + P.o_mj); st.match_s = (float *)(w + P.o_ms);
    st.uprev = (int32_t *)(w + P.o_uprev); st.uiter = (int32_t *)(w + P.o_uiter);
    st.basin = O.basin;
    st.k_bs = P.k_bs; st.cnt_bs = P.cnt_bs; st.n1_bs = P.N1;
    uint64_t *part = (uint64_t *)(w + P.o_part);
    uint32_t *ctl = (uint32_t *)(w + P.o_ctl);
    int32_t *marks = P.explicit_starts ? (int32_t *)(w + P.o_marks) : nullptr;

    // The one-workgroup output reads no dense match array, so unless start marks or a basin map
    // need clearing, the image-1-sized arrays are left alone.
    const bool bitmap_out = P.N1 <= output_bitmap_limit().load() && P.k <= OUT_NT * OUT_SPT;
    const int n1_clear = (bitmap_out && !marks && !O.basin) ? 0 : P.N1;
    // Grid seeds with nothing image-1-sized to clear and a first half-step launched on its own
    // need no init kernel: that sweep derives their pixels and resets the counts and control
    // words, its update writes their initial state.
    const int h_split = std::max(0, std::min(E.h_split, P.nhalf));
    const bool implicit_seeds = !P.explicit_starts && n1_clear == 0 && h_split >= 1 && P.k > 0;
    if (!implicit_seeds) {
        const int init_blocks = (int)std::min<long long>((std::max(P.k, n1_clear) + 255) / 256, 4096);
        hipLaunchKernelGGL(frm_init_kernel, dim3(std::max(init_blocks, 1), P.B), dim3(256), 0, s, st, P.k,
                           std::max(P.kx, 1), P.W1, P.S, n1_clear, P.nhalf, ctl, marks);
        DDM_CHECK_LAUNCH();
    }
    if (P.explicit_starts && P.k > 0) {
        // distinct starts, ascending: marks -> ordered compaction into u / qrows[0], count into counts[0]
        const int mb = (int)std::min<long long>((P.k + 255) / 256, 4096);
        hipLaunchKernelGGL(frm_mark_starts_kernel, dim3(mb), dim3(256), 0, s, O.starts, P.k, P.N1, marks);
        DDM_CHECK_LAUNCH();
        rc = compact_run(marks, st.match_s, P.N1, P.N1, 1, P.nblk, (int32_t *)(w + P.o_bc), (int32_t *)(w + P.o_bo),
                         st.u, st.qrows[0], st.score, P.k, st.counts, s);
        if (rc) return rc;
        hipLaunchKernelGGL(frm_seeds_from_starts_kernel, dim3(mb), dim3(256), 0, s, st, P.k);
        DDM_CHECK_LAUNCH();
    }

    if (P.k > 0) {
        FrmArgs fa{};
        frm_dir_args(P, m1, m1r, m2, m2r, part, 0, &fa.sw[0], &fa.rs[0]);
        frm_dir_args(P, m1, m1r, m2, m2r, part, 1, &fa.sw[1], &fa.rs[1]);
        fa.st = st; fa.B = P.B; fa.nhalf = P.nhalf; fa.k = P.k; fa.qblocks = P.qblocks;
        fa.nch[0] = P.nch2; fa.nch[1] = P.nch1;
        fa.bar = ctl; fa.err = (int32_t *)(ctl + 32); fa.spin_limit = loop_spin_limit().load();
        fa.tail = ctl + 64;
        if (implicit_seeds) fa.g0 = GridSeeds{P.S, std::max(P.kx, 1), P.W1, P.k};
        const long long sweep_tasks = (long long)P.B * P.qblocks * std::max(P.nch1, P.nch2);
        const long long upd_tasks = (long long)P.B * ((P.k + 15) / 16);
        for (int h = 0; h < h_split; ++h) {
            DDM_CHECK(with_events(2, s, [&] { return frm_switch(f, 0, &fa, h, P.loop_lds, sweep_tasks, s, true); }));
            DDM_DT_SWITCH(f.dtype, frm_update_kernel, dim3((unsigned)capped_grid(std::min<long long>(upd_tasks, 2048))),
                          dim3(256), 0, s, fa, h);
            DDM_CHECK_LAUNCH();
        }
        if (h_split < P.nhalf) {
            const int qb = nw_for(f.dtype) * 64 / 16;
            const long long ntask = std::max(sweep_tasks, (long long)P.B * ((P.k + qb - 1) / qb));
            const int which = E.tail == 2 ? 2 : 1;
            DDM_CHECK(with_events(2, s, [&] { return frm_switch(f, which, &fa, h_split, P.loop_lds, ntask, s, true); }));
        }
    }
    if (bitmap_out) {
        // one workgroup per pair: collection and ordered output through an LDS bitmap
        hipLaunchKernelGGL(frm_output_kernel, dim3(P.B), dim3(OUT_NT), (size_t)(P.N1 + 31) / 32 * 8, s, st, P.k,
                           seed_state, (const int32_t *)st.counts, query_counts, P.nhalf, P.W1, O.pixel_tol,
                           P.explicit_starts ? 1 : 0, P.N1, out_i, out_j, out_score, (long long)capacity, capacity,
                           out_count, (const int32_t *)(ctl + 32));
        DDM_CHECK_LAUNCH();
        return DDM_OK;
    }
    const int col_blocks = (int)std::min<long long>((std::max(P.k, 1) + 255) / 256, 4096);
    hipLaunchKernelGGL(frm_collect_kernel, dim3(col_blocks, P.B), dim3(256), 0, s, st, P.k, seed_state,
                       (const int32_t *)st.counts, query_counts, P.nhalf, P.W1, O.pixel_tol,
                       P.explicit_starts ? 1 : 0);
    DDM_CHECK_LAUNCH();
    return compact_run(st.match_j, st.match_s, P.N1, P.N1, P.B, P.nblk, (int32_t *)(w + P.o_bc),
                       (int32_t *)(w + P.o_bo), out_i, out_j, out_score, capacity, out_count, s,
                       (const int32_t *)(ctl + 32));
}

// ------------------------------------------------------ coarse-to-fine plan
struct C2fPlan {
    MapFmt f;
    int H1, W1, H2, W2, d, dtype, factor, Hc1, Wc1, Hc2, Wc2, CH, CW, ntx, nty, ntiles, words;
    int kc, kf, nblk;
    FrmPlan pc, pf;           // coarse FRM (one pair) and fine FRM (one pair per tile)
    size_t o_c1, o_c2, o_cws, o_ci, o_cj, o_cs, o_cc, o_info, o_b1, o_b2, o_fws, o_fi, o_fj, o_fs, o_fc, o_owner,
        o_mj, o_ms, o_bc, o_bo, o_err, total;
    CropGeom geom() const {
        return CropGeom{H1, W1, H2, W2, CH, CW, ntx, nty, factor, Wc1, Wc2};
    }
};

int c2f_plan(int H1, int W1, int H2, int W2, int d, int dtype, int factor, int cs, int cit, int CH, int CW, int fs,
             int fit, C2fPlan *p) {
    if (!pix_ok(H1, W1) || !pix_ok(H2, W2) || factor < 1) return DDM_ERR_INVALID;
    if (CH < 1 || CW < 1 || CH > H1 || CH > H2 || CW > W1 || CW > W2) return DDM_ERR_INVALID;
    if (dtype != DT_F32 && dtype != DT_F16 && dtype != DT_BF16) return DDM_ERR_UNSUPPORTED;
    if (!make_fmt(dtype, d, &p->f)) return DDM_ERR_UNSUPPORTED;
    if ((d * p->f.esz) % 4 != 0) return DDM_ERR_UNSUPPORTED;           // crops move whole 32-bit words
    if ((long long)W2 + H2 + 1 > 16384) return DDM_ERR_UNSUPPORTED;     // median histograms live in LDS
    p->H1 = H1; p->W1 = W1; p->H2 = H2; p->W2 = W2; p->d = d; p->dtype = dtype; p->factor = factor;
    p->Hc1 = (H1 + factor - 1) / factor; p->Wc1 = (W1 + factor - 1) / factor;
    p->Hc2 = (H2 + factor - 1) / factor; p->Wc2 = (W2 + factor - 1) / factor;
    p->CH = CH; p->CW = CW;
    p->nty = (H1 + CH - 1) / CH; p->ntx = (W1 + CW - 1) / CW; p->ntiles = p->nty * p->ntx;
    p->words = d * p->f.esz / 4;
    int rc = frm_plan(1, p->Hc1, p->Wc1, p->Hc2, p->Wc2, d, dtype, cs, cit, &p->pc);
    if (rc) return rc;
    rc = frm_plan(p->ntiles, CH, CW, CH, CW, d, dtype, fs, fit, &p->pf);
    if (rc) return rc;
    p->kc = std::max(p->pc.k, 1); p->kf = std::max(p->pf.k, 1);
    p->nblk = (H1 * W1 + CB - 1) / CB;
    const size_t row = (size_t)d * p->f.esz;
    Bump b;
    p->o_c1 = b.take((size_t)p->Hc1 * p->Wc1 * row);
    p->o_c2 = b.take((size_t)p->Hc2 * p->Wc2 * row);
    p->o_cws = b.take(p->pc.total);
    p->o_ci = b.take((size_t)p->kc * 4); p->o_cj = b.take((size_t)p->kc * 4); p->o_cs = b.take((size_t)p->kc * 4);
    p->o_cc = b.take(4);
    p->o_info = b.take((size_t)p->ntiles * 5 * 4);
    p->o_b1 = b.take((size_t)p->ntiles * CH * CW * row);
    p->o_b2 = b.take((size_t)p->ntiles * CH * CW * row);
    p->o_fws = b.take(p->pf.total);
    const size_t nf = (size_t)p->ntiles * p->kf;
    p->o_fi = b.take(nf * 4); p->o_fj = b.take(nf * 4); p->o_fs = b.take(nf * 4);
    p->o_fc = b.take((size_t)p->ntiles * 4);
    const size_t n1 = (size_t)H1 * W1;
    p->o_owner = b.take(n1 * 4); p->o_mj = b.take(n1 * 4); p->o_ms = b.take(n1 * 4);
    p->o_bc = b.take((size_t)p->nblk * 4); p->o_bo = b.take((size_t)p->nblk * 4);
    p->o_err = b.take(4);
    p->total = b.off;
    return DDM_OK;
}

int c2f_run(const C2fPlan &P, const void *F1, const void *F2, int32_t *out_i, int32_t *out_j, float *out_score,
            int32_t capacity, int32_t *out_count, int32_t *crop_info, void *ws, hipStream_t s, int mode) {
    unsigned char *w = (unsigned char *)ws;
    const CropGeom g = P.geom();
    // coarse maps and coarse FRM
    const long long nc1 = (long long)P.Hc1 * P.Wc1 * P.words, nc2 = (long long)P.Hc2 * P.Wc2 * P.words;
    hipLaunchKernelGGL(subsample_kernel, dim3((int)std::min<long long>((nc1 + 255) / 256, 4096)), dim3(256), 0, s,
                       (const uint32_t *)F1, P.W1, P.words, P.factor, P.Hc1, P.Wc1, (uint32_t *)(w + P.o_c1));
    DDM_CHECK_LAUNCH();
    hipLaunchKernelGGL(subsample_kernel, dim3((int)std::min<long long>((nc2 + 255) / 256, 4096)), dim3(256), 0, s,
                       (const uint32_t *)F2, P.W2, P.words, P.factor, P.Hc2, P.Wc2, (uint32_t *)(w + P.o_c2));
    DDM_CHECK_LAUNCH();
    int32_t *ci = (int32_t *)(w + P.o_ci), *cj = (int32_t *)(w + P.o_cj), *cc = (int32_t *)(w + P.o_cc);
    int rc = frm_run(P.pc, FrmOpts{}, w + P.o_c1, w + P.o_c2, ci, cj, (float *)(w + P.o_cs), P.kc, cc, nullptr,
                     nullptr, w + P.o_cws, s, frm_exec(mode, P.pc));
    if (rc) return rc;
    // crop windows, crop batches, fine FRM
    int32_t *info = crop_info ? crop_info : (int32_t *)(w + P.o_info);
    const size_t hist = (size_t)(P.W2 + P.H2 + 1) * sizeof(int);
    hipLaunchKernelGGL(crop_stats_kernel, dim3(P.ntiles), dim3(256), hist, s, (const int32_t *)ci,
                       (const int32_t *)cj, (const int32_t *)cc, g, info);
    DDM_CHECK_LAUNCH();
    const long long per = (long long)P.CH * P.CW * P.words;
    hipLaunchKernelGGL(crop_gather_kernel, dim3((int)std::min<long long>((per + 255) / 256, 2048), P.ntiles),
                       dim3(256), 0, s, (const uint32_t *)F1, (const uint32_t *)F2, P.words, g,
                       (const int32_t *)info, (uint32_t *)(w + P.o_b1), (uint32_t *)(w + P.o_b2));
    DDM_CHECK_LAUNCH();
    int32_t *fi = (int32_t *)(w + P.o_fi), *fj = (int32_t *)(w + P.o_fj), *fc = (int32_t *)(w + P.o_fc);
    float *fsc = (float *)(w + P.o_fs);
    rc = frm_run(P.pf, FrmOpts{}, w + P.o_b1, w + P.o_b2, fi, fj, fsc, P.kf, fc, nullptr, nullptr, w + P.o_fws, s,
                 frm_exec(mode, P.pf));
    if (rc) return rc;
    // merge into full resolution, first tile wins, ordered output
    const int n1 = P.H1 * P.W1;
    int32_t *owner = (int32_t *)(w + P.o_owner), *mj = (int32_t *)(w + P.o_mj);
    float *ms = (float *)(w + P.o_ms);
    hipLaunchKernelGGL(c2f_clear_kernel, dim3(std::min((n1 + 255) / 256, 4096)), dim3(256), 0, s, owner, mj, n1);
    DDM_CHECK_LAUNCH();
    const dim3 mg((unsigned)std::min((P.kf + 255) / 256, 1024), (unsigned)P.ntiles);
    hipLaunchKernelGGL(crop_owner_kernel, mg, dim3(256), 0, s, (const int32_t *)fi, (const int32_t *)fc, P.kf, g,
                       (const int32_t *)info, owner);
    DDM_CHECK_LAUNCH();
    hipLaunchKernelGGL(crop_write_kernel, mg, dim3(256), 0, s, (const int32_t *)fi, (const int32_t *)fj,
                       (const float *)fsc, (const int32_t *)fc, P.kf, g, (const int32_t *)info,
                       (const int32_t *)owner, mj, ms);
    DDM_CHECK_LAUNCH();
    int32_t *err = (int32_t *)(w + P.o_err);
    hipLaunchKernelGGL(c2f_status_kernel, dim3(1), dim3(256), 0, s, (const int32_t *)cc, (const int32_t *)fc,
                       P.ntiles, err);
    DDM_CHECK_LAUNCH();
    return compact_run(mj, ms, n1, n1, 1, P.nblk, (int32_t *)(w + P.o_bc), (int32_t *)(w + P.o_bo), out_i, out_j,
                       out_score, capacity, out_count, s, (const int32_t *)err);
}

// -------------------------------------------------------------- mutual plan
struct MutualPlan {
    MapFmt f;
    int N1, N2, chunk, nchunks, sb_per_wg, qblocks, nblk;
    size_t o_rowkey, o_colkey, o_owner, o_mj, o_ms, o_bc, o_bo, o_r1, o_r2, total;
};

int mutual_plan(int H1, int W1, int H2, int W2, int d, int dtype, MutualPlan *p, int metric = DDM_DOT) {
    if (!pix_ok(H1, W1) || !pix_ok(H2, W2)) return DDM_ERR_INVALID;
    if (dtype != DT_F32 && dtype != DT_F16 && dtype != DT_BF16) return DDM_ERR_UNSUPPORTED;
    if (!make_fmt(dtype, d, &p->f, metric)) return DDM_ERR_UNSUPPORTED;
    p->N1 = H1 * W1; p->N2 = H2 * W2;
    const int sbr = p->f.sb_rows();
    const int nsb = (p->N1 + sbr - 1) / sbr;
    int chunk = chunk_limit(p->f, true);
    // at least ~2 workgroups per CU along the chunk axis alone when the map is small
    while (chunk > p->f.group() && (long long)nsb * ((p->N2 + chunk - 1) / chunk) < 512) chunk -= p->f.group();
    p->chunk = chunk;
    p->nchunks = (p->N2 + chunk - 1) / chunk;
    // query sub-blocks per workgroup: aim at ~512 workgroups (two rounds of one workgroup per CU). Longer
    // workgroups merge fewer column keys (one atomic per column and query block) and spread the last unit's
    // tail over more work; sweep at 512x384 on one machine: 4 query blocks 2.065 ms, 8 2.07-2.08, 64 2.23,
    // 256 2.57
    const long long want_qblocks = std::max<long long>(1, 512 / p->nchunks);
    p->sb_per_wg = (int)std::max<long long>(1, (nsb + want_qblocks - 1) / want_qblocks);
    p->qblocks = (nsb + p->sb_per_wg - 1) / p->sb_per_wg;
    p->nblk = (p->N1 + CB - 1) / CB;
    Bump b;
    p->o_rowkey = b.take((size_t)p->N1 * 8);
    p->o_colkey = b.take((size_t)p->N2 * 8);
    p->o_owner = b.take((size_t)p->N2 * 4);
    p->o_mj = b.take((size_t)p->N1 * 4);
    p->o_ms = b.take((size_t)p->N1 * 4);
    p->o_bc = b.take((size_t)p->nblk * 4);
    p->o_bo = b.take((size_t)p->nblk * 4);
    p->o_r1 = p->f.repack ? b.take((size_t)p->N1 * p->f.ld * p->f.esz) : 0;
    p->o_r2 = p->f.repack ? b.take((size_t)p->N2 * p->f.ld * p->f.esz) : 0;
    p->total = b.off;
    return DDM_OK;
}

// ------------------------------------------------------------- FRM mode
std::atomic<int> &frm_mode() { static std::atomic<int> m{DDM_FRM_TAIL}; return m; }

bool cooperative_ok(int dev) {
    static std::mutex mu;
    static std::vector<int> known;      // per device: 0 unknown, 1 yes, 2 no
    std::lock_guard<std::mutex> g(mu);
    if ((int)known.size() <= dev) known.resize(dev + 1, 0);
    if (known[dev] == 0) {
        int v = 0;
        known[dev] = (hipDeviceGetAttribute(&v, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess && v) ? 1 : 2;
    }
    return known[dev] == 1;
}

// The process-wide mode as it applies on device dev.
int effective_mode(int dev) {
    const int m = frm_mode().load();
    return (m == DDM_FRM_LOOP && !cooperative_ok(dev)) ? DDM_FRM_PER_HALF_STEP : m;
}

// ---------------------------------------------------------- graph replay
// An FRM call is up to ~4*max_iter small launches whose host-side enqueue cost
// exceeds their GPU time once the active set has shrunk. The sequence depends
// only on the call's arguments, so it is captured once into a HIP graph on a
// private capture stream, instantiated, cached (a few entries, most recently
// used first) and replayed on the caller's stream with a single launch. An
// event recorded after every replay tells when the last replay of an entry has
// finished, so an entry is destroyed (on eviction or release) only once its
// work is done. The cache owns these objects; ddm_release_cached_resources
// destroys them, which must happen before the HIP runtime shuts down.
using GraphKey = std::array<uint64_t, 28>;

struct GraphEntry {
    GraphKey key;
    hipGraphExec_t exec;
    hipEvent_t done;      // recorded on the caller's stream after each replay
};

struct GraphCache {
    std::mutex mu;
    std::list<GraphEntry> lru;
    std::vector<hipStream_t> cap;     // per device: private capture stream (default priority)
    static constexpr size_t kMax = 8;
};
GraphCache &graphs() { static GraphCache g; return g; }

// Wait for the entry's last replay, then destroy its objects (on the entry's device).
hipError_t destroy_entry(GraphEntry &e) {
    int cur = 0;
    hipError_t st = hipGetDevice(&cur);
    const int dev = (int)e.key[0];
    if (st == hipSuccess && dev != cur) st = hipSetDevice(dev);
    auto keep = [&](hipError_t x) { if (st == hipSuccess) st = x; };
    if (e.done) { keep(hipEventSynchronize(e.done)); keep(hipEventDestroy(e.done)); }
    if (e.exec) keep(hipGraphExecDestroy(e.exec));
    e.done = nullptr; e.exec = nullptr;
    if (dev != cur) keep(hipSetDevice(cur));
    return st;
}

int replay(GraphEntry &e, hipStream_t stream) {
    if (hipGraphLaunch(e.exec, stream) != hipSuccess) return DDM_ERR_HIP;
    return hipEventRecord(e.done, stream) == hipSuccess ? DDM_OK : DDM_ERR_HIP;
}

template <class Enqueue>
int run_graphed(const GraphKey &key, hipStream_t stream, Enqueue enqueue) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return DDM_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone || (prof().mask & 2)) return enqueue(stream);   // direct launches
    GraphCache &G = graphs();
    std::lock_guard<std::mutex> lock(G.mu);
    for (auto it = G.lru.begin(); it != G.lru.end(); ++it) {
        if (it->key == key) {
            G.lru.splice(G.lru.begin(), G.lru, it);
            return replay(G.lru.front(), stream);
        }
    }
    const int dev = (int)key[0];
    if ((int)G.cap.size() <= dev) G.cap.resize(dev + 1, nullptr);
    hipStream_t &cap = G.cap[dev];
    if (!cap && hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess) return DDM_ERR_HIP;
    if (hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal) != hipSuccess) return DDM_ERR_HIP;
    const int rc = enqueue(cap);
    hipGraph_t graph = nullptr;
    const hipError_t ec = hipStreamEndCapture(cap, &graph);
    if (rc != DDM_OK || ec != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc != DDM_OK ? rc : DDM_ERR_HIP;
    }
    GraphEntry e{key, nullptr, nullptr};
    const hipError_t ei = hipGraphInstantiate(&e.exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) return DDM_ERR_HIP;
    if (hipEventCreateWithFlags(&e.done, hipEventDisableTiming) != hipSuccess) {
        e.done = nullptr;
        (void)destroy_entry(e);
        return DDM_ERR_HIP;
    }
    if (G.lru.size() >= GraphCache::kMax) {
        const hipError_t ed = destroy_entry(G.lru.back());
        G.lru.pop_back();
        if (ed != hipSuccess) { (void)destroy_entry(e); return DDM_ERR_HIP; }
    }
    G.lru.push_front(e);
    return replay(G.lru.front(), stream);
}

// Destroy every cached graph, capture stream and timing event (the library
// recreates them on demand).
int release_cached() {
    int rc = DDM_OK;
    {
        GraphCache &G = graphs();
        std::lock_guard<std::mutex> lock(G.mu);
        for (GraphEntry &e : G.lru)
            if (destroy_entry(e) != hipSuccess) rc = DDM_ERR_HIP;
        G.lru.clear();
        // HIP is only called for objects that exist (a process that never launched makes no call)
        const bool any_stream = std::any_of(G.cap.begin(), G.cap.end(), [](hipStream_t x) { return x != nullptr; });
        if (any_stream) {
            int cur = 0;
            if (hipGetDevice(&cur) != hipSuccess) rc = DDM_ERR_HIP;
            for (size_t dev = 0; dev < G.cap.size(); ++dev) {
                if (!G.cap[dev]) continue;
                if (hipSetDevice((int)dev) != hipSuccess || hipStreamSynchronize(G.cap[dev]) != hipSuccess ||
                    hipStreamDestroy(G.cap[dev]) != hipSuccess)
                    rc = DDM_ERR_HIP;
                G.cap[dev] = nullptr;
            }
            if (hipSetDevice(cur) != hipSuccess) rc = DDM_ERR_HIP;
        }
    }
    Profiler &P = prof();
    std::lock_guard<std::mutex> g(P.mu);
    for (auto *v : {&P.pending, &P.pool}) {
        for (auto &ev : *v) {
            if (hipEventSynchronize(ev.second) != hipSuccess || hipEventDestroy(ev.first) != hipSuccess ||
                hipEventDestroy(ev.second) != hipSuccess)
                rc = DDM_ERR_HIP;
        }
        v->clear();
    }
    return rc;
}

}  // namespace

// ===================================================================== C ABI
extern "C" {

const char *ddm_status_str(int status) {
    switch (status) {
    case DDM_OK: return "ok";
    case DDM_ERR_INVALID: return "invalid argument";
    case DDM_ERR_CAPACITY: return "output capacity too small";
    case DDM_ERR_WORKSPACE: return "workspace missing or too small";
    case DDM_ERR_UNSUPPORTED: return "unsupported dtype or descriptor dimension";
    case DDM_ERR_HIP: return "HIP error while enqueueing";
    default: return "unknown status";
    }
}

int64_t ddm_seed_count(int H, int W, int grid_stride) { return seed_count(H, W, grid_stride); }

int ddm_frm_stats(const int32_t *qc, int B, int max_iter, int64_t N1, int64_t N2, ddm_stats *stats) {
    if (!qc || !stats || B < 1 || max_iter < 1 || max_iter > DDM_MAX_ITER || N1 < 0 || N2 < 0)
        return DDM_ERR_INVALID;
    for (int b = 0; b < B; ++b) {
        const int32_t *c = qc + (size_t)b * 2 * max_iter;
        for (int h = 0; h < 2 * max_iter; ++h)
            if (c[h] < 0) return DDM_ERR_INVALID;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t *c = qc + (size_t)b * 2 * max_iter;
        ddm_stats &st = stats[b];
        std::memset(&st, 0, sizeof(st));
        for (int t = 0; t < max_iter; ++t) {
            st.active[2 * t] = c[2 * t];
            st.active[2 * t + 1] = c[2 * t + 1];
            if (c[2 * t] > 0) st.iters = t + 1;
            st.dot_products += (int64_t)c[2 * t] * N2 + (int64_t)c[2 * t + 1] * N1;
        }
    }
    return DDM_OK;
}

int ddm_frm_set_mode(int mode) {
    if (mode != DDM_FRM_PER_HALF_STEP && mode != DDM_FRM_LOOP && mode != DDM_FRM_TAIL) return DDM_ERR_INVALID;
    frm_mode().store(mode);
    return DDM_OK;
}

int ddm_frm_set_tail_after(int iterations) {
    if (iterations < -1 || iterations > DDM_MAX_ITER) return DDM_ERR_INVALID;
    tail_after().store(iterations);
    return DDM_OK;
}

int ddm_frm_get_mode(void) { return frm_mode().load(); }

int ddm_debug_set_output_bitmap_limit(int max_pixels) {
    if (max_pixels < -1) return DDM_ERR_INVALID;
    output_bitmap_limit().store(max_pixels < 0 ? OUT_MAX_PIXELS : std::min(max_pixels, OUT_MAX_PIXELS));
    return DDM_OK;
}

int ddm_debug_set_grid_cap(int max_workgroups) {
    if (max_workgroups < 0) return DDM_ERR_INVALID;
    frm_grid_cap().store(max_workgroups);
    return DDM_OK;
}

int ddm_frm_set_barrier_polls(int polls) {
    if (polls < 0) return DDM_ERR_INVALID;
    loop_spin_limit().store(polls == 0 ? kSpinLimit : polls);
    return DDM_OK;
}

int ddm_release_cached_resources(void) { return release_cached(); }

int ddm_profile_enable(int mask) {
    if (mask < 0 || mask > 3) return DDM_ERR_INVALID;
    std::lock_guard<std::mutex> g(prof().mu);
    prof().mask = mask;
    return DDM_OK;
}

int ddm_profile_read(double *total_ms, int64_t *launches) {
    if (!total_ms || !launches) return DDM_ERR_INVALID;
    Profiler &P = prof();
    std::lock_guard<std::mutex> g(P.mu);
    double sum = 0.0;
    int64_t n = 0;
    int rc = DDM_OK;
    for (auto &ev : P.pending) {
        float ms = 0.f;
        if (hipEventSynchronize(ev.second) != hipSuccess || hipEventElapsedTime(&ms, ev.first, ev.second) != hipSuccess)
            rc = DDM_ERR_HIP;
        sum += ms; ++n;
        P.pool.push_back(ev);
    }
    P.pending.clear();
    *total_ms = sum; *launches = n;
    return rc;
}

}  // extern "C"

extern "C" {

size_t ddm_nn_ex_workspace_bytes(int NQ, int M, int N, int d, int dtype, int metric) {
    NnPlan P;
    return nn_plan(NQ, M, N, d, dtype, &P, metric) == DDM_OK ? P.total : 0;
}

size_t ddm_nn_workspace_bytes(int NQ, int M, int N, int d, int dtype) {
    return ddm_nn_ex_workspace_bytes(NQ, M, N, d, dtype, DDM_DOT);
}

int ddm_nn_ex(const void *Q, int NQ, const int32_t *q_rows, int M, const void *R, int N, int d, int dtype,
              int metric, int32_t *out_idx, float *out_score, void *workspace, size_t workspace_bytes,
              hipStream_t stream) {
    NnPlan P;
    int rc = nn_plan(NQ, M, N, d, dtype, &P, metric);
    if (rc) return rc;
    if (!map_ok(Q, P.f) || !map_ok(R, P.f) || !out_idx || !out_score) return DDM_ERR_INVALID;
    if (!q_rows && NQ < M) return DDM_ERR_INVALID;
    if (!workspace || workspace_bytes < P.total) return DDM_ERR_WORKSPACE;
    if (prepare_kernels() != hipSuccess) return DDM_ERR_HIP;
    unsigned char *w = (unsigned char *)workspace;
    const void *q, *r;
    rc = maybe_repack(P.f, Q, NQ, w + P.o_rq, stream, &q);
    if (rc) return rc;
    rc = maybe_repack(P.f, R, N, w + P.o_rr, stream, &r, 1);
    if (rc) return rc;
    const int32_t *rows = nullptr;          // the caller's list with out-of-map entries replaced
    if (q_rows) {
        int32_t *safe = (int32_t *)(w + P.o_rows);
        hipLaunchKernelGGL(nn_rows_kernel, dim3(std::min((M + 255) / 256, 4096)), dim3(256), 0, stream, q_rows, M, NQ,
                           safe);
        DDM_CHECK_LAUNCH();
        rows = safe;
    }
    SweepArgs a{};
    a.Q = (const unsigned char *)q; a.R = (const unsigned char *)r; a.qrows = rows;
    a.rowpart = (uint64_t *)(w + P.o_part);
    a.nq = M; a.nref = N; a.ld = P.f.ld; a.chunk = P.chunk; a.nchunks = P.nchunks; a.sb_per_wg = 1;
    a.rowcap = M;
    DDM_CHECK(launch_sweep(P.f, false, a, dim3(P.nchunks, P.qblocks, 1), stream));
    ResolveArgs ra{};
    ra.rowpart = a.rowpart; ra.nchunks = P.nchunks; ra.rowcap = M;
    ra.Q = a.Q; ra.qrows = rows; ra.nq = M; ra.R = a.R; ra.nref = N; ra.ld = P.f.ld; ra.d = P.f.d;
    ra.neg_out = P.f.l2 ? 1 : 0;
    const int qb = resolve_qb(M);
    DDM_DT_QB_SWITCH(P.f.dtype, qb, nn_resolve_kernel, dim3((M + qb - 1) / qb), dim3(256), 0, stream, ra, q_rows,
                     NQ, out_idx, out_score);
    DDM_CHECK_LAUNCH();
    return DDM_OK;
}

int ddm_nn(const void *Q, int NQ, const int32_t *q_rows, int M, const void *R, int N, int d, int dtype,
           int32_t *out_idx, float *out_score, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return ddm_nn_ex(Q, NQ, q_rows, M, R, N, d, dtype, DDM_DOT, out_idx, out_score, workspace, workspace_bytes,
                     stream);
}

size_t ddm_frm_workspace_bytes(int B, int H1, int W1, int H2, int W2, int d, int dtype, int grid_stride,
                               int max_iter) {
    FrmPlan P;
    return frm_plan(B, H1, W1, H2, W2, d, dtype, grid_stride, max_iter, &P) == DDM_OK ? P.total : 0;
}

static int frm_entry(int B, const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype,
                     int metric, int grid_stride, int max_iter, const FrmOpts &O, int32_t *out_i, int32_t *out_j,
                     float *out_score, int32_t capacity, int32_t *out_count, int32_t *seed_state,
                     int32_t *query_counts, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    FrmPlan P;
    if (O.starts && O.n_starts < 0) return DDM_ERR_INVALID;
    if (!O.starts && O.n_starts != 0) return DDM_ERR_INVALID;
    {
        // finite and not negative, decided on the bits (NaN and infinities have an all-ones exponent)
        uint64_t b;
        std::memcpy(&b, &O.pixel_tol, sizeof(b));
        if (((b >> 52) & 0x7ff) == 0x7ff || ((b >> 63) && (b << 1) != 0)) return DDM_ERR_INVALID;
    }
    if (O.pixel_tol > 0.0 && !O.starts) return DDM_ERR_INVALID;       // the routine has no grid form of it
    int rc = frm_plan(B, H1, W1, H2, W2, d, dtype, grid_stride, max_iter, &P, O.starts ? O.n_starts : -1, metric);
    if (rc) return rc;
    if (!map_ok(D1, P.f) || !map_ok(D2, P.f)) return DDM_ERR_INVALID;
    if (!out_i || !out_j || !out_score || !out_count) return DDM_ERR_INVALID;
    if (capacity < P.k) return DDM_ERR_CAPACITY;
    if (!workspace || workspace_bytes < P.total) return DDM_ERR_WORKSPACE;
    if (prepare_kernels() != hipSuccess) return DDM_ERR_HIP;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DDM_ERR_HIP;
    uint64_t tol_bits;
    std::memcpy(&tol_bits, &O.pixel_tol, sizeof(tol_bits));
    const FrmExec E = frm_exec(effective_mode(dev), P);
    const GraphKey key = {(uint64_t)dev, (uint64_t)B, (uint64_t)(uintptr_t)D1, (uint64_t)H1, (uint64_t)W1,
                          (uint64_t)(uintptr_t)D2, (uint64_t)H2, (uint64_t)W2, (uint64_t)d, (uint64_t)dtype,
                          (uint64_t)grid_stride, (uint64_t)max_iter, (uint64_t)(uintptr_t)out_i,
                          (uint64_t)(uintptr_t)out_j, (uint64_t)(uintptr_t)out_score, (uint64_t)capacity,
                          (uint64_t)(uintptr_t)out_count, (uint64_t)(uintptr_t)seed_state,
                          (uint64_t)(uintptr_t)query_counts, (uint64_t)(uintptr_t)workspace,
                          (uint64_t)(uint32_t)E.h_split | ((uint64_t)E.tail << 32),
                          (uint64_t)(uintptr_t)O.starts, (uint64_t)(uint32_t)O.n_starts, tol_bits,
                          (uint64_t)(uintptr_t)O.basin, (uint64_t)metric,
                          (uint64_t)(E.h_split < P.nhalf ? loop_spin_limit().load() : 0),
                          (uint64_t)(uint32_t)frm_grid_cap().load() |
                              ((uint64_t)(uint32_t)output_bitmap_limit().load() << 32)};
    return run_graphed(key, stream, [&](hipStream_t s) {
        return frm_run(P, O, D1, D2, out_i, out_j, out_score, capacity, out_count, seed_state, query_counts,
                       workspace, s, E);
    });
}

int ddm_frm_match(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype,
                  int grid_stride, int max_iter, int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity,
                  int32_t *out_count, int32_t *seed_state, int32_t *query_counts, void *workspace,
                  size_t workspace_bytes, hipStream_t stream) {
    return frm_entry(1, D1, H1, W1, D2, H2, W2, d, dtype, DDM_DOT, grid_stride, max_iter, FrmOpts{}, out_i, out_j,
                     out_score,
                     capacity, out_count, seed_state, query_counts, workspace, workspace_bytes, stream);
}

int ddm_frm_match_noalloc(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype,
                          int grid_stride, int max_iter, int32_t *out_i, int32_t *out_j, float *out_score,
                          int32_t capacity, int32_t *out_count, int32_t *seed_state, int32_t *query_counts,
                          hipStream_t stream) {
    FrmPlan P;
    int rc = frm_plan(1, H1, W1, H2, W2, d, dtype, grid_stride, max_iter, &P);
    if (rc) return rc;
    if (!map_ok(D1, P.f) || !map_ok(D2, P.f)) return DDM_ERR_INVALID;
    if (!out_i || !out_j || !out_score || !out_count) return DDM_ERR_INVALID;
    if (capacity < P.k) return DDM_ERR_CAPACITY;
    if (P.total > (size_t)DDM_NOALLOC_SCRATCH_BYTES) return DDM_ERR_WORKSPACE;   // before any HIP call
    if (prepare_kernels() != hipSuccess) return DDM_ERR_HIP;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DDM_ERR_HIP;
    void *ws = nullptr;
    rc = scratch_ptr(dev, &ws);
    if (rc) return rc;
    // direct launches (no graph is instantiated), no timing events, no cooperative launch: the loop
    // mode runs as the tail mode, which gives the same bits
    const int mode = effective_mode(dev) == DDM_FRM_LOOP ? DDM_FRM_TAIL : effective_mode(dev);
    t_no_events = true;
    rc = frm_run(P, FrmOpts{}, D1, D2, out_i, out_j, out_score, capacity, out_count, seed_state, query_counts, ws,
                 stream, frm_exec(mode, P));
    t_no_events = false;
    return rc;
}

int ddm_frm_match_batched(int B, const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype,
                          int grid_stride, int max_iter, int32_t *out_i, int32_t *out_j, float *out_score,
                          int32_t capacity, int32_t *out_count, int32_t *seed_state, int32_t *query_counts,
                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return frm_entry(B, D1, H1, W1, D2, H2, W2, d, dtype, DDM_DOT, grid_stride, max_iter, FrmOpts{}, out_i, out_j,
                     out_score,
                     capacity, out_count, seed_state, query_counts, workspace, workspace_bytes, stream);
}

size_t ddm_frm_ex_workspace_bytes(int H1, int W1, int H2, int W2, int d, int dtype, int metric, int grid_stride,
                                  int n_starts, int max_iter) {
    FrmPlan P;
    return frm_plan(1, H1, W1, H2, W2, d, dtype, grid_stride, max_iter, &P, n_starts < 0 ? -1 : n_starts,
                    metric) == DDM_OK
               ? P.total
               : 0;
}

int ddm_frm_match_ex(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype, int metric,
                     int grid_stride, const int32_t *starts, int n_starts, int max_iter, double pixel_tol,
                     int32_t *basin, int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity,
                     int32_t *out_count, int32_t *seed_state, int32_t *query_counts, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    FrmOpts O;
    O.starts = starts; O.n_starts = starts ? n_starts : 0; O.pixel_tol = pixel_tol; O.basin = basin;
    if (!starts && n_starts > 0) return DDM_ERR_INVALID;
    return frm_entry(1, D1, H1, W1, D2, H2, W2, d, dtype, metric, grid_stride, max_iter, O, out_i, out_j, out_score,
                     capacity, out_count, seed_state, query_counts, workspace, workspace_bytes, stream);
}

size_t ddm_c2f_workspace_bytes(int H1, int W1, int H2, int W2, int d, int dtype, int factor, int coarse_stride,
                               int coarse_iter, int crop_h, int crop_w, int fine_stride, int fine_iter) {
    C2fPlan P;
    return c2f_plan(H1, W1, H2, W2, d, dtype, factor, coarse_stride, coarse_iter, crop_h, crop_w, fine_stride,
                    fine_iter, &P) == DDM_OK
               ? P.total
               : 0;
}

int ddm_c2f_match(const void *F1, int H1, int W1, const void *F2, int H2, int W2, int d, int dtype, int factor,
                  int coarse_stride, int coarse_iter, int crop_h, int crop_w, int fine_stride, int fine_iter,
                  int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity, int32_t *out_count,
                  int32_t *crop_info, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    C2fPlan P;
    int rc = c2f_plan(H1, W1, H2, W2, d, dtype, factor, coarse_stride, coarse_iter, crop_h, crop_w, fine_stride,
                      fine_iter, &P);
    if (rc) return rc;
    if (!map_ok(F1, P.f) || !map_ok(F2, P.f) || ((uintptr_t)F1 | (uintptr_t)F2) % 4 != 0) return DDM_ERR_INVALID;
    if (!out_i || !out_j || !out_score || !out_count) return DDM_ERR_INVALID;
    if ((long long)capacity < std::min<long long>((long long)H1 * W1, (long long)P.ntiles * P.pf.k))
        return DDM_ERR_CAPACITY;
    if (!workspace || workspace_bytes < P.total) return DDM_ERR_WORKSPACE;
    if (prepare_kernels() != hipSuccess) return DDM_ERR_HIP;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DDM_ERR_HIP;
    const int mode = effective_mode(dev);
    const GraphKey key = {(uint64_t)dev, 0xC2F, (uint64_t)(uintptr_t)F1, (uint64_t)H1, (uint64_t)W1,
                          (uint64_t)(uintptr_t)F2, (uint64_t)H2, (uint64_t)W2, (uint64_t)d, (uint64_t)dtype,
                          (uint64_t)factor, (uint64_t)coarse_stride, (uint64_t)coarse_iter, (uint64_t)crop_h,
                          (uint64_t)crop_w, (uint64_t)fine_stride, (uint64_t)fine_iter, (uint64_t)(uintptr_t)out_i,
                          (uint64_t)(uintptr_t)out_j, (uint64_t)(uintptr_t)out_score, (uint64_t)capacity,
                          (uint64_t)(uintptr_t)out_count, (uint64_t)(uintptr_t)crop_info,
                          (uint64_t)(uintptr_t)workspace, (uint64_t)mode | ((uint64_t)(uint32_t)(tail_after().load() + 1) << 8),
                          (uint64_t)(mode != DDM_FRM_PER_HALF_STEP ? loop_spin_limit().load() : 0),
                          (uint64_t)(uint32_t)frm_grid_cap().load() |
                              ((uint64_t)(uint32_t)output_bitmap_limit().load() << 32)};
    return run_graphed(key, stream, [&](hipStream_t s) {
        return c2f_run(P, F1, F2, out_i, out_j, out_score, capacity, out_count, crop_info, workspace, s, mode);
    });
}

size_t ddm_mutual_ex_workspace_bytes(int H1, int W1, int H2, int W2, int d, int dtype, int metric) {
    MutualPlan P;
    return mutual_plan(H1, W1, H2, W2, d, dtype, &P, metric) == DDM_OK ? P.total : 0;
}

size_t ddm_mutual_workspace_bytes(int H1, int W1, int H2, int W2, int d, int dtype) {
    return ddm_mutual_ex_workspace_bytes(H1, W1, H2, W2, d, dtype, DDM_DOT);
}

int ddm_mutual_nn_ex(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype, int metric,
                     int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity, int32_t *out_count,
                     int32_t *nn12, float *s12, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    MutualPlan P;
    int rc = mutual_plan(H1, W1, H2, W2, d, dtype, &P, metric);
    if (rc) return rc;
    if (!map_ok(D1, P.f) || !map_ok(D2, P.f)) return DDM_ERR_INVALID;
    if (!out_i || !out_j || !out_score || !out_count) return DDM_ERR_INVALID;
    if ((nn12 == nullptr) != (s12 == nullptr)) return DDM_ERR_INVALID;
    if (capacity < std::min(P.N1, P.N2)) return DDM_ERR_CAPACITY;
    if (!workspace || workspace_bytes < P.total) return DDM_ERR_WORKSPACE;
    if (prepare_kernels() != hipSuccess) return DDM_ERR_HIP;
    unsigned char *w = (unsigned char *)workspace;
    const void *m1, *m2;
    rc = maybe_repack(P.f, D1, P.N1, w + P.o_r1, stream, &m1);
    if (rc) return rc;
    rc = maybe_repack(P.f, D2, P.N2, w + P.o_r2, stream, &m2, 1);
    if (rc) return rc;
    uint64_t *rowkey = (uint64_t *)(w + P.o_rowkey), *colkey = (uint64_t *)(w + P.o_colkey);
    int32_t *owner = (int32_t *)(w + P.o_owner);
    hipLaunchKernelGGL(mutual_init_kernel, dim3((int)std::min<long long>((std::max(P.N1, P.N2) + 255) / 256, 2048)),
                       dim3(256), 0, stream, rowkey, P.N1, colkey, owner, P.N2);
    DDM_CHECK_LAUNCH();
    SweepArgs a{};
    a.Q = (const unsigned char *)m1; a.R = (const unsigned char *)m2;
    a.rowpart = rowkey;
    a.colkey = colkey;
    a.nq = P.N1; a.nref = P.N2; a.ld = P.f.ld; a.chunk = P.chunk; a.nchunks = P.nchunks;
    a.sb_per_wg = P.sb_per_wg; a.rowcap = P.N1;
    DDM_CHECK(launch_sweep(P.f, true, a, dim3(P.nchunks, P.qblocks, 1), stream));
    ResolveArgs ra{};
    ra.rowpart = rowkey; ra.nchunks = 1; ra.rowcap = P.N1;
    ra.Q = a.Q; ra.nq = P.N1; ra.R = a.R; ra.nref = P.N2; ra.ld = P.f.ld; ra.d = P.f.d;
    ra.neg_out = P.f.l2 ? 1 : 0;
    int32_t *mj = (int32_t *)(w + P.o_mj);
    float *ms = (float *)(w + P.o_ms);
    const int qb = resolve_qb(P.N1);
    DDM_DT_QB_SWITCH(P.f.dtype, qb, mutual_rows_kernel, dim3((P.N1 + qb - 1) / qb), dim3(256), 0, stream, ra,
                     (const uint64_t *)colkey, P.sb_per_wg * P.f.sb_rows(), owner, mj, ms, nn12, s12);
    DDM_CHECK_LAUNCH();
    // rows that lost their column's claim to a lower row drop out in the compaction
    return compact_run(mj, ms, P.N1, P.N1, 1, P.nblk, (int32_t *)(w + P.o_bc), (int32_t *)(w + P.o_bo), out_i, out_j,
                       out_score, capacity, out_count, stream, nullptr, (const int32_t *)owner);
}

int ddm_mutual_nn(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype, int32_t *out_i,
                  int32_t *out_j, float *out_score, int32_t capacity, int32_t *out_count, int32_t *nn12, float *s12,
                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return ddm_mutual_nn_ex(D1, H1, W1, D2, H2, W2, d, dtype, DDM_DOT, out_i, out_j, out_score, capacity, out_count,
                            nn12, s12, workspace, workspace_bytes, stream);
}

}  // extern "C"
