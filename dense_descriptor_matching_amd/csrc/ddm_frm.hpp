// ddm_frm.hpp -- the FRM iteration: sweep and update phases, run as one pair
// of launches per half-step, as one cooperative loop kernel, or per half-step
// for the first iterations and then as one tail kernel.
//
// Both phases enumerate only the active work of every pair (query blocks with
// queries, times sub-chunks of the runtime split; query blocks of the update)
// and stride it over a grid that the device keeps resident, so a half-step
// with few or no active seeds costs little whatever the grid of a full one.
//
// The loop kernel runs half-steps h_begin.. with a grid barrier after each
// phase. All workgroups read the same active counts after a barrier, so they
// leave the loop together once every pair's count is zero; later half-steps
// cost nothing. Its grid never exceeds the workgroups the device keeps
// resident at once (cooperative launch), and each barrier wait is bounded:
// past the bound the workgroup sets the error word and leaves the loop, so the
// kernel always ends; the output count then reports the failure.
//
// The tail kernel runs half-steps h_begin.. in one plain launch without grid
// barriers: workgroups take the tasks of all phases in one global order from a
// ticket counter and wait only for tasks with earlier tickets, which
// workgroups already running hold, so it needs no co-residency and ends as
// soon as a half-step has no active seed.
#pragma once
#include "ddm_aux.hpp"

namespace ddm {

struct FrmArgs {
    SweepArgs sw[2];      // forward (0) and backward (1) sweeps; qrows and qcount set per half-step
    ResolveArgs rs[2];
    FrmState st;
    int B, nhalf, k, qblocks;
    int nch[2];
    uint32_t *bar;        // loop kernel: barrier arrivals, zero at launch
    int32_t *err;         // loop and tail kernels: set to 1 when a wait ran past its bound
    int spin_limit;       // loop and tail kernels: polls per wait before giving up
    uint32_t *tail;       // tail kernel: ticket, done and ready words at +0, +32, +64, zero at launch
    GridSeeds g0;         // grid seeds implicit in half-step 0 (g0.S = 0: the init kernel wrote them)
};

// Active queries of pair pr at half-step h. Every helper below takes the grid
// seeds of half-step 0 separately: the per-half-step kernels pass a.g0, the
// loop and tail kernels (which never start at an implicit half-step 0) pass a
// zero constant, so that path is compiled out of them.
__device__ __forceinline__ int frm_count(const FrmArgs &a, GridSeeds g0, int h, int pr) {
    return (h == 0 && g0.S > 0) ? g0.k : a.st.counts[pr * a.st.cnt_bs + h];
}

// Start of a call whose grid seeds are implicit in half-step 0 (one workgroup
// of the first sweep): the active counts (k, then zero) and the control words.
__device__ __forceinline__ void frm_grid_start(const FrmArgs &a) {
    if (threadIdx.x < 5) a.bar[threadIdx.x * 32] = 0;
    const int per = a.nhalf + 1;
    for (int i = threadIdx.x; i < a.B * per; i += blockDim.x)
        a.st.counts[(i / per) * a.st.cnt_bs + i % per] = (i % per == 0) ? a.k : 0;
}

// Task t of a phase -> (pair, task within the pair), given the per-pair counts.
template <class Count>
__device__ __forceinline__ int task_locate(int B, int t, Count count, int *pair) {
    int pr = 0;
    for (; pr < B; ++pr) {
        const int c = count(pr);
        if (t < c) break;
        t -= c;
    }
    *pair = pr;
    return t;
}

// Sweep arguments of half-step h: its direction, query list and counts.
__device__ __forceinline__ SweepArgs frm_sweep_args(const FrmArgs &a, GridSeeds g0, int h) {
    SweepArgs p = a.sw[h & 1];
    if (h == 0 && g0.S > 0) {             // implicit grid seeds: rows from the grid, k of them
        p.qrows = nullptr;
        p.qcount = nullptr;
        p.nq = g0.k;
        p.grid_s = g0.S; p.grid_kx = g0.kx; p.grid_w = g0.W;
        return p;
    }
    p.qrows = a.st.qrows[h & 1];
    p.qcount = a.st.counts + h;
    p.grid_s = 0;
    return p;
}

// Sweep tasks of pair pr at half-step h: reference chunks x query groups of
// the runtime split (0 when the pair has no active query).
template <int DT>
__device__ __forceinline__ int frm_sweep_tasks(const FrmArgs &a, GridSeeds g0, const SweepArgs &p, int h,
                                           int pr) {
    constexpr int GROUP = TILE * group_tiles(DT);
    const int nq = frm_count(a, g0, h, pr);
    if (nq <= 0) return 0;
    const int nch = a.nch[h & 1];
    const SplitGeom sg = split_geom(p.split, nq, p.split_rows, p.qblocks, p.chunk / GROUP, nch, p.rowcap);
    return nch * sg.need * sg.s;
}

template <int DT>
__device__ __forceinline__ int frm_sweep_total(const FrmArgs &a, GridSeeds g0, const SweepArgs &p, int h) {
    int total = 0;
    for (int pr = 0; pr < a.B; ++pr) total += frm_sweep_tasks<DT>(a, g0, p, h, pr);
    return total;
}

// Sweep task t (over all pairs) of half-step h.
template <int DT, int NP, int NKB, int RQ, int NW>
__device__ __forceinline__ void frm_sweep_run(const FrmArgs &a, GridSeeds g0, const SweepArgs &p, int h,
                                              int t, unsigned char *lds) {
    int pr;
    const int tt = task_locate(a.B, t, [&](int q) { return frm_sweep_tasks<DT>(a, g0, p, h, q); }, &pr);
    const int nch = a.nch[h & 1];
    sweep_task<DT, NP, NKB, RQ, NW, false>(p, pr, tt % nch, tt / nch, lds);
}

// Sweep phase of half-step h over the workgroups of the grid.
template <int DT, int NP, int NKB, int RQ, int NW>
__device__ __forceinline__ void frm_sweep_phase(const FrmArgs &a, GridSeeds g0, int h, unsigned char *lds) {
    const SweepArgs p = frm_sweep_args(a, g0, h);
    const int total = frm_sweep_total<DT>(a, g0, p, h);
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        __syncthreads();                       // the previous task's waves are done with the LDS
        frm_sweep_run<DT, NP, NKB, RQ, NW>(a, g0, p, h, t, lds);
    }
}

// Update tasks of pair pr at half-step h: blocks of QB active queries.
template <int QB>
__device__ __forceinline__ int frm_update_tasks(const FrmArgs &a, GridSeeds g0, int h, int pr) {
    return (frm_count(a, g0, h, pr) + QB - 1) / QB;
}

template <int QB>
__device__ __forceinline__ int frm_update_total(const FrmArgs &a, GridSeeds g0, int h) {
    int total = 0;
    for (int pr = 0; pr < a.B; ++pr) total += frm_update_tasks<QB>(a, g0, h, pr);
    return total;
}

// Update task t (over all pairs) of half-step h with NT threads, NT/16 queries.
template <int DT, int NT>
__device__ __forceinline__ void frm_update_run(const FrmArgs &a, GridSeeds g0, int h, int t, uint64_t *red) {
    constexpr int QB = NT / 16;
    int pr;
    const int blk = task_locate(a.B, t, [&](int q) { return frm_update_tasks<QB>(a, g0, h, q); }, &pr);
    frm_update_task<DT, QB, NT>(a.rs[h & 1], a.st, h, h & 1, h / 2 + 1, pr, blk, red, g0);
}

// Update phase of half-step h over the workgroups of the grid.
template <int DT, int NT>
__device__ __forceinline__ void frm_update_phase(const FrmArgs &a, GridSeeds g0, int h, uint64_t *red) {
    const int total = frm_update_total<NT / 16>(a, g0, h);
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        __syncthreads();
        frm_update_run<DT, NT>(a, g0, h, t, red);
    }
}

template <int DT, int NP, int NKB, int RQ, int NW>
__global__ void __launch_bounds__(NW * 64) frm_sweep_kernel(FrmArgs a, int h) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    if (h == 0 && a.g0.S > 0 && blockIdx.x == 0) frm_grid_start(a);
    frm_sweep_phase<DT, NP, NKB, RQ, NW>(a, a.g0, h, lds);
}

template <int DT>
__global__ void __launch_bounds__(256) frm_update_kernel(FrmArgs a, int h) {
    __shared__ uint64_t red[256];
    frm_update_phase<DT, 256>(a, a.g0, h, red);
}

constexpr int kSpinLimit = 1 << 20;   // default polls per barrier wait (each an uncached load + s_sleep): ~1 s

// Grid-wide barrier on a monotonically increasing arrival counter: each
// workgroup adds one arrival and waits for `target` (= barriers so far x
// workgroups). Release/acquire at agent scope make the global writes before the
// barrier visible to every workgroup after it. Returns false, uniformly over
// the workgroup, if the wait timed out (then or at an earlier barrier).
__device__ __forceinline__ bool grid_sync(uint32_t *bar, uint32_t target, int32_t *err, int spin_limit, int *flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int ok = 1, spins = 0;
        while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++spins > spin_limit) {
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (ok && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) ok = 0;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *flag = ok;
    }
    __syncthreads();
    return *flag != 0;
}

template <int DT, int NP, int NKB, int RQ, int NW>
__global__ void __launch_bounds__(NW * 64) frm_loop_kernel(FrmArgs a, int h_begin) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ int flag;
    constexpr GridSeeds none{};
    uint32_t target = 0;
    for (int h = h_begin; h < a.nhalf; ++h) {
        bool any = false;
        for (int pr = 0; pr < a.B; ++pr) any |= frm_count(a, none, h, pr) > 0;
        if (!any) break;
        frm_sweep_phase<DT, NP, NKB, RQ, NW>(a, none, h, lds);
        target += gridDim.x;
        if (!grid_sync(a.bar, target, a.err, a.spin_limit, &flag)) return;
        frm_update_phase<DT, NW * 64>(a, none, h, reinterpret_cast<uint64_t *>(lds));
        target += gridDim.x;
        if (!grid_sync(a.bar, target, a.err, a.spin_limit, &flag)) return;
    }
}

// Bounded wait of the tail kernel until *w >= target: thread 0 polls, the
// workgroup follows, with agent-scope acquire after the wait. False, uniformly
// over the workgroup, when the bound ran out here or another workgroup already
// reported a timeout.
__device__ __forceinline__ bool tail_wait(const uint32_t *w, uint32_t target, int32_t *err, int spin_limit,
                                          int *flag) {
    __syncthreads();                           // every wave has read the previous flag
    if (threadIdx.x == 0) {
        int ok = 1, spins = 0;
        while (__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++spins > spin_limit) {
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *flag = ok;
    }
    __syncthreads();
    return *flag != 0;
}

// Half-steps h_begin.. until one has no active seed, in one plain launch.
// Tickets order the tasks: the sweep tasks of half-step h, then its update
// tasks, then those of h + 1. Every workgroup walks the same sequence of
// half-steps and derives each one's task counts from the active counts, so
// all agree on where a ticket falls. An update task first waits until the
// done counter covers every sweep task of its half-step (no later task can
// finish before that); the workgroup finishing the last update task of h
// publishes h + 1 through the ready word, after which its active counts are
// final. A wait therefore only ever depends on tickets handed out earlier,
// to workgroups already running: any grid completes, down to one workgroup.
template <int DT, int NP, int NKB, int RQ, int NW>
__global__ void __launch_bounds__(NW * 64) frm_tail_kernel(FrmArgs a, int h_begin) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ int flag;
    __shared__ uint32_t tk;
    constexpr int QB = NW * 64 / 16;
    constexpr GridSeeds none{};
    uint32_t *ticket = a.tail, *done = a.tail + 32, *ready = a.tail + 64;
    int h = h_begin;
    if (h >= a.nhalf) return;
    SweepArgs p = frm_sweep_args(a, none, h);
    uint32_t sb = 0;                                           // first ticket of half-step h
    uint32_t ns = frm_sweep_total<DT>(a, none, p, h), nu = frm_update_total<QB>(a, none, h);
    if (ns == 0) return;
    for (;;) {
        __syncthreads();                                       // the LDS and tk are free again
        if (threadIdx.x == 0) tk = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const uint32_t t = tk;
        while (t >= sb + ns + nu) {                            // past half-step h: wait until h + 1 is known
            if (!tail_wait(ready, (uint32_t)(h + 1 - h_begin), a.err, a.spin_limit, &flag)) return;
            sb += ns + nu;
            if (++h >= a.nhalf) return;
            p = frm_sweep_args(a, none, h);
            ns = frm_sweep_total<DT>(a, none, p, h);
            if (ns == 0) return;
            nu = frm_update_total<QB>(a, none, h);
        }
        const bool upd = t >= sb + ns;
        if (upd) {
            if (!tail_wait(done, sb + ns, a.err, a.spin_limit, &flag)) return;
            frm_update_run<DT, NW * 64>(a, none, h, (int)(t - sb - ns), reinterpret_cast<uint64_t *>(lds));
        } else {
            frm_sweep_run<DT, NP, NKB, RQ, NW>(a, none, p, h, (int)(t - sb), lds);
        }
        __syncthreads();                                       // every wave's writes of the task are issued
        if (threadIdx.x == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const uint32_t prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (upd && prev + 1 == sb + ns + nu) {             // last task of half-step h
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
                __hip_atomic_store(ready, (uint32_t)(h + 1 - h_begin), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

}  // namespace ddm
