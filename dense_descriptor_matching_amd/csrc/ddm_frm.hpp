// ddm_frm.hpp -- the FRM iteration: sweep and update phases, run either as one
// pair of launches per half-step or as one cooperative loop kernel.
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
    int32_t *err;         // loop kernel: set to 1 when a barrier wait ran past its bound
    int spin_limit;       // loop kernel: polls per barrier wait before giving up
};

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

// Sweep phase of half-step h over the workgroups of the grid.
template <int DT, int NP, int NKB, int RQ, int NW>
__device__ __forceinline__ void frm_sweep_phase(const FrmArgs &a, int h, unsigned char *lds) {
    constexpr int GROUP = TILE * group_tiles(DT);
    const int dir = h & 1;
    const int32_t *cnt = a.st.counts + h;
    SweepArgs p = a.sw[dir];
    p.qrows = a.st.qrows[h & 1];
    p.qcount = cnt;
    const int nch = a.nch[dir];
    auto tasks = [&](int pr) {
        const int nq = cnt[pr * a.st.cnt_bs];
        if (nq <= 0) return 0;
        const SplitGeom sg = split_geom(p.split, nq, p.split_rows, p.qblocks, p.chunk / GROUP, nch, p.rowcap);
        return nch * sg.need * sg.s;
    };
    int total = 0;
    for (int pr = 0; pr < a.B; ++pr) total += tasks(pr);
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        int pr;
        const int tt = task_locate(a.B, t, tasks, &pr);
        __syncthreads();                       // the previous task's waves are done with the LDS
        sweep_task<DT, NP, NKB, RQ, NW, false>(p, pr, tt % nch, tt / nch, lds);
    }
}

// Update phase of half-step h: NT threads per workgroup, NT/16 queries per task.
template <int DT, int NT>
__device__ __forceinline__ void frm_update_phase(const FrmArgs &a, int h, uint64_t *red) {
    constexpr int QB = NT / 16;
    const int dir = h & 1;
    const int32_t *cnt = a.st.counts + h;
    auto tasks = [&](int pr) { return (cnt[pr * a.st.cnt_bs] + QB - 1) / QB; };
    int total = 0;
    for (int pr = 0; pr < a.B; ++pr) total += tasks(pr);
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        int pr;
        const int blk = task_locate(a.B, t, tasks, &pr);
        __syncthreads();
        frm_update_task<DT, QB, NT>(a.rs[dir], a.st, h, dir, h / 2 + 1, pr, blk, red);
    }
}

template <int DT, int NP, int NKB, int RQ, int NW>
__global__ void __launch_bounds__(NW * 64) frm_sweep_kernel(FrmArgs a, int h) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    frm_sweep_phase<DT, NP, NKB, RQ, NW>(a, h, lds);
}

template <int DT>
__global__ void __launch_bounds__(256) frm_update_kernel(FrmArgs a, int h) {
    __shared__ uint64_t red[256];
    frm_update_phase<DT, 256>(a, h, red);
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
    uint32_t target = 0;
    for (int h = h_begin; h < a.nhalf; ++h) {
        bool any = false;
        for (int pr = 0; pr < a.B; ++pr) any |= a.st.counts[pr * a.st.cnt_bs + h] > 0;
        if (!any) break;
        frm_sweep_phase<DT, NP, NKB, RQ, NW>(a, h, lds);
        target += gridDim.x;
        if (!grid_sync(a.bar, target, a.err, a.spin_limit, &flag)) return;
        frm_update_phase<DT, NW * 64>(a, h, reinterpret_cast<uint64_t *>(lds));
        target += gridDim.x;
        if (!grid_sync(a.bar, target, a.err, a.spin_limit, &flag)) return;
    }
}

}  // namespace ddm
