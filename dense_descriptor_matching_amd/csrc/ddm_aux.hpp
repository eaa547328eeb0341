// ddm_aux.hpp -- the kernels around the sweep: index resolution, the FRM state
// machine (seed grid, cycle tests, active-set compaction), the mutual check and
// the ordered output compaction.
//
// FRM follows the fast_reciprocal_NNs routine quoted in "DUSt3R和MASt3R论文阅读"
// (Staskaer blog, section MASt3R matching): seeds on the stride-S grid, one
// forward and one backward NN query per iteration for the seeds still active,
// a seed stops once its new image-2 pixel equals the previous one (forward
// test) or its new image-1 pixel equals the previous one (backward test), at
// most max_iter iterations, and the stopped seeds give unique pairs sorted by
// the image-1 index. The reciprocal set follows the FRM paragraph of the
// "MASt3R" note on cv-learn.com (section 手法とアーキテクチャ).
#pragma once
#include "ddm_sweep.hpp"

namespace ddm {

// ---------------------------------------------------------------------------
// Index resolution. A query's row partials (one per reference chunk) hold the
// maximum score and the (group, slot) that produced it; the exact reference
// is one of the G consecutive references group*GROUP + slot*G + t. Sixteen
// lanes recompute those dots (fp32 FMA on the stored values, G/16 each) and
// keep the largest, lowest t on ties. The reported score is the matrix-core
// maximum.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float dot_rows(const unsigned char *a, const unsigned char *b, int d) {
    float s = 0.f;
#pragma unroll 8      // loads of eight elements in flight together; the fma chain keeps element order
    for (int k = 0; k < d; ++k) s = fmaf(Tr<DT>::elem(a, k), Tr<DT>::elem(b, k), s);
    return s;
}

// The 8 products of one 16-byte piece (fp16 or bf16), accumulated in element order.
template <int DT>
__device__ __forceinline__ float dot_piece(u32x4_t a, u32x4_t b, float s) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float a0, a1, b0, b1;
        if constexpr (DT == DT_F16) {
            a0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(a[w] & 0xffffu));
            a1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(a[w] >> 16));
            b0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(b[w] & 0xffffu));
            b1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(b[w] >> 16));
        } else {
            a0 = __uint_as_float(a[w] << 16); a1 = __uint_as_float(a[w] & 0xffff0000u);
            b0 = __uint_as_float(b[w] << 16); b1 = __uint_as_float(b[w] & 0xffff0000u);
        }
        s = fmaf(a0, b0, s);
        s = fmaf(a1, b1, s);
    }
    return s;
}

// Rescan of one query's winning (group, slot): called by the 16 lanes of a row
// (sub = lane & 15) with the query's merged partial key. Lane sub takes the
// candidates t = sub, sub + 16, ... of the G; fp16/bf16 rows are read as whole
// 16-byte pieces (rows hold ld = 8 * pieces elements, zero beyond d).
template <int DT>
__device__ __forceinline__ void rescan_one(uint64_t k, const unsigned char *qp, const unsigned char *R, int nref,
                                           int ld, int d, int sub, int *j_out, float *s_out) {
    constexpr int ESZ = Tr<DT>::ESZ;
    constexpr int G = group_tiles(DT), GROUP = TILE * G;
    const float mval = fkey_inv((uint32_t)(k >> 32));
    const uint32_t id = ~(uint32_t)k;
    const int j0 = (int)((id >> 4) * GROUP + (id & 15u) * G);
    float s = -INFINITY;
    int bj = 0x7fffffff;
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int t = sub; t < G; t += 16) {      // ascending t: strict > keeps the lowest
            const int j = j0 + t;
            if (j < nref) {
                const float v = dot_rows<DT>(qp, R + (long long)j * ld * ESZ, d);
                if (v > s || bj == 0x7fffffff) { s = v; bj = j; }
            }
        }
    } else {
        constexpr int C = G / 16;
        const u32x4_t *q4 = reinterpret_cast<const u32x4_t *>(qp);
        const u32x4_t *r4[C];
        float acc[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int j = j0 + sub + 16 * c;
            r4[c] = reinterpret_cast<const u32x4_t *>(R + (long long)(j < nref ? j : nref - 1) * ld * ESZ);
            acc[c] = 0.f;
        }
        const int np = ld / 8;
#pragma unroll 4      // four pieces' loads in flight together instead of one latency per piece
        for (int p = 0; p < np; ++p) {
            const u32x4_t qv = q4[p];
#pragma unroll
            for (int c = 0; c < C; ++c) acc[c] = dot_piece<DT>(qv, r4[c][p], acc[c]);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {            // ascending t: strict > keeps the lowest
            const int j = j0 + sub + 16 * c;
            if (j < nref && (acc[c] > s || bj == 0x7fffffff)) { s = acc[c]; bj = j; }
        }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
        const float os = __shfl_xor(s, m, 16);
        const int oj = __shfl_xor(bj, m, 16);
        if (os > s || (os == s && oj < bj)) { s = os; bj = oj; }
    }
    // every valid query has a partial from every chunk, so bj < nref; clamp anyway so
    // that a bad index can never become an out-of-range gather downstream
    *j_out = bj < nref ? bj : nref - 1;
    *s_out = mval;
}

// Resolution of query block blk (QB consecutive queries) by an NT-thread
// workgroup. Phase 1: TPQ = NT / QB threads per query take the maximum of its
// per-chunk partial keys, consecutive threads on consecutive queries so that
// each chunk's slice is read contiguously; the TPQ maxima meet in red[NT] (LDS).
// Phase 2: sixteen lanes per query rescan the winning group's candidates,
// NT / 16 queries per round. emit(valid, x, j, s, sub) is called by every lane
// in every round (wave-wide ballots may follow). A block past nq returns at
// once (nq may come from device memory; the test is uniform over the block).
// The caller separates two uses of red by a barrier. mid() runs on every
// thread between the phases (loads issued there travel with the candidates').
template <int DT, int QB, int NT, class QPtr, class Emit, class Mid>
__device__ __forceinline__ void resolve_block(int blk, uint64_t *red, const uint64_t *part, int nchunks,
                                              long long rowcap, int nq, const unsigned char *R, int nref, int ld,
                                              int d, QPtr qptr, Emit emit, Mid mid) {
    static_assert(QB % 16 == 0 && NT % QB == 0 && QB % (NT / 16) == 0, "QB and NT");
    constexpr int TPQ = NT / QB, PER_ROUND = NT / 16;
    const int x0 = blk * QB;
    if (x0 >= nq) return;
    {
        const int q = (int)threadIdx.x % QB, slice = (int)threadIdx.x / QB;
        const int x = x0 + q;
        uint64_t k = 0;
        if (x < nq) {
#pragma unroll 8
            for (int ch = slice; ch < nchunks; ch += TPQ) {
                const uint64_t v = part[(long long)ch * rowcap + x];
                k = v > k ? v : k;
            }
        }
        red[threadIdx.x] = k;
    }
    __syncthreads();
    if (TPQ > 1 && threadIdx.x < QB) {
        uint64_t k = red[threadIdx.x];
#pragma unroll
        for (int t = 1; t < TPQ; ++t) {
            const uint64_t v = red[t * QB + threadIdx.x];
            k = v > k ? v : k;
        }
        red[threadIdx.x] = k;
    }
    if (TPQ > 1) __syncthreads();
    mid();
    const int sub = threadIdx.x & 15;
#pragma unroll 1
    for (int round = 0; round < QB / PER_ROUND; ++round) {
        const int r = round * PER_ROUND + (int)(threadIdx.x >> 4);
        const int x = x0 + r;
        const bool valid = x < nq;
        int j = 0;
        float s = 0.f;
        if (valid) rescan_one<DT>(red[r], qptr(x), R, nref, ld, d, sub, &j, &s);
        emit(valid, x, j, s, sub);
    }
}

template <int DT, int QB, int NT, class QPtr, class Emit>
__device__ __forceinline__ void resolve_block(int blk, uint64_t *red, const uint64_t *part, int nchunks,
                                              long long rowcap, int nq, const unsigned char *R, int nref, int ld,
                                              int d, QPtr qptr, Emit emit) {
    resolve_block<DT, QB, NT>(blk, red, part, nchunks, rowcap, nq, R, nref, ld, d, qptr, emit, [] {});
}

struct ResolveArgs {
    const uint64_t *rowpart; long long rowpart_bs; int nchunks; int rowcap;
    const unsigned char *Q; long long q_bs; const int32_t *qrows; long long qrows_bs;
    const int32_t *qcount; long long qcount_bs; int nq;
    const unsigned char *R; long long r_bs; int nref; int ld; int d;
    int split, qblocks, split_rows, chunk_groups;   // runtime split of the sweep (SweepArgs)
    int neg_out;     // Euclidean metric: report -score (the squared distance, clamped at 0)
};

__device__ __forceinline__ float reported(float s, int neg_out) { return neg_out ? fmaxf(-s, 0.f) : s; }

// Caller gather list -> the rows the sweep reads: entries outside [0, nrows)
// become row 0 (so no access leaves the map) and are reported as -1 later.
__global__ void __launch_bounds__(256) nn_rows_kernel(const int32_t *qrows, int n, int nrows, int32_t *safe) {
    for (int x = blockIdx.x * 256 + threadIdx.x; x < n; x += gridDim.x * 256) {
        const int r = qrows[x];
        safe[x] = (r >= 0 && r < nrows) ? r : 0;
    }
}

// Plain NN output: out_idx[x], out_score[x] for every query (-1 and NaN for a
// caller row outside the query map; `given` holds the caller's list).
template <int DT, int QB>
__global__ void __launch_bounds__(256) nn_resolve_kernel(ResolveArgs a, const int32_t *given, int nrows,
                                                         int32_t *out_idx, float *out_score) {
    __shared__ uint64_t red[256];
    resolve_block<DT, QB, 256>(blockIdx.x, red, a.rowpart, a.nchunks, a.rowcap, a.nq, a.R, a.nref, a.ld, a.d,
                      [&](int x) {
                          const int qrow = a.qrows ? a.qrows[x] : x;
                          return a.Q + (long long)qrow * a.ld * Tr<DT>::ESZ;
                      },
                      [&](bool valid, int x, int j, float s, int sub) {
                          if (valid && sub == 0) {
                              const bool ok = !given || (given[x] >= 0 && given[x] < nrows);
                              out_idx[x] = ok ? j : -1;
                              // the quiet-NaN pattern is stored as an integer: no floating-point NaN is formed
                              reinterpret_cast<uint32_t *>(out_score)[x] =
                                  ok ? __float_as_uint(reported(s, a.neg_out)) : 0x7fc00000u;
                          }
                      });
}

// ---------------------------------------------------------------------------
// Mutual NN: the fused sweep leaves one key per row (maximum, winning (group,
// slot)) and one per column (maximum, first query block holding it), each
// merged over the whole sweep by atomic maxima. Row i with j = NN_2(i) is
// reciprocal iff column j's maximum equals row i's maximum (both are the same
// matrix-core value, compared as order-preserving keys) and no lower row reaches
// that maximum too (NN_1 takes the lowest index on ties). Lower rows of earlier
// query blocks are excluded by the column's first block; among the rows that
// pass, the lowest claims the column.
// ---------------------------------------------------------------------------
// Clears the merged keys (0 loses to every real key) and the column owners.
__global__ void __launch_bounds__(256) mutual_init_kernel(uint64_t *rowkey, int n1, uint64_t *colkey, int32_t *owner,
                                                          int n2) {
    for (int x = blockIdx.x * 256 + threadIdx.x; x < n1 || x < n2; x += gridDim.x * 256) {
        if (x < n1) rowkey[x] = 0;
        if (x < n2) { colkey[x] = 0; owner[x] = 0x7fffffff; }
    }
}

// One row per 16 lanes, QB rows per block in rounds of 16; the row key is the
// merged one (one slot per row). A row can only pass when one of the G
// candidates of its winning (group, slot) carries, in its column key, this
// row's maximum and this row's query block; a row with no such candidate skips
// the rescan (unless the caller asked for every row's NN) and is written as a
// non-match. Rows that pass claim their column with an atomic minimum; the
// compaction keeps a row only if it holds its column's claim.
template <int DT, int QB>
__global__ void __launch_bounds__(256) mutual_rows_kernel(ResolveArgs a, const uint64_t *colkey, int rows_per_qblk,
                                                          int32_t *owner, int32_t *match_j, float *match_s,
                                                          int32_t *nn12, float *s12) {
    static_assert(QB % 16 == 0, "rounds of 16 rows");
    constexpr int G = group_tiles(DT), GROUP = TILE * G;
    const int sub = (int)threadIdx.x & 15, lane = (int)threadIdx.x & 63;
#pragma unroll 1
    for (int round = 0; round < QB / 16; ++round) {
        const int x = (int)blockIdx.x * QB + round * 16 + (int)(threadIdx.x >> 4);
        const bool valid = x < a.nq;                 // the same for the row's 16 lanes
        uint64_t k = 0;
        bool hit = false;
        if (valid) {
            k = a.rowpart[x];
            const uint32_t id = ~(uint32_t)k, fk = (uint32_t)(k >> 32);
            const uint32_t qlow = ~(uint32_t)(x / rows_per_qblk);
            const int j0 = (int)((id >> 4) * GROUP + (id & 15u) * G);
            for (int t = sub; t < G; t += 16) {
                const int j = j0 + t;
                if (j < a.nref) {
                    const uint64_t ck = colkey[j];
                    hit |= (uint32_t)(ck >> 32) == fk && (uint32_t)ck == qlow;
                }
            }
        }
        // any candidate of the row: its 16 lanes are one 16-bit field of the wave's ballot
        hit = ((__ballot(hit) >> (lane & 48)) & 0xffffull) != 0;
        if (!valid) continue;
        int j = -1;
        float s = fkey_inv((uint32_t)(k >> 32));
        if (hit || nn12)
            rescan_one<DT>(k, a.Q + (long long)x * a.ld * Tr<DT>::ESZ, a.R, a.nref, a.ld, a.d, sub, &j, &s);
        if (sub == 0) {
            bool cand = false;
            if (hit) {
                const uint64_t ck = colkey[j];
                cand = (uint32_t)(ck >> 32) == fkey(s) && (uint32_t)(x / rows_per_qblk) == ~(uint32_t)ck;
            }
            if (cand) atomicMin(owner + j, x);
            const float rs = reported(s, a.neg_out);
            match_j[x] = cand ? j : -1;
            match_s[x] = rs;
            if (nn12) { nn12[x] = j; s12[x] = rs; }
        }
    }
}

// ---------------------------------------------------------------------------
// FRM state. Per pair: u[k], v[k], score[k], conv[k], two active lists (seed
// ids) with their query rows, and the per-half-step active counts
// counts[0 .. 2*max_iter] (counts[h] = queries of half-step h).
// ---------------------------------------------------------------------------
struct FrmState {
    int32_t *u, *v, *conv;
    float *score;
    int32_t *act[2], *qrows[2];
    int32_t *counts;
    int32_t *match_j; float *match_s;
    int32_t *uprev, *uiter;   // u before the seed's last backward step, and that step's iteration (-1 none)
    int32_t *basin;           // [pair][N1] or null: basin variant (forward test off, record every backward step)
    long long k_bs;        // elements between pairs for the k-sized arrays
    long long cnt_bs;      // elements between pairs for counts
    long long n1_bs;       // elements between pairs for match arrays
};

// Grid seeds left implicit in the first half-step (S = 0: none): the first
// sweep derives their pixels, the first update writes their initial state.
struct GridSeeds {
    int S, kx, W, k;
};

__device__ __forceinline__ void frm_seed_reset(const FrmState &st, long long ka, int a, int p) {
    st.u[ka] = p; st.v[ka] = -1; st.conv[ka] = -1; st.score[ka] = 0.f;
    st.act[0][ka] = a; st.qrows[0][ka] = p;
    st.uprev[ka] = p; st.uiter[ka] = -1;
}

// Initial state. Grid seeds (k > 0 of them: rows S/2 + S*n < H1, columns
// S/2 + S*n < W1, p = x + W1*y, ascending) are written here; with explicit
// starts (marks != null) the seeds come later from the start marks and the
// kernel only clears the marks. Also clears the first n1 entries of the dense
// match array, the marks and the basin map (n1 = 0 when none of them is read:
// the one-workgroup output), and the control words of the loop and tail
// kernels (barrier arrivals, error flag, ticket, done and ready counters).
__global__ void __launch_bounds__(256) frm_init_kernel(FrmState st, int k, int kx, int W1, int S, int N1,
                                                       int nhalf, uint32_t *ctl, int32_t *marks) {
    if (ctl && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 5) ctl[threadIdx.x * 32] = 0;
    const int pair = blockIdx.y;
    const long long ko = pair * st.k_bs;
    if (!marks)
        for (int a = blockIdx.x * 256 + threadIdx.x; a < k; a += gridDim.x * 256) {
            const int y = S / 2 + (a / kx) * S, x = S / 2 + (a % kx) * S;
            frm_seed_reset(st, ko + a, a, x + W1 * y);
        }
    for (int i = blockIdx.x * 256 + threadIdx.x; i < N1; i += gridDim.x * 256) {
        st.match_j[pair * st.n1_bs + i] = -1;
        if (marks) marks[pair * st.n1_bs + i] = -1;
        if (st.basin) st.basin[pair * st.n1_bs + i] = -1;
    }
    if (blockIdx.x == 0)
        for (int h = threadIdx.x; h <= nhalf; h += 256) st.counts[pair * st.cnt_bs + h] = (h == 0) ? k : 0;
}

// Explicit starts: mark every start inside image 1 (marks[p] = p); entries
// outside [0, N1) are ignored. An ordered compaction of the marks then lists
// the distinct starts in ascending order with their count.
__global__ void __launch_bounds__(256) frm_mark_starts_kernel(const int32_t *starts, int n, int N1, int32_t *marks) {
    for (int e = blockIdx.x * 256 + threadIdx.x; e < n; e += gridDim.x * 256) {
        const int p = starts[e];
        if (p >= 0 && p < N1) marks[p] = p;
    }
}

// Seeds from the compacted starts (u[a] and qrows[0][a] already hold them).
__global__ void __launch_bounds__(256) frm_seeds_from_starts_kernel(FrmState st, int kcap) {
    const int k = st.counts[0];
    for (int a = blockIdx.x * 256 + threadIdx.x; a < kcap && a < k; a += gridDim.x * 256)
        frm_seed_reset(st, a, a, st.u[a]);
}

// One half-step's update for query block blk of pair `pair`: resolve each
// active query, apply the cycle test and append the seeds that stay active to
// the next list. The block's survivors take one atomic on the pair's next
// count (one per block rather than per wave: the count is a single contended
// address); list order does not affect any result.
template <int DT, int QB, int NT>
__device__ __forceinline__ void frm_update_task(const ResolveArgs &a, const FrmState &st, int h, int backward,
                                                int iter, int pair, int blk, uint64_t *red, GridSeeds g0) {
    static_assert(QB <= 64, "survivors of a block are gathered by one wave");
    __shared__ int keep_seed[QB], keep_j[QB];
    const int cur = h & 1, nxt = cur ^ 1;
    const long long ko = pair * st.k_bs;
    int32_t *counts = st.counts + pair * st.cnt_bs;
    const bool implicit = h == 0 && g0.S > 0;       // seed x at its grid pixel, no state yet
    const int nq = implicit ? g0.k : counts[h];
    const int x0 = blk * QB;
    if (x0 >= nq) return;
    const unsigned char *Q = a.Q + pair * a.q_bs;
    const SplitGeom sg = split_geom(a.split, nq, a.split_rows, a.qblocks, a.chunk_groups, a.nchunks, a.rowcap);
    // The query of this thread's rescan (one round: QB = NT / 16): its row index and
    // seed are loaded before the partial merge, the seed's previous pixel between
    // merge and rescan, so that they arrive with the partials and the candidates.
    static_assert(QB == NT / 16, "one rescan round per block");
    const int xm = x0 + (int)(threadIdx.x >> 4);
    const bool vm = xm < nq;
    int pre_qrow = 0, pre_seed = 0, pre_prev = 0;
    if (vm) {
        pre_qrow = implicit ? grid_seed_pixel(xm, g0.S, g0.kx, g0.W) : st.qrows[cur][ko + xm];
        pre_seed = implicit ? xm : st.act[cur][ko + xm];
    }
    resolve_block<DT, QB, NT>(
        blk, red, a.rowpart + pair * a.rowpart_bs, a.nchunks * sg.s, sg.rowcap, nq, a.R + pair * a.r_bs, a.nref,
        a.ld, a.d,
        [&](int) { return Q + (long long)pre_qrow * a.ld * Tr<DT>::ESZ; },
        [&](bool valid, int x, int j, float s, int sub) {
            if (sub != 0) return;
            int seed = -1;
            if (valid) {
                seed = pre_seed;
                bool keep;
                if (!backward) {
                    keep = st.basin != nullptr || j != pre_prev;    // no forward test in the basin variant
                    st.v[ko + seed] = j;
                    st.score[ko + seed] = reported(s, a.neg_out);
                    if (implicit) {                                 // the seed's initial state
                        st.u[ko + seed] = pre_qrow; st.uprev[ko + seed] = pre_qrow;
                        st.uiter[ko + seed] = -1; st.conv[ko + seed] = -1;
                    }
                } else {
                    const int from = pre_prev;
                    keep = (j != from);
                    st.u[ko + seed] = j;
                    st.uprev[ko + seed] = from;
                    st.uiter[ko + seed] = iter;
                    if (st.basin) st.basin[pair * st.n1_bs + from] = j;
                }
                if (!keep) {
                    st.conv[ko + seed] = iter;
                    seed = -1;
                }
            }
            keep_seed[x - x0] = seed;
            keep_j[x - x0] = j;
        },
        [&] {
            if (vm) pre_prev = implicit ? -1 : backward ? st.u[ko + pre_seed] : st.v[ko + pre_seed];
        });
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const bool in = lane < QB && x0 + lane < nq;
        const int seed = in ? keep_seed[lane] : -1;
        const uint64_t ball = __ballot(seed >= 0);
        const int n = __popcll(ball);
        if (n > 0) {
            int base = 0;
            if (lane == 0) base = atomicAdd(counts + h + 1, n);
            base = __shfl(base, 0);
            if (seed >= 0) {
                const int pos = base + __popcll(ball & ((1ull << lane) - 1ull));
                st.act[nxt][ko + pos] = seed;
                st.qrows[nxt][ko + pos] = keep_j[lane];
            }
        }
    }
}

// Converged seeds -> dense match array indexed by image-1 pixel (every seed
// that reaches pixel u reports the same v and score), optional seed states.
// Kept seeds -> dense match array indexed by the reported image-1 pixel
// (every seed reporting pixel i reports the same j and score), optional seed
// states (u, v, iteration of convergence or -1, u_old; -1 rows past the seed
// count). u_old = u at the start of the last iteration when the loop ran
// iteration max_iter, else the final u. pixel_tol == 0: kept = not active,
// reported pixel u. pixel_tol > 0: kept = pixel distance |yx(u_old) - yx(u)|
// below pixel_tol (in double, as a Euclidean distance), reported pixel u_old
// when report_old (explicit starts), else u.
// One seed's part of the collection: its state row (when asked for) and the
// image-1 pixel it is kept at, or -1.
__device__ __forceinline__ int frm_collect_seed(const FrmState &st, long long ko, int a, int32_t *ss, bool ran_last,
                                                int max_iter, int W1, double pixel_tol, int report_old) {
    const int u = st.u[ko + a], v = st.v[ko + a], it = st.conv[ko + a];
    const int uold = (ran_last && st.uiter[ko + a] == max_iter) ? st.uprev[ko + a] : u;
    bool kept;
    int i = u;
    if (pixel_tol > 0.0) {
        const double dy = (double)(uold / W1 - u / W1), dx = (double)(uold % W1 - u % W1);
        kept = sqrt(dy * dy + dx * dx) < pixel_tol;
        if (report_old) i = uold;
    } else {
        kept = it >= 0;
    }
    if (ss) {
        ss[0] = u; ss[1] = v; ss[2] = it; ss[3] = uold;
    }
    return kept ? i : -1;
}

__global__ void __launch_bounds__(256) frm_collect_kernel(FrmState st, int kcap, int32_t *seed_state,
                                                          const int32_t *counts_in, int32_t *query_counts,
                                                          int nhalf, int W1, double pixel_tol, int report_old) {
    const int pair = blockIdx.y;
    const long long ko = pair * st.k_bs;
    const int32_t *cnt = counts_in + pair * st.cnt_bs;
    const int k = cnt[0];
    const bool ran_last = cnt[nhalf - 2] > 0;      // forward queries of the last iteration
    const int max_iter = nhalf / 2;
    for (int a = blockIdx.x * 256 + threadIdx.x; a < kcap; a += gridDim.x * 256) {
        int32_t *ss = seed_state ? seed_state + (pair * (long long)kcap + a) * 4 : nullptr;
        if (a >= k) {
            if (ss) {
                ss[0] = -1; ss[1] = -1; ss[2] = -1; ss[3] = -1;
            }
            continue;
        }
        const int i = frm_collect_seed(st, ko, a, ss, ran_last, max_iter, W1, pixel_tol, report_old);
        if (i >= 0) {
            st.match_j[pair * st.n1_bs + i] = st.v[ko + a];
            st.match_s[pair * st.n1_bs + i] = st.score[ko + a];
        }
    }
    if (query_counts && blockIdx.x == 0)
        for (int h = threadIdx.x; h < nhalf; h += 256)
            query_counts[pair * (long long)nhalf + h] = counts_in[pair * st.cnt_bs + h];
}

// Collection and ordered output of a pair in one workgroup, for problems whose
// image-1 pixels fit a bitmap in LDS and whose seeds fit the workgroup's
// registers (OUT_SPT per thread). Each thread loads all its seeds at once and
// keeps (pixel, j, score) of the kept ones; their pixels are marked in the
// bitmap; an exclusive scan of the words' population counts, kept in LDS,
// gives every marked pixel its rank, so each kept seed writes its pair straight
// to out[rank] (seeds reporting the same pixel report the same pair and write
// the same slot). The outputs equal those of frm_collect_kernel followed by
// the dense compaction; out_count = -1 when *err is set.
constexpr int OUT_NT = 1024, OUT_SPT = 4;   // up to 4096 seeds per pair (more: one workgroup falls behind)
__global__ void __launch_bounds__(OUT_NT) frm_output_kernel(FrmState st, int kcap, int32_t *seed_state,
                                                            const int32_t *counts_in, int32_t *query_counts,
                                                            int nhalf, int W1, double pixel_tol, int report_old,
                                                            int N1, int32_t *out_i, int32_t *out_j, float *out_s,
                                                            long long out_bs, int capacity, int32_t *out_count,
                                                            const int32_t *err) {
    extern __shared__ uint32_t obits[];     // bitmap [nwords], then exclusive word ranks [nwords]
    __shared__ int wsum[OUT_NT / 64];
    const int pair = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nwords = (N1 + 31) >> 5;
    uint32_t *bits = obits;
    int *rank0 = reinterpret_cast<int *>(obits + nwords);
    for (int q = tid; q < nwords; q += OUT_NT) bits[q] = 0u;
    const long long ko = pair * st.k_bs;
    const int32_t *cnt = counts_in + pair * st.cnt_bs;
    const int k = min(cnt[0], kcap);
    const bool ran_last = cnt[nhalf - 2] > 0;
    const int max_iter = nhalf / 2;

    // every load of this thread's seeds first, then the tests
    int u[OUT_SPT], v[OUT_SPT], it[OUT_SPT], ui[OUT_SPT], up[OUT_SPT];
    float sc[OUT_SPT];
#pragma unroll
    for (int r = 0; r < OUT_SPT; ++r) {
        const int a = r * OUT_NT + tid;
        if (a < k) {
            u[r] = st.u[ko + a]; v[r] = st.v[ko + a]; it[r] = st.conv[ko + a]; sc[r] = st.score[ko + a];
            ui[r] = st.uiter[ko + a]; up[r] = st.uprev[ko + a];
        }
    }
    int pix[OUT_SPT];
#pragma unroll
    for (int r = 0; r < OUT_SPT; ++r) {
        const int a = r * OUT_NT + tid;
        pix[r] = -1;
        if (a < k) {
            const int uold = (ran_last && ui[r] == max_iter) ? up[r] : u[r];
            bool kept;
            int i = u[r];
            if (pixel_tol > 0.0) {
                const double dy = (double)(uold / W1 - u[r] / W1), dx = (double)(uold % W1 - u[r] % W1);
                kept = sqrt(dy * dy + dx * dx) < pixel_tol;
                if (report_old) i = uold;
            } else {
                kept = it[r] >= 0;
            }
            if (kept) pix[r] = i;
            if (seed_state) {
                int32_t *ss = seed_state + (pair * (long long)kcap + a) * 4;
                ss[0] = u[r]; ss[1] = v[r]; ss[2] = it[r]; ss[3] = uold;
            }
        } else if (a < kcap && seed_state) {
            int32_t *ss = seed_state + (pair * (long long)kcap + a) * 4;
            ss[0] = -1; ss[1] = -1; ss[2] = -1; ss[3] = -1;
        }
    }
    if (query_counts)
        for (int h = tid; h < nhalf; h += OUT_NT) query_counts[pair * (long long)nhalf + h] = cnt[h];
    __syncthreads();                           // the bitmap is clear
#pragma unroll
    for (int r = 0; r < OUT_SPT; ++r)
        if (pix[r] >= 0) atomicOr(&bits[pix[r] >> 5], 1u << (pix[r] & 31));
    __syncthreads();                           // the bitmap is complete

    // exclusive rank of each word: thread t owns a run of words
    const int per = (nwords + OUT_NT - 1) / OUT_NT;
    const int w0 = min(tid * per, nwords), w1 = min(w0 + per, nwords);
    int c = 0;
    for (int q = w0; q < w1; ++q) c += __popc(bits[q]);
    int incl = c;
    for (int m = 1; m < 64; m <<= 1) {
        const int o = __shfl_up(incl, m);
        if (lane >= m) incl += o;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = incl - c, total = 0;
    for (int q = 0; q < OUT_NT / 64; ++q) {
        if (q < w) base += wsum[q];
        total += wsum[q];
    }
    for (int q = w0; q < w1; ++q) {
        rank0[q] = base;
        base += __popc(bits[q]);
    }
    __syncthreads();                           // every word's rank is in place
#pragma unroll
    for (int r = 0; r < OUT_SPT; ++r) {
        const int i = pix[r];
        if (i >= 0) {
            const int rank = rank0[i >> 5] + __popc(bits[i >> 5] & ((1u << (i & 31)) - 1u));
            if (rank < capacity) {
                const long long o = pair * out_bs + rank;
                out_i[o] = i; out_j[o] = v[r]; out_s[o] = sc[r];
            }
        }
    }
    if (tid == 0) out_count[pair] = (err && *err) ? -1 : (total < capacity ? total : capacity);
}

// ---------------------------------------------------------------------------
// Ordered compaction of a dense match array (j >= 0 marks a pair) into sorted
// (i, j, score) lists: per-block counts, one scan per pair, scatter. With
// column owners (the mutual check), entry i is kept only if it holds the claim
// on its column (owner[j] == i): rows that lost their column to a lower row
// drop out here.
// ---------------------------------------------------------------------------
constexpr int CB = 1024;   // entries per compaction block (256 threads x 4)

__device__ __forceinline__ bool kept_entry(const int32_t *mj, const int32_t *owner, int i, int n) {
    if (i >= n) return false;
    const int j = mj[i];
    return j >= 0 && (!owner || owner[j] == i);
}

__global__ void __launch_bounds__(256) compact_count_kernel(const int32_t *match_j, long long n_bs, int n,
                                                            int32_t *blockcnt, int nblk, const int32_t *owner) {
    const int pair = blockIdx.y;
    const int32_t *mj = match_j + pair * n_bs;
    int c = 0;
    const int base = blockIdx.x * CB;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = base + t * 256 + threadIdx.x;
        c += kept_entry(mj, owner, i, n) ? 1 : 0;
    }
    __shared__ int red[4];
    for (int m = 32; m > 0; m >>= 1) c += __shfl_xor(c, m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) blockcnt[pair * nblk + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// out_count = -1 when *err is set (a grid barrier of the loop kernel timed out).
__global__ void __launch_bounds__(256) compact_scan_kernel(const int32_t *blockcnt, int32_t *blockoff, int nblk,
                                                           int32_t *out_count, int capacity, const int32_t *err) {
    const int pair = blockIdx.x;
    __shared__ int carry;
    __shared__ int wsum[4];
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int b0 = 0; b0 < nblk; b0 += 256) {
        const int b = b0 + threadIdx.x;
        const int v = b < nblk ? blockcnt[pair * nblk + b] : 0;
        int incl = v;
        for (int m = 1; m < 64; m <<= 1) {
            const int o = __shfl_up(incl, m);
            if (lane >= m) incl += o;
        }
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        int woff = 0;
        for (int q = 0; q < w; ++q) woff += wsum[q];
        if (b < nblk) blockoff[pair * nblk + b] = carry + woff + incl - v;
        __syncthreads();
        if (threadIdx.x == 0) carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
    }
    if (threadIdx.x == 0) out_count[pair] = (err && *err) ? -1 : (carry < capacity ? carry : capacity);
}

__global__ void __launch_bounds__(256) compact_scatter_kernel(const int32_t *match_j, const float *match_s,
                                                              long long n_bs, int n, const int32_t *blockoff,
                                                              int nblk, int32_t *out_i, int32_t *out_j,
                                                              float *out_s, long long out_bs, int capacity,
                                                              const int32_t *owner) {
    const int pair = blockIdx.y;
    const int32_t *mj = match_j + pair * n_bs;
    const float *ms = match_s + pair * n_bs;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __shared__ int wcnt[4];
    int off = blockoff[pair * nblk + blockIdx.x];
    for (int t = 0; t < 4; ++t) {
        const int i = blockIdx.x * CB + t * 256 + threadIdx.x;
        const bool valid = kept_entry(mj, owner, i, n);
        const uint64_t ball = __ballot(valid);
        if (lane == 0) wcnt[w] = __popcll(ball);
        __syncthreads();
        int woff = 0;
        for (int q = 0; q < w; ++q) woff += wcnt[q];
        const int rank = off + woff + __popcll(ball & ((1ull << lane) - 1ull));
        if (valid && rank < capacity) {
            const long long pos = pair * out_bs + rank;
            out_i[pos] = i; out_j[pos] = mj[i]; out_s[pos] = ms[i];
        }
        off += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
        __syncthreads();
    }
}

// Zero-padded copy [n][d] -> [n][ld] for maps whose rows are not a whole
// number of 16-byte pieces of a supported width.
// Euclidean metric: rows of d floats become rows of d + 2 whose dot products
// are minus the squared distances, so the dot-product sweep finds the nearest
// point and its negated score is the squared distance:
//   query side     [2x, -|x|^2, 1]
//   reference side [x, 1, -|x|^2]        (2 q.r - |q|^2 - |r|^2 = -|q - r|^2)
__global__ void __launch_bounds__(256) l2_augment_kernel(const float *src, int d, long long n, int ref_side,
                                                         float *dst) {
    const int ld = d + 2;
    for (long long r = (long long)blockIdx.x * 256 + threadIdx.x; r < n; r += (long long)gridDim.x * 256) {
        const float *x = src + r * d;
        float *o = dst + r * ld;
        float nrm = 0.f;
        for (int c = 0; c < d; ++c) nrm = fmaf(x[c], x[c], nrm);
        for (int c = 0; c < d; ++c) o[c] = ref_side ? x[c] : 2.f * x[c];
        o[d] = ref_side ? 1.f : -nrm;
        o[d + 1] = ref_side ? -nrm : 1.f;
    }
}

__global__ void __launch_bounds__(256) repack_kernel(const uint16_t *src, int d, uint16_t *dst, int ld, long long n) {
    const long long total = n * ld;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
        const long long r = e / ld;
        const int k = (int)(e - r * ld);
        dst[e] = k < d ? src[r * d + k] : (uint16_t)0;
    }
}

}  // namespace ddm
