// ddm_sweep.hpp -- fused dot-product + running arg-max sweep on CDNA4 matrix cores.
//
// One launch scores a set of query rows against every row of a reference map
// without ever materialising the score matrix. Nearest neighbour = arg-max of
// the dot product ("MASt3R" note on cv-learn.com, section
// 手法とアーキテクチャ, FRM paragraph); the exhaustive reciprocal set of the
// same paragraph additionally needs every column's maximum, which the COLMAX
// variant produces in the same pass.
//
// Work decomposition
//   grid.x  = reference chunk (whole index groups: 512 references, 128 for fp32),
//             staged once in LDS
//   grid.y  = query block (sb_per_wg sub-blocks of NW*RQ*16 rows)
//   grid.z  = independent pair (batched calls)
//   (The FRM kernels enumerate the same tasks from device counts instead.)
//   A sub-block has NW query slots; slot w is the 16-row query tiles w, w + NW,
//   ... (RQ of them, fewer when the sub-block is short). The waves of a
//   workgroup take (sub-block, slot) units from an LDS counter, so a wave that
//   the SIMD's issue favours takes more of them and both waves of a SIMD
//   finish together; a unit's tiles stay resident in VGPRs as MFMA A operands
//   while the chunk's 16-row reference tiles stream from LDS as B operands
//   with v_mfma_f32_16x16x32_{f16,bf16} (v_mfma_f32_16x16x4_f32 for fp32
//   maps), K padded to 32 with zeros in A only.
//
// Epilogue (the part that bounds this kernel at d = 24)
//   MFMA output lane l holds reference slot c = l % 16 and query rows
//   4*(l/16) + r, r = 0..3. Row direction: per register a running maximum over
//   a group of G = 32 tiles with one v_max3_f32 per two scores, then one
//   compare + select per register and group to remember which group held the
//   maximum (lazy index). Inside a group the 512 references are laid out so
//   that slot c of tile t is reference 32*c + t: the 32 candidates of one
//   (group, slot) are contiguous, and (group, slot, t) order equals reference
//   order, so the lowest-index tie-break survives. The exact index inside the
//   group is recovered later by recomputing 32 candidate dots (resolve_one).
//   Column direction (COLMAX): in-lane v_max3 chain over the unit's rows, then
//   one ds_max_f32 per tile into an LDS column array (the four lanes that hold
//   one column meet there), flushed once per workgroup as order-preserving keys.
//
// Reference slots past the end of the map (the tail of the last index group)
// hold copies of the last valid reference: their scores repeat one of the
// group's own scores, so no row maximum changes, and a tie with the original
// resolves to the lower (group, slot), which is the original's (a copy's slot
// index is never lower); their column maxima are not written. Query rows past
// the query count repeat the last valid row, which changes no column maximum
// and is never written back. No NaN or infinity ever enters a score.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ddm {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

constexpr int TILE = 16;            // references per MFMA tile
// Tiles per index group: 32 for fp16/bf16 maps; 8 for fp32 maps, whose wider
// rows would otherwise not fit one group of up to 128 components in LDS.
constexpr int group_tiles(int dt) { return dt == 0 ? 8 : 32; }

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Order-preserving map float -> uint32 (larger float, larger key); -0 == +0.
__device__ __forceinline__ uint32_t fkey(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

template <int DT> struct Tr;
template <> struct Tr<DT_F16> {
    static constexpr int E = 8, PS = 16, ESZ = 2;     // elements / bytes per lane piece
    using raw = u32x4_t;
    __device__ static f32x4_t mma(raw a, raw b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    }
    __device__ static raw zero() { return raw{0u, 0u, 0u, 0u}; }
    __device__ static float elem(const unsigned char *p, int k) {
        return (float)reinterpret_cast<const _Float16 *>(p)[k];
    }
};
template <> struct Tr<DT_BF16> {
    static constexpr int E = 8, PS = 16, ESZ = 2;
    using raw = u32x4_t;
    __device__ static f32x4_t mma(raw a, raw b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    __device__ static raw zero() { return raw{0u, 0u, 0u, 0u}; }
    __device__ static float elem(const unsigned char *p, int k) {
        uint32_t u = (uint32_t)reinterpret_cast<const uint16_t *>(p)[k] << 16;
        return __uint_as_float(u);
    }
};
template <> struct Tr<DT_F32> {
    static constexpr int E = 1, PS = 4, ESZ = 4;
    using raw = uint32_t;
    __device__ static f32x4_t mma(raw a, raw b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a), __uint_as_float(b), c, 0, 0, 0);
    }
    __device__ static raw zero() { return 0u; }
    __device__ static float elem(const unsigned char *p, int k) {
        return reinterpret_cast<const float *>(p)[k];
    }
};

struct SweepArgs {
    const unsigned char *Q;      // query map of pair 0
    const unsigned char *R;      // reference map of pair 0
    const int32_t *qrows;        // optional gather list (row of Q for each query)
    const int32_t *qcount;       // optional device query count (else nq)
    uint64_t *rowpart;           // [pair][nchunks][rowcap] row partial keys; COLMAX: [nq] row keys merged
                                 // by atomic maximum over all chunks
    uint64_t *colkey;            // COLMAX: [nref] column keys merged by atomic maximum over all query
                                 // blocks: high word = order-preserving key of the column maximum,
                                 // low word = ~(first query block holding it)
    long long q_bs, r_bs;        // bytes between pairs
    long long qrows_bs, qcount_bs, rowpart_bs;   // elements between pairs
    int nq;                      // query count (upper bound when qcount is set)
    int nref;                    // reference rows per pair
    int ld;                      // row stride in elements
    int chunk;                   // references per chunk (multiple of GROUP)
    int nchunks;
    int sb_per_wg;               // query sub-blocks per workgroup
    int rowcap;                  // rows per chunk slice of rowpart (without split)
    // Runtime split (used with a device query count), aiming at `split` tasks
    // per pair: when the count leaves query blocks idle and the pair's busy
    // workgroups fall short of it, each reference chunk is cut into s
    // sub-chunks (whole index groups) handled by the idle blocks, partial slot
    // chunk*s + sub; when the count gives at least twice as many (chunk,
    // sub-block) tasks, consecutive sub-blocks are grouped into one task so the
    // staged chunk serves several of them.
    int split;                   // tasks per pair to aim for; 0 = off
    int qblocks;                 // query blocks in the grid
    int split_rows;              // query rows per query block
    // Implicit query rows (qrows null) of a one-way sweep: query x is the x-th seed
    // of the stride-grid_s grid over a map of width grid_w with grid_kx seeds per
    // row; 0 = rows 0, 1, ... (always so in the two-way sweep)
    int grid_s, grid_kx, grid_w;
};

// Pixel of grid seed a: rows and columns S/2 + S*n, p = x + W*y, ascending.
__device__ __forceinline__ int grid_seed_pixel(int a, int S, int kx, int W) {
    return S / 2 + (a % kx) * S + W * (S / 2 + (a / kx) * S);
}

// Geometry of the runtime split for nq queries: query tasks per chunk (need),
// sub-chunks per chunk (s), rows per partial slot (rowcap) and sub-blocks per
// query task (spw; 0 = the launch's sb_per_wg). The sweep and the resolve of
// one half-step evaluate it on the same count.
struct SplitGeom { int need, s, rowcap, spw; };
__device__ __forceinline__ SplitGeom split_geom(int split, int nq, int rows, int qblocks, int groups_per_chunk,
                                                int nchunks, int rowcap) {
    if (!split) return SplitGeom{qblocks, 1, rowcap, 0};
    const int nsb = max(1, (nq + rows - 1) / rows);
    const int busy = nsb * nchunks;
    if (busy >= 2 * split) {
        const int spw = min(nsb, busy / split);
        return SplitGeom{(nsb + spw - 1) / spw, 1, nsb * rows, spw};
    }
    const int want = (split + busy - 1) / busy;
    const int s = max(1, min(want, min(qblocks / nsb, groups_per_chunk)));
    return SplitGeom{nsb, s, nsb * rows, 1};
}

// Row-partial key: high word = order-preserving key of the row maximum, low
// word = ~(global group << 4 | slot): the u64 maximum prefers the larger score,
// then the lower (group, slot), i.e. the lower reference index.
__device__ __forceinline__ uint64_t row_key(float m, uint32_t gslot) {
    return ((uint64_t)fkey(m) << 32) | (uint64_t)(~gslot);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
// All-reduce over the 16 lanes of a DPP row: xor 1, xor 2 (quad permutes),
// half-row mirror, row mirror.
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    return x;
}
__device__ __forceinline__ uint32_t row16_min(uint32_t x) {
    x = min(x, dpp_u<0xB1>(x));
    x = min(x, dpp_u<0x4E>(x));
    x = min(x, dpp_u<0x141>(x));
    x = min(x, dpp_u<0x140>(x));
    return x;
}

// Queries of one unit against the staged chunk: the sub-block's 16-row tiles
// ws, ws + NW, ..., RQ of them; rows past the query count repeat the last
// valid row (no column maximum changes) and are not written back.
template <int DT, int NP, int NKB, int RQ, int NW, bool COLMAX>
__device__ __forceinline__ void sweep_rows(const SweepArgs &p, const unsigned char *Q, const int32_t *qrows, int nq,
                                           int sb_row0, int ws, int np, int TB, int nkb, int ngroups,
                                           const int (&boff)[NKB], uint32_t gbase, uint64_t *rp, float *colmax_lds,
                                           const unsigned char *lds) {
    constexpr int G = group_tiles(DT);
    using T = Tr<DT>;
    using raw = typename T::raw;
    constexpr int PS = T::PS, ESZ = T::ESZ;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
    auto row_of = [&](int qt) { return sb_row0 + (ws + qt * NW) * 16; };

    raw a[RQ][NKB];
#pragma unroll
    for (int qt = 0; qt < RQ; ++qt) {
        int rr = min(row_of(qt) + c, nq - 1);
        const int qrow = qrows ? qrows[rr]
                              : (!COLMAX && p.grid_s > 0) ? grid_seed_pixel(rr, p.grid_s, p.grid_kx, p.grid_w) : rr;
        const unsigned char *qp = Q + (long long)qrow * p.ld * ESZ;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int pc = kb * 4 + g;
            a[qt][kb] = (pc < np) ? *reinterpret_cast<const raw *>(qp + pc * PS) : T::zero();
        }
    }

    // Running row state lives in two register sets that swap roles every
    // group, so no copies are needed between groups.
    float bA[RQ][4], bB[RQ][4];
    int gid[RQ][4];
#pragma unroll
    for (int qt = 0; qt < RQ; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r) { bA[qt][r] = -INFINITY; gid[qt][r] = 0; }

    // ---- per tile pair: B fragments from LDS, MFMAs, epilogue
    auto load_pair = [&](int tile, raw (&b0)[NKB], raw (&b1)[NKB]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            b0[kb] = *reinterpret_cast<const raw *>(lds + tile * TB + boff[kb]);
            b1[kb] = *reinterpret_cast<const raw *>(lds + (tile + 1) * TB + boff[kb]);
        }
    };
    auto mma_pair = [&](const raw (&b0)[NKB], const raw (&b1)[NKB], f32x4_t (&c0)[RQ],
                        f32x4_t (&c1)[RQ]) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < RQ; ++qt) {
            c0[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            c1[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                if (NP > 0 || kb < nkb) {
                    c0[qt] = T::mma(a[qt][kb], b0[kb], c0[qt]);
                    c1[qt] = T::mma(a[qt][kb], b1[kb], c1[qt]);
                }
            }
        }
    };
    // Row state: running maximum of each (row, slot) over the group's tiles,
    // v_max3 consumes one score of each tile of the pair. Columns: in-lane
    // maximum over the unit's rows, one LDS float-max per tile (the four
    // lanes of a column, one per row group, meet in LDS).
    auto epi_pair = [&](const f32x4_t (&c0)[RQ], const f32x4_t (&c1)[RQ], int tile, bool first,
                        float (&bin)[RQ][4], float (&bout)[RQ][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < RQ; ++qt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                bout[qt][r] = fmaxf(fmaxf(first ? bin[qt][r] : bout[qt][r], c0[qt][r]), c1[qt][r]);
        if constexpr (COLMAX) {
            float m0 = fmaxf(c0[0][0], c0[0][1]);
            float m1 = fmaxf(c1[0][0], c1[0][1]);
            m0 = fmaxf(fmaxf(m0, c0[0][2]), c0[0][3]);
            m1 = fmaxf(fmaxf(m1, c1[0][2]), c1[0][3]);
#pragma unroll
            for (int qt = 1; qt < RQ; ++qt) {
                m0 = fmaxf(fmaxf(m0, c0[qt][0]), c0[qt][1]);
                m0 = fmaxf(fmaxf(m0, c0[qt][2]), c0[qt][3]);
                m1 = fmaxf(fmaxf(m1, c1[qt][0]), c1[qt][1]);
                m1 = fmaxf(fmaxf(m1, c1[qt][2]), c1[qt][3]);
            }
            float *cm = colmax_lds + tile * TILE + c;
            __hip_atomic_fetch_max(cm, m0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_max(cm + TILE, m1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    };
    auto mark = [&](int grp, float (&bin)[RQ][4], float (&bout)[RQ][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < RQ; ++qt)
#pragma unroll
            for (int r = 0; r < 4; ++r) gid[qt][r] = (bout[qt][r] > bin[qt][r]) ? grp : gid[qt][r];
    };

    if constexpr (DT == DT_F32) {
        // fp32 maps (narrow K blocks, small maps): plain loop, tile loop kept rolled
        for (int grp = 0; grp < ngroups; ++grp) {
            for (int tp = 0; tp < G; tp += 2) {
                raw b0[NKB], b1[NKB];
                f32x4_t c0[RQ], c1[RQ];
                load_pair(grp * G + tp, b0, b1);
                mma_pair(b0, b1, c0, c1);
                epi_pair(c0, c1, grp * G + tp, tp == 0, bA, bB);
            }
            mark(grp, bA, bB);
#pragma unroll
            for (int qt = 0; qt < RQ; ++qt)
#pragma unroll
                for (int r = 0; r < 4; ++r) bA[qt][r] = bB[qt][r];
        }
    } else {
        // Software pipeline over tile pairs: the next pair's B fragments and
        // MFMAs are issued before the current pair's epilogue, so the matrix
        // cores work while the VALU reduces. Two accumulator sets alternate;
        // the row state alternates between bA and bB every group.
        const int last_tile = ngroups * G - 2;
        raw b0[NKB], b1[NKB];
        f32x4_t xA0[RQ], xA1[RQ], xB0[RQ], xB1[RQ];
        load_pair(0, b0, b1);
        mma_pair(b0, b1, xA0, xA1);
        int grp = 0;
        for (; grp + 1 < ngroups; grp += 2) {
#pragma unroll
            for (int q = 0; q < G; ++q) {
                const int tile = grp * G + 2 * q;
                const int ntile = min(tile + 2, last_tile);
                const bool second = q >= G / 2;
                load_pair(ntile, b0, b1);
                if (q % 2 == 0) {
                    mma_pair(b0, b1, xB0, xB1);
                    if (!second) epi_pair(xA0, xA1, tile, q == 0, bA, bB);
                    else epi_pair(xA0, xA1, tile, q == G / 2, bB, bA);
                } else {
                    mma_pair(b0, b1, xA0, xA1);
                    if (!second) epi_pair(xB0, xB1, tile, false, bA, bB);
                    else epi_pair(xB0, xB1, tile, false, bB, bA);
                }
                if (q == G / 2 - 1) mark(grp, bA, bB);
                if (q == G - 1) mark(grp + 1, bB, bA);
            }
        }
        if (grp < ngroups) {
#pragma unroll
            for (int q = 0; q < G / 2; ++q) {
                const int tile = grp * G + 2 * q;
                const int ntile = min(tile + 2, last_tile);
                load_pair(ntile, b0, b1);
                if (q % 2 == 0) {
                    mma_pair(b0, b1, xB0, xB1);
                    epi_pair(xA0, xA1, tile, q == 0, bA, bB);
                } else {
                    mma_pair(b0, b1, xA0, xA1);
                    epi_pair(xB0, xB1, tile, false, bA, bB);
                }
            }
            mark(grp, bA, bB);
#pragma unroll
            for (int qt = 0; qt < RQ; ++qt)
#pragma unroll
                for (int r = 0; r < 4; ++r) bA[qt][r] = bB[qt][r];
        }
    }

    // ---- row flush: max over the 16 slots of each row, lowest (group, slot) among equals. Every
    // key is computed first, without branches, so the independent DPP chains of all registers
    // can interleave; the stores follow.
    uint64_t key[RQ][4];
#pragma unroll
    for (int qt = 0; qt < RQ; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float bv = bA[qt][r];
            const float m = row16_max(bv);
            const uint32_t id = ((gbase + (uint32_t)gid[qt][r]) << 4) | (uint32_t)c;
            key[qt][r] = row_key(m, row16_min(bv == m ? id : 0xffffffffu));
        }
    if (c == 0) {
#pragma unroll
        for (int qt = 0; qt < RQ; ++qt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = row_of(qt) + 4 * g + r;
                if (row < nq) {
                    if constexpr (COLMAX)     // one key per row, merged over the chunks
                        __hip_atomic_fetch_max(rp + row, key[qt][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else
                        rp[row] = key[qt][r];
                }
            }
    }
}

// sweep_rows with as few query tiles per unit as the sub-block needs (tpw = 16-row
// tiles of its fullest slot): a half-step with few active queries costs a
// fraction of a full one. The fused column-maximum sweep always takes RQ.
template <int DT, int NP, int NKB, int RQ, int NW, bool COLMAX>
__device__ __forceinline__ void sweep_rows_fit(int tpw, const SweepArgs &p, const unsigned char *Q,
                                               const int32_t *qrows, int nq, int sb_row0, int ws, int np, int TB,
                                               int nkb,
                                               int ngroups, const int (&boff)[NKB], uint32_t gbase, uint64_t *rp,
                                               float *colmax_lds, const unsigned char *lds) {
#define DDM_SWEEP_ROWS(RQV) \
    sweep_rows<DT, NP, NKB, RQV, NW, COLMAX>(p, Q, qrows, nq, sb_row0, ws, np, TB, nkb, ngroups, boff, gbase, rp, \
                                             colmax_lds, lds)
    if constexpr (COLMAX) {
        DDM_SWEEP_ROWS(RQ);
    } else {
        if (tpw <= 1) { DDM_SWEEP_ROWS(1); return; }
        if constexpr (RQ > 2) { if (tpw <= 2) { DDM_SWEEP_ROWS(2); return; } }
        if constexpr (RQ > 3) { if (tpw <= 3) { DDM_SWEEP_ROWS(3); return; } }
        if constexpr (RQ > 1) DDM_SWEEP_ROWS(RQ);
    }
#undef DDM_SWEEP_ROWS
}

// NP = pieces (of E elements) per stored row; 0 = runtime (fp32 path).
// NKB = 32-wide (fp16/bf16) or 4-wide (fp32) K blocks.
// One workgroup task: reference chunk chunk_id of pair `pair` against query
// block qblk. The caller owns the LDS (at least sweep_lds bytes: the staged
// chunk, COLMAX's column array, the unit counter) and makes sure no wave still
// reads it from a previous task.
template <int DT, int NP, int NKB, int RQ, int NW, bool COLMAX>
__device__ __forceinline__ void sweep_task(const SweepArgs &p, int pair, int chunk_id, int qblk, unsigned char *lds)
{
    constexpr int G = group_tiles(DT), GROUP = TILE * G;
    using T = Tr<DT>;
    using raw = typename T::raw;
    constexpr int E = T::E, PS = T::PS, ESZ = T::ESZ;
    constexpr int SB_ROWS = NW * RQ * 16;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nq = p.qcount ? p.qcount[pair * p.qcount_bs] : p.nq;
    const SplitGeom sg = split_geom(p.split, nq, p.split_rows, p.qblocks, p.chunk / GROUP, p.nchunks, p.rowcap);
    int qb = qblk, sub = 0;
    if (p.split) {
        qb = qblk % sg.need;
        sub = qblk / sg.need;
        if (sub >= sg.s) return;
    }
    const int spw = sg.spw > 0 ? sg.spw : p.sb_per_wg;
    const int n_sb = (nq + SB_ROWS - 1) / SB_ROWS;
    const int sb_first = qb * spw;
    if (sb_first >= n_sb) return;
    const int sb_last = min(sb_first + spw, n_sb);
    uint64_t *rp = COLMAX ? p.rowpart + pair * p.rowpart_bs
                          : p.rowpart + pair * p.rowpart_bs + (long long)(chunk_id * sg.s + sub) * sg.rowcap;

    const unsigned char *Q = p.Q + pair * p.q_bs;
    const unsigned char *R = p.R + pair * p.r_bs;
    const int32_t *qrows = p.qrows ? p.qrows + pair * p.qrows_bs : nullptr;

    const int np = NP > 0 ? NP : p.ld / E;          // pieces per row
    const int TB = np * 16 * PS;                    // LDS bytes per tile
    const int nkb = NP > 0 ? NKB : (np + 3) / 4;    // K blocks in use
    const int gpc = p.chunk / GROUP;
    const int g0 = gpc * sub / sg.s, g1 = gpc * (sub + 1) / sg.s;
    const int r0 = chunk_id * p.chunk + g0 * GROUP;
    const int nvalid = min((g1 - g0) * GROUP, p.nref - r0);
    if (nvalid <= 0) {
        // a sub-chunk past the last reference: its partials lose to every real one
        for (int row = sb_first * SB_ROWS + tid; row < min(sb_last * SB_ROWS, nq); row += NW * 64) rp[row] = 0;
        return;
    }
    const int ngroups = (nvalid + GROUP - 1) / GROUP;
    const int nslots = ngroups * GROUP;

    // ---- stage the chunk in LDS: slot c of tile t of group q <- reference q*GROUP + G*c + t.
    // The LDS image is written in address order (piece slot qq at byte qq*PS:
    // tile, then piece, then slot); the matching global reads gather 16 rows G
    // apart, which the cache serves since each group's rows are read whole.
    if constexpr (PS == 16) {
        // 16-byte pieces: global_load_lds_dwordx4 moves each lane's piece straight
        // into LDS at the wave's base + 16 * lane, so a wave fills 1 KB per
        // instruction with no register round trip, and every load of the chunk is
        // in flight before the single wait. Slots past the map read the last valid row.
        const int total = nslots * np;
        for (int base = wave * 64; base < total; base += NW * 64) {
            const int qq = base + lane;
            const int tile = qq / (np * 16), rem = qq - tile * (np * 16);
            const int pc = rem >> 4, c = rem & 15;
            const int r = (tile / G) * GROUP + G * c + tile % G;
            const unsigned char *src = R + ((long long)(r0 + min(r, nvalid - 1)) * p.ld + pc * E) * ESZ;
            if (qq < total)
                __builtin_amdgcn_global_load_lds(
                    (const void __attribute__((address_space(1))) *)src,
                    (void __attribute__((address_space(3))) *)(lds + (size_t)base * 16), 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);        // every counter at zero: this wave's LDS loads have landed
    } else {
        // 4-byte pieces (fp32 maps): SU loads per thread in flight before their stores.
        constexpr int SU = 8;
        const int total = nslots * np;
        for (int base = 0; base < total; base += SU * NW * 64) {
            raw v[SU];
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int qq = base + u * NW * 64 + tid;
                const int tile = qq / (np * 16), rem = qq - tile * (np * 16);
                const int pc = rem >> 4, c = rem & 15;
                const int r = (tile / G) * GROUP + G * c + tile % G;
                v[u] = T::zero();
                if (qq < total)
                    v[u] = *reinterpret_cast<const raw *>(R + ((long long)(r0 + min(r, nvalid - 1)) * p.ld + pc * E) * ESZ);
            }
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int qq = base + u * NW * 64 + tid;
                if (qq >= total) break;
                *reinterpret_cast<raw *>(lds + (size_t)qq * PS) = v[u];
            }
        }
    }
    float *colmax_lds = reinterpret_cast<float *>(lds + (size_t)(p.chunk / TILE) * TB);
    int *next_unit = reinterpret_cast<int *>(lds + (size_t)(p.chunk / TILE) * TB + (COLMAX ? (size_t)p.chunk * 4 : 0));
    if constexpr (COLMAX) {
        for (int s = tid; s < nslots; s += NW * 64) colmax_lds[s] = -INFINITY;
    }
    if (tid == 0) *next_unit = NW;
    __syncthreads();

    const int c = lane & 15, g = lane >> 4;
    int boff[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        const int pc = min(kb * 4 + g, np - 1);     // lanes past the last piece re-read it; A is 0 there
        boff[kb] = pc * 16 * PS + c * PS;
    }
    const uint32_t gbase = (uint32_t)(r0 / GROUP);

    // units u = (sub-block sb_first + u / NW, slot u % NW): wave w starts with unit w, the later ones
    // go in order to whichever wave asks next (no counter traffic when a task has one sub-block); a
    // unit's rows and results do not depend on the wave that runs it
    const int units = (sb_last - sb_first) * NW;
    int u = __builtin_amdgcn_readfirstlane(wave);     // uniform over the wave: scalar unit arithmetic
    while (u < units) {
        const int sb_row0 = (sb_first + u / NW) * SB_ROWS, ws = u % NW;
        const int tiles = (min(SB_ROWS, nq - sb_row0) + 15) / 16;     // 16-row tiles holding queries
        if (ws < tiles)
            sweep_rows_fit<DT, NP, NKB, RQ, NW, COLMAX>((tiles + NW - 1) / NW, p, Q, qrows, nq, sb_row0, ws, np,
                                                        TB, nkb, ngroups, boff, gbase, rp, colmax_lds, lds);
        if (units <= NW) break;
        int next = 0;
        if (lane == 0) next = atomicAdd(next_unit, 1);
        u = __builtin_amdgcn_readfirstlane(next);       // lane 0's value: every lane is active here
    }

    if constexpr (COLMAX) {
        __syncthreads();
        // column maxima of this query block, merged into the column keys: the larger maximum wins,
        // the lower query block among equal maxima (its complement is the larger low word)
        uint64_t *ck = p.colkey + r0;
        const uint64_t low = (uint64_t)(~(uint32_t)qblk);
        for (int s = tid; s < nslots; s += NW * 64) {
            const int tile = s / TILE, slot = s % TILE;
            const int r = (tile / G) * GROUP + slot * G + (tile % G);
            if (r < nvalid)
                __hip_atomic_fetch_max(ck + r, ((uint64_t)fkey(colmax_lds[s]) << 32) | low, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int DT, int NP, int NKB, int RQ, int NW, bool COLMAX>
__global__ void __launch_bounds__(NW * 64)
sweep_kernel(SweepArgs p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    sweep_task<DT, NP, NKB, RQ, NW, COLMAX>(p, blockIdx.z, blockIdx.x, blockIdx.y, lds);
}

}  // namespace ddm
