/*
 * ddm.h -- C ABI of the MI355X (gfx950) dense descriptor matching library.
 *
 * What is computed (cited by page title and section):
 *  - Descriptor maps: D1 in R^{H1 x W1 x d}, D2 in R^{H2 x W2 x d}, one d-vector
 *    per pixel, unit L2 norm as produced by MASt3R's matching head ("MASt3R"
 *    note on cv-learn.com, section 手法とアーキテクチャ, matching-head paragraph).
 *  - NN_2(x): the pixel j of image 2 maximising the dot product <x, D2_j>, the
 *    lowest j on exact ties; NN_1 likewise over image 1 (same note, FRM
 *    paragraph, where NN is the nearest-neighbour function of the reciprocal set).
 *  - Exhaustive reciprocal set M = {(i, j) : j = NN_2(D1_i) and i = NN_1(D2_j)}
 *    (same note, FRM paragraph).
 *  - Fast Reciprocal Matching: k seeds on a regular grid, NN round trips
 *    U^t -> V^t -> U^{t+1}, keep the seeds whose trajectory cycles (same note,
 *    FRM paragraph), run as the fast_reciprocal_NNs routine quoted in
 *    "DUSt3R和MASt3R论文阅读" (Staskaer blog, section MASt3R matching): seed grid,
 *    forward query, test against the previous image-2 pixel, backward query,
 *    test against the previous image-1 pixel, at most max_iter iterations,
 *    converged = no longer active, unique pairs sorted by the image-1 index.
 *
 * Conventions shared by every entry point:
 *  - Maps are row-major [H][W][d] (pixel p = x + W*y, then d components),
 *    contiguous, in device memory, 16-byte aligned (fp16/bf16) or 4-byte
 *    aligned (fp32). Values must be finite, and dot products within the fp32
 *    range (unit-norm descriptors are far inside). Element types: DDM_F32 (float),
 *    DDM_F16 (IEEE binary16), DDM_BF16 (bfloat16); products are accumulated in
 *    fp32 (fp16/bf16 products are exact in fp32).
 *  - All device buffers (inputs, outputs, workspace) belong to the caller. The
 *    library never allocates device memory; it asks for a workspace of the size
 *    the matching *_workspace_bytes function returns and uses it as scratch.
 *  - Calls only enqueue work on `stream` and return; outputs (including device
 *    counts) are valid once the stream has reached that point.
 *  - Argument errors are detected on the host before anything is enqueued and
 *    leave every output untouched. Status codes are the ddm_status values; a HIP
 *    launch failure is reported as DDM_ERR_HIP. Calls that share a workspace
 *    must not overlap on the device.
 *  - Scores are the fp32 dot products computed by the matrix cores.
 *  - Limits: 1 <= d <= 128, H*W < 2^31 / 16 pixels per map.
 */
#ifndef DDM_H
#define DDM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DDM_F32 = 0, DDM_F16 = 1, DDM_BF16 = 2 } ddm_dtype;

/* Similarity of the *_ex entry points.
 *   DDM_DOT: NN = arg-max of the dot product (descriptor maps; every other entry point).
 *   DDM_L2:  NN = arg-min of the Euclidean distance, for 3D points (pointmaps, d = 3), which
 *            the pages match with K-d trees ("DUSt3R和MASt3R论文阅读", section MASt3R
 *            matching); here by the same brute-force sweep: fp32 maps only, d <= DDM_MAX_D - 2,
 *            lowest index on exact ties, reported scores are squared distances (>= 0). */
typedef enum { DDM_DOT = 0, DDM_L2 = 1 } ddm_metric;

typedef enum {
    DDM_OK = 0,
    DDM_ERR_INVALID = -1,     /* null pointer, bad size, misaligned or bad parameter */
    DDM_ERR_CAPACITY = -2,    /* output capacity below the largest possible result */
    DDM_ERR_WORKSPACE = -3,   /* workspace null or smaller than required */
    DDM_ERR_UNSUPPORTED = -4, /* dtype or d outside what the kernels handle */
    DDM_ERR_HIP = -5          /* a HIP call failed while enqueueing */
} ddm_status;

#define DDM_MAX_D 128
#define DDM_MAX_ITER 64

/* Human-readable name of a status code (static string). */
const char *ddm_status_str(int status);

/* Number of grid seeds for an H x W image with stride S: the seed grid of the
 * quoted fast_reciprocal_NNs routine, rows S/2, S/2+S, ... < H and columns
 * S/2, S/2+S, ... < W. Returns -1 for S <= 0 or negative sizes. */
int64_t ddm_seed_count(int H, int W, int grid_stride);

/* ---------------------------------------------------------------- NN ----
 * Brute-force nearest neighbour (argmax of the dot product, lowest index on
 * exact ties) of M query rows against all N reference rows.
 *   Q       [NQ][d] query map; query a is row q_rows[a] (or row a when q_rows
 *           is NULL, which needs NQ >= M)
 *   q_rows  device int32[M] with entries in [0, NQ), or NULL; an entry outside
 *           [0, NQ) reads no memory outside Q and yields out_idx -1, out_score NaN
 *   R       [N][d] reference map
 *   out_idx device int32[M]: NN index in [0, N)
 *   out_score device float[M]: the fp32 dot product of the pair
 */
size_t ddm_nn_workspace_bytes(int NQ, int M, int N, int d, int dtype);
int ddm_nn(const void *Q, int NQ, const int32_t *q_rows, int M, const void *R, int N, int d, int dtype,
           int32_t *out_idx, float *out_score, void *workspace, size_t workspace_bytes,
           hipStream_t stream);
/* The same with a metric (ddm_metric); DDM_DOT is exactly ddm_nn. */
size_t ddm_nn_ex_workspace_bytes(int NQ, int M, int N, int d, int dtype, int metric);
int ddm_nn_ex(const void *Q, int NQ, const int32_t *q_rows, int M, const void *R, int N, int d, int dtype,
              int metric, int32_t *out_idx, float *out_score, void *workspace, size_t workspace_bytes,
              hipStream_t stream);

/* ---------------------------------------------------------------- FRM ---
 * Fast Reciprocal Matching from the stride-`grid_stride` seed grid of image 1
 * with at most `max_iter` iterations (1..DDM_MAX_ITER). Outputs are the unique
 * converged pairs (i in image 1, j in image 2) as linear pixel indices,
 * strictly ascending in i, with their fp32 scores:
 *   out_i, out_j, out_score  device arrays of `capacity` entries;
 *                            capacity >= ddm_seed_count(H1, W1, grid_stride)
 *   out_count                device int32: number of pairs written
 *   seed_state               device int32[k][4] or NULL: per seed (in grid
 *                            order) u, v, iteration in which it converged
 *                            (-1 if it did not), u_old (see ddm_frm_match_ex)
 *   query_counts             device int32[2*max_iter] or NULL: number of
 *                            forward / backward NN queries in each iteration
 *                            (entry 2t = forward, 2t+1 = backward of iteration t+1)
 * k = 0 (stride larger than the image) is valid and yields 0 pairs.
 * out_count = -1 reports a failed device-wide synchronisation of the loop
 * kernel (modes below); the other outputs are then undefined. Not expected in
 * normal operation: that mode never launches more workgroups than the device
 * keeps resident, and its barrier waits are bounded so the call always ends. */
size_t ddm_frm_workspace_bytes(int B, int H1, int W1, int H2, int W2, int d, int dtype,
                               int grid_stride, int max_iter);
int ddm_frm_match(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype,
                  int grid_stride, int max_iter,
                  int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity, int32_t *out_count,
                  int32_t *seed_state, int32_t *query_counts,
                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ddm_frm_match for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). Same arguments, kernels and results as
 * ddm_frm_match, without the workspace: the call uses a device array the library holds, one per
 * device, DDM_NOALLOC_SCRATCH_BYTES in size, until the process ends. It calls no allocating
 * routine and instantiates no graph (launches go straight onto `stream`, so they can be captured
 * into the caller's graph); DDM_FRM_LOOP runs as DDM_FRM_TAIL (identical results) and no timing
 * events are recorded. A problem whose ddm_frm_workspace_bytes(1, ...) exceeds
 * DDM_NOALLOC_SCRATCH_BYTES is rejected with DDM_ERR_WORKSPACE before anything is enqueued.
 * Every call on one device shares that device's array and leaves its contents behind (each call
 * initialises what it reads): calls that may overlap on one device (different streams, or
 * threads) race and must be serialised by the caller. */
#define DDM_NOALLOC_SCRATCH_BYTES (64u << 20)
int ddm_frm_match_noalloc(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype,
                          int grid_stride, int max_iter,
                          int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity, int32_t *out_count,
                          int32_t *seed_state, int32_t *query_counts, hipStream_t stream);

/* Statistics of one FRM call, derived on the host from its query_counts (copied to host memory
 * after the stream has passed the call; the call itself never waits for the device):
 *   iters         iterations that ran, the last one with at least one forward query
 *   active[2t]    seeds active in the forward half-step of iteration t+1 (= its forward queries),
 *   active[2t+1]  seeds still active for its backward half-step; zero past iters
 *   dot_products  sum over iterations of forward queries x N2 + backward queries x N1
 * ddm_frm_stats fills stats[b] for each of B pairs from query_counts_host [B][2*max_iter].
 * Returns DDM_ERR_INVALID for null pointers, B < 1, max_iter outside 1..DDM_MAX_ITER or negative
 * sizes or counts. */
typedef struct {
    int32_t iters;
    int32_t active[2 * DDM_MAX_ITER];
    int64_t dot_products;
} ddm_stats;
int ddm_frm_stats(const int32_t *query_counts_host, int B, int max_iter, int64_t N1, int64_t N2, ddm_stats *stats);

/* B independent pairs in one call: D1 is [B][H1][W1][d], D2 is [B][H2][W2][d].
 * Pair b writes its pairs at out_*[b * capacity ...] and its count at
 * out_count[b]; seed_state is [B][k][4] and query_counts [B][2*max_iter].
 * Each pair's result equals a single ddm_frm_match call on that pair. */
int ddm_frm_match_batched(int B, const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d,
                          int dtype, int grid_stride, int max_iter,
                          int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity,
                          int32_t *out_count, int32_t *seed_state, int32_t *query_counts,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* FRM with the routine's other options ("DUSt3R和MASt3R论文阅读", section MASt3R matching, the quoted
 * fast_reciprocal_NNs routine; one pair):
 *   starts      NULL: seeds on the stride-`grid_stride` grid as in ddm_frm_match.
 *               Else device int32[n_starts] linear image-1 pixels (p = x + W1*y); entries outside
 *               [0, H1*W1) are ignored, the rest are made unique and ascending (k = their number).
 *               The routine runs one iteration for such starts; max_iter is still the caller's.
 *   pixel_tol   0: a seed's pair is kept when the seed is no longer active at the end (as in
 *               ddm_frm_match). > 0 (explicit starts only, else DDM_ERR_INVALID): a seed is kept
 *               when the Euclidean distance in pixels between u_old and u is below pixel_tol, and
 *               its pair is reported at u_old, where u_old is the seed's image-1 pixel at the start
 *               of the last iteration if the loop ran all max_iter iterations, else its final pixel
 *               (with max_iter = 1: the start itself).
 *   basin       NULL, or device int32[H1*W1]: the basin variant. The forward test is off (a seed
 *               stops only when its backward query returns the pixel it started the iteration
 *               from) and every backward query of a seed standing at pixel p stores the pixel it
 *               moved to at basin[p]; pixels never left by a backward query hold -1.
 *   metric      ddm_metric (DDM_L2 for pointmaps; scores are then squared distances).
 *   capacity    >= k (ddm_seed_count for the grid, n_starts for explicit starts).
 *   seed_state  as for ddm_frm_match, with entry 3 = u_old; rows past the number of distinct
 *               starts are -1.
 * The workspace size comes from ddm_frm_ex_workspace_bytes with n_starts = -1 for the grid. */
size_t ddm_frm_ex_workspace_bytes(int H1, int W1, int H2, int W2, int d, int dtype, int metric,
                                  int grid_stride, int n_starts, int max_iter);
int ddm_frm_match_ex(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype,
                     int metric, int grid_stride, const int32_t *starts, int n_starts, int max_iter,
                     double pixel_tol,
                     int32_t *basin,
                     int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity, int32_t *out_count,
                     int32_t *seed_state, int32_t *query_counts,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* How FRM calls are executed (process-wide; results are identical):
 *   DDM_FRM_PER_HALF_STEP: a sweep and an update launch for every
 *     half-step of all max_iter iterations. Both kernels stride over the
 *     active work only, so the half-steps after convergence cost a few
 *     microseconds each.
 *   DDM_FRM_LOOP: every iteration in one cooperative kernel that loops over
 *     the half-steps with grid barriers and stops as soon as no seed is active
 *     (the device must support cooperative launches, else per half-step).
 *     Its barriers cost more than kernel boundaries on large maps; on small
 *     ones it beats per-half-step launches but not DDM_FRM_TAIL.
 *   DDM_FRM_TAIL (default): the first iterations per half-step (see
 *     ddm_frm_set_tail_after), the rest in one plain kernel launch whose
 *     workgroups take the remaining tasks in a global order from a ticket
 *     counter and stop as soon as no seed is active, so the iterations after
 *     convergence cost nothing. No co-residency is needed: a workgroup only
 *     waits for tasks handed out before its own. Its waits are bounded like
 *     the loop kernel's barriers (out_count = -1 past the bound).
 * The launch sequence of a call is recorded once into a HIP graph, cached under
 * the call's argument values and the mode, and replayed; on a stream that is
 * being captured it is recorded into the caller's graph.
 * ddm_frm_set_mode returns DDM_ERR_INVALID for other values. */
typedef enum { DDM_FRM_PER_HALF_STEP = 0, DDM_FRM_LOOP = 1, DDM_FRM_TAIL = 2 } ddm_frm_mode;
int ddm_frm_set_mode(int mode);
int ddm_frm_get_mode(void);
/* Iterations run per half-step before the tail kernel takes over in DDM_FRM_TAIL (0..DDM_MAX_ITER;
 * 0 runs every half-step in the tail kernel). -1 (the default) chooses by size, in half-steps:
 * with w = pairs x seeds x image-2 pixels, the tail kernel starts after 2 half-steps when
 * w <= 2^24, 3 when w <= 2^27, 5 when w <= 2^31, else 8. Process-wide; DDM_ERR_INVALID outside
 * -1..DDM_MAX_ITER. */
int ddm_frm_set_tail_after(int iterations);
/* Test aid for the failure path of DDM_FRM_LOOP and DDM_FRM_TAIL: the number of polls a wait makes
 * before giving up (0 restores the default of 2^20, about 1 s). A tiny value makes the loop
 * kernel's barriers time out on purpose (and any tail-kernel wait that does not end at once); the
 * kernel still ends and out_count reads -1. Process-wide; the value is part of the graph-cache
 * key (a changed value records a new graph). */
int ddm_frm_set_barrier_polls(int polls);
/* Test aid against races between workgroups: caps the grid of the FRM sweep, update, loop and
 * tail kernels (which spread their tasks over whatever grid they get) at max_workgroups; 0 removes
 * the cap. Outputs must be bit-identical with any cap; 1 runs every task in one workgroup.
 * Process-wide; the value is part of the graph-cache key (a changed value records a new graph). */
int ddm_debug_set_grid_cap(int max_workgroups);
/* Test aid for the two output paths of FRM: a call whose image 1 has at most max_pixels pixels (and
 * at most 4096 seeds per pair) collects and orders its pairs in one workgroup per pair through a
 * bitmap of image-1 pixels in LDS; larger ones use a collection kernel and a multi-workgroup
 * compaction of a dense match array. Both give identical outputs. -1 restores the default (2^19,
 * also the maximum); 0 sends every call down the multi-workgroup path. Process-wide;
 * the value is part of the graph-cache key (a changed value records a new graph). DDM_ERR_INVALID below -1. */
int ddm_debug_set_output_bitmap_limit(int max_pixels);

/* ----------------------------------------------------- coarse-to-fine ---
 * Matching of maps larger than the network's 512-px input ("MASt3R" note on cv-learn.com,
 * section 手法とアーキテクチャ, 粗密マッチング paragraph: coarse matching first, the coarse
 * correspondences guide the matching of enumerated local crops, fine matches mapped back to
 * the original resolution). Steps, as read here (the page gives no further rule):
 *   1. coarse maps: every `factor`-th row and column of F1 and F2 (from 0);
 *   2. coarse pairs: FRM on them (grid stride coarse_stride, coarse_iter iterations);
 *   3. image-1 crops: the tiling of image 1 by crop_h x crop_w windows, raster order, the last
 *      window of a row / column moved back to end at the border;
 *   4. image-2 crop of each tile: same size, centred on the lower medians of the image-2 x and y
 *      (full resolution) of the coarse pairs whose image-1 pixel lies in the tile (offset =
 *      median - size / 2, clamped into image 2); tiles without coarse pairs are skipped;
 *   5. fine pairs: FRM on every crop pair (grid stride fine_stride, fine_iter iterations), mapped
 *      to full-resolution indices; a pixel reported by several tiles keeps the first tile's pair.
 * Outputs as for ddm_frm_match (unique, ascending in i, fp32 dot products);
 * capacity >= min(H1*W1, tiles * ddm_seed_count(crop_h, crop_w, fine_stride)).
 *   crop_info  device int32[tiles][5] or NULL: x0_1, y0_1, x0_2, y0_2, coarse pairs in the tile.
 * Requires crop sizes within both maps, factor >= 1, d * element size a multiple of 4 bytes,
 * W2 + H2 < 16384. FRM calls inside follow ddm_frm_set_mode; out_count = -1 when one of them
 * reported a failed synchronisation (as for ddm_frm_match). */
size_t ddm_c2f_workspace_bytes(int H1, int W1, int H2, int W2, int d, int dtype, int factor,
                               int coarse_stride, int coarse_iter, int crop_h, int crop_w,
                               int fine_stride, int fine_iter);
int ddm_c2f_match(const void *F1, int H1, int W1, const void *F2, int H2, int W2, int d, int dtype,
                  int factor, int coarse_stride, int coarse_iter, int crop_h, int crop_w,
                  int fine_stride, int fine_iter,
                  int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity, int32_t *out_count,
                  int32_t *crop_info, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------- mutual NN ---
 * Exhaustive reciprocal nearest neighbours M (ascending in i), computed in a
 * single pass over all N1 x N2 scores with row arg-max and column max fused.
 *   capacity >= min(H1*W1, H2*W2); out_count as for FRM.
 *   nn12, s12  device int32[N1] / float[N1] or NULL: NN_2 of every pixel of
 *              image 1 and its score.
 * Ties: both nearest neighbours take the lowest index, so every j appears at most once.
 * (i, j) needs NN_2(i) = j, score(i, j) equal to column j's maximum, no earlier block of
 * query rows reaching that maximum, and no lower row of the same block passing the same
 * test; a lower row of that block whose own maximum lies elsewhere but ties in column j is
 * not looked for (the pair is then reciprocal up to an exact tie). */
size_t ddm_mutual_workspace_bytes(int H1, int W1, int H2, int W2, int d, int dtype);
int ddm_mutual_nn(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype,
                  int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity, int32_t *out_count,
                  int32_t *nn12, float *s12,
                  void *workspace, size_t workspace_bytes, hipStream_t stream);
/* The same with a metric (ddm_metric); DDM_DOT is exactly ddm_mutual_nn. */
size_t ddm_mutual_ex_workspace_bytes(int H1, int W1, int H2, int W2, int d, int dtype, int metric);
int ddm_mutual_nn_ex(const void *D1, int H1, int W1, const void *D2, int H2, int W2, int d, int dtype,
                     int metric, int32_t *out_i, int32_t *out_j, float *out_score, int32_t capacity,
                     int32_t *out_count, int32_t *nn12, float *s12,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------- kernel timing ---
 * Benchmark aid, off by default. ddm_profile_enable(mask) makes later calls
 * bracket each fused NN sweep launch with two HIP events on the call's stream:
 * mask bit 0 = the mutual-NN sweep, bit 1 = the NN / FRM sweeps (and the FRM
 * loop kernel as a whole), 0 = off (the library then creates no events). Bit 1
 * also makes FRM calls launch directly instead of through the graph cache. ddm_profile_read waits for the recorded
 * events, returns the summed elapsed milliseconds and the number of launches,
 * and forgets them. Events are created on first use and kept for reuse. */
int ddm_profile_enable(int mask);
int ddm_profile_read(double *total_ms, int64_t *launches);

/* ------------------------------------------------------------ resources ---
 * Per process the library keeps the instantiated HIP graphs of recent FRM and
 * coarse-to-fine calls (each with an event recorded after its latest replay), one
 * private capture stream per device and the timing events of ddm_profile_enable.
 * ddm_release_cached_resources waits until each cached graph's latest replay has
 * finished, then destroys all of them; later calls recreate what they need. Call it
 * while the HIP runtime is still up: before leaving main, before hipDeviceReset
 * (the Python binding registers it to run at interpreter exit). It must not overlap
 * another call into the library. Returns DDM_OK, or DDM_ERR_HIP if a HIP call failed
 * (everything is released regardless). */
int ddm_release_cached_resources(void);

#ifdef __cplusplus
}
#endif
#endif /* DDM_H */
