// ddm_c2f.hpp -- coarse-to-fine crop matching around the FRM kernels.
//
// The "MASt3R" note on cv-learn.com (section 手法とアーキテクチャ, 粗密マッチング
// paragraph): the network takes at most 512 px per side, so high-resolution
// images are matched coarsely first, the coarse correspondences guide the
// matching of enumerated local crops, and the fine matches are mapped back to
// the original resolution. Reading used here (the page gives no further rule):
// coarse maps = every factor-th row and column; coarse pairs = FRM on them;
// image-1 crops = the tiling of image 1 by crop_h x crop_w windows (the last
// window of a row / column moved back to end at the border); image-2 crop of a
// tile = the window of the same size centred on the lower medians of the
// image-2 x and y of the tile's coarse pairs, clamped into image 2; fine pairs
// = batched FRM over the crop pairs, mapped to full-resolution indices, the
// first crop (raster order) keeping a pixel reported by several.
#pragma once
#include "ddm_aux.hpp"

namespace ddm {

// Every factor-th row and column of a [H][W] map of rows of `words` 32-bit words.
__global__ void __launch_bounds__(256) subsample_kernel(const uint32_t *src, int W, int words, int factor, int Hc,
                                                        int Wc, uint32_t *dst) {
    const long long total = (long long)Hc * Wc * words;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
        const long long p = e / words;
        const int w = (int)(e - p * words);
        const int yc = (int)(p / Wc), xc = (int)(p - (long long)yc * Wc);
        dst[e] = src[((long long)yc * factor * W + (long long)xc * factor) * words + w];
    }
}

struct CropGeom {
    int H1, W1, H2, W2, CH, CW, ntx, nty, factor, Wc1, Wc2;
};

__device__ __forceinline__ void tile_origin(const CropGeom &g, int t, int *x0, int *y0) {
    const int ty = t / g.ntx, tx = t - ty * g.ntx;
    *y0 = min(ty * g.CH, g.H1 - g.CH);
    *x0 = min(tx * g.CW, g.W1 - g.CW);
}

// One workgroup per image-1 tile: histograms (LDS, W2 + H2 counters) of the
// image-2 x and y of the coarse pairs whose image-1 position lies in the tile,
// lower medians, image-2 window. crop_info[t] = (x0_1, y0_1, x0_2, y0_2, n).
__global__ void __launch_bounds__(256) crop_stats_kernel(const int32_t *ci, const int32_t *cj, const int32_t *ccount,
                                                         CropGeom g, int32_t *crop_info) {
    extern __shared__ int hist[];          // [W2] x counts, [H2] y counts, [1] total
    int *hx = hist, *hy = hist + g.W2, *hn = hist + g.W2 + g.H2;
    const int t = blockIdx.x;
    int x0, y0;
    tile_origin(g, t, &x0, &y0);
    for (int k = threadIdx.x; k <= g.W2 + g.H2; k += 256) hist[k] = 0;
    __syncthreads();
    const int n = ccount[0];
    for (int e = threadIdx.x; e < n; e += 256) {
        const int a = ci[e], b = cj[e];
        const int x1 = (a % g.Wc1) * g.factor, y1 = (a / g.Wc1) * g.factor;
        if (x1 < x0 || x1 >= x0 + g.CW || y1 < y0 || y1 >= y0 + g.CH) continue;
        const int x2 = (b % g.Wc2) * g.factor, y2 = (b / g.Wc2) * g.factor;
        atomicAdd(&hx[x2], 1);
        atomicAdd(&hy[y2], 1);
        atomicAdd(hn, 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int m = *hn;
        int x02 = 0, y02 = 0;
        if (m > 0) {
            const int target = (m - 1) / 2;      // lower median: the (target+1)-th smallest value
            int mx = 0, my = 0, c = 0;
            for (int v = 0; v < g.W2; ++v) { c += hx[v]; if (c > target) { mx = v; break; } }
            c = 0;
            for (int v = 0; v < g.H2; ++v) { c += hy[v]; if (c > target) { my = v; break; } }
            x02 = min(max(mx - g.CW / 2, 0), g.W2 - g.CW);
            y02 = min(max(my - g.CH / 2, 0), g.H2 - g.CH);
        }
        int32_t *o = crop_info + 5 * t;
        o[0] = x0; o[1] = y0; o[2] = x02; o[3] = y02; o[4] = m;
    }
}

// Copy every crop pair into the batch [tile][CH][CW] (rows of `words` words).
__global__ void __launch_bounds__(256) crop_gather_kernel(const uint32_t *F1, const uint32_t *F2, int words,
                                                          CropGeom g, const int32_t *crop_info, uint32_t *b1,
                                                          uint32_t *b2) {
    const int t = blockIdx.y;
    const int32_t *o = crop_info + 5 * t;
    const int x01 = o[0], y01 = o[1], x02 = o[2], y02 = o[3];
    const long long per = (long long)g.CH * g.CW * words;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < per; e += (long long)gridDim.x * 256) {
        const long long p = e / words;
        const int w = (int)(e - p * words);
        const int y = (int)(p / g.CW), x = (int)(p - (long long)y * g.CW);
        b1[t * per + e] = F1[((long long)(y + y01) * g.W1 + x + x01) * words + w];
        b2[t * per + e] = F2[((long long)(y + y02) * g.W2 + x + x02) * words + w];
    }
}

// Full-resolution image-1 index of crop-local pixel i of tile t.
__device__ __forceinline__ int crop_to_full1(const CropGeom &g, const int32_t *o, int i) {
    return (i / g.CW + o[1]) * g.W1 + i % g.CW + o[0];
}

// Merge, pass 1: owner[I] = first tile (lowest index) whose fine pairs report I.
__global__ void __launch_bounds__(256) crop_owner_kernel(const int32_t *fi, const int32_t *fcount, int kf, CropGeom g,
                                                         const int32_t *crop_info, int32_t *owner) {
    const int t = blockIdx.y;
    const int32_t *o = crop_info + 5 * t;
    if (o[4] == 0) return;
    const int n = fcount[t];
    for (int e = blockIdx.x * 256 + threadIdx.x; e < n; e += gridDim.x * 256)
        atomicMin(&owner[crop_to_full1(g, o, fi[(long long)t * kf + e])], t);
}

// Merge, pass 2: the owner writes its pair into the dense full-resolution arrays.
__global__ void __launch_bounds__(256) crop_write_kernel(const int32_t *fi, const int32_t *fj, const float *fs,
                                                         const int32_t *fcount, int kf, CropGeom g,
                                                         const int32_t *crop_info, const int32_t *owner,
                                                         int32_t *match_j, float *match_s) {
    const int t = blockIdx.y;
    const int32_t *o = crop_info + 5 * t;
    if (o[4] == 0) return;
    const int n = fcount[t];
    for (int e = blockIdx.x * 256 + threadIdx.x; e < n; e += gridDim.x * 256) {
        const long long q = (long long)t * kf + e;
        const int I = crop_to_full1(g, o, fi[q]);
        if (owner[I] != t) continue;
        const int j = fj[q];
        match_j[I] = (j / g.CW + o[3]) * g.W2 + j % g.CW + o[2];
        match_s[I] = fs[q];
    }
}

// flag = 1 when the coarse FRM or any tile's fine FRM reported failure (count -1).
__global__ void __launch_bounds__(256) c2f_status_kernel(const int32_t *ccount, const int32_t *fcount, int ntiles,
                                                         int32_t *flag) {
    int bad = threadIdx.x == 0 && ccount[0] < 0;
    for (int t = threadIdx.x; t < ntiles; t += 256) bad |= fcount[t] < 0;
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) *flag = bad;
}

__global__ void __launch_bounds__(256) c2f_clear_kernel(int32_t *owner, int32_t *match_j, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
        owner[i] = 0x7fffffff;
        match_j[i] = -1;
    }
}

}  // namespace ddm
