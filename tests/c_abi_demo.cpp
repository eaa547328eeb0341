// c_abi_demo.cpp -- drives the C ABI of libddm.so from plain host code (no torch):
// device buffers from hipMalloc, workspace sizes from the *_workspace_bytes
// queries, one FRM call and one mutual-NN call on the default stream.
//
// usage: c_abi_demo IN OUT
//   IN : int32 H1 W1 H2 W2 d dtype grid_stride max_iter, then the two maps' bytes
//   OUT: int32 status_frm, count_frm, pairs (i, j) as int32 and scores as float;
//        then status_mutual, count_mutual, pairs and scores likewise
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "ddm.h"

namespace {

bool check(hipError_t e, const char *what) {
    if (e != hipSuccess) std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return e == hipSuccess;
}

struct Pairs {
    int status = 0, count = 0;
    std::vector<int32_t> i, j;
    std::vector<float> s;
};

bool fetch(Pairs &p, const int32_t *di, const int32_t *dj, const float *ds, const int32_t *dcount) {
    if (!check(hipMemcpy(&p.count, dcount, 4, hipMemcpyDeviceToHost), "count")) return false;
    if (p.count < 0) return true;
    p.i.resize(p.count); p.j.resize(p.count); p.s.resize(p.count);
    if (p.count == 0) return true;
    return check(hipMemcpy(p.i.data(), di, p.count * 4, hipMemcpyDeviceToHost), "i") &&
           check(hipMemcpy(p.j.data(), dj, p.count * 4, hipMemcpyDeviceToHost), "j") &&
           check(hipMemcpy(p.s.data(), ds, p.count * 4, hipMemcpyDeviceToHost), "s");
}

void put(FILE *f, const Pairs &p) {
    std::fwrite(&p.status, 4, 1, f);
    std::fwrite(&p.count, 4, 1, f);
    if (p.count > 0) {
        std::fwrite(p.i.data(), 4, p.count, f);
        std::fwrite(p.j.data(), 4, p.count, f);
        std::fwrite(p.s.data(), 4, p.count, f);
    }
}

}  // namespace

int main(int argc, char **argv) {
    if (argc != 3) { std::fprintf(stderr, "usage: %s IN OUT\n", argv[0]); return 2; }
    FILE *in = std::fopen(argv[1], "rb");
    if (!in) { std::perror(argv[1]); return 2; }
    int32_t hdr[8];
    if (std::fread(hdr, 4, 8, in) != 8) { std::fprintf(stderr, "short header\n"); return 2; }
    const int H1 = hdr[0], W1 = hdr[1], H2 = hdr[2], W2 = hdr[3], d = hdr[4], dtype = hdr[5];
    const int S = hdr[6], max_iter = hdr[7];
    const size_t esz = dtype == DDM_F32 ? 4 : 2;
    const size_t b1 = (size_t)H1 * W1 * d * esz, b2 = (size_t)H2 * W2 * d * esz;
    std::vector<unsigned char> h1(b1), h2(b2);
    if (std::fread(h1.data(), 1, b1, in) != b1 || std::fread(h2.data(), 1, b2, in) != b2) {
        std::fprintf(stderr, "short maps\n");
        return 2;
    }
    std::fclose(in);

    void *D1 = nullptr, *D2 = nullptr;
    if (!check(hipMalloc(&D1, b1), "D1") || !check(hipMalloc(&D2, b2), "D2")) return 1;
    if (!check(hipMemcpy(D1, h1.data(), b1, hipMemcpyHostToDevice), "copy D1") ||
        !check(hipMemcpy(D2, h2.data(), b2, hipMemcpyHostToDevice), "copy D2"))
        return 1;
    const int cap = (int)std::max<int64_t>(1, ddm_seed_count(H1, W1, S));
    const int mcap = std::min(H1 * W1, H2 * W2);
    const int ocap = std::max(cap, mcap);
    int32_t *oi = nullptr, *oj = nullptr, *ocount = nullptr;
    float *os = nullptr;
    if (!check(hipMalloc(&oi, ocap * 4), "oi") || !check(hipMalloc(&oj, ocap * 4), "oj") ||
        !check(hipMalloc(&os, ocap * 4), "os") || !check(hipMalloc(&ocount, 4), "count"))
        return 1;

    Pairs frm, mut;
    const size_t wf = ddm_frm_workspace_bytes(1, H1, W1, H2, W2, d, dtype, S, max_iter);
    const size_t wm = ddm_mutual_workspace_bytes(H1, W1, H2, W2, d, dtype);
    void *ws = nullptr;
    if (!check(hipMalloc(&ws, std::max<size_t>(std::max(wf, wm), 1)), "workspace")) return 1;

    frm.status = ddm_frm_match(D1, H1, W1, D2, H2, W2, d, dtype, S, max_iter, oi, oj, os, cap, ocount, nullptr,
                               nullptr, ws, wf, 0);
    if (frm.status == DDM_OK && (!check(hipStreamSynchronize(0), "frm") || !fetch(frm, oi, oj, os, ocount))) return 1;
    mut.status = ddm_mutual_nn(D1, H1, W1, D2, H2, W2, d, dtype, oi, oj, os, mcap, ocount, nullptr, nullptr, ws, wm,
                               0);
    if (mut.status == DDM_OK && (!check(hipStreamSynchronize(0), "mutual") || !fetch(mut, oi, oj, os, ocount)))
        return 1;

    FILE *out = std::fopen(argv[2], "wb");
    if (!out) { std::perror(argv[2]); return 2; }
    put(out, frm);
    put(out, mut);
    std::fclose(out);
    std::printf("frm: status %d (%s), %d pairs; mutual: status %d (%s), %d pairs\n", frm.status,
                ddm_status_str(frm.status), frm.count, mut.status, ddm_status_str(mut.status), mut.count);
    (void)hipFree(D1); (void)hipFree(D2); (void)hipFree(oi); (void)hipFree(oj); (void)hipFree(os);
    (void)hipFree(ocount); (void)hipFree(ws);
    const int rel = ddm_release_cached_resources();     // the library's graphs, while HIP is still up
    if (rel != DDM_OK) std::fprintf(stderr, "release: %s\n", ddm_status_str(rel));
    return frm.status == DDM_OK && mut.status == DDM_OK && rel == DDM_OK ? 0 : 1;
}
