// One decode step through the C ABI from a plain host program (no Python,
// no torch): HIP runtime allocations, the descriptors of abs.h, centroid
// build, score + select, sparse decode; then the same step through
// abs_select_decode, which must give the same bytes (exit status 1 if not).
// Inputs come from raw files written by the test (fp32 caches), outputs go
// to raw files it compares.
//
//   decode_step DIR B HQ HKV D MAXPAGES NPAGES BUDGET BS_0 .. BS_{HKV-1}
//
// DIR holds k.bin v.bin q.bin (fp32), pt.bin lens.bin (int32); the program
// writes sel.bin count.bin (int32), out.bin lse.bin (fp32).
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include <string>
#include <vector>

#include "abs.h"

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
            return 2;                                                               \
        }                                                                           \
    } while (0)
#define ABS_OK_(x)                                                                  \
    do {                                                                            \
        abs_status s_ = (x);                                                        \
        if (s_ != ABS_OK) {                                                         \
            std::fprintf(stderr, "%s: %s (%s)\n", #x, abs_status_str(s_), abs_last_error()); \
            return 3;                                                               \
        }                                                                           \
    } while (0)

template <typename T>
static bool read_file(const std::string& path, std::vector<T>& out, size_t n) {
    out.resize(n);
    FILE* f = std::fopen(path.c_str(), "rb");
    if (!f) return false;
    const size_t got = std::fread(out.data(), sizeof(T), n, f);
    std::fclose(f);
    return got == n;
}

template <typename T>
static bool write_file(const std::string& path, const std::vector<T>& v) {
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f) return false;
    const size_t put = std::fwrite(v.data(), sizeof(T), v.size(), f);
    std::fclose(f);
    return put == v.size();
}

template <typename T>
static T* to_device(const std::vector<T>& h) {
    void* d = nullptr;
    if (hipMalloc(&d, h.size() * sizeof(T)) != hipSuccess) return nullptr;
    if (hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
    return static_cast<T*>(d);
}

int main(int argc, char** argv) {
    if (argc < 9) {
        std::fprintf(stderr, "usage: decode_step DIR B HQ HKV D MAXPAGES NPAGES BUDGET BS...\n");
        return 1;
    }
    const std::string dir = argv[1];
    const int B = std::atoi(argv[2]), Hq = std::atoi(argv[3]), Hkv = std::atoi(argv[4]), D = std::atoi(argv[5]);
    const int max_pages = std::atoi(argv[6]);
    const int64_t npages = std::atoll(argv[7]);
    const int budget = std::atoi(argv[8]);
    if (argc != 9 + Hkv) {
        std::fprintf(stderr, "need %d block sizes\n", Hkv);
        return 1;
    }
    std::vector<int32_t> bs(Hkv);
    for (int h = 0; h < Hkv; ++h) bs[h] = std::atoi(argv[9 + h]);

    std::vector<float> k, v, q;
    std::vector<int32_t> pt, lens;
    const size_t cache_n = (size_t)npages * Hkv * 16 * D;
    if (!read_file(dir + "/k.bin", k, cache_n) || !read_file(dir + "/v.bin", v, cache_n) ||
        !read_file(dir + "/q.bin", q, (size_t)B * Hq * D) || !read_file(dir + "/pt.bin", pt, (size_t)B * max_pages) ||
        !read_file(dir + "/lens.bin", lens, (size_t)B)) {
        std::fprintf(stderr, "cannot read the inputs in %s\n", dir.c_str());
        return 1;
    }

    float* dk = to_device(k);
    float* dv = to_device(v);
    float* dq = to_device(q);
    int32_t* dpt = to_device(pt);
    int32_t* dlens = to_device(lens);
    int32_t* dbs = to_device(bs);
    if (!dk || !dv || !dq || !dpt || !dlens || !dbs) return 2;

    abs_paged_kv kv = {};
    kv.num_seqs = B;
    kv.num_q_heads = Hq;
    kv.num_kv_heads = Hkv;
    kv.head_dim = D;
    kv.page_size = 16;
    kv.max_pages_per_seq = max_pages;
    kv.num_pages = npages;
    kv.kv_dtype = ABS_F32;
    kv.k_cache = dk;
    kv.v_cache = dv;
    kv.page_table = dpt;
    kv.seq_lens = dlens;
    kv.seq_lens_host = lens.data();

    std::vector<int64_t> off((size_t)B * Hkv + 1);
    abs_block_map map = {bs.data(), dbs, nullptr};
    ABS_OK_(abs_centroid_offsets(&kv, &map, off.data()));
    int64_t* doff = to_device(off);
    if (!doff) return 2;
    map.centroid_off = doff;

    int64_t row_bytes = 0;
    ABS_OK_(abs_centroid_row_bytes(D, ABS_CENT_INT4, &row_bytes));
    abs_centroids cents = {};
    cents.format = ABS_CENT_INT4;
    HIP_OK(hipMalloc((void**)&cents.codes, (size_t)off.back() * row_bytes));
    HIP_OK(hipMalloc((void**)&cents.scale, (size_t)B * Hkv * D * sizeof(float)));
    HIP_OK(hipMalloc((void**)&cents.lo, (size_t)B * Hkv * D * sizeof(float)));

    size_t ws_bytes[4];
    for (int op = 0; op < 4; ++op) ABS_OK_(abs_workspace_bytes(&kv, &map, budget, (abs_op)op, &ws_bytes[op]));
    void* ws[4];
    for (int op = 0; op < 4; ++op) {
        HIP_OK(hipMalloc(&ws[op], ws_bytes[op] ? ws_bytes[op] : 256));
        HIP_OK(hipMemset(ws[op], 0, ws_bytes[op] ? ws_bytes[op] : 256));   // the decode workspace starts zeroed
    }
    int32_t sel_cap = 0;
    ABS_OK_(abs_select_capacity(&kv, &map, budget, &sel_cap));
    int32_t *dsel = nullptr, *dcnt = nullptr;
    float *dout = nullptr, *dlse = nullptr;
    HIP_OK(hipMalloc((void**)&dsel, (size_t)B * Hkv * sel_cap * sizeof(int32_t)));
    HIP_OK(hipMemset(dsel, 0xFF, (size_t)B * Hkv * sel_cap * sizeof(int32_t)));
    HIP_OK(hipMalloc((void**)&dcnt, (size_t)B * Hkv * sizeof(int32_t)));
    HIP_OK(hipMalloc((void**)&dout, (size_t)B * Hq * D * sizeof(float)));
    HIP_OK(hipMalloc((void**)&dlse, (size_t)B * Hq * sizeof(float)));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    const float sm_scale = 1.0f / std::sqrt((float)D);
    ABS_OK_(abs_build_centroids(&kv, &map, &cents, ws[ABS_OP_BUILD], ws_bytes[ABS_OP_BUILD], stream));
    ABS_OK_(abs_score_select(&kv, &map, &cents, dq, budget, dsel, sel_cap, dcnt, ws[ABS_OP_SELECT],
                             ws_bytes[ABS_OP_SELECT], stream));
    ABS_OK_(abs_sparse_decode(&kv, &map, dq, dsel, sel_cap, dcnt, budget, sm_scale, dout, dlse, ws[ABS_OP_DECODE],
                              ws_bytes[ABS_OP_DECODE], stream));
    HIP_OK(hipStreamSynchronize(stream));

    std::vector<int32_t> sel((size_t)B * Hkv * sel_cap), cnt((size_t)B * Hkv);
    std::vector<float> out((size_t)B * Hq * D), lse((size_t)B * Hq);
    HIP_OK(hipMemcpy(sel.data(), dsel, sel.size() * sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(cnt.data(), dcnt, cnt.size() * sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out.data(), dout, out.size() * sizeof(float), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse.data(), dlse, lse.size() * sizeof(float), hipMemcpyDeviceToHost));

    // the same step through abs_select_decode, into fresh outputs: it must
    // give the same bytes
    int32_t *dsel2 = nullptr, *dcnt2 = nullptr;
    float *dout2 = nullptr, *dlse2 = nullptr;
    HIP_OK(hipMalloc((void**)&dsel2, sel.size() * sizeof(int32_t)));
    HIP_OK(hipMemset(dsel2, 0xFF, sel.size() * sizeof(int32_t)));
    HIP_OK(hipMalloc((void**)&dcnt2, cnt.size() * sizeof(int32_t)));
    HIP_OK(hipMalloc((void**)&dout2, out.size() * sizeof(float)));
    HIP_OK(hipMalloc((void**)&dlse2, lse.size() * sizeof(float)));
    ABS_OK_(abs_select_decode(&kv, &map, &cents, dq, budget, sm_scale, dsel2, sel_cap, dcnt2, dout2, dlse2,
                              ws[ABS_OP_SELECT_DECODE], ws_bytes[ABS_OP_SELECT_DECODE], stream));
    HIP_OK(hipStreamSynchronize(stream));
    std::vector<int32_t> sel2(sel.size()), cnt2(cnt.size());
    std::vector<float> out2(out.size()), lse2(lse.size());
    HIP_OK(hipMemcpy(sel2.data(), dsel2, sel2.size() * sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(cnt2.data(), dcnt2, cnt2.size() * sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out2.data(), dout2, out2.size() * sizeof(float), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse2.data(), dlse2, lse2.size() * sizeof(float), hipMemcpyDeviceToHost));
    bool same = cnt2 == cnt && std::memcmp(out2.data(), out.data(), out.size() * sizeof(float)) == 0 &&
                std::memcmp(lse2.data(), lse.data(), lse.size() * sizeof(float)) == 0;
    for (size_t r = 0; same && r < cnt.size(); ++r)
        same = std::memcmp(&sel2[r * sel_cap], &sel[r * sel_cap], (size_t)cnt[r] * sizeof(int32_t)) == 0;
    if (!same) {
        std::fprintf(stderr, "abs_select_decode differs from abs_score_select + abs_sparse_decode\n");
        return 1;
    }
    for (void* p : {(void*)dsel2, (void*)dcnt2, (void*)dout2, (void*)dlse2}) HIP_OK(hipFree(p));

    if (!write_file(dir + "/sel.bin", sel) || !write_file(dir + "/count.bin", cnt) ||
        !write_file(dir + "/out.bin", out) || !write_file(dir + "/lse.bin", lse))
        return 1;
    std::printf("sel_cap %d\n", sel_cap);

    HIP_OK(hipStreamDestroy(stream));
    for (void* p : {(void*)dk, (void*)dv, (void*)dq, (void*)dpt, (void*)dlens, (void*)dbs, (void*)doff,
                    (void*)cents.codes, (void*)cents.scale, (void*)cents.lo, ws[0], ws[1], ws[2], ws[3], (void*)dsel,
                    (void*)dcnt, (void*)dout, (void*)dlse})
        HIP_OK(hipFree(p));
    return 0;
}
