// C ABI of the AB-Sparse decode library (declared in include/abs.h).
//
// This layer owns everything the host knows before a launch: it validates
// the descriptors, derives the block geometry (N_{b,h} = ceil(L_b / bs_h),
// K_{b,h} = min(N, max(1, floor(budget / bs_h))), the CSR centroid offsets,
// the page count each head reads), carves the caller's workspace, sizes the
// grids, and enqueues the kernels on the caller's stream.  It never
// allocates, frees or synchronizes, and nothing is read back from the device
// (except with the debug checks on, abs_set_debug_checks).
#include "abs.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <vector>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "decode_layout.hpp"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

abs_status fail(abs_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

abs_status ok() {
    g_err[0] = '\0';
    return ABS_OK;
}

// Compute units of the current device, read once per device (256 on an
// MI355X; fewer on a partitioned one).  Without a device (host-only use of
// the sizing calls) the MI355X figure is assumed.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_compute_units() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        n = 256;
    }
    g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

std::atomic<int> g_debug_checks{0};

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Everything derived on the host from the descriptors (and budget).
struct Plan {
    absk::Geom g{};
    absk::DType dt{};
    int64_t total_blocks = 0;
    int max_n = 0;            // largest N_{b,h}
    int max_len = 0;          // largest L_b
    int sel_cap = 0;          // largest K_{b,h}
    int max_pages_read = 0;   // largest K_{b,h} * (bs_h / 16)
    const int32_t* block_size_dev = nullptr;   // the descriptor's device copy (kernels use the host values)
};

abs_status check_geometry(const abs_paged_kv* kv, const abs_block_map* map, Plan* p) {
    if (kv == nullptr || map == nullptr) return fail(ABS_ERR_INVALID_ARG, "null descriptor");
    if (kv->num_seqs < 1 || kv->num_q_heads < 1 || kv->num_kv_heads < 1)
        return fail(ABS_ERR_INVALID_ARG, "num_seqs, num_q_heads, num_kv_heads must be >= 1");
    if (kv->num_q_heads % kv->num_kv_heads != 0)
        return fail(ABS_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                    kv->num_q_heads, kv->num_kv_heads);
    if (kv->num_kv_heads > absk::kMaxKvHeads)
        return fail(ABS_ERR_UNSUPPORTED, "num_kv_heads %d > %d", kv->num_kv_heads, absk::kMaxKvHeads);
    if ((int64_t)kv->num_seqs * kv->num_kv_heads > 65536)   // (b, h) pairs index a grid dimension
        return fail(ABS_ERR_UNSUPPORTED, "num_seqs * num_kv_heads = %lld > 65536",
                    (long long)kv->num_seqs * kv->num_kv_heads);
    const int G = kv->num_q_heads / kv->num_kv_heads;
    if (G > 8) return fail(ABS_ERR_UNSUPPORTED, "query group size %d > 8", G);
    if (kv->head_dim != 64 && kv->head_dim != 128)
        return fail(ABS_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", kv->head_dim);
    if (kv->page_size != 16) return fail(ABS_ERR_UNSUPPORTED, "page_size %d (supported: 16)", kv->page_size);
    if (kv->kv_dtype != ABS_F32 && kv->kv_dtype != ABS_BF16)
        return fail(ABS_ERR_UNSUPPORTED, "kv_dtype %d", kv->kv_dtype);
    if (kv->reserved0 != 0) return fail(ABS_ERR_INVALID_ARG, "reserved0 must be 0");
    if (kv->max_pages_per_seq < 1 || kv->num_pages < 1)
        return fail(ABS_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
    if (kv->seq_lens_host == nullptr) return fail(ABS_ERR_INVALID_ARG, "seq_lens_host is null");
    if (map->block_size_host == nullptr) return fail(ABS_ERR_INVALID_ARG, "block_size_host is null");
    const int64_t max_len = (int64_t)kv->max_pages_per_seq * 16;
    for (int b = 0; b < kv->num_seqs; ++b) {
        const int L = kv->seq_lens_host[b];
        if (L < 1 || L > max_len)
            return fail(ABS_ERR_INVALID_ARG, "seq_lens[%d] = %d outside [1, %lld]", b, L, (long long)max_len);
    }
    for (int h = 0; h < kv->num_kv_heads; ++h) {
        const int bs = map->block_size_host[h];
        if (bs < 1) return fail(ABS_ERR_INVALID_ARG, "block_size[%d] = %d", h, bs);
        if (bs != 16 && bs != 32 && bs != 64)
            return fail(ABS_ERR_UNSUPPORTED, "block_size[%d] = %d (supported: 16, 32, 64)", h, bs);
    }
    p->dt = kv->kv_dtype == ABS_BF16 ? absk::DType::BF16 : absk::DType::F32;
    absk::Geom& g = p->g;
    g.B = kv->num_seqs;
    g.Hq = kv->num_q_heads;
    g.Hkv = kv->num_kv_heads;
    g.D = kv->head_dim;
    g.G = G;
    g.hkv_magic = absk::div_magic(g.Hkv);
    g.max_pages = kv->max_pages_per_seq;
    g.num_pages = kv->num_pages;
    g.k = kv->k_cache;
    g.v = kv->v_cache;
    g.page_table = kv->page_table;
    g.seq_lens = kv->seq_lens;
    g.off = map->centroid_off;
    p->block_size_dev = map->block_size;
    g.bs_log2[0] = g.bs_log2[1] = 0;
    for (int h = 0; h < g.Hkv; ++h) {
        const int bs = map->block_size_host[h];   // validated: 16, 32 or 64
        g.bs_log2[h / 32] |= (uint64_t)(bs == 16 ? 0 : bs == 32 ? 1 : 2) << (2 * (h % 32));
    }
    p->total_blocks = 0;
    p->max_n = 0;
    p->max_len = 0;
    for (int b = 0; b < g.B; ++b) p->max_len = std::max(p->max_len, kv->seq_lens_host[b]);
    g.max_len = p->max_len;
    for (int b = 0; b < g.B; ++b)
        for (int h = 0; h < g.Hkv; ++h) {
            const int64_t n = ceil_div64(kv->seq_lens_host[b], map->block_size_host[h]);
            p->total_blocks += n;
            p->max_n = std::max<int>(p->max_n, (int)n);
        }
    return ok();
}

abs_status plan_budget(const abs_paged_kv* kv, const abs_block_map* map, int32_t budget, Plan* p) {
    if (budget < 1) return fail(ABS_ERR_INVALID_ARG, "token_budget %d < 1", budget);
    p->sel_cap = 0;
    p->max_pages_read = 0;
    for (int b = 0; b < kv->num_seqs; ++b)
        for (int h = 0; h < kv->num_kv_heads; ++h) {
            const int bs = map->block_size_host[h];
            const int64_t n = ceil_div64(kv->seq_lens_host[b], bs);
            const int64_t k = std::min<int64_t>(n, std::max<int64_t>(1, budget / bs));
            p->sel_cap = std::max<int>(p->sel_cap, (int)k);
            p->max_pages_read = std::max<int>(p->max_pages_read, (int)(k * (bs / 16)));
        }
    return ok();
}

abs_status require_device(const Plan& p, bool need_v) {
    const absk::Geom& g = p.g;
    if (g.k == nullptr || (need_v && g.v == nullptr)) return fail(ABS_ERR_INVALID_ARG, "null cache pointer");
    if (g.page_table == nullptr || g.seq_lens == nullptr)
        return fail(ABS_ERR_INVALID_ARG, "null page_table or seq_lens");
    if (g.off == nullptr) return fail(ABS_ERR_INVALID_ARG, "null centroid_off");
    return ok();
}

// Debug checks (abs_set_debug_checks): read the device copies back and compare
// them with what the host sized the launch from.  Synchronizes the stream.
abs_status debug_check(const Plan& p, const abs_paged_kv* kv, const abs_block_map* map, hipStream_t st) {
    if (g_debug_checks.load(std::memory_order_relaxed) == 0) return ok();
    const absk::Geom& g = p.g;
    std::vector<int32_t> lens(g.B), bs(g.Hkv), pt((size_t)g.B * g.max_pages);
    hipError_t e = hipMemcpyAsync(lens.data(), g.seq_lens, lens.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess && map->block_size != nullptr)
        e = hipMemcpyAsync(bs.data(), map->block_size, bs.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(pt.data(), g.page_table, pt.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(ABS_ERR_HIP, "debug check read-back: %s", hipGetErrorString(e));
    for (int b = 0; b < g.B; ++b) {
        if (lens[b] != kv->seq_lens_host[b])
            return fail(ABS_ERR_INVALID_ARG, "debug check: seq_lens[%d] = %d on the device, %d on the host", b,
                        lens[b], kv->seq_lens_host[b]);
        const int np = (kv->seq_lens_host[b] + 15) / 16;
        for (int i = 0; i < np; ++i) {
            const int32_t id = pt[(size_t)b * g.max_pages + i];
            if (id < 0 || id >= g.num_pages)
                return fail(ABS_ERR_INVALID_ARG, "debug check: page_table[%d][%d] = %d outside [0, %lld)", b, i, id,
                            (long long)g.num_pages);
        }
    }
    if (map->block_size != nullptr)
        for (int h = 0; h < g.Hkv; ++h)
            if (bs[h] != map->block_size_host[h])
                return fail(ABS_ERR_INVALID_ARG, "debug check: block_size[%d] = %d on the device, %d on the host", h,
                            bs[h], map->block_size_host[h]);
    return ok();
}

// ---- workspace layouts ----------------------------------------------------

struct BuildLayout {
    int tiles = 0;
    size_t staging = 0, pmin = 0, pmax = 0, bytes = 0;
};

BuildLayout build_layout(const Plan& p) {
    BuildLayout l;
    l.tiles = (int)ceil_div64(p.max_len, absk::kBuildTileTokens);
    const size_t part = align_up((size_t)p.g.B * p.g.Hkv * l.tiles * p.g.D * sizeof(float));
    l.staging = 0;   // per (b, h): max N rows, whatever the centroid offsets
    l.pmin = align_up((size_t)p.g.B * p.g.Hkv * p.max_n * p.g.D * sizeof(float));
    l.pmax = l.pmin + part;
    l.bytes = l.pmax + part;
    return l;
}

int score_stride(const Plan& p) { return (p.max_n + 3) / 4 * 4; }

int range_stride(const Plan& p) { return (int)ceil_div64(p.max_n, absk::kScoreBlocksPerWg); }

// The select workspace: fp32 score rows, then each 256-block tile's (min, max).
size_t select_scores_bytes(const Plan& p) {
    return align_up((size_t)p.g.B * p.g.Hkv * score_stride(p) * sizeof(float));
}

size_t select_bytes(const Plan& p) {
    return select_scores_bytes(p) + align_up((size_t)p.g.B * p.g.Hkv * range_stride(p) * 2 * sizeof(float));
}

absk::DecodeLayout decode_layout(const Plan& p) {
    return absk::decode_layout(p.g.B, p.g.Hkv, p.g.Hq, p.g.D, p.max_pages_read, device_compute_units());
}

abs_status check_centroids(const abs_centroids* c) {
    if (c == nullptr || c->codes == nullptr || c->scale == nullptr || c->lo == nullptr)
        return fail(ABS_ERR_INVALID_ARG, "null centroid store");
    if (c->format < ABS_CENT_INT4 || c->format > ABS_CENT_BF16)
        return fail(ABS_ERR_INVALID_ARG, "unknown centroid format %d", c->format);
    if (c->reserved0 != 0) return fail(ABS_ERR_INVALID_ARG, "abs_centroids.reserved0 must be 0");
    if (reinterpret_cast<uintptr_t>(c->codes) % 16 != 0)
        return fail(ABS_ERR_INVALID_ARG, "centroid codes are not 16-byte aligned");
    return ok();
}

char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

abs_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ABS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Checks shared by the calls that select (after plan_budget).
abs_status check_select(const Plan& p, const abs_centroids* cents, const void* q, const int32_t* sel,
                        int32_t sel_cap, const int32_t* sel_count) {
    if (abs_status st = check_centroids(cents)) return st;
    if (q == nullptr || sel == nullptr || sel_count == nullptr)
        return fail(ABS_ERR_INVALID_ARG, "null q, sel or sel_count");
    if (sel_cap < p.sel_cap) return fail(ABS_ERR_INVALID_ARG, "sel_cap %d < required %d", sel_cap, p.sel_cap);
    if (p.max_n > absk::kMaxBlocksPerHead)
        return fail(ABS_ERR_UNSUPPORTED, "%d blocks in one head (max %d)", p.max_n, absk::kMaxBlocksPerHead);
    return ok();
}

// Launch arguments of the select stage; `scores` is its workspace, `tiles`
// storage for the score tile list (read during the launch).
void fill_select_args(const Plan& p, const abs_paged_kv* kv, const abs_block_map* map, const abs_centroids* cents,
                      const void* q, int32_t token_budget, int32_t* sel, int32_t sel_cap, int32_t* sel_count,
                      void* scores, uint32_t* tiles, absk::SelectArgs* a) {
    a->codes = cents->codes;
    a->scale = cents->scale;
    a->lo = cents->lo;
    a->fmt = cents->format;
    a->q = q;
    a->scores = reinterpret_cast<float*>(scores);
    a->stride = score_stride(p);
    a->ranges = scores != nullptr ? reinterpret_cast<float2*>(ws_at(scores, select_scores_bytes(p))) : nullptr;
    a->range_stride = range_stride(p);
    a->sel = sel;
    a->count = sel_count;
    a->sel_cap = sel_cap;
    a->budget = token_budget;
    a->max_n = p.max_n;
    a->max_len = p.max_len;
    a->total_blocks = p.total_blocks;
    a->zero_counters = nullptr;
    a->n_zero = 0;
    // the exact list of score tiles, when it fits the kernel arguments
    a->ntiles = 0;
    for (int b = 0; b < p.g.B; ++b)
        for (int h = 0; h < p.g.Hkv; ++h) {
            const int64_t n = ceil_div64(ceil_div64(kv->seq_lens_host[b], map->block_size_host[h]),
                                         absk::kScoreBlocksPerWg);
            for (int64_t t = 0; t < n; ++t, ++a->ntiles)
                if (a->ntiles < absk::kMaxScoreTiles) tiles[a->ntiles] = (uint32_t)(b * p.g.Hkv + h) << 8 | (uint32_t)t;
        }
    a->tiles_host = a->ntiles <= absk::kMaxScoreTiles ? tiles : nullptr;
    // per-head cumulative tiles of the longest sequence (the grid when the list does not fit)
    a->head_tiles.cum[0] = 0;
    for (int h = 0; h < p.g.Hkv; ++h)
        a->head_tiles.cum[h + 1] =
            a->head_tiles.cum[h] +
            (uint32_t)ceil_div64(ceil_div64(p.max_len, map->block_size_host[h]), absk::kScoreBlocksPerWg);
}

// Launch arguments of the decode stage; `ws` is its workspace.
void fill_decode_args(const absk::DecodeLayout& l, const void* q, const int32_t* sel, int32_t sel_cap,
                      const int32_t* sel_count, float sm_scale, void* out, float* lse, void* ws,
                      absk::DecodeArgs* a) {
    a->q = q;
    a->sel = sel;
    a->count = sel_count;
    a->sel_cap = sel_cap;
    a->sm_scale = sm_scale;
    a->out = out;
    a->lse = lse;
    a->part_ml = reinterpret_cast<float*>(ws_at(ws, l.ml));
    a->part_o = reinterpret_cast<float*>(ws_at(ws, l.o));
    a->arrive = ABS_DECODE_FUSED_MERGE ? reinterpret_cast<int32_t*>(ws_at(ws, l.arrive)) : nullptr;
    a->pages_per_wg = l.ppw;
    a->ppw_magic = absk::div_magic(l.ppw);
    a->chunk = l.chunk;
    a->pipelined = l.pipelined;
    a->splits = l.splits;
    a->compute_units = device_compute_units();
}

}  // namespace

extern "C" {

const char* abs_status_str(abs_status s) {
    switch (s) {
        case ABS_OK: return "ok";
        case ABS_ERR_INVALID_ARG: return "invalid argument";
        case ABS_ERR_UNSUPPORTED: return "unsupported configuration";
        case ABS_ERR_WORKSPACE: return "workspace too small";
        case ABS_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* abs_last_error(void) { return g_err; }

abs_status abs_total_blocks(const abs_paged_kv* kv, const abs_block_map* map, int64_t* total) {
    if (total == nullptr) return fail(ABS_ERR_INVALID_ARG, "null output");
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    *total = p.total_blocks;
    return ok();
}

abs_status abs_centroid_offsets(const abs_paged_kv* kv, const abs_block_map* map, int64_t* off_host) {
    if (off_host == nullptr) return fail(ABS_ERR_INVALID_ARG, "null output");
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    int64_t run = 0;
    for (int b = 0; b < kv->num_seqs; ++b)
        for (int h = 0; h < kv->num_kv_heads; ++h) {
            off_host[(int64_t)b * kv->num_kv_heads + h] = run;
            run += ceil_div64(kv->seq_lens_host[b], map->block_size_host[h]);
        }
    off_host[(int64_t)kv->num_seqs * kv->num_kv_heads] = run;
    return ok();
}

abs_status abs_centroid_offsets_capacity(const abs_paged_kv* kv, const abs_block_map* map, int32_t capacity_tokens,
                                         int64_t* off_host) {
    if (off_host == nullptr) return fail(ABS_ERR_INVALID_ARG, "null output");
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    for (int b = 0; b < kv->num_seqs; ++b)
        if (capacity_tokens < kv->seq_lens_host[b])
            return fail(ABS_ERR_INVALID_ARG, "capacity_tokens %d < seq_lens[%d] = %d", capacity_tokens, b,
                        kv->seq_lens_host[b]);
    int64_t run = 0;
    for (int b = 0; b < kv->num_seqs; ++b)
        for (int h = 0; h < kv->num_kv_heads; ++h) {
            off_host[(int64_t)b * kv->num_kv_heads + h] = run;
            run += ceil_div64(capacity_tokens, map->block_size_host[h]);
        }
    off_host[(int64_t)kv->num_seqs * kv->num_kv_heads] = run;
    return ok();
}

abs_status abs_centroid_row_bytes(int32_t head_dim, int32_t format, int64_t* bytes) {
    if (bytes == nullptr) return fail(ABS_ERR_INVALID_ARG, "null output");
    if (head_dim < 1) return fail(ABS_ERR_INVALID_ARG, "head_dim %d < 1", head_dim);
    if (format < ABS_CENT_INT4 || format > ABS_CENT_BF16)
        return fail(ABS_ERR_INVALID_ARG, "unknown centroid format %d", format);
    *bytes = absk::row_bytes(head_dim, format);
    return ok();
}

abs_status abs_select_capacity(const abs_paged_kv* kv, const abs_block_map* map, int32_t token_budget,
                               int32_t* sel_cap) {
    if (sel_cap == nullptr) return fail(ABS_ERR_INVALID_ARG, "null output");
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    if (abs_status st = plan_budget(kv, map, token_budget, &p)) return st;
    *sel_cap = p.sel_cap;
    return ok();
}

abs_status abs_workspace_bytes(const abs_paged_kv* kv, const abs_block_map* map, int32_t token_budget, abs_op op,
                               size_t* bytes) {
    if (bytes == nullptr) return fail(ABS_ERR_INVALID_ARG, "null output");
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    switch (op) {
        case ABS_OP_BUILD: *bytes = build_layout(p).bytes; return ok();
        case ABS_OP_SELECT: *bytes = select_bytes(p); return ok();
        case ABS_OP_DECODE:
            if (abs_status st = plan_budget(kv, map, token_budget, &p)) return st;
            *bytes = decode_layout(p).bytes;
            return ok();
        case ABS_OP_SELECT_DECODE:
            if (abs_status st = plan_budget(kv, map, token_budget, &p)) return st;
            *bytes = select_bytes(p) + decode_layout(p).bytes;
            return ok();
    }
    return fail(ABS_ERR_INVALID_ARG, "unknown op %d", (int)op);
}

abs_status abs_build_centroids(const abs_paged_kv* kv, const abs_block_map* map, const abs_centroids* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    if (abs_status st = require_device(p, false)) return st;
    if (abs_status st = check_centroids(out)) return st;
    const BuildLayout l = build_layout(p);
    if (workspace == nullptr || workspace_bytes < l.bytes)
        return fail(ABS_ERR_WORKSPACE, "build needs %zu workspace bytes, got %zu", l.bytes, workspace_bytes);
    absk::BuildArgs a;
    a.codes = out->codes;
    a.scale = out->scale;
    a.lo = out->lo;
    a.staging = reinterpret_cast<float*>(ws_at(workspace, l.staging));
    a.pmin = reinterpret_cast<float*>(ws_at(workspace, l.pmin));
    a.pmax = reinterpret_cast<float*>(ws_at(workspace, l.pmax));
    a.tiles = l.tiles;
    a.stage_rows = p.max_n;
    a.fmt = out->format;
    if (abs_status st = debug_check(p, kv, map, static_cast<hipStream_t>(stream))) return st;
    return hip_status(absk::launch_build(p.g, p.dt, a, static_cast<hipStream_t>(stream)), "build_centroids");
}

abs_status abs_update_centroids(const abs_paged_kv* kv, const abs_block_map* map, const abs_centroids* cents,
                                int32_t appended, int32_t* out_of_range, void* stream) {
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    if (abs_status st = require_device(p, false)) return st;
    if (abs_status st = check_centroids(cents)) return st;
    if (appended < 0) return fail(ABS_ERR_INVALID_ARG, "appended %d < 0", appended);
    absk::UpdateArgs a;
    a.scale = cents->scale;
    a.lo = cents->lo;
    a.codes = cents->codes;
    a.out_of_range = out_of_range;
    a.appended = appended;
    a.fmt = cents->format;
    if (abs_status st = debug_check(p, kv, map, static_cast<hipStream_t>(stream))) return st;
    return hip_status(absk::launch_update(p.g, p.dt, a, static_cast<hipStream_t>(stream)), "update_centroids");
}

abs_status abs_score_select(const abs_paged_kv* kv, const abs_block_map* map, const abs_centroids* cents,
                            const void* q, int32_t token_budget, int32_t* sel, int32_t sel_cap,
                            int32_t* sel_count, void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    if (abs_status st = require_device(p, false)) return st;
    if (abs_status st = plan_budget(kv, map, token_budget, &p)) return st;
    if (abs_status st = check_select(p, cents, q, sel, sel_cap, sel_count)) return st;
    const size_t need = select_bytes(p);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ABS_ERR_WORKSPACE, "select needs %zu workspace bytes, got %zu", need, workspace_bytes);
    absk::SelectArgs a;
    uint32_t tiles[absk::kMaxScoreTiles];
    fill_select_args(p, kv, map, cents, q, token_budget, sel, sel_cap, sel_count, workspace, tiles, &a);
    if (abs_status st = debug_check(p, kv, map, static_cast<hipStream_t>(stream))) return st;
    return hip_status(absk::launch_select(p.g, p.dt, a, static_cast<hipStream_t>(stream)), "score_select");
}

abs_status abs_sparse_decode(const abs_paged_kv* kv, const abs_block_map* map, const void* q, const int32_t* sel,
                             int32_t sel_cap, const int32_t* sel_count, int32_t token_budget, float sm_scale,
                             void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    if (abs_status st = require_device(p, true)) return st;
    if (abs_status st = plan_budget(kv, map, token_budget, &p)) return st;
    if (q == nullptr || sel == nullptr || sel_count == nullptr || out == nullptr)
        return fail(ABS_ERR_INVALID_ARG, "null q, sel, sel_count or out");
    if (sel_cap < p.sel_cap) return fail(ABS_ERR_INVALID_ARG, "sel_cap %d < required %d", sel_cap, p.sel_cap);
    if (!std::isfinite(sm_scale)) return fail(ABS_ERR_INVALID_ARG, "sm_scale is not finite");
    const absk::DecodeLayout l = decode_layout(p);
    if (workspace == nullptr || workspace_bytes < l.bytes)
        return fail(ABS_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", l.bytes, workspace_bytes);
    absk::DecodeArgs a;
    fill_decode_args(l, q, sel, sel_cap, sel_count, sm_scale, out, lse, workspace, &a);
    if (abs_status st = debug_check(p, kv, map, static_cast<hipStream_t>(stream))) return st;
    return hip_status(absk::launch_decode(p.g, p.dt, a, static_cast<hipStream_t>(stream)), "sparse_decode");
}

}  // extern "C"

namespace {

// The stages of abs_select_decode: Estimation alone (abs_estimate), Top-K and
// Attention on the scores already in the workspace (abs_topk_decode), or all
// three.
enum class Stages { All, Estimate, TopkDecode };

// abs_select_decode's stages on the workspace `workspace` of
// `workspace_bytes` bytes (validated here), or, with scratch_of_device, on
// the static scratch of the current device (workspace_bytes is then its
// size).
abs_status select_decode_on(const abs_paged_kv* kv, const abs_block_map* map, const abs_centroids* cents,
                            const void* q, int32_t token_budget, float sm_scale, int32_t* sel, int32_t sel_cap,
                            int32_t* sel_count, void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream, void* (*scratch_of_device)(), Stages stages) {
    const bool estimate = stages != Stages::TopkDecode, decode = stages != Stages::Estimate;
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    if (abs_status st = require_device(p, decode)) return st;
    if (abs_status st = plan_budget(kv, map, token_budget, &p)) return st;
    if (estimate) {
        if (abs_status st = check_centroids(cents)) return st;
    }
    if (q == nullptr) return fail(ABS_ERR_INVALID_ARG, "null q");
    if (decode) {
        if (sel == nullptr || sel_count == nullptr || out == nullptr)
            return fail(ABS_ERR_INVALID_ARG, "null sel, sel_count or out");
        if (sel_cap < p.sel_cap) return fail(ABS_ERR_INVALID_ARG, "sel_cap %d < required %d", sel_cap, p.sel_cap);
        if (!std::isfinite(sm_scale)) return fail(ABS_ERR_INVALID_ARG, "sm_scale is not finite");
    }
    if (p.max_n > absk::kMaxBlocksPerHead)
        return fail(ABS_ERR_UNSUPPORTED, "%d blocks in one head (max %d)", p.max_n, absk::kMaxBlocksPerHead);
    const size_t sbytes = select_bytes(p);
    const absk::DecodeLayout l = decode_layout(p);
    if (scratch_of_device != nullptr) {
        if (sbytes + l.bytes > workspace_bytes)
            return fail(ABS_ERR_WORKSPACE, "this layer needs %zu scratch bytes; the static scratch holds %zu",
                        sbytes + l.bytes, workspace_bytes);
        workspace = scratch_of_device();
        if (workspace == nullptr) return ABS_ERR_HIP;   // the message is set
    }
    if (workspace == nullptr || workspace_bytes < sbytes + l.bytes)
        return fail(ABS_ERR_WORKSPACE, "select_decode needs %zu workspace bytes, got %zu", sbytes + l.bytes,
                    workspace_bytes);
    const abs_centroids none{};
    absk::SelectArgs sa;
    uint32_t tiles[absk::kMaxScoreTiles];
    fill_select_args(p, kv, map, estimate ? cents : &none, q, token_budget, sel, sel_cap, sel_count, workspace, tiles,
                     &sa);
    absk::DecodeArgs da;
    fill_decode_args(l, q, sel, sel_cap, sel_count, sm_scale, out, lse, ws_at(workspace, sbytes), &da);
    // the score launch zero-fills the decode's arrival counters, so the
    // decode region needs no zero-filling by the caller
    sa.zero_counters = da.arrive;
    sa.n_zero = da.arrive != nullptr ? p.g.B * p.g.Hkv : 0;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (abs_status e = debug_check(p, kv, map, st)) return e;
    if (estimate) {
        if (abs_status e = hip_status(absk::launch_scores(p.g, p.dt, sa, st), "select_decode (scores)")) return e;
    }
    if (!decode) return ok();
    if (absk::select_decode_fusable(p.g, p.dt, sa, da))
        return hip_status(absk::launch_select_decode(p.g, p.dt, sa, da, st), "select_decode");
    if (abs_status e = hip_status(absk::launch_topk(p.g, sa, st), "select_decode (top-K)")) return e;
    return hip_status(absk::launch_decode(p.g, p.dt, da, st), "select_decode (decode)");
}

// ---- the static scratch of abs_select_decode_static ------------------------
//
// One array per GPU, in device memory for the life of the process.  Its name
// is only a host-side handle: host code uses the address that
// hipGetSymbolAddress returns for the current device, taken once per device
// on the first call there and kept in g_scratch.
constexpr size_t kStaticScratchBytes = ABS_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];

void* scratch_of_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        fail(ABS_ERR_HIP, "no current device (or device id beyond %d)", kMaxDevices - 1);
        return nullptr;
    }
    void* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr != nullptr) return ptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        fail(ABS_ERR_HIP, "hipGetSymbolAddress: %s", hipGetErrorString(e));
        return nullptr;
    }
    g_scratch[dev].store(ptr, std::memory_order_release);   // the same address if two threads race here
    return ptr;
}

}  // namespace

extern "C" {

abs_status abs_select_decode(const abs_paged_kv* kv, const abs_block_map* map, const abs_centroids* cents,
                             const void* q, int32_t token_budget, float sm_scale, int32_t* sel, int32_t sel_cap,
                             int32_t* sel_count, void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return select_decode_on(kv, map, cents, q, token_budget, sm_scale, sel, sel_cap, sel_count, out, lse, workspace,
                            workspace_bytes, stream, nullptr, Stages::All);
}

abs_status abs_estimate(const abs_paged_kv* kv, const abs_block_map* map, const abs_centroids* cents, const void* q,
                        int32_t token_budget, void* workspace, size_t workspace_bytes, void* stream) {
    return select_decode_on(kv, map, cents, q, token_budget, 1.0f, nullptr, 0, nullptr, nullptr, nullptr, workspace,
                            workspace_bytes, stream, nullptr, Stages::Estimate);
}

abs_status abs_topk_decode(const abs_paged_kv* kv, const abs_block_map* map, const void* q, int32_t token_budget,
                           float sm_scale, int32_t* sel, int32_t sel_cap, int32_t* sel_count, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return select_decode_on(kv, map, nullptr, q, token_budget, sm_scale, sel, sel_cap, sel_count, out, lse,
                            workspace, workspace_bytes, stream, nullptr, Stages::TopkDecode);
}

abs_status abs_select_decode_static(const abs_paged_kv* kv, const abs_block_map* map, const abs_centroids* cents,
                                    const void* q, int32_t token_budget, float sm_scale, int32_t* sel,
                                    int32_t sel_cap, int32_t* sel_count, void* out, float* lse, void* stream) {
    return select_decode_on(kv, map, cents, q, token_budget, sm_scale, sel, sel_cap, sel_count, out, lse, nullptr,
                            kStaticScratchBytes, stream, scratch_of_current_device, Stages::All);
}

abs_status abs_describe_launch(const abs_paged_kv* kv, const abs_block_map* map, int32_t token_budget,
                               abs_launch_plan* plan) {
    if (plan == nullptr) return fail(ABS_ERR_INVALID_ARG, "null output");
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    if (abs_status st = plan_budget(kv, map, token_budget, &p)) return st;
    const absk::DecodeLayout l = decode_layout(p);
    absk::SelectArgs sa{};
    uint32_t tiles[absk::kMaxScoreTiles];
    abs_centroids none{};
    fill_select_args(p, kv, map, &none, nullptr, token_budget, nullptr, p.sel_cap, nullptr, nullptr, tiles, &sa);
    absk::DecodeArgs da{};
    // a placeholder workspace address (never dereferenced): the arrival
    // counters' presence decides the merge form
    void* const ws_placeholder = reinterpret_cast<void*>(uintptr_t{kAlign});
    fill_decode_args(l, nullptr, nullptr, p.sel_cap, nullptr, 1.0f, nullptr, nullptr, ws_placeholder, &da);
    std::memset(plan, 0, sizeof *plan);
    plan->splits = l.splits;
    plan->pages_per_wg = l.ppw;
    plan->chunk = l.chunk;
    plan->pipelined = l.pipelined ? 1 : 0;
    plan->fused = absk::select_decode_fusable(p.g, p.dt, sa, da) ? 1 : 0;
    plan->score_workgroups = sa.ntiles <= absk::kMaxScoreTiles ? sa.ntiles : (int32_t)(sa.head_tiles.cum[p.g.Hkv] * p.g.B);
    plan->max_blocks = p.max_n;
    plan->sel_cap = p.sel_cap;
    plan->compute_units = da.compute_units;
    return ok();
}

abs_status abs_reset_workspace(const abs_paged_kv* kv, const abs_block_map* map, int32_t token_budget, abs_op op,
                               void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    if (abs_status st = check_geometry(kv, map, &p)) return st;
    if (abs_status st = plan_budget(kv, map, token_budget, &p)) return st;
    if (op != ABS_OP_DECODE && op != ABS_OP_SELECT_DECODE)
        return fail(ABS_ERR_INVALID_ARG, "op %d has no state to reset (ABS_OP_DECODE or ABS_OP_SELECT_DECODE)",
                    (int)op);
    const absk::DecodeLayout l = decode_layout(p);
    const size_t at = op == ABS_OP_DECODE ? 0 : select_bytes(p);
    if (workspace == nullptr || workspace_bytes < at + l.bytes)
        return fail(ABS_ERR_WORKSPACE, "workspace of %zu bytes, op %d needs %zu", workspace_bytes, (int)op,
                    at + l.bytes);
    return hip_status(absk::launch_zero(reinterpret_cast<int32_t*>(ws_at(workspace, at + l.arrive)),
                                        p.g.B * p.g.Hkv, static_cast<hipStream_t>(stream)),
                      "reset_workspace");
}

int32_t abs_set_debug_checks(int32_t enable) { return g_debug_checks.exchange(enable != 0 ? 1 : 0); }

abs_status abs_head_recall(const abs_paged_kv* kv, const float* lse_sel, const float* lse_full, float* recall,
                           void* stream) {
    if (kv == nullptr) return fail(ABS_ERR_INVALID_ARG, "null descriptor");
    if (kv->num_seqs < 1 || kv->num_q_heads < 1 || kv->num_kv_heads < 1)
        return fail(ABS_ERR_INVALID_ARG, "num_seqs, num_q_heads, num_kv_heads must be >= 1");
    if (kv->num_q_heads % kv->num_kv_heads != 0)
        return fail(ABS_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                    kv->num_q_heads, kv->num_kv_heads);
    if (lse_sel == nullptr || lse_full == nullptr || recall == nullptr)
        return fail(ABS_ERR_INVALID_ARG, "null lse_sel, lse_full or recall");
    return hip_status(absk::launch_head_recall(kv->num_seqs, kv->num_q_heads, kv->num_kv_heads, lse_sel, lse_full,
                                               recall, static_cast<hipStream_t>(stream)),
                      "head_recall");
}

abs_status abs_gather_tiles(const uint64_t* tile_addr, int32_t num_tiles, int32_t tile_bytes, int32_t workgroups,
                            int32_t in_flight, uint32_t* xor_out, void* stream) {
    if (tile_addr == nullptr || xor_out == nullptr) return fail(ABS_ERR_INVALID_ARG, "null tile_addr or xor_out");
    if (tile_bytes != 4096) return fail(ABS_ERR_INVALID_ARG, "tile_bytes %d: only 4096 is supported", tile_bytes);
    if (num_tiles < 1) return fail(ABS_ERR_INVALID_ARG, "num_tiles %d < 1", num_tiles);
    if (workgroups < 1 || workgroups > 65535)
        return fail(ABS_ERR_INVALID_ARG, "workgroups %d outside [1, 65535]", workgroups);
    if (in_flight != 1 && in_flight != 2 && in_flight != 4 && in_flight != 8)
        return fail(ABS_ERR_INVALID_ARG, "in_flight %d not 1, 2, 4 or 8", in_flight);
    return hip_status(absk::launch_gather_tiles(tile_addr, num_tiles, workgroups, in_flight, xor_out,
                                                static_cast<hipStream_t>(stream)),
                      "gather_tiles");
}

abs_status abs_assign_block_sizes(int32_t num_kv_heads, const float* recall_host, float threshold,
                                  int32_t* block_size_host) {
    if (num_kv_heads < 1) return fail(ABS_ERR_INVALID_ARG, "num_kv_heads %d < 1", num_kv_heads);
    if (recall_host == nullptr || block_size_host == nullptr)
        return fail(ABS_ERR_INVALID_ARG, "null recall or block size array");
    if (!std::isfinite(threshold) || threshold <= 0.0f)
        return fail(ABS_ERR_INVALID_ARG, "threshold must be finite and > 0");
    for (int i = 0; i < 3 * num_kv_heads; ++i)
        if (!(recall_host[i] >= 0.0f && recall_host[i] <= 1.0f))
            return fail(ABS_ERR_INVALID_ARG, "recall[%d] = %g outside [0, 1]", i, (double)recall_host[i]);
    static constexpr int kSizes[3] = {16, 32, 64};
    for (int h = 0; h < num_kv_heads; ++h) {
        const double base = recall_host[h];
        int bs = kSizes[0];
        for (int k = 2; k >= 1; --k) {
            const double ratio = base > 0.0 ? (double)recall_host[k * num_kv_heads + h] / base : 1.0;
            if (ratio >= (double)threshold) {
                bs = kSizes[k];
                break;
            }
        }
        block_size_host[h] = bs;
    }
    return ok();
}

}  // extern "C"
