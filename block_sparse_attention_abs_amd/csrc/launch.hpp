// Internal interface between the C-ABI layer (abs_api.cpp) and the kernel
// launchers (*.hip).  Everything here has already been validated by the
// caller; launchers only size grids and enqueue kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace absk {

// Geometry of one layer's paged cache and block map, passed by value to kernels.
// The block sizes travel in the kernel arguments, 2 bits per KV head
// (log2(bs / 16)), so no workgroup waits on a memory read for them.
constexpr int kMaxKvHeads = 64;
struct Geom {
    int B, Hq, Hkv, D, G, max_pages;
    uint32_t hkv_magic;   // div_magic(Hkv): b = bh / Hkv without a division
    int max_len;          // the longest L_b on the host: every buffer is sized from it
    int64_t num_pages;
    const void* k;
    const void* v;
    const int32_t* page_table;
    const int32_t* seq_lens;
    const int64_t* off;
    uint64_t bs_log2[kMaxKvHeads / 32];
};

// L_b as the kernels use it: the device copy, clamped to [1, the host's
// longest length], so that a device value that disagrees with the host's
// (which sized every buffer and grid) cannot index past them.
__device__ __forceinline__ int seq_len(const Geom& g, int b) { return min(max(g.seq_lens[b], 1), g.max_len); }

// The same length read by a vector load, for kernels with a workgroup
// barrier before its first use: a barrier waits for every scalar load in
// flight, a vector load only where its value is used.  seq_len_issue()
// issues the load (the offset is an opaque zero in a vector register, so
// the load cannot be made scalar), seq_len_use() takes the value, uniform;
// its empty volatile statement keeps the wait for the load after any
// barrier that precedes the call.
__device__ __forceinline__ int seq_len_issue(const Geom& g, int b) {
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    return g.seq_lens[b + zero];
}
__device__ __forceinline__ int seq_len_use(const Geom& g, int issued) {
    asm volatile("" : "+v"(issued));
    return min(max(__builtin_amdgcn_readfirstlane(issued), 1), g.max_len);
}

// Centroid rows of (b, h) = bh that the kernels touch: its N blocks, capped
// by the rows the offsets give it (so that a device length that disagrees
// with the host's cannot index past the centroid store).
__device__ __forceinline__ int centroid_rows(const Geom& g, int bh, int N) {
    return (int)min((int64_t)N, g.off[bh + 1] - g.off[bh]);
}

// Division by a small runtime divisor d (1..64) without a division: with
// magic = ceil(2^32 / d), floor(n / d) = (n * magic) >> 32 for 0 <= n < 2^26
// (the rounding of the magic, n * (magic - 2^32 / d) < n * d / 2^32, stays
// below 1/d, the smallest gap between n/d and the next integer).  d = 1 has
// magic 0: the product vanishes and n is added back by a select, not a
// branch (a branch here splits the kernel's entry block, and the kernel
// argument loads after it then wait for a second round trip).
__host__ __device__ constexpr uint32_t div_magic(int d) {
    return d <= 1 ? 0u : (uint32_t)(((uint64_t)1 << 32) / (uint64_t)d + (((uint64_t)1 << 32) % (uint64_t)d != 0));
}
__host__ __device__ __forceinline__ constexpr int fast_div(int n, int d, uint32_t magic) {
    return (int)((uint32_t)(((uint64_t)(uint32_t)n * magic) >> 32) + (d == 1 ? (uint32_t)n : 0u));
}

// (b, h) of a flat index bh = b * Hkv + h.
__device__ __forceinline__ void split_bh(const Geom& g, int bh, int& b, int& h) {
    b = fast_div(bh, g.Hkv, g.hkv_magic);
    h = bh - b * g.Hkv;
}

// Block sizes are 16 << {0, 1, 2}: log2 of head h's block size.
__device__ __forceinline__ int block_shift_of(const Geom& g, int h) {
    const uint64_t w = h < 32 ? g.bs_log2[0] : g.bs_log2[1];
    return 4 + (int)((w >> (2 * (h & 31))) & 3u);
}

__device__ __forceinline__ int block_size_of(const Geom& g, int h) { return 1 << block_shift_of(g, h); }

// ceil(x / 2^s) for x >= 0.
__device__ __forceinline__ int shr_ceil(int x, int s) { return (x + (1 << s) - 1) >> s; }

enum class DType { F32 = 0, BF16 = 1 };

// Centroid storage formats (values of abs_centroid_format): bits per channel
// and bytes per centroid row.
enum CentFmt { kInt4 = 0, kInt4Sym = 1, kInt8 = 2, kInt4Tensor = 3, kBf16 = 4 };
__host__ __device__ constexpr int fmt_bits(int fmt) { return fmt == kInt8 ? 8 : fmt == kBf16 ? 16 : 4; }
__host__ __device__ constexpr int64_t row_bytes(int D, int fmt) { return (int64_t)D * fmt_bits(fmt) / 8; }

// Centroid build: a workgroup tile covers kBuildTileTokens tokens of one
// (b, h), i.e. kBuildTileTokens / bs_h blocks (64 at block size 16), so every
// tile holds the same number of keys whatever the head's block size.
constexpr int kBuildTileTokens = 1024;

struct BuildArgs {
    uint8_t* codes;
    float* scale;
    float* lo;
    float* staging;   // [B*Hkv][stage_rows][D] fp32 centroids
    float* pmin;      // [B*Hkv][tiles][D]
    float* pmax;      // [B*Hkv][tiles][D]
    int tiles;        // ceil(max L / kBuildTileTokens)
    int stage_rows;   // largest N_{b,h}
    int fmt;          // CentFmt
};

hipError_t launch_build(const Geom& g, DType dt, const BuildArgs& a, hipStream_t s);

// Centroids of the blocks touched by the last `appended` tokens, coded with
// the stored range.
struct UpdateArgs {
    const float* scale;
    const float* lo;
    uint8_t* codes;
    int32_t* out_of_range;   // [B*Hkv] or null
    int appended;
    int fmt;                 // CentFmt
};

hipError_t launch_update(const Geom& g, DType dt, const UpdateArgs& a, hipStream_t s);

// Score + select.
constexpr int kMaxBlocksPerHead = 65536;   // top-K keeps N_{b,h} keys in registers: 1024 x 64

// The score launch: 256 blocks per workgroup.
// When the tiles of all heads fit kMaxScoreTiles, they are listed in the
// kernel arguments ((b*Hkv + h) << 8 | tile) and the grid has exactly that
// many workgroups.  Otherwise the grid is (sum over heads of the tiles that
// head needs for the longest sequence, B): x is mapped to (head, tile)
// through the per-head cumulative tile counts in HeadTiles, and only the
// workgroups past a shorter sequence's blocks have nothing to do.
constexpr int kScoreBlocksPerWg = 256;             // 2^8: the top-K shifts by 8 to count tiles
constexpr int kMaxScoreTiles = 512;
struct ScoreTiles {
    uint32_t t[kMaxScoreTiles];
};
struct HeadTiles {
    uint32_t cum[kMaxKvHeads + 1];   // cum[0] = 0, cum[h + 1] - cum[h] = tiles of head h
};

struct SelectArgs {
    const uint8_t* codes;
    const float* scale;
    const float* lo;
    int fmt;          // CentFmt
    const void* q;
    float* scores;    // [B*Hkv][stride]
    int stride;       // max N_{b,h} rounded up to a multiple of 4
    float2* ranges;   // [B*Hkv][range_stride]: (min, max) score of each 256-block tile
    int range_stride; // tiles of the longest head
    int32_t* sel;
    int32_t* count;
    int sel_cap;
    int budget;
    int max_n;        // largest N_{b,h}
    int max_len;      // largest L_b
    int64_t total_blocks;   // sum of N_{b,h}
    int32_t* zero_counters;   // the score launch zero-fills these n_zero ints first (or null)
    int n_zero;
    int ntiles;       // score tiles over all heads
    const uint32_t* tiles_host;   // their list (host, valid during the call) or null
    HeadTiles head_tiles;         // per-head cumulative tiles for the longest sequence
};

hipError_t launch_select(const Geom& g, DType dt, const SelectArgs& a, hipStream_t s);

// Split-K sparse decode + merge.
struct DecodeArgs {
    const void* q;
    const int32_t* sel;
    const int32_t* count;
    int sel_cap;
    float sm_scale;
    void* out;
    float* lse;       // may be null
    float* part_ml;   // [B*Hq][splits][2]
    float* part_o;    // [B*Hq][splits][D]
    int32_t* arrive;  // [B*Hkv] arrival counters, zero between calls; null: separate merge launch
    int pages_per_wg; // <= kMaxPagesPerWg, a multiple of chunk
    uint32_t ppw_magic;   // div_magic(pages_per_wg)
    int chunk;        // pages held in registers at a time: 1, 2, 4 or 8
    bool pipelined;   // two chunks in flight (chunk 8, pages_per_wg a multiple of 16)
    int splits;
    int compute_units;   // of the device the launch runs on
};

constexpr int kMaxPagesPerWg = 64;

hipError_t launch_decode(const Geom& g, DType dt, const DecodeArgs& a, hipStream_t s);

// abs_select_decode: the score launch alone (launch_scores), then one launch
// that runs the top-K inside the split decode (launch_select_decode), when
// select_decode_fusable(); otherwise launch_select and launch_decode.
// The fused launch's workgroup: 256 threads (the decode's four wavefronts)
// when every head has at most kFusedSmallMaxN blocks, else 512 (eight
// wavefronts share the top-K of larger heads; four of them decode).
constexpr int kFusedThreads = 512;
constexpr int kFusedSmallMaxN = 256 * 16;
constexpr int kFusedTopkMaxN = kFusedThreads * 32;
hipError_t launch_scores(const Geom& g, DType dt, const SelectArgs& a, hipStream_t s);
hipError_t launch_topk(const Geom& g, const SelectArgs& a, hipStream_t s);   // the top-K launch alone
bool select_decode_fusable(const Geom& g, DType dt, const SelectArgs& s, const DecodeArgs& a);
hipError_t launch_select_decode(const Geom& g, DType dt, const SelectArgs& s, const DecodeArgs& a, hipStream_t st);

// Calibration: recall[h] = mean over (b, query heads of h) of exp(lse_sel - lse_full).
// Zero n ints at p (a fill kernel: no memset node, so it can be captured).
hipError_t launch_zero(int32_t* p, int n, hipStream_t s);

hipError_t launch_head_recall(int B, int Hq, int Hkv, const float* lse_sel, const float* lse_full, float* recall,
                              hipStream_t s);

// Measurement: n tiles of 4 KiB at the device addresses addr, read as the
// decode reads its K/V tiles; out[g] = XOR of the words workgroup g read.
hipError_t launch_gather_tiles(const uint64_t* addr, int n, int workgroups, int in_flight, uint32_t* out,
                               hipStream_t s);

}  // namespace absk
