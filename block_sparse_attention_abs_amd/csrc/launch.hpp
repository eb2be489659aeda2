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
    int64_t num_pages;
    const void* k;
    const void* v;
    const int32_t* page_table;
    const int32_t* seq_lens;
    const int64_t* off;
    uint64_t bs_log2[kMaxKvHeads / 32];
};

__device__ __forceinline__ int block_size_of(const Geom& g, int h) {
    const uint64_t w = h < 32 ? g.bs_log2[0] : g.bs_log2[1];
    return 16 << (int)((w >> (2 * (h & 31))) & 3u);
}

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
constexpr int kScoreBlocksPerWg = 256;
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
    int32_t* sel;
    int32_t* count;
    int sel_cap;
    int budget;
    int max_n;        // largest N_{b,h}
    int max_len;      // largest L_b
    int64_t total_blocks;   // sum of N_{b,h}
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
    int chunk;        // pages held in registers at a time: 1, 2, 4 or 8
    bool pipelined;   // two chunks in flight (chunk 8, pages_per_wg a multiple of 16)
    int splits;
};

constexpr int kMaxPagesPerWg = 64;

hipError_t launch_decode(const Geom& g, DType dt, const DecodeArgs& a, hipStream_t s);

// abs_select_decode: the score launch alone (launch_scores), then one launch
// that runs the top-K inside the split decode (launch_select_decode), when
// select_decode_fusable(); otherwise launch_select and launch_decode.
constexpr int kFusedThreads = 512;                 // the fused launch's workgroup: the top-K launch's width
constexpr int kFusedTopkMaxN = kFusedThreads * 32;
constexpr int kComputeUnits = 256;                 // MI355X
hipError_t launch_scores(const Geom& g, DType dt, const SelectArgs& a, hipStream_t s);
bool select_decode_fusable(const Geom& g, DType dt, const SelectArgs& s, const DecodeArgs& a);
hipError_t launch_select_decode(const Geom& g, DType dt, const SelectArgs& s, const DecodeArgs& a, hipStream_t st);

// Calibration: recall[h] = mean over (b, query heads of h) of exp(lse_sel - lse_full).
hipError_t launch_head_recall(int B, int Hq, int Hkv, const float* lse_sel, const float* lse_full, float* recall,
                              hipStream_t s);

}  // namespace absk
