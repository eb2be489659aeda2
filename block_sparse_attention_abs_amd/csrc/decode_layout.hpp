// Launch layout of the split decode (pages per workgroup, chunk, splits) and
// its workspace carve-up, from the layer's size alone.  Kept apart from the
// C-ABI layer because it decides the kernel's traffic as much as the kernel
// source does.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "launch.hpp"

namespace absk {

inline int64_t layout_ceil(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t layout_align(size_t x) { return (x + 255) / 256 * 256; }

struct DecodeLayout {
    int ppw = 8, chunk = 8, splits = 1;
    bool pipelined = false;
    size_t arrive = 0, ml = 0, o = 0, bytes = 0;
};

// Build-time tuning of the decode launch (see decode_layout).
#ifndef ABS_DECODE_TARGET_WGS
#define ABS_DECODE_TARGET_WGS 1024
#endif
#ifndef ABS_DECODE_MAX_CHUNK
#define ABS_DECODE_MAX_CHUNK 8
#endif
// Workgroups of the double-buffered layout; 0: one per compute unit of the
// device (read at run time).
#ifndef ABS_DECODE_PIPE_WGS
#define ABS_DECODE_PIPE_WGS 0
#endif
// At most this many splits per (b, h) outside the double-buffered layout:
// the merging workgroup reads the splits' partials 8 at a time, so a
// small layer does better with more pages per workgroup than with a long
// merge.
#ifndef ABS_DECODE_MAX_SPLITS
#define ABS_DECODE_MAX_SPLITS 16
#endif
// 1: the last split workgroup of each (b, h) merges (one launch); 0: a merge launch.
#ifndef ABS_DECODE_FUSED_MERGE
#define ABS_DECODE_FUSED_MERGE 1
#endif

// Pages per workgroup: enough workgroups to fill the chip (about
// ABS_DECODE_TARGET_WGS) but at most kMaxPagesPerWg pages each; pages are
// held in registers `chunk` at a time.  `compute_units`: of the device the
// launch runs on.
inline DecodeLayout decode_layout(int B, int Hkv, int Hq, int D, int max_pages_read, int compute_units) {
    DecodeLayout l;
    const int64_t heads = (int64_t)B * Hkv;
    const int64_t maxp = std::max(max_pages_read, 1);
    const int64_t ideal = std::max<int64_t>(1, layout_ceil(heads * maxp, ABS_DECODE_TARGET_WGS));
    const int64_t cmax = ABS_DECODE_MAX_CHUNK;
    l.chunk = (int)std::min<int64_t>(cmax, ideal >= 8 ? 8 : ideal >= 4 ? 4 : ideal >= 2 ? 2 : 1);
    l.ppw = (int)std::min<int64_t>(kMaxPagesPerWg, layout_ceil(ideal, l.chunk) * l.chunk);
    l.splits = (int)layout_ceil(maxp, l.ppw);
    if (l.splits > ABS_DECODE_MAX_SPLITS) {
        const int64_t need = layout_ceil(maxp, ABS_DECODE_MAX_SPLITS);
        l.chunk = (int)std::min<int64_t>(cmax, need >= 8 ? 8 : need >= 4 ? 4 : need >= 2 ? 2 : 1);
        l.ppw = (int)std::min<int64_t>(kMaxPagesPerWg, layout_ceil(need, l.chunk) * l.chunk);
        l.splits = (int)layout_ceil(maxp, l.ppw);
    }
    // Enough pages for two chunks of 8 per workgroup at one workgroup per
    // compute unit: stream them double-buffered instead.
    const int64_t pipe_wgs = ABS_DECODE_PIPE_WGS > 0 ? ABS_DECODE_PIPE_WGS : std::max(1, compute_units);
    if (heads * maxp >= pipe_wgs * 16) {
        const int64_t per = layout_ceil(heads * maxp, pipe_wgs);
        l.chunk = 8;
        l.pipelined = true;
        l.ppw = (int)std::min<int64_t>(kMaxPagesPerWg, std::max<int64_t>(16, layout_ceil(per, 16) * 16));
        l.splits = (int)layout_ceil(maxp, l.ppw);
    }
    const size_t rows = (size_t)B * Hq * l.splits;
    l.arrive = 0;
    l.ml = layout_align((size_t)B * Hkv * sizeof(int32_t));
    l.o = l.ml + layout_align(rows * 2 * sizeof(float));
    l.bytes = l.o + layout_align(rows * D * sizeof(float));
    return l;
}

}  // namespace absk
