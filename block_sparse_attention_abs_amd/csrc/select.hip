// Dot-product estimation and top-K selection (AB-Sparse page, Figure 1:
// importance score = query . block representation, then Top-K; the mapping
// figure after Figure 8: each head keeps K blocks, K set by its block size
// so every head reads the same number of pages).
//
// score:  one workgroup per (tile of 256 blocks, b*Hkv + h);
//         the tiles are listed in the launch when the list is short.  The group query
//         qbar = sum of the G query heads of KV head h is folded with the
//         per-channel dequantization once per workgroup:
//             w_d = qbar_d * scale_d,   c0 = sum_d qbar_d * lo_d,
//             score_j = c0 + sum_d w_d * code_{j,d}
//         (fp64 inside, stored as fp32 in a [b*Hkv+h][stride] scratch with
//         16-byte aligned rows).  The lanes of one block row load 16 bytes
//         of codes each (head_dim/32 lanes for INT4, head_dim/16 for INT8,
//         head_dim/8 for bf16 centroids, whose w_d is qbar_d and c0 = 0),
//         so one load instruction reads a contiguous 1 KiB run per
//         wavefront.  Every load is unconditional (offsets clamped), the
//         query, scale and lo first, then all of a lane's code rows, so
//         the fold waits only for the former.
// top-K:  one workgroup per (b, h) running topk_rows (topk.hpp): a value
//         histogram, the exact rank of the threshold bin's candidates (or a
//         radix select when that bin is crowded), the kept indices written
//         in ascending order.
#include "device.hpp"
#include "topk.hpp"

namespace absk {
namespace {

// Build-time tuning: threads of a score workgroup (256 or 512).
#ifndef ABS_SCORE_NT
#define ABS_SCORE_NT 256
#endif

// One tile of 256 blocks of (b, h) = bh, by an ABS_SCORE_NT-thread
// workgroup; BITS = 4 (INT4 codes), 8 (INT8 codes) or 16 (bf16 centroids).
template <typename T, int D, int GT, int BITS>
__device__ __forceinline__ void score_tile(const Geom& g, const uint8_t* __restrict__ codes,
                                           const float* __restrict__ scale, const float* __restrict__ lo,
                                           const T* __restrict__ q, float* __restrict__ scores, int stride, int bh,
                                           int tile) {
    constexpr int NT = ABS_SCORE_NT;
    constexpr int CPL = 128 / BITS;           // channels per lane (16 B of codes)
    constexpr int LPB = D / CPL;              // lanes per block row
    constexpr int GPW = NT / LPB;             // lane groups per workgroup
    constexpr int RPL = kScoreBlocksPerWg / GPW;   // block rows per lane group
    constexpr int RB = D * BITS / 8;          // bytes per row
    constexpr int PER = 32 / BITS;            // channels per 32-bit word
    static_assert(NT >= D, "one thread per channel folds the query");
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int64_t row0 = g.off[bh];
    const int N = ceil_div(g.seq_lens[b], block_size_of(g, h));
    const int j0 = tile * kScoreBlocksPerWg;
    const int sub = threadIdx.x % LPB;
    const int grp = threadIdx.x / LPB;

    // Every load below is unconditional (offsets clamped), so all of them are
    // in flight together and none waits on a branch; the query group, scale
    // and lo go first, so that the fold below waits only for them.  A tile
    // past the end of a shorter sequence (j0 >= N, in the per-sequence grid)
    // runs through and stores nothing.
    const int dch = min((int)threadIdx.x, D - 1);    // this thread's channel (threads < D)
    float qv[GT], sc = 0.0f, zp = 0.0f;
#pragma unroll
    for (int gg = 0; gg < GT; ++gg)
        qv[gg] = Elem<T>::load1(q + ((int64_t)b * g.Hq + h * g.G + min(gg, g.G - 1)) * D + dch);
    if constexpr (BITS != 16) {
        sc = scale[(int64_t)bh * D + dch];
        zp = lo[(int64_t)bh * D + dch];
    }
    // RPL block rows per lane group, GPW consecutive rows per step (contiguous
    // runs); a row at or beyond N reads row N - 1 again (N >= 1) and is not
    // stored
    uint4 v[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int j = min(j0 + r * GPW + grp, N - 1);
        const Words<4> cw = load_words_stream<4>(codes + (row0 + j) * RB + sub * 16);
        v[r] = make_uint4(cw.w[0], cw.w[1], cw.w[2], cw.w[3]);
    }

    // per channel: w_d = qbar_d * scale_d and z_d = qbar_d * lo_d (fp64, LDS);
    // bf16 centroids are values already: w_d = qbar_d, z_d = 0.  Every thread
    // writes its slot (those past D are never read), so no branch holds the
    // loads above back.
    // one padding slot after each lane's CPL channels: the LPB lanes of a
    // row, which read the same n-th channel of their own runs, then hit
    // different LDS banks (unpadded, their addresses are 256 B apart for
    // INT4 and conflict)
    constexpr int CS = CPL + 1;
    __shared__ double w[NT + NT / CPL], z[NT + NT / CPL];
    {
        // the group's G heads count, the padding slots (G < GT) add +0; the
        // mask is opaque to the optimizer, which would otherwise move a
        // padding slot's load into a branch behind the code loads
        double qbar = 0.0;
#pragma unroll
        for (int gg = 0; gg < GT; ++gg) {
            uint32_t keep = gg < g.G ? ~0u : 0u;
            asm volatile("" : "+v"(keep));
            qbar += (double)__uint_as_float(__float_as_uint(qv[gg]) & keep);
        }
        const int slot = threadIdx.x + threadIdx.x / CPL;
        w[slot] = BITS == 16 ? qbar : qbar * (double)sc;
        z[slot] = BITS == 16 ? 0.0 : qbar * (double)zp;
    }
    __syncthreads();

    // this lane's CPL channels: its share of sum_d z_d once, then sum_d w_d *
    // value_d per row (two accumulators per row); the LPB lanes of a row then
    // add up
    double wr[CPL], c0 = 0.0;
#pragma unroll
    for (int n = 0; n < CPL; ++n) {
        wr[n] = w[sub * CS + n];
        if constexpr (BITS != 16) c0 += z[sub * CS + n];
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const uint32_t wd[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
        double acc[2] = {c0, 0.0};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int n = 0; n < PER; ++n) {
                double x;
                if constexpr (BITS == 16)
                    x = (double)__uint_as_float(n == 0 ? wd[i] << 16 : wd[i] & 0xFFFF0000u);
                else
                    x = (double)((wd[i] >> (BITS * n)) & ((1u << BITS) - 1u));
                acc[i >> 1] = fma(wr[i * PER + n], x, acc[i >> 1]);
            }
        const double sum = lanes_sum_f64<LPB>(acc[0] + acc[1]);
        const int j = j0 + r * GPW + grp;
        if (j < N && sub == 0) scores[(int64_t)bh * stride + j] = (float)sum;
    }
}

// Grid (tiles per sequence, B): x -> (head, tile) by a binary search of the
// per-head cumulative tile counts (uniform, kernel-argument reads only).
template <typename T, int D, int GT, int BITS>
__global__ __launch_bounds__(ABS_SCORE_NT) void k_score_seq(Geom g, const uint8_t* __restrict__ codes,
                                                   const float* __restrict__ scale, const float* __restrict__ lo,
                                                   const T* __restrict__ q, float* __restrict__ scores, int stride,
                                                   const HeadTiles ht) {
    const uint32_t x = blockIdx.x;
    int hl = 0, hh = g.Hkv;                          // ht.cum[hl] <= x < ht.cum[hh]
    while (hh - hl > 1) {
        const int mid = (hl + hh) >> 1;
        if (ht.cum[mid] <= x) hl = mid;
        else hh = mid;
    }
    score_tile<T, D, GT, BITS>(g, codes, scale, lo, q, scores, stride, (int)blockIdx.y * g.Hkv + hl,
                               (int)(x - ht.cum[hl]));
}

template <typename T, int D, int GT, int BITS>
__global__ __launch_bounds__(ABS_SCORE_NT) void k_score_list(Geom g, const uint8_t* __restrict__ codes,
                                                    const float* __restrict__ scale, const float* __restrict__ lo,
                                                    const T* __restrict__ q, float* __restrict__ scores, int stride,
                                                    const ScoreTiles tl) {
    const uint32_t e = tl.t[blockIdx.x];
    score_tile<T, D, GT, BITS>(g, codes, scale, lo, q, scores, stride, (int)(e >> 8), (int)(e & 255u));
}

// Build-time tuning: threads of the top-K workgroup.
#ifndef ABS_TOPK_NT
#define ABS_TOPK_NT 512
#endif

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void k_topk(Geom g, const float* __restrict__ scores, int stride, int max_len,
                                             int budget, int32_t* __restrict__ sel, int sel_cap,
                                             int32_t* __restrict__ count) {
    const int bh = blockIdx.x;
    int32_t* out = sel + (int64_t)bh * sel_cap;
    const int K = topk_rows<NT, KPT>(g, bh, scores + (int64_t)bh * stride, stride, max_len, budget,
                                     [&](uint32_t p, int32_t j) { out[p] = j; });
    if (threadIdx.x == 0) count[bh] = K;
}

template <typename T, int D, int BITS>
void launch_score(const Geom& g, const SelectArgs& a, hipStream_t s) {
    const T* q = reinterpret_cast<const T*>(a.q);
    if (a.tiles_host != nullptr && a.ntiles <= kMaxScoreTiles) {
        ScoreTiles tl;
        for (int i = 0; i < a.ntiles; ++i) tl.t[i] = a.tiles_host[i];
#define ABS_SCORE(GT_)                                                                                    \
    hipLaunchKernelGGL((k_score_list<T, D, GT_, BITS>), dim3(a.ntiles), dim3(ABS_SCORE_NT), 0, s, g, a.codes, \
                       a.scale, a.lo, q, a.scores, a.stride, tl)
        if (g.G <= 1) ABS_SCORE(1);
        else if (g.G <= 2) ABS_SCORE(2);
        else if (g.G <= 4) ABS_SCORE(4);
        else ABS_SCORE(8);
#undef ABS_SCORE
    } else {
        const dim3 sgrid(a.head_tiles.cum[g.Hkv], g.B);
#define ABS_SCORE(GT_)                                                                                       \
    hipLaunchKernelGGL((k_score_seq<T, D, GT_, BITS>), sgrid, dim3(ABS_SCORE_NT), 0, s, g, a.codes, a.scale, a.lo, \
                       q, a.scores, a.stride, a.head_tiles)
        if (g.G <= 1) ABS_SCORE(1);
        else if (g.G <= 2) ABS_SCORE(2);
        else if (g.G <= 4) ABS_SCORE(4);
        else ABS_SCORE(8);
#undef ABS_SCORE
    }
}

template <typename T, int D>
hipError_t select_impl(const Geom& g, const SelectArgs& a, bool with_topk, hipStream_t s) {
    const int bits = fmt_bits(a.fmt);
    if (bits == 8) launch_score<T, D, 8>(g, a, s);
    else if (bits == 16) launch_score<T, D, 16>(g, a, s);
    else launch_score<T, D, 4>(g, a, s);
    if (!with_topk) return hipGetLastError();
    const dim3 tgrid(g.B * g.Hkv);
#define ABS_TOPK(NT_, KPT_)                                                                                  \
    hipLaunchKernelGGL((k_topk<NT_, KPT_>), tgrid, dim3(NT_), 0, s, g, a.scores, a.stride, a.max_len, a.budget, \
                       a.sel, a.sel_cap, a.count)
    // ABS_TOPK_NT threads, each holding up to 32 keys; 1024 x 64 beyond that
    constexpr int NT = ABS_TOPK_NT;
    const int n = a.max_n;
    if (n <= NT * 1) ABS_TOPK(NT, 1);
    else if (n <= NT * 2) ABS_TOPK(NT, 2);
    else if (n <= NT * 4) ABS_TOPK(NT, 4);
    else if (n <= NT * 8) ABS_TOPK(NT, 8);
    else if (n <= NT * 16) ABS_TOPK(NT, 16);
    else if (n <= NT * 32) ABS_TOPK(NT, 32);
    else ABS_TOPK(1024, 64);
#undef ABS_TOPK
    return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const Geom& g, DType dt, const SelectArgs& a, hipStream_t s) {
    if (dt == DType::BF16)
        return g.D == 128 ? select_impl<uint16_t, 128>(g, a, true, s) : select_impl<uint16_t, 64>(g, a, true, s);
    return g.D == 128 ? select_impl<float, 128>(g, a, true, s) : select_impl<float, 64>(g, a, true, s);
}

hipError_t launch_scores(const Geom& g, DType dt, const SelectArgs& a, hipStream_t s) {
    if (dt == DType::BF16)
        return g.D == 128 ? select_impl<uint16_t, 128>(g, a, false, s) : select_impl<uint16_t, 64>(g, a, false, s);
    return g.D == 128 ? select_impl<float, 128>(g, a, false, s) : select_impl<float, 64>(g, a, false, s);
}

}  // namespace absk
