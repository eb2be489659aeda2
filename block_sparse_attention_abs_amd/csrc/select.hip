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
//         (stored as fp32 in a [b*Hkv+h][stride] scratch with 16-byte
//         aligned rows; exact integer sums of the codes against 30-bit
//         rounded weights for the 4- and 8-bit formats, see the fold, and
//         fp64 for bf16 centroids).  The lanes of one block row load 16 bytes
//         of codes each (head_dim/32 lanes for INT4, head_dim/16 for INT8,
//         head_dim/8 for bf16 centroids, whose w_d is qbar_d and c0 = 0),
//         so one load instruction reads a contiguous 1 KiB run per
//         wavefront.  Every load is unconditional (offsets clamped): the
//         row's bounds, the query, scale and lo, then all of a lane's code
//         rows, so the fold waits only for the query, scale and lo.
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
                                           const T* __restrict__ q, float* __restrict__ scores, int stride,
                                           float2* __restrict__ ranges, int range_stride, int bh, int tile) {
    constexpr int NT = ABS_SCORE_NT;
    constexpr int CPL = 128 / BITS;           // channels per lane (16 B of codes)
    constexpr int LPB = D / CPL;              // lanes per block row
    constexpr int GPW = NT / LPB;             // lane groups per workgroup
    constexpr int RPL = kScoreBlocksPerWg / GPW;   // block rows per lane group
    constexpr int RB = D * BITS / 8;          // bytes per row
    constexpr int PER = 32 / BITS;            // channels per 32-bit word
    static_assert(NT >= D, "one thread per channel folds the query");
    int b, h;
    split_bh(g, bh, b, h);
    const int j0 = tile * kScoreBlocksPerWg;
    const int sub = threadIdx.x % LPB;
    const int grp = threadIdx.x / LPB;

    // Every load below is unconditional (offsets clamped), so all of them are
    // in flight together and none waits on a branch.  First the row's bounds
    // (centroid offsets and length) by vector loads, then the query group,
    // scale and lo, which need only (b, h) and so go out at once, then the
    // code rows, which wait for the bounds only (scalar loads of the bounds
    // would put a round trip before every load, and barriers wait for them).
    // A tile past the end of a shorter sequence (j0 >= N, in the per-sequence
    // grid) runs through and stores nothing.
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const int64_t off0 = g.off[bh + zero], off1 = g.off[bh + 1 + zero];
    const int len = g.seq_lens[b + zero];
    const int dch = min((int)threadIdx.x, D - 1);    // this thread's channel (threads < D)
    T qraw[GT];                                       // converted after the code loads are out
    float sc = 0.0f, zp = 0.0f;
#pragma unroll
    for (int gg = 0; gg < GT; ++gg) qraw[gg] = q[((int64_t)b * g.Hq + h * g.G + min(gg, g.G - 1)) * D + dch];
    if constexpr (BITS != 16) {
        sc = scale[(int64_t)bh * D + dch];
        zp = lo[(int64_t)bh * D + dch];
    }
    __builtin_amdgcn_sched_barrier(0);
    // 64-bit offsets through scalar registers, each half as unsigned (readfirstlane
    // returns int: a sign-extended low half would fill the high half with ones)
    const int64_t row0 = (int64_t)((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)off0) |
                                   ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off0 >> 32)) << 32));
    const int64_t rows = (int64_t)((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)off1) |
                                   ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off1 >> 32)) << 32)) -
                         row0;
    const int L = min(max(__builtin_amdgcn_readfirstlane(len), 1), g.max_len);
    const int N = (int)min((int64_t)shr_ceil(L, block_shift_of(g, h)), rows);   // as centroid_rows()
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
    // integer weights (4- and 8-bit codes): one run per lane's channels (32
    // for 4-bit codes, 16 for 8-bit), NKW words of digits each, KRS words
    // apart (padding: 16-byte aligned, and the runs of a row's lanes in
    // different banks)
    constexpr bool INT = BITS == 4 || BITS == 8;
    constexpr int NKW = BITS == 4 ? 32 : 16;
    constexpr int KRS = BITS == 4 ? 36 : 20;
    __shared__ __align__(16) uint32_t kq[INT ? (D / CPL) * KRS : 1];
    __shared__ int kE[INT ? D / CPL : 1];
    {
        // the group's G heads count, the padding slots (G < GT) add +0; the
        // mask is opaque to the optimizer, which would otherwise move a
        // padding slot's load into a branch behind the code loads
        double qbar = 0.0;
#pragma unroll
        for (int gg = 0; gg < GT; ++gg) {
            uint32_t keep = gg < g.G ? ~0u : 0u;
            asm volatile("" : "+v"(keep));
            qbar += (double)__uint_as_float(__float_as_uint(Elem<T>::cvt(qraw[gg])) & keep);
        }
        const int slot = threadIdx.x + threadIdx.x / CPL;
        w[slot] = BITS == 16 ? qbar : qbar * (double)sc;
        z[slot] = BITS == 16 ? 0.0 : qbar * (double)zp;
        if constexpr (INT) {
            // 4- and 8-bit codes: each run of channels one lane of a row reads
            // (32 or 16) gets a scale 2^E from its largest |w_d| (a max over
            // the run's threads), and each weight becomes an integer k_d =
            // rint(w_d / 2^E), |k_d| <= 2^30, stored as four signed base-256
            // digits, so that sum_d code_d k_d is exact in int32 dot products
            // of four 8-bit pairs (v_dot4_i32_i8; 8-bit codes enter as code -
            // 128, and 128 sum_d k_d is added back).  Each weight then carries
            // |w_d - k_d 2^E| <= 2^-30 max_run |w|, a score at most 128 x
            // (2^BITS - 1) x 2^-30 max_d |w_d| <= 2.4e-7 M (M = sum_d |qbar_d|
            // max(|lo_d|, |hi_d|) >= (2^BITS - 1) max_d |w_d| / 2), and equal
            // codes give equal sums.
            const double wv = qbar * (double)sc;
            int ev = 0;
            (void)frexp(wv, &ev);                    // |wv| < 2^ev
            const float ef = wv != 0.0 ? (float)ev : -4096.0f;
            const float emax = BITS == 4 ? half32_max(ef) : row16_max(ef);
            const int E = (int)emax - 30;
            const int k = (int)rint(ldexp(wv, -E));
            const int d0 = ((k + 128) & 255) - 128, k1 = (k - d0) / 256;
            const int d1 = ((k1 + 128) & 255) - 128, k2 = (k1 - d1) / 256;
            const int d2 = ((k2 + 128) & 255) - 128, d3 = (k2 - d2) / 256;   // |d3| <= 65
            if ((int)threadIdx.x < D) {
                const int c = threadIdx.x % CPL, run = threadIdx.x / CPL;
                // 4-bit: word ((8-channel group) * 2 + parity) * 4 + digit of the run, byte = position in the
                // group's pair (a word of codes holds the group's even channels in its low nibbles, the odd
                // ones in its high nibbles); 8-bit: word (4-channel group) * 4 + digit, byte = position in
                // the group
                int8_t* dst = reinterpret_cast<int8_t*>(kq + run * KRS) +
                              (BITS == 4 ? ((c >> 3) * 2 + (c & 1)) * 16 + ((c & 7) >> 1) : (c >> 2) * 16 + (c & 3));
                dst[0] = (int8_t)d0;
                dst[4] = (int8_t)d1;
                dst[8] = (int8_t)d2;
                dst[12] = (int8_t)d3;
                if (c == 0) kE[run] = E;
            }
        }
    }
    __syncthreads();

    // this lane's CPL channels: its share of sum_d z_d once, then sum_d w_d *
    // value_d per row (two accumulators per row); the LPB lanes of a row then
    // add up
    double wr[CPL], c0 = 0.0;
#pragma unroll
    for (int n = 0; n < CPL; ++n) {
        if constexpr (BITS == 16) wr[n] = w[sub * CS + n];
        if constexpr (BITS != 16) c0 += z[sub * CS + n];
    }
    uint32_t kw[NKW];                                // 4- and 8-bit codes: this lane's run of integer weights
    int E = 0;
    int64_t bias = 0;                                // 8-bit codes: 128 sum_d k_d over the run (codes enter as code - 128)
    if constexpr (INT) {
#pragma unroll
        for (int n = 0; n < NKW; ++n) kw[n] = kq[sub * KRS + n];
        E = kE[sub];
    }
    if constexpr (BITS == 8) {
#pragma unroll
        for (int L = 0; L < 4; ++L) {
            int s = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) s = __builtin_amdgcn_sdot4((int)kw[i * 4 + L], 0x01010101, s, false);
            bias += (int64_t)s << (8 * L);
        }
        bias *= 128;
    }
    float tmn = __builtin_inff(), tmx = -__builtin_inff();   // the tile's range of stored scores
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const uint32_t wd[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
        double part;
        if constexpr (BITS == 4) {
            // digit sums: |s_L| <= 32 x 15 x 128; sum_L s_L 256^L is sum code k exactly (< 2^40)
            int sd[4] = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ev = (int)(wd[i] & 0x0F0F0F0Fu);          // channels 8i + 0, 2, 4, 6 (one per byte)
                const int od = (int)((wd[i] >> 4) & 0x0F0F0F0Fu);   // channels 8i + 1, 3, 5, 7
#pragma unroll
                for (int L = 0; L < 4; ++L) {
                    sd[L] = __builtin_amdgcn_sdot4(ev, (int)kw[(2 * i) * 4 + L], sd[L], false);
                    sd[L] = __builtin_amdgcn_sdot4(od, (int)kw[(2 * i + 1) * 4 + L], sd[L], false);
                }
            }
            const int64_t sum_k = (int64_t)sd[0] + (int64_t)sd[1] * 256 + (int64_t)sd[2] * 65536 +
                                  (int64_t)sd[3] * 16777216;
            part = c0 + ldexp((double)sum_k, E);
        } else if constexpr (BITS == 8) {
            // digit sums: |s_L| <= 16 x 128 x 128; sum_L s_L 256^L + 128 sum_d k_d is sum code k exactly
            int sd[4] = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int cv = (int)(wd[i] ^ 0x80808080u);           // channels 4i .. 4i + 3 as code - 128
#pragma unroll
                for (int L = 0; L < 4; ++L) sd[L] = __builtin_amdgcn_sdot4(cv, (int)kw[i * 4 + L], sd[L], false);
            }
            const int64_t sum_k = (int64_t)sd[0] + (int64_t)sd[1] * 256 + (int64_t)sd[2] * 65536 +
                                  (int64_t)sd[3] * 16777216 + bias;
            part = c0 + ldexp((double)sum_k, E);
        } else {
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
            part = acc[0] + acc[1];
        }
        const double sum = lanes_sum_f64<LPB>(part);
        const int j = j0 + r * GPW + grp;
        if (j < N && sub == 0) scores[(int64_t)bh * stride + j] = (float)sum;
        tmn = j < N ? fminf(tmn, (float)sum) : tmn;
        tmx = j < N ? fmaxf(tmx, (float)sum) : tmx;
    }
    // (min, max) over the tile's stored scores, for the top-K's binning
    // (a tile past the row's end writes the empty range)
    __shared__ float s_rng[2][NT / 64];
    tmx = wave_max(tmx);
    tmn = -wave_max(-tmn);
    if ((threadIdx.x & 63) == 0) {
        s_rng[0][threadIdx.x >> 6] = tmn;
        s_rng[1][threadIdx.x >> 6] = tmx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) {
            tmn = fminf(tmn, s_rng[0][w]);
            tmx = fmaxf(tmx, s_rng[1][w]);
        }
        ranges[(int64_t)bh * range_stride + tile] = make_float2(tmn, tmx);
    }
}

// The decode's arrival counters, zeroed by the first score workgroup when
// the decode follows in the same call (zc null: nothing to do).
__device__ __forceinline__ void zero_ints(int32_t* zc, int nz) {
    if (zc != nullptr)
        for (int i = threadIdx.x; i < nz; i += ABS_SCORE_NT) zc[i] = 0;
}

// Grid (tiles per sequence, B): x -> (head, tile) by a binary search of the
// per-head cumulative tile counts (uniform, kernel-argument reads only).
template <typename T, int D, int GT, int BITS>
__global__ __launch_bounds__(ABS_SCORE_NT) void k_score_seq(Geom g, const uint8_t* __restrict__ codes,
                                                   const float* __restrict__ scale, const float* __restrict__ lo,
                                                   const T* __restrict__ q, float* __restrict__ scores, int stride,
                                                   float2* __restrict__ ranges, int range_stride,
                                                   const HeadTiles ht, int32_t* __restrict__ zc, int nz) {
    const uint32_t x = blockIdx.x;
    int hl = 0, hh = g.Hkv;                          // ht.cum[hl] <= x < ht.cum[hh]
    while (hh - hl > 1) {
        const int mid = (hl + hh) >> 1;
        if (ht.cum[mid] <= x) hl = mid;
        else hh = mid;
    }
    score_tile<T, D, GT, BITS>(g, codes, scale, lo, q, scores, stride, ranges, range_stride,
                               (int)blockIdx.y * g.Hkv + hl, (int)(x - ht.cum[hl]));
    if (x == 0 && blockIdx.y == 0) zero_ints(zc, nz);
}

template <typename T, int D, int GT, int BITS>
__global__ __launch_bounds__(ABS_SCORE_NT) void k_score_list(Geom g, const uint8_t* __restrict__ codes,
                                                    const float* __restrict__ scale, const float* __restrict__ lo,
                                                    const T* __restrict__ q, float* __restrict__ scores, int stride,
                                                    float2* __restrict__ ranges, int range_stride,
                                                    const ScoreTiles tl, int32_t* __restrict__ zc, int nz) {
    const uint32_t e = tl.t[blockIdx.x];
    score_tile<T, D, GT, BITS>(g, codes, scale, lo, q, scores, stride, ranges, range_stride, (int)(e >> 8),
                               (int)(e & 255u));
    if (blockIdx.x == 0) zero_ints(zc, nz);
}

// Build-time tuning: threads of the top-K workgroup.
#ifndef ABS_TOPK_NT
#define ABS_TOPK_NT 512
#endif

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void k_topk(Geom g, const float* __restrict__ scores, int stride,
                                             const float2* __restrict__ ranges, int range_stride, int max_len,
                                             int budget, int32_t* __restrict__ sel, int sel_cap,
                                             int32_t* __restrict__ count) {
    const int bh = blockIdx.x;
    int32_t* out = sel + (int64_t)bh * sel_cap;
    int L;
    const int K = topk_rows<NT, KPT>(g, bh, scores + (int64_t)bh * stride, stride,
                                     ranges + (int64_t)bh * range_stride, max_len, budget,
                                     [&](uint32_t p, int32_t j) {
                                         if (p < (uint32_t)sel_cap) out[p] = j;
                                     }, L);
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
                       a.scale, a.lo, q, a.scores, a.stride, a.ranges, a.range_stride, tl, a.zero_counters, \
                       a.n_zero)
        if (g.G <= 1) ABS_SCORE(1);
        else if (g.G <= 2) ABS_SCORE(2);
        else if (g.G <= 4) ABS_SCORE(4);
        else ABS_SCORE(8);
#undef ABS_SCORE
    } else {
        const dim3 sgrid(a.head_tiles.cum[g.Hkv], g.B);
#define ABS_SCORE(GT_)                                                                                       \
    hipLaunchKernelGGL((k_score_seq<T, D, GT_, BITS>), sgrid, dim3(ABS_SCORE_NT), 0, s, g, a.codes, a.scale, a.lo, \
                       q, a.scores, a.stride, a.ranges, a.range_stride, a.head_tiles, a.zero_counters, a.n_zero)
        if (g.G <= 1) ABS_SCORE(1);
        else if (g.G <= 2) ABS_SCORE(2);
        else if (g.G <= 4) ABS_SCORE(4);
        else ABS_SCORE(8);
#undef ABS_SCORE
    }
}

hipError_t topk_impl(const Geom& g, const SelectArgs& a, hipStream_t s) {
    const dim3 tgrid(g.B * g.Hkv);
#define ABS_TOPK(NT_, KPT_)                                                                                  \
    hipLaunchKernelGGL((k_topk<NT_, KPT_>), tgrid, dim3(NT_), 0, s, g, a.scores, a.stride, a.ranges,            \
                       a.range_stride, a.max_len, a.budget,                                                \
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

template <typename T, int D>
hipError_t select_impl(const Geom& g, const SelectArgs& a, bool with_topk, hipStream_t s) {
    const int bits = fmt_bits(a.fmt);
    if (bits == 8) launch_score<T, D, 8>(g, a, s);
    else if (bits == 16) launch_score<T, D, 16>(g, a, s);
    else launch_score<T, D, 4>(g, a, s);
    if (!with_topk) return hipGetLastError();
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    return topk_impl(g, a, s);
}

}  // namespace

hipError_t launch_select(const Geom& g, DType dt, const SelectArgs& a, hipStream_t s) {
    if (dt == DType::BF16)
        return g.D == 128 ? select_impl<uint16_t, 128>(g, a, true, s) : select_impl<uint16_t, 64>(g, a, true, s);
    return g.D == 128 ? select_impl<float, 128>(g, a, true, s) : select_impl<float, 64>(g, a, true, s);
}

hipError_t launch_topk(const Geom& g, const SelectArgs& a, hipStream_t s) { return topk_impl(g, a, s); }

hipError_t launch_scores(const Geom& g, DType dt, const SelectArgs& a, hipStream_t s) {
    if (dt == DType::BF16)
        return g.D == 128 ? select_impl<uint16_t, 128>(g, a, false, s) : select_impl<uint16_t, 64>(g, a, false, s);
    return g.D == 128 ? select_impl<float, 128>(g, a, false, s) : select_impl<float, 64>(g, a, false, s);
}

}  // namespace absk
