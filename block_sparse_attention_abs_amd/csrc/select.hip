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
// top-K:  one workgroup per (b, h); thread t owns block indices
//         [t*KPT, (t+1)*KPT) as order-preserving 32-bit keys in registers.
//         1. min/max of the scores; a 2048-bin histogram of the scores'
//            position in [min, max] (a monotone binning, spread over the
//            bins, so LDS atomics rarely collide);
//         2. the bin b* holding the K-th largest score, and how many scores
//            lie in higher bins;
//         3. the few candidates in b* are ranked exactly by (score desc,
//            index asc), giving the threshold pair (tau_key, tau_index);
//            if b* is crowded (heavy ties) an 8-bit radix select over the
//            keys gives the same pair instead;
//         4. keep key > tau_key, or key == tau_key and index <= tau_index;
//            a block scan writes the kept indices in ascending order.
#include <type_traits>

#include "device.hpp"

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
    __shared__ double w[NT], z[NT];
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
        w[threadIdx.x] = BITS == 16 ? qbar : qbar * (double)sc;
        z[threadIdx.x] = BITS == 16 ? 0.0 : qbar * (double)zp;
    }
    __syncthreads();

    // this lane's CPL channels: its share of sum_d z_d once, then sum_d w_d *
    // value_d per row (two accumulators per row); the LPB lanes of a row then
    // add up
    double wr[CPL], c0 = 0.0;
#pragma unroll
    for (int n = 0; n < CPL; ++n) {
        wr[n] = w[sub * CPL + n];
        if constexpr (BITS != 16) c0 += z[sub * CPL + n];
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

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is folded onto +0 so that equal scores give equal keys.
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Exclusive prefix sum over a workgroup of NT threads (one barrier); `total`
// gets the sum.  s_wave must not be written again before the next barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const uint32_t t = s_wave[i];
        before += i < wave ? t : 0u;
        all += t;
    }
    *total = all;
    return before + x - v;
}

// Build-time tuning: threads of the top-K workgroup.
#ifndef ABS_TOPK_NT
#define ABS_TOPK_NT 512
#endif

constexpr int kBins = 2048;
constexpr int kCandCap = 512;

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void k_topk(Geom g, const float* __restrict__ scores, int stride, int max_len,
                                             int budget, int32_t* __restrict__ sel, int sel_cap,
                                             int32_t* __restrict__ count) {
    const int bh = blockIdx.x;
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int bs = block_size_of(g, h);

    // Thread t owns indices [t*KPT, t*KPT + nv).  Its scores are loaded before
    // the row length is known (that takes a read of seq_lens), so the two
    // reads overlap.  The loads are unconditional, their offsets clamped to
    // the head's longest row, rounded up to a multiple of 4 (cap: at least N,
    // at most the stride): a clamped slot is at or beyond N and never used.
    const int base = threadIdx.x * KPT;
    const float* row = scores + (int64_t)bh * stride;
    const int cap = min(stride, (ceil_div(max_len, bs) + 3) & ~3);
    float f[KPT];
    if constexpr (KPT % 4 == 0) {
#pragma unroll
        for (int e = 0; e < KPT; e += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + min(base + e, cap - 4));
            f[e] = v.x;
            f[e + 1] = v.y;
            f[e + 2] = v.z;
            f[e + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < KPT; ++e) f[e] = row[min(base + e, cap - 1)];
    }

    const int N = ceil_div(g.seq_lens[b], bs);
    const int K = min(N, max(1, budget / bs));
    int32_t* out = sel + (int64_t)bh * sel_cap;
    if (threadIdx.x == 0) count[bh] = K;
    if (K >= N) {
        for (int j = threadIdx.x; j < N; j += NT) out[j] = j;
        return;
    }
    // most threads are full (nv = KPT) and run the unguarded forms of the
    // loops below
    const int nv = min(max(N - base, 0), KPT);
    const bool full = nv == KPT;
    float mn = __builtin_inff(), mx = -__builtin_inff();
    if (full) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            mn = fminf(mn, f[e]);
            mx = fmaxf(mx, f[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            if (e < nv) {
                mn = fminf(mn, f[e]);
                mx = fmaxf(mx, f[e]);
            }
        }
    }

    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t s_wave[3][NT / 64];          // one per scan: no barrier between reuses
    __shared__ float s_wmax[NT / 64], s_wmin[NT / 64];
    __shared__ float s_cand_val[kCandCap];
    __shared__ int32_t s_cand_idx[kCandCap];
    __shared__ uint32_t s_bin, s_above, s_ncand, s_tau_key;
    __shared__ int32_t s_tau_idx;

    for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0u;
    if (threadIdx.x == 0) s_ncand = 0u;
    // min and max of the row: wavefront shuffles, then one barrier
    mx = wave_max(mx);
    mn = -wave_max(-mn);
    if ((threadIdx.x & 63) == 0) {
        s_wmax[threadIdx.x >> 6] = mx;
        s_wmin[threadIdx.x >> 6] = mn;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        mx = fmaxf(mx, s_wmax[i]);
        mn = fminf(mn, s_wmin[i]);
    }
    const float range = mx - mn;
    const float inv = (float)kBins / range;
    const bool binned = range > 0.0f && range <= 3.0e38f && inv > 0.0f && inv <= 3.0e38f;

    // The threshold: the K-th element in (score desc, index asc) order, as
    // (tau score, tau index).  Scores compare as floats (-0 == +0).
    float tau_f = 0.0f;
    int32_t tau_idx = -1;
    bool resolved = false;
    if (binned) {
        // bin of a score: monotone non-decreasing in the score; -1 marks an empty slot
        int bin[KPT];
        if (full) {
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                bin[e] = min(kBins - 1, (int)((f[e] - mn) * inv));
                atomicAdd(&hist[bin[e]], 1u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                bin[e] = e < nv ? min(kBins - 1, (int)((f[e] - mn) * inv)) : -1;
                if (e < nv) atomicAdd(&hist[bin[e]], 1u);
            }
        }
        __syncthreads();
        // thread t sums bins kBins-1-t*BPT ... downwards; scan from the top
        constexpr int BPT = kBins / NT;
        uint32_t c[BPT], mine = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            c[i] = hist[kBins - 1 - threadIdx.x * BPT - i];
            mine += c[i];
        }
        uint32_t total;
        const uint32_t excl = block_exclusive_scan<NT>(mine, s_wave[0], &total);
        if (excl < (uint32_t)K && (uint32_t)K <= excl + mine) {     // exactly one thread
            uint32_t above = excl;
#pragma unroll
            for (int i = 0; i < BPT; ++i) {
                if (above + c[i] >= (uint32_t)K) {
                    s_bin = kBins - 1 - threadIdx.x * BPT - i;
                    s_above = above;
                    break;
                }
                above += c[i];
            }
        }
        __syncthreads();
        const int bstar = (int)s_bin;
        const uint32_t need = (uint32_t)K - s_above;                 // 1 <= need <= |bin b*|
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            if (bin[e] == bstar) {
                const uint32_t slot = atomicAdd(&s_ncand, 1u);
                if (slot < (uint32_t)kCandCap) {
                    s_cand_val[slot] = f[e];
                    s_cand_idx[slot] = base + e;
                }
            }
        }
        __syncthreads();
        const uint32_t nc = s_ncand;
        if (nc <= (uint32_t)kCandCap) {
            for (uint32_t t = threadIdx.x; t < nc; t += NT) {
                const float vt = s_cand_val[t];
                const int32_t it = s_cand_idx[t];
                uint32_t rank = 0;
                for (uint32_t u = 0; u < nc; ++u) {
                    const float vu = s_cand_val[u];
                    rank += (vu > vt || (vu == vt && s_cand_idx[u] < it)) ? 1u : 0u;
                }
                if (rank == need - 1) {
                    s_tau_key = __float_as_uint(vt);
                    s_tau_idx = it;
                }
            }
            __syncthreads();
            tau_f = __uint_as_float(s_tau_key);
            tau_idx = s_tau_idx;
            resolved = true;
        }
    }
    if (!resolved) {
        // crowded threshold bin or degenerate range: 8-bit radix select on the
        // order-preserving keys
        uint32_t prefix = 0, mask = 0, need = (uint32_t)K;
        for (int shift = 24; shift >= 0; shift -= 8) {
            __syncthreads();
            for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const uint32_t k = float_key(f[e]);
                if (e < nv && (k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (threadIdx.x < 64) {
                const int lane = threadIdx.x;   // lane l holds digits 255-4l .. 252-4l
                uint32_t c[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) c[i] = hist[255 - 4 * lane - i];
                const uint32_t mine = c[0] + c[1] + c[2] + c[3];
                const uint32_t incl = wave_inclusive_scan(mine);
                const uint32_t excl = incl - mine;
                if (excl < need && need <= incl) {
                    uint32_t above = excl;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (above + c[i] >= need) {
                            s_bin = 255u - 4u * lane - i;
                            s_above = need - above;
                            break;
                        }
                        above += c[i];
                    }
                }
            }
            __syncthreads();
            prefix |= s_bin << shift;
            mask |= 255u << shift;
            need = s_above;
        }
        // the need-th lowest index among keys equal to the threshold key
        uint32_t n_eq = 0;
#pragma unroll
        for (int e = 0; e < KPT; ++e) n_eq += (e < nv && float_key(f[e]) == prefix) ? 1u : 0u;
        uint32_t total;
        uint32_t r = block_exclusive_scan<NT>(n_eq, s_wave[1], &total);
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            if (e < nv && float_key(f[e]) == prefix) {
                if (r == need - 1) s_tau_idx = base + e;
                ++r;
            }
        }
        __syncthreads();
        tau_f = key_float(prefix);
        tau_idx = s_tau_idx;
    }

    // keep (score > tau) or (score == tau and index <= tau index): exactly K
    using Mask = std::conditional_t<(KPT > 32), uint64_t, uint32_t>;
    Mask keep = 0;
    const int tau_rel = tau_idx - base;                 // the tie cut in this thread's indices
    if (full) {
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            keep |= (f[e] > tau_f || (f[e] == tau_f && e <= tau_rel)) ? (Mask)1 << e : (Mask)0;
    } else {
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            keep |= (e < nv && (f[e] > tau_f || (f[e] == tau_f && e <= tau_rel))) ? (Mask)1 << e : (Mask)0;
    }
    uint32_t total;
    const uint32_t pos = block_exclusive_scan<NT>((uint32_t)__builtin_popcountll((uint64_t)keep), s_wave[2], &total);
    if (keep != 0) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const uint32_t p = pos + (uint32_t)__builtin_popcountll((uint64_t)(keep & (((Mask)1 << e) - 1)));
            if (((keep >> e) & 1) && p < (uint32_t)K) out[p] = base + e;
        }
    }
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
hipError_t select_impl(const Geom& g, const SelectArgs& a, hipStream_t s) {
    const int bits = fmt_bits(a.fmt);
    if (bits == 8) launch_score<T, D, 8>(g, a, s);
    else if (bits == 16) launch_score<T, D, 16>(g, a, s);
    else launch_score<T, D, 4>(g, a, s);
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
    if (dt == DType::BF16) return g.D == 128 ? select_impl<uint16_t, 128>(g, a, s) : select_impl<uint16_t, 64>(g, a, s);
    return g.D == 128 ? select_impl<float, 128>(g, a, s) : select_impl<float, 64>(g, a, s);
}

}  // namespace absk
