// Top-K selection of one head's blocks by one workgroup (AB-Sparse page,
// Figure 1: keep the blocks of highest estimated importance; the mapping
// figure after Figure 8: K per head set by its block size).  Shared by the
// select launch (one workgroup per (b, h)) and the fused select + decode
// launch (each split workgroup of a head selects for itself).
//
// Thread t owns block indices [t*KPT, (t+1)*KPT) as fp32 scores in registers;
// the steps are listed at topk_rows.
#pragma once

#include <type_traits>

#include "device.hpp"

namespace absk {

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

constexpr int kBins = 2048;
constexpr int kCandCap = 512;
constexpr int kMaxRangeLoads = (kMaxBlocksPerHead / kScoreBlocksPerWg + 63) / 64;   // tile ranges per lane

// Keys of thread t as a bit mask: bit e stands for block t*KPT + e.
template <int KPT>
using KeyMask = std::conditional_t<(KPT > 32), uint64_t, uint32_t>;

// Exact (score desc, index asc) rank of the threshold bin's candidates by
// one wavefront, every wavefront for itself: lane t takes candidate t (nc <=
// 64) and counts the candidates ranked before it, reading them from the
// other lanes; the lane of rank need - 1 holds the threshold pair, which a
// ballot and readlane hand to every lane.
__device__ __forceinline__ void rank_in_wave(const float* s_val, const int32_t* s_idx, uint32_t nc, uint32_t need,
                                             float* tau_f, int32_t* tau_idx) {
    const uint32_t t = threadIdx.x & 63;
    const float vt = s_val[min(t, nc - 1)];              // nc >= need >= 1
    const int32_t it = s_idx[min(t, nc - 1)];
    uint32_t rank = 0;
    for (uint32_t u = 0; u < nc; ++u) {
        const float vu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vt), (int)u));
        const int32_t iu = __builtin_amdgcn_readlane(it, (int)u);
        rank += ((vu > vt) | ((vu == vt) & (iu < it))) ? 1u : 0u;
    }
    const uint64_t hit = __ballot(t < nc && rank == need - 1);
    const int src = (int)__builtin_ctzll(hit);           // exactly one lane
    *tau_f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vt), src));
    *tau_idx = __builtin_amdgcn_readlane(it, src);
}

// The top-K of (b, h) = bh by a workgroup of NT threads, each holding KPT
// keys: returns K and calls emit(p, j) for the kept block indices j, p their
// position in ascending order (0 <= p < K; each p once, from some thread).
// `row` is the head's score row, `stride` its allocated length (at least N),
// `ranges` the (min, max) of each 256-block tile of the row that the score
// launch wrote, `max_len` the longest L_b of the layer.  Every thread of the
// workgroup must call it (it has barriers).
//
//   1. the row's range from the tile ranges (no pass over the keys); a
//      2048-bin histogram of the keys' position in it (a monotone binning);
//   2. the bin b* holding the K-th largest key, and how many keys lie above
//      it: a block scan, after which every wavefront finds b* itself;
//   3. the few keys in b* are ranked exactly by (score desc, index asc), by
//      every wavefront for itself when there are at most 64 of them, giving
//      the threshold pair (tau, tau index); a crowded b* (heavy ties) or a
//      degenerate range takes an 8-bit radix select over the keys instead;
//   4. keep the keys above b*, and those in b* ranked up to the threshold;
//      a block scan gives the kept indices' positions in ascending order.
// Every per-key step works on bit masks without data-dependent branches
// (padding keys take a slot below the scanned bins and count into spill
// slots past them), and the kept keys are emitted by a loop over the set
// bits of the keep mask, so the cost per thread grows with KPT by a few
// instructions per key.
template <int NT, int KPT, class Emit>
__device__ __forceinline__ int topk_rows(const Geom& g, int bh, const float* __restrict__ row, int stride,
                                         const float2* __restrict__ ranges, int max_len, int budget, Emit&& emit,
                                         int& L) {
    using Mask = KeyMask<KPT>;
    constexpr int NW = NT / 64;
    int b, h;
    split_bh(g, bh, b, h);
    const int sb = block_shift_of(g, h);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int len_issued = seq_len_issue(g, b);       // first: its wait does not take the loads below

    // Thread t owns indices [t*KPT, t*KPT + nv).  Its scores and the tile
    // ranges are loaded before the row length is known (that takes a read of
    // seq_lens, issued first), so the reads overlap.  The loads are unconditional, their
    // offsets clamped to the head's longest row (keys: rounded up to a
    // multiple of 4, at least N, at most the stride): a clamped slot is at or
    // beyond N and never used.
    const int base = threadIdx.x * KPT;
    const int n_max = shr_ceil(max_len, sb);
    const int cap = min(stride, (n_max + 3) & ~3);
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
    const int tiles_max = shr_ceil(n_max, 8);                  // 256-block tiles
    constexpr int RL = (KPT * NT + kScoreBlocksPerWg * 64 - 1) / (kScoreBlocksPerWg * 64);   // range loads per lane
    static_assert(RL <= kMaxRangeLoads, "tile ranges per lane");
    float2 rr[RL];
#pragma unroll
    for (int k = 0; k < RL; ++k) rr[k] = ranges[min(lane + 64 * k, tiles_max - 1)];


    __shared__ uint32_t hist[kBins + 1 + 64];         // bin i -> slot i + 1; then one padding spill slot per lane
    __shared__ uint32_t s_wave[3][NW];                // one per scan: no barrier between reuses
    __shared__ float s_cand_val[kCandCap];
    __shared__ int32_t s_cand_idx[kCandCap];
    __shared__ uint32_t s_bin, s_above, s_ncand;
    __shared__ float s_tau_f;
    __shared__ int32_t s_tau_idx;
    for (int i = threadIdx.x; i <= kBins + 64; i += NT) hist[i] = 0u;
    if (threadIdx.x == 0) s_ncand = 0u;
    __syncthreads();                                  // (the loads above are still in flight)

    L = seq_len_use(g, len_issued);
    const int N = shr_ceil(L, sb);
    const int K = min(N, max(1, budget >> sb));
    if (K >= N) {
        for (int j = threadIdx.x; j < N; j += NT) emit((uint32_t)j, (int32_t)j);
        return K;
    }
    // padding keys (e >= nv: the tail of one thread, and every key of the
    // threads past the row) become -inf: below every score (finite), so no
    // later comparison needs to test e < nv
    const int nv = min(max(N - base, 0), KPT);
    if (nv < KPT) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) f[e] = e < nv ? f[e] : -__builtin_inff();
    }
    // the row's range: min and max over its tiles' ranges (every wavefront)
    const int nt = shr_ceil(N, 8);
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < RL; ++k) {
        const bool ok = lane + 64 * k < nt;
        mn = fminf(mn, ok ? rr[k].x : __builtin_inff());
        mx = fmaxf(mx, ok ? rr[k].y : -__builtin_inff());
    }
    mx = wave_max(mx);
    mn = -wave_max(-mn);
    const float range = mx - mn;
    const float inv = (float)kBins / range;
    const bool binned = range > 0.0f && range <= 3.0e38f && inv > 0.0f && inv <= 3.0e38f;

    // The threshold: the K-th element in (score desc, index asc) order, as
    // (tau score, tau index).  Scores compare as floats (-0 == +0).
    float tau_f = 0.0f;
    int32_t tau_idx = -1;
    Mask keep = 0;
    bool resolved = false;
    if (binned) {
        // slot of a key: clamp(f inv + 1 - mn inv, 1, kBins) truncated, one
        // fma then a truncation, monotone non-decreasing in the score (the
        // bin offset 1 folded into the constant).  A wavefront with padding
        // keys gives them slot 0, below every bin, and counts them into each
        // lane's own spill slot past the bins (one LDS address taking the
        // atomics of whole wavefronts of padding would serialize them, 64
        // cycles per instruction); the others skip those selects.
        const float c1 = 1.0f - mn * inv;
        int slot[KPT];
        if (__builtin_amdgcn_ballot_w64(nv < KPT) == 0) {       // every key of this wavefront is valid
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                slot[e] = (int)fminf(fmaxf(fmaf(f[e], inv, c1), 1.0f), (float)kBins);
                atomicAdd(&hist[slot[e]], 1u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                slot[e] = e < nv ? (int)fminf(fmaxf(fmaf(f[e], inv, c1), 1.0f), (float)kBins) : 0;
                atomicAdd(&hist[e < nv ? slot[e] : kBins + 1 + lane], 1u);
            }
        }
        __syncthreads();
        // thread t sums the bins of slots kBins - t*BPT ... downwards; scan from the top
        constexpr int BPT = kBins / NT;
        uint32_t mine = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) mine += hist[kBins - threadIdx.x * BPT - i];
        const uint32_t x = wave_inclusive_scan(mine);
        if (lane == 63) s_wave[0][wave] = x;
        __syncthreads();
        // every wavefront finds the thread whose bins hold the K-th key (wc,
        // lane lc), then redoes that wavefront's scan of its bins to find the
        // slot b* and the count above it
        uint32_t before = 0;
        int wc = NW - 1;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t tw = s_wave[0][w];
            if (w < wc && before + tw >= (uint32_t)K) wc = w;
            before += w < wc ? tw : 0u;
        }
        uint32_t cw[BPT], mw = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            cw[i] = hist[kBins - (wc * 64 + lane) * BPT - i];
            mw += cw[i];
        }
        const uint32_t xw = wave_inclusive_scan(mw) + before;
        const uint64_t past = __ballot(xw >= (uint32_t)K);
        const int lc = (int)__builtin_ctzll(past);                    // first lane reaching K
        uint32_t above = xw - mw;                                     // keys above this lane's bins
        int bstar = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const bool here = bstar == 0 && above + cw[i] >= (uint32_t)K;
            bstar = here ? kBins - (wc * 64 + lane) * BPT - i : bstar;
            above += bstar == 0 ? cw[i] : 0u;
        }
        bstar = __builtin_amdgcn_readlane(bstar, lc);
        above = __builtin_amdgcn_readlane(above, lc);
        const uint32_t need = (uint32_t)K - above;                    // 1 <= need <= |bin b*|
        // this thread's keys above b* and in b*; those in b* go to the candidate list
        Mask in_bin = 0;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            keep |= slot[e] > bstar ? (Mask)1 << e : (Mask)0;
            in_bin |= slot[e] == bstar ? (Mask)1 << e : (Mask)0;
        }
        uint32_t c_slot = 0;
        if (in_bin != 0) {
            c_slot = atomicAdd(&s_ncand, (uint32_t)__builtin_popcountll((uint64_t)in_bin));
            uint32_t at = c_slot;
            for (Mask m = in_bin; m != 0; m &= m - 1, ++at) {
                const int e = __builtin_ctzll((uint64_t)m);
                if (at < (uint32_t)kCandCap) {
                    s_cand_val[at] = f[e];
                    s_cand_idx[at] = base + e;
                }
            }
        }
        __syncthreads();
        const uint32_t nc = __builtin_amdgcn_readfirstlane(s_ncand);
        if (nc <= 64u) {
            rank_in_wave(s_cand_val, s_cand_idx, nc, need, &tau_f, &tau_idx);   // no barrier needed
            resolved = true;
        } else if (nc <= (uint32_t)kCandCap) {
            for (uint32_t t = threadIdx.x; t < nc; t += NT) {
                const float vt = s_cand_val[t];
                const int32_t it = s_cand_idx[t];
                uint32_t rank = 0;
                for (uint32_t u = 0; u < nc; ++u) {
                    const float vu = s_cand_val[u];
                    rank += ((vu > vt) | ((vu == vt) & (s_cand_idx[u] < it))) ? 1u : 0u;
                }
                if (rank == need - 1) {
                    s_tau_f = vt;
                    s_tau_idx = it;
                }
            }
            __syncthreads();
            tau_f = s_tau_f;
            tau_idx = s_tau_idx;
            resolved = true;
        }
        if (resolved) {
            // this thread's keys in b*: kept when ranked up to the threshold
            for (Mask m = in_bin; m != 0; m &= m - 1) {
                const int e = __builtin_ctzll((uint64_t)m);
                const bool kept = (f[e] > tau_f) | ((f[e] == tau_f) & (base + e <= tau_idx));
                keep |= kept ? (Mask)1 << e : (Mask)0;
            }
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
                uint32_t c[4];                  // lane l holds digits 255-4l .. 252-4l
#pragma unroll
                for (int i = 0; i < 4; ++i) c[i] = hist[255 - 4 * lane - i];
                const uint32_t m4 = c[0] + c[1] + c[2] + c[3];
                const uint32_t incl = wave_inclusive_scan(m4);
                const uint32_t excl = incl - m4;
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
        // keep (score > tau) or (score == tau and index <= tau index); padding keys are -inf
        const int tau_rel = tau_idx - base;
        keep = 0;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const bool kept = (f[e] > tau_f) | ((f[e] == tau_f) & (e <= tau_rel));
            keep |= kept ? (Mask)1 << e : (Mask)0;
        }
    }

    // exactly K keys kept; their positions in ascending index order
    uint32_t total;
    uint32_t p = block_exclusive_scan<NT>((uint32_t)__builtin_popcountll((uint64_t)keep), s_wave[2], &total);
    for (Mask m = keep; m != 0; m &= m - 1, ++p) {
        const int e = __builtin_ctzll((uint64_t)m);
        if (p < (uint32_t)K) emit(p, (int32_t)(base + e));
    }
    return K;
}

}  // namespace absk
