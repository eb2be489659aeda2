// Top-K selection of one head's blocks by one workgroup (AB-Sparse page,
// Figure 1: keep the blocks of highest estimated importance; the mapping
// figure after Figure 8: K per head set by its block size).  Shared by the
// select launch (one workgroup per (b, h)) and the fused select + decode
// launch (each split workgroup of a head selects for itself).
//
// Thread t owns block indices [t*KPT, (t+1)*KPT) as order-preserving 32-bit
// keys in registers.
//   1. min/max of the scores; a 2048-bin histogram of the scores' position
//      in [min, max] (a monotone binning, spread over the bins, so LDS
//      atomics rarely collide);
//   2. the bin b* holding the K-th largest score, and how many scores lie in
//      higher bins;
//   3. the few candidates in b* are ranked exactly by (score desc, index
//      asc), by one wavefront when there are at most 64 of them, giving the
//      threshold pair (tau_key, tau_index); if b* is crowded
//      (heavy ties) an 8-bit radix select over the keys gives the same pair
//      instead;
//   4. keep key > tau_key, or key == tau_key and index <= tau_index; a block
//      scan gives the kept indices' positions in ascending order.
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

// The top-K of (b, h) = bh by a workgroup of NT threads, each holding KPT
// keys: returns K and calls emit(p, j) for the kept block indices j, p their
// position in ascending order (0 <= p < K; each p once, from some thread).
// `row` is the head's score row, `stride` its allocated length (at least N),
// `max_len` the longest L_b of the layer.  Every thread of the workgroup must
// call it (it has barriers).
template <int NT, int KPT, class Emit>
__device__ __forceinline__ int topk_rows(const Geom& g, int bh, const float* __restrict__ row, int stride,
                                         int max_len, int budget, Emit&& emit) {
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int bs = block_size_of(g, h);

    // Thread t owns indices [t*KPT, t*KPT + nv).  Its scores are loaded before
    // the row length is known (that takes a read of seq_lens), so the two
    // reads overlap.  The loads are unconditional, their offsets clamped to
    // the head's longest row, rounded up to a multiple of 4 (cap: at least N,
    // at most the stride): a clamped slot is at or beyond N and never used.
    const int base = threadIdx.x * KPT;
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

    const int N = ceil_div(seq_len(g, b), bs);
    const int K = min(N, max(1, budget / bs));
    if (K >= N) {
        for (int j = threadIdx.x; j < N; j += NT) emit((uint32_t)j, (int32_t)j);
        return K;
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
        const uint32_t nc = __builtin_amdgcn_readfirstlane(s_ncand);
        if (nc <= 64u) {
            // the usual case, a few candidates: lane t of wavefront 0 holds
            // candidate t and counts the ones ranked before it, reading them
            // from the other lanes (readlane) rather than from LDS
            if (threadIdx.x < 64) {
                const uint32_t t = threadIdx.x;
                const float vt = s_cand_val[min(t, nc - 1)];         // nc >= need >= 1
                const int32_t it = s_cand_idx[min(t, nc - 1)];
                uint32_t rank = 0;
                for (uint32_t u = 0; u < nc; ++u) {
                    const float vu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vt), (int)u));
                    const int32_t iu = __builtin_amdgcn_readlane(it, (int)u);
                    rank += (vu > vt || (vu == vt && iu < it)) ? 1u : 0u;
                }
                if (t < nc && rank == need - 1) {
                    s_tau_key = __float_as_uint(vt);
                    s_tau_idx = it;
                }
            }
            __syncthreads();
            tau_f = __uint_as_float(s_tau_key);
            tau_idx = s_tau_idx;
            resolved = true;
        } else if (nc <= (uint32_t)kCandCap) {
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
            if (((keep >> e) & 1) && p < (uint32_t)K) emit(p, (int32_t)(base + e));
        }
    }
    return K;
}

}  // namespace absk
