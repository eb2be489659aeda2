// Dot-product estimation and top-K selection (AB-Sparse page, Figure 1:
// importance score = query . block representation, then Top-K; the mapping
// figure after Figure 8: each head keeps K blocks, K set by its block size
// so every head reads the same number of pages).
//
// score:  one workgroup per (tile of blocks, b*Hkv + h).  The group query
//         qbar = sum of the G query heads of KV head h is folded with the
//         per-channel dequantization once per workgroup:
//             w_d = qbar_d * scale_d,   c0 = sum_d qbar_d * lo_d,
//             score_j = c0 + sum_d w_d * code_{j,d}
//         (fp64 inside, stored as fp32).  head_dim/32 lanes share one block
//         row of INT4 codes, 16 bytes each, so one load instruction reads a
//         contiguous 1 KiB run.
// top-K:  one 1024-thread workgroup per (b, h).  Thread t owns the block
//         indices [t*KPT, (t+1)*KPT) as order-preserving 32-bit keys in
//         registers.  An 8-bit radix select (4 passes over an LDS histogram)
//         finds the K-th largest key tau and how many keys equal to tau to
//         keep; two block-wide scans then write the kept indices in ascending
//         order (keys > tau, plus the lowest-index keys == tau).
#include "device.hpp"

namespace absk {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void k_score(Geom g, const uint8_t* __restrict__ codes,
                                               const float* __restrict__ scale, const float* __restrict__ lo,
                                               const T* __restrict__ q, float* __restrict__ scores) {
    constexpr int LPB = D / 32;               // lanes per block row (16 B of codes each)
    constexpr int BPW = 256 / LPB;            // blocks per workgroup
    const int bh = blockIdx.y;
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int N = ceil_div(g.seq_lens[b], g.block_size[h]);
    const int j0 = blockIdx.x * BPW;
    if (j0 >= N) return;
    const int64_t row0 = g.off[bh];

    __shared__ double w[D];
    __shared__ double c0_part[D / 64 > 0 ? D / 64 : 1];
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        double qbar = 0.0;
        for (int gg = 0; gg < g.G; ++gg)
            qbar += (double)Elem<T>::load1(q + ((int64_t)b * g.Hq + h * g.G + gg) * D + d);
        w[d] = qbar * (double)scale[(int64_t)bh * D + d];
        double part = qbar * (double)lo[(int64_t)bh * D + d];
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
        if ((d & 63) == 0) c0_part[d / 64] = part;
    }
    __syncthreads();
    double c0 = 0.0;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) c0 += c0_part[i];

    const int sub = threadIdx.x % LPB;
    const int j = j0 + threadIdx.x / LPB;
    double acc = 0.0;
    if (j < N) {
        const uint4 v = *reinterpret_cast<const uint4*>(codes + (row0 + j) * (D / 2) + sub * 16);
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
        const double* ws = w + sub * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int n = 0; n < 8; ++n) acc += ws[i * 8 + n] * (double)((wd[i] >> (4 * n)) & 15u);
    }
#pragma unroll
    for (int off = 1; off < LPB; off <<= 1) acc += __shfl_xor(acc, off);
    if (j < N && sub == 0) scores[row0 + j] = (float)(c0 + acc);
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is folded onto +0 so that equal scores give equal keys.
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup (blockDim.x == kTopkThreads).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kTopkThreads / 64; ++i) {
        const uint32_t t = s_wave[i];
        before += i < wave ? t : 0u;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void k_topk(Geom g, const float* __restrict__ scores, int budget,
                                                       int32_t* __restrict__ sel, int sel_cap,
                                                       int32_t* __restrict__ count) {
    const int bh = blockIdx.x;
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int bs = g.block_size[h];
    const int N = ceil_div(g.seq_lens[b], bs);
    const int K = min(N, max(1, budget / bs));
    const int64_t row0 = g.off[bh];
    int32_t* out = sel + (int64_t)bh * sel_cap;
    if (threadIdx.x == 0) count[bh] = K;
    if (K >= N) {
        for (int j = threadIdx.x; j < N; j += blockDim.x) out[j] = j;
        return;
    }

    const int base = threadIdx.x * KPT;
    uint32_t key[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) key[e] = base + e < N ? float_key(scores[row0 + base + e]) : 0u;

    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_digit, s_need;
    __shared__ uint32_t s_wave[kTopkThreads / 64];
    uint32_t prefix = 0, mask = 0, need = (uint32_t)K;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            if (base + e < N && (key[e] & mask) == prefix) atomicAdd(&hist[(key[e] >> shift) & 255u], 1u);
        __syncthreads();
        if (threadIdx.x < 64) {
            // lane l holds bins 255-4l .. 252-4l (descending digit order)
            const int lane = threadIdx.x;
            uint32_t c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) c[i] = hist[255 - 4 * lane - i];
            const uint32_t mine = c[0] + c[1] + c[2] + c[3];
            uint32_t incl = mine;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_up(incl, off);
                if (lane >= off) incl += y;
            }
            const uint32_t excl = incl - mine;       // keys in bins above this lane's
            if (excl < need && need <= incl) {        // exactly one lane
                uint32_t above = excl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (above + c[i] >= need) {
                        s_digit = 255u - 4u * lane - i;
                        s_need = need - above;
                        break;
                    }
                    above += c[i];
                }
            }
        }
        __syncthreads();
        prefix |= s_digit << shift;
        mask |= 255u << shift;
        need = s_need;
    }
    const uint32_t tau = prefix;

    // keys > tau are kept; of the keys == tau, the `need` lowest indices.
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) n_eq += (base + e < N && key[e] == tau) ? 1u : 0u;
    uint32_t total;
    const uint32_t eq_base = block_exclusive_scan(n_eq, s_wave, &total);
    uint32_t r = eq_base, n_keep = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        if (base + e < N) {
            if (key[e] > tau) ++n_keep;
            else if (key[e] == tau && r++ < need) ++n_keep;
        }
    }
    uint32_t pos = block_exclusive_scan(n_keep, s_wave, &total);
    r = eq_base;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        if (base + e < N) {
            bool keep = key[e] > tau;
            if (key[e] == tau) keep = r++ < need;
            if (keep && pos < (uint32_t)K) out[pos++] = base + e;
        }
    }
}

template <typename T, int D>
hipError_t select_impl(const Geom& g, const SelectArgs& a, hipStream_t s) {
    constexpr int BPW = 256 / (D / 32);
    const dim3 sgrid(ceil_div(a.max_n, BPW), g.B * g.Hkv);
    hipLaunchKernelGGL((k_score<T, D>), sgrid, dim3(256), 0, s, g, a.codes, a.scale, a.lo,
                       reinterpret_cast<const T*>(a.q), a.scores);
    const dim3 tgrid(g.B * g.Hkv);
    const int kpt = ceil_div(a.max_n, kTopkThreads);
#define ABS_TOPK(KPT_)                                                                                     \
    hipLaunchKernelGGL((k_topk<KPT_>), tgrid, dim3(kTopkThreads), 0, s, g, a.scores, a.budget, a.sel, \
                       a.sel_cap, a.count)
    if (kpt <= 1) ABS_TOPK(1);
    else if (kpt <= 2) ABS_TOPK(2);
    else if (kpt <= 4) ABS_TOPK(4);
    else if (kpt <= 8) ABS_TOPK(8);
    else if (kpt <= 16) ABS_TOPK(16);
    else if (kpt <= 32) ABS_TOPK(32);
    else ABS_TOPK(64);
#undef ABS_TOPK
    return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const Geom& g, DType dt, const SelectArgs& a, hipStream_t s) {
    if (dt == DType::BF16) return g.D == 128 ? select_impl<uint16_t, 128>(g, a, s) : select_impl<uint16_t, 64>(g, a, s);
    return g.D == 128 ? select_impl<float, 128>(g, a, s) : select_impl<float, 64>(g, a, s);
}

}  // namespace absk
