// Centroid build and INT4 asymmetric per-channel quantization (AB-Sparse page:
// Figure 1's block representation; Figure 8's INT4 asymmetric per-channel
// centroids; the mapping figure after Figure 8 for pages -> blocks).
//
// Three launches per layer (staging rows are (b*Hkv + h) * max N + j, so
// they do not depend on the caller's centroid offsets):
//   mean:     one workgroup per (tile of 1024 tokens, b*Hkv + h), i.e. 64,
//             32 or 16 blocks.  16 lanes own a cache row (16 x head_dim/16
//             channels); 16 row-groups work on 16 blocks at a time,
//             streaming each page's 16 rows with 16 independent wide
//             non-temporal loads.  Sums are fp64 in token order, as the
//             oracle's (exact unless a block's keys in one channel span
//             more than about 39 binades for bf16, 23 for fp32), so the fp32
//             centroid is the correctly rounded mean.  Per-channel min/max
//             of the tile is reduced with shuffles + LDS.
//   range:    per (b, h, channel): min/max over tiles -> lo, scale (fp32).
//   quantize: code = clamp(rint((c - lo) / scale), 0, 15), two per byte.
// The other storage formats (Figure 8's precision comparison) change only
// range and quantize: INT4 symmetric (scale = max|c| / 7, q = clamp(rint(c /
// scale), -7, 7) stored as q + 8, lo reported as -8 * scale), INT8 (255
// levels, one byte per channel), INT4 with one range per (sequence, head)
// (min/max over every block and channel), and bf16 (the fp32 mean rounded to
// nearest even; scale and lo are 0).
#include "device.hpp"

namespace absk {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void k_centroid_mean(Geom g, float* __restrict__ staging,
                                                        float* __restrict__ pmin, float* __restrict__ pmax,
                                                        int tiles, int stage_rows) {
    constexpr int VEC = D / kRowLanes;                    // channels per lane
    constexpr int NW = VEC * Elem<T>::kBytes / 4;         // 32-bit words per lane per row
    constexpr int GROUPS = 256 / kRowLanes;               // 16 blocks in flight
    const int bh = blockIdx.y;
    int b, h;
    split_bh(g, bh, b, h);
    const int L = seq_len(g, b);
    const int sb = block_shift_of(g, h);
    const int bs = 1 << sb;
    const int N = shr_ceil(L, sb);
    const int bpt = kBuildTileTokens >> sb;               // blocks per tile
    const int j0 = blockIdx.x * bpt;
    if (j0 >= N) return;                                  // uniform: whole workgroup leaves
    const int lane = threadIdx.x & (kRowLanes - 1);
    const int grp = threadIdx.x / kRowLanes;
    const T* kbase = reinterpret_cast<const T*>(g.k);

    float mn[VEC], mx[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        mn[e] = __builtin_inff();
        mx[e] = -__builtin_inff();
    }

    for (int jj = grp; jj < bpt; jj += GROUPS) {
        const int j = j0 + jj;
        if (j >= N) break;
        const int t0 = j * bs;
        const int t1 = min(t0 + bs, L);
        double acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
        for (int t = t0; t < t1; t += kPage) {
            const int page = g.page_table[(int64_t)b * g.max_pages + t / kPage];
            if (page < 0 || page >= g.num_pages) continue;
            const T* src = kbase + ((int64_t)page * g.Hkv + h) * kPage * D + lane * VEC;
            const int rows = min(kPage, t1 - t);
            Words<NW> w[kPage];
#pragma unroll
            for (int r = 0; r < kPage; ++r) w[r] = r < rows ? load_words_stream<NW>(src + r * D) : zero_words<NW>();
#pragma unroll
            for (int r = 0; r < kPage; ++r)
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] += (double)Elem<T>::get(w[r], e);
        }
        const double n = (double)(t1 - t0);
        float c[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            c[e] = (float)(acc[e] / n);
            mn[e] = fminf(mn[e], c[e]);
            mx[e] = fmaxf(mx[e], c[e]);
        }
        float* dst = staging + ((int64_t)bh * stage_rows + j) * D + lane * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
            *reinterpret_cast<float4*>(dst + e) = make_float4(c[e], c[e + 1], c[e + 2], c[e + 3]);
    }

    // min/max over the 16 row-groups: 4 per wavefront by shuffles, then LDS.
    __shared__ float smn[4][D], smx[4][D];
    const int wave = threadIdx.x / 64;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        mn[e] = rows4_min(mn[e]);
        mx[e] = rows4_max(mx[e]);
    }
    if ((threadIdx.x & 63) < kRowLanes) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            smn[wave][lane * VEC + e] = mn[e];
            smx[wave][lane * VEC + e] = mx[e];
        }
    }
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float a = fminf(fminf(smn[0][d], smn[1][d]), fminf(smn[2][d], smn[3][d]));
        float z = fmaxf(fmaxf(smx[0][d], smx[1][d]), fmaxf(smx[2][d], smx[3][d]));
        pmin[((int64_t)bh * tiles + blockIdx.x) * D + d] = a;
        pmax[((int64_t)bh * tiles + blockIdx.x) * D + d] = z;
    }
}

// One workgroup of kRangeThreads per (b, h): S = kRangeThreads / D stripes
// of tiles per channel, four tiles' loads in flight per thread, then LDS.
constexpr int kRangeThreads = 1024;

template <int D>
__global__ __launch_bounds__(kRangeThreads) void k_centroid_range(Geom g, const float* __restrict__ pmin,
                                                                  const float* __restrict__ pmax, int tiles, int fmt,
                                                                  float* __restrict__ scale, float* __restrict__ lo) {
    constexpr int S = kRangeThreads / D;
    const int bh = blockIdx.x;
    int b, h;
    split_bh(g, bh, b, h);
    const int sb = block_shift_of(g, h);
    const int nt = shr_ceil(shr_ceil(seq_len(g, b), sb), __builtin_ctz(kBuildTileTokens) - sb);
    const int d = threadIdx.x % D, stripe = threadIdx.x / D;
    const float* pn = pmin + (int64_t)bh * tiles * D + d;
    const float* px = pmax + (int64_t)bh * tiles * D + d;
    float a = __builtin_inff(), z = -__builtin_inff();
    int t = stripe;
    for (; t + 3 * S < nt; t += 4 * S) {
        float an[4], zx[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            an[k] = pn[(int64_t)(t + k * S) * D];
            zx[k] = px[(int64_t)(t + k * S) * D];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a = fminf(a, an[k]);
            z = fmaxf(z, zx[k]);
        }
    }
    for (; t < nt; t += S) {
        a = fminf(a, pn[(int64_t)t * D]);
        z = fmaxf(z, px[(int64_t)t * D]);
    }
    __shared__ float s_mn[S][D], s_mx[S][D];
    __shared__ float s_hmn[D / 64], s_hmx[D / 64];
    s_mn[stripe][d] = a;
    s_mx[stripe][d] = z;
    __syncthreads();
    // stripe 0 (the first D threads: whole wavefronts) finishes; every thread
    // still reaches each barrier
    const bool mine = stripe == 0;
    if (mine) {
#pragma unroll
        for (int k = 1; k < S; ++k) {
            a = fminf(a, s_mn[k][d]);
            z = fmaxf(z, s_mx[k][d]);
        }
    }
    if (fmt == kInt4Tensor) {   // one range for the whole head: min/max over the channels too
        if (mine) {
            for (int o = 32; o > 0; o >>= 1) {
                a = fminf(a, __shfl_xor(a, o));
                z = fmaxf(z, __shfl_xor(z, o));
            }
            if ((d & 63) == 0) {
                s_hmn[d / 64] = a;
                s_hmx[d / 64] = z;
            }
        }
        __syncthreads();
        if (mine) {
            a = s_hmn[0];
            z = s_hmx[0];
#pragma unroll
            for (int w = 1; w < D / 64; ++w) {
                a = fminf(a, s_hmn[w]);
                z = fmaxf(z, s_hmx[w]);
            }
        }
    }
    if (!mine) return;
    float s = 0.0f, zp = 0.0f;
    if (fmt == kInt4Sym) {
        const float amax = -a > z ? -a : z;   // max |c|
        s = amax / 7.0f;                      // IEEE fp32 division
        zp = -8.0f * s;
    } else if (fmt != kBf16) {
        const float range = z - a;            // fp32
        s = range / (fmt == kInt8 ? 255.0f : 15.0f);
        zp = a;
    }
    scale[(int64_t)bh * D + d] = s;
    lo[(int64_t)bh * D + d] = zp;
}

// Code of one fp32 centroid value under format FMT with the head's (s, z).
// `clamped` is set when the value lies outside what the code can express.
template <int FMT>
__device__ __forceinline__ uint32_t code_of(float c, float s, float z, bool* clamped) {
    if constexpr (FMT == kBf16) {
        const uint32_t u = __float_as_uint(c);
        const uint32_t hb = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;   // round to nearest even
        *clamped = ((hb & 0x7FFFu) == 0x7F80u) && ((u & 0x7FFFFFFFu) < 0x7F800000u);   // finite -> inf
        return hb;
    } else if constexpr (FMT == kInt4Sym) {
        float r = 0.0f;
        if (s > 0.0f) {
            const float quot = c / s;            // IEEE fp32 division
            r = rintf(quot);
            *clamped = r < -7.0f || r > 7.0f;
            r = fminf(fmaxf(r, -7.0f), 7.0f);
        } else {
            *clamped = c != 0.0f;
        }
        return (uint32_t)(r + 8.0f);
    } else {
        constexpr float top = FMT == kInt8 ? 255.0f : 15.0f;
        float r = 0.0f;
        if (s > 0.0f) {
            const float diff = c - z;
            const float quot = diff / s;         // IEEE fp32 division
            r = rintf(quot);
            *clamped = r < 0.0f || r > top;
            r = fminf(fmaxf(r, 0.0f), top);
        } else {
            *clamped = c != z;
        }
        return (uint32_t)r;
    }
}

// One thread per (block, 8 channels): reads 32 B of fp32 centroid, writes
// the 8 codes (4, 8 or 16 B).
template <int D, int FMT>
__global__ __launch_bounds__(256) void k_centroid_quantize(Geom g, const float* __restrict__ staging,
                                                           const float* __restrict__ scale,
                                                           const float* __restrict__ lo,
                                                           uint8_t* __restrict__ codes, int stage_rows) {
    constexpr int TPB = D / 8;                 // threads per block row
    constexpr int ROWS = 256 / TPB;            // block rows per pass
    constexpr int BITS = fmt_bits(FMT);
    constexpr int64_t RB = row_bytes(D, FMT);
    const int bh = blockIdx.y;
    int b, h;
    split_bh(g, bh, b, h);
    const int sb = block_shift_of(g, h);
    const int N = centroid_rows(g, bh, shr_ceil(seq_len(g, b), sb));
    const int bpt = kBuildTileTokens >> sb;
    const int j0 = blockIdx.x * bpt;
    if (j0 >= N) return;
    const int64_t row0 = g.off[bh];
    const int c8 = threadIdx.x % TPB;
    float s[8], z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s[e] = scale[(int64_t)bh * D + c8 * 8 + e];
        z[e] = lo[(int64_t)bh * D + c8 * 8 + e];
    }
    for (int jj = threadIdx.x / TPB; jj < bpt; jj += ROWS) {
        const int j = j0 + jj;
        if (j >= N) break;
        const float* src = staging + ((int64_t)bh * stage_rows + j) * D + c8 * 8;
        const float4 u0 = reinterpret_cast<const float4*>(src)[0];
        const float4 u1 = reinterpret_cast<const float4*>(src)[1];
        const float c[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        uint32_t code[8];
        bool unused;
#pragma unroll
        for (int e = 0; e < 8; ++e) code[e] = code_of<FMT>(c[e], s[e], z[e], &unused);
        uint8_t* dst = codes + (row0 + j) * RB + c8 * BITS;   // 8 channels = BITS bytes
        if constexpr (BITS == 4) {
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) packed |= code[e] << (4 * e);
            *reinterpret_cast<uint32_t*>(dst) = packed;
        } else if constexpr (BITS == 8) {
            *reinterpret_cast<uint2*>(dst) =
                make_uint2(code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24,
                           code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24);
        } else {
            *reinterpret_cast<uint4*>(dst) = make_uint4(code[0] | code[1] << 16, code[2] | code[3] << 16,
                                                        code[4] | code[5] << 16, code[6] | code[7] << 16);
        }
    }
}

template <typename T, int D>
hipError_t build_impl(const Geom& g, const BuildArgs& a, hipStream_t s) {
    const dim3 grid(a.tiles, g.B * g.Hkv);
    hipLaunchKernelGGL((k_centroid_mean<T, D>), grid, dim3(256), 0, s, g, a.staging, a.pmin, a.pmax, a.tiles,
                       a.stage_rows);
    hipLaunchKernelGGL((k_centroid_range<D>), dim3(g.B * g.Hkv), dim3(kRangeThreads), 0, s, g, a.pmin, a.pmax,
                       a.tiles, a.fmt, a.scale, a.lo);
#define ABS_QUANT(F_)                                                                                         \
    hipLaunchKernelGGL((k_centroid_quantize<D, F_>), grid, dim3(256), 0, s, g, a.staging, a.scale, a.lo, a.codes, \
                       a.stage_rows)
    switch (a.fmt) {
        case kInt4Sym: ABS_QUANT(kInt4Sym); break;
        case kInt8: ABS_QUANT(kInt8); break;
        case kBf16: ABS_QUANT(kBf16); break;
        default: ABS_QUANT(kInt4); break;   // kInt4 and kInt4Tensor: the same coding, per-channel (s, lo)
    }
#undef ABS_QUANT
    return hipGetLastError();
}

// Centroids kept current while decoding (the page fixes static per-head
// block sizes, Figure 5's text, and INT4 per-channel centroids, Figure 8;
// how they follow appended tokens is read as: recompute every block holding
// one of the tokens [L - appended - 1, L) -- always at least the last,
// possibly partial block -- and code it with the head's stored (scale, lo),
// clamped to the format's code range, counting the clamped codes).  One workgroup per (b, h).
// Each 16-lane row group loads one 16-token page of a recomputed block (all
// pages at once) and sums its rows in order in fp64; the page sums are then
// added in page order (exact, and so equal to the build's in-order sums,
// unless a block's keys in one channel span more than about 39 binades for
// bf16, 23 for fp32) and the mean is coded by one thread per channel.
template <typename T, int D, int FMT>
__global__ __launch_bounds__(256) void k_centroid_update(Geom g, int appended, const float* __restrict__ scale,
                                                         const float* __restrict__ lo, uint8_t* __restrict__ codes,
                                                         int32_t* __restrict__ out_of_range) {
    constexpr int VEC = D / kRowLanes;                    // channels per lane
    constexpr int NW = VEC * Elem<T>::kBytes / 4;
    constexpr int GROUPS = 256 / kRowLanes;               // pages in flight
    constexpr int BITS = fmt_bits(FMT);
    constexpr int64_t RB = row_bytes(D, FMT);
    const int bh = blockIdx.x;
    int b, h;
    split_bh(g, bh, b, h);
    const int L = seq_len(g, b);
    const int sb = block_shift_of(g, h);
    const int bs = 1 << sb;
    const int sp = sb - 4;                                // log2(pages per block)
    const int ppb = 1 << sp;                              // pages per block
    const int N = centroid_rows(g, bh, shr_ceil(L, sb));
    const int j_first = (max(1, L - appended) - 1) >> sb;
    const int64_t row0 = g.off[bh];
    const int lane = threadIdx.x & (kRowLanes - 1);
    const int grp = threadIdx.x / kRowLanes;
    const T* kbase = reinterpret_cast<const T*>(g.k);
    __shared__ double s_part[GROUPS][D];                  // per page: sum of its valid rows
    __shared__ int s_clamped;
    if (threadIdx.x == 0) s_clamped = 0;
    int clamped = 0;
    // (block, page) items, GROUPS at a time; blocks of a pass are whole
    const int bpp = max(1, GROUPS >> sp);                 // blocks per pass
    for (int jb = j_first; jb < N; jb += bpp) {
        const int nb = min(bpp, N - jb);
        {
            const int item = grp, j = jb + (item >> sp), pg_in = item & (ppb - 1);
            double acc[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
            if (item < nb * ppb) {
                const int t = j * bs + pg_in * kPage;
                const int rows = min(kPage, L - t);      // <= 0: page past the end of the sequence
                if (rows > 0) {
                    const int page = g.page_table[(int64_t)b * g.max_pages + t / kPage];
                    if (page >= 0 && page < g.num_pages) {
                        const T* src = kbase + ((int64_t)page * g.Hkv + h) * kPage * D + lane * VEC;
                        Words<NW> w[kPage];
#pragma unroll
                        for (int r = 0; r < kPage; ++r)
                            w[r] = r < rows ? load_words<NW>(src + r * D) : zero_words<NW>();
#pragma unroll
                        for (int r = 0; r < kPage; ++r)
#pragma unroll
                            for (int e = 0; e < VEC; ++e) acc[e] += (double)Elem<T>::get(w[r], e);
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) s_part[grp][lane * VEC + e] = acc[e];
        }
        __syncthreads();
        // one thread per (block of this pass, channel): page sums in order, mean, code
        for (int idx = threadIdx.x; idx < nb * D; idx += blockDim.x) {
            const int k = idx / D, d = idx - k * D, j = jb + k;
            double sum = 0.0;
            for (int p = 0; p < ppb; ++p) sum += s_part[k * ppb + p][d];
            const int n = min(bs, L - j * bs);
            const float c = (float)(sum / (double)n);
            const float sc = scale[(int64_t)bh * D + d], z = lo[(int64_t)bh * D + d];
            bool out;
            const uint32_t code = code_of<FMT>(c, sc, z, &out);
            clamped += out ? 1 : 0;
            if constexpr (BITS == 4) {
                // two channels per byte: the even channel's thread writes the pair
                const uint32_t other = __shfl_xor(code, 1);
                if ((d & 1) == 0) codes[(row0 + j) * RB + d / 2] = (uint8_t)(code | (other << 4));
            } else if constexpr (BITS == 8) {
                codes[(row0 + j) * RB + d] = (uint8_t)code;
            } else {
                reinterpret_cast<uint16_t*>(codes + (row0 + j) * RB)[d] = (uint16_t)code;
            }
        }
        __syncthreads();
    }
    if (clamped != 0) atomicAdd(&s_clamped, clamped);
    __syncthreads();
    if (threadIdx.x == 0 && out_of_range != nullptr) out_of_range[bh] = s_clamped;
}

template <typename T, int D>
hipError_t update_impl(const Geom& g, const UpdateArgs& a, hipStream_t s) {
#define ABS_UPDATE(F_)                                                                                         \
    hipLaunchKernelGGL((k_centroid_update<T, D, F_>), dim3(g.B * g.Hkv), dim3(256), 0, s, g, a.appended, a.scale, \
                       a.lo, a.codes, a.out_of_range)
    switch (a.fmt) {
        case kInt4Sym: ABS_UPDATE(kInt4Sym); break;
        case kInt8: ABS_UPDATE(kInt8); break;
        case kBf16: ABS_UPDATE(kBf16); break;
        default: ABS_UPDATE(kInt4); break;   // kInt4 and kInt4Tensor
    }
#undef ABS_UPDATE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_build(const Geom& g, DType dt, const BuildArgs& a, hipStream_t s) {
    if (dt == DType::BF16) return g.D == 128 ? build_impl<uint16_t, 128>(g, a, s) : build_impl<uint16_t, 64>(g, a, s);
    return g.D == 128 ? build_impl<float, 128>(g, a, s) : build_impl<float, 64>(g, a, s);
}

hipError_t launch_update(const Geom& g, DType dt, const UpdateArgs& a, hipStream_t s) {
    if (dt == DType::BF16)
        return g.D == 128 ? update_impl<uint16_t, 128>(g, a, s) : update_impl<uint16_t, 64>(g, a, s);
    return g.D == 128 ? update_impl<float, 128>(g, a, s) : update_impl<float, 64>(g, a, s);
}

}  // namespace absk
