// Centroid build and INT4 asymmetric per-channel quantization (AB-Sparse page:
// Figure 1's block representation; Figure 8's INT4 asymmetric per-channel
// centroids; the mapping figure after Figure 8 for pages -> blocks).
//
// Three launches per layer (staging rows are (b*Hkv + h) * tiles*64 + j, so
// they do not depend on the caller's centroid offsets):
//   mean:     one workgroup per (tile of 64 blocks, b*Hkv + h).  16 lanes own a
//             cache row (16 x head_dim/16 channels); 16 row-groups work on 16
//             blocks at a time, streaming each page's 16 rows with 16
//             independent wide loads.  Sums are fp64 (exact for bf16 keys), so
//             the fp32 centroid is the correctly rounded mean.  Per-channel
//             min/max of the tile is reduced with shuffles + LDS.
//   range:    per (b, h, channel): min/max over tiles -> lo, scale (fp32).
//   quantize: code = clamp(rint((c - lo) / scale), 0, 15), two per byte.
#include "device.hpp"

namespace absk {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void k_centroid_mean(Geom g, float* __restrict__ staging,
                                                        float* __restrict__ pmin, float* __restrict__ pmax,
                                                        int tiles) {
    constexpr int VEC = D / kRowLanes;                    // channels per lane
    constexpr int NW = VEC * Elem<T>::kBytes / 4;         // 32-bit words per lane per row
    constexpr int GROUPS = 256 / kRowLanes;               // 16 blocks in flight
    const int bh = blockIdx.y;
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int L = g.seq_lens[b];
    const int bs = block_size_of(g, h);
    const int N = ceil_div(L, bs);
    const int j0 = blockIdx.x * kBuildTile;
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

    for (int jj = grp; jj < kBuildTile; jj += GROUPS) {
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
            for (int r = 0; r < kPage; ++r) w[r] = r < rows ? load_words<NW>(src + r * D) : zero_words<NW>();
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
        float* dst = staging + ((int64_t)bh * tiles * kBuildTile + j) * D + lane * VEC;
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

template <int D>
__global__ __launch_bounds__(D) void k_centroid_range(Geom g, const float* __restrict__ pmin,
                                                      const float* __restrict__ pmax, int tiles,
                                                      float* __restrict__ scale, float* __restrict__ lo) {
    const int bh = blockIdx.x;
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int N = ceil_div(g.seq_lens[b], block_size_of(g, h));
    const int nt = ceil_div(N, kBuildTile);
    const int d = threadIdx.x;
    float a = __builtin_inff(), z = -__builtin_inff();
    for (int t = 0; t < nt; ++t) {
        a = fminf(a, pmin[((int64_t)bh * tiles + t) * D + d]);
        z = fmaxf(z, pmax[((int64_t)bh * tiles + t) * D + d]);
    }
    const float range = z - a;        // fp32
    const float s = range / 15.0f;    // IEEE fp32 division
    scale[(int64_t)bh * D + d] = s;
    lo[(int64_t)bh * D + d] = a;
}

// One thread per (block, 8 channels): reads 32 B of fp32 centroid, writes 4 B of codes.
template <int D>
__global__ __launch_bounds__(256) void k_centroid_quantize(Geom g, const float* __restrict__ staging,
                                                           const float* __restrict__ scale,
                                                           const float* __restrict__ lo,
                                                           uint8_t* __restrict__ codes, int tiles) {
    constexpr int TPB = D / 8;                 // threads per block row
    constexpr int ROWS = 256 / TPB;            // block rows per pass
    const int bh = blockIdx.y;
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int N = ceil_div(g.seq_lens[b], block_size_of(g, h));
    const int j0 = blockIdx.x * kBuildTile;
    if (j0 >= N) return;
    const int64_t row0 = g.off[bh];
    const int c8 = threadIdx.x % TPB;
    float s[8], z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s[e] = scale[(int64_t)bh * D + c8 * 8 + e];
        z[e] = lo[(int64_t)bh * D + c8 * 8 + e];
    }
    for (int jj = threadIdx.x / TPB; jj < kBuildTile; jj += ROWS) {
        const int j = j0 + jj;
        if (j >= N) break;
        const float* src = staging + ((int64_t)bh * tiles * kBuildTile + j) * D + c8 * 8;
        const float4 u0 = reinterpret_cast<const float4*>(src)[0];
        const float4 u1 = reinterpret_cast<const float4*>(src)[1];
        const float c[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t code = 0;
            if (s[e] > 0.0f) {
                const float diff = c[e] - z[e];
                const float quot = diff / s[e];          // IEEE fp32 division
                const float r = fminf(fmaxf(rintf(quot), 0.0f), 15.0f);
                code = (uint32_t)r;
            }
            packed |= code << (4 * e);
        }
        *reinterpret_cast<uint32_t*>(codes + (row0 + j) * (D / 2) + c8 * 4) = packed;
    }
}

template <typename T, int D>
hipError_t build_impl(const Geom& g, const BuildArgs& a, hipStream_t s) {
    const dim3 grid(a.tiles, g.B * g.Hkv);
    hipLaunchKernelGGL((k_centroid_mean<T, D>), grid, dim3(256), 0, s, g, a.staging, a.pmin, a.pmax, a.tiles);
    hipLaunchKernelGGL((k_centroid_range<D>), dim3(g.B * g.Hkv), dim3(D), 0, s, g, a.pmin, a.pmax, a.tiles,
                       a.scale, a.lo);
    hipLaunchKernelGGL((k_centroid_quantize<D>), grid, dim3(256), 0, s, g, a.staging, a.scale, a.lo, a.codes,
                       a.tiles);
    return hipGetLastError();
}

// Centroids kept current while decoding (the page fixes static per-head
// block sizes, Figure 5's text, and INT4 per-channel centroids, Figure 8;
// how they follow appended tokens is read as: recompute every block holding
// one of the tokens [L - appended - 1, L) -- always at least the last,
// possibly partial block -- and code it with the head's stored (scale, lo),
// clamped to 0..15, counting the clamped codes).  One workgroup per (b, h).
// Each 16-lane row group loads one 16-token page of a recomputed block (all
// pages at once) and sums its rows in order in fp64; the page sums are then
// added in page order (exact for bf16 keys, like the build's sums) and the
// mean is coded by one thread per channel.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_centroid_update(Geom g, int appended, const float* __restrict__ scale,
                                                         const float* __restrict__ lo, uint8_t* __restrict__ codes,
                                                         int32_t* __restrict__ out_of_range) {
    constexpr int VEC = D / kRowLanes;                    // channels per lane
    constexpr int NW = VEC * Elem<T>::kBytes / 4;
    constexpr int GROUPS = 256 / kRowLanes;               // pages in flight
    const int bh = blockIdx.x;
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int L = g.seq_lens[b];
    const int bs = block_size_of(g, h);
    const int ppb = bs / kPage;                           // pages per block
    const int N = ceil_div(L, bs);
    const int j_first = (max(1, L - appended) - 1) / bs;
    const int64_t row0 = g.off[bh];
    const int lane = threadIdx.x & (kRowLanes - 1);
    const int grp = threadIdx.x / kRowLanes;
    const T* kbase = reinterpret_cast<const T*>(g.k);
    __shared__ double s_part[GROUPS][D];                  // per page: sum of its valid rows
    __shared__ int s_clamped;
    if (threadIdx.x == 0) s_clamped = 0;
    int clamped = 0;
    // (block, page) items, GROUPS at a time; blocks of a pass are whole
    const int bpp = max(1, GROUPS / ppb);                 // blocks per pass
    for (int jb = j_first; jb < N; jb += bpp) {
        const int nb = min(bpp, N - jb);
        {
            const int item = grp, j = jb + item / ppb, pg_in = item % ppb;
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
            uint32_t code = 0;
            if (sc > 0.0f) {
                const float diff = c - z;
                const float quot = diff / sc;             // IEEE fp32 division
                const float r = rintf(quot);
                clamped += (r < 0.0f || r > 15.0f) ? 1 : 0;
                code = (uint32_t)fminf(fmaxf(r, 0.0f), 15.0f);
            } else {
                clamped += c != z ? 1 : 0;
            }
            // two channels per byte: the even channel's thread writes the pair
            const uint32_t other = __shfl_xor(code, 1);
            if ((d & 1) == 0) codes[(row0 + j) * (D / 2) + d / 2] = (uint8_t)(code | (other << 4));
        }
        __syncthreads();
    }
    if (clamped != 0) atomicAdd(&s_clamped, clamped);
    __syncthreads();
    if (threadIdx.x == 0 && out_of_range != nullptr) out_of_range[bh] = s_clamped;
}

template <typename T, int D>
hipError_t update_impl(const Geom& g, const UpdateArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((k_centroid_update<T, D>), dim3(g.B * g.Hkv), dim3(256), 0, s, g, a.appended, a.scale, a.lo,
                       a.codes, a.out_of_range);
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
