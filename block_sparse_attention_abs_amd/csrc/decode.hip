// Sparse decode attention over the selected blocks (AB-Sparse page, Figure 1:
// sparse attention over the Top-K blocks; the mapping figure after Figure 8:
// block j of a head with stride s covers logical pages j*s .. j*s+s-1).
// Exact softmax attention, split over pages with an fp32 online softmax and
// a log-sum-exp merge (FlashAttention, in the page's references).
//
// split:  one 256-thread workgroup per (split, b*Hkv + h) handles PPW of the
//         head's selected pages for all G query heads of the group (the K/V
//         page is read once for the group).  Lane (row r, lane c) of the
//         16x16 layout holds channels [c*D/16, (c+1)*D/16) of token r of each
//         page; every K and V load of the workgroup is issued before any math.
//         q.k is reduced over the 16 lanes of a DPP row; logits are kept in
//         log2 units (q pre-scaled by sm_scale*log2 e).  The workgroup writes
//         (m, l, o[D]) per query head to fp32 partials.
// merge:  one workgroup per (b, query head): M = max m_s, l = sum 2^(m_s-M) l_s,
//         out = sum 2^(m_s-M) o_s / l, lse = (M + log2 l) * ln 2.
#include "device.hpp"

namespace absk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T, int D, int GT, int PPW>
__global__ __launch_bounds__(256) void k_decode_split(Geom g, const T* __restrict__ q,
                                                      const int32_t* __restrict__ sel, int sel_cap,
                                                      const int32_t* __restrict__ count, float qscale,
                                                      float* __restrict__ part_ml, float* __restrict__ part_o,
                                                      int splits) {
    constexpr int VEC = D / kRowLanes;
    constexpr int NW = VEC * Elem<T>::kBytes / 4;
    const int split = blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / g.Hkv, h = bh - b * g.Hkv;
    const int L = g.seq_lens[b];
    const int bs = g.block_size[h];
    const int spb = bs / kPage;                        // pages per block (stride)
    const int npages = ceil_div(L, kPage);
    const int N = ceil_div(L, bs);
    const int K = min(max(count[bh], 0), sel_cap);
    const int total = K * spb;
    const int p0 = split * PPW;
    const int row = threadIdx.x / kRowLanes;
    const int lane = threadIdx.x & (kRowLanes - 1);
    const int wave = threadIdx.x / 64;
    const T* kc = reinterpret_cast<const T*>(g.k);
    const T* vc = reinterpret_cast<const T*>(g.v);

    // physical page and first token of each of this workgroup's pages (uniform)
    int64_t phys[PPW];
    int tok0[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        const int gp = p0 + i;
        phys[i] = -1;
        tok0[i] = 0;
        if (gp < total) {
            const int blk = min(max(sel[(int64_t)bh * sel_cap + gp / spb], 0), N - 1);
            const int lp = blk * spb + gp % spb;
            if (lp < npages) {
                const int pg = g.page_table[(int64_t)b * g.max_pages + lp];
                if (pg >= 0 && pg < g.num_pages) {
                    phys[i] = pg;
                    tok0[i] = lp * kPage;
                }
            }
        }
    }

    Words<NW> kw[PPW], vw[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        if (phys[i] >= 0) {
            const int64_t off = ((phys[i] * g.Hkv + h) * kPage + row) * D + lane * VEC;
            kw[i] = load_words<NW>(kc + off);
            vw[i] = load_words<NW>(vc + off);
        } else {
            kw[i] = zero_words<NW>();
            vw[i] = zero_words<NW>();
        }
    }

    float qv[GT][VEC];
#pragma unroll
    for (int gg = 0; gg < GT; ++gg) {
        const bool on = gg < g.G;
        const T* qp = q + ((int64_t)b * g.Hq + h * g.G + (on ? gg : 0)) * D + lane * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) qv[gg][e] = on ? Elem<T>::load1(qp + e) * qscale : 0.0f;
    }

    float sc[PPW][GT];
    float m[GT];
#pragma unroll
    for (int gg = 0; gg < GT; ++gg) m[gg] = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        const bool valid = phys[i] >= 0 && tok0[i] + row < L;
#pragma unroll
        for (int gg = 0; gg < GT; ++gg) {
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc += qv[gg][e] * Elem<T>::template get<NW>(kw[i], e);
            acc = row16_sum(acc);
            sc[i][gg] = valid ? acc : -__builtin_inff();
            m[gg] = fmaxf(m[gg], sc[i][gg]);
        }
    }

    __shared__ float s_m[4][GT];
    __shared__ float s_l[4][GT];
    __shared__ float s_o[4][GT][D];
#pragma unroll
    for (int gg = 0; gg < GT; ++gg) {
        m[gg] = rows4_max(m[gg]);
        if ((threadIdx.x & 63) == 0) s_m[wave][gg] = m[gg];
    }
    __syncthreads();
#pragma unroll
    for (int gg = 0; gg < GT; ++gg) m[gg] = fmaxf(fmaxf(s_m[0][gg], s_m[1][gg]), fmaxf(s_m[2][gg], s_m[3][gg]));

    float l[GT], o[GT][VEC];
#pragma unroll
    for (int gg = 0; gg < GT; ++gg) {
        l[gg] = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[gg][e] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
#pragma unroll
        for (int gg = 0; gg < GT; ++gg) {
            const float p = sc[i][gg] == -__builtin_inff() ? 0.0f : exp2f(sc[i][gg] - m[gg]);
            l[gg] += p;
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[gg][e] += p * Elem<T>::template get<NW>(vw[i], e);
        }
    }
#pragma unroll
    for (int gg = 0; gg < GT; ++gg) {
        l[gg] = rows4_sum(l[gg]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[gg][e] = rows4_sum(o[gg][e]);
    }
    if ((threadIdx.x & 63) < kRowLanes) {
#pragma unroll
        for (int gg = 0; gg < GT; ++gg) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) s_o[wave][gg][lane * VEC + e] = o[gg][e];
            if (lane == 0) s_l[wave][gg] = l[gg];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < GT * D; idx += blockDim.x) {
        const int gg = idx / D, d = idx - gg * D;
        if (gg >= g.G) continue;
        const int64_t prow = ((int64_t)b * g.Hq + h * g.G + gg) * splits + split;
        part_o[prow * D + d] = s_o[0][gg][d] + s_o[1][gg][d] + s_o[2][gg][d] + s_o[3][gg][d];
        if (d == 0) {
            part_ml[prow * 2 + 0] = m[gg];
            part_ml[prow * 2 + 1] = s_l[0][gg] + s_l[1][gg] + s_l[2][gg] + s_l[3][gg];
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void k_decode_merge(Geom g, const float* __restrict__ part_ml,
                                                    const float* __restrict__ part_o, int splits,
                                                    T* __restrict__ out, float* __restrict__ lse) {
    const int bi = blockIdx.x;                 // b * Hq + query head
    const int d = threadIdx.x;
    const float* ml = part_ml + (int64_t)bi * splits * 2;
    float M = -__builtin_inff();
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[2 * s]);
    float lsum = 0.0f, acc = 0.0f;
    if (M != -__builtin_inff()) {
        for (int s = 0; s < splits; ++s) {
            const float ms = ml[2 * s];
            if (ms == -__builtin_inff()) continue;
            const float w = exp2f(ms - M);
            lsum += w * ml[2 * s + 1];
            acc += w * part_o[((int64_t)bi * splits + s) * D + d];
        }
    }
    Elem<T>::store1(out + (int64_t)bi * D + d, lsum > 0.0f ? acc / lsum : 0.0f);
    if (lse != nullptr && d == 0) lse[bi] = lsum > 0.0f ? (M + log2f(lsum)) * kLn2 : -__builtin_inff();
}

template <typename T, int D, int GT>
hipError_t decode_gt(const Geom& g, const DecodeArgs& a, hipStream_t s) {
    const dim3 grid(a.splits, g.B * g.Hkv);
    const float qscale = a.sm_scale * kLog2e;
    const T* q = reinterpret_cast<const T*>(a.q);
#define ABS_SPLIT(PPW_)                                                                                   \
    hipLaunchKernelGGL((k_decode_split<T, D, GT, PPW_>), grid, dim3(256), 0, s, g, q, a.sel, a.sel_cap, \
                       a.count, qscale, a.part_ml, a.part_o, a.splits)
    switch (a.pages_per_wg) {
        case 1: ABS_SPLIT(1); break;
        case 2: ABS_SPLIT(2); break;
        case 4: ABS_SPLIT(4); break;
        default: ABS_SPLIT(8); break;
    }
#undef ABS_SPLIT
    hipLaunchKernelGGL((k_decode_merge<T, D>), dim3(g.B * g.Hq), dim3(D), 0, s, g, a.part_ml, a.part_o, a.splits,
                       reinterpret_cast<T*>(a.out), a.lse);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t decode_impl(const Geom& g, const DecodeArgs& a, hipStream_t s) {
    if (g.G <= 1) return decode_gt<T, D, 1>(g, a, s);
    if (g.G <= 2) return decode_gt<T, D, 2>(g, a, s);
    if (g.G <= 4) return decode_gt<T, D, 4>(g, a, s);
    return decode_gt<T, D, 8>(g, a, s);
}

}  // namespace

hipError_t launch_decode(const Geom& g, DType dt, const DecodeArgs& a, hipStream_t s) {
    if (dt == DType::BF16) return g.D == 128 ? decode_impl<uint16_t, 128>(g, a, s) : decode_impl<uint16_t, 64>(g, a, s);
    return g.D == 128 ? decode_impl<float, 128>(g, a, s) : decode_impl<float, 64>(g, a, s);
}

}  // namespace absk
