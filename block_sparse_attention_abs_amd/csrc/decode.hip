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
//         page for the V side; pages are streamed in chunks of up to 8, two
//         chunks in flight when the workgroup has enough pages.  For bf16,
//         q.k runs on the matrix cores (each wavefront owns two pages of a
//         chunk); otherwise it is reduced over the 16 lanes of a DPP row.
//         Logits are kept in log2 units (q pre-scaled by sm_scale*log2 e).
//         The workgroup's (m, l, o[D]) per query head is its partial.
//         bf16 layers with D = 128 and groups of up to 4 heads use the
//         wavefront-split form instead (k_sparse_decode_ws): each wavefront
//         streams its own pages with its own softmax state, and the four
//         states meet only at the end.
// merge:  M = max m_s, l = sum 2^(m_s-M) l_s, out = sum 2^(m_s-M) o_s / l,
//         lse = (M + log2 l) * ln 2.  Done in the split launch by the last
//         workgroup to finish each (b, h): partials are written with
//         agent-scope stores, an agent-scope counter per (b, h) finds the
//         last arrival, which reads the partials with agent-scope loads (no
//         L2 writeback is needed, unlike an agent-scope fence).  A build
//         switch keeps the older form, a second launch with one workgroup
//         per (b, query head).
#include "device.hpp"
#include "topk.hpp"

// Build-time tuning: partials the merging workgroup loads per pass.
#ifndef ABS_DECODE_MERGE_BATCH
#define ABS_DECODE_MERGE_BATCH 8
#endif

namespace absk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// 2^x by the hardware's exp2 (v_exp_f32, about 1 ulp); -inf gives 0.  The
// arguments here are <= 0 and results below 2^-126 only weigh tokens that
// are negligible next to the row maximum (weight 1).
__device__ __forceinline__ float exp2_approx(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLn2 = 0.6931471805599453f;

// Waves per SIMD the split kernel is compiled for: 4 (all of a typical
// grid resident at once) unless the group or the row width needs more registers.
// (PIPE: two chunks of K/V in registers at once; MF: the query in the A-operand
// layout as well.)
template <typename T, int D, int GT, bool PIPE, bool MF>
struct DecodeOccupancy {
    static constexpr int value = (PIPE || GT >= 8 || D * (int)sizeof(T) > 256) ? 2
                                 : (MF && GT >= 4 && D * (int)sizeof(T) >= 256) ? 3
                                                                                : 4;
};

// The double-buffered form fits the register file (no spills) only for
// 2-byte elements and up to 4 query heads per group at D = 128.
template <typename T, int D, int GT>
constexpr bool kPipeFits = sizeof(T) == 2 && (D == 64 || GT <= 4);

// Build-time switch: 0 keeps q.k on the vector ALUs for bf16 as well.
#ifndef ABS_DECODE_MATRIX
#define ABS_DECODE_MATRIX 1
#endif
// 1: bf16 layers with D = 128 and up to 4 query heads per KV head use the
// wavefront-split kernel for 8-page and double-buffered layouts.
#ifndef ABS_DECODE_WAVES
#define ABS_DECODE_WAVES 1
#endif
// Page buffers per wavefront in the wavefront-split kernel (1 measured best).
#ifndef ABS_DECODE_WS_DEPTH
#define ABS_DECODE_WS_DEPTH 1
#endif
// Row groups of the double-buffered matrix-core kernel (1 or 2).
#ifndef ABS_DECODE_ROWGROUPS
#define ABS_DECODE_ROWGROUPS 1
#endif

// Agent-scope (device-coherent) 8-byte store and load: relaxed atomics, which
// write through and read past the per-XCD L2.
__device__ __forceinline__ void store2_agent(float* p, float a, float b) {
    const uint64_t u = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load2_agent(const float* p) {
    const uint64_t u = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}

// Final output of query row bi, channels d and d+1, from the merged state
// (sum o, max m in log2 units, sum l).
template <typename T>
__device__ __forceinline__ void write_output(T* out, float* lse, int64_t bi, int d, float2 acc, float m, float l, int D) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    Elem<T>::store1(out + bi * D + d, acc.x * inv);
    Elem<T>::store1(out + bi * D + d + 1, acc.y * inv);
    if (lse != nullptr && d == 0) lse[bi] = l > 0.0f ? (m + log2f(l)) * kLn2 : -__builtin_inff();
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// MF: q.k on the matrix cores (bf16 only, CH == 8).  Each wavefront owns two
// pages of a chunk and loads their K in the B-operand layout of
// v_mfma_f32_16x16x32_bf16 (lane l: token l%16, channels 8*(l/16)..+7 of the
// step's 32, so a step reads 64 contiguous bytes of each key row).  The query
// rows of the A operand are the group's heads repeated 4x, so lane l receives
// S[head][token l%16] for all heads.  The scores go through LDS (one barrier
// per chunk, double-buffered) to the row layout the V side uses.
//
// RG row groups (RG = 2 only with MF): 256*RG threads; row group rg folds the
// pages rg, rg + RG, ... of each chunk into its own 16 rows, so each
// wavefront does 1/RG of the softmax and P.V work of a chunk and RG
// wavefronts share each SIMD.
template <typename T, int D, int GT, int CH, bool PIPE, bool MF, int RG>
__global__ __launch_bounds__(256 * RG, (DecodeOccupancy<T, D, GT, PIPE, MF>::value)) void k_sparse_decode(Geom g, const T* __restrict__ q,
                                                          const int32_t* __restrict__ sel, int sel_cap,
                                                          const int32_t* __restrict__ count, float qscale,
                                                          float* __restrict__ part_ml, float* __restrict__ part_o,
                                                          int splits, int ppw, uint32_t ppw_magic,
                                                          int32_t* __restrict__ arrive,
                                                          T* __restrict__ out, float* __restrict__ lse) {
    constexpr int VEC = D / kRowLanes;
    constexpr int NW = VEC * Elem<T>::kBytes / 4;
    constexpr float NEG = -__builtin_inff();
    const int split = blockIdx.x;
    const int bh = blockIdx.y;
    int b, h;
    split_bh(g, bh, b, h);
    const int row = (threadIdx.x & 255) / kRowLanes;
    const int rg = threadIdx.x >> 8;                     // row group
    const int lane = threadIdx.x & (kRowLanes - 1);
    const int wave = threadIdx.x / 64;
    const int wl = threadIdx.x & 63;

    constexpr int KSTEPS = D / 32;                       // MFMA k-steps per key row
    constexpr int GP = (GT + 3) / 4;                     // MFMA passes (4 heads each)
    constexpr int PPC = CH / RG;                         // pages of a chunk per row group (V side)
    constexpr int PWV = 2 / RG;                          // MF: pages of a chunk per wavefront (K side)
    constexpr int KW = MF ? PWV * KSTEPS : CH;           // K words held per chunk
    static_assert(!MF || (CH == 8 && sizeof(T) == 2), "matrix-core path: bf16, 8-page chunks");
    static_assert(RG == 1 || (MF && RG == 2), "two row groups only with the matrix-core path");

    // Resolve this workgroup's pages lane-parallel: lane i of every wavefront
    // follows selection entry -> logical page -> physical page for page p0 + i
    // (the selection row is read speculatively up to sel_cap, before the
    // sequence length and the count arrive); readlane then broadcasts them.
    const int sh = block_shift_of(g, h) - 4;          // log2(pages per block)
    const int spb = 1 << sh;                           // pages per block (stride): 1, 2 or 4
    const int p0 = split * ppw;                        // ppw <= 64
    const int gp = p0 + wl;
    const bool in_row = wl < ppw && gp < sel_cap * spb;
    const int sv = sel[(int64_t)bh * sel_cap + min(gp >> sh, sel_cap - 1)];   // unconditional, clamped
    const int L = seq_len(g, b);
    const int npages = shr_ceil(L, 4);
    const int N = shr_ceil(L, sh + 4);
    const int K = min(max(count[bh], 0), sel_cap);
    const int total = min(K * spb, splits * ppw);      // selected pages of (b, h)
    int ph = -1, lp = 0;
    if (in_row) {
        lp = min(max(sv, 0), N - 1) * spb + (gp & (spb - 1));
        if (lp < npages) {
            const int pg = g.page_table[(int64_t)b * g.max_pages + lp];
            if (pg >= 0 && pg < g.num_pages) ph = pg;
        }
    }
    if (gp >= total) ph = -1;

    // The group's queries, issued after the page resolution's first load so
    // that they do not queue ahead of it.
    Words<NW> qw[MF ? 1 : GT];
    Words<4> qa[MF ? GP : 1][MF ? KSTEPS : 1];
    if constexpr (MF) {
        const int m4 = (wl & 15) & 3;
#pragma unroll
        for (int pp = 0; pp < GP; ++pp) {
            const int head = h * g.G + min(4 * pp + m4, g.G - 1);
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st)
                qa[pp][st] = load_words<4>(q + ((int64_t)b * g.Hq + head) * D + st * 32 + (wl >> 4) * 8);
        }
    } else {
#pragma unroll
        for (int gg = 0; gg < GT; ++gg) {
            const int head = h * g.G + min(gg, g.G - 1);
            qw[gg] = load_words<NW>(q + ((int64_t)b * g.Hq + head) * D + lane * VEC);
        }
    }

    __shared__ float s_red[4 * RG][GT];
    constexpr int kRows = 256 * RG / kRowLanes;
    __shared__ __align__(16) float s_o[kRows][GT][D];   // epilogue: each row's rescaled output
    __shared__ float s_l[kRows][GT];
    __shared__ float s_sc[MF ? 2 : 1][MF ? CH : 1][MF ? 16 : 1][GT];   // MF: scores, double-buffered per chunk
    int sbuf = 0;

    // Per-row running softmax state (each row of 16 lanes sees one token per page).
    float m[GT], l[GT], o[GT][VEC];
#pragma unroll
    for (int gg = 0; gg < GT; ++gg) {
        m[gg] = NEG;
        l[gg] = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[gg][e] = 0.0f;
    }
    // Selected pages are contiguous from the start of the list, so a
    // workgroup whose first page is empty has nothing to do.
    const bool active = __builtin_amdgcn_readfirstlane(ph) >= 0;
    if (active) {
        const T* kc = reinterpret_cast<const T*>(g.k);
        const T* vc = reinterpret_cast<const T*>(g.v);
        const uint32_t lane_off = (uint32_t)((row * D + lane * VEC) * sizeof(T));
        // issue every K and V load of the chunk of CH pages starting at c0
        auto issue = [&](int c0, Words<MF ? 4 : NW>(&kw)[KW], Words<NW>(&vw)[PPC]) {
            if constexpr (MF) {
                // this wavefront's pages (wave, wave + 4*RG), B-operand layout
                const uint32_t k_off = (uint32_t)(((wl & 15) * D + (wl >> 4) * 8) * sizeof(T));
#pragma unroll
                for (int j = 0; j < PWV; ++j) {
                    const int pg = __builtin_amdgcn_readlane(ph, c0 + wave + 4 * RG * j);
                    const int64_t base = ((int64_t)(pg >= 0 ? pg : 0) * g.Hkv + h) * (kPage * D);
#pragma unroll
                    for (int st = 0; st < KSTEPS; ++st)
                        kw[j * KSTEPS + st] = load_words_stream_at<4>(kc + base + st * 32, k_off);
                }
            } else {
#pragma unroll
                for (int i = 0; i < CH; ++i) {   // branch-free: empty slots re-read page 0 and are masked later
                    const int pg = __builtin_amdgcn_readlane(ph, c0 + i);
                    const int64_t base = ((int64_t)(pg >= 0 ? pg : 0) * g.Hkv + h) * (kPage * D);
                    kw[i] = load_words_stream_at<NW>(kc + base, lane_off);
                }
            }
#pragma unroll
            for (int k = 0; k < PPC; ++k) {   // this row group's pages rg, rg + RG, ...
                const int pg = __builtin_amdgcn_readlane(ph, c0 + RG * k + rg);
                const int64_t base = ((int64_t)(pg >= 0 ? pg : 0) * g.Hkv + h) * (kPage * D);
                vw[k] = load_words_stream_at<NW>(vc + base, lane_off);
            }
        };
        // fold the chunk at c0 into this row's running (m, l, o)
        auto consume = [&](int c0, const Words<MF ? 4 : NW>(&kw)[KW], const Words<NW>(&vw)[PPC]) {
            float sc[PPC][GT], cm[GT];
#pragma unroll
            for (int gg = 0; gg < GT; ++gg) cm[gg] = m[gg];
            if constexpr (MF) {
#pragma unroll
                for (int j = 0; j < PWV; ++j) {
                    const int pi = wave + 4 * RG * j;
                    const int pg = __builtin_amdgcn_readlane(ph, c0 + pi);
                    const int t0 = __builtin_amdgcn_readlane(lp, c0 + pi) * kPage;
                    const bool valid = pg >= 0 && t0 + (wl & 15) < L;
#pragma unroll
                    for (int pp = 0; pp < GP; ++pp) {
                        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int st = 0; st < KSTEPS; ++st)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, qa[pp][st]), __builtin_bit_cast(bf16x8_t, kw[j * KSTEPS + st]),
                                acc, 0, 0, 0);
                        if (wl < 16) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (4 * pp + i < GT) s_sc[sbuf][pi][wl][4 * pp + i] = valid ? acc[i] * qscale : NEG;
                        }
                    }
                }
                __syncthreads();
#pragma unroll
                for (int k = 0; k < PPC; ++k)
#pragma unroll
                    for (int gg = 0; gg < GT; ++gg) {
                        sc[k][gg] = s_sc[sbuf][RG * k + rg][row][gg];
                        cm[gg] = fmaxf(cm[gg], sc[k][gg]);
                    }
                sbuf ^= 1;
            } else {
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int pg = __builtin_amdgcn_readlane(ph, c0 + i);
                    const int t0 = __builtin_amdgcn_readlane(lp, c0 + i) * kPage;
                    const bool valid = pg >= 0 && t0 + row < L;
#pragma unroll
                    for (int gg = 0; gg < GT; ++gg) {
                        const float z = row16_sum(dot_words<T, NW>(qw[gg], kw[i])) * qscale;
                        sc[i][gg] = valid ? z : NEG;
                        cm[gg] = fmaxf(cm[gg], sc[i][gg]);
                    }
                }
            }
            // Exponents are taken against ms, the new running max, or 0 while a
            // row has seen no valid token: exp2(-inf) = 0 then covers masked
            // tokens and the empty state (l = o = 0) without further tests.
            float ms[GT];
#pragma unroll
            for (int gg = 0; gg < GT; ++gg) {
                ms[gg] = cm[gg] == NEG ? 0.0f : cm[gg];
                const float alpha = exp2_approx(m[gg] - ms[gg]);
                m[gg] = cm[gg];
                l[gg] *= alpha;
#pragma unroll
                for (int e = 0; e < VEC; ++e) o[gg][e] *= alpha;
            }
#pragma unroll
            for (int i = 0; i < PPC; ++i) {
                float p[GT];
#pragma unroll
                for (int gg = 0; gg < GT; ++gg) {
                    p[gg] = exp2_approx(sc[i][gg] - ms[gg]);
                    l[gg] += p[gg];
                }
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float v = Elem<T>::template get<NW>(vw[i], e);
#pragma unroll
                    for (int gg = 0; gg < GT; ++gg) o[gg][e] = fmaf(p[gg], v, o[gg][e]);
                }
            }
        };
        auto has_chunk = [&](int c0) { return c0 < ppw && __builtin_amdgcn_readlane(ph, c0) >= 0; };
        if constexpr (PIPE) {
            // double-buffered: the next chunk's loads are in flight while this one is folded
            Words<MF ? 4 : NW> ka[KW], kb[KW];
            Words<NW> va[PPC], vb[PPC];
            issue(0, ka, va);
            for (int c0 = 0;; c0 += 2 * CH) {
                const bool nb = has_chunk(c0 + CH);
                if (nb) issue(c0 + CH, kb, vb);
                consume(c0, ka, va);
                if (!nb) break;
                const bool na = has_chunk(c0 + 2 * CH);
                if (na) issue(c0 + 2 * CH, ka, va);
                consume(c0 + CH, kb, vb);
                if (!na) break;
            }
        } else {
            for (int c0 = 0; has_chunk(c0); c0 += CH) {
                Words<MF ? 4 : NW> kw[KW];
                Words<NW> vw[PPC];
                issue(c0, kw, vw);
                consume(c0, kw, vw);
            }
        }

        // rows -> workgroup: the common max (shuffles within a wavefront, LDS
        // across the four), then each row's rescaled state goes to LDS and
        // every thread sums two channels over the 16 rows.
        float M[GT];
#pragma unroll
        for (int gg = 0; gg < GT; ++gg) M[gg] = rows4_max(m[gg]);
#pragma unroll
        for (int gg = 0; gg < GT; ++gg)
            if (wl == 0) s_red[wave][gg] = M[gg];
        __syncthreads();
#pragma unroll
        for (int gg = 0; gg < GT; ++gg) {
            M[gg] = s_red[0][gg];
#pragma unroll
            for (int w = 1; w < 4 * RG; ++w) M[gg] = fmaxf(M[gg], s_red[w][gg]);
            const float f = m[gg] == NEG ? 0.0f : exp2_approx(m[gg] - M[gg]);
            const int r = rg * 16 + row;
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                *reinterpret_cast<float4*>(&s_o[r][gg][lane * VEC + e]) =
                    make_float4(o[gg][e] * f, o[gg][e + 1] * f, o[gg][e + 2] * f, o[gg][e + 3] * f);
            if (lane == 0) s_l[r][gg] = l[gg] * f;
        }
        __syncthreads();
    }

    // This workgroup's share of (b, h), per (query head, channel pair): the
    // row sums from LDS, or an empty partial (m = -inf) when the workgroup is
    // in the selected range but all of its pages are empty.
    const bool fused = arrive != nullptr;
    const bool holds = p0 < total;                      // active implies holds
    const int nact = fast_div(total + ppw - 1, ppw, ppw_magic);   // workgroups holding pages of (b, h)
    if (holds) {
        for (int idx = 2 * (int)threadIdx.x; idx < GT * D; idx += 2 * (int)blockDim.x) {
            const int gg = idx / D, d = idx - gg * D;
            if (gg >= g.G) continue;
            float2 acc = make_float2(0.0f, 0.0f);
            float mg = NEG, ls = 0.0f;
            if (active) {
#pragma unroll
                for (int r = 0; r < kRows; ++r) {
                    const float2 v = *reinterpret_cast<const float2*>(&s_o[r][gg][d]);
                    acc.x += v.x;
                    acc.y += v.y;
                }
#pragma unroll
                for (int r = 0; r < kRows; ++r) ls += s_l[r][gg];
                mg = s_red[0][gg];
#pragma unroll
                for (int w = 1; w < 4 * RG; ++w) mg = fmaxf(mg, s_red[w][gg]);
            }
            const int64_t bi = (int64_t)b * g.Hq + h * g.G + gg;
            const int64_t prow = bi * splits + split;
            if (fused && nact == 1) {
                write_output(out, lse, bi, d, acc, mg, ls, D);        // the only workgroup of (b, h)
            } else if (fused) {
                store2_agent(part_o + prow * D + d, acc.x, acc.y);
                if (d == 0) store2_agent(part_ml + prow * 2, mg, ls);
            } else {
                *reinterpret_cast<float2*>(part_o + prow * D + d) = acc;
                if (d == 0) {
                    part_ml[prow * 2 + 0] = mg;
                    part_ml[prow * 2 + 1] = ls;
                }
            }
        }
    } else if (fused && total == 0 && split == 0) {
        // nothing selected for (b, h): zero output, lse = -inf
        for (int idx = 2 * (int)threadIdx.x; idx < GT * D; idx += 2 * (int)blockDim.x) {
            const int gg = idx / D, d = idx - gg * D;
            if (gg < g.G)
                write_output(out, lse, (int64_t)b * g.Hq + h * g.G + gg, d, make_float2(0.0f, 0.0f), NEG, 0.0f, D);
        }
    }
    if (!fused || !holds || nact == 1) return;

    // Hand-off: partials are written with agent-scope (L2 write-through)
    // stores; once every thread's stores have completed, one agent-scope
    // atomic counts the arrival.  The last of the nact workgroups resets the
    // counter for the next call and merges, reading with agent-scope loads.
    __shared__ int s_last;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = __hip_atomic_fetch_add(arrive + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == nact - 1;
        if (prev == nact - 1) __hip_atomic_store(arrive + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    constexpr int MB = ABS_DECODE_MERGE_BATCH;   // partials per merge pass
    for (int idx = 2 * (int)threadIdx.x; idx < GT * D; idx += 2 * (int)blockDim.x) {
        const int gg = idx / D, d = idx - gg * D;
        if (gg >= g.G) continue;
        const int64_t bi = (int64_t)b * g.Hq + h * g.G + gg;
        const float* ml = part_ml + bi * splits * 2;
        const float* po = part_o + bi * splits * D + d;
        float mg = NEG, ls = 0.0f;
        float2 acc = make_float2(0.0f, 0.0f);
        for (int s0 = 0; s0 < nact; s0 += MB) {
            // 2 MB loads in flight (indices clamped, so no load waits on a
            // branch), then one max and one weighted sum over the MB splits
            float2 mlv[MB], ov[MB];
#pragma unroll
            for (int k = 0; k < MB; ++k) {
                const int sk = min(s0 + k, nact - 1);
                mlv[k] = load2_agent(ml + 2 * sk);
                ov[k] = load2_agent(po + (int64_t)sk * D);
            }
            float bm = NEG;
#pragma unroll
            for (int k = 0; k < MB; ++k)
                if (s0 + k < nact) bm = fmaxf(bm, mlv[k].x);
            const float mn = fmaxf(mg, bm);
            if (mn == NEG) continue;                      // only empty partials so far
            const float a = mg == NEG ? 0.0f : exp2f(mg - mn);
            ls *= a;
            acc.x *= a;
            acc.y *= a;
#pragma unroll
            for (int k = 0; k < MB; ++k) {
                const float w = s0 + k < nact ? exp2f(mlv[k].x - mn) : 0.0f;   // empty partial: m = -inf, w = 0
                ls = fmaf(mlv[k].y, w, ls);
                acc.x = fmaf(ov[k].x, w, acc.x);
                acc.y = fmaf(ov[k].y, w, acc.y);
            }
            mg = mn;
        }
        write_output(out, lse, bi, d, acc, mg, ls, D);
    }
}

// WS: the wavefront-split form of the split kernel (bf16, D = 128, q.k on
// the matrix cores).  Wavefront w owns pages w, w + 4, w + 8, ... of the
// workgroup's range and keeps its own running (m, l, o) over them: the MFMA
// gives every lane S[head][token lane%16] of a page, the page's max and sum
// per head are DPP reductions over a 16-lane row (the four rows hold the
// same values), and P.V runs with each lane owning 2 of the 128 channels for
// all G heads, the 16 tokens' probabilities broadcast with readlane.  One
// page buffer per wavefront (ABS_DECODE_WS_DEPTH): the compiler issues the
// next page's loads while the current page is folded, and more buffers
// measured slower.  No LDS and no barrier until the four wavefronts' states
// are combined at the end.
// The body, for a lane whose page gp = split * ppw + lane lies in selected
// block sv (the selection entry at position gp >> log2(pages per block),
// clamped into the row) of a head with K selected blocks; NW wavefronts in
// the workgroup, of which 0-3 do the work.
template <int GT, int NW>
__device__ __forceinline__ void ws_decode(const Geom& g, const uint16_t* __restrict__ q, int L, int sv, int K, int sel_cap,
                                          float qscale, float* __restrict__ part_ml, float* __restrict__ part_o,
                                          int splits, int ppw, uint32_t ppw_magic, int32_t* __restrict__ arrive,
                                          uint16_t* __restrict__ out, float* __restrict__ lse) {
    using T = uint16_t;
    constexpr int D = 128;
    constexpr int KSTEPS = D / 32;
    constexpr int GP = (GT + 3) / 4;
    constexpr int DEPTH = ABS_DECODE_WS_DEPTH;           // page buffers per wavefront
    constexpr float NEG = -__builtin_inff();
    const int split = blockIdx.x;
    const int bh = blockIdx.y;
    int b, h;
    split_bh(g, bh, b, h);
    const int wave = threadIdx.x / 64;
    const int wl = threadIdx.x & 63;
    const bool worker = NW == 4 || wave < 4;

    const int sh = block_shift_of(g, h) - 4;          // log2(pages per block)
    const int spb = 1 << sh;                           // pages per block (stride): 1, 2 or 4
    const int p0 = split * ppw;                        // ppw <= 64
    const int gp = p0 + wl;
    const bool in_row = wl < ppw && gp < sel_cap * spb;
    const int npages = shr_ceil(L, 4);
    const int N = shr_ceil(L, sh + 4);
    const int total = min(K * spb, splits * ppw);      // selected pages of (b, h)
    int ph = -1, lp = 0;
    if (in_row) {
        lp = min(max(sv, 0), N - 1) * spb + (gp & (spb - 1));
        if (lp < npages) {
            const int pg = g.page_table[(int64_t)b * g.max_pages + lp];
            if (pg >= 0 && pg < g.num_pages) ph = pg;
        }
    }
    if (gp >= total) ph = -1;

    Words<4> qa[GP][KSTEPS];
    {
        const int m4 = (wl & 15) & 3;
#pragma unroll
        for (int pp = 0; pp < GP; ++pp) {
            const int head = h * g.G + min(4 * pp + m4, g.G - 1);
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st)
                qa[pp][st] = load_words<4>(q + ((int64_t)b * g.Hq + head) * D + st * 32 + (wl >> 4) * 8);
        }
    }

    __shared__ float s_red[4][GT];
    __shared__ __align__(16) float s_o[4][GT][D];
    __shared__ float s_l[4][GT];

    // this wavefront's running state; m and l are the same in every lane
    float m[GT], l[GT], o[GT][2];
#pragma unroll
    for (int gg = 0; gg < GT; ++gg) {
        m[gg] = NEG;
        l[gg] = 0.0f;
        o[gg][0] = o[gg][1] = 0.0f;
    }
    const bool active = __builtin_amdgcn_readfirstlane(ph) >= 0;
    if (active) {
        const T* kc = reinterpret_cast<const T*>(g.k);
        const T* vc = reinterpret_cast<const T*>(g.v);
        const uint32_t k_off = (uint32_t)(((wl & 15) * D + (wl >> 4) * 8) * sizeof(T));
        const uint32_t v_off = (uint32_t)(2 * wl * sizeof(T));
        const int nvalid = min(max(total - p0, 0), ppw);             // pages of this workgroup
        // ... of this wavefront; only wavefronts 0-3 stream pages (a launch
        // with more wavefronts, for the fused top-K, idles the others here)
        const int npw = worker && nvalid > wave ? (nvalid - wave + 3) / 4 : 0;
        auto issue = [&](int c, Words<4>(&kw)[KSTEPS], Words<1>(&vw)[kPage]) {
            const int pg = __builtin_amdgcn_readlane(ph, c);
            const int64_t base = ((int64_t)(pg >= 0 ? pg : 0) * g.Hkv + h) * (kPage * D);
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) kw[st] = load_words_stream_at<4>(kc + base + st * 32, k_off);
#pragma unroll
            for (int t = 0; t < kPage; ++t) vw[t] = load_words_stream_at<1>(vc + base + t * D, v_off);
        };
        auto consume = [&](int c, const Words<4>(&kw)[KSTEPS], const Words<1>(&vw)[kPage]) {
            const int pg = __builtin_amdgcn_readlane(ph, c);
            const int t0 = __builtin_amdgcn_readlane(lp, c) * kPage;
            const bool valid = pg >= 0 && t0 + (wl & 15) < L;
            float sc[GT];
#pragma unroll
            for (int pp = 0; pp < GP; ++pp) {
                f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int st = 0; st < KSTEPS; ++st)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[pp][st]),
                                                                  __builtin_bit_cast(bf16x8_t, kw[st]), acc, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * pp + i < GT) sc[4 * pp + i] = valid ? acc[i] * qscale : NEG;
            }
            float p[GT];
#pragma unroll
            for (int gg = 0; gg < GT; ++gg) {
                const float mn = fmaxf(m[gg], row16_max(sc[gg]));
                const float ms = mn == NEG ? 0.0f : mn;       // no valid token yet: exponents give 0
                const float alpha = exp2_approx(m[gg] - ms);
                p[gg] = exp2_approx(sc[gg] - ms);
                l[gg] = l[gg] * alpha + row16_sum(p[gg]);
                o[gg][0] *= alpha;
                o[gg][1] *= alpha;
                m[gg] = mn;
            }
#pragma unroll
            for (int t = 0; t < kPage; ++t) {
                const float v0 = bf16_lo(vw[t].w[0]), v1 = bf16_hi(vw[t].w[0]);
#pragma unroll
                for (int gg = 0; gg < GT; ++gg) {
                    const float pt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[gg]), t));
                    o[gg][0] = fmaf(pt, v0, o[gg][0]);
                    o[gg][1] = fmaf(pt, v1, o[gg][1]);
                }
            }
        };
        Words<4> kb[DEPTH][KSTEPS];
        Words<1> vb[DEPTH][kPage];
#pragma unroll
        for (int k = 0; k < DEPTH; ++k)
            if (k < npw) issue(wave + 4 * k, kb[k], vb[k]);
        for (int i0 = 0; i0 < npw; i0 += DEPTH) {
#pragma unroll
            for (int k = 0; k < DEPTH; ++k) {
                const int i = i0 + k;
                if (i < npw) {
                    consume(wave + 4 * i, kb[k], vb[k]);
                    if (i + DEPTH < npw) issue(wave + 4 * (i + DEPTH), kb[k], vb[k]);
                }
            }
        }

        // wavefronts -> workgroup: the common max, then each wavefront's
        // rescaled state to LDS; every thread then sums two channels over
        // the four wavefronts
        if (wl == 0 && worker) {
#pragma unroll
            for (int gg = 0; gg < GT; ++gg) s_red[wave][gg] = m[gg];
        }
        __syncthreads();
        if (worker) {
#pragma unroll
            for (int gg = 0; gg < GT; ++gg) {
                float M = s_red[0][gg];
#pragma unroll
                for (int w = 1; w < 4; ++w) M = fmaxf(M, s_red[w][gg]);
                const float f = m[gg] == NEG ? 0.0f : exp2_approx(m[gg] - M);
                *reinterpret_cast<float2*>(&s_o[wave][gg][2 * wl]) = make_float2(o[gg][0] * f, o[gg][1] * f);
                if (wl == 0) s_l[wave][gg] = l[gg] * f;
            }
        }
        __syncthreads();
    }

    // This workgroup's share of (b, h), per (query head, channel pair): the
    // wavefront sums from LDS, or an empty partial (m = -inf) when the workgroup is
    // in the selected range but all of its pages are empty.
    const bool fused = arrive != nullptr;
    const bool holds = p0 < total;                      // active implies holds
    const int nact = fast_div(total + ppw - 1, ppw, ppw_magic);   // workgroups holding pages of (b, h)
    if (holds) {
        for (int idx = 2 * (int)threadIdx.x; idx < GT * D; idx += 2 * (int)blockDim.x) {
            const int gg = idx / D, d = idx - gg * D;
            if (gg >= g.G) continue;
            float2 acc = make_float2(0.0f, 0.0f);
            float mg = NEG, ls = 0.0f;
            if (active) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float2 v = *reinterpret_cast<const float2*>(&s_o[r][gg][d]);
                    acc.x += v.x;
                    acc.y += v.y;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) ls += s_l[r][gg];
                mg = s_red[0][gg];
#pragma unroll
                for (int w = 1; w < 4; ++w) mg = fmaxf(mg, s_red[w][gg]);
            }
            const int64_t bi = (int64_t)b * g.Hq + h * g.G + gg;
            const int64_t prow = bi * splits + split;
            if (fused && nact == 1) {
                write_output(out, lse, bi, d, acc, mg, ls, D);        // the only workgroup of (b, h)
            } else if (fused) {
                store2_agent(part_o + prow * D + d, acc.x, acc.y);
                if (d == 0) store2_agent(part_ml + prow * 2, mg, ls);
            } else {
                *reinterpret_cast<float2*>(part_o + prow * D + d) = acc;
                if (d == 0) {
                    part_ml[prow * 2 + 0] = mg;
                    part_ml[prow * 2 + 1] = ls;
                }
            }
        }
    } else if (fused && total == 0 && split == 0) {
        // nothing selected for (b, h): zero output, lse = -inf
        for (int idx = 2 * (int)threadIdx.x; idx < GT * D; idx += 2 * (int)blockDim.x) {
            const int gg = idx / D, d = idx - gg * D;
            if (gg < g.G)
                write_output(out, lse, (int64_t)b * g.Hq + h * g.G + gg, d, make_float2(0.0f, 0.0f), NEG, 0.0f, D);
        }
    }
    if (!fused || !holds || nact == 1) return;

    // Hand-off: partials are written with agent-scope (L2 write-through)
    // stores; once every thread's stores have completed, one agent-scope
    // atomic counts the arrival.  The last of the nact workgroups resets the
    // counter for the next call and merges, reading with agent-scope loads.
    __shared__ int s_last;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = __hip_atomic_fetch_add(arrive + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == nact - 1;
        if (prev == nact - 1) __hip_atomic_store(arrive + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    constexpr int MB = ABS_DECODE_MERGE_BATCH;   // partials per merge pass
    for (int idx = 2 * (int)threadIdx.x; idx < GT * D; idx += 2 * (int)blockDim.x) {
        const int gg = idx / D, d = idx - gg * D;
        if (gg >= g.G) continue;
        const int64_t bi = (int64_t)b * g.Hq + h * g.G + gg;
        const float* ml = part_ml + bi * splits * 2;
        const float* po = part_o + bi * splits * D + d;
        float mg = NEG, ls = 0.0f;
        float2 acc = make_float2(0.0f, 0.0f);
        for (int s0 = 0; s0 < nact; s0 += MB) {
            // 2 MB loads in flight (indices clamped, so no load waits on a
            // branch), then one max and one weighted sum over the MB splits
            float2 mlv[MB], ov[MB];
#pragma unroll
            for (int k = 0; k < MB; ++k) {
                const int sk = min(s0 + k, nact - 1);
                mlv[k] = load2_agent(ml + 2 * sk);
                ov[k] = load2_agent(po + (int64_t)sk * D);
            }
            float bm = NEG;
#pragma unroll
            for (int k = 0; k < MB; ++k)
                if (s0 + k < nact) bm = fmaxf(bm, mlv[k].x);
            const float mn = fmaxf(mg, bm);
            if (mn == NEG) continue;                      // only empty partials so far
            const float a = mg == NEG ? 0.0f : exp2f(mg - mn);
            ls *= a;
            acc.x *= a;
            acc.y *= a;
#pragma unroll
            for (int k = 0; k < MB; ++k) {
                const float w = s0 + k < nact ? exp2f(mlv[k].x - mn) : 0.0f;   // empty partial: m = -inf, w = 0
                ls = fmaf(mlv[k].y, w, ls);
                acc.x = fmaf(ov[k].x, w, acc.x);
                acc.y = fmaf(ov[k].y, w, acc.y);
            }
            mg = mn;
        }
        write_output(out, lse, bi, d, acc, mg, ls, D);
    }
}

// The selection read from sel / sel_count (abs_sparse_decode).
template <int GT>
__global__ __launch_bounds__(256, 2) void k_sparse_decode_ws(Geom g, const uint16_t* __restrict__ q,
                                                             const int32_t* __restrict__ sel, int sel_cap,
                                                             const int32_t* __restrict__ count, float qscale,
                                                             float* __restrict__ part_ml, float* __restrict__ part_o,
                                                             int splits, int ppw, uint32_t ppw_magic,
                                                             int32_t* __restrict__ arrive,
                                                             uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int bh = blockIdx.y;
    int b, h;
    split_bh(g, bh, b, h);
    const int sh = block_shift_of(g, h) - 4;
    const int gp = blockIdx.x * ppw + (int)(threadIdx.x & 63);
    const int sv = sel[(int64_t)bh * sel_cap + min(gp >> sh, sel_cap - 1)];   // unconditional, clamped
    const int K = min(max(count[bh], 0), sel_cap);
    ws_decode<GT, 4>(g, q, seq_len(g, b), sv, K, sel_cap, qscale, part_ml, part_o, splits, ppw, ppw_magic, arrive,
                     out, lse);
}

// Top-K and decode in one launch (abs_select_decode): every split workgroup
// of (b, h) runs the head's top-K over the score row itself (topk.hpp, 512
// threads of KPT keys, as the top-K launch), keeps in LDS the selected blocks
// at the positions its pages cover, and decodes them with wavefronts 0-3;
// split 0 also writes sel and sel_count.  The workgroups of a head compute
// the same selection from the same row.
template <int NT, int GT, int KPT>
__global__ __launch_bounds__(NT) void k_select_decode_ws(Geom g, const float* __restrict__ scores, int stride,
                                                          const float2* __restrict__ ranges, int range_stride,
                                                          int max_len, int budget, int32_t* __restrict__ sel,
                                                          int sel_cap, int32_t* __restrict__ count,
                                                          const uint16_t* __restrict__ q, float qscale,
                                                          float* __restrict__ part_ml, float* __restrict__ part_o,
                                                          int splits, int ppw, uint32_t ppw_magic,
                                                          int32_t* __restrict__ arrive,
                                                          uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int split = blockIdx.x;
    const int bh = blockIdx.y;
    int b, h;
    split_bh(g, bh, b, h);
    const int sb = block_shift_of(g, h);
    const int sh = sb - 4;
    const int first = (split * ppw) >> sh;            // selection positions first .. first + 63 (ppw <= 64)
    __shared__ int32_t s_blk[kMaxPagesPerWg];
    int32_t* row_out = sel + (int64_t)bh * sel_cap;
    auto emit = [&](uint32_t p, int32_t j) {
        if (split == 0 && p < (uint32_t)sel_cap) row_out[p] = j;
        const uint32_t r = p - (uint32_t)first;
        if (r < (uint32_t)kMaxPagesPerWg) s_blk[r] = j;
    };
    // keys per thread for this head's longest row (up to KPT, the layer's):
    // heads with larger blocks finish their top-K sooner
    const float* srow = scores + (int64_t)bh * stride;
    const float2* rrow = ranges + (int64_t)bh * range_stride;
    const int nh = shr_ceil(max_len, sb);
    int K, L;
    constexpr int K4 = KPT >= 16 ? KPT / 4 : KPT, K2 = KPT >= 8 ? KPT / 2 : KPT;
    if (KPT > K4 && nh <= NT * K4)
        K = topk_rows<NT, K4>(g, bh, srow, stride, rrow, max_len, budget, emit, L);
    else if (KPT > K2 && nh <= NT * K2)
        K = topk_rows<NT, K2>(g, bh, srow, stride, rrow, max_len, budget, emit, L);
    else
        K = topk_rows<NT, KPT>(g, bh, srow, stride, rrow, max_len, budget, emit, L);
    if (split == 0 && threadIdx.x == 0) count[bh] = K;
    __syncthreads();
    const int gp = split * ppw + (int)(threadIdx.x & 63);
    const int sv = s_blk[min(max((gp >> sh) - first, 0), kMaxPagesPerWg - 1)];   // positions >= K: unused
    ws_decode<GT, NT / 64>(g, q, L, sv, min(K, sel_cap), sel_cap, qscale, part_ml, part_o, splits, ppw,
                           ppw_magic, arrive, out, lse);
}

// One workgroup per (b, query head): merge the partials of the splits that
// held pages of (b, h).  Thread (group sg, channel d) folds splits sg,
// sg + NG, ... with an online max/sum (its loads are independent, so they are
// all in flight together); the NG groups are then combined through LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_decode_merge(Geom g, const int32_t* __restrict__ count, int sel_cap,
                                                      int ppw, int splits, const float* __restrict__ part_ml,
                                                      const float* __restrict__ part_o, T* __restrict__ out,
                                                      float* __restrict__ lse) {
    constexpr float NEG = -__builtin_inff();
    constexpr int NG = 256 / D;
    const int bi = blockIdx.x;                       // b * Hq + query head
    const int b = bi / g.Hq, head = bi - b * g.Hq;
    const int h = head / g.G;
    const int bh = b * g.Hkv + h;
    const int spb = block_size_of(g, h) / kPage;
    const int K = min(max(count[bh], 0), sel_cap);
    const int total = min(K * spb, splits * ppw);
    const int nact = max(1, ceil_div(total, ppw));
    const int d = threadIdx.x % D, sg = threadIdx.x / D;
    const float* ml = part_ml + (int64_t)bi * splits * 2;
    const float* po = part_o + (int64_t)bi * splits * D + d;

    float m = NEG, ls = 0.0f, acc = 0.0f;
#pragma unroll 8
    for (int s = sg; s < nact; s += NG) {
        const float ms = ml[2 * s];
        const float lv = ml[2 * s + 1];
        const float ov = po[(int64_t)s * D];
        if (ms != NEG) {
            const float mn = fmaxf(m, ms);
            const float a = m == NEG ? 0.0f : exp2f(m - mn);
            const float w = exp2f(ms - mn);
            ls = ls * a + lv * w;
            acc = acc * a + ov * w;
            m = mn;
        }
    }
    __shared__ float s_m[NG][D], s_l[NG][D], s_a[NG][D];
    s_m[sg][d] = m;
    s_l[sg][d] = ls;
    s_a[sg][d] = acc;
    __syncthreads();
    if (sg != 0) return;
    float M = s_m[0][d];
#pragma unroll
    for (int i = 1; i < NG; ++i) M = fmaxf(M, s_m[i][d]);
    float lsum = 0.0f, o = 0.0f;
    if (M != NEG) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            if (s_m[i][d] == NEG) continue;
            const float w = exp2f(s_m[i][d] - M);
            lsum += s_l[i][d] * w;
            o += s_a[i][d] * w;
        }
    }
    Elem<T>::store1(out + (int64_t)bi * D + d, lsum > 0.0f ? o / lsum : 0.0f);
    if (lse != nullptr && d == 0) lse[bi] = lsum > 0.0f ? (M + log2f(lsum)) * kLn2 : NEG;
}

// One split launch: 256 * RG threads per workgroup, as the kernel assumes.
template <typename T, int D, int GT, int CH, bool PIPE, bool MF, int RG>
void launch_split(dim3 grid, const Geom& g, const DecodeArgs& a, float qscale, hipStream_t s) {
    constexpr int kThreads = 256 * RG;
    hipLaunchKernelGGL((k_sparse_decode<T, D, GT, CH, PIPE, MF, RG>), grid, dim3(kThreads), 0, s, g,
                       reinterpret_cast<const T*>(a.q), a.sel, a.sel_cap, a.count, qscale, a.part_ml, a.part_o,
                       a.splits, a.pages_per_wg, a.ppw_magic, a.arrive, reinterpret_cast<T*>(a.out), a.lse);
}

template <typename T, int D, int GT>
hipError_t decode_gt(const Geom& g, const DecodeArgs& a, hipStream_t s) {
    const dim3 grid(a.splits, g.B * g.Hkv);
    const float qscale = a.sm_scale * kLog2e;
    T* out = reinterpret_cast<T*>(a.out);
    constexpr bool kMatrix = ABS_DECODE_MATRIX && sizeof(T) == 2;   // bf16: q.k on the matrix cores
    constexpr int kRowGroups = kMatrix ? ABS_DECODE_ROWGROUPS : 1;
    // (a pipelined plan on a variant that does not fit runs the plain 8-page loop)
    // (fp32 rows of 8 query heads at D = 128 hold at most 4 pages at once)
    constexpr bool kWide = sizeof(T) == 4 && D * GT >= 1024;
    // bf16, D = 128, up to 4 query heads per group: the wavefront-split kernel
    // (at 8 heads its per-lane state outgrows the plain matrix-core kernel's)
    constexpr bool kWaveSplit = kMatrix && D == 128 && GT <= 4;
    if (ABS_DECODE_WAVES && kWaveSplit && (a.pipelined || a.chunk == 8)) {
        if constexpr (kWaveSplit)
            hipLaunchKernelGGL((k_sparse_decode_ws<GT>), grid, dim3(256), 0, s, g,
                               reinterpret_cast<const uint16_t*>(a.q), a.sel, a.sel_cap, a.count, qscale, a.part_ml,
                               a.part_o, a.splits, a.pages_per_wg, a.ppw_magic, a.arrive,
                               reinterpret_cast<uint16_t*>(a.out), a.lse);
    } else if (a.pipelined && kPipeFits<T, D, GT>) {
        if constexpr (kPipeFits<T, D, GT>) launch_split<T, D, GT, 8, true, kMatrix, kRowGroups>(grid, g, a, qscale, s);
    } else if ((a.chunk == 8 || a.pipelined) && !kWide) {
        if constexpr (!kWide) launch_split<T, D, GT, 8, false, kMatrix, 1>(grid, g, a, qscale, s);
    } else {
        switch (a.chunk) {
            case 1: launch_split<T, D, GT, 1, false, false, 1>(grid, g, a, qscale, s); break;
            case 2: launch_split<T, D, GT, 2, false, false, 1>(grid, g, a, qscale, s); break;
            default: launch_split<T, D, GT, 4, false, false, 1>(grid, g, a, qscale, s); break;
        }
    }
    if (a.arrive == nullptr)
        hipLaunchKernelGGL((k_decode_merge<T, D>), dim3(g.B * g.Hq), dim3(256), 0, s, g, a.count, a.sel_cap,
                           a.pages_per_wg, a.splits, a.part_ml, a.part_o, out, a.lse);
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

// The fused form covers the layers the wavefront-split decode serves (the
// same conditions as in decode_gt) whose heads have at most 512 x 32 blocks,
// and is used where it measured faster than the separate launches (every
// split workgroup repeats its head's top-K): heads of at most 6144 blocks on
// average, and either at most 4096 in every head or a split grid that fits
// the 256 compute units once.  Measured against the separate launches at
// 4 x 128K / 256K: drawn map (one head at block size 16) -1.1 / -0.7 us per
// step, every head at 16: +0.3 / +1.7 us; 16 x 128K (512 workgroups): +0.6.
// (The compute units are the device's, read at run time.)
bool select_decode_fusable(const Geom& g, DType dt, const SelectArgs& s, const DecodeArgs& a) {
    const bool served = ABS_DECODE_WAVES && ABS_DECODE_MATRIX && dt == DType::BF16 && g.D == 128 && g.G <= 4 &&
                        (a.pipelined || a.chunk == 8) && a.arrive != nullptr && s.max_n <= kFusedTopkMaxN;
    // measured faster than the separate launches: heads of at most 4096
    // blocks; heads of at most 8192 with the split grid within two
    // workgroups per compute unit (128K x 16, and every head at 16-token
    // blocks at 128K: 1-2 us faster; 128K x 32, four per unit: no gain);
    // longer heads (a 16384-block head) with the grid within the compute
    // units and at most 6144 blocks per head on average (256K x 4 with one
    // 16-token head: 2 us faster; every head at 16384 blocks: no gain)
    const int64_t grid = (int64_t)a.splits * g.B * g.Hkv;
    const bool faster = s.max_n <= 4096 || (s.max_n <= 8192 && grid <= 2 * (int64_t)a.compute_units) ||
                        (grid <= a.compute_units && s.total_blocks <= (int64_t)6144 * g.B * g.Hkv);
    return served && faster;
}

namespace {

template <int NT, int GT, int KPT>
void launch_fused(const Geom& g, const SelectArgs& s, const DecodeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_select_decode_ws<NT, GT, KPT>), dim3(a.splits, g.B * g.Hkv), dim3(NT), 0, st, g, s.scores,
                       s.stride, s.ranges, s.range_stride, s.max_len, s.budget, s.sel, s.sel_cap, s.count,
                       reinterpret_cast<const uint16_t*>(a.q), a.sm_scale * kLog2e, a.part_ml, a.part_o, a.splits,
                       a.pages_per_wg, a.ppw_magic, a.arrive, reinterpret_cast<uint16_t*>(a.out), a.lse);
}

// Heads of at most kFusedSmallMaxN blocks: 256 threads (the decode's
// wavefronts alone), measured faster there (-0.4 to -0.8 us per step at
// 32K x 1, 32K x 16 and 64K x 8); larger heads: 512 threads, whose top-K the
// eight wavefronts share (1.2 us faster at 128K x 4, where one head has 8192
// blocks).
template <int GT>
void launch_fused_gt(const Geom& g, const SelectArgs& s, const DecodeArgs& a, hipStream_t st) {
    if (s.max_n <= 256 * 4) launch_fused<256, GT, 4>(g, s, a, st);
    else if (s.max_n <= 256 * 8) launch_fused<256, GT, 8>(g, s, a, st);
    else if (s.max_n <= kFusedSmallMaxN) launch_fused<256, GT, 16>(g, s, a, st);
    else if (s.max_n <= kFusedThreads * 16) launch_fused<kFusedThreads, GT, 16>(g, s, a, st);
    else launch_fused<kFusedThreads, GT, 32>(g, s, a, st);
}

}  // namespace

hipError_t launch_select_decode(const Geom& g, DType dt, const SelectArgs& s, const DecodeArgs& a, hipStream_t st) {
    if (!select_decode_fusable(g, dt, s, a)) return hipErrorInvalidValue;
    if (g.G <= 1) launch_fused_gt<1>(g, s, a, st);
    else if (g.G <= 2) launch_fused_gt<2>(g, s, a, st);
    else launch_fused_gt<4>(g, s, a, st);
    return hipGetLastError();
}

}  // namespace absk
