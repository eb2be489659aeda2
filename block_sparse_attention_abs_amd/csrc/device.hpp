// Device-side helpers shared by the gfx950 kernels of the AB-Sparse library:
// element conversion, wide loads, and reductions across the 16 lanes of a
// DPP row (a row of 16 lanes holds one cache row: 16 lanes x head_dim/16
// channels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace absk {

constexpr int kPage = 16;       // tokens per physical page
constexpr int kRowLanes = 16;   // lanes that share one cache row

// ---- element conversion ---------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// A run of NW 32-bit words loaded with the widest aligned loads available.
template <int NW>
struct Words {
    uint32_t w[NW];
};

template <int NW>
__device__ __forceinline__ Words<NW> load_words(const void* p) {
    Words<NW> r;
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            uint4 v = reinterpret_cast<const uint4*>(p)[i];
            r.w[4 * i + 0] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    } else if constexpr (NW == 2) {
        uint2 v = *reinterpret_cast<const uint2*>(p);
        r.w[0] = v.x;
        r.w[1] = v.y;
    } else {
        static_assert(NW == 1, "unsupported width");
        r.w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
    return r;
}

// Load from a wavefront-uniform base plus a per-lane unsigned byte offset
// (lets the compiler use scalar-base addressing: one VGPR per lane, not two).
template <int NW>
__device__ __forceinline__ Words<NW> load_words_at(const void* uniform_base, uint32_t byte_off) {
    return load_words<NW>(static_cast<const char*>(uniform_base) + byte_off);
}

// The same with non-temporal loads, for data read once per call (key and
// value pages, centroid codes): they are kept out of the caches' way.
template <int NW>
__device__ __forceinline__ Words<NW> load_words_stream(const void* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    Words<NW> r;
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
            r.w[4 * i + 0] = u.x;
            r.w[4 * i + 1] = u.y;
            r.w[4 * i + 2] = u.z;
            r.w[4 * i + 3] = u.w;
        }
    } else if constexpr (NW == 2) {
        const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        r.w[0] = u.x;
        r.w[NW - 1] = u.y;
    } else {
        static_assert(NW == 1, "1, 2 or a multiple of 4 words");
        r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    return r;
}

template <int NW>
__device__ __forceinline__ Words<NW> load_words_stream_at(const void* uniform_base, uint32_t byte_off) {
    return load_words_stream<NW>(static_cast<const char*>(uniform_base) + byte_off);
}

template <int NW>
__device__ __forceinline__ Words<NW> zero_words() {
    Words<NW> r;
#pragma unroll
    for (int i = 0; i < NW; ++i) r.w[i] = 0u;
    return r;
}

// Storage traits: element e of a Words run as fp32.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static constexpr int kBytes = 4;
    template <int NW>
    __device__ static __forceinline__ float get(const Words<NW>& w, int e) { return __uint_as_float(w.w[e]); }
    __device__ static __forceinline__ float load1(const float* p) { return *p; }
    __device__ static __forceinline__ float cvt(float v) { return v; }
    __device__ static __forceinline__ void store1(float* p, float v) { *p = v; }
};

template <>
struct Elem<uint16_t> {  // bf16 bit patterns
    static constexpr int kBytes = 2;
    template <int NW>
    __device__ static __forceinline__ float get(const Words<NW>& w, int e) {
        return (e & 1) ? bf16_hi(w.w[e >> 1]) : bf16_lo(w.w[e >> 1]);
    }
    __device__ static __forceinline__ float load1(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
    __device__ static __forceinline__ float cvt(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
    __device__ static __forceinline__ void store1(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16(v); }
};

// Partial dot product of one lane's run of a query row and a key row (raw
// storage words, fp32 result).  bf16: v_dot2c_f32_bf16 on packed pairs (exact
// products, fp32 accumulation, no unpacking); fp32: plain fma.
template <typename T, int NW>
__device__ __forceinline__ float dot_words(const Words<NW>& a, const Words<NW>& b);

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <>
__device__ __forceinline__ float dot_words<uint16_t, 2>(const Words<2>& a, const Words<2>& b) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w[i]),
                                              __builtin_bit_cast(bf16x2_t, b.w[i]), acc, false);
    return acc;
}

template <>
__device__ __forceinline__ float dot_words<uint16_t, 4>(const Words<4>& a, const Words<4>& b) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w[i]),
                                              __builtin_bit_cast(bf16x2_t, b.w[i]), acc, false);
    return acc;
}

template <>
__device__ __forceinline__ float dot_words<float, 4>(const Words<4>& a, const Words<4>& b) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(a.w[i]), __uint_as_float(b.w[i]), acc);
    return acc;
}

template <>
__device__ __forceinline__ float dot_words<float, 8>(const Words<8>& a, const Words<8>& b) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(__uint_as_float(a.w[i]), __uint_as_float(b.w[i]), acc);
    return acc;
}

// ---- cross-lane reductions --------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets the sum.
// quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v;
}

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
}

// Combine the four 16-lane rows of a wavefront (lanes l, l^16, l^32, l^48)
// with the gfx950 row swaps: v_permlane16_swap exchanges rows 0<->1 and
// 2<->3 between its two operands and v_permlane32_swap the two halves, so
// after a swap of (v, v) every lane holds {own value, partner's value}.
__device__ __forceinline__ float swap16_other_plus(float v, bool is_max) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    return is_max ? fmaxf(a, b) : a + b;
}

__device__ __forceinline__ float swap32_other_plus(float v, bool is_max) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    return is_max ? fmaxf(a, b) : a + b;
}

__device__ __forceinline__ float rows4_sum(float v) {
    return swap32_other_plus(swap16_other_plus(v, false), false);
}

__device__ __forceinline__ float rows4_max(float v) {
    return swap32_other_plus(swap16_other_plus(v, true), true);
}

__device__ __forceinline__ float rows4_min(float v) {
    return -rows4_max(-v);
}

// Whole-wavefront max (every lane gets it): DPP within rows, row swaps across.
__device__ __forceinline__ float wave_max(float v) { return rows4_max(row16_max(v)); }

// Max over each half of the wavefront (lanes 0-31, 32-63): the rows, then
// the swap of rows 0<->1 and 2<->3.
__device__ __forceinline__ float half32_max(float v) { return swap16_other_plus(row16_max(v), true); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);   // out-of-row lanes read 0
}

// Inclusive prefix sum over the 64 lanes: row_shr 1/2/4/8 inside each
// 16-lane row, then the totals of the rows below are added (readlane).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += dpp_u32<0x111>(x);   // row_shr:1
    x += dpp_u32<0x112>(x);   // row_shr:2
    x += dpp_u32<0x114>(x);   // row_shr:4
    x += dpp_u32<0x118>(x);   // row_shr:8
    const uint32_t t0 = __builtin_amdgcn_readlane(x, 15);
    const uint32_t t1 = t0 + __builtin_amdgcn_readlane(x, 31);
    const uint32_t t2 = t1 + __builtin_amdgcn_readlane(x, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return x + (row == 1 ? t0 : row == 2 ? t1 : row == 3 ? t2 : 0u);
}

// Sum over aligned groups of N lanes (N = 2, 4, 8 or 16), fp64: both halves
// of the double move with DPP -- quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror -- each step adding the partner group's sum.
template <int N>
__device__ __forceinline__ double lanes_sum_f64(double v) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16, "2, 4, 8 or 16 lanes");
    constexpr int kSteps = N == 2 ? 1 : N == 4 ? 2 : N == 8 ? 3 : 4;
#pragma unroll
    for (int step = 0; step < kSteps; ++step) {
        const uint64_t u = __double_as_longlong(v);
        const int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
        int lo2, hi2;
        if (step == 0) {
            lo2 = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, true);
            hi2 = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, true);
        } else if (step == 1) {
            lo2 = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, true);
            hi2 = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, true);
        } else if (step == 2) {
            lo2 = __builtin_amdgcn_mov_dpp(lo, 0x141, 0xF, 0xF, true);
            hi2 = __builtin_amdgcn_mov_dpp(hi, 0x141, 0xF, 0xF, true);
        } else {
            lo2 = __builtin_amdgcn_mov_dpp(lo, 0x140, 0xF, 0xF, true);
            hi2 = __builtin_amdgcn_mov_dpp(hi, 0x140, 0xF, 0xF, true);
        }
        v += __longlong_as_double((int64_t)(((uint64_t)(uint32_t)hi2 << 32) | (uint32_t)lo2));
    }
    return v;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace absk
