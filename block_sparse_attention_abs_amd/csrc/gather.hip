// Measurement: the decode's K/V gather without its arithmetic.
//
// The split decode reads, for every selected page of a head, the page's K
// tile and V tile: [page][kv head][16][head_dim] storage, 4 KiB per tile for
// bf16 and head_dim 128, scattered over the cache as the page table places
// them.  k_gather_tiles reads a list of such tiles at the device addresses
// it is given, with the same non-temporal 16-byte loads, U tiles in flight
// per wavefront and nothing between the loads but an XOR of the words (so
// no load is dead).  Timed over the tiles one decode step selects, it is the
// rate at which this GPU gathers those bytes with no dependent chain before
// or after them: the reference for the decode's page loop.
//
// Wavefront w reads tiles [w * per_wave, (w + 1) * per_wave) of the list in
// runs of 64, lane l holding the address of the run's tile l; each tile is
// read by the whole wavefront, 16 bytes per lane per load, four loads (1 KiB
// per wavefront each).  Workgroup g writes the XOR of all the 32-bit words
// its four wavefronts read to out[g].
#include "device.hpp"

namespace absk {
namespace {

constexpr int kTileBytes = 4096;
constexpr int kLoadsPerTile = kTileBytes / (64 * 16);

template <int U>
__global__ __launch_bounds__(256) void k_gather_tiles(const uint64_t* __restrict__ addr, int n, int per_wave,
                                                      uint32_t* __restrict__ out) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    const int64_t first = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * per_wave;
    const int64_t mine = min((int64_t)per_wave, max((int64_t)n - first, (int64_t)0));   // tiles of this wavefront
    uint32_t acc = 0;
    for (int64_t r0 = 0; r0 < mine; r0 += 64) {
        const int cnt = (int)min((int64_t)64, mine - r0);            // >= 1
        const uint64_t a = addr[first + r0 + min(lane, cnt - 1)];
        const uint32_t a_lo = (uint32_t)a, a_hi = (uint32_t)(a >> 32);
        for (int i = 0; i < cnt; i += U) {
            u32x4 v[U][kLoadsPerTile];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (i + u < cnt) {                                    // the run's last slots load nothing
                    // both halves as unsigned: readlane returns int, and a sign-extended
                    // low half would set every bit of the high half
                    const uint64_t t = (uint64_t)(uint32_t)__builtin_amdgcn_readlane(a_lo, i + u) |
                                       ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(a_hi, i + u) << 32);
                    const u32x4* p = reinterpret_cast<const u32x4*>(t) + lane;
#pragma unroll
                    for (int s = 0; s < kLoadsPerTile; ++s) v[u][s] = __builtin_nontemporal_load(p + s * 64);
                } else {
#pragma unroll
                    for (int s = 0; s < kLoadsPerTile; ++s) v[u][s] = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int s = 0; s < kLoadsPerTile; ++s) acc ^= v[u][s].x ^ v[u][s].y ^ v[u][s].z ^ v[u][s].w;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    __shared__ uint32_t s_acc[4];
    if (lane == 0) s_acc[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

}  // namespace

hipError_t launch_gather_tiles(const uint64_t* addr, int n, int workgroups, int in_flight, uint32_t* out,
                               hipStream_t s) {
    const int64_t waves = (int64_t)workgroups * 4;
    const int per_wave = (int)((n + waves - 1) / waves);
#define ABS_GATHER(U_) hipLaunchKernelGGL(k_gather_tiles<U_>, dim3(workgroups), dim3(256), 0, s, addr, n, per_wave, out)
    if (in_flight == 1) ABS_GATHER(1);
    else if (in_flight == 2) ABS_GATHER(2);
    else if (in_flight == 4) ABS_GATHER(4);
    else ABS_GATHER(8);
#undef ABS_GATHER
    return hipGetLastError();
}

}  // namespace absk
