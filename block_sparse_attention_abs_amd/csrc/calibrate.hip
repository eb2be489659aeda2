// Small service kernels: the zero fill of a decode workspace's arrival
// counters, and the per-head recall for the offline block-size calibration (AB-Sparse page:
// Figure 3's normalized recall against block size, and the per-head
// block-size heatmap printed after it).
//
// The recall of a selection for query head i is the share of i's exact
// attention over all its tokens that the selection keeps.  Both softmax
// normalizers come out of abs_sparse_decode as log-sum-exps: lse_sel over
// the kept tokens and lse_full over every token (every block selected), so
// the share is exp(lse_sel - lse_full).  One wavefront per KV head averages
// it over the sequences and the head's query group, in fp64.
#include "device.hpp"

namespace absk {
namespace {

__global__ __launch_bounds__(64) void k_head_recall(int B, int Hq, int Hkv, const float* __restrict__ lse_sel,
                                                    const float* __restrict__ lse_full, float* __restrict__ recall) {
    const int h = blockIdx.x;
    const int G = Hq / Hkv;
    const int n = B * G;
    double acc = 0.0;
    for (int e = threadIdx.x; e < n; e += 64) {
        const int b = e / G, i = h * G + (e - (e / G) * G);
        const int64_t at = (int64_t)b * Hq + i;
        acc += exp((double)lse_sel[at] - (double)lse_full[at]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (threadIdx.x == 0) recall[h] = (float)(acc / (double)n);
}

__global__ __launch_bounds__(256) void k_zero(int32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_zero(int32_t* p, int n, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_zero, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_head_recall(int B, int Hq, int Hkv, const float* lse_sel, const float* lse_full, float* recall,
                              hipStream_t s) {
    hipLaunchKernelGGL(k_head_recall, dim3(Hkv), dim3(64), 0, s, B, Hq, Hkv, lse_sel, lse_full, recall);
    return hipGetLastError();
}

}  // namespace absk
