// kda_gate: g = g_min * sigmoid(exp(A_h) * z), elementwise over [T, H, d_k].
//
// Source: "NLP——技术报告解读-Kimi-K3", Model Architecture / Kimi Delta
// Attention (KDA), lower-bounded decay (scaled sigmoid replacing the negative
// softplus, g_min = -5); "Kimi K3 技术报告 · 大白话版" §2.1.1 (at most 99.33%
// forgotten per step).
//
// g may alias z (in place); each element is read before it is written by the
// same thread.  HBM-bound streaming kernel: 8 elements per thread per iteration with 16-byte
// (bf16) or 2x16-byte (fp32) accesses, grid-stride so one launch of a few
// thousand workgroups covers any size.  Computed in fp32, rounded once; g is
// written with streaming (non-temporal) stores.
#pragma once

#include "kda_common.hpp"

namespace kda {

__device__ __forceinline__ float gate_value(float z, float scale, float g_min)
{
    // g_min / (1 + e^{-x}); for x -> -inf the denominator is +inf and g -> -0.
    const float x = scale * z;
    return g_min / (1.0f + __expf(-x));
}

template <typename DT>
__global__ void __launch_bounds__(256) gate_kernel_vec8(const typename DT::storage* z,
                                                        const float* __restrict__ A,
                                                        typename DT::storage* g,
                                                        int64_t n_groups, int H, int dk, float g_min)
{
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t grp = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; grp < n_groups;
         grp += stride) {
        const int64_t e0 = grp * 8;
        float x[8];
        load8<DT>(z + e0, x);
        // d_k is a multiple of 8 here, so all 8 elements share one head.
        const int h = int((e0 / dk) % H);
        const float s = __expf(A[h]);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = gate_value(x[i], s, g_min);
        store8<DT, true>(g + e0, x);
    }
}

template <typename DT>
__global__ void __launch_bounds__(256) gate_kernel_scalar(const typename DT::storage* z,
                                                          const float* __restrict__ A,
                                                          typename DT::storage* g,
                                                          int64_t n, int H, int dk, float g_min)
{
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) {
        const int h = int((e / dk) % H);
        store_elem<DT>(g, e, gate_value(load_elem<DT>(z, e), __expf(A[h]), g_min));
    }
}

template <typename DT>
hipError_t launch_gate(const void* z, const float* A, void* g, int64_t n_tokens, int H, int dk,
                       float g_min, hipStream_t stream)
{
    using S = typename DT::storage;
    const int64_t n = n_tokens * H * int64_t(dk);
    if (n == 0) return hipSuccess;
    const bool aligned = (reinterpret_cast<uintptr_t>(z) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(g) % 16 == 0) && (dk % 8 == 0);
    const int threads = 256;
    if (aligned) {
        const int64_t groups = n / 8;
        int64_t blocks = (groups + threads - 1) / threads;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(gate_kernel_vec8<DT>, dim3(unsigned(blocks)), dim3(threads), 0, stream,
                           static_cast<const S*>(z), A, static_cast<S*>(g), groups, H, dk, g_min);
    } else {
        int64_t blocks = (n + threads - 1) / threads;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(gate_kernel_scalar<DT>, dim3(unsigned(blocks)), dim3(threads), 0, stream,
                           static_cast<const S*>(z), A, static_cast<S*>(g), n, H, dk, g_min);
    }
    return hipGetLastError();
}

}  // namespace kda
