// libkda_roofs: measurement kernels for the rooflines the benchmark reports
// against (not part of libkda's path).  Each entry point times its own
// launches with HIP events on the given stream and returns the mean
// milliseconds per launch; the caller turns that into GB/s or TFLOP/s.
//   kda_roof_stream : read, write, copy or in-place update of a device
//                     buffer with 16-byte vector accesses: grid-stride over a
//                     given number of workgroups, or one vector per thread.
//   kda_roof_state_inplace : in-place update of 64 KB fp32 states in the
//                     decode step's access pattern (the read + write roof of
//                     a working set of the decode step's size).
//   kda_roof_mfma   : back-to-back independent 16x16x32 bf16 matrix-core
//                     instructions on every SIMD (the issue ceiling of the
//                     instruction the prefill's products use).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "kda_roofs.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// Grid-stride over `n` 16-byte vectors, four in flight per thread.  Mode 0:
// read (each thread folds what it reads into one word, written once per
// thread so the loads cannot be dropped), 1: write, 2: copy, 3: in place
// (each word + 1, written back where it was read).
template <int MODE>
__global__ void __launch_bounds__(256) stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t n, uint32_t* __restrict__ sink)
{
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {  // four independent vectors in flight per thread
        if constexpr (MODE == 1) {
            const u32x4 w = {uint32_t(i), 0u, 0u, 0u};
            dst[i] = w;
            dst[i + stride] = w;
            dst[i + 2 * stride] = w;
            dst[i + 3 * stride] = w;
        } else {
            const u32x4* in = MODE == 3 ? dst : src;
            const u32x4 a = in[i], b = in[i + stride], c = in[i + 2 * stride], d = in[i + 3 * stride];
            if constexpr (MODE == 0) {
                acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
                acc ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
            } else {
                const uint32_t inc = MODE == 3 ? 1u : 0u;
                dst[i] = a + inc;
                dst[i + stride] = b + inc;
                dst[i + 2 * stride] = c + inc;
                dst[i + 3 * stride] = d + inc;
            }
        }
    }
    for (; i < n; i += stride) {
        if constexpr (MODE == 1) {
            dst[i] = u32x4{uint32_t(i), 0u, 0u, 0u};
        } else {
            const u32x4 a = (MODE == 3 ? dst : src)[i];
            if constexpr (MODE == 0) acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
            else dst[i] = MODE == 3 ? a + 1u : a;
        }
    }
    if constexpr (MODE == 0) sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

// One 16-byte vector per thread, the grid covering all `n` (modes 1-3 as
// above): every load of a workgroup is in flight at once.
template <int MODE>
__global__ void __launch_bounds__(256) tile_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n)
{
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    if constexpr (MODE == 1) dst[i] = u32x4{uint32_t(i), 0u, 0u, 0u};
    else if constexpr (MODE == 2) dst[i] = src[i];
    else dst[i] = dst[i] + 1u;
}

// In place over 64 KB blocks laid out as 128 x 128 fp32 states, in the
// decode step's access pattern: a workgroup per block, wave w = 32 columns,
// lane = (row group of 16 rows, 4 columns); all 16 loads of a
// lane in flight, then `delay` rounds of dependent arithmetic on the values,
// then 16 streaming stores.  The delay spreads the workgroups' write bursts
// apart from their read bursts (it is what the decode step's own arithmetic
// does); the caller sweeps it.
__global__ void __launch_bounds__(256) state_inplace_kernel(float* __restrict__ x, int delay)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int cgl = lane & 7, rg = lane >> 3;
    float* S = x + int64_t(blockIdx.x) * 128 * 128 + w * 32 + 4 * cgl;
    f32x4 v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = *reinterpret_cast<const f32x4*>(S + (rg * 16 + r) * 128);
    for (int d = 0; d < delay; ++d) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = v[r] * 0.999f + 0.001f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) __builtin_nontemporal_store(v[r] + 1.f, reinterpret_cast<f32x4*>(S + (rg * 16 + r) * 128));
}

// Each wave keeps NACC independent accumulators and issues ITERS rounds of
// NACC matrix instructions; the results are folded into one word per lane so
// nothing is dead code.
constexpr int NACC = 8;
__global__ void __launch_bounds__(256) mfma_kernel(int iters, float* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * float(lane + e));
        b[e] = (__bf16)(0.002f * float(lane - e));
    }
    f32x4 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// Mean milliseconds per launch of `reps` back-to-back launches of `launch`
// on stream s, between two events; 0 on success, 2 on a HIP error.
template <typename F>
int timed(F&& launch, int reps, hipStream_t s, float* ms_per_launch)
{
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    if (e == hipSuccess) {
        for (int r = 0; r < reps; ++r) launch();
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (e != hipSuccess) return 2;
    *ms_per_launch = ms / float(reps);
    return 0;
}

}  // namespace

extern "C" {

int kda_roof_stream(int mode, const void* src, void* dst, int64_t bytes, void* sink, int64_t sink_words,
                    int workgroups, int reps, void* stream, float* ms_per_launch)
{
    if (mode < 0 || mode > 3 || bytes < 16 || bytes % 16 != 0 || workgroups < 0 || reps < 1 || !ms_per_launch)
        return 1;
    if (workgroups == 0 && (mode == 0 || bytes / 16 > int64_t(0x7fffffff) * 256)) return 1;
    if ((mode == 0 || mode == 2) && !src) return 1;
    if (mode != 0 && !dst) return 1;
    if (mode == 0 && (!sink || sink_words < int64_t(workgroups) * 256)) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = bytes / 16;
    const u32x4* in = static_cast<const u32x4*>(src);
    u32x4* out = static_cast<u32x4*>(dst);
    uint32_t* sk = static_cast<uint32_t*>(sink);
    const unsigned tiles = unsigned((n + 255) / 256);
    auto launch = [&]() {
        if (workgroups == 0) {
            if (mode == 1) hipLaunchKernelGGL(tile_kernel<1>, dim3(tiles), dim3(256), 0, s, in, out, n);
            else if (mode == 2) hipLaunchKernelGGL(tile_kernel<2>, dim3(tiles), dim3(256), 0, s, in, out, n);
            else hipLaunchKernelGGL(tile_kernel<3>, dim3(tiles), dim3(256), 0, s, in, out, n);
        } else if (mode == 0) {
            hipLaunchKernelGGL(stream_kernel<0>, dim3(workgroups), dim3(256), 0, s, in, out, n, sk);
        } else if (mode == 1) {
            hipLaunchKernelGGL(stream_kernel<1>, dim3(workgroups), dim3(256), 0, s, in, out, n, sk);
        } else if (mode == 2) {
            hipLaunchKernelGGL(stream_kernel<2>, dim3(workgroups), dim3(256), 0, s, in, out, n, sk);
        } else {
            hipLaunchKernelGGL(stream_kernel<3>, dim3(workgroups), dim3(256), 0, s, in, out, n, sk);
        }
    };
    launch();  // first launch loads the code object
    if (hipGetLastError() != hipSuccess) return 2;
    return timed(launch, reps, s, ms_per_launch);
}

int kda_roof_state_inplace(void* buf, int64_t bytes, int delay, int reps, void* stream, float* ms_per_launch)
{
    if (!buf || bytes < 65536 || bytes % 65536 != 0 || bytes / 65536 > int64_t(0x7fffffff) || delay < 0 ||
        delay > 4096 || reps < 1 || !ms_per_launch)
        return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* x = static_cast<float*>(buf);
    const unsigned blocks = unsigned(bytes / 65536);
    auto launch = [&]() { hipLaunchKernelGGL(state_inplace_kernel, dim3(blocks), dim3(256), 0, s, x, delay); };
    launch();
    if (hipGetLastError() != hipSuccess) return 2;
    return timed(launch, reps, s, ms_per_launch);
}

int kda_roof_mfma(int workgroups, int iters, void* sink, void* stream, float* ms_per_launch, double* flops_per_launch)
{
    if (workgroups < 1 || iters < 1 || !sink || !ms_per_launch || !flops_per_launch) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* sk = static_cast<float*>(sink);
    auto launch = [&]() { hipLaunchKernelGGL(mfma_kernel, dim3(workgroups), dim3(256), 0, s, iters, sk); };
    launch();
    if (hipGetLastError() != hipSuccess) return 2;
    const int r = timed(launch, 1, s, ms_per_launch);
    if (r != 0) return r;
    // 4 waves per workgroup, NACC instructions per round, 16*16*32 multiply-adds each
    *flops_per_launch = double(workgroups) * 4.0 * double(iters) * NACC * 2.0 * 16 * 16 * 32;
    return 0;
}

}  // extern "C"
