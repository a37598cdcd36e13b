// Shared device helpers for the libkda kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Device-side bounds checks, compiled only with -DKDA_DEVICE_CHECKS (the
// library's checked build): each kernel checks, at its work item's set-up,
// that the index ranges its accesses are derived from lie inside the
// buffers' extents; a failed check sets its bit in kda_check_bits (read back
// by kda_debug_check_bits) and the kernel carries on.  The release build
// compiles every check away.
enum CheckBit {
    CK_TOKENS = 0,   // a token range outside [0, T_total)
    CK_SEQ = 1,      // a sequence or state index outside [0, N)
    CK_WS = 2,       // a workspace index (segment, summary, flag) outside its plan's count
    CK_CKPT = 3,     // a checkpoint row read outside [0, capacity)
    CK_BLOCK = 4,    // a block or sub-chunk length outside [1, its size]
};
#ifdef KDA_DEVICE_CHECKS
__device__ unsigned int kda_check_bits;
#define KDA_CHECK(cond, bit)                                                        \
    do {                                                                            \
        if (!(cond)) atomicOr(&::kda::kda_check_bits, 1u << (unsigned)(::kda::bit)); \
    } while (0)
#else
#define KDA_CHECK(cond, bit) \
    do {                     \
    } while (0)
#endif

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// ---- bf16 <-> fp32 (bit exact; fp32 -> bf16 rounds to nearest even in hardware)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    f32x2 v = {a, b};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a)
{
    return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// Token-tensor element type tags.
struct F32 {
    using storage = float;
    static constexpr bool is_bf16 = false;
};
struct BF16 {
    using storage = uint16_t;
    static constexpr bool is_bf16 = true;
};

template <typename DT>
__device__ __forceinline__ float load_elem(const typename DT::storage* p, int64_t i)
{
    if constexpr (DT::is_bf16) return bf16_to_f32(p[i]);
    else return p[i];
}
template <typename DT>
__device__ __forceinline__ void store_elem(typename DT::storage* p, int64_t i, float x)
{
    if constexpr (DT::is_bf16) p[i] = f32_to_bf16(x);
    else p[i] = x;
}

// Eight consecutive elements (16-byte aligned for bf16, 32-byte pair of float4 for f32).
template <typename DT>
__device__ __forceinline__ void load8(const typename DT::storage* p, float (&x)[8])
{
    if constexpr (DT::is_bf16) {
        u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w[i]);
            x[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
        f32x4 a = *reinterpret_cast<const f32x4*>(p);
        f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = a[i];
            x[4 + i] = b[i];
        }
    }
}
// Stores are streaming (non-temporal) when NT: the data is not kept in the
// caches on its way to HBM.
template <typename T, bool NT>
__device__ __forceinline__ void store_vec(T* p, const T& v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}
template <typename DT, bool NT = false>
__device__ __forceinline__ void store8(typename DT::storage* p, const float (&x)[8])
{
    if constexpr (DT::is_bf16) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        store_vec<u32x4, NT>(reinterpret_cast<u32x4*>(p), w);
    } else {
        f32x4 a = {x[0], x[1], x[2], x[3]};
        f32x4 b = {x[4], x[5], x[6], x[7]};
        store_vec<f32x4, NT>(reinterpret_cast<f32x4*>(p), a);
        store_vec<f32x4, NT>(reinterpret_cast<f32x4*>(p + 4), b);
    }
}

// The gate g = g_min sigmoid(e^{A_h} z) ("NLP——技术报告解读-Kimi-K3", Model
// Architecture / Kimi Delta Attention (KDA), lower-bounded decay), fused into
// a kernel that consumes g: g = g_min / (1 + 2^{s2 z}) with
// s2 = -e^{A_h} log2(e), in fp32 (hardware exp2 and reciprocal), so the decay
// input never goes through HBM as g.  Off, it passes its argument through.
struct GateZ {
    bool on;
    float s2, g_min;
    __device__ __forceinline__ float operator()(float z) const
    {
        return on ? g_min * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(s2 * z)) : z;
    }
    // the gate of head h, or the identity when A is null
    static __device__ __forceinline__ GateZ of_head(const float* A, int h, float g_min)
    {
        GateZ gz{A != nullptr, 0.f, g_min};
        if (gz.on) gz.s2 = -__expf(A[h]) * 1.4426950408889634f;
        return gz;
    }
};

}  // namespace kda
