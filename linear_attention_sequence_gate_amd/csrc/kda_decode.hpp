// kda_decode_step: one token per (sequence, head) against a resident fp32
// state, updated in place.
//
// Source: "NLP——技术报告解读-Kimi-K3", Model Architecture / Kimi Delta
// Attention (KDA), state update and read-out; "Kimi K3 技术报告 · 大白话版"
// §2.1.1 (decay, then delta correction, then read) and §5.4 (decode updates
// the board in place token by token).
//
// Per (b, h), with alpha = exp(g) and D = Diag(alpha):
//   pk = (D S)^T k,  pq = (D S)^T q,  u = beta (v - pk)
//   S  <- D S + k u^T                       (written back in place)
//   o  = S_new^T q = pq + (k^T q) u
// which is the recurrence's single step rearranged so the state is read once
// and written once.  The step is HBM-bound (about 0.9 flop per byte), so the
// design is one streaming pass: one 256-thread workgroup per (b, h); thread t
// owns 4 consecutive value columns (a 16-byte slice of a state row) for
// d_k / (1024 / d_v) rows, so one wave's loads cover whole 512-byte rows.  The
// column sums over d_k are reduced through LDS; no atomics, so results are
// deterministic.  The state write-back is a streaming (non-temporal) store:
// measured on MI355X it lifts the in-place read+write stream from about 5.1
// to about 6.6 TB/s, while streaming loads do not help.
#pragma once

#include "kda_common.hpp"

namespace kda {

template <typename DT, int DK, int DV>
__global__ void __launch_bounds__(256) decode_kernel(const typename DT::storage* __restrict__ q,
                                                     const typename DT::storage* __restrict__ k,
                                                     const typename DT::storage* __restrict__ v,
                                                     const typename DT::storage* __restrict__ g,
                                                     const typename DT::storage* __restrict__ beta,
                                                     float* __restrict__ state,
                                                     typename DT::storage* __restrict__ o, int H,
                                                     const float* __restrict__ gate_A, float g_min)
{
    constexpr int CG = DV / 4;       // column groups of 4
    constexpr int RG = 256 / CG;     // row groups
    constexpr int R = DK / RG;       // rows per thread
    static_assert(R >= 1 && DK % RG == 0, "unsupported decode shape");

    __shared__ f32x4 red_pk[RG][CG];
    __shared__ f32x4 red_pq[RG][CG];
    __shared__ float red_kq[RG];

    const int bh = blockIdx.x;
    const int t = threadIdx.x;
    const int cg = t % CG;
    const int rg = t / CG;
    const int c0 = rg * R;

    // gate_A non-null: g holds the gate's input z, and the gate runs here
    const GateZ gz = GateZ::of_head(gate_A, bh % H, g_min);
    float* S = state + int64_t(bh) * DK * DV;
    const auto* qb = q + int64_t(bh) * DK;
    const auto* kb = k + int64_t(bh) * DK;
    const auto* gb = g + int64_t(bh) * DK;

    f32x4 s[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        s[r] = *reinterpret_cast<const f32x4*>(S + (c0 + r) * DV + cg * 4);

    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
    float kr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float a = __expf(gz(load_elem<DT>(gb, c0 + r)));
        const float kc = load_elem<DT>(kb, c0 + r);
        const float qc = load_elem<DT>(qb, c0 + r);
        kr[r] = kc;
        s[r] *= a;
        pk += kc * s[r];
        pq += qc * s[r];
        kq += kc * qc;
    }
    red_pk[rg][cg] = pk;
    red_pq[rg][cg] = pq;
    if (cg == 0) red_kq[rg] = kq;
    __syncthreads();

    f32x4 tk = {0.f, 0.f, 0.f, 0.f}, tq = {0.f, 0.f, 0.f, 0.f};
    float tkq = 0.f;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
        tk += red_pk[i][cg];
        tq += red_pq[i][cg];
        tkq += red_kq[i];
    }
    const float b = load_elem<DT>(beta, bh);
    const auto* vb = v + int64_t(bh) * DV + cg * 4;
    f32x4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = b * (load_elem<DT>(vb, j) - tk[j]);

    if (rg == 0) {
        auto* ob = o + int64_t(bh) * DV + cg * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) store_elem<DT>(ob, j, tq[j] + tkq * u[j]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        s[r] += kr[r] * u;
        store_vec<f32x4, true>(reinterpret_cast<f32x4*>(S + (c0 + r) * DV + cg * 4), s[r]);
    }
}

template <typename DT, int DK, int DV>
hipError_t launch_decode_t(const void* q, const void* k, const void* v, const void* g,
                           const void* beta, float* state, void* o, int BH, int H, const float* gate_A,
                           float g_min, hipStream_t stream)
{
    using S = typename DT::storage;
    hipLaunchKernelGGL((decode_kernel<DT, DK, DV>), dim3(BH), dim3(256), 0, stream,
                       static_cast<const S*>(q), static_cast<const S*>(k), static_cast<const S*>(v),
                       static_cast<const S*>(g), static_cast<const S*>(beta), state,
                       static_cast<S*>(o), H, gate_A, g_min);
    return hipGetLastError();
}

template <typename DT>
hipError_t launch_decode(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, float* state, void* o, int BH, int dk, int dv,
                         hipStream_t stream, int H = 1, const float* gate_A = nullptr, float g_min = -5.f)
{
#define KDA_DEC(DKV, DVV)                                                                      \
    if (dk == DKV && dv == DVV)                                                                \
        return launch_decode_t<DT, DKV, DVV>(q, k, v, g, beta, state, o, BH, H, gate_A, g_min, stream);
    KDA_DEC(32, 32) KDA_DEC(32, 64) KDA_DEC(32, 128)
    KDA_DEC(64, 32) KDA_DEC(64, 64) KDA_DEC(64, 128)
    KDA_DEC(128, 32) KDA_DEC(128, 64) KDA_DEC(128, 128)
#undef KDA_DEC
    return hipErrorInvalidValue;
}

}  // namespace kda
