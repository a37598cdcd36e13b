// kda_verify / kda_commit: speculative multi-token decode against a resident
// state, with roll-back by replay.
//
// Sources: "NLP——技术报告解读-Kimi-K3", Infrastructure / 推理与在线服务,
// high-performance kernels, KDA decoding (under multi-token-prediction
// speculative decoding the projected inputs are cached instead of states, and
// the state is rebuilt on demand by replay); "Kimi K3 技术报告 · 大白话版" §5.4
// (a rejected guess cannot be undone on an in-place state, so the raw inputs
// are kept and replayed on chip); "详解Kimi K3：强到冲击Anthropic估值的模型什么样？",
// section 先分后合，和一条没有开源的流水线 (store a small per-token
// projection, replay the accepted tokens from the last checkpoint).
//
// verify: for each (b, h), K draft tokens run through the recurrence from the
//   resident state S, which is read and NOT written; o is emitted for every
//   draft token (the values an in-place decode of those tokens would give).
// commit: the first n_b <= K of the same cached tokens are replayed onto S in
//   place (o is not written): the state after the accepted prefix.
// Per token, with alpha = exp(g) and D = Diag(alpha), the step is the decode
// step (pk = (D S)^T k, pq = (D S)^T q, u = beta (v - pk), S <- D S + k u^T,
// o = pq + (k^T q) u); the state stays in registers across the K tokens, so it
// is read once (and, for commit, written once) per call.
#pragma once

#include "kda_common.hpp"

namespace kda {

template <typename DT, int DK, int DV, bool COMMIT>
__global__ void __launch_bounds__(256) spec_kernel(const typename DT::storage* __restrict__ q,
                                                   const typename DT::storage* __restrict__ k,
                                                   const typename DT::storage* __restrict__ v,
                                                   const typename DT::storage* __restrict__ g,
                                                   const typename DT::storage* __restrict__ beta,
                                                   const int32_t* __restrict__ n_accept, float* state,
                                                   typename DT::storage* __restrict__ o, int K, int H)
{
    constexpr int CG = DV / 4;    // column groups of 4
    constexpr int RG = 256 / CG;  // row groups
    constexpr int R = DK / RG;    // rows per thread
    static_assert(R >= 1 && DK % RG == 0, "unsupported shape");

    __shared__ f32x4 red_pk[2][RG][CG];
    __shared__ f32x4 red_pq[2][RG][CG];
    __shared__ float red_kq[2][RG];

    const int bh = blockIdx.x;  // b * H + h
    const int b = bh / H, h = bh % H;
    const int t = threadIdx.x;
    const int cg = t % CG;
    const int rg = t / CG;
    const int c0 = rg * R;

    int steps = K;
    if (COMMIT) {
        const int na = n_accept[b];
        steps = na < 0 ? 0 : (na > K ? K : na);
        if (steps == 0) return;  // nothing accepted: the state is left untouched
    }

    float* S = state + int64_t(bh) * DK * DV;
    f32x4 s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = *reinterpret_cast<const f32x4*>(S + (c0 + r) * DV + cg * 4);

    for (int i = 0; i < steps; ++i) {
        // token i of sequence b: tensors are [B, K, H, d]
        const int64_t row = (int64_t(b) * K + i) * H + h;
        const auto* qb = q + row * DK;
        const auto* kb = k + row * DK;
        const auto* gb = g + row * DK;
        f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
        float kq = 0.f;
        float kr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float a = __expf(load_elem<DT>(gb, c0 + r));
            const float kc = load_elem<DT>(kb, c0 + r);
            const float qc = COMMIT ? 0.f : load_elem<DT>(qb, c0 + r);
            kr[r] = kc;
            s[r] *= a;
            pk += kc * s[r];
            if (!COMMIT) {
                pq += qc * s[r];
                kq += kc * qc;
            }
        }
        const int pb = i & 1;  // alternating reduction buffers: one barrier per token
        red_pk[pb][rg][cg] = pk;
        if (!COMMIT) {
            red_pq[pb][rg][cg] = pq;
            if (cg == 0) red_kq[pb][rg] = kq;
        }
        __syncthreads();
        f32x4 tk = {0.f, 0.f, 0.f, 0.f}, tq = {0.f, 0.f, 0.f, 0.f};
        float tkq = 0.f;
#pragma unroll
        for (int j = 0; j < RG; ++j) {
            tk += red_pk[pb][j][cg];
            if (!COMMIT) {
                tq += red_pq[pb][j][cg];
                tkq += red_kq[pb][j];
            }
        }
        const float bt = load_elem<DT>(beta, row);
        const auto* vb = v + row * DV + cg * 4;
        f32x4 u;
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = bt * (load_elem<DT>(vb, j) - tk[j]);
        if (!COMMIT && rg == 0) {
            auto* ob = o + row * DV + cg * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) store_elem<DT>(ob, j, tq[j] + tkq * u[j]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] += kr[r] * u;
    }
    if (COMMIT) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            store_vec<f32x4, true>(reinterpret_cast<f32x4*>(S + (c0 + r) * DV + cg * 4), s[r]);
    }
}

template <typename DT, int DK, int DV>
hipError_t launch_spec_t(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const int32_t* n_accept, float* state, void* o, int B, int K, int H, bool commit,
                         hipStream_t stream)
{
    using S = typename DT::storage;
    const dim3 grid(unsigned(B * H)), block(256);
    if (commit)
        hipLaunchKernelGGL((spec_kernel<DT, DK, DV, true>), grid, block, 0, stream, static_cast<const S*>(q),
                           static_cast<const S*>(k), static_cast<const S*>(v), static_cast<const S*>(g),
                           static_cast<const S*>(beta), n_accept, state, static_cast<S*>(o), K, H);
    else
        hipLaunchKernelGGL((spec_kernel<DT, DK, DV, false>), grid, block, 0, stream, static_cast<const S*>(q),
                           static_cast<const S*>(k), static_cast<const S*>(v), static_cast<const S*>(g),
                           static_cast<const S*>(beta), n_accept, state, static_cast<S*>(o), K, H);
    return hipGetLastError();
}

template <typename DT>
hipError_t launch_spec(const void* q, const void* k, const void* v, const void* g, const void* beta,
                       const int32_t* n_accept, float* state, void* o, int B, int K, int H, int dk, int dv,
                       bool commit, hipStream_t stream)
{
#define KDA_SPEC(DKV, DVV)                                                                            \
    if (dk == DKV && dv == DVV)                                                                       \
        return launch_spec_t<DT, DKV, DVV>(q, k, v, g, beta, n_accept, state, o, B, K, H, commit, stream);
    KDA_SPEC(32, 32) KDA_SPEC(32, 64) KDA_SPEC(32, 128)
    KDA_SPEC(64, 32) KDA_SPEC(64, 64) KDA_SPEC(64, 128)
    KDA_SPEC(128, 32) KDA_SPEC(128, 64) KDA_SPEC(128, 128)
#undef KDA_SPEC
    return hipErrorInvalidValue;
}

}  // namespace kda
