// Token-serial fp32 prefill: the fp32 head shapes the chunk kernels are not
// built for (d_k > 32, or d_v = 128).  Their fp32 operand tiles would need
// twice the LDS of the bf16 ones, more than one compute unit holds, so these
// shapes advance the recurrence one token at a time instead, in fp32
// throughout, with the state in registers.
//
// Sources: "NLP——技术报告解读-Kimi-K3", Model Architecture / Kimi Delta
// Attention (KDA) (the recurrence and its read-out); "Kimi K3 技术报告 ·
// 大白话版" §2.1.1 (decay, then delta correction, then read after the
// update).
//
// Per token, with alpha = exp(g) and D = Diag(alpha), the decode step's form:
//   pk = (D S)^T k,  pq = (D S)^T q,  u = beta (v - pk),
//   S <- D S + k u^T,  o = S_new^T q = pq + (k^T q) u.
// Lane layout as the decode step: one wave owns a 32-column slice of one
// (sequence, head) state, lane 8 rg + cgl holding 4 consecutive columns of
// d_k / 8 consecutive rows; the column sums over d_k are lane exchanges
// inside the wave.  One workgroup is the d_v / 32 slices of one (sequence,
// head).  The tokens' inputs go through LDS in groups of 8, double-buffered:
// the workgroup reads each token's g, k, q, v rows once as 16-byte pieces
// spread over its threads, two groups ahead of their use, and the staging
// pass turns g into the decay alpha = exp(g) once (with the gate fused: from
// z), so each token's arithmetic reads only LDS and the memory latency stays
// off the chain from token to token.
#pragma once

#include "kda_common.hpp"
#include "kda_prefill.hpp"
#include "kda_step.hpp"

namespace kda {

// whether an fp32 prefill of this head shape takes the token-serial kernel
constexpr bool serial_shape_f32(int dk, int dv) { return !(dk == 32 && dv <= 64); }

template <int DK, int DV, bool GATED>
__global__ void __launch_bounds__(64 * (DV / 32)) prefill_serial_kernel(PrefillDev p)
{
    constexpr int R = DK / 8;            // rows per lane
    constexpr int RH = 4;                // rows per run of LDS reads
    constexpr int NT = 64 * (DV / 32);   // threads of the workgroup
    constexpr int E = 4;                 // floats per 16-byte piece
    constexpr int OQ = 2 * DK, OV = 3 * DK;
    constexpr int TS = OV + DV;          // staged token: alpha | k | q | v
    constexpr int PT = TS / E;           // pieces per token
    constexpr int G = 8;                 // tokens per group
    constexpr int NP = (G * PT + NT - 1) / NT;  // pieces per thread per group
    static_assert(DV % 32 == 0 && (R == 4 || R == 8 || R == 16), "unsupported shape");
    static_assert(NP <= 16, "pieces per thread");
    __shared__ __align__(16) float tok[2][G * TS];
    __shared__ float tbeta[2][G];

    const int H = p.H;
    const int n = blockIdx.x / H, h = blockIdx.x % H;
    const int tid = threadIdx.x;
    const int slice = tid >> 6;
    const int lane = tid & 63;
    const int cgl = lane & 7, rg = lane >> 3;
    const int c0 = rg * R;
    const int col = slice * 32 + 4 * cgl;
    const float* __restrict__ q = static_cast<const float*>(p.q);
    const float* __restrict__ k = static_cast<const float*>(p.k);
    const float* __restrict__ v = static_cast<const float*>(p.v);
    const float* __restrict__ g = static_cast<const float*>(p.g);
    const float* __restrict__ beta = static_cast<const float*>(p.beta);
    float* __restrict__ o = static_cast<float*>(p.o);

    const int32_t t0 = tab_cu(p, n);
    const int len = tab_cu(p, n + 1) - t0;
    KDA_CHECK(n < p.N, CK_SEQ);
    KDA_CHECK(t0 >= 0 && len >= 0 && int64_t(t0) + len <= p.T_total, CK_TOKENS);
    const GateZ gz = GateZ::of_head(GATED ? p.gate_A : nullptr, h, p.g_min);

    // piece j of this thread in the group starting at token i0: piece
    // pi = tid + j NT of the group, token pi / PT, elements E (pi % PT) ..
    // + E of the staged row, which sits at E pi in the group's LDS buffer
    u32x4 buf[NP];
    float bbuf = 0.f;
    auto fetch = [&](int i0) {
        const int m = min(G, len - i0);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pi = tid + j * NT;
            if (pi < m * PT) {
                const int t = pi / PT, c = (pi - t * PT) * E;
                const int64_t row = int64_t(t0 + i0 + t) * H + h;
                const float* src = c < DK   ? g + row * DK + c
                                   : c < OQ ? k + row * DK + (c - DK)
                                   : c < OV ? q + row * DK + (c - OQ)
                                            : v + row * DV + (c - OV);
                buf[j] = *reinterpret_cast<const u32x4*>(src);
            }
        }
        if (tid < m) bbuf = beta[int64_t(t0 + i0 + tid) * H + h];
    };
    auto stage = [&](int i0, int sb) {
        const int m = min(G, len - i0);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pi = tid + j * NT;
            if (pi < m * PT) {
                f32x4 x = __builtin_bit_cast(f32x4, buf[j]);
                if ((pi - pi / PT * PT) * E < DK) {  // g: the decay alpha = exp(g)
#pragma unroll
                    for (int e = 0; e < E; ++e) x[e] = __expf(gz(x[e]));
                }
                *reinterpret_cast<f32x4*>(&tok[sb][pi * E]) = x;
            }
        }
        if (tid < m) tbeta[sb][tid] = bbuf;
    };

    // this lane's part of the state: rows c0 .. c0 + R - 1, columns col .. col + 3
    const int64_t soff = (int64_t(n) * H + h) * DK * DV + int64_t(c0) * DV + col;
    if (len > 0) fetch(0);
    f32x4 s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (p.init) {
            const float* src = p.init + soff + r * DV;
            s[r] = f32x4{src[0], src[1], src[2], src[3]};
        } else {
            s[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    int64_t ck_row = p.ckpt ? tab_ck(p, n) : 0;  // the next checkpoint's row
    int to_ck = p.ckpt_interval;                 // tokens until it
    if (len > 0) {
        stage(0, 0);
        if (G < len) fetch(G);
    }
    __syncthreads();

    int sb = 0;
    for (int i0 = 0; i0 < len; i0 += G, sb ^= 1) {
        const int m = min(G, len - i0);
#pragma unroll 1
        for (int t = 0; t < m; ++t) {
            const float* tk = &tok[sb][t * TS];
            f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
            float kq = 0.f;
#pragma unroll
            for (int r0 = 0; r0 < R; r0 += RH) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(tk + c0 + r0);
                const f32x4 kk = *reinterpret_cast<const f32x4*>(tk + DK + c0 + r0);
                const f32x4 qq = *reinterpret_cast<const f32x4*>(tk + OQ + c0 + r0);
#pragma unroll
                for (int r = 0; r < RH; ++r) {
                    s[r0 + r] *= a[r];
                    pk += kk[r] * s[r0 + r];
                    pq += qq[r] * s[r0 + r];
                    kq += kk[r] * qq[r];
                }
            }
            // column sums over the 8 row groups (lane bits 3..5); pk and pq
            // as a reduce-scatter: afterwards the lanes of quarter Q = lane / 16
            // hold column 4 cgl + Q
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                pk[mm] += lane_xor_8_16_32(pk[mm], 8, lane);
                pq[mm] += lane_xor_8_16_32(pq[mm], 8, lane);
            }
            kq += lane_xor_8_16_32(kq, 8, lane);
            kq += lane_xor_8_16_32(kq, 16, lane);
            kq += lane_xor_8_16_32(kq, 32, lane);
            const float pkq = fold32(fold16(pk[0], pk[1]), fold16(pk[2], pk[3]));
            const float pqq = fold32(fold16(pq[0], pq[1]), fold16(pq[2], pq[3]));
            const int cq = col + (lane >> 4);  // this lane's column
            const float uq = tbeta[sb][t] * (tk[OV + cq] - pkq);
            if ((lane & 8) == 0) o[(int64_t(t0 + i0 + t) * H + h) * DV + cq] = pqq + kq * uq;
            const f32x4 u = gather_quarters(uq);
#pragma unroll
            for (int r0 = 0; r0 < R; r0 += RH) {
                const f32x4 kk = *reinterpret_cast<const f32x4*>(tk + DK + c0 + r0);
#pragma unroll
                for (int r = 0; r < RH; ++r) s[r0 + r] += kk[r] * u;
            }
            if (p.ckpt && --to_ck == 0) {  // the state after a multiple of the interval
                to_ck = p.ckpt_interval;
                if (ck_row < p.ckpt_cap) {
                    float* dst = p.ckpt + (ck_row * H + h) * DK * DV + int64_t(c0) * DV + col;
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int e = 0; e < 4; ++e) dst[r * DV + e] = s[r][e];
                }
                ++ck_row;
            }
        }
        // the next group into the other buffer (its loads were issued a group
        // ago), then the loads of the group after it; the barrier keeps any
        // wave from staging into a buffer another wave still reads
        if (i0 + G < len) {
            stage(i0 + G, sb ^ 1);
            if (i0 + 2 * G < len) fetch(i0 + 2 * G);
        }
        __syncthreads();
    }
    if (p.fin) {
        float* dst = p.fin + soff;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[r * DV + e] = s[r][e];
    }
}

// The serial plan: one segment per sequence; the workspace holds only the
// table the plan kernel writes for packed sequences (clamped cu_seqlens and
// checkpoint offsets).
inline PrefillPlan serial_plan(int64_t T_total, int N)
{
    PrefillPlan p;
    const int64_t max_seq_chunks = (T_total + CH - 1) / CH;
    p.seg_chunks = int(max_seq_chunks > 0 ? max_seq_chunks : 1);
    p.warm = 0;
    p.nseg_max = N;
    p.np1_max = 0;
    p.off_table = 0;
    p.workspace_bytes = align256(sizeof(int32_t) * 5 * size_t(N + 1));
    return p;
}

template <int DK, int DV>
hipError_t launch_serial_t(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t stream)
{
    int32_t* tab = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(a.ws) + plan.off_table);
    const bool single = a.cu == nullptr && a.N == 1;
    const int64_t len = a.T_total > 0 ? a.T_total : 0;
    const int single_nck = (single && a.ckpt && a.ckpt_interval > 0) ? int(len / a.ckpt_interval) : 0;
    PrefillDev d{a.q, a.k, a.v, a.g, a.beta, tab, a.N, a.T_total, a.H, plan.seg_chunks,
                 a.init, a.fin, a.o, nullptr, nullptr,
                 a.ckpt, a.ckpt_interval, a.ckpt_cap, single ? 1 : 0, 1, single_nck,
                 a.gate_A, a.g_min, nullptr, 0, plan.nseg_max, 0};
    hipError_t e = hipSuccess;
    if (!single) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, a.cu, a.N, a.T_total, plan.seg_chunks,
                           a.ckpt ? a.ckpt_interval : 0, tab);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const dim3 grid(unsigned(int64_t(a.N) * a.H)), block(64 * (DV / 32));
    if (a.gate_A)
        hipLaunchKernelGGL((prefill_serial_kernel<DK, DV, true>), grid, block, 0, stream, d);
    else
        hipLaunchKernelGGL((prefill_serial_kernel<DK, DV, false>), grid, block, 0, stream, d);
    return hipGetLastError();
}

inline hipError_t launch_serial(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t stream)
{
#define KDA_PS(DKV, DVV) \
    if (a.dk == DKV && a.dv == DVV) return launch_serial_t<DKV, DVV>(a, plan, stream);
    KDA_PS(32, 128)
    KDA_PS(64, 32) KDA_PS(64, 64) KDA_PS(64, 128)
    KDA_PS(128, 32) KDA_PS(128, 64) KDA_PS(128, 128)
#undef KDA_PS
    return hipErrorInvalidValue;
}

inline void describe_serial(int64_t N, int H, int dv, bool packed, std::string& out)
{
    char line[256];
    int n = 0;
    if (packed) {
        snprintf(line, sizeof(line), "launch %d: plan_kernel grid 1 x 256 threads, 0 B LDS; clamped cu_seqlens "
                 "and checkpoint offsets of the packed sequences\n", ++n);
        out += line;
    }
    snprintf(line, sizeof(line), "launch %d: prefill_serial_kernel grid %lld x %d threads, 0 B LDS; every "
             "(sequence, head) token by token in fp32, state in registers\n", ++n, (long long)N * H, 64 * (dv / 32));
    out += line;
}

}  // namespace kda
