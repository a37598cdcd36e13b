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
// inside the wave.  The tokens' inputs go through LDS in groups of 8,
// double-buffered: the workgroup reads each token's g, k, q, v rows once as
// 16-byte pieces spread over its threads, two groups ahead of their use, and
// the staging pass turns g into the decay alpha = exp(g) once (with the gate
// fused: from z), so each token's arithmetic reads only LDS and the memory
// latency stays off the chain from token to token.
//
// Long sequences are cut into segments that run in parallel, each taking its
// incoming state from a warm-up window, as the chunk kernels do: the
// workgroup of segment s > 0 first runs the `warm` tokens before it from a
// zero state, with the window's transition M carried beside the state by d_k
// more columns (M's columns start as the identity and see v = 0).  The state
// entering the segment is M S(window start) + S~; where every entry of the
// computed M is exactly zero it is the window's own state S~, and the segment
// runs on.  Otherwise the workgroup flags its segment and ends, and a second
// launch reruns every flagged chain (sequence, head) from its start, token by
// token: exact either way.
#pragma once

#include "kda_common.hpp"
#include "kda_prefill.hpp"
#include "kda_step.hpp"

namespace kda {

// whether an fp32 prefill of this head shape takes the token-serial kernel
constexpr bool serial_shape_f32(int dk, int dv) { return !(dk == 32 && dv <= 64); }

// WINDOWED: one workgroup per (segment, head), d_v / 32 state slices plus
// d_k / 32 transition slices for the window.  Otherwise: one workgroup per
// (sequence, head), the whole sequence, only for chains the windowed launch
// flagged (every chain when p.flags is null).
template <int DK, int DV, bool GATED, bool WINDOWED>
__global__ void __launch_bounds__(64 * ((DV + (WINDOWED ? DK : 0)) / 32)) prefill_serial_kernel(PrefillDev p)
{
    constexpr int R = DK / 8;            // rows per lane
    constexpr int RH = 4;                // rows per run of LDS reads
    constexpr int NSW = DV / 32;         // state slices
    constexpr int NT = 64 * ((DV + (WINDOWED ? DK : 0)) / 32);  // threads of the workgroup
    constexpr int E = 4;                 // floats per 16-byte piece
    constexpr int OQ = 2 * DK, OV = 3 * DK;
    constexpr int TS = OV + DV;          // staged token: alpha | k | q | v
    constexpr int PT = TS / E;           // pieces per token
    constexpr int G = 8;                 // tokens per group
    constexpr int NP = (G * PT + NT - 1) / NT;  // pieces per thread per group
    static_assert(DV % 32 == 0 && DK % 32 == 0 && (R == 4 || R == 8 || R == 16), "unsupported shape");
    static_assert(NP <= 16, "pieces per thread");
    static_assert(WARM_DEFAULT % G == 0, "windows end on a group boundary");
    __shared__ __align__(16) float tok[2][G * TS];
    __shared__ float tbeta[2][G];
    __shared__ int s_live;  // the window's M is not zero

    const int H = p.H;
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x;
    const int slice = tid >> 6;
    const int lane = tid & 63;
    const int cgl = lane & 7, rg = lane >> 3;
    const int c0 = rg * R;
    const bool mwave = slice >= NSW;  // carries 32 columns of M during the window
    const int col = (mwave ? slice - NSW : slice) * 32 + 4 * cgl;
    const float* __restrict__ q = static_cast<const float*>(p.q);
    const float* __restrict__ k = static_cast<const float*>(p.k);
    const float* __restrict__ v = static_cast<const float*>(p.v);
    const float* __restrict__ g = static_cast<const float*>(p.g);
    const float* __restrict__ beta = static_cast<const float*>(p.beta);
    float* __restrict__ o = static_cast<float*>(p.o);

    // ---- work item
    int n, s, nseg, item;
    if (WINDOWED) {
        item = blockIdx.x / H;
        if (item >= tab_seg(p, p.N)) return;
        n = p.single ? 0 : find_seq(p.tab + (p.N + 1), p.N, item);
        s = item - tab_seg(p, n);
        nseg = tab_seg(p, n + 1) - tab_seg(p, n);
        if (tid == 0) p.flags[int64_t(item) * H + h] = 0;
    } else {
        n = blockIdx.x / H;
        s = 0;
        nseg = 1;
        item = tab_seg(p, n);
        if (p.flags && !chain_flagged(p, item, tab_seg(p, n + 1) - item, h)) return;
    }
    const int64_t seq0 = tab_cu(p, n), seq1 = tab_cu(p, n + 1);
    const int64_t t_begin = WINDOWED ? seq0 + int64_t(s) * p.L * CH : seq0;
    const int64_t t_end = WINDOWED ? (t_begin + int64_t(p.L) * CH < seq1 ? t_begin + int64_t(p.L) * CH : seq1) : seq1;
    int64_t ws = t_begin;  // the window [ws, t_begin)
    if (WINDOWED && s > 0) ws = t_begin - p.warm > seq0 ? t_begin - p.warm : seq0;
    const bool from_zero = ws > seq0;  // else the window starts at the sequence start, from the initial state
    const int len = int(t_end - ws);   // tokens this workgroup runs
    const int nwin = int(t_begin - ws);
    const bool last_seg = s == nseg - 1;
    KDA_CHECK(n < p.N, CK_SEQ);
    KDA_CHECK(seq0 >= 0 && seq0 <= ws && ws <= t_begin && t_begin <= t_end && t_end <= seq1 && seq1 <= p.T_total,
              CK_TOKENS);
    KDA_CHECK(!WINDOWED || item < p.nseg_cap, CK_WS);
    const GateZ gz = GateZ::of_head(GATED ? p.gate_A : nullptr, h, p.g_min);

    // piece j of this thread in the group starting at token ws + i0: piece
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
                const int64_t row = (ws + i0 + t) * H + h;
                const float* src = c < DK   ? g + row * DK + c
                                   : c < OQ ? k + row * DK + (c - DK)
                                   : c < OV ? q + row * DK + (c - OQ)
                                            : v + row * DV + (c - OV);
                buf[j] = *reinterpret_cast<const u32x4*>(src);
            }
        }
        if (tid < m) bbuf = beta[(ws + i0 + tid) * H + h];
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
    f32x4 st[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (mwave) {  // M starts as the identity: column col + e has its 1 in row col + e
#pragma unroll
            for (int e = 0; e < 4; ++e) st[r][e] = (c0 + r == col + e) ? 1.f : 0.f;
        } else if (!from_zero && p.init) {
            // the chains' rerun reads the copy segment 0 made (p.init_snap)
            const float* src = (!WINDOWED && p.init_snap ? p.sin : p.init) + soff + r * DV;
            st[r] = f32x4{src[0], src[1], src[2], src[3]};
        } else {
            st[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // checkpoints: the state after every multiple of the interval tokens of
    // the sequence, counted from the segment's first token
    const int64_t pos0 = t_begin - seq0;
    // in place: segment 0 keeps a copy of the initial state for the chains'
    // rerun, since a last segment may write the final state over it first
    if (WINDOWED && p.init_snap && s == 0 && !mwave) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.sin[soff + r * DV + e] = st[r][e];
    }
    int64_t ck_row = 0;
    int to_ck = 0;
    if (p.ckpt) {
        ck_row = tab_ck(p, n) + pos0 / p.ckpt_interval;
        to_ck = p.ckpt_interval - int(pos0 % p.ckpt_interval);
    }
    if (tid == 0) s_live = 0;
    if (len > 0) {
        stage(0, 0);
        if (G < len) fetch(G);
    }
    __syncthreads();

    int sb = 0;
    for (int i0 = 0; i0 < len; i0 += G, sb ^= 1) {
        if (WINDOWED && from_zero && i0 == nwin) {
            // the window ends here: its state is the incoming one only where
            // every entry of M is exactly zero
            if (mwave) {
                bool nz = false;
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int e = 0; e < 4; ++e) nz = nz || st[r][e] != 0.f;
                if (__ballot(nz) != 0 && lane == 0) atomicOr(&s_live, 1);
            }
            __syncthreads();
            if (s_live) {
                if (tid == 0) p.flags[int64_t(item) * H + h] = 1;
                return;
            }
        }
        // M's columns run during the window only
        const bool run = !mwave || (from_zero && i0 < nwin);
        const bool emit = !mwave && i0 >= nwin;  // windows end on a group boundary
        const int m = min(G, len - i0);
        if (run) {
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
                        st[r0 + r] *= a[r];
                        pk += kk[r] * st[r0 + r];
                        pq += qq[r] * st[r0 + r];
                        kq += kk[r] * qq[r];
                    }
                }
                // column sums over the 8 row groups (lane bits 3..5); pk and
                // pq as a reduce-scatter: afterwards the lanes of quarter
                // Q = lane / 16 hold column 4 cgl + Q
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
                const float uq = tbeta[sb][t] * ((mwave ? 0.f : tk[OV + cq]) - pkq);
                if (emit && (lane & 8) == 0) o[((ws + i0 + t) * H + h) * DV + cq] = pqq + kq * uq;
                const f32x4 u = gather_quarters(uq);
#pragma unroll
                for (int r0 = 0; r0 < R; r0 += RH) {
                    const f32x4 kk = *reinterpret_cast<const f32x4*>(tk + DK + c0 + r0);
#pragma unroll
                    for (int r = 0; r < RH; ++r) st[r0 + r] += kk[r] * u;
                }
                if (emit && p.ckpt && --to_ck == 0) {  // the state after a multiple of the interval
                    to_ck = p.ckpt_interval;
                    if (ck_row < p.ckpt_cap) {
                        float* dst = p.ckpt + (ck_row * H + h) * DK * DV + int64_t(c0) * DV + col;
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int e = 0; e < 4; ++e) dst[r * DV + e] = st[r][e];
                    }
                    ++ck_row;
                }
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
    if (!mwave && last_seg && p.fin) {
        float* dst = p.fin + soff;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[r * DV + e] = st[r][e];
    }
}

// The serial plan: segments of L chunks as the chunk planner cuts them where
// the warm-up windows apply (for one sequence, one (segment, head) item per
// compute unit, at least 4 chunks each; for packed sequences an eighth of a
// unit's share), each with a 128-token window (force_L and warm_req as for
// prefill_plan; a zero window flags every segment after the first, so the
// chains run whole); the workspace holds the table
// the plan kernel writes (clamped cu_seqlens, segment and checkpoint offsets)
// and one flag per (segment, head), then room for a copy of the initial
// states (read by the chains' rerun when the initial state is the final state).
inline PrefillPlan serial_plan(int64_t T_total, int N, int H, int dk, int dv, int force_L = 0, int warm_req = -1)
{
    PrefillPlan p = prefill_plan(T_total, N, H, 32, 32, force_L, warm_req);  // the warm-up planner's segments
    p.np1_max = 0;
    p.off_ms = 0;
    size_t off = align256(sizeof(int32_t) * 5 * size_t(N + 1));
    p.off_table = 0;
    p.off_flags = off;
    off = align256(off + sizeof(int32_t) * size_t(p.nseg_max) * H);
    p.off_sin = off;
    off = align256(off + sizeof(float) * size_t(N) * H * dk * dv);
    p.workspace_bytes = off;
    return p;
}

template <int DK, int DV>
hipError_t launch_serial_t(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t stream)
{
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    int32_t* tab = reinterpret_cast<int32_t*>(ws + plan.off_table);
    const bool single = a.cu == nullptr && a.N == 1;
    int single_nseg = 1, single_nck = 0;
    if (single) {  // the plan kernel's arithmetic for the one sequence [0, T_total)
        const int64_t len = a.T_total > 0 ? a.T_total : 0;
        const int64_t ch = (len + CH - 1) / CH;
        const int64_t ns = (ch + plan.seg_chunks - 1) / plan.seg_chunks;
        single_nseg = int(ns < 1 ? 1 : ns);
        single_nck = (a.ckpt && a.ckpt_interval > 0) ? int(len / a.ckpt_interval) : 0;
    }
    PrefillDev d{a.q, a.k, a.v, a.g, a.beta, tab, a.N, a.T_total, a.H, plan.seg_chunks,
                 a.init, a.fin, a.o, nullptr, reinterpret_cast<float*>(ws + plan.off_sin),
                 a.ckpt, a.ckpt_interval, a.ckpt_cap, single ? 1 : 0, single_nseg, single_nck,
                 a.gate_A, a.g_min, reinterpret_cast<int32_t*>(ws + plan.off_flags), plan.warm,
                 plan.nseg_max, 0};
    d.init_snap = a.init_snap;
    hipError_t e = hipSuccess;
    if (!single) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, a.cu, a.N, a.T_total, plan.seg_chunks,
                           a.ckpt ? a.ckpt_interval : 0, tab);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const dim3 gw(unsigned(plan.nseg_max * a.H)), bw(64 * ((DV + DK) / 32));
    if (a.gate_A) hipLaunchKernelGGL((prefill_serial_kernel<DK, DV, true, true>), gw, bw, 0, stream, d);
    else hipLaunchKernelGGL((prefill_serial_kernel<DK, DV, false, true>), gw, bw, 0, stream, d);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // one segment for the one sequence: no window can fail
    if (single && single_nseg == 1) return hipSuccess;
    const dim3 gf(unsigned(int64_t(a.N) * a.H)), bf(64 * (DV / 32));
    if (a.gate_A) hipLaunchKernelGGL((prefill_serial_kernel<DK, DV, true, false>), gf, bf, 0, stream, d);
    else hipLaunchKernelGGL((prefill_serial_kernel<DK, DV, false, false>), gf, bf, 0, stream, d);
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

inline void describe_serial(const PrefillPlan& plan, int64_t N, int H, int dk, int dv, bool packed, std::string& out)
{
    char line[320];
    int n = 0;
    if (packed) {
        snprintf(line, sizeof(line), "launch %d: plan_kernel grid 1 x 256 threads, 0 B LDS; segment table and "
                 "checkpoint offsets of the packed sequences\n", ++n);
        out += line;
    }
    snprintf(line, sizeof(line), "launch %d: prefill_serial_kernel (windowed) grid %lld x %d threads; every "
             "(segment, head) token by token in fp32 after its warm-up window; flags the chains where the "
             "window's transition is not zero\n", ++n, (long long)plan.nseg_max * H, 64 * ((dv + dk) / 32));
    out += line;
    if (packed || plan.nseg_max > 1) {
        snprintf(line, sizeof(line), "launch %d: prefill_serial_kernel (chains) grid %lld x %d threads; the "
                 "flagged chains from their start (returns at once elsewhere)\n", ++n, (long long)N * H,
                 64 * (dv / 32));
        out += line;
    }
}

}  // namespace kda
