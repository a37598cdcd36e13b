// One-wave recurrence steps against a resident fp32 state: the decode step
// (one token, state updated in place), verify (K draft tokens, state read
// only) and commit (replay of the accepted prefix, state written once).
//
// Sources: "NLP——技术报告解读-Kimi-K3", Model Architecture / Kimi Delta
// Attention (KDA), state update and read-out, and Infrastructure / 推理与在线服务
// (KDA decoding under speculative decoding: cached projected inputs, state
// rebuilt by replay); "Kimi K3 技术报告 · 大白话版" §2.1.1 (decay, then delta
// correction, then read) and §5.4 (in-place state; replay of the accepted
// guesses).
//
// Per token, with alpha = exp(g) and D = Diag(alpha):
//   pk = (D S)^T k,  pq = (D S)^T q,  u = beta (v - pk),
//   S <- D S + k u^T,  o = S_new^T q = pq + (k^T q) u.
// The columns of the state are independent: column c needs only column c of
// the state and the column sums over d_k.  So one wave owns a 32-column slice
// of one (b, h) state, all d_k rows of it, in registers: lane = 8 * rg + cgl
// holds 4 consecutive columns (cgl) of d_k / 8 consecutive rows (rg).  The
// sums over d_k are three lane exchanges inside the wave (row groups differ in
// lane bits 3..5): no LDS and no barrier in the arithmetic.  Each row of the
// slice is 128 contiguous bytes, read by the 8 lanes of one row group.
#pragma once

#include "kda_common.hpp"

namespace kda {

// The value held by lane `lane ^ dist` for dist in {8, 16, 32}: a DPP rotate
// by half a row, v_permlane16_swap, v_permlane32_swap.
__device__ __forceinline__ float lane_xor_8_16_32(float x, int dist, int lane)
{
    const unsigned u = __float_as_uint(x);
    if (dist == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __uint_as_float(lane >= 32 ? r[0] : r[1]);
    }
    if (dist == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __uint_as_float((lane & 16) ? r[0] : r[1]);
    }
    return __int_as_float(__builtin_amdgcn_update_dpp(0, int(u), 0x128, 0xf, 0xf, false));  // row_ror:8
}

// a and b each summed over lane bit 4 in one exchange: lanes with bit 4 clear
// get a + a', the others b' + b (x' the value of lane ^ 16)
__device__ __forceinline__ float fold16(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// the same over lane bit 5: lanes below 32 get a + a', the others b' + b
__device__ __forceinline__ float fold32(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x holds value Q in the lanes of quarter Q (lanes 16 Q .. 16 Q + 15): every
// lane gets the four values, each from the lane of its quarter at its own
// position in the quarter
__device__ __forceinline__ f32x4 gather_quarters(float x)
{
    const unsigned w = __float_as_uint(x);
    const auto h = __builtin_amdgcn_permlane32_swap(w, w, false, false);  // [0]: values 0 | 1, [1]: 2 | 3
    const auto a = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
    return f32x4{__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(c[0]), __uint_as_float(c[1])};
}

// R consecutive elements (R = 4, 8 or 16) from an address aligned to their size
template <typename DT, int R>
__device__ __forceinline__ void load_run(const typename DT::storage* p, float (&x)[R])
{
    if constexpr (R >= 8) {
#pragma unroll
        for (int j = 0; j < R / 8; ++j) {
            float y[8];
            load8<DT>(p + 8 * j, y);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[8 * j + e] = y[e];
        }
    } else {
        static_assert(R == 4, "runs of 4, 8 or 16");
        if constexpr (DT::is_bf16) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(p);
            x[0] = bf16_lo(w[0]);
            x[1] = bf16_hi(w[0]);
            x[2] = bf16_lo(w[1]);
            x[3] = bf16_hi(w[1]);
        } else {
            const f32x4 w = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = w[e];
        }
    }
}

// EMIT_O: write o per token (decode).  WRITE_S: write the state back (decode,
// commit).  Decode runs K = 1 token; commit the first n_accept[b] (clamped to
// [0, K]) of K and emits nothing; verify has a kernel of its own below.  The
// workgroup is the d_v / 32 waves of one state (one slice each): they share
// nothing and never synchronise, but run side by side, so each 512-byte state
// row is read (and written) by the four waves at about the same time.
template <typename DT, int DK, int DV, bool EMIT_O, bool WRITE_S, bool GATED>
__global__ void __launch_bounds__(64 * (DV / 32)) step_wave_kernel(const typename DT::storage* __restrict__ q,
                                                       const typename DT::storage* __restrict__ k,
                                                       const typename DT::storage* __restrict__ v,
                                                       const typename DT::storage* __restrict__ g,
                                                       const typename DT::storage* __restrict__ beta,
                                                       const int32_t* __restrict__ n_accept, float* state,
                                                       typename DT::storage* __restrict__ o, int K, int H,
                                                       const float* __restrict__ gate_A, float g_min)
{
    constexpr int R = DK / 8;  // rows per lane
    static_assert(DV % 32 == 0 && (R == 4 || R == 8 || R == 16), "unsupported shape");
    const int bh = blockIdx.x;
    const int slice = threadIdx.x >> 6;  // waves of one workgroup: the slices of one state
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x & 63;
    const int cgl = lane & 7, rg = lane >> 3;
    const int c0 = rg * R;
    const int col = slice * 32 + 4 * cgl;

    int steps = K;
    if (!EMIT_O) {  // commit: the accepted prefix only
        const int na = n_accept[b];
        steps = na < 0 ? 0 : (na > K ? K : na);
        if (steps == 0) return;  // nothing accepted: the state is left untouched
    }

    // GATED: g holds the gate's input z, and the gate runs here (a separate
    // instantiation, so the plain kernel keeps its register budget)
    const GateZ gz = GateZ::of_head(GATED ? gate_A : nullptr, h, g_min);
    float* S = state + int64_t(bh) * DK * DV + col;
    f32x4 s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = *reinterpret_cast<const f32x4*>(S + (c0 + r) * DV);

    for (int i = 0; i < steps; ++i) {
        const int64_t row = (int64_t(b) * K + i) * H + h;  // token tensors are [B, K, H, d]
        float a[R], kk[R], qq[R];
        load_run<DT, R>(g + row * DK + c0, a);
        load_run<DT, R>(k + row * DK + c0, kk);
        if (EMIT_O) load_run<DT, R>(q + row * DK + c0, qq);
        f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
        float kq = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            s[r] *= __expf(GATED ? gz(a[r]) : a[r]);
            pk += kk[r] * s[r];
            if (EMIT_O) {
                pq += qq[r] * s[r];
                kq += kk[r] * qq[r];
            }
        }
        // column sums over all d_k rows: the 8 row groups of the wave
#pragma unroll
        for (int d = 8; d < 64; d <<= 1) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                pk[m] += lane_xor_8_16_32(pk[m], d, lane);
                if (EMIT_O) pq[m] += lane_xor_8_16_32(pq[m], d, lane);
            }
            if (EMIT_O) kq += lane_xor_8_16_32(kq, d, lane);
        }
        float vv[4];
        load_run<DT, 4>(v + row * DV + col, vv);
        const float bt = load_elem<DT>(beta, row);
        f32x4 u;
#pragma unroll
        for (int m = 0; m < 4; ++m) u[m] = bt * (vv[m] - pk[m]);
        if (EMIT_O && rg == 0) {
            const f32x4 ov = pq + kq * u;
            auto* ob = o + row * DV + col;
            if constexpr (DT::is_bf16) {
                *reinterpret_cast<u32x2*>(ob) = u32x2{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
            } else {
                *reinterpret_cast<f32x4*>(ob) = ov;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] += kk[r] * u;
    }
    if (WRITE_S) {
#pragma unroll
        for (int r = 0; r < R; ++r) store_vec<f32x4, true>(reinterpret_cast<f32x4*>(S + (c0 + r) * DV), s[r]);
    }
}

// Verify: K draft tokens scored from the resident state, which is read once
// and never written.  Same lane layout as step_wave_kernel and the same
// arithmetic per token (every sum pairs the same addends), so its outputs
// equal K decode steps bit for bit; but the tokens' inputs are staged
// through LDS, G tokens at a time: the workgroup reads each token's g, k, q,
// v rows once, as 16-byte pieces spread over its threads (where every lane
// would otherwise read its d_k / 8 rows of them from the caches, token after
// token), and the first group's loads are issued before the state's, so
// they arrive while the state streams in.  The staging also does, once per workgroup, the work
// every lane would repeat on its rows: the rows go to LDS as fp32, and g as
// the decay alpha = exp(g).  In the kernels that write the state (decode,
// commit) the staging measured slower, so they keep the direct form.
template <typename DT, int DK, int DV>
__global__ void __launch_bounds__(64 * (DV / 32)) verify_wave_kernel(const typename DT::storage* __restrict__ q,
                                                         const typename DT::storage* __restrict__ k,
                                                         const typename DT::storage* __restrict__ v,
                                                         const typename DT::storage* __restrict__ g,
                                                         const typename DT::storage* __restrict__ beta,
                                                         const float* __restrict__ state,
                                                         typename DT::storage* __restrict__ o, int K, int H)
{
    using ST = typename DT::storage;
    constexpr int R = DK / 8;                     // rows per lane
    constexpr int RH = 4;                         // rows per run of LDS reads
    constexpr int NT = 64 * (DV / 32);            // threads of the workgroup
    constexpr int E = 16 / int(sizeof(ST));       // elements per 16-byte piece
    constexpr int OQ = 2 * DK;                    // staged token: alpha, k, q, v (fp32)
    constexpr int OV = 3 * DK;
    constexpr int TS = OV + DV;                   // elements per staged token
    constexpr int PT = TS / E;                    // pieces per token
    constexpr int G = (2 * NT) / PT < 1 ? 1 : (2 * NT) / PT > 8 ? 8 : (2 * NT) / PT;  // tokens per group
    constexpr int NP = (G * PT + NT - 1) / NT;    // pieces per thread per group (at most 2)
    static_assert(DV % 32 == 0 && (R == 4 || R == 8 || R == 16), "unsupported shape");
    static_assert(NP <= 2, "at most two pieces per thread");
    __shared__ __align__(16) float tok[G * TS];
    __shared__ float tbeta[G];

    const int bh = blockIdx.x;
    const int slice = threadIdx.x >> 6;  // waves of one workgroup: the slices of one state
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x & 63;
    const int cgl = lane & 7, rg = lane >> 3;
    const int c0 = rg * R;
    const int col = slice * 32 + 4 * cgl;

    // piece p of the group starting at token i0: token p / PT of the group,
    // elements [E (p % PT), E (p % PT) + E) of its staged row, which sits at
    // tok + E p in LDS
    u32x4 buf[NP];
    ST bbuf = 0;  // raw: converted once staged, so no wait falls before the state's loads
    auto fetch = [&](int i0) {
        const int n = min(G, K - i0);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int p = int(threadIdx.x) + j * NT;
            if (p < n * PT) {
                const int t = p / PT, c = (p - t * PT) * E;
                const int64_t row = (int64_t(b) * K + i0 + t) * H + h;  // token tensors are [B, K, H, d]
                const ST* src = c < DK   ? g + row * DK + c
                                : c < OQ ? k + row * DK + (c - DK)
                                : c < OV ? q + row * DK + (c - OQ)
                                         : v + row * DV + (c - OV);
                buf[j] = *reinterpret_cast<const u32x4*>(src);
            }
        }
        if (int(threadIdx.x) < n) bbuf = beta[(int64_t(b) * K + i0 + threadIdx.x) * H + h];
    };
    auto stage = [&](int i0) {
        const int n = min(G, K - i0);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int p = int(threadIdx.x) + j * NT;
            if (p < n * PT) {
                const bool is_g = (p - p / PT * PT) * E < DK;
                float x[E];
                if constexpr (DT::is_bf16) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[2 * e] = bf16_lo(buf[j][e]);
                        x[2 * e + 1] = bf16_hi(buf[j][e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(buf[j][e]);
                }
                if (is_g) {
#pragma unroll
                    for (int e = 0; e < E; ++e) x[e] = __expf(x[e]);
                }
#pragma unroll
                for (int e = 0; e < E; e += 4)
                    *reinterpret_cast<f32x4*>(tok + p * E + e) = f32x4{x[e], x[e + 1], x[e + 2], x[e + 3]};
            }
        }
        if (int(threadIdx.x) < n) tbeta[threadIdx.x] = load_elem<DT>(&bbuf, 0);
    };

    fetch(0);
    const float* S = state + int64_t(bh) * DK * DV + col;
    f32x4 s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = *reinterpret_cast<const f32x4*>(S + (c0 + r) * DV);

    for (int i0 = 0; i0 < K; i0 += G) {
        stage(i0);
        __syncthreads();
        const int n = min(G, K - i0);
#pragma unroll 1
        for (int t = 0; t < n; ++t) {
            const float* tk = tok + t * TS;
            f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
            float kq = 0.f;
            // the rows in runs of RH, read from LDS as they are needed (LDS
            // reads are cheap to repeat; registers for all of them are not)
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
                asm volatile("" ::: "memory");  // keep the next run's LDS reads here
            }
            // column sums over all d_k rows (the 8 row groups, lane bits 3..5),
            // pairing the addends as step_wave_kernel's butterfly does (bit 3,
            // then 4, then 5), but as a reduce-scatter: afterwards the lane in
            // quarter Q = lane / 16 holds column 4 cgl + Q of pk and pq
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                pk[m] += lane_xor_8_16_32(pk[m], 8, lane);
                pq[m] += lane_xor_8_16_32(pq[m], 8, lane);
            }
            kq += lane_xor_8_16_32(kq, 8, lane);
            kq += lane_xor_8_16_32(kq, 16, lane);
            kq += lane_xor_8_16_32(kq, 32, lane);
            const float pkq = fold32(fold16(pk[0], pk[1]), fold16(pk[2], pk[3]));
            const float pqq = fold32(fold16(pq[0], pq[1]), fold16(pq[2], pq[3]));
            const int cq = col + (lane >> 4);  // this lane's column
            const float uq = tbeta[t] * (tk[OV + cq] - pkq);
            if ((lane & 8) == 0) {  // one lane per column
                const float ov = pqq + kq * uq;
                auto* ob = o + ((int64_t(b) * K + i0 + t) * H + h) * DV + cq;
                if constexpr (DT::is_bf16) *ob = uint16_t(pack_bf16x2(ov, 0.f));
                else *ob = ov;
            }
            const f32x4 u = gather_quarters(uq);
#pragma unroll
            for (int r0 = 0; r0 < R; r0 += RH) {
                const f32x4 kk = *reinterpret_cast<const f32x4*>(tk + DK + c0 + r0);
#pragma unroll
                for (int r = 0; r < RH; ++r) s[r0 + r] += kk[r] * u;
                asm volatile("" ::: "memory");
            }
        }
        if (i0 + G < K) {
            __syncthreads();  // the group is read before the next one is staged
            fetch(i0 + G);
        }
    }
}

// 16-byte alignment of every token tensor (the kernel's vector loads and stores)
inline bool step_wave_aligned(const void* q, const void* k, const void* v, const void* g, const void* o)
{
    auto al = [](const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    return al(q) && al(k) && al(v) && al(g) && al(o);
}

template <typename DT, int DK, int DV, bool EMIT_O, bool WRITE_S, bool GATED = false>
hipError_t launch_step_wave_t(const void* q, const void* k, const void* v, const void* g, const void* beta,
                              const int32_t* n_accept, float* state, void* o, int B, int K, int H,
                              const float* gate_A, float g_min, hipStream_t stream)
{
    using S = typename DT::storage;
    hipLaunchKernelGGL((step_wave_kernel<DT, DK, DV, EMIT_O, WRITE_S, GATED>), dim3(unsigned(B * H)),
                       dim3(64 * (DV / 32)), 0, stream, static_cast<const S*>(q), static_cast<const S*>(k),
                       static_cast<const S*>(v), static_cast<const S*>(g), static_cast<const S*>(beta), n_accept,
                       state, static_cast<S*>(o), K, H, gate_A, g_min);
    return hipGetLastError();
}

// mode: 0 decode (one token, o, state written), 1 verify (K tokens, o), 2 commit (n_accept tokens, state)
template <typename DT, int DKV, int DVV>
hipError_t launch_step_wave_shape(int mode, const void* q, const void* k, const void* v, const void* g,
                                  const void* beta, const int32_t* n_accept, float* state, void* o, int B, int K,
                                  int H, const float* gate_A, float g_min, hipStream_t stream)
{
    if (mode == 0 && gate_A)  // decode with the gate fused
        return launch_step_wave_t<DT, DKV, DVV, true, true, true>(q, k, v, g, beta, n_accept, state, o, B, K, H,
                                                                  gate_A, g_min, stream);
    if (mode == 0)
        return launch_step_wave_t<DT, DKV, DVV, true, true>(q, k, v, g, beta, n_accept, state, o, B, K, H, gate_A,
                                                            g_min, stream);
    if (mode == 1) {
        using S = typename DT::storage;
        hipLaunchKernelGGL((verify_wave_kernel<DT, DKV, DVV>), dim3(unsigned(B * H)), dim3(64 * (DVV / 32)), 0,
                           stream, static_cast<const S*>(q), static_cast<const S*>(k), static_cast<const S*>(v),
                           static_cast<const S*>(g), static_cast<const S*>(beta), state, static_cast<S*>(o), K, H);
        return hipGetLastError();
    }
    return launch_step_wave_t<DT, DKV, DVV, false, true>(q, k, v, g, beta, n_accept, state, o, B, K, H, gate_A,
                                                         g_min, stream);
}

template <typename DT>
hipError_t launch_step_wave(int mode, const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const int32_t* n_accept, float* state, void* o, int B, int K,
                            int H, int dk, int dv, hipStream_t stream, const float* gate_A = nullptr,
                            float g_min = -5.f)
{
#define KDA_STEP(DKV, DVV)                                                                                       \
    if (dk == DKV && dv == DVV)                                                                                  \
        return launch_step_wave_shape<DT, DKV, DVV>(mode, q, k, v, g, beta, n_accept, state, o, B, K, H, gate_A, \
                                                    g_min, stream);
    KDA_STEP(32, 32) KDA_STEP(32, 64) KDA_STEP(32, 128)
    KDA_STEP(64, 32) KDA_STEP(64, 64) KDA_STEP(64, 128)
    KDA_STEP(128, 32) KDA_STEP(128, 64) KDA_STEP(128, 128)
#undef KDA_STEP
    return hipErrorInvalidValue;
}

}  // namespace kda
