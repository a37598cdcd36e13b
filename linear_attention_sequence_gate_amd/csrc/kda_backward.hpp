// kda_backward: gradients of the KDA recurrence for training.
//
// Sources: "NLP——技术报告解读-Kimi-K3", Model Architecture / Kimi Delta
// Attention (KDA) (the state update and read-out; the pages give no backward,
// so it is the chain rule applied to that step), and Infrastructure / KDA
// algorithm-system co-design (FlashKDA serves training as well as inference).
//
// For L = sum_t <dO_t, o_t> + <dS_fin, S_T>, per token, with a = exp(g),
// Sp = Diag(a) S_prev, r = v - Sp^T k, u = beta r, S = Sp + k u^T, o = S^T q:
//   dS += q dO^T,   dq = S dO,   du = dS^T k,   dv = beta du,   dbeta = <du, r>,
//   dw = -beta du,  dk = dS u + Sp dw,  dSp = dS + k dw^T,
//   dg_c = a_c <dSp[c,:], S_prev[c,:]>,   dS_prev = Diag(a) dSp.
// Like the forward, dS evolves column by column: column j of dS needs only
// column j of the states and the per-token scalars and vectors.  So the
// layout is the one-wave step kernel's: one workgroup per (sequence, head),
// one wave per 32 state columns, lane = 8 rg + c holding 4 columns of d_k / 8
// rows of both S and dS in registers.  Sums over d_k (du, and r through
// Sp^T k) are three lane exchanges inside the wave; sums over d_v (dq, dk, dg,
// dbeta) are three exchanges across the 8 lanes of a row group, then one LDS
// round (one barrier per token) across the waves.
//
// States come backwards chunk by chunk (64 tokens): the chunk's start state
// is the forward's checkpoint (kda_prefill_ckpt at interval 64) or, where
// none is given, is recomputed from the initial state; the chunk is run
// forward once, each state before a token is kept in a per-workgroup scratch
// slot in HBM, and the chunk's tokens are then taken in reverse.
#pragma once

#include "kda_common.hpp"

namespace kda {

constexpr int BWD_CHUNK = 64;  // tokens per backward chunk (the checkpoint interval it reads)
constexpr int BWD_MAX_WG = 256;

struct BackwardArgs {
    const void *q, *k, *v, *g, *beta;
    const int32_t* cu;  // [N + 1] device, or null (one sequence)
    int N;
    int64_t T_total;
    int H;
    const float* init;      // [N, H, dk, dv] or null
    const float* ckpt;      // checkpoints every 64 tokens, or null
    int64_t ckpt_cap;
    const void* d_o;        // [T, H, dv] or null
    const float* d_fin;     // [N, H, dk, dv] or null
    float *dq, *dk, *dv, *dg, *dbeta, *d_init;
    float* scratch;         // [grid][BWD_CHUNK][dk][dv]
};

// the sum over the 8 lanes of a row group, in every lane of the group
// (DPP quad_perm [1,0,3,2] and [2,3,0,1], then the other quad by a lane xor 4)
__device__ __forceinline__ float sum8(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
    x += __shfl_xor(x, 4, 64);
    return x;
}

// the sum over the 8 row groups (lane bits 3..5), in every lane
__device__ __forceinline__ float sum_rows(float x, int lane)
{
    const unsigned u8 = __float_as_uint(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, int(u8), 0x128, 0xf, 0xf, false));  // row_ror:8
    {
        const unsigned u = __float_as_uint(x);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        x += __uint_as_float((lane & 16) ? r[0] : r[1]);
    }
    {
        const unsigned u = __float_as_uint(x);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        x += __uint_as_float(lane >= 32 ? r[0] : r[1]);
    }
    return x;
}

template <typename DT, int R>
__device__ __forceinline__ void bwd_load_rows(const typename DT::storage* p, float (&x)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] = load_elem<DT>(p, r);
}

template <typename DT, int DK, int DV>
__global__ void __launch_bounds__(64 * (DV / 32)) backward_kernel(BackwardArgs a)
{
    constexpr int NS = DV / 32;  // waves (32-column slices)
    constexpr int R = DK / 8;    // rows per lane
    constexpr int NRED = 3 * DK + 1;  // dq, dk, dg rows and dbeta
    static_assert(R == 4 || R == 8 || R == 16, "unsupported shape");
    using ST = typename DT::storage;
    __shared__ float red[2][NS][NRED];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cgl = lane & 7, rg = lane >> 3;
    const int r0 = rg * R;              // first row of the lane
    const int col = wave * 32 + 4 * cgl;  // first column of the lane
    const int H = a.H;
    const ST* q = static_cast<const ST*>(a.q);
    const ST* k = static_cast<const ST*>(a.k);
    const ST* v = static_cast<const ST*>(a.v);
    const ST* g = static_cast<const ST*>(a.g);
    const ST* beta = static_cast<const ST*>(a.beta);
    const ST* dO = static_cast<const ST*>(a.d_o);
    // this workgroup's scratch slot: [token of chunk][wave][row of lane][lane] f32x4
    f32x4* scr = reinterpret_cast<f32x4*>(a.scratch) + int64_t(blockIdx.x) * BWD_CHUNK * (DK * DV / 4);
    auto scr_at = [&](int i, int r) { return scr + ((int64_t(i) * NS + wave) * R + r) * 64 + lane; };

    for (int item = blockIdx.x; item < a.N * H; item += gridDim.x) {
        const int n = item / H, h = item % H;
        // the sequence's tokens and its first checkpoint row (offsets clamped
        // into [0, T_total] and made non-decreasing, as the prefill's planner does)
        int64_t c0 = 0, c1 = a.T_total, ck0 = 0;
        if (a.cu) {
            int64_t prev = 0;
            for (int m = 0; m <= n; ++m) {
                int64_t x = a.cu[m + 1];
                x = x < 0 ? 0 : (x > a.T_total ? a.T_total : x);
                x = x < prev ? prev : x;
                if (m < n) ck0 += (x - prev) / BWD_CHUNK;
                else {
                    c0 = prev;
                    c1 = x;
                }
                prev = x;
            }
        }
        const int64_t len = c1 - c0;
        const int64_t unit = int64_t(n) * H + h;

        // one forward token on S (this lane's rows and columns)
        auto fwd = [&](f32x4 (&S)[R], int64_t t) {
            const int64_t th = t * H + h;
            float gg[R], kk[R];
            bwd_load_rows<DT, R>(g + th * DK + r0, gg);
            bwd_load_rows<DT, R>(k + th * DK + r0, kk);
            f32x4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < R; ++r) {
                S[r] *= __expf(gg[r]);
                w += kk[r] * S[r];
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) w[m] = sum_rows(w[m], lane);
            const float bt = load_elem<DT>(beta, th);
            f32x4 u;
#pragma unroll
            for (int m = 0; m < 4; ++m) u[m] = bt * (load_elem<DT>(v + th * DV + col, m) - w[m]);
#pragma unroll
            for (int r = 0; r < R; ++r) S[r] += kk[r] * u;
        };
        auto load_state = [&](f32x4 (&S)[R], const float* src) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                S[r] = src ? *reinterpret_cast<const f32x4*>(src + (r0 + r) * DV + col) : f32x4{0.f, 0.f, 0.f, 0.f};
        };

        // dS starts as the gradient of the final state
        f32x4 dS[R];
        load_state(dS, a.d_fin ? a.d_fin + unit * DK * DV : nullptr);
        const int64_t nch = (len + BWD_CHUNK - 1) / BWD_CHUNK;
        for (int64_t j = nch - 1; j >= 0; --j) {
            const int64_t t0 = c0 + j * BWD_CHUNK;
            const int clen = int((c1 - t0) < BWD_CHUNK ? (c1 - t0) : BWD_CHUNK);
            // the state before token t0
            f32x4 S[R];
            const float* init = a.init ? a.init + unit * DK * DV : nullptr;
            const int64_t ckrow = ck0 + j - 1;
            if (j > 0 && a.ckpt && ckrow < a.ckpt_cap) {
                load_state(S, a.ckpt + (ckrow * H + h) * DK * DV);
            } else {
                load_state(S, init);
                for (int64_t t = c0; t < t0; ++t) fwd(S, t);  // no checkpoint: from the start
            }
            // forward through the chunk, keeping each state before its token
            for (int i = 0; i < clen; ++i) {
#pragma unroll
                for (int r = 0; r < R; ++r) *scr_at(i, r) = S[r];
                fwd(S, t0 + i);
            }
            // the chunk's tokens in reverse
            for (int i = clen - 1; i >= 0; --i) {
                const int64_t t = t0 + i;
                const int64_t th = t * H + h;
                f32x4 Sprev[R];
#pragma unroll
                for (int r = 0; r < R; ++r) Sprev[r] = *scr_at(i, r);
                float gg[R], kk[R], qq[R], ea[R];
                bwd_load_rows<DT, R>(g + th * DK + r0, gg);
                bwd_load_rows<DT, R>(k + th * DK + r0, kk);
                bwd_load_rows<DT, R>(q + th * DK + r0, qq);
                f32x4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    ea[r] = __expf(gg[r]);
                    w += kk[r] * (ea[r] * Sprev[r]);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) w[m] = sum_rows(w[m], lane);
                const float bt = load_elem<DT>(beta, th);
                f32x4 rv, u, dOv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    rv[m] = load_elem<DT>(v + th * DV + col, m) - w[m];
                    u[m] = bt * rv[m];
                    if (dO) dOv[m] = load_elem<DT>(dO + th * DV + col, m);
                }
                // o = S^T q:  dS += q dO^T,  dq = S dO  (S = Sp + k u^T)
                float pq[R];
                f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const f32x4 Sc = ea[r] * Sprev[r] + kk[r] * u;
                    pq[r] = Sc[0] * dOv[0] + Sc[1] * dOv[1] + Sc[2] * dOv[2] + Sc[3] * dOv[3];
                    dS[r] += qq[r] * dOv;
                    du += kk[r] * dS[r];
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) du[m] = sum_rows(du[m], lane);
                // dv = beta du (one row group writes), dbeta = <du, r>, dw = -beta du
                if (rg == 0)
                    *reinterpret_cast<f32x4*>(a.dv + th * DV + col) = bt * du;
                const float pb = du[0] * rv[0] + du[1] * rv[1] + du[2] * rv[2] + du[3] * rv[3];
                const f32x4 dw = -bt * du;
                // dk = dS u + Sp dw;  dSp = dS + k dw^T;  dg = a <dSp, S_prev>;  dS <- a dSp
                float pk[R], pg[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const f32x4 Sp = ea[r] * Sprev[r];
                    const f32x4 x = dS[r] * u + Sp * dw;
                    pk[r] = x[0] + x[1] + x[2] + x[3];
                    const f32x4 dSp = dS[r] + kk[r] * dw;
                    const f32x4 y = dSp * Sprev[r];
                    pg[r] = ea[r] * (y[0] + y[1] + y[2] + y[3]);
                    dS[r] = ea[r] * dSp;
                }
                // sums over the columns: the 8 lanes of the row group, then the waves
                const int pb_ = int(t & 1);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float sq = sum8(pq[r]), sk = sum8(pk[r]), sg = sum8(pg[r]);
                    if (cgl == 0) {
                        red[pb_][wave][r0 + r] = sq;
                        red[pb_][wave][DK + r0 + r] = sk;
                        red[pb_][wave][2 * DK + r0 + r] = sg;
                    }
                }
                const float sb = sum8(pb);
                if (lane == 0) red[pb_][wave][3 * DK] = sb;
                __syncthreads();
                for (int e = threadIdx.x; e < NRED; e += 64 * NS) {
                    float s = 0.f;
#pragma unroll
                    for (int w2 = 0; w2 < NS; ++w2) s += red[pb_][w2][e];
                    if (e < DK) a.dq[th * DK + e] = s;
                    else if (e < 2 * DK) a.dk[th * DK + e - DK] = s;
                    else if (e < 3 * DK) a.dg[th * DK + e - 2 * DK] = s;
                    else a.dbeta[th] = s;
                }
            }
        }
        // the gradient of the initial state
#pragma unroll
        for (int r = 0; r < R; ++r)
            *reinterpret_cast<f32x4*>(a.d_init + unit * DK * DV + (r0 + r) * DV + col) = dS[r];
        __syncthreads();  // every wave is done with the reduction buffers before the next item
    }
}

inline int backward_grid(int N, int H) { return N * H < BWD_MAX_WG ? N * H : BWD_MAX_WG; }

inline size_t backward_scratch_bytes(int N, int H, int dk, int dv)
{
    return size_t(backward_grid(N, H)) * BWD_CHUNK * size_t(dk) * dv * sizeof(float);
}

template <typename DT, int DK, int DV>
hipError_t launch_backward_t(const BackwardArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((backward_kernel<DT, DK, DV>), dim3(unsigned(backward_grid(a.N, a.H))), dim3(64 * (DV / 32)),
                       0, stream, a);
    return hipGetLastError();
}

template <typename DT>
hipError_t launch_backward(const BackwardArgs& a, int dk, int dv, hipStream_t stream)
{
#define KDA_BWD(DKV, DVV) \
    if (dk == DKV && dv == DVV) return launch_backward_t<DT, DKV, DVV>(a, stream);
    KDA_BWD(32, 32) KDA_BWD(32, 64) KDA_BWD(32, 128)
    KDA_BWD(64, 32) KDA_BWD(64, 64) KDA_BWD(64, 128)
    KDA_BWD(128, 32) KDA_BWD(128, 64) KDA_BWD(128, 128)
#undef KDA_BWD
    return hipErrorInvalidValue;
}

}  // namespace kda
