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
//
// Segments run in parallel, as in the forward's segment composition: the
// step dS_prev = F^T (dS + q dO^T), F = (I - beta k k^T) Diag(a) the forward
// transition, is affine in dS and needs no forward state.  So for a segment
// dS_start = M^T dS_end + C, with M the segment's forward transition and C the
// segment's own contribution (dS_end = 0).  A summary pass computes [C | M^T]
// per (segment, head) by running that step on an extended dS whose extra
// d_k columns start as the identity and see no dO; a scan takes
// dS_start = M^T dS_end + C backwards over each sequence's segments; the full
// backward then runs every segment from its true dS_end, in parallel.
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
    int64_t Lseg;           // tokens per segment (a multiple of BWD_CHUNK)
    float* cm;              // per (segment, head): C [dk][dv] then M^T [dk][dk], fp32
    float* dsend;           // per (segment, head): dS at the segment's end [dk][dv], fp32
};

// Where segment `seg` (0 .. total) of the packed sequences lies.  Offsets are
// clamped into [0, T_total] and made non-decreasing, as the prefill's planner
// does; every sequence has at least one segment.  n = -1 past the last one.
struct SegLoc {
    int n = -1, s = 0, nseg = 0, seg0 = 0;  // sequence, segment in it, its segment count and first index
    int64_t c0 = 0, c1 = 0;                 // the sequence's tokens
    int64_t t0 = 0, t1 = 0;                 // the segment's tokens
    int64_t ck0 = 0;                        // the sequence's first checkpoint row
};

__device__ inline int64_t seg_count(int64_t len, int64_t Lseg) { return len <= 0 ? 1 : (len + Lseg - 1) / Lseg; }

__device__ inline SegLoc bwd_locate(const BackwardArgs& a, int seg)
{
    SegLoc L;
    int64_t prev = 0, ck = 0;
    int acc = 0;
    for (int m = 0; m < a.N; ++m) {
        int64_t x = a.cu ? int64_t(a.cu[m + 1]) : a.T_total;
        x = x < 0 ? 0 : (x > a.T_total ? a.T_total : x);
        x = x < prev ? prev : x;
        const int ns = int(seg_count(x - prev, a.Lseg));
        if (seg < acc + ns) {
            L.n = m;
            L.s = seg - acc;
            L.nseg = ns;
            L.seg0 = acc;
            L.c0 = prev;
            L.c1 = x;
            L.t0 = prev + int64_t(L.s) * a.Lseg;
            L.t1 = L.t0 + a.Lseg < x ? L.t0 + a.Lseg : x;
            if (L.t0 > x) L.t0 = x;
            L.ck0 = ck;
            return L;
        }
        acc += ns;
        ck += (x - prev) / BWD_CHUNK;
        prev = x;
    }
    return L;
}

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

    // items are (segment, head) pairs; the loop ends at the first segment past the last sequence
    for (int item = blockIdx.x;; item += gridDim.x) {
        const int h = item % H;
        const SegLoc L = bwd_locate(a, item / H);
        if (L.n < 0) break;
        const int n = L.n;
        const int64_t c0 = L.c0, ck0 = L.ck0;
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

        // dS starts as the gradient at the segment's end (the scan's result)
        f32x4 dS[R];
        load_state(dS, a.dsend + int64_t(item) * DK * DV);
        // the segment's 64-token chunks, numbered within the sequence
        const int64_t j0 = (L.t0 - c0) / BWD_CHUNK, j1 = (L.t1 - c0 + BWD_CHUNK - 1) / BWD_CHUNK;
        for (int64_t j = j1 - 1; j >= j0; --j) {
            const int64_t t0 = c0 + j * BWD_CHUNK;
            const int clen = int((L.t1 - t0) < BWD_CHUNK ? (L.t1 - t0) : BWD_CHUNK);
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
        __syncthreads();  // every wave is done with the reduction buffers before the next item
    }
}

// Summary pass: one workgroup per (segment, head), one wave per 32 columns of
// the extended dS = [dS | N] (d_v + d_k columns).  Runs dS_prev =
// Diag(a) (I - beta k k^T) (dS + q dO^T) over the segment backwards from
// [dS_end | I] with dS_end = 0 (the sequence's last segment: the final
// state's gradient) and no dO on the N columns, giving [C | M^T].  The last
// segment needs no M^T.  No forward state, no scratch, no barrier.
template <typename DT, int DK, int DV>
__global__ void __launch_bounds__(64 * ((DV + DK) / 32)) bwd_summary_kernel(BackwardArgs a)
{
    constexpr int R = DK / 8;
    using ST = typename DT::storage;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cgl = lane & 7, rg = lane >> 3;
    const int r0 = rg * R;
    const int H = a.H;
    const int item = blockIdx.x, h = item % H;
    const SegLoc L = bwd_locate(a, item / H);
    if (L.n < 0) return;
    const bool last = L.s == L.nseg - 1;
    const bool mcols = wave >= DV / 32;  // a wave of the N (identity) columns
    if (mcols && last) return;
    const int col = (mcols ? wave - DV / 32 : wave) * 32 + 4 * cgl;  // column within its part
    const ST* q = static_cast<const ST*>(a.q);
    const ST* k = static_cast<const ST*>(a.k);
    const ST* g = static_cast<const ST*>(a.g);
    const ST* beta = static_cast<const ST*>(a.beta);
    const ST* dO = static_cast<const ST*>(a.d_o);
    f32x4 X[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (mcols) {
#pragma unroll
            for (int m = 0; m < 4; ++m) X[r][m] = (r0 + r == col + m) ? 1.f : 0.f;
        } else if (last && a.d_fin) {
            X[r] = *reinterpret_cast<const f32x4*>(a.d_fin + (int64_t(L.n) * H + h) * DK * DV + (r0 + r) * DV + col);
        } else {
            X[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    for (int64_t t = L.t1 - 1; t >= L.t0; --t) {
        const int64_t th = t * H + h;
        float gg[R], kk[R], qq[R];
        bwd_load_rows<DT, R>(g + th * DK + r0, gg);
        bwd_load_rows<DT, R>(k + th * DK + r0, kk);
        f32x4 dOv = {0.f, 0.f, 0.f, 0.f};
        if (!mcols && dO) {
            bwd_load_rows<DT, R>(q + th * DK + r0, qq);
#pragma unroll
            for (int m = 0; m < 4; ++m) dOv[m] = load_elem<DT>(dO + th * DV + col, m);
#pragma unroll
            for (int r = 0; r < R; ++r) X[r] += qq[r] * dOv;
        }
        f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < R; ++r) du += kk[r] * X[r];
#pragma unroll
        for (int m = 0; m < 4; ++m) du[m] = sum_rows(du[m], lane);
        const float bt = load_elem<DT>(beta, th);
#pragma unroll
        for (int r = 0; r < R; ++r) X[r] = __expf(gg[r]) * (X[r] - (bt * kk[r]) * du);
    }
    float* out = a.cm + int64_t(item) * (DK * DV + DK * DK) + (mcols ? DK * DV : 0);
    const int ld = mcols ? DK : DV;
#pragma unroll
    for (int r = 0; r < R; ++r) *reinterpret_cast<f32x4*>(out + (r0 + r) * ld + col) = X[r];
}

// Scan: one workgroup of 256 threads per (sequence, head, 32 columns of dS).
// Backwards over the sequence's segments: dS_end of segment s is dS_start of
// segment s + 1, and dS_start(s) = M_s^T dS_end(s) + C_s, in fp32.  Writes
// every segment's dS_end for the full pass and the initial state's gradient.
template <int DK, int DV>
__global__ void __launch_bounds__(256) bwd_scan_kernel(BackwardArgs a)
{
    constexpr int RPT = DK / 8;  // rows per thread (8 row groups x 32 columns)
    __shared__ float sd[DK][33];
    const int H = a.H;
    const int slice = blockIdx.x % (DV / 32), unit = blockIdx.x / (DV / 32);
    const int n = unit / H, h = unit % H;
    const int t = threadIdx.x, jj = t & 31, rgp = t >> 5;
    const int col = slice * 32 + jj;
    // this sequence's segments: the first segment of sequence n is the sum of
    // the earlier sequences' counts
    int seg0 = 0, nseg = 1;
    {
        int64_t prev = 0;
        for (int m = 0; m <= n; ++m) {
            int64_t x = a.cu ? int64_t(a.cu[m + 1]) : a.T_total;
            x = x < 0 ? 0 : (x > a.T_total ? a.T_total : x);
            x = x < prev ? prev : x;
            const int ns = int(seg_count(x - prev, a.Lseg));
            if (m < n) seg0 += ns;
            else nseg = ns;
            prev = x;
        }
    }
    auto cm_of = [&](int s) { return a.cm + (int64_t(seg0 + s) * H + h) * (DK * DV + DK * DK); };
    auto dsend_of = [&](int s) { return a.dsend + (int64_t(seg0 + s) * H + h) * DK * DV; };
    // the last segment ends at the final state: its dS_end is the final state's gradient
    for (int r = rgp; r < DK; r += 8) {
        dsend_of(nseg - 1)[r * DV + col] = a.d_fin ? a.d_fin[unit * int64_t(DK) * DV + r * DV + col] : 0.f;
        sd[r][jj] = cm_of(nseg - 1)[r * DV + col];  // dS_start of the last segment
    }
    __syncthreads();
    for (int s = nseg - 2; s >= 0; --s) {
        const float* C = cm_of(s);
        const float* MT = C + DK * DV;
        float acc[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rgp * RPT + i;
            float x = C[r * DV + col];
            for (int c = 0; c < DK; ++c) x += MT[r * DK + c] * sd[c][jj];
            acc[i] = x;
        }
        for (int r = rgp; r < DK; r += 8) dsend_of(s)[r * DV + col] = sd[r][jj];
        __syncthreads();  // every thread has read dS_end(s)
#pragma unroll
        for (int i = 0; i < RPT; ++i) sd[rgp * RPT + i][jj] = acc[i];
        __syncthreads();
    }
    for (int r = rgp; r < DK; r += 8) a.d_init[unit * int64_t(DK) * DV + r * DV + col] = sd[r][jj];
}

struct BwdPlan {
    int64_t Lseg = 0, segs_max = 0;
    int grid = 0;
    size_t off_scratch = 0, off_cm = 0, off_dsend = 0, bytes = 0;
};

// Segment length: enough (segment, head) items to cover the compute units
// about once (each runs its tokens one by one), at least one 64-token chunk.
inline BwdPlan backward_plan(int64_t T_total, int N, int H, int dk, int dv)
{
    BwdPlan p;
    const int64_t T = T_total > 0 ? T_total : 1;
    if (int64_t(N) * H >= BWD_MAX_WG / 2) {
        p.Lseg = (T + BWD_CHUNK - 1) / BWD_CHUNK * BWD_CHUNK;  // one segment per sequence
    } else {
        const int64_t per = (T * H + int64_t(BWD_MAX_WG) * BWD_CHUNK - 1) / (int64_t(BWD_MAX_WG) * BWD_CHUNK);
        p.Lseg = BWD_CHUNK * (per > 0 ? per : 1);
    }
    if (const char* e = getenv("KDA_BWD_SEG_TOKENS")) {  // tests: force a segment length
        const long v = atol(e);
        if (v > 0) p.Lseg = (v + BWD_CHUNK - 1) / BWD_CHUNK * BWD_CHUNK;
    }
    p.segs_max = T / p.Lseg + 1 + N;  // >= the sum over sequences of max(1, ceil(len / Lseg))
    const int64_t items = p.segs_max * H;
    p.grid = int(items < BWD_MAX_WG ? items : BWD_MAX_WG);
    size_t off = 0;
    p.off_scratch = off;
    off = align256(off + size_t(p.grid) * BWD_CHUNK * size_t(dk) * dv * sizeof(float));
    p.off_cm = off;
    off = align256(off + size_t(items) * (size_t(dk) * dv + size_t(dk) * dk) * sizeof(float));
    p.off_dsend = off;
    off = align256(off + size_t(items) * dk * dv * sizeof(float));
    p.bytes = off;
    return p;
}

template <typename DT, int DK, int DV>
hipError_t launch_backward_t(BackwardArgs a, const BwdPlan& plan, hipStream_t stream)
{
    unsigned char* ws = reinterpret_cast<unsigned char*>(a.scratch);
    a.Lseg = plan.Lseg;
    a.scratch = reinterpret_cast<float*>(ws + plan.off_scratch);
    a.cm = reinterpret_cast<float*>(ws + plan.off_cm);
    a.dsend = reinterpret_cast<float*>(ws + plan.off_dsend);
    hipLaunchKernelGGL((bwd_summary_kernel<DT, DK, DV>), dim3(unsigned(plan.segs_max * a.H)),
                       dim3(64 * ((DV + DK) / 32)), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_scan_kernel<DK, DV>), dim3(unsigned(a.N * a.H * (DV / 32))), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((backward_kernel<DT, DK, DV>), dim3(unsigned(plan.grid)), dim3(64 * (DV / 32)), 0, stream, a);
    return hipGetLastError();
}

template <typename DT>
hipError_t launch_backward(const BackwardArgs& a, const BwdPlan& plan, int dk, int dv, hipStream_t stream)
{
#define KDA_BWD(DKV, DVV) \
    if (dk == DKV && dv == DVV) return launch_backward_t<DT, DKV, DVV>(a, plan, stream);
    KDA_BWD(32, 32) KDA_BWD(32, 64) KDA_BWD(32, 128)
    KDA_BWD(64, 32) KDA_BWD(64, 64) KDA_BWD(64, 128)
    KDA_BWD(128, 32) KDA_BWD(128, 64) KDA_BWD(128, 128)
#undef KDA_BWD
    return hipErrorInvalidValue;
}

}  // namespace kda
