// kda_bwd_chunk: the backward of the KDA recurrence in chunk form, on the
// matrix cores.
//
// Sources: "NLP——技术报告解读-Kimi-K3", Model Architecture / Kimi Delta
// Attention (KDA) (the step, the read-out and the bounded decay g >= -5 that
// keeps every decay ratio of a 16-token span inside fp32 range; the pages give
// no backward, so this is the chain rule applied to the forward's chunk form)
// and Infrastructure / KDA algorithm-system co-design (the chunkwise kernel
// serves training as well; inside a chunk in parallel, chunk to chunk in
// series).
//
// Per sub-chunk of n <= 16 tokens, with G the running sum of g from the
// sub-chunk's start (per key channel), G_last its last row, gamma = e^{G_last},
// the incoming state S and
//   K^ = K.e^{G},  K- = K.e^{-G},  Q^ = Q.e^{G},  K~ = K.e^{G_last - G}
// the forward is
//   A' = strict(K^ K-^T),  P = incl(Q^ K-^T),  T = (I + Diag(beta) A')^{-1}
//   X = V - K^ S,  Y = Diag(beta) X,  U = T Y
//   O = Q^ S + P U,  S' = Diag(gamma) S + K~^T U
// and, from dS' (the gradient of S') and dO, the backward is
//   dU = K~ dS' + P^T dO,  dY = T^T dU,  dX = Diag(beta) dY  (= dV)
//   dS = Diag(gamma) dS' + Q^^T dO - K^^T dX                 (to the previous sub-chunk)
//   dA' = -Diag(beta) strict(dY U^T),   dP = incl(dO U^T)
//   dbeta_r = <dY_r, X_r> - sum_{i<r} (dY U^T)_ri A'_ri
//   dQ^ = dO S^T + dP K-,   dK^ = -dX S^T + dA' K-,   dK~ = U dS'^T,   dK- = dA'^T K^ + dP^T Q^
//   dq = dQ^.e^{G},  dk = dK^.e^{G} + dK-.e^{-G} + dK~.e^{G_last - G}
//   dG = dQ^.Q^ + dK^.K^ - dK-.K- - dK~.K~,   dG_last = sum_r dK~.K~ + gamma.rowsum(S.dS')
//   dg_r = dG_last + sum_{r' >= r} dG_r'.
// Rows past the sequence's end have k = q = v = dO = g = beta = 0, so they
// reach no output, state or gradient.
//
// Two kernels, one workgroup per (segment, head) each:
//   - bwd_chunk_summary_kernel: the state-free part only (dU, dY, dX, dS) over
//     an extended dS = [dS | N] whose N columns start as I and see no dO; it
//     gives [C | M^T] of dS_start = M^T dS_end + C for the segment scan.
//   - bwd_chunk_full_kernel: from the segment's true dS_end, every gradient.
//     Per 64-token chunk it runs the forward once from the chunk's checkpoint,
//     keeping the state at each 16-token sub-chunk start in a per-workgroup
//     scratch slot (4 states, not one per token), then takes the sub-chunks in
//     reverse.
// dS (and, in the forward, S) lives in registers as 16x16 accumulator tiles:
// 16 columns per wave in the full pass, 32 in the summary.  Products that
// contract over d_v (dQ^, dK^, dK~, dP) run per 16-channel unit of d_k, one
// unit per wave, with S and dS' staged in LDS.
#pragma once

#include "kda_prefill.hpp"
#include "kda_backward.hpp"

namespace kda {

constexpr int BSUB = 16;                 // tokens per sub-chunk
constexpr int BNSUB = BWD_CHUNK / BSUB;  // sub-chunks per checkpoint chunk

template <typename DT, int DKV, int DVV, bool FULL, bool DSN_LDS_, bool S_LDS_ = false>
struct BwdLayout {
    static constexpr int DK = DKV, DV = DVV;
    static constexpr int NCOL = FULL ? DV : DV + DK;  // dS columns (extended in the summary)
    // 16-column tiles of dS per chain wave: one in the full pass (eight waves,
    // two per SIMD); two in the summary (its 16-wave variant was slower)
    static constexpr int CT = FULL ? 1 : 2;
    static constexpr int NCW = NCOL / (16 * CT);      // waves holding dS columns
    static constexpr int NU = DK / 16;                // 16-channel units of d_k (per-slice products)
    static constexpr int NW = FULL ? (NCW > NU ? NCW : NU) : NCW;
    static constexpr int NT = 64 * NW;
    static constexpr bool DSN_LDS = DSN_LDS_;
    static constexpr bool S_LDS = FULL && S_LDS_;  // the sub-chunk's incoming state staged in LDS for the slices
    using OT = typename Op<DT>::T;
    static constexpr int ES = sizeof(OT);
    static constexpr int PAD = 16 / ES;
    static constexpr int SK = DK + PAD;   // [16][SK]   token-major tiles
    static constexpr int S16 = 16 + PAD;  // [DK][S16]  channel-major tiles, 16x16 tiles
    static constexpr int ST = S16, SD = S16;  // strides diag_inverse reads and writes
    static constexpr int SV = DV + PAD;   // [16][SV] value-side tiles, [DK][SV] dS'
    static constexpr int TK = BSUB * SK * ES;
    static constexpr int TT = DK * S16 * ES;
    static constexpr int TV = BSUB * SV * ES;
    static constexpr int T16 = BSUB * S16 * ES;
    static constexpr int O_KH = 0;                              // K^
    static constexpr int O_KM = O_KH + TK;                      // K-
    static constexpr int O_QH = O_KM + TK;                      // Q^
    static constexpr int O_KT = O_QH + TK;                      // K~
    static constexpr int O_KHT = O_KT + TK;                     // K^^T
    static constexpr int O_KMT = O_KHT + TT;                    // K-^T (backward) or K~^T (forward sub-chunks)
    static constexpr int O_QHT = O_KMT + (FULL ? TT : 0);       // Q^^T
    static constexpr int O_VY = O_QHT + TT;                     // v, then dY (column by column)
    static constexpr int O_DO = O_VY + (FULL ? TV : 0);         // dO
    static constexpr int O_U = O_DO + (FULL ? TV : 0);          // U
    static constexpr int O_DOT = O_U + (FULL ? TV : 0);         // dO^T [DV][S16]
    static constexpr int O_DSN = O_DOT + DV * S16 * ES;         // dS' [DK][SV]
    static constexpr int O_SS = O_DSN + ((FULL && DSN_LDS) ? DK * SV * ES : 0);  // S [DK][SV]
    static constexpr int O_QA = O_SS + (S_LDS ? DK * SV * ES : 0);  // -Diag(beta) A'
    static constexpr int O_T = O_QA + T16;                      // T
    static constexpr int O_P = O_T + T16;                       // P
    static constexpr int O_F32 = (O_P + T16 + 15) / 16 * 16;
    static constexpr int O_AP = O_F32;                          // A' fp32 [16][17]
    static constexpr int O_G = O_AP + (FULL ? BSUB * 17 * 4 : 0);  // G fp32 [16][DK]
    static constexpr int O_GAM = O_G + (FULL ? BSUB * DK * 4 : 0);  // gamma [DK]
    static constexpr int O_BETA = O_GAM + DK * 4;               // beta [16]
    static constexpr int O_RB = O_BETA + BSUB * 4;              // dbeta partials [NW][16]
    static constexpr int LDS = O_RB + (FULL ? NW * BSUB * 4 : 0);
};

template <typename DT, int DK, int DV, bool FULL>
struct BwdCfgSel {
    // dS', then the incoming state, go through LDS where they fit; otherwise
    // (fp32 at the larger heads) through scratch slots
    static constexpr bool FIT = BwdLayout<DT, DK, DV, FULL, true>::LDS <= 160 * 1024;
    static constexpr bool FIT_S = BwdLayout<DT, DK, DV, FULL, FIT, true>::LDS <= 160 * 1024;
    using type = BwdLayout<DT, DK, DV, FULL, FIT, FIT_S>;
};
template <typename DT, int DK, int DV, bool FULL>
using BwdCfg = typename BwdCfgSel<DT, DK, DV, FULL>::type;

// state slots per workgroup in the scratch: per sub-chunk start the state as
// the chain waves' accumulator tiles, and row-major too when the slices cannot
// read it from LDS; then dS' when it does not fit in LDS
template <typename DT, int DK, int DV>
constexpr int bwd_slots()
{
    using C = BwdCfg<DT, DK, DV, true>;
    return BNSUB * (C::S_LDS ? 1 : 2) + (C::DSN_LDS ? 0 : 1);
}

// A 16x16x16 operand whose lane (l16 + 16 q4) holds p[l16][4 q4 .. 4 q4 + 3]:
// as A it is the matrix p, as B its transpose.
template <typename O>
__device__ __forceinline__ typename O::Frag4 frag_rows(const typename O::T* p, int stride, int lane)
{
    return O::load4(p + (lane & 15) * stride + 4 * (lane >> 4));
}
// ... holding p[4 q4 + j][l16]: as A the transpose of p, as B p itself.
template <typename O>
__device__ __forceinline__ typename O::Frag4 frag_cols(const typename O::T* p, int stride, int lane)
{
    const int l16 = lane & 15, q4 = lane >> 4;
    f32x4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = O::from_op(p[(4 * q4 + j) * stride + l16]);
    return O::make4(x);
}
template <typename O>
__device__ __forceinline__ f32x4 unpack4(const typename O::Frag4& f)
{
    if constexpr (sizeof(typename O::T) == 2) {
        const u32x2 w = __builtin_bit_cast(u32x2, f);
        return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
    } else {
        return __builtin_bit_cast(f32x4, f);
    }
}

// The lane index, re-read behind an empty asm: values derived from it (LDS
// addresses, masks, lane offsets) are then formed where a phase needs them
// instead of being hoisted to the kernel's start and kept live throughout.
__device__ __forceinline__ int fresh_lane()
{
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
}
__device__ __forceinline__ int fresh_tid()
{
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// sum over the 16 lanes of a row of 16 (lane bits 0..3)
__device__ __forceinline__ float sum16(float x)
{
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

// Lanes per channel in the prep: the largest power of two up to NT / DK,
// at most the sub-chunk's 16 tokens.
constexpr int bwd_prep_parts(int nt, int dk)
{
    int p = 1;
    while (p * 2 <= nt / dk && p * 2 <= BSUB) p *= 2;
    return p;
}

// Every state-independent operand of one sub-chunk (tokens t_s .. t_s + n - 1
// of head h), by the whole workgroup.  FWD: a forward sub-chunk (K~^T in the
// shared slot, no dO or Q^ tiles); otherwise a backward one (K-^T, dO).
template <typename C, typename DT, bool FULL>
__device__ __forceinline__ void bwd_prep(const BackwardArgs& a, unsigned char* sm, int64_t t_s, int n, int h,
                                         bool fwd)
{
    using O = Op<DT>;
    using OT = typename O::T;
    using STG = typename DT::storage;
    constexpr int DK = C::DK, DV = C::DV;
    const int tid = fresh_tid();
    const int64_t H = a.H;
    OT* sKH = reinterpret_cast<OT*>(sm + C::O_KH);
    OT* sKM = reinterpret_cast<OT*>(sm + C::O_KM);
    OT* sQH = reinterpret_cast<OT*>(sm + C::O_QH);
    OT* sKT = reinterpret_cast<OT*>(sm + C::O_KT);
    OT* sKHT = reinterpret_cast<OT*>(sm + C::O_KHT);
    OT* sKMT = reinterpret_cast<OT*>(sm + C::O_KMT);
    OT* sQHT = reinterpret_cast<OT*>(sm + C::O_QHT);
    float* sG = reinterpret_cast<float*>(sm + C::O_G);
    float* sGam = reinterpret_cast<float*>(sm + C::O_GAM);
    const STG* g = static_cast<const STG*>(a.g);
    const STG* k = static_cast<const STG*>(a.k);
    const STG* q = static_cast<const STG*>(a.q);
    // uniform bases at the sub-chunk's first row; lanes add 32-bit offsets
    const int64_t row0 = t_s * H + h;
    const uint32_t rsk = uint32_t(H) * DK, rsv = uint32_t(H) * DV;
    // PARTS adjacent lanes per channel, each over a run of TPT tokens: the
    // running sum of g crosses the runs as a lane scan.  Rows past the end
    // re-read the last valid row (so every load is issued up front) and count as 0.
    constexpr int PARTS = bwd_prep_parts(C::NT, DK), TPT = BSUB / PARTS;
    if (tid < DK * PARTS) {
        const int c = tid / PARTS, part = tid % PARTS, r0 = part * TPT;
        const STG* gb = g + row0 * DK;
        const STG* kb = k + row0 * DK;
        const STG* qb = q + row0 * DK;
        float gr[TPT], kr[TPT], qr[TPT];
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int r = r0 + i;
            const uint32_t off = uint32_t(r < n ? r : n - 1) * rsk + uint32_t(c);
            gr[i] = load_elem<DT>(gb, off);
            kr[i] = load_elem<DT>(kb, off);
            if (!fwd) qr[i] = load_elem<DT>(qb, off);
        }
        float G[TPT];
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            run += r0 + i < n ? gr[i] : 0.f;
            G[i] = run;
        }
        // exclusive prefix over the runs before this one, and the sub-chunk's total
        float incl = run;
#pragma unroll
        for (int d = 1; d < PARTS; d *= 2) {
            const float y = __shfl_up(incl, d, PARTS);
            if (part >= d) incl += y;
        }
        const float total = __shfl(incl, PARTS - 1, PARTS);
        const float excl = incl - run;
        if (part == PARTS - 1) sGam[c] = __expf(total);
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int r = r0 + i;
            const bool ok = r < n;
            const float Gr = excl + G[i];
            if (FULL && !fwd) sG[r * DK + c] = Gr;
            const float kv = ok ? kr[i] : 0.f;
            const float eG = __expf(Gr), eM = __expf(-Gr), eT = __expf(total - Gr);
            const OT kh = O::to_op(kv * eG), km = O::to_op(kv * eM), kt = O::to_op(kv * eT);
            sKH[r * C::SK + c] = kh;
            sKM[r * C::SK + c] = km;
            if (!fwd) {  // the forward sub-chunks read K^ (rows), K- and K~^T only
                sKHT[c * C::S16 + r] = kh;
                sKT[r * C::SK + c] = kt;
            }
            if (FULL) sKMT[c * C::S16 + r] = fwd ? kt : km;
            if (!fwd) {
                const OT qh = O::to_op((ok ? qr[i] : 0.f) * eG);
                sQH[r * C::SK + c] = qh;
                sQHT[c * C::S16 + r] = qh;
            }
        }
    }
    if (FULL || !fwd) {
        // v and dO rows in 8-element units, all loads first
        OT* sV = reinterpret_cast<OT*>(sm + C::O_VY);
        OT* sDO = reinterpret_cast<OT*>(sm + C::O_DO);
        OT* sDOT = reinterpret_cast<OT*>(sm + C::O_DOT);
        const STG* v = static_cast<const STG*>(a.v);
        const STG* dO = static_cast<const STG*>(a.d_o);
        constexpr int UPR = DV / 8, NU = BSUB * UPR, UPT = (NU + C::NT - 1) / C::NT;
        float xv[UPT][8], xd[UPT][8];
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * C::NT;
            if (NU % C::NT == 0 || u < NU) {
                const int r = u / UPR, col = (u % UPR) * 8;
                const uint32_t off = uint32_t(r < n ? r : n - 1) * rsv + uint32_t(col);
                if (FULL) load8<DT>(v + row0 * DV + off, xv[i]);
                if (!fwd && dO) load8<DT>(dO + row0 * DV + off, xd[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * C::NT;
            if (NU % C::NT == 0 || u < NU) {
                const int r = u / UPR, col = (u % UPR) * 8;
                const bool ok = r < n;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (FULL) sV[r * C::SV + col + e] = O::to_op(ok ? xv[i][e] : 0.f);
                    if (!fwd) {
                        const OT d = O::to_op((ok && dO) ? xd[i][e] : 0.f);
                        if (FULL) sDO[r * C::SV + col + e] = d;
                        sDOT[(col + e) * C::S16 + r] = d;
                    }
                }
            }
        }
    }
    if (tid < BSUB) {
        float* sB = reinterpret_cast<float*>(sm + C::O_BETA);
        sB[tid] = tid < n ? load_elem<DT>(static_cast<const STG*>(a.beta) + row0, uint32_t(tid) * uint32_t(H)) : 0.f;
    }
}

// P (lower with the diagonal), by one wave on the matrix cores.
template <typename C, typename DT>
__device__ __forceinline__ void bwd_small_p(unsigned char* sm, int lane)
{
    using O = Op<DT>;
    using OT = typename O::T;
    const int l16 = lane & 15, q4 = lane >> 4;
    const OT* sKM = reinterpret_cast<const OT*>(sm + C::O_KM);
    const OT* sQH = reinterpret_cast<const OT*>(sm + C::O_QH);
    OT* sP = reinterpret_cast<OT*>(sm + C::O_P);
    f32x4 aP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < C::DK / 16; ++kt)
        O::mma4(aP, frag_rows<O>(sQH + 16 * kt, C::SK, lane), frag_rows<O>(sKM + 16 * kt, C::SK, lane));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * q4 + j;
        sP[r * C::S16 + l16] = O::to_op(l16 <= r ? aP[j] : 0.f);
    }
}

// A' (strictly lower), T = (I + Diag(beta) A')^{-1} and, with need_p, P,
// by one wave on the matrix cores.
template <typename C, typename DT, bool FULL>
__device__ __forceinline__ void bwd_small(unsigned char* sm, int lane, bool need_p)
{
    using O = Op<DT>;
    using OT = typename O::T;
    const int l16 = lane & 15, q4 = lane >> 4;
    const OT* sKH = reinterpret_cast<const OT*>(sm + C::O_KH);
    const OT* sKM = reinterpret_cast<const OT*>(sm + C::O_KM);
    const OT* sQH = reinterpret_cast<const OT*>(sm + C::O_QH);
    OT* sQA = reinterpret_cast<OT*>(sm + C::O_QA);
    OT* sT = reinterpret_cast<OT*>(sm + C::O_T);
    OT* sP = reinterpret_cast<OT*>(sm + C::O_P);
    float* sAP = reinterpret_cast<float*>(sm + C::O_AP);
    const float* sB = reinterpret_cast<const float*>(sm + C::O_BETA);
    f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aP = aA;
#pragma unroll
    for (int kt = 0; kt < C::DK / 16; ++kt) {
        const auto bkm = frag_rows<O>(sKM + 16 * kt, C::SK, lane);  // B = K-^T
        O::mma4(aA, frag_rows<O>(sKH + 16 * kt, C::SK, lane), bkm);
        if (need_p) O::mma4(aP, frag_rows<O>(sQH + 16 * kt, C::SK, lane), bkm);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * q4 + j;
        const float av = l16 < r ? aA[j] : 0.f;
        sQA[r * C::S16 + l16] = O::to_op(-sB[r] * av);
        if (need_p) sP[r * C::S16 + l16] = O::to_op(l16 <= r ? aP[j] : 0.f);
        if (FULL) sAP[r * 17 + l16] = av;
    }
    diag_inverse<C, O>(sQA, sT, 0, lane);
}

// The state-free backward step of one sub-chunk for a wave's 32 columns of dS
// (HASDO: the columns see dO).  Returns dY and, through dS, the gradient at
// the sub-chunk's start.  Before the update, hook(dS') sees the incoming dS.
template <typename C, typename DT, bool HASDO, typename Hook>
__device__ __forceinline__ void bwd_dstep(unsigned char* sm, f32x4 (&dS)[C::DK / 16][C::CT], int col0, int lane,
                                          f32x4 (&dY)[C::CT], f32x4 (&dX)[C::CT], Hook&& hook)
{
    using O = Op<DT>;
    using OT = typename O::T;
    const int q4 = lane >> 4, l16 = lane & 15;
    const OT* sKT = reinterpret_cast<const OT*>(sm + C::O_KT);
    const OT* sKHT = reinterpret_cast<const OT*>(sm + C::O_KHT);
    const OT* sQHT = reinterpret_cast<const OT*>(sm + C::O_QHT);
    const OT* sDOT = reinterpret_cast<const OT*>(sm + C::O_DOT);
    const OT* sT = reinterpret_cast<const OT*>(sm + C::O_T);
    const OT* sP = reinterpret_cast<const OT*>(sm + C::O_P);
    const float* sB = reinterpret_cast<const float*>(sm + C::O_BETA);
    const float* sGam = reinterpret_cast<const float*>(sm + C::O_GAM);
    typename O::Frag4 bdo[C::CT];
    if constexpr (HASDO) {
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) bdo[ct] = frag_rows<O>(sDOT + (col0 + 16 * ct) * C::S16, C::S16, lane);  // B = dO
    }
    const auto aTt = frag_cols<O>(sT, C::S16, lane);  // A = T^T
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
        f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < C::DK / 16; ++kt)
            O::mma4(du, frag_rows<O>(sKT + 16 * kt, C::SK, lane), O::make4(dS[kt][ct]));  // K~ dS'
        if constexpr (HASDO) O::mma4(du, frag_cols<O>(sP, C::S16, lane), bdo[ct]);  // + P^T dO
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        O::mma4(y, aTt, O::make4(du));
        dY[ct] = y;
#pragma unroll
        for (int j = 0; j < 4; ++j) dX[ct][j] = sB[4 * q4 + j] * y[j];
    }
    hook();
    typename O::Frag4 ndx[C::CT];
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) ndx[ct] = O::make4(-dX[ct]);
#pragma unroll
    for (int rt = 0; rt < C::DK / 16; ++rt) {
        const auto aq = frag_rows<O>(sQHT + 16 * rt * C::S16, C::S16, lane);  // A = Q^^T
        const auto ak = frag_rows<O>(sKHT + 16 * rt * C::S16, C::S16, lane);  // A = K^^T
        f32x4 gm;
#pragma unroll
        for (int j = 0; j < 4; ++j) gm[j] = sGam[16 * rt + 4 * q4 + j];
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) {
            f32x4 s = gm * dS[rt][ct];
            if constexpr (HASDO) O::mma4(s, aq, bdo[ct]);
            O::mma4(s, ak, ndx[ct]);
            dS[rt][ct] = s;
        }
    }
    (void)l16;
}

// Summary pass: [C | M^T] of dS_start = M^T dS_end + C per (segment, head).
template <typename DT, int DK, int DV>
__global__ void __launch_bounds__((BwdCfg<DT, DK, DV, false>::NT)) bwd_chunk_summary_kernel(BackwardArgs a)
{
    using C = BwdCfg<DT, DK, DV, false>;
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int H = a.H;
    const int item = blockIdx.x, h = item % H;
    const SegLoc L = bwd_locate(a, item / H);
    // a sequence of one segment needs no summary: the full pass gives its
    // initial state's gradient directly
    if (L.n < 0 || L.nseg == 1) return;
    const bool last = L.s == L.nseg - 1;
    constexpr int CT = C::CT, CW = 16 * CT;  // columns per wave
    const bool mcols = wave >= DV / CW;  // a wave of the N (identity) columns
    const bool active = !(mcols && last);
    const int col0 = (mcols ? wave - DV / CW : wave) * CW;
    f32x4 dS[DK / 16][CT];
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * rt + 4 * q4 + j, col = col0 + 16 * ct + l16;
                float x = 0.f;
                if (mcols) x = row == col ? 1.f : 0.f;
                else if (last && a.d_fin) x = a.d_fin[(int64_t(L.n) * H + h) * DK * DV + row * DV + col];
                dS[rt][ct][j] = x;
            }
    if (L.t1 > L.t0) {
        const int64_t m0 = (L.t0 - L.c0) / BSUB, m1 = (L.t1 - 1 - L.c0) / BSUB;
        for (int64_t m = m1; m >= m0; --m) {
            const int64_t t_s = L.c0 + m * BSUB;
            const int n = int(L.t1 - t_s < BSUB ? L.t1 - t_s : BSUB);
            bwd_prep<C, DT, false>(a, sm, t_s, n, h, false);
            __syncthreads();
            if (wave == 0) bwd_small<C, DT, false>(sm, fresh_lane(), false);
            else if (wave == 1) bwd_small_p<C, DT>(sm, fresh_lane());
            __syncthreads();
            if (active) {
                f32x4 dY[CT], dX[CT];
                if (mcols) bwd_dstep<C, DT, false>(sm, dS, col0, fresh_lane(), dY, dX, [] {});
                else bwd_dstep<C, DT, true>(sm, dS, col0, fresh_lane(), dY, dX, [] {});
            }
            __syncthreads();
        }
    }
    if (!active) return;
    const int ln = fresh_lane(), ol16 = ln & 15, oq4 = ln >> 4;
    float* out = a.cm + int64_t(item) * (DK * DV + DK * DK) + (mcols ? DK * DV : 0);
    const int ld = mcols ? DK : DV;
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                out[(16 * rt + 4 * oq4 + j) * ld + col0 + 16 * ct + ol16] = dS[rt][ct][j];
}

// Full pass: every gradient, per (segment, head), from the segment's dS_end.
template <typename DT, int DK, int DV>
__global__ void __launch_bounds__((BwdCfg<DT, DK, DV, true>::NT)) bwd_chunk_full_kernel(BackwardArgs a)
{
    using C = BwdCfg<DT, DK, DV, true>;
    using O = Op<DT>;
    using OT = typename O::T;
    using STG = typename DT::storage;
    constexpr int NCT = DK / 16;
    constexpr int CT = C::CT;  // 16-column tiles per chain wave
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    const int wave = threadIdx.x >> 6;
    const bool chain = wave < C::NCW;  // holds 32 columns of dS
    const int col0 = wave * 16 * CT;
    const int H = a.H;
    const STG* q = static_cast<const STG*>(a.q);
    const STG* k = static_cast<const STG*>(a.k);
    OT* sVY = reinterpret_cast<OT*>(sm + C::O_VY);
    OT* sDO = reinterpret_cast<OT*>(sm + C::O_DO);
    OT* sU = reinterpret_cast<OT*>(sm + C::O_U);
    OT* sDSN = reinterpret_cast<OT*>(sm + C::O_DSN);
    const OT* sKH = reinterpret_cast<const OT*>(sm + C::O_KH);
    const OT* sKMT = reinterpret_cast<const OT*>(sm + C::O_KMT);
    const OT* sKHT = reinterpret_cast<const OT*>(sm + C::O_KHT);
    const OT* sQHT = reinterpret_cast<const OT*>(sm + C::O_QHT);
    const OT* sT = reinterpret_cast<const OT*>(sm + C::O_T);
    const float* sAP = reinterpret_cast<const float*>(sm + C::O_AP);
    const float* sG = reinterpret_cast<const float*>(sm + C::O_G);
    const float* sGam = reinterpret_cast<const float*>(sm + C::O_GAM);
    const float* sB = reinterpret_cast<const float*>(sm + C::O_BETA);
    float* sRB = reinterpret_cast<float*>(sm + C::O_RB);
    // this workgroup's scratch: the state at each sub-chunk start of the
    // current chunk (row-major [DK][DV] fp32), then dS' when it is not in LDS
    float* slots = a.scratch + int64_t(blockIdx.x) * bwd_slots<DT, DK, DV>() * DK * DV;
    float* slotsB = slots + BNSUB * DK * DV;  // row-major copies (when the state is not staged in LDS)
    float* gdsn = slots + BNSUB * (C::S_LDS ? 1 : 2) * DK * DV;
    OT* sS = reinterpret_cast<OT*>(sm + C::O_SS);

    // X = V - K^ S and U = T Diag(beta) X for this wave's columns; S tiles from st(kt, ct)
    auto fwd_xu = [&](auto&& st, f32x4 (&X)[CT], f32x4 (&U)[CT]) {
        const int lane = fresh_lane(), l16 = lane & 15, q4 = lane >> 4;
        const auto aT = frag_rows<O>(sT, C::S16, lane);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < NCT; k4 += 4) {
#pragma unroll
                for (int kt = k4; kt < k4 + 4 && kt < NCT; ++kt)
                    O::mma4(acc, frag_rows<O>(sKH + 16 * kt, C::SK, lane), O::make4(st(kt, ct)));
                __builtin_amdgcn_sched_barrier(0);
            }
            f32x4 y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * q4 + j;
                X[ct][j] = O::from_op(sVY[r * C::SV + col0 + 16 * ct + l16]) - acc[j];
                y[j] = sB[r] * X[ct][j];
            }
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
            O::mma4(u, aT, O::make4(y));
            U[ct] = u;
        }
    };
    // one forward sub-chunk on the register state S (prep and small already done)
    auto fwd_update = [&](f32x4 (&S)[NCT][CT]) {
        f32x4 X[CT], U[CT];
        fwd_xu([&](int kt, int ct) { return S[kt][ct]; }, X, U);
        const int lane = fresh_lane(), q4 = lane >> 4;
        typename O::Frag4 bu[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bu[ct] = O::make4(U[ct]);
#pragma unroll
        for (int rt = 0; rt < NCT; ++rt) {
            const auto ak = frag_rows<O>(sKMT + 16 * rt * C::S16, C::S16, lane);  // A = K~^T
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                f32x4 s;
#pragma unroll
                for (int j = 0; j < 4; ++j) s[j] = sGam[16 * rt + 4 * q4 + j] * S[rt][ct][j];
                O::mma4(s, ak, bu[ct]);
                S[rt][ct] = s;
            }
        }
    };
    auto fwd_sub = [&](f32x4 (&S)[NCT][CT], int64_t t_s, int n, int h) {
        bwd_prep<C, DT, true>(a, sm, t_s, n, h, true);
        __syncthreads();
        if (wave == 0) bwd_small<C, DT, true>(sm, fresh_lane(), false);
        __syncthreads();
        if (chain) fwd_update(S);
        __syncthreads();
    };
    auto store_tiles = [&](const f32x4 (&S)[NCT][CT], float* dst) {
        const int lane = fresh_lane(), l16 = lane & 15, q4 = lane >> 4;
#pragma unroll
        for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    dst[uint32_t((16 * rt + 4 * q4 + j) * DV + col0 + 16 * ct + l16)] = S[rt][ct][j];
    };
    auto load_tiles = [&](f32x4 (&S)[NCT][CT], const float* src) {
        const int lane = fresh_lane(), l16 = lane & 15, q4 = lane >> 4;
#pragma unroll
        for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    S[rt][ct][j] = src ? src[uint32_t((16 * rt + 4 * q4 + j) * DV + col0 + 16 * ct + l16)] : 0.f;
    };

    for (int item = blockIdx.x;; item += gridDim.x) {
        const int h = item % H;
        const SegLoc L = bwd_locate(a, item / H);
        if (L.n < 0) break;
        const int64_t c0 = L.c0, ck0 = L.ck0;
        const int64_t unit = int64_t(L.n) * H + h;
        f32x4 dS[NCT][CT];
        if (chain) load_tiles(dS, a.dsend + int64_t(item) * DK * DV);
        const int64_t j0 = (L.t0 - c0) / BWD_CHUNK, j1 = (L.t1 - c0 + BWD_CHUNK - 1) / BWD_CHUNK;
        for (int64_t j = j1 - 1; j >= j0; --j) {
            const int64_t t0 = c0 + j * BWD_CHUNK;
            const int clen = int((L.t1 - t0) < BWD_CHUNK ? (L.t1 - t0) : BWD_CHUNK);
            const int nsub = (clen + BSUB - 1) / BSUB;
            // the state before token t0: the checkpoint, or recomputed from the initial state
            {
                f32x4 S[NCT][CT];
                const float* init = a.init ? a.init + unit * DK * DV : nullptr;
                const int64_t ckrow = ck0 + j - 1;
                const bool have_ck = j > 0 && a.ckpt && ckrow < a.ckpt_cap;
                if (chain) load_tiles(S, have_ck ? a.ckpt + (ckrow * H + h) * DK * DV : init);
                if (!have_ck)
                    for (int64_t t = c0; t < t0; t += BSUB) fwd_sub(S, t, BSUB, h);
                // forward through the chunk, keeping the state at each sub-chunk start
                for (int s = 0; s < nsub; ++s) {
                    if (chain) {
                        const int lane = fresh_lane(), l16 = lane & 15, q4 = lane >> 4;
                        float* dst = slots + s * DK * DV;  // accumulator tiles, one 16-byte vector per tile
#pragma unroll
                        for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct)
                                *reinterpret_cast<f32x4*>(dst + acc_tile_off<DV>(rt, CT * wave + ct, lane)) = S[rt][ct];
                        if constexpr (!C::S_LDS) {
                            float* dstB = slotsB + s * DK * DV;
#pragma unroll
                            for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
                                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                                    for (int jj = 0; jj < 4; ++jj)
                                        dstB[uint32_t((16 * rt + 4 * q4 + jj) * DV + col0 + 16 * ct + l16)] = S[rt][ct][jj];
                        }
                    }
                    if (s + 1 < nsub) fwd_sub(S, t0 + s * BSUB, BSUB, h);
                }
            }
            __syncthreads();  // every slot is written
            for (int s = nsub - 1; s >= 0; --s) {
                const int64_t t_s = t0 + s * BSUB;
                const int n = clen - s * BSUB < BSUB ? clen - s * BSUB : BSUB;
                const float* SslotA = slots + s * DK * DV;
                const float* Sslot = slotsB + s * DK * DV;  // row-major (when not staged in LDS)
                const int64_t row0 = t_s * H + h;
                const uint32_t rsk = uint32_t(H) * DK, rsv = uint32_t(H) * DV;
                float* dqb = a.dq + row0 * DK;
                float* dkb = a.dk + row0 * DK;
                float* dgb = a.dg + row0 * DK;
                float* dvb = a.dv + row0 * DV;
                bwd_prep<C, DT, true>(a, sm, t_s, n, h, false);
                __syncthreads();
                if (wave == 0) bwd_small<C, DT, true>(sm, fresh_lane(), false);
                else if (wave == 1) bwd_small_p<C, DT>(sm, fresh_lane());
                __syncthreads();
                if (chain) {
                    const int lane = fresh_lane(), l16 = lane & 15, q4 = lane >> 4;
                    f32x4 X[CT], U[CT], dY[CT], dX[CT];
                    f32x4 Sf[NCT][CT];
#pragma unroll
                    for (int kt = 0; kt < NCT; ++kt)
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct)
                            Sf[kt][ct] = *reinterpret_cast<const f32x4*>(SslotA + acc_tile_off<DV>(kt, CT * wave + ct, lane));
                    fwd_xu([&](int kt, int ct) { return Sf[kt][ct]; }, X, U);
                    if constexpr (C::S_LDS) {
                        // the state for the slices' products (row-major, operand precision)
#pragma unroll
                        for (int kt = 0; kt < NCT; ++kt)
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj)
                                    sS[(16 * kt + 4 * q4 + jj) * C::SV + col0 + 16 * ct + l16] = O::to_op(Sf[kt][ct][jj]);
                    }
                    bwd_dstep<C, DT, true>(sm, dS, col0, lane, dY, dX, [&] {
                        // dS' for the per-slice products, before dS moves on
#pragma unroll
                        for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj) {
                                    const int row = 16 * rt + 4 * q4 + jj, col = col0 + 16 * ct + l16;
                                    if constexpr (C::DSN_LDS) sDSN[row * C::SV + col] = O::to_op(dS[rt][ct][jj]);
                                    else gdsn[uint32_t(row * DV + col)] = dS[rt][ct][jj];
                                }
                    });
                    // dv = dX; dbeta's <dY, X> part; U and dY for the slices
                    float pb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int r = 4 * q4 + jj, col = col0 + 16 * ct + l16;
                            if (r < n) dvb[uint32_t(r) * rsv + uint32_t(col)] = dX[ct][jj];
                            pb[jj] += dY[ct][jj] * X[ct][jj];
                            sU[r * C::SV + col] = O::to_op(U[ct][jj]);
                            sVY[r * C::SV + col] = O::to_op(dY[ct][jj]);
                        }
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float s = sum16(pb[jj]);
                        if (l16 == 0) sRB[wave * BSUB + 4 * q4 + jj] = s;
                    }
                }
                __syncthreads();
                if (wave < C::NU) {
                    const int lane = fresh_lane(), l16 = lane & 15, q4 = lane >> 4;
                    const int ch0 = 16 * wave, c = ch0 + l16;  // this wave's 16 channels
                    // raw k and q of this lane's elements (rows past the end re-read the last one)
                    float kq[4][2];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r = 4 * q4 + jj;
                        const uint32_t off = uint32_t(r < n ? r : n - 1) * rsk + uint32_t(c);
                        kq[jj][0] = load_elem<DT>(k + row0 * DK, off);
                        kq[jj][1] = load_elem<DT>(q + row0 * DK, off);
                    }
                    // dP = incl(dO U^T), dA' = -Diag(beta) strict(dY U^T), each with its transpose
                    f32x4 dP = {0.f, 0.f, 0.f, 0.f}, dPT = dP, M1 = dP, M1T = dP;
#pragma unroll
                    for (int kt = 0; kt < DV / 16; ++kt) {
                        const auto fo = frag_rows<O>(sDO + 16 * kt, C::SV, lane);
                        const auto fu = frag_rows<O>(sU + 16 * kt, C::SV, lane);
                        const auto fy = frag_rows<O>(sVY + 16 * kt, C::SV, lane);
                        O::mma4(dP, fo, fu);
                        O::mma4(dPT, fu, fo);
                        O::mma4(M1, fy, fu);
                        O::mma4(M1T, fu, fy);
                    }
                    float tb[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r4 = 4 * q4 + jj;
                        const float m1 = M1[jj];
                        tb[jj] = l16 < r4 ? -m1 * sAP[r4 * 17 + l16] : 0.f;
                        dP[jj] = l16 <= r4 ? dP[jj] : 0.f;
                        dPT[jj] = r4 <= l16 ? dPT[jj] : 0.f;
                        M1[jj] = l16 < r4 ? -sB[r4] * m1 : 0.f;
                        M1T[jj] = r4 < l16 ? -sB[l16] * M1T[jj] : 0.f;
                    }
                    if (wave == 0) {
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const float s = sum16(tb[jj]);
                            const int r = 4 * q4 + jj;
                            if (l16 == 0 && r < n) {
                                float t = s;
                                for (int w2 = 0; w2 < C::NCW; ++w2) t += sRB[w2 * BSUB + r];
                                a.dbeta[row0 + uint32_t(r) * uint32_t(H)] = t;
                            }
                        }
                    }
                    const auto fdP = O::make4(dPT);   // A = dP
                    const auto fdPT = O::make4(dP);   // A = dP^T
                    const auto fdA = O::make4(M1T);   // A = dA'
                    const auto fdAT = O::make4(M1);   // A = dA'^T
                    f32x4 aQ = {0.f, 0.f, 0.f, 0.f}, aK = aQ, aT = aQ;
                    float dot = 0.f;
#pragma unroll
                    for (int kt = 0; kt < DV / 16; ++kt) {
                        f32x4 sv;
                        typename O::Frag4 bs;  // B = S^T
                        if constexpr (C::S_LDS) {
                            bs = O::load4(sS + c * C::SV + 16 * kt + 4 * q4);
                            sv = unpack4<O>(bs);
                        } else {
                            sv = *reinterpret_cast<const f32x4*>(Sslot + uint32_t(c * DV + 16 * kt + 4 * q4));
                            bs = O::make4(sv);
                        }
                        typename O::Frag4 bd;  // B = dS'^T
                        f32x4 dv;
                        if constexpr (C::DSN_LDS) {
                            bd = O::load4(sDSN + c * C::SV + 16 * kt + 4 * q4);
                            dv = unpack4<O>(bd);
                        } else {
                            dv = *reinterpret_cast<const f32x4*>(gdsn + uint32_t(c * DV + 16 * kt + 4 * q4));
                            bd = O::make4(dv);
                        }
                        dot += sv[0] * dv[0] + sv[1] * dv[1] + sv[2] * dv[2] + sv[3] * dv[3];
                        O::mma4(aQ, frag_rows<O>(sDO + 16 * kt, C::SV, lane), bs);
                        O::mma4(aK, frag_rows<O>(sVY + 16 * kt, C::SV, lane), bs);
                        O::mma4(aT, frag_rows<O>(sU + 16 * kt, C::SV, lane), bd);
                    }
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) aK[jj] *= -sB[4 * q4 + jj];
                    const auto bkm = frag_rows<O>(sKMT + ch0 * C::S16, C::S16, lane);  // B = K-
                    O::mma4(aQ, fdP, bkm);
                    O::mma4(aK, fdA, bkm);
                    f32x4 aM = {0.f, 0.f, 0.f, 0.f};
                    O::mma4(aM, fdAT, frag_rows<O>(sKHT + ch0 * C::S16, C::S16, lane));  // dA'^T K^
                    O::mma4(aM, fdPT, frag_rows<O>(sQHT + ch0 * C::S16, C::S16, lane));  // + dP^T Q^
                    const float Gl = sG[(BSUB - 1) * DK + c];
                    float gl = 0.f, dGr[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r = 4 * q4 + jj;
                        const bool ok = r < n;
                        const uint32_t off = uint32_t(r) * rsk + uint32_t(c);
                        const float kv = ok ? kq[jj][0] : 0.f;
                        const float qv = ok ? kq[jj][1] : 0.f;
                        const float G = sG[r * DK + c];
                        const float eG = __expf(G), eM = __expf(-G), eT = __expf(Gl - G);
                        const float Qh = qv * eG, Kh = kv * eG, Km = kv * eM, Kt = kv * eT;
                        const float dq = aQ[jj] * eG;
                        const float dk = aK[jj] * eG + aM[jj] * eM + aT[jj] * eT;
                        const float dG = aQ[jj] * Qh + aK[jj] * Kh - aM[jj] * Km - aT[jj] * Kt;
                        gl += aT[jj] * Kt;
                        if (ok) {
                            dqb[off] = dq;
                            dkb[off] = dk;
                        }
                        dGr[jj] = dG;
                    }
                    float tot = gl + sGam[c] * dot;
                    tot += xor_lanes(tot, 16, lane);
                    tot += xor_lanes(tot, 32, lane);
                    // dg: reverse running sum over the sub-chunk's rows (this lane's
                    // four, then the row groups after it), plus dG_last
                    float suf[4];
                    suf[3] = dGr[3];
#pragma unroll
                    for (int jj = 2; jj >= 0; --jj) suf[jj] = suf[jj + 1] + dGr[jj];
                    float after = 0.f;
#pragma unroll
                    for (int qq = 1; qq < 4; ++qq) {
                        const float b = __shfl(suf[0], l16 + 16 * qq, 64);
                        after += qq > q4 ? b : 0.f;
                    }
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r = 4 * q4 + jj;
                        if (r < n) dgb[uint32_t(r) * rsk + uint32_t(c)] = tot + after + suf[jj];
                    }
                }
                __syncthreads();
            }
        }
        // the first segment of a sequence ends at the initial state's gradient
        if (L.s == 0 && chain) store_tiles(dS, a.d_init + unit * DK * DV);
    }
}

template <typename DT, int DK, int DV>
hipError_t launch_bwd_chunk(const BackwardArgs& a, const BwdPlan& plan, hipStream_t stream)
{
    using C1 = BwdCfg<DT, DK, DV, false>;
    using C3 = BwdCfg<DT, DK, DV, true>;
    auto k1 = bwd_chunk_summary_kernel<DT, DK, DV>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C1::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k1, dim3(unsigned(plan.segs_max * a.H)), dim3(C1::NT), C1::LDS, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    auto ks = bwd_scan_kernel<DK, DV>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(ks), hipFuncAttributeMaxDynamicSharedMemorySize,
                            BwdScanCfg<DK>::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ks, dim3(unsigned(a.N * a.H * (DV / BWD_SCAN_COLS))), dim3(256), BwdScanCfg<DK>::LDS, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    auto k3 = bwd_chunk_full_kernel<DT, DK, DV>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k3), hipFuncAttributeMaxDynamicSharedMemorySize, C3::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k3, dim3(unsigned(plan.grid)), dim3(C3::NT), C3::LDS, stream, a);
    return hipGetLastError();
}

template <typename DT>
hipError_t launch_backward(const BackwardArgs& a, const BwdPlan& plan, int dk, int dv, hipStream_t stream)
{
    BackwardArgs b = a;
    unsigned char* ws = reinterpret_cast<unsigned char*>(a.scratch);
    b.Lseg = plan.Lseg;
    b.scratch = reinterpret_cast<float*>(ws + plan.off_scratch);
    b.cm = reinterpret_cast<float*>(ws + plan.off_cm);
    b.dsend = reinterpret_cast<float*>(ws + plan.off_dsend);
#define KDA_BWD(DKV, DVV) \
    if (dk == DKV && dv == DVV) return launch_bwd_chunk<DT, DKV, DVV>(b, plan, stream);
    KDA_BWD(32, 32) KDA_BWD(32, 64) KDA_BWD(32, 128)
    KDA_BWD(64, 32) KDA_BWD(64, 64) KDA_BWD(64, 128)
    KDA_BWD(128, 32) KDA_BWD(128, 64) KDA_BWD(128, 128)
#undef KDA_BWD
    return hipErrorInvalidValue;
}

}  // namespace kda
