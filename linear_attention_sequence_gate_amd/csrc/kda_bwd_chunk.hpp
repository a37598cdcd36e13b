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
    static constexpr int O_U = O_DO + TV;                       // U
    static constexpr int O_DSN = O_U + (FULL ? TV : 0);         // dS' [DK][SV]
    static constexpr int O_SS = O_DSN + ((FULL && DSN_LDS) ? DK * SV * ES : 0);  // S [DK][SV]
    static constexpr int O_QA = O_SS + (S_LDS ? DK * SV * ES : 0);  // -Diag(beta) A'
    static constexpr int O_T = O_QA + T16;                      // T
    static constexpr int O_P = O_T + T16;                       // P
    static constexpr int O_F32 = (O_P + T16 + 15) / 16 * 16;
    static constexpr int O_AP = O_F32;                          // A' fp32 [16][17]
    // G fp32 [16][SG]: rows padded by 4 floats, so the rows four apart that one
    // wave touches together start 16 banks apart
    static constexpr int SG = DK + 4;
    static constexpr int O_G = O_AP + (FULL ? BSUB * 17 * 4 : 0);
    static constexpr int O_GAM = O_G + (FULL ? BSUB * SG * 4 : 0);  // gamma [DK]
    static constexpr int O_BETA = O_GAM + DK * 4;               // beta [16]
    static constexpr int O_RB = O_BETA + BSUB * 4;              // dbeta partials [NW][16]
    static constexpr int LDS0 = O_RB + (FULL ? NW * BSUB * 4 : 0);
    // the full pass keeps T and A' of a chunk's forward sub-chunks (all but the
    // last) for the backward sub-chunks of the same tokens, where they fit
    static constexpr int TC_ONE = (T16 + BSUB * 17 * 4 + 15) / 16 * 16;
    static constexpr int O_TC = (LDS0 + 15) / 16 * 16;
    static constexpr bool TCACHE = FULL && O_TC + (BNSUB - 1) * TC_ONE <= 160 * 1024;
    static constexpr int LDS = TCACHE ? O_TC + (BNSUB - 1) * TC_ONE : LDS0;
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
// (DPP rotations inside each row of 16 lanes, on the VALU: no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum16(float x)
{
    x += dpp_row<0x128>(x);  // row_ror:8
    x += dpp_row<0x124>(x);  // row_ror:4
    x += dpp_row<0x122>(x);  // row_ror:2
    x += dpp_row<0x121>(x);  // row_ror:1
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

// N consecutive LDS elements from registers in 16-byte (or smaller) vector
// writes; p is aligned to the write size (N * sizeof(T), or 16 beyond it).
template <int B>
struct LdsVec;
template <>
struct LdsVec<2> { using T = uint16_t; };
template <>
struct LdsVec<4> { using T = uint32_t; };
template <>
struct LdsVec<8> { using T = u32x2; };
template <>
struct LdsVec<16> { using T = u32x4; };
template <typename T, int N>
__device__ __forceinline__ void st_run(T* p, const T (&x)[N])
{
    constexpr int B = N * int(sizeof(T));
    if constexpr (B <= 16) {
        typename LdsVec<B>::T w;
        __builtin_memcpy(&w, x, B);
        *reinterpret_cast<typename LdsVec<B>::T*>(p) = w;
    } else {
        constexpr int M = 16 / int(sizeof(T));
#pragma unroll
        for (int h = 0; h < N / M; ++h) {
            u32x4 w;
            __builtin_memcpy(&w, x + h * M, 16);
            *reinterpret_cast<u32x4*>(p + h * M) = w;
        }
    }
}

// One sub-chunk's raw inputs in a prep thread's registers, loaded ahead of
// their use (the loads stay in flight across the barriers of the sub-chunk
// before).  PARTS adjacent lanes per channel, each over a run of TPT tokens of
// g, k and q; 16-byte units of the v and dO rows; one beta per thread of the
// first BSUB.
template <typename C, typename DT>
struct BwdRaw {
    using STG = typename DT::storage;
    static constexpr int PARTS = bwd_prep_parts(C::NT, C::DK), TPT = BSUB / PARTS;
    static constexpr int EPU = 16 / int(sizeof(STG));           // elements per 16-byte unit
    static constexpr int UPR = C::DV / EPU, NUV = BSUB * UPR;   // units per row, per sub-chunk
    static constexpr int UPT = (NUV + C::NT - 1) / C::NT;       // units per thread
    STG g[TPT], k[TPT], q[TPT];
    u32x4 v[UPT], d[UPT];
    STG b;
    // Wait for these loads here: called before a thread's next global store.
    // A later wait on them (after stores issued since) is counted in one
    // in-order counter with those stores, and would wait for them too.
    __device__ __forceinline__ void settle() const
    {
#pragma unroll
        for (int i = 0; i < TPT; ++i) asm volatile("" ::"v"(g[i]), "v"(k[i]), "v"(q[i]));
#pragma unroll
        for (int i = 0; i < UPT; ++i) asm volatile("" ::"v"(v[i]), "v"(d[i]));
        asm volatile("" ::"v"(b));
    }
};

// Issue the loads of sub-chunk (tokens t_s .. t_s + n - 1 of head h).  FWD
// sub-chunks need no q or dO.  Rows past the end re-read the last valid row,
// so every load stays inside the sequence.
template <typename C, typename DT, bool FULL, bool fwd>
__device__ __forceinline__ void bwd_prep_load(BwdRaw<C, DT>& R, const BackwardArgs& a, int64_t t_s, int n, int h)
{
    using RW = BwdRaw<C, DT>;
    using STG = typename DT::storage;
    constexpr int DK = C::DK, DV = C::DV;
    const int tid = fresh_tid();
    const int64_t H = a.H;
    const int64_t row0 = t_s * H + h;
    KDA_CHECK(t_s >= 0 && t_s + n <= a.T_total, CK_TOKENS);
    KDA_CHECK(n >= 1 && n <= BSUB, CK_BLOCK);
    const uint32_t rsk = uint32_t(H) * DK, rsv = uint32_t(H) * DV;
    if (DK * RW::PARTS >= C::NT || tid < DK * RW::PARTS) {
        const int c = tid / RW::PARTS, part = tid % RW::PARTS, r0 = part * RW::TPT;
        const STG* gb = static_cast<const STG*>(a.g) + row0 * DK;
        const STG* kb = static_cast<const STG*>(a.k) + row0 * DK;
        const STG* qb = static_cast<const STG*>(a.q) + row0 * DK;
#pragma unroll
        for (int i = 0; i < RW::TPT; ++i) {
            const int r = r0 + i;
            const uint32_t off = uint32_t(r < n ? r : n - 1) * rsk + uint32_t(c);
            R.g[i] = gb[off];
            R.k[i] = kb[off];
            if (!fwd) R.q[i] = qb[off];
        }
    }
    if (FULL || !fwd) {
        const STG* v = static_cast<const STG*>(a.v) + row0 * DV;
        const STG* dO = static_cast<const STG*>(a.d_o);
#pragma unroll
        for (int i = 0; i < RW::UPT; ++i) {
            const int u = tid + i * C::NT;
            if (RW::NUV % C::NT == 0 || u < RW::NUV) {
                const int r = u / RW::UPR, col = (u % RW::UPR) * RW::EPU;
                const uint32_t off = uint32_t(r < n ? r : n - 1) * rsv + uint32_t(col);
                if (FULL) R.v[i] = *reinterpret_cast<const u32x4*>(v + off);
                if (!fwd && dO) R.d[i] = *reinterpret_cast<const u32x4*>(dO + row0 * DV + off);
            }
        }
    }
    if (tid < BSUB && tid < n) R.b = static_cast<const STG*>(a.beta)[row0 + int64_t(tid) * H];
}

template <typename DT>
__device__ __forceinline__ float raw_elem(const u32x4& w, int e)
{
    if constexpr (DT::is_bf16) return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    else return __uint_as_float(w[e]);
}

// Every state-independent operand of one sub-chunk from its raw inputs, into
// LDS, by the whole workgroup.  FWD: a forward sub-chunk (K~^T in the shared
// slot, no dO or Q^ tiles); otherwise a backward one (K-^T, dO).
template <typename C, typename DT, bool FULL, bool fwd>
__device__ __forceinline__ void bwd_prep_store(const BwdRaw<C, DT>& R, const BackwardArgs& a, unsigned char* sm, int n)
{
    using O = Op<DT>;
    using OT = typename O::T;
    using RW = BwdRaw<C, DT>;
    constexpr int DK = C::DK;
    const int tid = fresh_tid();
    OT* sKH = reinterpret_cast<OT*>(sm + C::O_KH);
    OT* sKM = reinterpret_cast<OT*>(sm + C::O_KM);
    OT* sQH = reinterpret_cast<OT*>(sm + C::O_QH);
    OT* sKT = reinterpret_cast<OT*>(sm + C::O_KT);
    OT* sKHT = reinterpret_cast<OT*>(sm + C::O_KHT);
    OT* sKMT = reinterpret_cast<OT*>(sm + C::O_KMT);
    OT* sQHT = reinterpret_cast<OT*>(sm + C::O_QHT);
    float* sG = reinterpret_cast<float*>(sm + C::O_G);
    float* sGam = reinterpret_cast<float*>(sm + C::O_GAM);
    auto cvt = [](typename DT::storage x) {
        if constexpr (DT::is_bf16) return bf16_to_f32(x);
        else return float(x);
    };
    // the running sum of g crosses the runs as a lane scan; rows past the end
    // count as 0
    constexpr int PARTS = RW::PARTS, TPT = RW::TPT;
    if (DK * PARTS >= C::NT || tid < DK * PARTS) {
        const int c = tid / PARTS, part = tid % PARTS, r0 = part * TPT;
        float G[TPT];
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            run += r0 + i < n ? cvt(R.g[i]) : 0.f;
            G[i] = run;
        }
        // exclusive prefix over the runs before this one, and the sub-chunk's
        // total: within a quad of lanes by DPP quad permutes, else by shuffles
        float incl = run, total;
        if constexpr (PARTS == 4) {
            const float y1 = dpp_row<0x90>(incl);  // quad_perm [0,0,1,2]
            incl += part >= 1 ? y1 : 0.f;
            const float y2 = dpp_row<0x40>(incl);  // quad_perm [0,0,0,1]
            incl += part >= 2 ? y2 : 0.f;
            total = dpp_row<0xFF>(incl);           // quad_perm [3,3,3,3]
        } else if constexpr (PARTS == 2) {
            const float y1 = dpp_row<0xA0>(incl);  // quad_perm [0,0,2,2]
            incl += part >= 1 ? y1 : 0.f;
            total = dpp_row<0xF5>(incl);           // quad_perm [1,1,3,3]
        } else {
#pragma unroll
            for (int d = 1; d < PARTS; d *= 2) {
                const float y = __shfl_up(incl, d, PARTS);
                if (part >= d) incl += y;
            }
            total = __shfl(incl, PARTS - 1, PARTS);
        }
        const float excl = incl - run;
        const float eTot = __expf(total);  // e^{G_last}, in [e^-80, 1]
        if (part == PARTS - 1) sGam[c] = eTot;
        // token-major tiles element by element; this thread's run of tokens
        // of a channel-major tile in one vector write
        OT khr[TPT], kmtr[TPT], qhr[TPT];
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int r = r0 + i;
            const bool ok = r < n;
            const float Gr = excl + G[i];
            if (FULL && !fwd) sG[r * C::SG + c] = Gr;
            const float kv = ok ? cvt(R.k[i]) : 0.f;
            // e^{G_last - G} = e^{G_last} e^{-G} (<= 1; one exponential less per element)
            const float eG = __expf(Gr), eM = __expf(-Gr), eT = eTot * eM;
            const OT kh = O::to_op(kv * eG), km = O::to_op(kv * eM), kt = O::to_op(kv * eT);
            sKH[r * C::SK + c] = kh;
            sKM[r * C::SK + c] = km;
            if (!fwd) sKT[r * C::SK + c] = kt;  // the forward sub-chunks read K^ (rows), K- and K~^T only
            khr[i] = kh;
            kmtr[i] = fwd ? kt : km;
            if (!fwd) {
                const OT qh = O::to_op((ok ? cvt(R.q[i]) : 0.f) * eG);
                sQH[r * C::SK + c] = qh;
                qhr[i] = qh;
            }
        }
        if (!fwd) st_run(sKHT + c * C::S16 + r0, khr);
        if (FULL) st_run(sKMT + c * C::S16 + r0, kmtr);
        if (!fwd) st_run(sQHT + c * C::S16 + r0, qhr);
    }
    if (FULL || !fwd) {
        // v and dO rows: the 16-byte units as loaded (the operand type is the
        // storage type), zero past the end
        OT* sV = reinterpret_cast<OT*>(sm + C::O_VY);
        OT* sDO = reinterpret_cast<OT*>(sm + C::O_DO);
        const bool has_do = a.d_o != nullptr;
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < RW::UPT; ++i) {
            const int u = tid + i * C::NT;
            if (RW::NUV % C::NT == 0 || u < RW::NUV) {
                const int r = u / RW::UPR, col = (u % RW::UPR) * RW::EPU;
                const bool ok = r < n;
                if (FULL) *reinterpret_cast<u32x4*>(sV + r * C::SV + col) = ok ? R.v[i] : zero;
                if (!fwd) *reinterpret_cast<u32x4*>(sDO + r * C::SV + col) = (ok && has_do) ? R.d[i] : zero;
            }
        }
    }
    if (tid < BSUB) {
        float* sB = reinterpret_cast<float*>(sm + C::O_BETA);
        sB[tid] = tid < n ? cvt(R.b) : 0.f;
    }
}

// Where a prep reads: tokens t .. t + n - 1, forward or backward sub-chunk.
struct BwdPrepAt {
    int64_t t;
    int n;
    bool fwd, valid;
};

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

// T and A' of one sub-chunk between their live tiles and cache slot `slot`
// (put: live -> slot), as 16-byte pieces, by one wave after its own writes
template <typename C>
__device__ __forceinline__ void tcache_copy(unsigned char* sm, int slot, int lane, bool put)
{
    static_assert(C::T16 % 16 == 0 && (BSUB * 17 * 4) % 16 == 0, "16-byte pieces");
    constexpr int NT16 = C::T16 / 16, NAP = BSUB * 17 * 4 / 16;
    unsigned char* kept = sm + C::O_TC + slot * C::TC_ONE;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int i = lane; i < NT16 + NAP; i += 64) {
        unsigned char* live = i < NT16 ? sm + C::O_T + 16 * i : sm + C::O_AP + 16 * (i - NT16);
        u32x4* dst = reinterpret_cast<u32x4*>(put ? kept + 16 * i : live);
        const u32x4* src = reinterpret_cast<const u32x4*>(put ? live : kept + 16 * i);
        *dst = *src;
    }
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
    const OT* sDO = reinterpret_cast<const OT*>(sm + C::O_DO);
    const OT* sT = reinterpret_cast<const OT*>(sm + C::O_T);
    const OT* sP = reinterpret_cast<const OT*>(sm + C::O_P);
    const float* sB = reinterpret_cast<const float*>(sm + C::O_BETA);
    const float* sGam = reinterpret_cast<const float*>(sm + C::O_GAM);
    typename O::Frag4 bdo[C::CT];
    if constexpr (HASDO) {
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) bdo[ct] = frag_cols<O>(sDO + col0 + 16 * ct, C::SV, lane);  // B = dO
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
// WINDOW: per (segment, head), dS at the segment's end from the window of
// a.warm tokens after it (see kda_backward.hpp): written to dsend when the
// window's M^T is exactly zero or the window reaches the sequence end (then it
// starts from d_fin and is exact); otherwise the (segment, head) is flagged.
// A sequence's last segment takes d_fin itself.  Without WINDOW: the
// segment's [C | M^T] for the scan, for the chains a window flagged.
template <typename DT, int DK, int DV, bool WINDOW>
__global__ void __launch_bounds__((BwdCfg<DT, DK, DV, false>::NT)) bwd_chunk_summary_kernel(BackwardArgs a)
{
    using C = BwdCfg<DT, DK, DV, false>;
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    __shared__ int s_live;  // WINDOW: some wave's M^T columns are still non-zero
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int H = a.H;
    const int item = blockIdx.x, h = item % H;
    const SegLoc L = bwd_locate(a, item / H);
    if (L.n < 0) return;
    KDA_CHECK(L.n < a.N, CK_SEQ);
    KDA_CHECK(L.c0 >= 0 && L.c0 <= L.t0 && L.t0 <= L.t1 && L.t1 <= L.c1 && L.c1 <= a.T_total, CK_TOKENS);
    KDA_CHECK(item < a.segs_cap * H, CK_WS);
    const bool last = L.s == L.nseg - 1;
    const int64_t unit = int64_t(L.n) * H + h;
    // the tokens this workgroup runs backwards over, and where dS starts
    int64_t r0 = L.t0, r1 = L.t1;
    bool from_fin = last;  // dS starts at d_fin (else at 0)
    if constexpr (WINDOW) {
        float* dst = a.dsend + int64_t(item) * DK * DV;
        if (last) {  // the sequence's last segment ends at the final state
            const float* src = a.d_fin ? a.d_fin + unit * DK * DV : nullptr;
            for (int e = threadIdx.x; e < DK * DV; e += C::NT) dst[e] = src ? src[e] : 0.f;
            if (threadIdx.x == 0) a.flags[item] = 0;
            return;
        }
        r0 = L.t1;
        r1 = L.t1 + a.warm < L.c1 ? L.t1 + a.warm : L.c1;
        from_fin = r1 == L.c1;
        if (threadIdx.x == 0) s_live = 0;
        __syncthreads();
    } else {
        // a sequence of one segment needs no summary (the full pass gives its
        // initial state's gradient directly), nor does its first segment (the
        // scan stops at the second), nor a chain every window served
        if (L.nseg == 1 || L.s == 0) return;
        if (!bwd_chain_flagged(a, L.seg0, L.nseg, h)) return;
    }
    constexpr int CT = C::CT, CW = 16 * CT;  // columns per wave
    const bool mcols = wave >= DV / CW;  // a wave of the N (identity) columns
    const bool active = !(mcols && from_fin);
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
                else if (from_fin && a.d_fin) x = a.d_fin[unit * DK * DV + row * DV + col];
                dS[rt][ct][j] = x;
            }
    if (r1 > r0) {
        const int64_t m0 = (r0 - L.c0) / BSUB, m1 = (r1 - 1 - L.c0) / BSUB;
        auto sub_len = [&](int64_t m) {
            const int64_t t_s = L.c0 + m * BSUB;
            return int(r1 - t_s < BSUB ? r1 - t_s : BSUB);
        };
        // each sub-chunk's inputs are loaded one sub-chunk ahead (no global
        // stores happen inside the loop, so no wait on them is held up)
        BwdRaw<C, DT> R;
        bwd_prep_load<C, DT, false, false>(R, a, L.c0 + m1 * BSUB, sub_len(m1), h);
        for (int64_t m = m1; m >= m0; --m) {
            bwd_prep_store<C, DT, false, false>(R, a, sm, sub_len(m));
            if (m > m0) bwd_prep_load<C, DT, false, false>(R, a, L.c0 + (m - 1) * BSUB, sub_len(m - 1), h);
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
    if constexpr (WINDOW) {
        // the window's M^T: exactly zero, or the chain goes through the scan
        if (!from_fin) {
            if (mcols) {
                bool nz = false;
#pragma unroll
                for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                        for (int j = 0; j < 4; ++j) nz = nz || (dS[rt][ct][j] != 0.f);
                if (__ballot(nz) != 0 && fresh_lane() == 0) atomicOr(&s_live, 1);
            }
            __syncthreads();
        }
        const bool fail = !from_fin && s_live != 0;
        if (threadIdx.x == 0) a.flags[item] = fail ? 1 : 0;
        if (fail || mcols) return;
        const int ln = fresh_lane(), ol16 = ln & 15, oq4 = ln >> 4;
        float* out = a.dsend + int64_t(item) * DK * DV;
#pragma unroll
        for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    out[(16 * rt + 4 * oq4 + j) * DV + col0 + 16 * ct + ol16] = dS[rt][ct][j];
        return;
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
    // phases (timing build): 0-2 forward sub-chunk prep / small / update,
    // 3 checkpoint load and state slots, 4-7 backward prep / small / chain
    // waves / slices, 8 the item's end
    PhaseClock pclk;
#ifdef KDA_PHASE_TIMING
    pclk.on = threadIdx.x == KDA_PHASE_TID;
    pclk.last = clock64();
#endif

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
    // one forward sub-chunk; prep() puts its operands into LDS; T and A' go to
    // cache slot cslot (when >= 0) for the backward sub-chunk of the same tokens
    auto fwd_sub = [&](f32x4 (&S)[NCT][CT], auto&& prep, int cslot) {
        prep();
        __syncthreads();
        KDA_PHASE(0);
        if (wave == 0) {
            bwd_small<C, DT, true>(sm, fresh_lane(), false);
            if (C::TCACHE && cslot >= 0) tcache_copy<C>(sm, cslot, fresh_lane(), true);
        }
        __syncthreads();
        KDA_PHASE(1);
        if (chain) fwd_update(S);
        __syncthreads();
        KDA_PHASE(2);
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
        KDA_CHECK(L.n < a.N, CK_SEQ);
        KDA_CHECK(L.c0 >= 0 && L.c0 <= L.t0 && L.t0 <= L.t1 && L.t1 <= L.c1 && L.c1 <= a.T_total, CK_TOKENS);
        KDA_CHECK(item < a.segs_cap * H, CK_WS);
        const int64_t c0 = L.c0, ck0 = L.ck0;
        const int64_t unit = int64_t(L.n) * H + h;
        f32x4 dS[NCT][CT];
        if (chain) load_tiles(dS, a.dsend + int64_t(item) * DK * DV);
        const int64_t j0 = (L.t0 - c0) / BWD_CHUNK, j1 = (L.t1 - c0 + BWD_CHUNK - 1) / BWD_CHUNK;
        // Chunk j: its first token, length, sub-chunks, and the checkpoint the
        // state before it is rebuilt from: the nearest one at or before its
        // start that the buffer holds (with interval 64, the one at its start),
        // else the initial state, m = the sequence's checkpoints used.
        auto chunk_t0 = [&](int64_t j) { return c0 + j * BWD_CHUNK; };
        auto chunk_len = [&](int64_t j) {
            const int64_t r = L.t1 - chunk_t0(j);
            return int(r < BWD_CHUNK ? r : BWD_CHUNK);
        };
        auto chunk_ck = [&](int64_t j) {
            int64_t m = j * BWD_CHUNK / a.ckpt_interval;
            if (m > a.ckpt_cap - ck0) m = a.ckpt_cap - ck0;
            return a.ckpt ? m : int64_t(0);
        };
        // The item's sub-chunk preps in order: per chunk (last to first) the
        // forward sub-chunks from the rebuild point up to the chunk's last
        // sub-chunk start, then the chunk's sub-chunks in reverse.  Each prep's
        // loads are issued as soon as the one before has gone into LDS.
        auto first_prep = [&](int64_t j) -> BwdPrepAt {
            const int64_t t0 = chunk_t0(j);
            const int clen = chunk_len(j), nsub = (clen + BSUB - 1) / BSUB;
            const int64_t fend = t0 + int64_t(nsub - 1) * BSUB, m = chunk_ck(j);
            const int64_t from = m >= 1 ? c0 + m * a.ckpt_interval : c0;
            if (from < fend) return {from, BSUB, true, true};
            return {fend, clen - (nsub - 1) * BSUB, false, true};
        };
        auto next_prep = [&](const BwdPrepAt& c, int64_t j) -> BwdPrepAt {
            const int64_t t0 = chunk_t0(j);
            const int clen = chunk_len(j), nsub = (clen + BSUB - 1) / BSUB;
            const int64_t fend = t0 + int64_t(nsub - 1) * BSUB;
            if (c.fwd) {
                if (c.t + BSUB < fend) return {c.t + BSUB, BSUB, true, true};
                return {fend, clen - (nsub - 1) * BSUB, false, true};
            }
            if (c.t > t0) return {c.t - BSUB, BSUB, false, true};
            if (j - 1 >= j0) return first_prep(j - 1);
            return {0, 0, false, false};
        };
        BwdRaw<C, DT> R;
        auto load_prep = [&](const BwdPrepAt& p) {
            if (p.fwd) bwd_prep_load<C, DT, true, true>(R, a, p.t, p.n, h);
            else bwd_prep_load<C, DT, true, false>(R, a, p.t, p.n, h);
        };
        BwdPrepAt cur = {0, 0, false, false};
        if (j1 > j0) {
            cur = first_prep(j1 - 1);
            load_prep(cur);
        }
        auto consume = [&](int64_t j) {
            if (cur.fwd) bwd_prep_store<C, DT, true, true>(R, a, sm, cur.n);
            else bwd_prep_store<C, DT, true, false>(R, a, sm, cur.n);
            const BwdPrepAt nx = next_prep(cur, j);
            if (nx.valid) load_prep(nx);
            cur = nx;
        };
        for (int64_t j = j1 - 1; j >= j0; --j) {
            const int64_t t0 = chunk_t0(j);
            const int clen = chunk_len(j);
            const int nsub = (clen + BSUB - 1) / BSUB;
            // the chunk's start state where it already lies in memory, row-major
            // (its checkpoint row, or the initial state): where the slices read
            // S from LDS, sub-chunk 0 takes it from there and its slot is not written
            const float* s0 = nullptr;
            // the forward's state; after the loop below, the state before the
            // chunk's last sub-chunk, which the backward takes first, from here.
            // With bf16 operands (registers to spare) the state before the one
            // before it stays in registers too (S2).
            constexpr bool KEEP2 = DT::is_bf16;
            f32x4 S[NCT][CT], S2[NCT][CT];
            {
                const float* init = a.init ? a.init + unit * DK * DV : nullptr;
                const int64_t m = chunk_ck(j);
                const int64_t from = m >= 1 ? c0 + m * a.ckpt_interval : c0;
                KDA_CHECK(m < 1 || (ck0 + m - 1 >= 0 && ck0 + m - 1 < a.ckpt_cap), CK_CKPT);
                const float* src = m >= 1 ? a.ckpt + ((ck0 + m - 1) * H + h) * DK * DV : init;
                if (C::S_LDS && from == t0) s0 = src;
                if (chain) load_tiles(S, src);
                for (int64_t t = from; t < t0; t += BSUB) fwd_sub(S, [&] { consume(j); }, -1);
                // forward through the chunk, keeping the state at each sub-chunk start
                for (int s = 0; s < nsub; ++s) {
                    // accumulator-tile slots for all but the last sub-chunk (and
                    // with KEEP2 the one before), and not for sub-chunk 0 where it
                    // reads s0
                    const bool in_s0 = s == 0 && s0, in_s2 = KEEP2 && s == nsub - 2 && !in_s0;
                    const bool acc_slot = s + 1 < nsub && !in_s0 && !in_s2;
                    if (chain && in_s2) {
#pragma unroll
                        for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct) S2[rt][ct] = S[rt][ct];
                    }
                    if (chain && (acc_slot || !C::S_LDS)) {
                        R.settle();
                        const int lane = fresh_lane(), l16 = lane & 15, q4 = lane >> 4;
                        float* dst = slots + s * DK * DV;  // accumulator tiles, one 16-byte vector per tile
                        if (acc_slot) {
#pragma unroll
                            for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
                                for (int ct = 0; ct < CT; ++ct)
                                    *reinterpret_cast<f32x4*>(dst + acc_tile_off<DV>(rt, CT * wave + ct, lane)) =
                                        S[rt][ct];
                        }
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
                    KDA_PHASE(3);
                    if (s + 1 < nsub) fwd_sub(S, [&] { consume(j); }, s);
                }
            }
            __syncthreads();  // every slot is written
            KDA_PHASE(3);
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
                consume(j);
                __syncthreads();
                KDA_PHASE(4);
                // T and A' of the sub-chunks the forward pass ran were kept;
                // the chunk's last sub-chunk computes them here
                if (wave == 0) {
                    if (C::TCACHE && s + 1 < nsub) tcache_copy<C>(sm, s, fresh_lane(), false);
                    else bwd_small<C, DT, true>(sm, fresh_lane(), false);
                } else if (wave == 1) {
                    bwd_small_p<C, DT>(sm, fresh_lane());
                }
                __syncthreads();
                KDA_PHASE(5);
                if (chain) {
                    const int lane = fresh_lane(), l16 = lane & 15, q4 = lane >> 4;
                    f32x4 X[CT], U[CT], dY[CT], dX[CT];
                    f32x4 Sf[NCT][CT];
                    if (s == nsub - 1) {
#pragma unroll
                        for (int kt = 0; kt < NCT; ++kt)
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct) Sf[kt][ct] = S[kt][ct];
                    } else if (KEEP2 && s == nsub - 2 && !(s == 0 && s0)) {
#pragma unroll
                        for (int kt = 0; kt < NCT; ++kt)
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct) Sf[kt][ct] = S2[kt][ct];
                    } else if (s == 0 && s0) {
#pragma unroll
                        for (int kt = 0; kt < NCT; ++kt)
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj)
                                    Sf[kt][ct][jj] = s0[uint32_t((16 * kt + 4 * q4 + jj) * DV + col0 + 16 * ct + l16)];
                    } else {
#pragma unroll
                        for (int kt = 0; kt < NCT; ++kt)
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct)
                                Sf[kt][ct] =
                                    *reinterpret_cast<const f32x4*>(SslotA + acc_tile_off<DV>(kt, CT * wave + ct, lane));
                    }
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
                    KDA_PHASE(9);
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
                    KDA_PHASE(10);
                    R.settle();
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
                KDA_PHASE(6);
                if (wave < C::NU) {
                    if (!chain) R.settle();
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
                    // one pass over d_v: dP = incl(dO U^T) and dA' = -Diag(beta) strict(dY U^T)
                    // (masked below), dO S^T, dY S^T and U dS'^T for the channel
                    // products, and this lane's share of <S, dS'>
                    f32x4 dP = {0.f, 0.f, 0.f, 0.f}, M1 = dP, aQ = dP, aK = dP, aT = dP;
                    float dot = 0.f;
#pragma unroll
                    for (int kt = 0; kt < DV / 16; ++kt) {
                        const auto fo = frag_rows<O>(sDO + 16 * kt, C::SV, lane);
                        const auto fu = frag_rows<O>(sU + 16 * kt, C::SV, lane);
                        const auto fy = frag_rows<O>(sVY + 16 * kt, C::SV, lane);
                        O::mma4(dP, fo, fu);
                        O::mma4(M1, fy, fu);
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
                        O::mma4(aQ, fo, bs);
                        O::mma4(aK, fy, bs);
                        O::mma4(aT, fu, bd);
                    }
                    // every lane reads (all indices are in range), then masks
                    float tb[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r4 = 4 * q4 + jj;
                        const float m1 = M1[jj];
                        const float ap = sAP[r4 * 17 + l16], br = sB[r4];
                        tb[jj] = l16 < r4 ? -m1 * ap : 0.f;
                        dP[jj] = l16 <= r4 ? dP[jj] : 0.f;
                        M1[jj] = l16 < r4 ? -br * m1 : 0.f;
                    }
                    // their transposes: an accumulator tile as the A operand is its
                    // matrix transposed, so X^T = (that operand) x I, one product
                    // each (exact: the operand is what the products below use)
                    f32x4 dPT = {0.f, 0.f, 0.f, 0.f}, M1T = dPT;
                    {
                        f32x4 x;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) x[jj] = (4 * q4 + jj == l16) ? 1.f : 0.f;
                        const auto iden = O::make4(x);
                        O::mma4(dPT, O::make4(dP), iden);
                        O::mma4(M1T, O::make4(M1), iden);
                    }
                    if (wave == 0) {
                        // dbeta_r: this row's sum of tb plus the chain waves'
                        // <dY_r, X_r> partials, lane l16 < NCW adding wave l16's
                        static_assert(C::NCW <= 16, "one partial per lane of a row");
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int r = 4 * q4 + jj;
                            const float pr = sRB[(l16 < C::NCW ? l16 : 0) * BSUB + r];
                            const float s = sum16(tb[jj] + (l16 < C::NCW ? pr : 0.f));
                            if (l16 == 0 && r < n) a.dbeta[row0 + uint32_t(r) * uint32_t(H)] = s;
                        }
                    }
                    KDA_PHASE(12);
                    const auto fdP = O::make4(dPT);   // A = dP
                    const auto fdPT = O::make4(dP);   // A = dP^T
                    const auto fdA = O::make4(M1T);   // A = dA'
                    const auto fdAT = O::make4(M1);   // A = dA'^T
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) aK[jj] *= -sB[4 * q4 + jj];
                    KDA_PHASE(13);
                    const auto bkm = frag_rows<O>(sKMT + ch0 * C::S16, C::S16, lane);  // B = K-
                    O::mma4(aQ, fdP, bkm);
                    O::mma4(aK, fdA, bkm);
                    f32x4 aM = {0.f, 0.f, 0.f, 0.f};
                    O::mma4(aM, fdAT, frag_rows<O>(sKHT + ch0 * C::S16, C::S16, lane));  // dA'^T K^
                    O::mma4(aM, fdPT, frag_rows<O>(sQHT + ch0 * C::S16, C::S16, lane));  // + dP^T Q^
                    const float eGl = sGam[c];  // e^{G_last}
                    float gl = 0.f, dGr[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r = 4 * q4 + jj;
                        const bool ok = r < n;
                        const uint32_t off = uint32_t(r) * rsk + uint32_t(c);
                        const float kv = ok ? kq[jj][0] : 0.f;
                        const float qv = ok ? kq[jj][1] : 0.f;
                        const float G = sG[r * C::SG + c];
                        const float eG = __expf(G), eM = __expf(-G), eT = eGl * eM;  // e^{G_last - G}
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
                    KDA_PHASE(14);
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
                KDA_PHASE(7);
            }
        }
        // the first segment of a sequence ends at the initial state's gradient
        if (L.s == 0 && chain) store_tiles(dS, a.d_init + unit * DK * DV);
        KDA_PHASE(8);
    }
    pclk.save();
}

template <typename DT, int DK, int DV>
hipError_t launch_bwd_chunk(const BackwardArgs& a, const BwdPlan& plan, hipStream_t stream)
{
    using C1 = BwdCfg<DT, DK, DV, false>;
    using C3 = BwdCfg<DT, DK, DV, true>;
    hipError_t e = hipSuccess;
    BackwardArgs b = a;
    if (plan.warm > 0) {  // the windows: dS_end of every segment, flags where M^T did not vanish
        auto kw = bwd_chunk_summary_kernel<DT, DK, DV, true>;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kw), hipFuncAttributeMaxDynamicSharedMemorySize,
                                C1::LDS);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kw, dim3(unsigned(plan.segs_max * a.H)), dim3(C1::NT), C1::LDS, stream, b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
        b.flags = nullptr;  // every chain through the summary and the scan
    }
    // the summary pass and the scan: flagged chains only (all of them without
    // windows, where the scan also hands each sequence's last segment d_fin);
    // with windows and one segment per sequence there is nothing to compose
    if (b.flags == nullptr || plan.Lseg < a.T_total) {
        auto k1 = bwd_chunk_summary_kernel<DT, DK, DV, false>;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1), hipFuncAttributeMaxDynamicSharedMemorySize,
                                C1::LDS);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k1, dim3(unsigned(plan.segs_max * a.H)), dim3(C1::NT), C1::LDS, stream, b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        auto ks = bwd_scan_kernel<DK, DV>;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(ks), hipFuncAttributeMaxDynamicSharedMemorySize,
                                BwdScanCfg<DK>::LDS);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(ks, dim3(unsigned(a.N * a.H * (DV / BWD_SCAN_COLS))), dim3(256), BwdScanCfg<DK>::LDS,
                           stream, b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    auto k3 = bwd_chunk_full_kernel<DT, DK, DV>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k3), hipFuncAttributeMaxDynamicSharedMemorySize, C3::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k3, dim3(unsigned(plan.grid)), dim3(C3::NT), C3::LDS, stream, b);
    return hipGetLastError();
}

// The launches launch_bwd_chunk makes for this plan, as text (host only).
template <typename DT, int DK, int DV>
void describe_backward_t(const BwdPlan& plan, int64_t T_total, int N, int H, std::string& out)
{
    using C1 = BwdCfg<DT, DK, DV, false>;
    using C3 = BwdCfg<DT, DK, DV, true>;
    char line[256];
    int n = 0;
    auto add = [&](const char* kernel, int64_t grid, int threads, int lds, const char* what) {
        snprintf(line, sizeof(line), "launch %d: %s grid %lld x %d threads, %d B LDS; %s\n", ++n, kernel,
                 (long long)grid, threads, lds, what);
        out += line;
    };
    if (plan.warm > 0)
        add("bwd_chunk_summary_kernel (window)", plan.segs_max * H, C1::NT, C1::LDS,
            "every segment's end-of-segment state gradient from the window after it; flags the chains where the "
            "window's transposed transition is not zero");
    if (plan.warm == 0 || plan.Lseg < T_total) {
        add("bwd_chunk_summary_kernel", plan.segs_max * H, C1::NT, C1::LDS,
            plan.warm > 0 ? "[C | M^T] of the flagged chains' segments 1.. (returns at once elsewhere)"
                          : "[C | M^T] of every segment but a sequence's first");
        add("bwd_scan_kernel", int64_t(N) * H * (DV / BWD_SCAN_COLS), 256, BwdScanCfg<DK>::LDS,
            plan.warm > 0 ? "end-of-segment gradients of the flagged chains" : "every end-of-segment gradient");
    }
    add("bwd_chunk_full_kernel", plan.grid, C3::NT, C3::LDS,
        "every (segment, head) from its end-of-segment gradient: dq, dk, dv, dg, dbeta, the initial state's "
        "gradient; the states rebuilt from the checkpoints");
}

template <typename DT>
bool describe_backward(const BwdPlan& plan, int64_t T_total, int N, int H, int dk, int dv, std::string& out)
{
#define KDA_BWD(DKV, DVV)                                                                                  \
    if (dk == DKV && dv == DVV) {                                                                          \
        describe_backward_t<DT, DKV, DVV>(plan, T_total, N, H, out);                                       \
        return true;                                                                                       \
    }
    KDA_BWD(32, 32) KDA_BWD(32, 64) KDA_BWD(32, 128)
    KDA_BWD(64, 32) KDA_BWD(64, 64) KDA_BWD(64, 128)
    KDA_BWD(128, 32) KDA_BWD(128, 64) KDA_BWD(128, 128)
#undef KDA_BWD
    return false;
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
    b.flags = reinterpret_cast<int32_t*>(ws + plan.off_flags);
    b.warm = plan.warm;
    b.segs_cap = plan.segs_max;
#define KDA_BWD(DKV, DVV) \
    if (dk == DKV && dv == DVV) return launch_bwd_chunk<DT, DKV, DVV>(b, plan, stream);
    KDA_BWD(32, 32) KDA_BWD(32, 64) KDA_BWD(32, 128)
    KDA_BWD(64, 32) KDA_BWD(64, 64) KDA_BWD(64, 128)
    KDA_BWD(128, 32) KDA_BWD(128, 64) KDA_BWD(128, 128)
#undef KDA_BWD
    return hipErrorInvalidValue;
}

}  // namespace kda
