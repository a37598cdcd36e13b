// kda_prefill: chunkwise KDA forward with state in / state out, varlen packing
// and intra-device segment parallelism.
//
// Sources: "NLP——技术报告解读-Kimi-K3", Model Architecture / Kimi Delta
// Attention (KDA) (recurrence, read-out, bounded decay that keeps every
// decay ratio inside the matrix units' range) and Infrastructure / KDA
// algorithm-system co-design (chunkwise prefill kernel; one sequence split
// across the compute units with each segment's transition computed
// independently and composed exactly; the KCP identity S = S~ + M S_in);
// "Kimi K3 技术报告 · 大白话版" §5.1 (inside a chunk in parallel, chunk to
// chunk in series).
//
// Per (segment, head) and chunk of C = 64 tokens, with G the running sum of g
// inside the chunk (per key channel), incoming state S (d_k x d_v):
//   A[r][i] = beta_r sum_c k_rc k_ic e^{G_rc - G_ic}   (i < r)
//   P[r][i] =        sum_c q_rc k_ic e^{G_rc - G_ic}   (i <= r)
//   T = (I + A)^{-1} Diag(beta)                          (UT/WY solve)
//   X = V - (K . e^{G}) S ;  U = T X
//   O = (Q . e^{G}) S + P U
//   S <- Diag(e^{G_last}) S + (K . e^{G_last - G})^T U
// (U = T V - T (K.e^G) S is the WY form; grouping it as T (V - (K.e^G) S)
// needs no separate W tile.)
//
// Decay ratios e^{G_r - G_i} never leave fp32 range: G is referenced per
// 16-token sub-tile.  With R_a = G before sub-tile a and E_b = G at the end
// of sub-tile b (so E_b = R_{b+1}), one sub-tile spans at most 16 * 5 = 80 in
// log space (g >= -5), hence
//   diagonal (a == b):  e^{G_r - R_a} (<= 1)  x  e^{R_a - G_i} (<= e^80)
//   off-diagonal b < a: e^{G_r - R_a} e^{R_a - E_b} (<= 1)  x  e^{R_b - G_i} e^{E_b - R_b} (<= 1)
// and the products run on the matrix cores for every tile.
//
// Work decomposition (gfx950, wave64, 16x16x32 bf16 / 16x16x4 f32 MFMA):
//   - one workgroup per (segment, head); the (extended) state's columns are
//     split across waves, 32 per wave, and stay in registers for the whole
//     segment, so the chunk-to-chunk chain needs no cross-wave traffic.
//   - per chunk the shared operands (decayed q/k tiles, T, P) are built in
//     LDS by all waves, then each wave runs its columns' chain.
//   - the next chunk's raw tiles are prefetched into registers during the
//     chain.
//   - long sequences are cut into segments: pass 1 (SUMMARY) computes each
//     non-final segment's transition M and zero-start state S~ as one
//     extended state [S~ | M] (M's columns have v = 0 and start at I); a
//     scan composes S_in(s+1) = M_s S_in(s) + S~_s; pass 3 (OUT) reruns every
//     segment from its true incoming state and writes the outputs.
#pragma once

#include "kda_common.hpp"

namespace kda {

// Optional per-phase cycle counters of the chunk kernel (built only with
// -DKDA_PHASE_TIMING; the default build compiles the markers away).
#ifdef KDA_PHASE_TIMING
#ifndef KDA_PHASE_TID
#define KDA_PHASE_TID 0
#endif
__device__ unsigned long long kda_phase_cycles[16384 * 16];
#define KDA_PHASE(i)                                    \
    do {                                                \
        if (tid == KDA_PHASE_TID) {                     \
            const long long t_ = clock64();             \
            phase_acc[i] += t_ - phase_last;            \
            phase_last = t_;                            \
        }                                               \
    } while (0)
#else
#define KDA_PHASE(i) \
    do {             \
    } while (0)
#endif

constexpr int CH = 64;  // tokens per chunk
constexpr int NCU_TARGET = 256;

// ---------------------------------------------------------------- host plan
struct PrefillPlan {
    int seg_chunks = 1;        // chunks per segment (L)
    int64_t nseg_max = 0;      // upper bound on the number of segments
    int64_t np1_max = 0;       // upper bound on the number of non-final segments
    size_t off_table = 0, off_ms = 0, off_sin = 0;
    size_t workspace_bytes = 0;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline PrefillPlan prefill_plan(int64_t T_total, int N, int H, int dk, int dv)
{
    PrefillPlan p;
    const int64_t chunks_bound = (T_total + CH - 1) / CH + N;  // >= total chunks over sequences
    int64_t per_cu = (int64_t(H) * chunks_bound + NCU_TARGET - 1) / NCU_TARGET;
    int64_t L = per_cu / 2;
    if (L < 16) L = 16;
    if (const char* e = getenv("KDA_SEG_CHUNKS")) {
        const long v = atol(e);
        if (v > 0) L = v;
    }
    const int64_t max_seq_chunks = (T_total + CH - 1) / CH;
    if (L >= max_seq_chunks) L = max_seq_chunks > 0 ? max_seq_chunks : 1;  // nothing splits
    p.seg_chunks = int(L);
    p.nseg_max = chunks_bound / L + N + 1;
    p.np1_max = (max_seq_chunks > L) ? chunks_bound / L + 1 : 0;
    size_t off = 0;
    p.off_table = off;
    off = align256(off + sizeof(int32_t) * 3 * size_t(N + 1));
    if (p.np1_max > 0) {
        p.off_ms = off;
        off = align256(off + sizeof(float) * size_t(p.np1_max) * H * dk * (dk + dv));
        p.off_sin = off;
        off = align256(off + sizeof(float) * size_t(p.nseg_max) * H * dk * dv);
    }
    p.workspace_bytes = off;
    return p;
}

struct PrefillArgs {
    const void *q, *k, *v, *g, *beta;
    const int32_t* cu;
    int N;
    int64_t T_total;
    int H, dk, dv;
    const float* init;
    float* fin;
    void* o;
    void* ws;
};

// Device-side view shared by the prefill kernels.
struct PrefillDev {
    const void *q, *k, *v, *g, *beta;
    const int32_t* tab;  // cuc[N+1] | seg_off[N+1] | p1_off[N+1]
    int N;
    int64_t T_total;
    int H;
    int L;  // chunks per segment
    const float* init;
    float* fin;
    void* o;
    float* ms;   // [np1][H][dk][dk+dv]
    float* sin;  // [nseg][H][dk][dv]
};

// ------------------------------------------------------------- plan kernel
// One workgroup: clamps cu_seqlens into a non-decreasing sequence inside
// [0, T_total] and writes the per-sequence segment / pass-1 offsets.
__global__ void __launch_bounds__(256) plan_kernel(const int32_t* __restrict__ cu, int N,
                                                   int64_t T_total, int L, int32_t* __restrict__ tab)
{
    __shared__ int32_t s_seg[256], s_p1[256], s_cu[256];
    __shared__ int32_t carry_seg, carry_p1, carry_cu;
    int32_t* cuc = tab;
    int32_t* seg_off = tab + (N + 1);
    int32_t* p1_off = tab + 2 * (N + 1);
    const int t = threadIdx.x;
    if (t == 0) {
        carry_seg = 0;
        carry_p1 = 0;
        carry_cu = 0;
        cuc[0] = 0;
        seg_off[0] = 0;
        p1_off[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + t;
        // running max of clamped offsets = a non-decreasing sequence
        int32_t c1 = 0;
        if (n < N) {
            int64_t x = cu ? int64_t(cu[n + 1]) : T_total;
            if (x < 0) x = 0;
            if (x > T_total) x = T_total;
            c1 = int32_t(x);
        }
        s_cu[t] = c1;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {  // inclusive max-scan
            const int32_t y = (t >= d) ? s_cu[t - d] : 0;
            __syncthreads();
            if (y > s_cu[t]) s_cu[t] = y;
            __syncthreads();
        }
        const int32_t c1m = s_cu[t] > carry_cu ? s_cu[t] : carry_cu;
        __syncthreads();
        s_cu[t] = c1m;
        __syncthreads();
        const int32_t c0m = (t == 0) ? carry_cu : s_cu[t - 1];
        int32_t nseg = 0, np1 = 0;
        if (n < N) {
            const int64_t len = int64_t(c1m) - c0m;
            const int64_t ch = (len + CH - 1) / CH;
            int64_t ns = (ch + L - 1) / L;
            if (ns < 1) ns = 1;
            nseg = int32_t(ns);
            np1 = int32_t(ns - 1);
        }
        s_seg[t] = nseg;
        s_p1[t] = np1;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {  // inclusive sum-scans
            const int32_t a = (t >= d) ? s_seg[t - d] : 0;
            const int32_t b = (t >= d) ? s_p1[t - d] : 0;
            __syncthreads();
            s_seg[t] += a;
            s_p1[t] += b;
            __syncthreads();
        }
        if (n < N) {
            cuc[n + 1] = c1m;
            seg_off[n + 1] = carry_seg + s_seg[t];
            p1_off[n + 1] = carry_p1 + s_p1[t];
        }
        __syncthreads();
        if (t == 255) {
            carry_seg += s_seg[255];
            carry_p1 += s_p1[255];
            carry_cu = s_cu[255];
        }
        __syncthreads();
    }
}

// index n with off[n] <= item < off[n+1] (off non-decreasing, off[0] = 0)
__device__ __forceinline__ int find_seq(const int32_t* off, int N, int item)
{
    int lo = 0, hi = N;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= item) lo = mid;
        else hi = mid;
    }
    return lo;
}

// ------------------------------------------------------- operand plumbing
// MFMA operand tiles in LDS keep each 32-column block in a permuted order:
// logical column c = 16h + 4q + j (h in {0,1}, q, j in 0..3) is stored at
// position 8q + 4h + j.  Lane group q of a 16x16x32 MFMA then reads its eight
// K-values k(q, e) = 16*(e/4) + 4q + e%4 (e = 0..7) as one contiguous 16-byte
// (bf16) load.  The same k(q, e) order lets a pair of 16x16 accumulator tiles
// (rows 4q..4q+3 of rows 0-15 and of rows 16-31) serve directly as the other
// operand, so the state, X and U never leave registers.
__host__ __device__ constexpr int pcol(int c)
{
    return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}
__device__ __forceinline__ int kperm(int q, int e) { return ((e >> 2) << 4) + (q << 2) + (e & 3); }

// 2^x with the hardware instruction (about 1 ulp; results below the fp32
// range flush to zero, which the decay factoring above tolerates: every
// flushed factor multiplies terms bounded by 1)
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename DT>
struct Op;
typedef __attribute__((ext_vector_type(4))) short s16x4;
template <>
struct Op<BF16> {
    using T = uint16_t;  // LDS operand element
    using Frag = bf16x8;  // 16x16x32 operand
    using Frag4 = s16x4;  // 16x16x16 operand
    static __device__ __forceinline__ Frag make(const float (&x)[8])
    {
        u32x4 w;
        w[0] = pack_bf16x2(x[0], x[1]);
        w[1] = pack_bf16x2(x[2], x[3]);
        w[2] = pack_bf16x2(x[4], x[5]);
        w[3] = pack_bf16x2(x[6], x[7]);
        return __builtin_bit_cast(Frag, w);
    }
    static __device__ __forceinline__ Frag load(const T* p)  // 8 consecutive elements
    {
        return __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(p));
    }
    static __device__ __forceinline__ void unpack(const Frag& f, float (&x)[8])
    {
        const u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w[i]);
            x[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    static __device__ __forceinline__ Frag4 load4(const T* p)
    {
        return __builtin_bit_cast(Frag4, *reinterpret_cast<const u32x2*>(p));
    }
    static __device__ __forceinline__ Frag4 make4(const f32x4& v)
    {
        u32x2 w;
        w[0] = pack_bf16x2(v[0], v[1]);
        w[1] = pack_bf16x2(v[2], v[3]);
        return __builtin_bit_cast(Frag4, w);
    }
    static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b)
    {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void mma4(f32x4& acc, const Frag4& a, const Frag4& b)
    {
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ T to_op(float x) { return f32_to_bf16(x); }
    static __device__ __forceinline__ float from_op(T x) { return bf16_to_f32(x); }
    // two adjacent elements (channels 2m, 2m+1)
    using Pair = uint32_t;
    static __device__ __forceinline__ Pair ldp(const T* p) { return *reinterpret_cast<const uint32_t*>(p); }
    static __device__ __forceinline__ float p0(Pair w) { return bf16_lo(w); }
    static __device__ __forceinline__ float p1(Pair w) { return bf16_hi(w); }
    static __device__ __forceinline__ void stp(T* p, float a, float b)
    {
        *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
    }
    static __device__ __forceinline__ void st4(T* p, const f32x4& v)
    {
        u32x2 w;
        w[0] = pack_bf16x2(v[0], v[1]);
        w[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(p) = w;
    }
};
struct f32x8 {
    float v[8];
};
template <>
struct Op<F32> {
    using T = float;
    using Frag = f32x8;
    using Frag4 = f32x4;
    static __device__ __forceinline__ Frag make(const float (&x)[8])
    {
        Frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f.v[i] = x[i];
        return f;
    }
    static __device__ __forceinline__ Frag load(const T* p)
    {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
        Frag f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f.v[i] = a[i];
            f.v[4 + i] = b[i];
        }
        return f;
    }
    static __device__ __forceinline__ void unpack(const Frag& f, float (&x)[8])
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = f.v[i];
    }
    static __device__ __forceinline__ Frag4 load4(const T* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ Frag4 make4(const f32x4& v) { return v; }
    static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b)
    {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
    }
    // K = 16 with lane group q holding k = 4q..4q+3: MFMA s takes element s (k = 4q + s)
    static __device__ __forceinline__ void mma4(f32x4& acc, const Frag4& a, const Frag4& b)
    {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    }
    static __device__ __forceinline__ T to_op(float x) { return x; }
    static __device__ __forceinline__ float from_op(T x) { return x; }
    using Pair = f32x2;
    static __device__ __forceinline__ Pair ldp(const T* p) { return *reinterpret_cast<const f32x2*>(p); }
    static __device__ __forceinline__ float p0(Pair w) { return w[0]; }
    static __device__ __forceinline__ float p1(Pair w) { return w[1]; }
    static __device__ __forceinline__ void stp(T* p, float a, float b)
    {
        *reinterpret_cast<f32x2*>(p) = f32x2{a, b};
    }
    static __device__ __forceinline__ void st4(T* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
};

// operand fragment from two accumulator tiles (rows 0-15 and 16-31 of a K-block)
template <typename DT>
__device__ __forceinline__ typename Op<DT>::Frag acc_frag(const f32x4& lo, const f32x4& hi)
{
    float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return Op<DT>::make(x);
}

// ------------------------------------------------------------ chunk kernel
template <typename DT, int DK, int DV, bool SUMMARY>
struct ChunkCfg {
    static constexpr int NCOL = SUMMARY ? DV + DK : DV;  // extended state columns
    // state columns per chain wave: 16 for the output pass (two waves per SIMD
    // hide LDS latency), 32 for the summary pass (twice the columns, no outputs)
    static constexpr int CW = (SUMMARY || NCOL <= 32) ? 32 : 16;
    static constexpr int NCT = CW / 16;                   // 16-wide column tiles per wave
    static constexpr int NCW = NCOL / CW;                 // chain waves
    static constexpr int NW0 = NCW > DK / 64 ? NCW : DK / 64;
    static constexpr int NW = NW0 <= 1 ? 1 : NW0 <= 2 ? 2 : NW0 <= 4 ? 4 : 8;
    static constexpr int NT = NW * 64;
    static constexpr int CP = DK / 2;          // channel pairs
    static constexpr int PARTS = NT / CP;      // threads per channel pair (elementwise phases)
    static constexpr int TPT = CH / PARTS;     // tokens per thread
    static constexpr int SL = TPT < 16 ? TPT : 16;
    static constexpr int NSLOT = CH / SL;
    using OT = typename Op<DT>::T;
    static constexpr int ES = sizeof(OT);
    static constexpr int SK = DK + 16 / ES;  // padded row strides (elements)
    static constexpr int SV = DV + 16 / ES;
    static constexpr int ST = CH + 16 / ES;
    static constexpr int SD = 16 + 16 / ES;
    static constexpr int TILE_K = CH * SK * ES;
    // LDS layout (bytes)
    static constexpr int O_Q = 0;                       // raw q -> q.e^{G-R_a}
    static constexpr int O_K = O_Q + TILE_K;            // raw k -> k.e^{G-R_a}
    static constexpr int O_G = O_K + TILE_K;            // raw g -> k.e^{R_a-G}
    static constexpr int O_V = O_G + TILE_K;            // raw v
    static constexpr int O_QG = O_V + CH * SV * ES;     // q.e^{G}
    static constexpr int O_KG = O_QG + TILE_K;          // -k.e^{G}
    static constexpr int O_KH = O_KG + TILE_K;          // (k.e^{G_last-G})^T  [DK][ST]
    static constexpr int O_A = O_KH + DK * ST * ES;     // -A (x beta_r), natural columns
    static constexpr int O_P = O_A + CH * ST * ES;      // P, permuted columns
    static constexpr int O_D = O_P + CH * ST * ES;      // (I + A_aa)^{-1}, 4 blocks
    static constexpr int O_DS = O_D + 4 * 16 * SD * ES;  // N^2, N^4 per diagonal block (inverse scratch)
    static constexpr int O_VEC = O_DS + 8 * 16 * SD * ES;  // 16 x DK fp32 channel vectors
    static constexpr int O_SIG = O_VEC + 16 * DK * 4;   // NSLOT x DK fp32
    static constexpr int O_B = O_SIG + NSLOT * DK * 4;  // beta[64]
    static constexpr int LDS = O_B + CH * 4;
    // output staging in the -k.e^G tile: rows of DV storage elements (stride SO)
    static constexpr int SO = DV + 8;
    static constexpr bool STAGE_O = !SUMMARY && CH * SO * int(sizeof(typename DT::storage)) <= TILE_K;
    // raw tile loading: 16-byte units
    static constexpr int EPU = 16 / ES;           // elements per unit
    static constexpr int UPR_K = DK / EPU;        // units per row
    static constexpr int UPR_V = DV / EPU;
    static constexpr int U_K = CH * UPR_K;        // units per q/k/g tile
    static constexpr int U_V = CH * UPR_V;
    static constexpr int NTILE_K = SUMMARY ? 2 : 3;  // pass 1 needs no q
    static constexpr int UPT_K = (U_K + NT - 1) / NT;  // units per thread, per q/k/g tile
    static constexpr int UPT_V = (U_V + NT - 1) / NT;
    static constexpr int UPT = NTILE_K * UPT_K + UPT_V;
    static_assert(LDS <= 160 * 1024, "LDS budget exceeded");
    static_assert(PARTS >= 1 && CH % PARTS == 0, "bad elementwise split");
    static_assert((TPT % 16 == 0) || (16 % TPT == 0), "sub-tile alignment");
};

// channel-vector slots (each DK fp32, permuted channel order):
//   V_ER + a : e^{R_a}                              (q, k decayed to the chunk start)
//   V_YS + t : e^{R_a - R_b} for off-diagonal block t = (a, b), key side
//   V_GC     : e^{G_last}
enum { V_ER = 0, V_YS = 4, V_GC = 10 };
// off-diagonal blocks in task order (1,0),(2,0),(2,1),(3,0),(3,1),(3,2) -> slot
__host__ __device__ constexpr int ys_slot(int a, int b) { return (a * (a - 1)) / 2 + b; }

// Raw tile prefetch into registers: per tensor a uniform base pointer for the
// chunk and a fixed per-lane offset, so each 16-byte unit is one load.  Rows
// past the sequence end are re-read from its last row (only needed when the
// chunk ends past the tensor) and zeroed at commit.
template <typename C, typename DT>
__device__ __forceinline__ void raw_prefetch(u32x4 (&pre)[C::UPT], const typename DT::storage* gq,
                                             const typename DT::storage* gk,
                                             const typename DT::storage* gv,
                                             const typename DT::storage* gg, int64_t c0, int len,
                                             int64_t T_total, int H, int h, int tid, int dk, int dv)
{
    using ST = typename DT::storage;
    const bool clamp = c0 + CH > T_total;
    const int hdk = H * dk, hdv = H * dv;
    const ST* bases[3] = {gq, gk, gg};
#pragma unroll
    for (int t = 0; t < C::NTILE_K; ++t) {
        const ST* base = bases[C::NTILE_K == 3 ? t : t + 1] + (c0 * H + h) * int64_t(dk);
#pragma unroll
        for (int j = 0; j < C::UPT_K; ++j) {
            const int uu = tid + j * C::NT;
            if (C::U_K % C::NT == 0 || uu < C::U_K) {
                int row = uu / C::UPR_K;
                if (clamp) row = row < len ? row : len - 1;
                pre[t * C::UPT_K + j] =
                    *reinterpret_cast<const u32x4*>(base + (row * hdk + (uu % C::UPR_K) * C::EPU));
            }
        }
    }
    const ST* vbase = gv + (c0 * H + h) * int64_t(dv);
#pragma unroll
    for (int j = 0; j < C::UPT_V; ++j) {
        const int uu = tid + j * C::NT;
        if (C::U_V % C::NT == 0 || uu < C::U_V) {
            int row = uu / C::UPR_V;
            if (clamp) row = row < len ? row : len - 1;
            pre[C::NTILE_K * C::UPT_K + j] =
                *reinterpret_cast<const u32x4*>(vbase + (row * hdv + (uu % C::UPR_V) * C::EPU));
        }
    }
}

// raw tiles into LDS, each 16-byte unit placed at its permuted column position
// (rows at or past `len` are written as zeros)
template <typename C>
__device__ __forceinline__ void raw_commit(const u32x4 (&pre)[C::UPT], unsigned char* smem, int tid, int len)
{
    using OT = typename C::OT;
    constexpr int offs[3] = {C::NTILE_K == 3 ? C::O_Q : C::O_K, C::NTILE_K == 3 ? C::O_K : C::O_G, C::O_G};
#pragma unroll
    for (int i = 0; i < C::UPT; ++i) {
        const bool isv = i >= C::NTILE_K * C::UPT_K;
        const int t = isv ? 0 : i / C::UPT_K;
        const int j = isv ? i - C::NTILE_K * C::UPT_K : i % C::UPT_K;
        const int uu = tid + j * C::NT;
        const int UPR = isv ? C::UPR_V : C::UPR_K;
        if ((isv ? C::U_V : C::U_K) % C::NT == 0 || uu < (isv ? C::U_V : C::U_K)) {
            const int row = uu / UPR, c0 = (uu % UPR) * C::EPU;
            OT* row_base = isv ? reinterpret_cast<OT*>(smem + C::O_V) + row * C::SV
                               : reinterpret_cast<OT*>(smem + offs[t]) + row * C::SK;
            const bool keep = row < len;
            const u32x4 w = {keep ? pre[i][0] : 0u, keep ? pre[i][1] : 0u, keep ? pre[i][2] : 0u,
                             keep ? pre[i][3] : 0u};
            if constexpr (C::ES == 2) {  // 8 columns -> two runs of 4 (8 bytes each)
                *reinterpret_cast<u32x2*>(row_base + pcol(c0)) = u32x2{w[0], w[1]};
                *reinterpret_cast<u32x2*>(row_base + pcol(c0 + 4)) = u32x2{w[2], w[3]};
            } else {  // 4 fp32 columns stay contiguous
                *reinterpret_cast<u32x4*>(row_base + pcol(c0)) = w;
            }
        }
    }
}

// four consecutive elements of a token tensor from fp32
template <typename DT>
__device__ __forceinline__ void store4(typename DT::storage* p, const f32x4& v)
{
    if constexpr (DT::is_bf16) {
        *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    } else {
        *reinterpret_cast<f32x4*>(p) = v;
    }
}

// copy a staged output tile (LDS rows of DV elements, row stride SO) to o, 16 bytes per unit
template <typename C, typename DT, int DV>
__device__ __forceinline__ void store_out_tile(const unsigned char* smem, typename DT::storage* go, int64_t c0,
                                               int len, int H, int h, int tid)
{
    using ST = typename DT::storage;
    constexpr int EPU = 16 / int(sizeof(ST));
    constexpr int UPR = DV / EPU;
    const ST* stage = reinterpret_cast<const ST*>(smem + C::O_KG);
    for (int u = tid; u < CH * UPR; u += C::NT) {
        const int row = u / UPR, cu = u % UPR;
        if (row < len)
            *reinterpret_cast<u32x4*>(go + ((c0 + row) * H + h) * DV + cu * EPU) =
                *reinterpret_cast<const u32x4*>(stage + row * C::SO + cu * EPU);
    }
}

// (I + N)^{-1} for one 16x16 diagonal block of the strictly lower N, by one
// full wave on the matrix cores.  N is nilpotent (N^16 = 0), so
//     (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8):
// three squarings and three products of 16x16 tiles.  A 16x16 accumulator tile
// is directly the B operand of the next 16x16x16 product; the A operand needs
// rows, so each power is written once to LDS (wave-private scratch, read back
// by the same wave: LDS operations of one wave complete in order).
// sA holds -N (natural column order); the result goes to sD.
template <typename C, typename O>
__device__ __forceinline__ void diag_inverse(const typename O::T* sA, typename O::T* sD, typename O::T* scr,
                                             int a, int lane)
{
    using OT = typename O::T;
    using Frag4 = typename O::Frag4;
    const int l16 = lane & 15, q4 = lane >> 4;
    const OT* Qrows = sA + (a * 16) * C::ST + a * 16;  // -N
    OT* n2 = scr + (2 * a) * 16 * C::SD;
    OT* n4 = scr + (2 * a + 1) * 16 * C::SD;
    auto rowfrag = [&](const OT* base, int ld) { return O::load4(base + l16 * ld + 4 * q4); };
    auto put = [&](OT* base, const f32x4& t) {  // accumulator tile -> natural rows
#pragma unroll
        for (int j = 0; j < 4; ++j) base[(4 * q4 + j) * C::SD + l16] = O::to_op(t[j]);
    };
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // B operand of -N: column l16, rows 4q..4q+3
    f32x4 qcol;
#pragma unroll
    for (int j = 0; j < 4; ++j) qcol[j] = O::from_op(Qrows[(4 * q4 + j) * C::ST + l16]);
    const Frag4 qa = rowfrag(Qrows, C::ST);
    f32x4 t2 = {0.f, 0.f, 0.f, 0.f};
    O::mma4(t2, qa, O::make4(qcol));  // N^2 = (-N)(-N)
    put(n2, t2);
    wave_sync();
    f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
    const Frag4 n2a = rowfrag(n2, C::SD);
    O::mma4(t4, n2a, O::make4(t2));  // N^4
    put(n4, t4);
    wave_sync();
    f32x4 t8 = {0.f, 0.f, 0.f, 0.f};
    const Frag4 n4a = rowfrag(n4, C::SD);
    O::mma4(t8, n4a, O::make4(t4));  // N^8
    // E1 = (I + N^4)(I + N^8) = I + N^4 + N^8 + N^4 N^8
    f32x4 e = t4 + t8;
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] += (4 * q4 + j == l16) ? 1.f : 0.f;
    O::mma4(e, n4a, O::make4(t8));
    // E2 = (I + N^2) E1
    f32x4 e2 = e;
    O::mma4(e2, n2a, O::make4(e));
    // D = (I - N) E2
    f32x4 d = e2;
    O::mma4(d, qa, O::make4(e2));
#pragma unroll
    for (int j = 0; j < 4; ++j) sD[(a * 16 + 4 * q4 + j) * C::SD + l16] = O::to_op(d[j]);
}

template <typename DT, int DK, int DV, bool SUMMARY>
__global__ void __launch_bounds__((ChunkCfg<DT, DK, DV, SUMMARY>::NT))
prefill_chunk_kernel(PrefillDev p)
{
    using C = ChunkCfg<DT, DK, DV, SUMMARY>;
    using O = Op<DT>;
    using OT = typename O::T;
    using Frag = typename O::Frag;
    using Frag4 = typename O::Frag4;
    using Pair = typename O::Pair;
    using ST = typename DT::storage;
    constexpr float LOG2E = 1.4426950408889634f;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    OT* sQ = reinterpret_cast<OT*>(smem + C::O_Q);
    OT* sK = reinterpret_cast<OT*>(smem + C::O_K);
    OT* sG = reinterpret_cast<OT*>(smem + C::O_G);
    OT* sV = reinterpret_cast<OT*>(smem + C::O_V);
    OT* sQG = reinterpret_cast<OT*>(smem + C::O_QG);
    OT* sKG = reinterpret_cast<OT*>(smem + C::O_KG);
    OT* sKH = reinterpret_cast<OT*>(smem + C::O_KH);
    OT* sA = reinterpret_cast<OT*>(smem + C::O_A);
    OT* sP = reinterpret_cast<OT*>(smem + C::O_P);
    OT* sD = reinterpret_cast<OT*>(smem + C::O_D);
    OT* sDS = reinterpret_cast<OT*>(smem + C::O_DS);
    ST* sO = reinterpret_cast<ST*>(smem + C::O_KG);  // output staging (reuses the -k.e^G tile)
    float* sVec = reinterpret_cast<float*>(smem + C::O_VEC);
    float* sSig = reinterpret_cast<float*>(smem + C::O_SIG);
    float* sB = reinterpret_cast<float*>(smem + C::O_B);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;
#ifdef KDA_PHASE_TIMING
    long long phase_acc[12] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    long long phase_last = clock64();
#endif

    // ---- work item
    const int H = p.H;
    const int item = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int32_t* cuc = p.tab;
    const int32_t* seg_off = p.tab + (p.N + 1);
    const int32_t* off = SUMMARY ? p.tab + 2 * (p.N + 1) : seg_off;
    if (item >= off[p.N]) return;
    const int n = find_seq(off, p.N, item);
    const int s = item - off[n];
    const int nseg = seg_off[n + 1] - seg_off[n];
    const int64_t seq0 = cuc[n], seq1 = cuc[n + 1];
    const int64_t t_begin = seq0 + int64_t(s) * p.L * CH;
    int64_t t_end = t_begin + int64_t(p.L) * CH;
    if (t_end > seq1) t_end = seq1;
    const bool last_seg = (s == nseg - 1);

    const ST* gq = static_cast<const ST*>(p.q);
    const ST* gk = static_cast<const ST*>(p.k);
    const ST* gv = static_cast<const ST*>(p.v);
    const ST* gg = static_cast<const ST*>(p.g);
    const ST* gb = static_cast<const ST*>(p.beta);
    ST* go = static_cast<ST*>(p.o);

    // ---- chain registers: wave owns columns [32*wave, 32*wave+32) of the extended state
    constexpr int RT = DK / 16;  // state row tiles
    const bool chain = wave < C::NCW;
    constexpr int NCT = C::NCT;
    const int colbase = C::CW * wave;
    const bool mcols = SUMMARY && colbase >= DV;
    f32x4 S[RT][NCT];
    {
        const float* src = nullptr;
        if (!SUMMARY) {
            if (s == 0) {
                if (p.init) src = p.init + (int64_t(n) * H + h) * DK * DV;
            } else {
                src = p.sin + (int64_t(seg_off[n] + s) * H + h) * DK * DV;
            }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = rt * 16 + 4 * q4 + j;
                    const int col = colbase + ct * 16 + l16;
                    float x = 0.f;
                    if (chain) {
                        if (mcols) x = (row == col - DV) ? 1.f : 0.f;
                        else if (src) x = src[row * DV + col];
                    }
                    S[rt][ct][j] = x;
                }
    }

    // strictly-upper 16x16 blocks of P are read by the P U product and never written
    if (!SUMMARY)
        for (int e = tid; e < CH * CH; e += C::NT) {
            const int r = e / CH, c = e % CH;
            if ((c >> 4) > (r >> 4)) sP[r * C::ST + pcol(c)] = O::to_op(0.f);
        }

    // identity fragments (exact) for X = V I: pick this wave's columns out of
    // the 32-column block that holds them
    Frag Iden[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (kperm(q4, e) == (colbase & 31) + ct * 16 + l16) ? 1.f : 0.f;
        Iden[ct] = O::make(x);
    }

    u32x4 pre[C::UPT];
    const int64_t nchunks = (t_end - t_begin + CH - 1) / CH;
    if (nchunks > 0)
        raw_prefetch<C, DT>(pre, gq, gk, gv, gg, t_begin, int(t_end - t_begin < CH ? t_end - t_begin : CH),
                            p.T_total, H, h, tid, DK, DV);

    const int cp = tid % C::CP;  // channel pair (elementwise phases)
    const int part = tid / C::CP;
    const int pc = pcol(2 * cp);  // stored position of channels 2cp, 2cp+1 (adjacent)
    const int tok0 = part * C::TPT;

    int64_t prev_c0 = 0;
    int prev_len = 0;
    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t c0 = t_begin + ci * CH;
        const int len = int(t_end - c0 < CH ? t_end - c0 : CH);
        __syncthreads();  // the previous chunk's operands are no longer read
        KDA_PHASE(0);
        if (!SUMMARY && C::STAGE_O && ci > 0) store_out_tile<C, DT, DV>(smem, go, prev_c0, prev_len, H, h, tid);
        raw_commit<C>(pre, smem, tid, len);
        __syncthreads();
        KDA_PHASE(1);

        // beta for this chunk: loaded now, first needed by the products (two phases later)
        float bload = 0.f;
        if (tid < CH) bload = load_elem<DT>(gb, (c0 + (tid < len ? tid : len - 1)) * H + h);
        // ---- phase A: per-slot sums of g (log2 domain), two channels per thread
#pragma unroll
        for (int sl = 0; sl < C::TPT / C::SL; ++sl) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int i = 0; i < C::SL; ++i) {
                const Pair w = O::ldp(sG + (tok0 + sl * C::SL + i) * C::SK + pc);
                a0 += O::p0(w);
                a1 += O::p1(w);
            }
            const int slot = tok0 / C::SL + sl;
            *reinterpret_cast<f32x2*>(sSig + slot * DK + pc) = f32x2{a0 * LOG2E, a1 * LOG2E};
        }
        __syncthreads();

        KDA_PHASE(2);
        // ---- phase B: decayed operand tiles and channel vectors
        {
            float R0[5], R1[5];  // G before sub-tile a (log2 domain); R[4] = G at chunk end
            R0[0] = R1[0] = 0.f;
            float r0 = 0.f, r1 = 0.f, G0 = 0.f, G1 = 0.f;
#pragma unroll
            for (int sl = 0; sl < C::NSLOT; ++sl) {
                if (sl == tok0 / C::SL) {
                    G0 = r0;
                    G1 = r1;
                }
                const f32x2 sg = *reinterpret_cast<const f32x2*>(sSig + sl * DK + pc);
                r0 += sg[0];
                r1 += sg[1];
                if (((sl + 1) * C::SL) % 16 == 0) {
                    R0[((sl + 1) * C::SL) / 16] = r0;
                    R1[((sl + 1) * C::SL) / 16] = r1;
                }
            }
            if (part == 0) {
                f32x2* vv = reinterpret_cast<f32x2*>(sVec);
#pragma unroll
                for (int a = 0; a < 4; ++a) vv[((V_ER + a) * DK + pc) / 2] = f32x2{fexp2(R0[a]), fexp2(R1[a])};
                // key side of block (a, b): e^{R_a - R_b} = e^{E_b - R_b} e^{R_a - E_b}; the
                // first factor is >= e^-80 (one sub-tile), the second may underflow only
                // when the true value is negligible; the multiply keeps denormals
#pragma unroll
                for (int a = 1; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < a; ++b)
                        vv[((V_YS + ys_slot(a, b)) * DK + pc) / 2] =
                            f32x2{fexp2(R0[b + 1] - R0[b]) * fexp2(R0[a] - R0[b + 1]),
                                  fexp2(R1[b + 1] - R1[b]) * fexp2(R1[a] - R1[b + 1])};
                vv[(V_GC * DK + pc) / 2] = f32x2{fexp2(R0[4]), fexp2(R1[4])};
            }
            // all loads of this thread's tokens first
            Pair wg[C::TPT], wk[C::TPT], wq[C::TPT];
#pragma unroll
            for (int i = 0; i < C::TPT; ++i) {
                const int r = tok0 + i;
                wg[i] = O::ldp(sG + r * C::SK + pc);
                wk[i] = O::ldp(sK + r * C::SK + pc);
                if (!SUMMARY) wq[i] = O::ldp(sQ + r * C::SK + pc);
            }
            float kh0[C::TPT], kh1[C::TPT];
            // the thread's tokens cover whole sub-tiles (TPT >= 16) or lie in one (TPT < 16)
            constexpr int SPAN = C::TPT < 16 ? C::TPT : 16;
#pragma unroll
            for (int i0 = 0; i0 < C::TPT; i0 += SPAN) {
                const int a = (tok0 + i0) >> 4;
                const float ra0 = a == 0 ? R0[0] : a == 1 ? R0[1] : a == 2 ? R0[2] : R0[3];
                const float ra1 = a == 0 ? R1[0] : a == 1 ? R1[1] : a == 2 ? R1[2] : R1[3];
                const float rb0 = a == 0 ? R0[1] : a == 1 ? R0[2] : a == 2 ? R0[3] : R0[4];  // E_a
                const float rb1 = a == 0 ? R1[1] : a == 1 ? R1[2] : a == 2 ? R1[3] : R1[4];
                const float er0 = fexp2(ra0), er1 = fexp2(ra1);  // e^{R_a}
                // e^{G_last - R_a} as e^{E_a - R_a} (>= e^-80) times e^{G_last - E_a}; the
                // product may be denormal, which fp32 multiplies keep
                const float fe0 = fexp2(rb0 - ra0) * fexp2(R0[4] - rb0);
                const float fe1 = fexp2(rb1 - ra1) * fexp2(R1[4] - rb1);
#pragma unroll
                for (int i = i0; i < i0 + SPAN; ++i) {
                    const int r = tok0 + i;
                    G0 += O::p0(wg[i]) * LOG2E;
                    G1 += O::p1(wg[i]) * LOG2E;
                    const float d0 = G0 - ra0, d1 = G1 - ra1;
                    const float e1a = fexp2(d0), e1b = fexp2(d1);    // e^{G - R_a} in [e^-80, 1]
                    const float e2a = fexp2(-d0), e2b = fexp2(-d1);  // e^{R_a - G} in [1, e^80]
                    const float ga = e1a * er0, gb2 = e1b * er1;                // e^{G}
                    const float k0 = O::p0(wk[i]), k1 = O::p1(wk[i]);
                    const float kf0 = k0 * e2a, kf1 = k1 * e2b;
                    O::stp(sK + r * C::SK + pc, k0 * e1a, k1 * e1b);
                    O::stp(sG + r * C::SK + pc, kf0, kf1);
                    O::stp(sKG + r * C::SK + pc, -k0 * ga, -k1 * gb2);
                    // k e^{G_last - G} = (k e^{R_a - G}) e^{G_last - R_a}
                    kh0[i] = kf0 * fe0;
                    kh1[i] = kf1 * fe1;
                    if (!SUMMARY) {
                        const float q0 = O::p0(wq[i]), q1 = O::p1(wq[i]);
                        O::stp(sQ + r * C::SK + pc, q0 * e1a, q1 * e1b);
                        O::stp(sQG + r * C::SK + pc, q0 * ga, q1 * gb2);
                    }
                }
            }
            if (tid < CH) sB[tid] = tid < len ? bload : 0.f;
            // transposed K-hat rows (channels 2cp, 2cp+1): 4 tokens per store when a
            // thread owns at least 4 (tokens 4m..4m+3 sit contiguously after pcol)
            if constexpr (C::TPT >= 4) {
#pragma unroll
                for (int i = 0; i < C::TPT; i += 4) {
                    const int tp = pcol(tok0 + i);
                    O::st4(sKH + (2 * cp) * C::ST + tp, f32x4{kh0[i], kh0[i + 1], kh0[i + 2], kh0[i + 3]});
                    O::st4(sKH + (2 * cp + 1) * C::ST + tp, f32x4{kh1[i], kh1[i + 1], kh1[i + 2], kh1[i + 3]});
                }
            } else {
#pragma unroll
                for (int i = 0; i < C::TPT; ++i) {
                    const int tp = pcol(tok0 + i);
                    sKH[(2 * cp) * C::ST + tp] = O::to_op(kh0[i]);
                    sKH[(2 * cp + 1) * C::ST + tp] = O::to_op(kh1[i]);
                }
            }
        }
        __syncthreads();

        KDA_PHASE(3);
        // ---- prefetch the next chunk while the chain runs
        if (ci + 1 < nchunks) {
            const int64_t n0 = c0 + CH;
            raw_prefetch<C, DT>(pre, gq, gk, gv, gg, n0, int(t_end - n0 < CH ? t_end - n0 : CH), p.T_total,
                                H, h, tid, DK, DV);
        }

        KDA_PHASE(4);
        // ---- chain part 1: X = V - (K . e^G) S   (rows = tokens; 4 row tiles x 2 column tiles)
        Frag Sb[DK / 32][NCT];
        f32x4 Xt[4][NCT];
        if (chain) {
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Sb[kb][ct] = acc_frag<DT>(S[2 * kb][ct], S[2 * kb + 1][ct]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Xt[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!mcols) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const Frag vf = O::load(sV + (rt * 16 + l16) * C::SV + (colbase & ~31) + 8 * q4);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) O::mma(Xt[rt][ct], vf, Iden[ct]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const Frag af = O::load(sKG + (rt * 16 + l16) * C::SK + kb * 32 + 8 * q4);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) O::mma(Xt[rt][ct], af, Sb[kb][ct]);
                }
        }
        KDA_PHASE(5);
        // ---- products per 16x16 block (a, b), b <= a, sharing the key-side fragment:
        //      -A x beta_r (strictly lower, natural columns) and P (lower incl. diagonal)
        // With 8 waves, waves 4..7 take the diagonal blocks and invert them at once
        // (their own LDS writes, so no barrier), while waves 0..3 take the six
        // off-diagonal blocks.  Otherwise blocks go round-robin and the
        // inversion follows in its own phase.
        constexpr bool DIAG_WAVES = C::NW == 8;
        const int ntask = DIAG_WAVES ? (wave < 4 ? (wave < 2 ? 2 : 1) : 1) : (10 - wave + C::NW - 1) / C::NW;
        for (int tk = 0; tk < ntask; ++tk) {
            int a, b;
            if (DIAG_WAVES) {
                if (wave >= 4) {
                    a = b = wave - 4;
                } else {
                    const int ot = wave + 4 * tk;  // off-diagonal (1,0),(2,0),(2,1),(3,0),(3,1),(3,2)
                    a = ot == 0 ? 1 : ot <= 2 ? 2 : 3;
                    b = ot == 0 ? 0 : ot == 1 ? 0 : ot == 2 ? 1 : ot - 3;
                }
            } else {
                int bi = wave + tk * C::NW;
                a = 0;
                while (bi > a) {
                    bi -= a + 1;
                    ++a;
                }
                b = bi;  // 0 <= b <= a
            }
            Frag yf[DK / 32], kf[DK / 32], qf[DK / 32];
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                yf[kb] = O::load(sG + (b * 16 + l16) * C::SK + kb * 32 + 8 * q4);
                kf[kb] = O::load(sK + (a * 16 + l16) * C::SK + kb * 32 + 8 * q4);
                if (!SUMMARY) qf[kb] = O::load(sQ + (a * 16 + l16) * C::SK + kb * 32 + 8 * q4);
            }
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag y = yf[kb];
                if (b < a) {  // off-diagonal: key side moved from R_b to R_a
                    float t[8];
                    O::unpack(y, t);
                    const f32x4* fv = reinterpret_cast<const f32x4*>(sVec + (V_YS + ys_slot(a, b)) * DK + kb * 32 + 8 * q4);
                    const f32x4 f0 = fv[0], f1 = fv[1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        t[e] *= f0[e];
                        t[4 + e] *= f1[e];
                    }
                    y = O::make(t);
                }
                O::mma(accA, y, kf[kb]);
                if (!SUMMARY) O::mma(accP, y, qf[kb]);
            }
            // acc: lane (col r = 16a + l16, rows i = 16b + 4*q4 + j)
            const int r = a * 16 + l16;
            const int i0 = b * 16 + 4 * q4;
            const float br = -sB[r];
            f32x4 v4;
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] = (i0 + j < r) ? br * accA[j] : 0.f;
            O::st4(sA + r * C::ST + i0, v4);
            if (!SUMMARY) {
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[j] = (i0 + j <= r) ? accP[j] : 0.f;
                O::st4(sP + r * C::ST + pcol(i0), v4);
            }
            if (DIAG_WAVES && wave >= 4) {
                // this wave's block is complete in LDS (in-order within the wave)
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                diag_inverse<C, O>(sA, sD, sDS, a, lane);
            }
        }
        __syncthreads();

        KDA_PHASE(6);
        // ---- diagonal blocks (I + A_aa)^{-1} (when not already done in the products phase)
        if (!DIAG_WAVES) {
            for (int a = wave; a < 4; a += C::NW) diag_inverse<C, O>(sA, sD, sDS, a, lane);
        }
        KDA_PHASE(7);
        if (!DIAG_WAVES) __syncthreads();
        KDA_PHASE(8);

        if (chain) {
            // ---- U = (I + A)^{-1} Diag(beta) X by block forward substitution:
            //      U_a = D_a (beta_a X_a - sum_{b<a} A_ab U_b)
            f32x4 Ut[4][NCT];
            Frag4 Uf[4][NCT];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 bv = *reinterpret_cast<const f32x4*>(sB + a * 16 + 4 * q4);
                f32x4 R[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) R[ct] = bv * Xt[a][ct];
#pragma unroll
                for (int b = 0; b < a; ++b) {
                    const Frag4 af = O::load4(sA + (a * 16 + l16) * C::ST + b * 16 + 4 * q4);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) O::mma4(R[ct], af, Uf[b][ct]);
                }
                const Frag4 df = O::load4(sD + (a * 16 + l16) * C::SD + 4 * q4);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    Ut[a][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                    O::mma4(Ut[a][ct], df, O::make4(R[ct]));
                    Uf[a][ct] = O::make4(Ut[a][ct]);
                }
            }
            KDA_PHASE(10);
            Frag Ub[2][NCT];
#pragma unroll
            for (int kbt = 0; kbt < 2; ++kbt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Ub[kbt][ct] = acc_frag<DT>(Ut[2 * kbt][ct], Ut[2 * kbt + 1][ct]);

            if (!SUMMARY) {
                // ---- O^T = S^T (Q . e^G)^T + U^T P^T: the register fragments of S and U
                //      serve as the left operand, so each lane ends up holding four
                //      consecutive value columns of one token (one 8-byte store)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f32x4 Ot[NCT];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) Ot[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < DK / 32; ++kb) {
                        const Frag bf = O::load(sQG + (rt * 16 + l16) * C::SK + kb * 32 + 8 * q4);
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) O::mma(Ot[ct], Sb[kb][ct], bf);
                    }
#pragma unroll
                    for (int kbt = 0; kbt <= rt / 2; ++kbt) {
                        const Frag pf = O::load(sP + (rt * 16 + l16) * C::ST + kbt * 32 + 8 * q4);
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) O::mma(Ot[ct], Ub[kbt][ct], pf);
                    }
                    const int row = rt * 16 + l16;  // token
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const int col = colbase + ct * 16 + 4 * q4;
                        if (C::STAGE_O) store4<DT>(sO + row * C::SO + col, Ot[ct]);
                        else if (row < len) store4<DT>(go + ((c0 + row) * H + h) * DV + col, Ot[ct]);
                    }
                }
            }

            KDA_PHASE(11);
            // ---- S <- Diag(e^{G_last}) S + (K . e^{G_last - G})^T U
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                // channels rt*16 + 4q .. +3 are stored contiguously (permuted position)
                const f32x4 gc = *reinterpret_cast<const f32x4*>(sVec + V_GC * DK + pcol(rt * 16 + 4 * q4));
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) S[rt][ct] *= gc;
#pragma unroll
                for (int kbt = 0; kbt < 2; ++kbt) {
                    const Frag kf = O::load(sKH + (rt * 16 + l16) * C::ST + kbt * 32 + 8 * q4);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) O::mma(S[rt][ct], kf, Ub[kbt][ct]);
                }
            }
        }
        prev_c0 = c0;
        prev_len = len;
    }
    if (!SUMMARY && C::STAGE_O && nchunks > 0) {
        __syncthreads();
        store_out_tile<C, DT, DV>(smem, go, prev_c0, prev_len, H, h, tid);
    }

    KDA_PHASE(9);
#ifdef KDA_PHASE_TIMING
    if (tid == KDA_PHASE_TID && blockIdx.x < 16384)
        for (int i = 0; i < 12; ++i) kda_phase_cycles[blockIdx.x * 16 + i] = phase_acc[i];
#endif
    // ---- write the segment result
    if (chain) {
        float* dst = nullptr;
        int ld = DV;
        if (SUMMARY) {
            dst = p.ms + (int64_t(item) * H + h) * DK * (DK + DV);  // [S~ | M], rows of DK + DV
            ld = DK + DV;
        } else if (last_seg && p.fin) {
            dst = p.fin + (int64_t(n) * H + h) * DK * DV;
        }
        if (dst) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        dst[(rt * 16 + 4 * q4 + j) * ld + colbase + ct * 16 + l16] = S[rt][ct][j];
        }
    }
}

// ------------------------------------------------------------- scan kernel
// Per (sequence, head, 32-column slice of the state):
//     S_in(s+1) = M_s S_in(s) + S~_s
// over the sequence's segments, on the matrix cores with fp32-level accuracy:
// each fp32 operand x is split as hi = bf16(x), lo = bf16(x - hi) and the
// product accumulates hi*hi + hi*lo + lo*hi in fp32.  Per step the workgroup
// stages M_s in LDS (next step's M prefetched into registers during this
// step's products) and keeps its S_in slice in LDS, transposed, as the other
// operand.  Wave w owns state row tiles w, w+4, ... and both column tiles.
constexpr int SCAN_COLS = 32;
template <int DK, int DV>
struct ScanCfg {
    static constexpr int SM = DK + 4;                 // fp32 row stride of M and S_in^T in LDS
    static constexpr int UNITS = DK * (DK / 4);       // 16-byte units of M
    static constexpr int UPT = (UNITS + 255) / 256;
    static constexpr int RTW = (DK / 16 + 3) / 4;     // row tiles per wave
    static constexpr int LDS = (DK + SCAN_COLS) * SM * 4;
};

__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo)
{
    float h[8], l[8];
    hi = Op<BF16>::make(x);
    Op<BF16>::unpack(hi, h);
#pragma unroll
    for (int e = 0; e < 8; ++e) l[e] = x[e] - h[e];
    lo = Op<BF16>::make(l);
}

template <int DK, int DV>
__global__ void __launch_bounds__(256) scan_kernel(PrefillDev p)
{
    using SC = ScanCfg<DK, DV>;
    constexpr int NB = DV / SCAN_COLS;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float* sM = reinterpret_cast<float*>(smem);  // [DK][SM]: M_s rows
    float* sT = sM + DK * SC::SM;                // [32][SM]: S_in slice, transposed (column j, row k)
    const int H = p.H;
    const int jb = blockIdx.x % NB;
    const int h = (blockIdx.x / NB) % H;
    const int n = blockIdx.x / (NB * H);
    const int32_t* seg_off = p.tab + (p.N + 1);
    const int32_t* p1_off = p.tab + 2 * (p.N + 1);
    const int nseg = seg_off[n + 1] - seg_off[n];
    if (nseg <= 1) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int col0 = jb * SCAN_COLS;
    auto ms_of = [&](int st) { return p.ms + (int64_t(p1_off[n] + st) * H + h) * DK * (DK + DV); };

    for (int e = tid; e < SCAN_COLS * DK; e += 256) {
        const int j = e / DK, k = e % DK;
        sT[j * SC::SM + k] = p.init ? p.init[(int64_t(n) * H + h) * DK * DV + k * DV + col0 + j] : 0.f;
    }
    f32x4 pre[SC::UPT];
    f32x4 nxt[SC::RTW][2];
    // M_st (columns DV .. DV+DK-1 of each row) and this wave's S~_st tiles
    // (columns 0 .. DV-1) into registers; consumed one step later.
    auto load_step = [&](int st) {
        const float* base = ms_of(st);
#pragma unroll
        for (int i = 0; i < SC::UPT; ++i) {
            const int u = tid + i * 256;
            if (SC::UNITS % 256 == 0 || u < SC::UNITS)
                pre[i] = *reinterpret_cast<const f32x4*>(base + DV + (u / (DK / 4)) * (DK + DV) + (u % (DK / 4)) * 4);
        }
#pragma unroll
        for (int i = 0; i < SC::RTW; ++i) {
            const int rt = wave + 4 * i;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    nxt[i][ct][j] = rt < DK / 16 ? base[(rt * 16 + 4 * q4 + j) * (DK + DV) + col0 + ct * 16 + l16] : 0.f;
        }
    };
    load_step(0);
    for (int s = 0; s + 1 < nseg; ++s) {
        __syncthreads();  // sM free
#pragma unroll
        for (int i = 0; i < SC::UPT; ++i) {
            const int u = tid + i * 256;
            if (SC::UNITS % 256 == 0 || u < SC::UNITS)
                *reinterpret_cast<f32x4*>(sM + (u / (DK / 4)) * SC::SM + (u % (DK / 4)) * 4) = pre[i];
        }
        f32x4 acc[SC::RTW][2];
#pragma unroll
        for (int i = 0; i < SC::RTW; ++i)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc[i][ct] = nxt[i][ct];
        __syncthreads();
        if (s + 2 < nseg) load_step(s + 1);  // in flight during the products
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            bf16x8 bh[2], bl[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const float* b = sT + (ct * 16 + l16) * SC::SM + kb * 32 + 4 * q4;
                const f32x4 b0 = *reinterpret_cast<const f32x4*>(b), b1 = *reinterpret_cast<const f32x4*>(b + 16);
                const float x[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                split_bf16(x, bh[ct], bl[ct]);
            }
#pragma unroll
            for (int i = 0; i < SC::RTW; ++i) {
                const int rt = wave + 4 * i;
                if (rt < DK / 16) {
                    const float* a = sM + (rt * 16 + l16) * SC::SM + kb * 32 + 4 * q4;
                    const f32x4 a0 = *reinterpret_cast<const f32x4*>(a), a1 = *reinterpret_cast<const f32x4*>(a + 16);
                    const float x[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                    bf16x8 ah, al;
                    split_bf16(x, ah, al);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        Op<BF16>::mma(acc[i][ct], ah, bh[ct]);
                        Op<BF16>::mma(acc[i][ct], ah, bl[ct]);
                        Op<BF16>::mma(acc[i][ct], al, bh[ct]);
                    }
                }
            }
        }
        __syncthreads();  // every wave is done reading sT
        float* out = p.sin + (int64_t(seg_off[n] + s + 1) * H + h) * DK * DV;
#pragma unroll
        for (int i = 0; i < SC::RTW; ++i) {
            const int rt = wave + 4 * i;
            if (rt < DK / 16) {
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const int j = ct * 16 + l16;
                    *reinterpret_cast<f32x4*>(sT + j * SC::SM + rt * 16 + 4 * q4) = acc[i][ct];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) out[(rt * 16 + 4 * q4 + jj) * DV + col0 + j] = acc[i][ct][jj];
                }
            }
        }
    }
}

// ------------------------------------------------------------------ launch
template <typename DT, int DK, int DV>
hipError_t launch_prefill_t(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t stream)
{
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    int32_t* tab = reinterpret_cast<int32_t*>(ws + plan.off_table);
    PrefillDev d{a.q, a.k, a.v, a.g, a.beta, tab, a.N, a.T_total, a.H, plan.seg_chunks,
                 a.init, a.fin, a.o,
                 plan.np1_max > 0 ? reinterpret_cast<float*>(ws + plan.off_ms) : nullptr,
                 plan.np1_max > 0 ? reinterpret_cast<float*>(ws + plan.off_sin) : nullptr};
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, a.cu, a.N, a.T_total,
                       plan.seg_chunks, tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (plan.np1_max > 0) {
        using C1 = ChunkCfg<DT, DK, DV, true>;
        auto k1 = prefill_chunk_kernel<DT, DK, DV, true>;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1),
                                hipFuncAttributeMaxDynamicSharedMemorySize, C1::LDS);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k1, dim3(unsigned(plan.np1_max * a.H)), dim3(C1::NT), C1::LDS, stream, d);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        auto ks = scan_kernel<DK, DV>;
        constexpr int scan_lds = ScanCfg<DK, DV>::LDS;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(ks), hipFuncAttributeMaxDynamicSharedMemorySize,
                                scan_lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(ks, dim3(unsigned(a.N * a.H * (DV / SCAN_COLS))), dim3(256), scan_lds, stream, d);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    using C3 = ChunkCfg<DT, DK, DV, false>;
    auto k3 = prefill_chunk_kernel<DT, DK, DV, false>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k3),
                            hipFuncAttributeMaxDynamicSharedMemorySize, C3::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k3, dim3(unsigned(plan.nseg_max * a.H)), dim3(C3::NT), C3::LDS, stream, d);
    return hipGetLastError();
}

template <typename DT>
hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t stream)
{
#define KDA_PF(DKV, DVV)                                                                       \
    if (a.dk == DKV && a.dv == DVV) return launch_prefill_t<DT, DKV, DVV>(a, plan, stream);
    if constexpr (DT::is_bf16) {
        KDA_PF(32, 32) KDA_PF(32, 64) KDA_PF(32, 128)
        KDA_PF(64, 32) KDA_PF(64, 64) KDA_PF(64, 128)
        KDA_PF(128, 32) KDA_PF(128, 64) KDA_PF(128, 128)
    } else {
        KDA_PF(32, 32) KDA_PF(32, 64)
    }
#undef KDA_PF
    return hipErrorInvalidValue;
}

}  // namespace kda
