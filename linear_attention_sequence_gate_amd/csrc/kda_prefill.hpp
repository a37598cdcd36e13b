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

#include <cmath>
#include <cstdio>
#include <string>
#include <type_traits>

#include "kda_common.hpp"

namespace kda {

// Optional per-phase cycle counters of the chunk kernel (built only with
// -DKDA_PHASE_TIMING; the default build compiles the markers away).
#ifdef KDA_PHASE_TIMING
#ifndef KDA_PHASE_TID
#define KDA_PHASE_TID 0
#endif
__device__ unsigned long long kda_phase_cycles[16384 * 16];
struct PhaseClock {
    long long acc[16] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    long long last = 0;
    bool on = false;
    __device__ void mark(int i)
    {
        if (on) {
            const long long t = clock64();
            acc[i] += t - last;
            last = t;
        }
    }
    __device__ void save(int base = 0)
    {
        if (on && base + blockIdx.x < 16384)
            for (int i = 0; i < 16; ++i) kda_phase_cycles[(base + blockIdx.x) * 16 + i] = acc[i];
    }
};
#else
struct PhaseClock {
    __device__ void mark(int) {}
    __device__ void save(int = 0) {}
};
#endif
#define KDA_PHASE(i) pclk.mark(i)

constexpr int CH = 64;  // tokens per chunk
constexpr int NCU_TARGET = 256;

// ---------------------------------------------------------------- host plan
// A long sequence is cut into segments of L chunks that run in parallel.  Two
// ways give each segment its incoming state:
//   warm-up (the default where d_k <= d_v): the workgroup of segment s > 0
//     first runs the `warm` tokens before the segment from a zero state,
//     carrying the window's transition M beside the state ([S~ | M], M's
//     columns start at I and see no v).  The incoming state is M S(window
//     start) + S~; when the computed M is exactly zero (every entry has
//     underflowed, as it does within about a hundred tokens of the decay the
//     gate's bound produces) it is S~, and the segment runs on.  A window that
//     reaches the sequence start begins from the initial state instead and
//     needs no check.  A segment whose M is not zero flags its (sequence,
//     head), and the exact passes below then run for every flagged chain.
//   exact passes: a summary pass computes every non-final segment's [S~ | M]
//     over the whole segment, a scan composes S_in(s+1) = M_s S_in(s) + S~_s,
//     and an output pass reruns every segment from its true incoming state.
struct PrefillPlan {
    int seg_chunks = 1;        // chunks per segment (L)
    int warm = 0;              // warm-up tokens (a multiple of the 32-token block); 0: exact passes only
    int64_t nseg_max = 0;      // upper bound on the number of segments
    int64_t np1_max = 0;       // upper bound on the number of non-final segments
    size_t off_table = 0, off_flags = 0, off_ms = 0, off_sin = 0;
    size_t workspace_bytes = 0;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int WARM_DEFAULT = 128;  // tokens

// Whether the warm-up kernel exists for this head shape: its chain waves own
// 16 state columns each and, during the warm-up, one 16-column tile of M
// beside them, so M's d_k columns must fit in d_v / 16 tiles.
constexpr bool warm_shape(int dk, int dv) { return dk <= dv; }

// force_L > 0 fixes the segment length (in chunks); warm_req < 0 takes the
// default warm-up, 0 turns it off, > 0 sets it (a multiple of 32 tokens).
inline PrefillPlan prefill_plan(int64_t T_total, int N, int H, int dk, int dv, int force_L = 0, int warm_req = -1)
{
    PrefillPlan p;
    p.warm = warm_req < 0 ? WARM_DEFAULT : warm_req;
    if (!warm_shape(dk, dv)) p.warm = 0;
    const int64_t chunks_bound = (T_total + CH - 1) / CH + N;  // >= total chunks over sequences
    const int64_t max_seq_chunks = (T_total + CH - 1) / CH;
    const int64_t per_cu = (int64_t(H) * chunks_bound + NCU_TARGET - 1) / NCU_TARGET;
    int64_t L;
    int64_t L_min = 16;  // the exact passes: a segment's summary and scan step must pay off
    if (p.warm > 0 && N == 1) {
        // one (segment, head) item per compute unit: a segment costs its own
        // blocks plus a short warm-up, so fewer, longer segments waste least;
        // with few heads segments may be as short as twice the default window
        const int64_t nseg = NCU_TARGET / H > 1 ? NCU_TARGET / H : 1;
        L = (max_seq_chunks + nseg - 1) / nseg;
        L_min = 4;
    } else if (p.warm > 0) {
        L = per_cu / 8;  // several items per unit, so long sequences do not end last (1.03M tokens
                         // in 64 sequences: 14.4 ms per call, against 15.7 with per_cu / 4)
    } else {
        L = per_cu / 2;  // the summary and output passes each fill the units once
    }
    if (L < L_min) L = L_min;
    if (force_L > 0) L = force_L;
    if (L >= max_seq_chunks) L = max_seq_chunks > 0 ? max_seq_chunks : 1;  // nothing splits
    p.seg_chunks = int(L);
    if (N == 1) {
        // one sequence of at most max_seq_chunks chunks: the count is exact,
        // so no launch carries workgroups that only return (at one workgroup
        // per compute unit they would take a dispatch round of their own)
        p.nseg_max = max_seq_chunks > L ? (max_seq_chunks + L - 1) / L : 1;
        p.np1_max = p.nseg_max - 1;
    } else {
        p.nseg_max = chunks_bound / L + N + 1;
        p.np1_max = (max_seq_chunks > L) ? chunks_bound / L + 1 : 0;
    }
    size_t off = 0;
    p.off_table = off;
    off = align256(off + sizeof(int32_t) * 5 * size_t(N + 1));
    if (p.warm > 0) {
        p.off_flags = off;
        off = align256(off + sizeof(int32_t) * size_t(p.nseg_max) * H);
    }
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
    float* ckpt = nullptr;  // state checkpoints (or null)
    int ckpt_interval = 0;  // tokens between checkpoints (multiple of CH), 0 = none
    int64_t ckpt_cap = 0;   // checkpoints the buffer holds
    const float* gate_A = nullptr;  // non-null: g holds the gate's input z, and g = g_min sigmoid(e^{A_h} z)
    float g_min = -5.f;
    int init_snap = 0;  // initial_state is final_state: passes after the first read a copy of it
};

// Device-side view shared by the prefill kernels.
struct PrefillDev {
    const void *q, *k, *v, *g, *beta;
    const int32_t* tab;  // cuc[N+1] | seg_off[N+1] | p1_off[N+1] | ckpt_off[N+1]
    int N;
    int64_t T_total;
    int H;
    int L;  // chunks per segment
    const float* init;
    float* fin;
    void* o;
    float* ms;   // [np1][H][dk][dk+dv]
    float* sin;  // [nseg][H][dk][dv]
    float* ckpt;  // [ckpt_cap][H][dk][dv] or null
    int ckpt_interval;
    int64_t ckpt_cap;
    // One sequence without cu_seqlens: the table is [0, T] | [0, nseg] |
    // [0, nseg - 1] | [0, nck], known on the host and carried here, so no
    // plan launch is needed.
    int single;
    int single_nseg;
    int single_nck;
    const float* gate_A;  // non-null: the gate is applied to g (which holds z) in the decay stage
    float g_min;
    int32_t* flags;  // [nseg_max][H]: 1 where a segment's warm-up left M non-zero; null: no warm-up pass
    int warm;        // warm-up tokens
    int64_t nseg_cap = 0, np1_cap = 0;  // the plan's segment and non-final segment counts (bounds checks)
    // 1: the initial state is also the final state, which a warm-up workgroup
    // may write before a later pass reads the initial state; so the warm-up
    // pass copies each sequence's initial state (row-major) into its segment
    // 0 slot of `sin` (the scan writes slots 1..) and the later passes read it
    // there
    int init_snap = 0;
};

// Table entries (cu_seqlens clamped, segment, pass-1 and checkpoint offsets)
__device__ __forceinline__ int32_t tab_cu(const PrefillDev& p, int n)
{
    return p.single ? (n ? int32_t(p.T_total) : 0) : p.tab[n];
}
__device__ __forceinline__ int32_t tab_seg(const PrefillDev& p, int n)
{
    return p.single ? (n ? p.single_nseg : 0) : p.tab[(p.N + 1) + n];
}
__device__ __forceinline__ int32_t tab_p1(const PrefillDev& p, int n)
{
    return p.single ? (n ? p.single_nseg - 1 : 0) : p.tab[2 * (p.N + 1) + n];
}
__device__ __forceinline__ int32_t tab_ck(const PrefillDev& p, int n)
{
    return p.single ? (n ? p.single_nck : 0) : p.tab[3 * (p.N + 1) + n];
}

// ------------------------------------------------------------- plan kernel
// One workgroup: clamps cu_seqlens into a non-decreasing sequence inside
// [0, T_total] and writes the per-sequence segment, pass-1 and checkpoint
// offsets (a sequence of length len holds len / ckpt_interval checkpoints),
// then the warm-up kernel's dispatch order of the sequences' final segments:
// longest first (a counting sort on the chunk count, PERM_BUCKETS buckets,
// the longest sharing the last), so no long item starts last.
constexpr int PERM_BUCKETS = 1024;
__global__ void __launch_bounds__(256) plan_kernel(const int32_t* __restrict__ cu, int N,
                                                   int64_t T_total, int L, int ckpt_interval,
                                                   int32_t* __restrict__ tab)
{
    __shared__ int32_t s_seg[256], s_p1[256], s_cu[256], s_ck[256];
    __shared__ int32_t carry_seg, carry_p1, carry_cu, carry_ck;
    int32_t* cuc = tab;
    int32_t* seg_off = tab + (N + 1);
    int32_t* p1_off = tab + 2 * (N + 1);
    int32_t* ck_off = tab + 3 * (N + 1);
    const int t = threadIdx.x;
    if (t == 0) {
        carry_seg = 0;
        carry_p1 = 0;
        carry_cu = 0;
        carry_ck = 0;
        cuc[0] = 0;
        seg_off[0] = 0;
        p1_off[0] = 0;
        ck_off[0] = 0;
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
        int32_t nseg = 0, np1 = 0, nck = 0;
        if (n < N) {
            const int64_t len = int64_t(c1m) - c0m;
            const int64_t ch = (len + CH - 1) / CH;
            int64_t ns = (ch + L - 1) / L;
            if (ns < 1) ns = 1;
            nseg = int32_t(ns);
            np1 = int32_t(ns - 1);
            nck = ckpt_interval > 0 ? int32_t(len / ckpt_interval) : 0;
        }
        s_seg[t] = nseg;
        s_p1[t] = np1;
        s_ck[t] = nck;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {  // inclusive sum-scans
            const int32_t a = (t >= d) ? s_seg[t - d] : 0;
            const int32_t b = (t >= d) ? s_p1[t - d] : 0;
            const int32_t c = (t >= d) ? s_ck[t - d] : 0;
            __syncthreads();
            s_seg[t] += a;
            s_p1[t] += b;
            s_ck[t] += c;
            __syncthreads();
        }
        if (n < N) {
            cuc[n + 1] = c1m;
            seg_off[n + 1] = carry_seg + s_seg[t];
            p1_off[n + 1] = carry_p1 + s_p1[t];
            ck_off[n + 1] = carry_ck + s_ck[t];
        }
        __syncthreads();
        if (t == 255) {
            carry_seg += s_seg[255];
            carry_p1 += s_p1[255];
            carry_cu = s_cu[255];
            carry_ck += s_ck[255];
        }
        __syncthreads();
    }
    // ---- final segments, longest first (the barrier above makes this
    // workgroup's table writes visible to all of it)
    __shared__ int32_t s_hist[PERM_BUCKETS];
    int32_t* perm = tab + 4 * (N + 1);
    auto bucket_of = [&](int n) {  // reversed chunk count of n's final segment: 0 = longest
        const int64_t len = int64_t(cuc[n + 1]) - cuc[n];
        const int64_t ch = (len + CH - 1) / CH;
        int64_t ns = (ch + L - 1) / L;
        if (ns < 1) ns = 1;
        int64_t f = ch - (ns - 1) * L;  // in [0, L]
        if (f > PERM_BUCKETS - 1) f = PERM_BUCKETS - 1;
        return PERM_BUCKETS - 1 - int(f);
    };
    for (int b = t; b < PERM_BUCKETS; b += 256) s_hist[b] = 0;
    __syncthreads();
    for (int n = t; n < N; n += 256) atomicAdd(&s_hist[bucket_of(n)], 1);
    __syncthreads();
    // exclusive scan of the buckets: each thread sums its four, the 256 sums
    // are scanned, then each thread writes its four starts
    constexpr int BPT = PERM_BUCKETS / 256;
    int32_t own = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) own += s_hist[BPT * t + i];
    s_seg[t] = own;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int32_t a = (t >= d) ? s_seg[t - d] : 0;
        __syncthreads();
        s_seg[t] += a;
        __syncthreads();
    }
    int32_t start = s_seg[t] - own;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int32_t c = s_hist[BPT * t + i];
        s_hist[BPT * t + i] = start;
        start += c;
    }
    __syncthreads();
    for (int n = t; n < N; n += 256) perm[atomicAdd(&s_hist[bucket_of(n)], 1)] = n;
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

// Offset of 16x16 tile (rt, ct) of a [d_k][DV] fp32 state held in the
// matrix-core accumulator layout: 64 lanes x 4 consecutive floats, lane
// l16 + 16 q holding column 16 ct + l16, rows 16 rt + 4 q .. +3.  The
// workspace keeps S~ and S_in this way, so each lane moves one 16-byte vector
// per tile.
template <int DV>
__host__ __device__ constexpr int acc_tile_off(int rt, int ct, int lane)
{
    return ((rt * (DV / 16) + ct) * 64 + lane) * 4;
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

// ------------------------------------------------------------ block kernel
// The recurrence advances in blocks of BC = 32 tokens (two 16-token sub-tiles).
// Waves have two roles inside a workgroup:
//   chain waves (NCW, 32 or 64 state columns each) hold their columns of the state
//   in registers for the whole segment and run X, U, O and the state update;
//   prep waves (4) build every state-independent operand of the NEXT block:
//   the decayed q/k tiles, the channel vectors, the products A and P and the
//   inverses of the diagonal blocks of (I + A).
// Two stages per block, one barrier each:
//   alpha:  chain X_b = V_b - (K.e^G)_b S        | prep: A_b, P_b, (I + A_aa)^{-1}
//   beta:   chain U_b, O_b, S <- ...             | prep: tiles of block b+1 from
//                                                   registers; loads of block b+2
// so the vector work of one block runs beside the matrix work of the other.
// Only the tiles that the two roles touch in the same stage are double
// buffered (q.e^G, K-hat^T, e^{G_last}, beta).
constexpr int BC = 32;

// The three passes of the block kernel: the output pass (from a known
// incoming state), the summary pass ([S~ | M] of a segment) and the warm-up
// output pass (incoming state from a warm-up window, see the plan above).
enum { MODE_OUT = 0, MODE_SUMMARY = 1, MODE_WARM = 2 };

template <typename DT, int DKV, int DVV, int MODE>
struct BlockCfg {
    static constexpr bool SUMMARY = MODE == MODE_SUMMARY;
    static constexpr bool WARM = MODE == MODE_WARM;
    static constexpr int DK = DKV, DV = DVV;
    static constexpr int NCOL = SUMMARY ? DV + DK : DV;  // extended state columns
    // state columns per chain wave (64 was measured slower for the summary
    // pass: the chain's vector work, not its LDS reads, competes with the
    // prep).  The warm-up pass holds 16 state columns per wave, plus one
    // 16-column tile of M during the warm-up: 16 waves fit at four per SIMD.
    static constexpr int CW = WARM ? 16 : 32;
    static constexpr int NCT = CW / 16;                   // 16-wide column tiles per chain wave
    static constexpr int NCW = NCOL / CW;                 // chain waves
    // prep waves: two per SIMD for heads with d_k >= 64 (their vector work,
    // the gate's included when it is fused, is the longer side of the
    // pipeline in both passes: the summary pass then runs 16 waves at 118
    // VGPRs), one otherwise
    static constexpr int NPW = (DKV >= 64) ? 8 : 4;
    static constexpr int NW = NCW + NPW;
    static constexpr int NT = 64 * NW;
    static constexpr int NPT = 64 * NPW;       // prep threads
    static constexpr int CP = DK / 2;          // channel pairs
    static constexpr int PARTS = NPT / CP;     // token runs per channel pair
    static constexpr int TPT = BC / PARTS;     // tokens per prep thread (one run)
    static constexpr int CPW = 64 / PARTS;     // channel pairs per prep wave
    using OT = typename Op<DT>::T;
    static constexpr int ES = sizeof(OT);
    static constexpr int SK = DK + 16 / ES;  // padded row strides (elements)
    static constexpr int SV = DV + 16 / ES;
    static constexpr int ST = BC + 16 / ES;
    static constexpr int SD = 16 + 16 / ES;
    static constexpr int TILE_K = BC * SK * ES;
    static constexpr int TILE_H = DK * ST * ES;
    static constexpr int TILE_S = BC * ST * ES;
    static constexpr int TILE_D = 16 * SD * ES;
    // LDS layout (bytes)
    static constexpr int O_KE = 0;                                  // k.e^{G-R_a}
    static constexpr int O_KF = O_KE + TILE_K;                      // k.e^{R_a-G}
    static constexpr int O_QE = O_KF + TILE_K;                      // q.e^{G-R_a}
    static constexpr int O_KG = O_QE + (SUMMARY ? 0 : TILE_K);      // -k.e^{G}
    static constexpr int O_V = O_KG + TILE_K;                       // v
    static constexpr int O_QG = O_V + BC * SV * ES;                 // q.e^{G}, 2 buffers
    static constexpr int O_KH = O_QG + (SUMMARY ? 0 : 2 * TILE_K);  // (k.e^{G_last-G})^T [DK][ST], 2 buffers
    static constexpr int O_A = O_KH + 2 * TILE_H;                   // -beta_r A, natural columns
    static constexpr int O_P = O_A + TILE_S;                        // P, permuted columns
    static constexpr int O_D = O_P + (SUMMARY ? 0 : TILE_S);        // (I + A_aa)^{-1}, 2 blocks
    static constexpr int O_VEC = O_D + 2 * TILE_D;                  // fp32 channel vectors
    static constexpr int O_B = O_VEC + 3 * DK * 4;                  // beta, 2 buffers
    static constexpr int O_FLAG = O_B + 2 * BC * 4;                 // warm-up: one word per chain wave (M non-zero)
    static constexpr int LDS_TILES = O_FLAG + (WARM ? 4 * ((NCW + 3) / 4 * 4) : 0);
    // summary pass, after the last block: each M-column wave stages its 32
    // columns (fp32, rows padded to 36) to write M split and permuted
    static constexpr int MSTAGE = 36;
    static constexpr int LDS_MSTAGE = SUMMARY ? (DK / 32) * DK * MSTAGE * 4 : 0;
    static constexpr int LDS = LDS_TILES > LDS_MSTAGE ? LDS_TILES : LDS_MSTAGE;
    // v tile: 16-byte units
    static constexpr int EPU = 16 / ES;
    static constexpr int UPR_V = DV / EPU;
    static constexpr int U_V = BC * UPR_V;
    static constexpr int UPT_V = (U_V + NPT - 1) / NPT;
    static_assert(NCOL % CW == 0 && NCW >= 1, "state columns come in whole chain-wave blocks");
    static_assert(!WARM || DK <= DV, "the warm-up holds one tile of M per chain wave");
    static_assert(LDS <= 160 * 1024, "LDS budget exceeded");
    static_assert(PARTS >= 2 && BC % PARTS == 0 && CP * PARTS == NPT, "bad elementwise split");
    static_assert(16 % TPT == 0, "a token run stays inside one sub-tile");
    static_assert(NT <= 1024, "workgroup too large");
};

// channel vectors (DK fp32 each, permuted channel order):
//   V_YS       : e^{R_1 - R_0}, key side of the off-diagonal block (1, 0)
//   V_GC + buf : e^{G_last}
enum { V_YS = 0, V_GC = 1 };

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

// (I + N)^{-1} for one 16x16 diagonal block of the strictly lower N, by one
// wave on the matrix cores, entirely in registers.  N is nilpotent (N^16 = 0):
// with Q = -N,  (I + N)^{-1} = (I + Q)(I + Q^2)(I + Q^4)(I + Q^8).
// A 16x16 accumulator tile of P serves directly as the B operand of P and as
// the A operand of P^T; a row read and a column read of Q give both operands
// of Q and of Q^T.  Each power needed later as a left operand is therefore
// formed together with its transpose (Q^2 and (Q^2)^T, Q^4 and (Q^4)^T), and
// nothing goes back through LDS.  sA holds Q = -N (natural column order); the
// result goes to rows 16a.. of sD.
template <typename C, typename O>
__device__ __forceinline__ void diag_inverse(const typename O::T* sA, typename O::T* sD, int a, int lane)
{
    using OT = typename O::T;
    using Frag4 = typename O::Frag4;
    const int l16 = lane & 15, q4 = lane >> 4;
    const OT* Qb = sA + (a * 16) * C::ST + a * 16;
    const Frag4 rQ = O::load4(Qb + l16 * C::ST + 4 * q4);  // A(Q) = B(Q^T)
    f32x4 c;
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = O::from_op(Qb[(4 * q4 + j) * C::ST + l16]);
    const Frag4 cQ = O::make4(c);  // B(Q) = A(Q^T)
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 q2 = z, q2t = z;
    O::mma4(q2, rQ, cQ);   // Q^2       -> B(Q^2), A((Q^2)^T)
    O::mma4(q2t, cQ, rQ);  // (Q^2)^T   -> B((Q^2)^T), A(Q^2)
    const Frag4 f2 = O::make4(q2), f2t = O::make4(q2t);
    f32x4 p4 = z, p4t = z;
    O::mma4(p4, f2t, f2);   // Q^4
    O::mma4(p4t, f2, f2t);  // (Q^4)^T
    const Frag4 f4 = O::make4(p4), f4t = O::make4(p4t);
    f32x4 q8 = z;
    O::mma4(q8, f4t, f4);  // Q^8
    // E1 = (I + Q^4)(I + Q^8) = I + Q^4 + Q^8 + Q^4 Q^8
    f32x4 e = p4 + q8;
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] += (4 * q4 + j == l16) ? 1.f : 0.f;
    O::mma4(e, f4t, O::make4(q8));
    // E2 = (I + Q^2) E1, D = (I + Q) E2
    f32x4 e2 = e;
    O::mma4(e2, f2t, O::make4(e));
    f32x4 d = e2;
    O::mma4(d, rQ, O::make4(e2));
#pragma unroll
    for (int j = 0; j < 4; ++j) sD[(a * 16 + 4 * q4 + j) * C::SD + l16] = O::to_op(d[j]);
}

// One product of the block substitution, acc += a b: a is a 16x16 tile of
// the operand type, b the fp32 right-hand side as computed.  bf16: b goes in
// as two bf16 parts, hi = bf16(b) and lo = bf16(b - hi), two matrix
// instructions, so the right-hand side keeps about 16 bits (fp32 accumulation
// throughout).  fp32 operands: the ordinary product.
template <typename O>
__device__ __forceinline__ void sub_mma(f32x4& acc, const typename O::Frag4& a, const f32x4& b)
{
    if constexpr (std::is_same<O, Op<BF16>>::value) {
        const typename O::Frag4 hi = O::make4(b);
        const u32x2 w = __builtin_bit_cast(u32x2, hi);
        const f32x4 hf = {bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
        O::mma4(acc, a, hi);
        O::mma4(acc, a, O::make4(b - hf));
    } else {
        O::mma4(acc, a, O::make4(b));
    }
}

// The value held by lane `lane ^ dist` (dist a power of two): rows of 16 lanes
// swap with v_permlane16_swap / v_permlane32_swap, half rows with a DPP
// rotate, and smaller distances go through ds_bpermute.
__device__ __forceinline__ float xor_lanes(float x, int dist, int lane)
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
    if (dist == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, int(u), 0x128, 0xf, 0xf, false));  // row_ror:8
    return __shfl_xor(x, dist);
}

// One block's raw inputs in a prep thread's registers: q, k, g of its token
// run (two adjacent channels per token), its 16-byte units of v and, for the
// first BC threads, one beta.  Rows at or past the block's valid length
// re-read the last valid row, so no load leaves the sequence.  Only their g
// (no decay past the end) and beta are zeroed: with beta = 0 a padded row's U
// row is 0, so its q, k and v reach no valid output or state.
template <typename C, typename DT>
struct PrepRegs {
    typename Op<DT>::Pair q[C::TPT], k[C::TPT], g[C::TPT];
    u32x4 v[C::UPT_V];
    typename DT::storage b;  // raw bits: converted where used, so the load is not waited on here
};

// Parts of a block's raw inputs, loaded separately as each one's registers
// become free in the tile pass of the block before
enum PrepPart { PP_ALL, PP_G, PP_KQ, PP_B, PP_V };

template <typename C, typename DT, bool SUMMARY, int PART = PP_ALL>
__device__ __forceinline__ void prep_load(PrepRegs<C, DT>& r, const PrefillDev& p, int64_t b0, int len, int h,
                                          int ptid, int cpair, int tok0)
{
    using ST = typename DT::storage;
    using Pair = typename Op<DT>::Pair;
    const int64_t H = p.H;
    KDA_CHECK(b0 >= 0 && b0 + len <= p.T_total, CK_TOKENS);
    KDA_CHECK(len >= 1 && len <= BC, CK_BLOCK);
    // uniform per-block byte bases + 32-bit lane byte offsets (a block spans 32
    // token rows, and the host caps H so that a row is below 2^24 bytes)
    const int64_t rk0 = (b0 * H + h) * C::DK * int64_t(sizeof(ST)), rv0 = (b0 * H + h) * C::DV * int64_t(sizeof(ST));
    const char* gq = static_cast<const char*>(p.q) + rk0;
    const char* gk = static_cast<const char*>(p.k) + rk0;
    const char* gg = static_cast<const char*>(p.g) + rk0;
    const char* gv = static_cast<const char*>(p.v) + rv0;
    const uint32_t rsk = uint32_t(H) * uint32_t(C::DK * sizeof(ST)), rsv = uint32_t(H) * uint32_t(C::DV * sizeof(ST));
    const uint32_t cb = uint32_t(2 * cpair * sizeof(ST));
    // all parts at once (the first block): beta and v first, since the running
    // sums wait for g, issued last, and loads complete in issue order, so that
    // one wait covers every load here
    if constexpr (PART == PP_ALL || PART == PP_B) {
        const char* gb = static_cast<const char*>(p.beta) + (b0 * H + h) * int64_t(sizeof(ST));
        r.b = *reinterpret_cast<const ST*>(gb + __umul24(uint32_t(ptid < len ? ptid : len - 1),
                                                         uint32_t(H * sizeof(ST))));
    }
    if constexpr (PART == PP_ALL || PART == PP_V) {
#pragma unroll
        for (int j = 0; j < C::UPT_V; ++j) {
            const int u = ptid + j * C::NPT;
            if (C::U_V % C::NPT == 0 || u < C::U_V) {
                int row = u / C::UPR_V;
                row = row < len ? row : len - 1;
                const uint32_t off = __umul24(uint32_t(row), rsv) + uint32_t((u % C::UPR_V) * 16);
                r.v[j] = *reinterpret_cast<const u32x4*>(gv + off);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
        const int row = tok0 + i < len ? tok0 + i : len - 1;
        const uint32_t off = __umul24(uint32_t(row), rsk) + cb;
        if constexpr (PART == PP_ALL || PART == PP_KQ) {
            if (!SUMMARY) r.q[i] = *reinterpret_cast<const Pair*>(gq + off);
            r.k[i] = *reinterpret_cast<const Pair*>(gk + off);
        }
        if constexpr (PART == PP_ALL || PART == PP_G) r.g[i] = *reinterpret_cast<const Pair*>(gg + off);
    }
}

// Prep stage of the beta step: every state-independent tile of one block from
// the registers.  A thread owns channels 2c, 2c+1 over a run of TPT tokens;
// the runs of one channel pair sit in one wave (lanes cpl + CPW * part), so the
// running sum of g across runs is a lane scan.  Sums are kept in natural-log
// units and scaled to log2 once, inside the exponent's FMA; R_a is G before
// sub-tile a (R_0 = 0).
// `next(r, part)` loads that part of the next block's raw inputs into r; it is
// called as soon as the pass has read the part's registers for the last time
// (g after the running sums, k and q after the tile loop, beta and v after
// their stores), which gives g the most time to land: the running sums of the
// next pass wait for it first.
template <typename C, typename DT, bool SUMMARY, typename Next>
__device__ __forceinline__ void prep_tiles(PrepRegs<C, DT>& r, unsigned char* smem, int buf, int len,
                                           int lane, int ptid, int cpair, int part, int tok0, const GateZ& gz,
                                           PhaseClock& pclk, Next&& next)
{
    using O = Op<DT>;
    using OT = typename O::T;
    constexpr int DK = C::DK;
    constexpr float LOG2E = 1.4426950408889634f;
    OT* sKE = reinterpret_cast<OT*>(smem + C::O_KE);
    OT* sKF = reinterpret_cast<OT*>(smem + C::O_KF);
    OT* sQE = reinterpret_cast<OT*>(smem + C::O_QE);
    OT* sKG = reinterpret_cast<OT*>(smem + C::O_KG);
    OT* sV = reinterpret_cast<OT*>(smem + C::O_V);
    OT* sQG = reinterpret_cast<OT*>(smem + C::O_QG + buf * C::TILE_K);
    OT* sKH = reinterpret_cast<OT*>(smem + C::O_KH + buf * C::TILE_H);
    float* sVec = reinterpret_cast<float*>(smem + C::O_VEC);
    float* sB = reinterpret_cast<float*>(smem + C::O_B) + buf * BC;
    const int pc = pcol(2 * cpair);

    // inclusive running sums of g inside the run (natural log units; rows at
    // or past the valid length add nothing)
    float c0[C::TPT], c1[C::TPT];
    float s0 = 0.f, s1 = 0.f;
#ifdef KDA_PHASE_TIMING
    asm volatile("" ::"v"(r.g[C::TPT - 1]));  // the raw loads have landed
    pclk.mark(11);
#endif
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
        const bool ok = tok0 + i < len;
        s0 += ok ? gz(O::p0(r.g[i])) : 0.f;
        s1 += ok ? gz(O::p1(r.g[i])) : 0.f;
        c0[i] = s0;
        c1[i] = s1;
    }
    next(r, std::integral_constant<int, PP_G>{});
    asm volatile("" ::: "memory");  // issue them here, not with the k and q loads below
    pclk.mark(7);
    // running sums across the runs of this channel pair (lanes cpl + CPW * part):
    // an exchange butterfly over the part index.  At level d every lane adds its
    // partner's block total; lanes in the upper half also add it to their
    // prefix.  Partners add the same two numbers, so every lane of a pair ends
    // with bit-identical totals.
    float G0 = 0.f, G1 = 0.f, R10 = 0.f, R11 = 0.f, GL0 = s0, GL1 = s1;  // G before the run, at token 15, at the end
#pragma unroll
    for (int d = 1; d < C::PARTS; d <<= 1) {
        const float p0 = xor_lanes(GL0, d * C::CPW, lane), p1 = xor_lanes(GL1, d * C::CPW, lane);
        if (d == 16 / C::TPT) {  // parts 0 .. 16/TPT - 1 hold sub-tile 0
            R10 = (part & d) ? p0 : GL0;
            R11 = (part & d) ? p1 : GL1;
        }
        if (part & d) {
            G0 += p0;
            G1 += p1;
        }
        GL0 += p0;
        GL1 += p1;
    }
    const bool hi = tok0 >= 16;  // sub-tile of the run
    // e^{R_1} and e^{G_last - R_1}, each in [e^-80, 1]; every other factor is
    // one of them or their product:  e^{R_a} = 1 or e^{R_1},  e^{G_last} =
    // e^{R_1} e^{G_last - R_1},  e^{G_last - R_a} = e^{G_last} or e^{G_last - R_1}.
    // A product may be denormal or flush to zero, which only ever scales terms
    // bounded by 1.
    const float ya0 = fexp2(R10 * LOG2E), ya1 = fexp2(R11 * LOG2E);
    const float za0 = fexp2((GL0 - R10) * LOG2E), za1 = fexp2((GL1 - R11) * LOG2E);
    const float er0 = hi ? ya0 : 1.f, er1 = hi ? ya1 : 1.f;  // e^{R_a}
    const float gc0 = ya0 * za0, gc1 = ya1 * za1;            // e^{G_last}
    const float fe0 = hi ? za0 : gc0, fe1 = hi ? za1 : gc1;  // e^{G_last - R_a}
    // log2 of e^{G - R_a} = (G before the run - R_a + running sum) log2(e)
    const float off0 = (G0 - (hi ? R10 : 0.f)) * LOG2E, off1 = (G1 - (hi ? R11 : 0.f)) * LOG2E;
    pclk.mark(8);
    float kh0[C::TPT], kh1[C::TPT];
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
        const int t = tok0 + i;
        const float d0 = __builtin_fmaf(c0[i], LOG2E, off0), d1 = __builtin_fmaf(c1[i], LOG2E, off1);
        const float e1a = fexp2(d0), e1b = fexp2(d1);    // e^{G - R_a} in [e^-80, 1]
        const float e2a = fexp2(-d0), e2b = fexp2(-d1);  // e^{R_a - G} in [1, e^80]
        const float ga = e1a * er0, gb = e1b * er1;      // e^{G}
        const float k0 = O::p0(r.k[i]), k1 = O::p1(r.k[i]);
        const float kf0 = k0 * e2a, kf1 = k1 * e2b;
        O::stp(sKE + t * C::SK + pc, k0 * e1a, k1 * e1b);
        O::stp(sKF + t * C::SK + pc, kf0, kf1);
        O::stp(sKG + t * C::SK + pc, -k0 * ga, -k1 * gb);
        kh0[i] = kf0 * fe0;  // k e^{G_last - G}
        kh1[i] = kf1 * fe1;
        if (!SUMMARY) {
            const float q0 = O::p0(r.q[i]), q1 = O::p1(r.q[i]);
            O::stp(sQE + t * C::SK + pc, q0 * e1a, q1 * e1b);
            O::stp(sQG + t * C::SK + pc, q0 * ga, q1 * gb);
        }
    }
    next(r, std::integral_constant<int, PP_KQ>{});
    pclk.mark(9);
    // K-hat^T rows 2c, 2c+1 (tokens 4m..4m+3 stay contiguous under pcol)
    if constexpr (C::TPT >= 4) {
#pragma unroll
        for (int i = 0; i < C::TPT; i += 4) {
            const int tp = pcol(tok0 + i);
            O::st4(sKH + (2 * cpair) * C::ST + tp, f32x4{kh0[i], kh0[i + 1], kh0[i + 2], kh0[i + 3]});
            O::st4(sKH + (2 * cpair + 1) * C::ST + tp, f32x4{kh1[i], kh1[i + 1], kh1[i + 2], kh1[i + 3]});
        }
    } else {
#pragma unroll
        for (int i = 0; i < C::TPT; ++i) {
            const int tp = pcol(tok0 + i);
            sKH[(2 * cpair) * C::ST + tp] = O::to_op(kh0[i]);
            sKH[(2 * cpair + 1) * C::ST + tp] = O::to_op(kh1[i]);
        }
    }
    if (part == 0) {
        f32x2* vv = reinterpret_cast<f32x2*>(sVec);
        vv[(V_YS * DK + pc) / 2] = f32x2{ya0, ya1};
        vv[((V_GC + buf) * DK + pc) / 2] = f32x2{gc0, gc1};
    }
    if (ptid < BC) {
        float bv;
        if constexpr (DT::is_bf16) bv = bf16_to_f32(r.b);
        else bv = r.b;
        sB[ptid] = ptid < len ? bv : 0.f;
    }
    next(r, std::integral_constant<int, PP_B>{});
    // v rows at their permuted column positions
#pragma unroll
    for (int j = 0; j < C::UPT_V; ++j) {
        const int u = ptid + j * C::NPT;
        if (C::U_V % C::NPT == 0 || u < C::U_V) {
            const int row = u / C::UPR_V, cc = (u % C::UPR_V) * C::EPU;
            const u32x4 w = r.v[j];
            OT* rb = sV + row * C::SV;
            if constexpr (C::ES == 2) {  // 8 columns -> two runs of 4
                *reinterpret_cast<u32x2*>(rb + pcol(cc)) = u32x2{w[0], w[1]};
                *reinterpret_cast<u32x2*>(rb + pcol(cc + 4)) = u32x2{w[2], w[3]};
            } else {
                *reinterpret_cast<u32x4*>(rb + pcol(cc)) = w;
            }
        }
    }
    next(r, std::integral_constant<int, PP_V>{});
}

// Prep stage of the alpha step: per 16x16 block (a, b), b <= a, of the block
// the products -beta_r A (strictly lower, natural columns) and P (lower with
// the diagonal, permuted columns), sharing the key-side fragment.  Task t:
// blocks (0,0), (1,1), (1,0) for t = 0, 1, 2; with eight prep waves the P
// products move to their own waves (t = 3, 4, 5).  The waves holding a
// diagonal A block then invert their block of (I + A) in place
// (wave-private, no barrier).
template <typename C, typename DT, bool SUMMARY>
__device__ __forceinline__ void prep_products(unsigned char* smem, int buf, int pw, int lane, PhaseClock& pclk)
{
    using O = Op<DT>;
    using OT = typename O::T;
    using Frag = typename O::Frag;
    constexpr int DK = C::DK;
    constexpr bool SPLIT = !SUMMARY && C::NPW >= 6;
    if (pw >= (SPLIT ? 6 : 3)) return;
    const bool doA = !SPLIT || pw < 3, doP = !SUMMARY && (!SPLIT || pw >= 3);
    const int t = SPLIT && pw >= 3 ? pw - 3 : pw;
    const OT* sKE = reinterpret_cast<const OT*>(smem + C::O_KE);
    const OT* sKF = reinterpret_cast<const OT*>(smem + C::O_KF);
    const OT* sQE = reinterpret_cast<const OT*>(smem + C::O_QE);
    OT* sA = reinterpret_cast<OT*>(smem + C::O_A);
    OT* sP = reinterpret_cast<OT*>(smem + C::O_P);
    OT* sD = reinterpret_cast<OT*>(smem + C::O_D);
    const float* sVec = reinterpret_cast<const float*>(smem + C::O_VEC);
    const float* sB = reinterpret_cast<const float*>(smem + C::O_B) + buf * BC;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int a = t == 0 ? 0 : 1, b = t == 1 ? 1 : 0;
    Frag yf[DK / 32], kf[DK / 32], qf[DK / 32];
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
        yf[kb] = O::load(sKF + (b * 16 + l16) * C::SK + kb * 32 + 8 * q4);
        if (doA) kf[kb] = O::load(sKE + (a * 16 + l16) * C::SK + kb * 32 + 8 * q4);
        if (doP) qf[kb] = O::load(sQE + (a * 16 + l16) * C::SK + kb * 32 + 8 * q4);
    }
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
        Frag y = yf[kb];
        if (b < a) {  // off-diagonal: key side moved from R_0 to R_1
            float tt[8];
            O::unpack(y, tt);
            const f32x4* fv = reinterpret_cast<const f32x4*>(sVec + V_YS * DK + kb * 32 + 8 * q4);
            const f32x4 f0 = fv[0], f1 = fv[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                tt[e] *= f0[e];
                tt[4 + e] *= f1[e];
            }
            y = O::make(tt);
        }
        if (doA) O::mma(accA, y, kf[kb]);
        if (doP) O::mma(accP, y, qf[kb]);
    }
    // acc: lane (column r = 16a + l16, rows i = 16b + 4*q4 + j)
    const int rr = a * 16 + l16;
    const int i0 = b * 16 + 4 * q4;
    f32x4 v4;
    if (doA) {
        const float br = -sB[rr];
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = (i0 + j < rr) ? br * accA[j] : 0.f;
        O::st4(sA + rr * C::ST + i0, v4);
    }
    if (doP) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = (i0 + j <= rr) ? accP[j] : 0.f;
        O::st4(sP + rr * C::ST + pcol(i0), v4);
    }
    KDA_PHASE(12);
    if (doA && a == b) {
        // this wave's block is complete in LDS (in-order within the wave)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        diag_inverse<C, O>(sA, sD, a, lane);
    }
}

// Whether any segment of the chain (sequence n, head h) left its warm-up's M
// non-zero: the exact passes that follow a warm-up pass run only for those
// chains.  Every thread reads the same words, so the answer is uniform.
__device__ __forceinline__ bool chain_flagged(const PrefillDev& p, int seg0, int nseg, int h)
{
    // lane j reads segment j's flag, all at once, and the wave's ballot
    // combines them (one memory round trip, not one per segment); every wave
    // reads the same words, so the result is uniform across the workgroup
    const int lane = threadIdx.x & 63;
    bool any = false;
    for (int j0 = 0; j0 < nseg; j0 += 64) {
        const int j = j0 + lane;
        const bool f = j < nseg && p.flags[int64_t(seg0 + j) * p.H + h] != 0;
        any = any || __ballot(f) != 0;
    }
    return any;
}

// The warm-up decision of a workgroup: the chain waves' words in LDS (written
// before the barrier that ends the last warm-up block).
template <typename C>
__device__ __forceinline__ bool warm_failed(const unsigned char* smem)
{
    const int32_t* f = reinterpret_cast<const int32_t*>(smem + C::O_FLAG);
    int32_t any = 0;
#pragma unroll
    for (int w = 0; w < C::NCW; ++w) any |= f[w];
    return any != 0;
}

// The prep waves' loop: one barrier after the prologue, two per block (see
// above).  Block bi covers tokens [blk0 + bi BC, ...) clipped at t_end.  After
// the second barrier of block check_bi (when >= 0) the role ends early if the
// warm-up flags are set; the chain waves take the same decision there.
template <typename C, typename DT>
__device__ __forceinline__ void prep_role(const PrefillDev& p, unsigned char* smem, int64_t blk0, int64_t t_end,
                                          int64_t nblk, int h, int tid, int wave, int lane, int64_t check_bi,
                                          PhaseClock& pclk)
{
    constexpr bool SUMMARY = C::SUMMARY;
    const int pw = wave - C::NCW;
    const int ptid = tid - 64 * C::NCW;
    const int part = lane / C::CPW;
    const int cpair = pw * C::CPW + lane % C::CPW;
    const int tok0 = part * C::TPT;
    auto blen = [&](int64_t bi) {
        const int64_t b0 = blk0 + bi * BC;
        return int(t_end - b0 < BC ? t_end - b0 : BC);
    };
    // with the fused gate, g comes from z here; every pass applies it to the
    // same z and gets the same g
    const GateZ gz = GateZ::of_head(p.gate_A, h, p.g_min);
    PrepRegs<C, DT> pr;
    // the loads of block nb, part by part (past the last block they re-read
    // it: unconditional loads keep the wait counts exact)
    auto loads_of = [&](int64_t nb) {
        const int64_t b = nb < nblk ? nb : nblk - 1;
        return [&, b](PrepRegs<C, DT>& r, auto part_t) {
            prep_load<C, DT, SUMMARY, decltype(part_t)::value>(r, p, blk0 + b * BC, blen(b), h, ptid, cpair, tok0);
        };
    };
    if (nblk > 0) {
        prep_load<C, DT, SUMMARY>(pr, p, blk0, blen(0), h, ptid, cpair, tok0);
        prep_tiles<C, DT, SUMMARY>(pr, smem, 0, blen(0), lane, ptid, cpair, part, tok0, gz, pclk, loads_of(1));
    }
    __syncthreads();
    KDA_PHASE(4);
    for (int64_t bi = 0; bi < nblk; ++bi) {
        const int buf = int(bi & 1);
        prep_products<C, DT, SUMMARY>(smem, buf, pw, lane, pclk);  // alpha: block bi
        KDA_PHASE(0);
        __syncthreads();
        KDA_PHASE(1);
        if (bi + 1 < nblk) {  // beta: tiles of block bi+1, loads of block bi+2
            prep_tiles<C, DT, SUMMARY>(pr, smem, buf ^ 1, blen(bi + 1), lane, ptid, cpair, part, tok0, gz, pclk,
                                       loads_of(bi + 2));
            KDA_PHASE(10);
        }
        KDA_PHASE(2);
        __syncthreads();
        KDA_PHASE(3);
        if (bi == check_bi && warm_failed<C>(smem)) return;
    }
}

template <typename DT, int DK, int DV, bool SUMMARY>
__global__ void __launch_bounds__((BlockCfg<DT, DK, DV, SUMMARY ? MODE_SUMMARY : MODE_OUT>::NT))
prefill_block_kernel(PrefillDev p)
{
    using C = BlockCfg<DT, DK, DV, SUMMARY ? MODE_SUMMARY : MODE_OUT>;
    using O = Op<DT>;
    using OT = typename O::T;
    using Frag = typename O::Frag;
    using Frag4 = typename O::Frag4;
    using ST = typename DT::storage;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const OT* sKG = reinterpret_cast<const OT*>(smem + C::O_KG);
    const OT* sV = reinterpret_cast<const OT*>(smem + C::O_V);
    const OT* sA = reinterpret_cast<const OT*>(smem + C::O_A);
    OT* sP = reinterpret_cast<OT*>(smem + C::O_P);
    const OT* sD = reinterpret_cast<const OT*>(smem + C::O_D);
    const float* sVec = reinterpret_cast<const float*>(smem + C::O_VEC);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;
    PhaseClock pclk;
#ifdef KDA_PHASE_TIMING
    pclk.on = tid == KDA_PHASE_TID;
    pclk.last = clock64();
#endif

    // ---- work item
    const int H = p.H;
    const int item = blockIdx.x / H;
    const int h = blockIdx.x % H;
    auto off = [&](int i) { return SUMMARY ? tab_p1(p, i) : tab_seg(p, i); };
    if (item >= off(p.N)) return;
    const int n = p.single ? 0 : find_seq(p.tab + (SUMMARY ? 2 : 1) * (p.N + 1), p.N, item);
    const int s = item - off(n);
    const int seg0 = tab_seg(p, n);
    const int nseg = tab_seg(p, n + 1) - seg0;
    // after a warm-up pass only the chains it flagged run again
    if (p.flags && !chain_flagged(p, seg0, nseg, h)) return;
    const int64_t seq0 = tab_cu(p, n), seq1 = tab_cu(p, n + 1);
    const int64_t t_begin = seq0 + int64_t(s) * p.L * CH;
    int64_t t_end = t_begin + int64_t(p.L) * CH;
    if (t_end > seq1) t_end = seq1;
    const bool last_seg = (s == nseg - 1);
    const int64_t nblk = (t_end - t_begin + BC - 1) / BC;
    KDA_CHECK(n >= 0 && n < p.N, CK_SEQ);
    KDA_CHECK(seq0 >= 0 && seq0 <= t_begin && t_begin <= t_end && t_end <= seq1 && seq1 <= p.T_total, CK_TOKENS);
    KDA_CHECK(SUMMARY ? item < p.np1_cap : seg0 + s < p.nseg_cap, CK_WS);
    ST* go = static_cast<ST*>(p.o);
    // first checkpoint slot of this sequence, read before the block loop (a
    // table read inside it would wait for every store in flight)
    const int64_t ck_first = (!SUMMARY && p.ckpt) ? int64_t(tab_ck(p, n)) : 0;

    // strictly-upper 16x16 block of P: read by the P U product, never written
    if (!SUMMARY)
        for (int e = tid; e < BC * BC; e += C::NT) {
            const int r = e / BC, c = e % BC;
            if ((c >> 4) > (r >> 4)) sP[r * C::ST + pcol(c)] = O::to_op(0.f);
        }
    auto blen = [&](int64_t bi) {
        const int64_t b0 = t_begin + bi * BC;
        return int(t_end - b0 < BC ? t_end - b0 : BC);
    };

    // The two roles run separate loops with the same barrier sequence (one
    // after the prologue, two per block), so their registers never overlap.
    if (wave >= C::NCW) {
        prep_role<C, DT>(p, smem, t_begin, t_end, nblk, h, tid, wave, lane, -1, pclk);
        pclk.save(SUMMARY ? 8192 : 0);
        return;
    }

    // ================= chain waves: CW columns of the extended state each, in registers
    constexpr int RT = DK / 16;  // state row tiles
    constexpr int NCT = C::NCT;
    const int colbase = C::CW * wave;
    const bool mcols = SUMMARY && colbase >= DV;
    f32x4 S[RT][NCT];
    {
        const float* src = nullptr;
        if (!SUMMARY && s == 0 && p.init)
            src = p.init_snap ? p.sin + (int64_t(seg0) * H + h) * DK * DV : p.init + (int64_t(n) * H + h) * DK * DV;
        if (!SUMMARY && s > 0) {
            // S_in from the scan, in accumulator tiles
            const float* tin = p.sin + (int64_t(seg0 + s) * H + h) * DK * DV;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    S[rt][ct] = *reinterpret_cast<const f32x4*>(tin + acc_tile_off<DV>(rt, colbase / 16 + ct, lane));
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int row = rt * 16 + 4 * q4 + j;
                        const int col = colbase + ct * 16 + l16;
                        float x = 0.f;
                        if (mcols) x = (row == col - DV) ? 1.f : 0.f;
                        else if (src) x = src[row * DV + col];
                        S[rt][ct][j] = x;
                    }
        }
    }
    __syncthreads();
    KDA_PHASE(4);
    for (int64_t bi = 0; bi < nblk; ++bi) {
        const int64_t b0 = t_begin + bi * BC;
        const int len = blen(bi);
        const int buf = int(bi & 1);
        // ---- alpha: X = V - (K . e^G) S, rows = the block's 32 tokens
        f32x4 Xt[2][NCT];
        {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Xt[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!mcols) {
                // V I with exact identity fragments picking column (ct%2)*16 + l16 of
                // the 32-column block ct/2
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = (kperm(q4, e) == (ct % 2) * 16 + l16) ? 1.f : 0.f;
                    const Frag iden = O::make(x);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
                        O::mma(Xt[rt][ct], O::load(sV + (rt * 16 + l16) * C::SV + colbase + 32 * (ct / 2) + 8 * q4),
                               iden);
                }
            }
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                const Frag a0 = O::load(sKG + l16 * C::SK + kb * 32 + 8 * q4);
                const Frag a1 = O::load(sKG + (16 + l16) * C::SK + kb * 32 + 8 * q4);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const Frag sb = acc_frag<DT>(S[2 * kb][ct], S[2 * kb + 1][ct]);
                    O::mma(Xt[0][ct], a0, sb);
                    O::mma(Xt[1][ct], a1, sb);
                }
            }
        }
        KDA_PHASE(0);
        __syncthreads();
        KDA_PHASE(1);
        // ---- beta: U = (I + A)^{-1} Diag(beta) X by block substitution, the
        // right-hand sides in two bf16 parts (sub_mma):
        //   U_0 = D_0 beta_0 X_0,  U_1 = D_1 (beta_1 X_1 - A_10 U_0)
        const float* sBb = reinterpret_cast<const float*>(smem + C::O_B) + buf * BC;
        f32x4 U0[NCT], U1[NCT];
        {
            const f32x4 bv0 = *reinterpret_cast<const f32x4*>(sBb + 4 * q4);
            const f32x4 bv1 = *reinterpret_cast<const f32x4*>(sBb + 16 + 4 * q4);
            const Frag4 d0 = O::load4(sD + l16 * C::SD + 4 * q4);
            const Frag4 d1 = O::load4(sD + (16 + l16) * C::SD + 4 * q4);
            const Frag4 a10 = O::load4(sA + (16 + l16) * C::ST + 4 * q4);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                U0[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                sub_mma<O>(U0[ct], d0, bv0 * Xt[0][ct]);
                f32x4 R = bv1 * Xt[1][ct];
                sub_mma<O>(R, a10, U0[ct]);
                U1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                sub_mma<O>(U1[ct], d1, R);
            }
        }
        Frag Ub[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Ub[ct] = acc_frag<DT>(U0[ct], U1[ct]);
        KDA_PHASE(5);
        if (!SUMMARY) {
            // O^T = S^T (Q . e^G)^T + U^T P^T: each lane ends up with four
            // consecutive value columns of one token
            const OT* sQG = reinterpret_cast<const OT*>(smem + C::O_QG + buf * C::TILE_K);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4 Ot[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Ot[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const Frag bf = O::load(sQG + (rt * 16 + l16) * C::SK + kb * 32 + 8 * q4);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        O::mma(Ot[ct], acc_frag<DT>(S[2 * kb][ct], S[2 * kb + 1][ct]), bf);
                }
                const Frag pf = O::load(sP + (rt * 16 + l16) * C::ST + 8 * q4);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) O::mma(Ot[ct], Ub[ct], pf);
                const int row = rt * 16 + l16;
                if (row < len) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        store4<DT>(go + ((b0 + row) * H + h) * DV + colbase + ct * 16 + 4 * q4, Ot[ct]);
                }
            }
        }
        KDA_PHASE(6);
        // S <- Diag(e^{G_last}) S + (K . e^{G_last - G})^T U
        const OT* sKH = reinterpret_cast<const OT*>(smem + C::O_KH + buf * C::TILE_H);
        const float* gcv = sVec + (V_GC + buf) * DK;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 gc = *reinterpret_cast<const f32x4*>(gcv + pcol(rt * 16 + 4 * q4));
            const Frag kf = O::load(sKH + (rt * 16 + l16) * C::ST + 8 * q4);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                S[rt][ct] *= gc;
                O::mma(S[rt][ct], kf, Ub[ct]);
            }
        }
        // state checkpoint when this block ends on a multiple of the interval
        // (intervals are multiples of 64, so checkpoints fall on block ends)
        if (!SUMMARY && p.ckpt) {
            const int64_t pos = b0 + len - seq0;  // tokens of the sequence consumed
            if (pos % p.ckpt_interval == 0) {
                const int64_t idx = ck_first + pos / p.ckpt_interval - 1;
                if (idx < p.ckpt_cap) {
                    // one lane pointer, formed here: hoisted out of the block
                    // loop, the 64 element addresses would live in (spilled)
                    // registers for the whole segment
                    uint32_t eo = uint32_t(4 * q4 * DV + colbase + l16);
                    asm volatile("" : "+v"(eo));
                    float* dst = p.ckpt + (idx * H + h) * DK * DV + eo;
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                __builtin_nontemporal_store(S[rt][ct][j], dst + (rt * 16 + j) * DV + ct * 16);
                }
            }
        }
        KDA_PHASE(2);
        __syncthreads();
        KDA_PHASE(3);
    }

    pclk.save(SUMMARY ? 8192 : 0);
    // ---- write the segment result.  Summary pass: S~ in fp32 accumulator tiles,
    // then M as two bf16 tiles (hi = bf16(M), lo = bf16(M - hi)) [d_k][d_k] with
    // the permuted column order of the operand tiles, ready as A operands of the
    // scan's split-precision products.
    if (SUMMARY) {
        float* base = p.ms + (int64_t(item) * H + h) * DK * (DK + DV);
        if (!mcols) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    *reinterpret_cast<f32x4*>(base + acc_tile_off<DV>(rt, colbase / 16 + ct, lane)) = S[rt][ct];
        } else {
            // every other wave is past its last LDS access (final barrier above)
            uint16_t* mhi = reinterpret_cast<uint16_t*>(base + DK * DV);
            uint16_t* mlo = mhi + DK * DK;
#pragma unroll
            for (int cb = 0; cb < NCT / 2; ++cb) {
                const int mw = (colbase - DV) / 32 + cb;  // a 32-column block of M
                float* stg = reinterpret_cast<float*>(smem) + mw * DK * C::MSTAGE;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            stg[(rt * 16 + 4 * q4 + j) * C::MSTAGE + ct * 16 + l16] = S[rt][2 * cb + ct][j];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                for (int r = lane; r < DK; r += 64) {
                    float x[32];
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const f32x4 w = *reinterpret_cast<const f32x4*>(stg + r * C::MSTAGE + 4 * m);
                        x[4 * m] = w[0];
                        x[4 * m + 1] = w[1];
                        x[4 * m + 2] = w[2];
                        x[4 * m + 3] = w[3];
                    }
                    // position p of the block holds column 16*((p>>2)&1) + 4*(p>>3) + (p&3)
                    u32x4 hv[4], lv[4];
#pragma unroll
                    for (int pp = 0; pp < 32; pp += 2) {
                        const int c0 = 16 * ((pp >> 2) & 1) + 4 * (pp >> 3) + (pp & 3);
                        const uint32_t hw = pack_bf16x2(x[c0], x[c0 + 1]);
                        hv[pp / 8][(pp / 2) % 4] = hw;
                        lv[pp / 8][(pp / 2) % 4] = pack_bf16x2(x[c0] - bf16_lo(hw), x[c0 + 1] - bf16_hi(hw));
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        *reinterpret_cast<u32x4*>(mhi + r * DK + mw * 32 + 8 * m) = hv[m];
                        *reinterpret_cast<u32x4*>(mlo + r * DK + mw * 32 + 8 * m) = lv[m];
                    }
                }
            }
        }
    } else if (last_seg && p.fin) {
        float* dst = p.fin + (int64_t(n) * H + h) * DK * DV;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    dst[(rt * 16 + 4 * q4 + j) * DV + colbase + ct * 16 + l16] = S[rt][ct][j];
    }
}

// ------------------------------------------------------------- scan kernel
// Per (sequence, head, 16-column slice of the state):
//     S_in(s+1) = M_s S_in(s) + S~_s
// over the sequence's segments, on the matrix cores with fp32-level accuracy:
// each fp32 operand x is split as hi = bf16(x), lo = bf16(x - hi) and the
// product accumulates hi*hi + hi*lo + lo*hi in fp32.  The summary pass stores
// M_s already split (hi and lo bf16 tiles, permuted columns) and S~_s in
// accumulator tiles.  Wave w owns state row tiles w, w+4, ...: it needs only
// those rows of M_s, so it loads their fragments straight from global memory
// into registers, two steps ahead.  The S_in slice, which every wave reads
// whole, sits in LDS transposed and split the same way, written once by the
// wave that computed it.
// The steps are bound by how fast one compute unit streams M_s in (all of it
// per workgroup and step; about 40 GB/s per unit here), not by the products:
// 16-column slices spread the sequence-head pairs over twice as many units as
// 32-column ones, at the price of reading M_s eight times instead of four.
constexpr int SCAN_COLS = 16;
template <int DK, int DV>
struct ScanCfg {
    static constexpr int SB = DK + 8;              // bf16 row stride of the S_in^T tiles in LDS
    static constexpr int RTW = (DK / 16 + 3) / 4;  // row tiles per wave
    static constexpr int LDS = 2 * SCAN_COLS * SB * 2;
};

// four consecutive fp32 values -> bf16 hi and lo parts (8 bytes each)
__device__ __forceinline__ void split4(const f32x4& x, u32x2& hi, u32x2& lo)
{
    hi = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    lo = u32x2{pack_bf16x2(x[0] - bf16_lo(hi[0]), x[1] - bf16_hi(hi[0])),
               pack_bf16x2(x[2] - bf16_lo(hi[1]), x[3] - bf16_hi(hi[1]))};
}

template <int DK, int DV>
__global__ void __launch_bounds__(256) scan_kernel(PrefillDev p)
{
    using SC = ScanCfg<DK, DV>;
    constexpr int NB = DV / SCAN_COLS;
    constexpr int SCT = SCAN_COLS / 16;  // 16-wide column tiles of the slice
    constexpr bool ALL_ROWS = (DK / 16) % 4 == 0;  // every wave owns RTW row tiles
    constexpr int KB = DK / 32;
    constexpr int RTW = SC::RTW;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t* sTh = reinterpret_cast<uint16_t*>(smem);  // [32][SB]: S_in slice^T, hi part, permuted rows
    uint16_t* sTl = sTh + SCAN_COLS * SC::SB;           // lo part
    const int H = p.H;
    // Workgroups go to the 8 XCDs round-robin by index; the NB column slices of
    // one (sequence, head) read the same M_s, so they are given indices that
    // share an XCD (and its L2): slices of unit u sit at u%8 + 8*(NB*(u/8) + jb).
    const int nunits = p.N * H;
    const int bx = blockIdx.x;
    int unit, jb;
    if ((nunits & 7) == 0) {
        jb = (bx >> 3) % NB;
        unit = (bx & 7) + 8 * ((bx >> 3) / NB);
    } else {
        jb = bx % NB;
        unit = bx / NB;
    }
    const int h = unit % H;
    const int n = unit / H;
    const int nseg = tab_seg(p, n + 1) - tab_seg(p, n);
    if (nseg <= 1) return;
    if (p.flags && !chain_flagged(p, tab_seg(p, n), nseg, h)) return;  // after a warm-up pass: flagged chains only
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int col0 = jb * SCAN_COLS;
    PhaseClock pclk;
#ifdef KDA_PHASE_TIMING
    pclk.on = tid == 0;
    pclk.last = clock64();
#endif
    // Table entries are read once, into registers: a re-read after the state
    // stores below would wait for every load in flight, the prefetch included.
    KDA_CHECK(tab_p1(p, n) + nseg - 1 <= p.np1_cap && tab_seg(p, n) + nseg <= p.nseg_cap, CK_WS);
    const float* const ms0 = p.ms + (int64_t(tab_p1(p, n)) * H + h) * DK * (DK + DV);
    float* const sin0 = p.sin + (int64_t(tab_seg(p, n)) * H + h) * DK * DV;
    auto ms_of = [&](int st) { return ms0 + int64_t(st) * H * DK * (DK + DV); };

    // S_in(0) slice: column j of the slice is row j of the tiles; state row k sits at pcol(k)
    for (int e = tid; e < SCAN_COLS * DK / 4; e += 256) {
        const int j = e / (DK / 4), k = (e % (DK / 4)) * 4;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (p.init) {
            const float* src = (p.init_snap ? sin0 : p.init + (int64_t(n) * H + h) * DK * DV) + col0 + j;
#pragma unroll
            for (int m = 0; m < 4; ++m) x[m] = src[(k + m) * DV];
        }
        u32x2 hi, lo;
        split4(x, hi, lo);
        *reinterpret_cast<u32x2*>(sTh + j * SC::SB + pcol(k)) = hi;
        *reinterpret_cast<u32x2*>(sTl + j * SC::SB + pcol(k)) = lo;
    }
    // this wave's rows of M_st (A operands: hi and lo fragments) and of S~_st
    // (accumulator layout), in two register sets: set st & 1 is loaded two
    // steps before it is used, so the loads have two steps to land.
    bf16x8 mh[2][RTW][KB], ml[2][RTW][KB];
    f32x4 stl[2][RTW][SCT];
    auto load_step = [&](const int set, int st) {
        const float* base = ms_of(st);
        const uint16_t* mhi = reinterpret_cast<const uint16_t*>(base + DK * DV);
        const uint16_t* mlo = mhi + DK * DK;
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + 4 * i;
            if (ALL_ROWS || rt < DK / 16) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    mh[set][i][kb] = Op<BF16>::load(mhi + (rt * 16 + l16) * DK + kb * 32 + 8 * q4);
                    ml[set][i][kb] = Op<BF16>::load(mlo + (rt * 16 + l16) * DK + kb * 32 + 8 * q4);
                }
#pragma unroll
                for (int ct = 0; ct < SCT; ++ct)
                    stl[set][i][ct] = *reinterpret_cast<const f32x4*>(base + acc_tile_off<DV>(rt, col0 / 16 + ct, lane));
            }
        }
    };
    const int nsteps = nseg - 1;
    // S_in(s + 1) = M_s S_in(s) + S~_s from register set `set`, which is then
    // refilled with step s + 2
    auto run_step = [&](const int set, int s) {
        f32x4 acc[RTW][SCT];
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct) acc[i][ct] = stl[set][i][ct];
        KDA_PHASE(1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            bf16x8 bh[SCT], bl[SCT];
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct) {
                bh[ct] = Op<BF16>::load(sTh + (ct * 16 + l16) * SC::SB + kb * 32 + 8 * q4);
                bl[ct] = Op<BF16>::load(sTl + (ct * 16 + l16) * SC::SB + kb * 32 + 8 * q4);
            }
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                if (ALL_ROWS || wave + 4 * i < DK / 16) {
#pragma unroll
                    for (int ct = 0; ct < SCT; ++ct) {
                        Op<BF16>::mma(acc[i][ct], mh[set][i][kb], bh[ct]);
                        Op<BF16>::mma(acc[i][ct], mh[set][i][kb], bl[ct]);
                        Op<BF16>::mma(acc[i][ct], ml[set][i][kb], bh[ct]);
                    }
                }
            }
        }
        // unconditional (the last steps re-read step nsteps - 1), so the two
        // register sets never merge with their old values at the loop head
        load_step(set, s + 2 < nsteps ? s + 2 : nsteps - 1);
        KDA_PHASE(2);
        __syncthreads();  // every wave is done reading the S_in tiles
        KDA_PHASE(3);
        float* out = sin0 + int64_t(s + 1) * H * DK * DV;
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + 4 * i;
            if (ALL_ROWS || rt < DK / 16) {
#pragma unroll
                for (int ct = 0; ct < SCT; ++ct) {
                    const int j = ct * 16 + l16;
                    u32x2 hi, lo;
                    split4(acc[i][ct], hi, lo);  // state rows rt*16 + 4q .. +3: contiguous under pcol
                    *reinterpret_cast<u32x2*>(sTh + j * SC::SB + pcol(rt * 16 + 4 * q4)) = hi;
                    *reinterpret_cast<u32x2*>(sTl + j * SC::SB + pcol(rt * 16 + 4 * q4)) = lo;
                    *reinterpret_cast<f32x4*>(out + acc_tile_off<DV>(rt, col0 / 16 + ct, lane)) = acc[i][ct];
                }
            }
        }
        __syncthreads();  // the new S_in slice is complete
        KDA_PHASE(4);
    };
    load_step(0, 0);
    load_step(1, nsteps > 1 ? 1 : 0);
    __syncthreads();
    KDA_PHASE(0);
    for (int s = 0; s < nsteps; s += 2) {
        run_step(0, s);
        if (s + 1 < nsteps) run_step(1, s + 1);
    }
    pclk.save(12288);
}

// ------------------------------------------------------- warm-up kernel
// One workgroup per (segment, head), as the output pass, but segment s > 0
// first runs the `warm` tokens before it (the plan above): chain wave w owns
// state columns 16w..16w+15 and, during the warm-up, columns 16w..16w+15 of
// the window's transition M as a second tile (M's columns start at I and see
// no v, so X = -(K.e^G) M for them).  A wave whose M tile has become exactly
// zero stops updating it (a zero tile stays zero).  After the window each
// wave writes whether its M tile is still non-zero; the next barrier makes the
// decision uniform: on zero the state is the warm-up's S~ and the segment runs
// on, else the workgroup flags its (segment, head) and ends, and the exact
// passes redo that chain.  A window that reaches the sequence start runs from
// the initial state and needs no check.  Warm-up blocks write no outputs and
// no checkpoints: those tokens belong to the previous segment.
template <typename DT, int DK, int DV>
__global__ void __launch_bounds__((BlockCfg<DT, DK, DV, MODE_WARM>::NT))
prefill_warm_kernel(PrefillDev p)
{
    using C = BlockCfg<DT, DK, DV, MODE_WARM>;
    using O = Op<DT>;
    using OT = typename O::T;
    using Frag = typename O::Frag;
    using Frag4 = typename O::Frag4;
    using ST = typename DT::storage;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const OT* sKG = reinterpret_cast<const OT*>(smem + C::O_KG);
    const OT* sV = reinterpret_cast<const OT*>(smem + C::O_V);
    const OT* sA = reinterpret_cast<const OT*>(smem + C::O_A);
    OT* sP = reinterpret_cast<OT*>(smem + C::O_P);
    const OT* sD = reinterpret_cast<const OT*>(smem + C::O_D);
    const float* sVec = reinterpret_cast<const float*>(smem + C::O_VEC);
    int32_t* sFlag = reinterpret_cast<int32_t*>(smem + C::O_FLAG);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;
    PhaseClock pclk;
#ifdef KDA_PHASE_TIMING
    pclk.on = tid == KDA_PHASE_TID;
    pclk.last = clock64();
#endif

    // ---- work item.  Packed sequences: every non-final segment first (all
    // of full length, in sequence order), then the sequences' final segments
    // longest first (the plan kernel's order), so long items start early.
    const int H = p.H;
    const int rank = blockIdx.x / H;
    const int h = blockIdx.x % H;
    if (rank >= tab_seg(p, p.N)) return;
    int n, s;
    if (p.single) {
        n = 0;
        s = rank;
    } else {
        const int np1 = tab_p1(p, p.N);
        if (rank < np1) {
            n = find_seq(p.tab + 2 * (p.N + 1), p.N, rank);
            s = rank - tab_p1(p, n);
        } else {
            n = p.tab[4 * (p.N + 1) + (rank - np1)];
            s = tab_seg(p, n + 1) - tab_seg(p, n) - 1;
        }
    }
    const int seg0 = tab_seg(p, n);
    const int item = seg0 + s;  // the segment's index in sequence order (its flag)
    const int nseg = tab_seg(p, n + 1) - seg0;
    const int64_t seq0 = tab_cu(p, n), seq1 = tab_cu(p, n + 1);
    const int64_t t_begin = seq0 + int64_t(s) * p.L * CH;
    int64_t t_end = t_begin + int64_t(p.L) * CH;
    if (t_end > seq1) t_end = seq1;
    const bool last_seg = (s == nseg - 1);
    // the warm-up window [ws, t_begin): whole 32-token blocks (segments start
    // on chunk boundaries and the window is a multiple of 32 tokens)
    int64_t ws = t_begin;
    if (s > 0) ws = t_begin - p.warm > seq0 ? t_begin - p.warm : seq0;
    const bool from_zero = ws > seq0;  // else the window starts at the sequence start
    const int64_t nwarm = (t_begin - ws) / BC;
    const int64_t nblk = nwarm + (t_end - t_begin + BC - 1) / BC;
    KDA_CHECK(n >= 0 && n < p.N, CK_SEQ);
    KDA_CHECK(seq0 >= 0 && seq0 <= ws && ws <= t_begin && t_begin <= t_end && t_end <= seq1 &&
                  seq1 <= p.T_total, CK_TOKENS);
    KDA_CHECK(item >= 0 && item < p.nseg_cap, CK_WS);
    ST* go = static_cast<ST*>(p.o);
    const int64_t ck_first = p.ckpt ? int64_t(tab_ck(p, n)) : 0;
    int32_t* gflag = p.flags + int64_t(item) * H + h;
    if (tid == 0) *gflag = 0;

    // strictly-upper 16x16 block of P: read by the P U product, never written
    for (int e = tid; e < BC * BC; e += C::NT) {
        const int r = e / BC, c = e % BC;
        if ((c >> 4) > (r >> 4)) sP[r * C::ST + pcol(c)] = O::to_op(0.f);
    }
    auto blen = [&](int64_t bi) {
        const int64_t b0 = ws + bi * BC;
        return int(t_end - b0 < BC ? t_end - b0 : BC);
    };

    if (wave >= C::NCW) {
        prep_role<C, DT>(p, smem, ws, t_end, nblk, h, tid, wave, lane, from_zero ? nwarm - 1 : -1, pclk);
        pclk.save(0);
        return;
    }

    // ================= chain waves
    constexpr int RT = DK / 16;  // state row tiles
    const int colbase = 16 * wave;
    const bool hasM = from_zero && colbase < DK;
    f32x4 S[RT][2];  // [.][0]: state columns colbase.., [.][1]: M columns colbase.. (warm-up only)
    {
        const float* src = (!from_zero && p.init) ? p.init + (int64_t(n) * H + h) * DK * DV : nullptr;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = rt * 16 + 4 * q4 + j;
                const int col = colbase + l16;
                S[rt][0][j] = src ? src[row * DV + col] : 0.f;
                S[rt][1][j] = (hasM && row == col) ? 1.f : 0.f;
            }
        if (p.init_snap && s == 0) {
            float* snap = p.sin + (int64_t(seg0) * H + h) * DK * DV;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) snap[(rt * 16 + 4 * q4 + j) * DV + colbase + l16] = S[rt][0][j];
        }
    }
    bool mlive = hasM;  // wave-uniform: the M tile is still non-zero
    __syncthreads();
    KDA_PHASE(4);

    // one block: EXT carries the M tile beside the state, EMIT writes outputs
    // and checkpoints
    auto step = [&](const int64_t bi, auto ext_t, auto emit_t) {
        constexpr bool EXT = decltype(ext_t)::value;
        constexpr bool EMIT = decltype(emit_t)::value;
        const int64_t b0 = ws + bi * BC;
        const int len = blen(bi);
        const int buf = int(bi & 1);
        const bool act1 = EXT && mlive;
        // ---- alpha: X = V - (K . e^G) S;  X_M = -(K . e^G) M
        f32x4 Xt[2][2];
        {
            // v in the accumulator layout: lane (l16, q4) takes column
            // 16 (wave & 1) + l16 of block wave / 2 (its permuted position in
            // the tile) of rows 4 q4 .. 4 q4 + 3 of each sub-tile
            const OT* vc = sV + 32 * (wave >> 1) + 8 * (l16 >> 2) + 4 * (wave & 1) + (l16 & 3);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
                for (int j = 0; j < 4; ++j) Xt[rt][0][j] = O::from_op(vc[(rt * 16 + 4 * q4 + j) * C::SV]);
                Xt[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            const Frag a0 = O::load(sKG + l16 * C::SK + kb * 32 + 8 * q4);
            const Frag a1 = O::load(sKG + (16 + l16) * C::SK + kb * 32 + 8 * q4);
            const Frag sb = acc_frag<DT>(S[2 * kb][0], S[2 * kb + 1][0]);
            O::mma(Xt[0][0], a0, sb);
            O::mma(Xt[1][0], a1, sb);
            if (act1) {
                const Frag sm = acc_frag<DT>(S[2 * kb][1], S[2 * kb + 1][1]);
                O::mma(Xt[0][1], a0, sm);
                O::mma(Xt[1][1], a1, sm);
            }
        }
        KDA_PHASE(0);
        __syncthreads();
        KDA_PHASE(1);
        // ---- beta: U = (I + A)^{-1} Diag(beta) X by block substitution
        const float* sBb = reinterpret_cast<const float*>(smem + C::O_B) + buf * BC;
        f32x4 U0[2], U1[2];
        Frag Ub[2];
        {
            const f32x4 bv0 = *reinterpret_cast<const f32x4*>(sBb + 4 * q4);
            const f32x4 bv1 = *reinterpret_cast<const f32x4*>(sBb + 16 + 4 * q4);
            const Frag4 d0 = O::load4(sD + l16 * C::SD + 4 * q4);
            const Frag4 d1 = O::load4(sD + (16 + l16) * C::SD + 4 * q4);
            const Frag4 a10 = O::load4(sA + (16 + l16) * C::ST + 4 * q4);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                if (ct == 1 && !act1) break;
                U0[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                sub_mma<O>(U0[ct], d0, bv0 * Xt[0][ct]);
                f32x4 R = bv1 * Xt[1][ct];
                sub_mma<O>(R, a10, U0[ct]);
                U1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                sub_mma<O>(U1[ct], d1, R);
                Ub[ct] = acc_frag<DT>(U0[ct], U1[ct]);
            }
        }
        KDA_PHASE(5);
        if constexpr (EMIT) {
            // O^T = S^T (Q . e^G)^T + U^T P^T: four consecutive value columns per lane
            const OT* sQG = reinterpret_cast<const OT*>(smem + C::O_QG + buf * C::TILE_K);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4 Ot = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const Frag bf = O::load(sQG + (rt * 16 + l16) * C::SK + kb * 32 + 8 * q4);
                    O::mma(Ot, acc_frag<DT>(S[2 * kb][0], S[2 * kb + 1][0]), bf);
                }
                const Frag pf = O::load(sP + (rt * 16 + l16) * C::ST + 8 * q4);
                O::mma(Ot, Ub[0], pf);
                const int row = rt * 16 + l16;
                if (row < len) store4<DT>(go + ((b0 + row) * H + h) * DV + colbase + 4 * q4, Ot);
            }
        }
        KDA_PHASE(6);
        // S <- Diag(e^{G_last}) S + (K . e^{G_last - G})^T U
        const OT* sKH = reinterpret_cast<const OT*>(smem + C::O_KH + buf * C::TILE_H);
        const float* gcv = sVec + (V_GC + buf) * DK;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 gc = *reinterpret_cast<const f32x4*>(gcv + pcol(rt * 16 + 4 * q4));
            const Frag kf = O::load(sKH + (rt * 16 + l16) * C::ST + 8 * q4);
            S[rt][0] *= gc;
            O::mma(S[rt][0], kf, Ub[0]);
            if (act1) {
                S[rt][1] *= gc;
                O::mma(S[rt][1], kf, Ub[1]);
            }
        }
        if constexpr (EMIT) {
            // state checkpoint when this block ends on a multiple of the interval
            if (p.ckpt) {
                const int64_t pos = b0 + len - seq0;  // tokens of the sequence consumed
                if (pos % p.ckpt_interval == 0) {
                    const int64_t idx = ck_first + pos / p.ckpt_interval - 1;
                    if (idx < p.ckpt_cap) {
                        // one lane pointer, formed here (see the output pass)
                        uint32_t eo = uint32_t(4 * q4 * DV + colbase + l16);
                        asm volatile("" : "+v"(eo));
                        float* dst = p.ckpt + (idx * H + h) * DK * DV + eo;
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                __builtin_nontemporal_store(S[rt][0][j], dst + (rt * 16 + j) * DV);
                    }
                }
            }
        }
        if constexpr (EXT) {
            if (act1) {
                bool nz = false;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) nz = nz || (S[rt][1][j] != 0.f);
                mlive = __ballot(nz) != 0;
            }
            if (bi == nwarm - 1 && lane == 0) sFlag[wave] = mlive ? 1 : 0;
        }
        KDA_PHASE(2);
        __syncthreads();
        KDA_PHASE(3);
    };

    int64_t bi = 0;
    if (from_zero) {
        for (; bi < nwarm; ++bi) step(bi, std::true_type{}, std::false_type{});
        if (warm_failed<C>(smem)) {  // the incoming state still matters: the exact passes take over
            if (tid == 0) *gflag = 1;
            return;
        }
    } else {
        for (; bi < nwarm; ++bi) step(bi, std::false_type{}, std::false_type{});
    }
    for (; bi < nblk; ++bi) step(bi, std::false_type{}, std::true_type{});
    pclk.save(0);

    if (last_seg && p.fin) {
        // one lane offset, formed here: formed before the block loop, the
        // compiler keeps the element addresses live across it
        uint32_t eo = uint32_t(4 * q4 * DV + colbase + l16);
        asm volatile("" : "+v"(eo));
        float* dst = p.fin + (int64_t(n) * H + h) * DK * DV + eo;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[(rt * 16 + j) * DV] = S[rt][0][j];
    }
}

// ------------------------------------------------------------------ launch
template <typename DT, int DK, int DV>
hipError_t launch_prefill_t(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t stream)
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
    const bool warm = plan.warm > 0 && warm_shape(DK, DV);
    PrefillDev d{a.q, a.k, a.v, a.g, a.beta, tab, a.N, a.T_total, a.H, plan.seg_chunks,
                 a.init, a.fin, a.o,
                 plan.np1_max > 0 ? reinterpret_cast<float*>(ws + plan.off_ms) : nullptr,
                 plan.np1_max > 0 ? reinterpret_cast<float*>(ws + plan.off_sin) : nullptr,
                 a.ckpt, a.ckpt_interval, a.ckpt_cap, single ? 1 : 0, single_nseg, single_nck,
                 a.gate_A, a.g_min,
                 warm ? reinterpret_cast<int32_t*>(ws + plan.off_flags) : nullptr, plan.warm,
                 plan.nseg_max, plan.np1_max};
    d.init_snap = (a.init_snap && warm && plan.np1_max > 0) ? 1 : 0;
    hipError_t e = hipSuccess;
    if (!single) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, a.cu, a.N, a.T_total,
                           plan.seg_chunks, a.ckpt ? a.ckpt_interval : 0, tab);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if constexpr (warm_shape(DK, DV)) {
        if (warm) {
            using CW_ = BlockCfg<DT, DK, DV, MODE_WARM>;
            auto kw = prefill_warm_kernel<DT, DK, DV>;
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(kw), hipFuncAttributeMaxDynamicSharedMemorySize,
                                    CW_::LDS);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(kw, dim3(unsigned(plan.nseg_max * a.H)), dim3(CW_::NT), CW_::LDS, stream, d);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            // every sequence is one segment: no warm-up can fail
            if (plan.np1_max == 0) return hipSuccess;
        }
    }
    // the exact passes (after a warm-up pass: only for the chains it flagged)
    if (plan.np1_max > 0) {
        using C1 = BlockCfg<DT, DK, DV, MODE_SUMMARY>;
        auto k1 = prefill_block_kernel<DT, DK, DV, true>;
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
    using C3 = BlockCfg<DT, DK, DV, MODE_OUT>;
    auto k3 = prefill_block_kernel<DT, DK, DV, false>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k3),
                            hipFuncAttributeMaxDynamicSharedMemorySize, C3::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k3, dim3(unsigned(plan.nseg_max * a.H)), dim3(C3::NT), C3::LDS, stream, d);
    return hipGetLastError();
}

// The launches launch_prefill_t makes for this plan, as text (host only): one
// line per kernel with its grid, block and LDS bytes.  packed: cu_seqlens is
// given (the plan kernel runs first).
template <typename DT, int DK, int DV>
void describe_prefill_t(const PrefillPlan& plan, int N, int H, bool packed, std::string& out)
{
    char line[256];
    int n = 0;
    auto add = [&](const char* kernel, int64_t grid, int threads, int lds, const char* what) {
        snprintf(line, sizeof(line), "launch %d: %s grid %lld x %d threads, %d B LDS; %s\n", ++n, kernel,
                 (long long)grid, threads, lds, what);
        out += line;
    };
    if (packed) add("plan_kernel", 1, 256, 0, "segment table of the packed sequences");
    const bool warm = plan.warm > 0 && warm_shape(DK, DV);
    if constexpr (warm_shape(DK, DV)) {
        if (warm) {
            using CW_ = BlockCfg<DT, DK, DV, MODE_WARM>;
            add("prefill_warm_kernel", plan.nseg_max * H, CW_::NT, CW_::LDS,
                "every (segment, head): its incoming state from the warm-up window, outputs and final states; "
                "flags the chains where the window's transition is not zero");
            if (plan.np1_max == 0) return;
        }
    }
    if (plan.np1_max > 0) {
        using C1 = BlockCfg<DT, DK, DV, MODE_SUMMARY>;
        add("prefill_block_kernel (summary)", plan.np1_max * H, C1::NT, C1::LDS,
            warm ? "[S~ | M] of the flagged chains' non-final segments (returns at once elsewhere)"
                 : "[S~ | M] of every non-final segment");
        add("scan_kernel", int64_t(N) * H * (DV / SCAN_COLS), 256, ScanCfg<DK, DV>::LDS,
            warm ? "incoming states of the flagged chains' segments" : "incoming state of every segment");
    }
    using C3 = BlockCfg<DT, DK, DV, MODE_OUT>;
    add("prefill_block_kernel (output)", plan.nseg_max * H, C3::NT, C3::LDS,
        warm ? "outputs and final states of the flagged chains (returns at once elsewhere)"
             : "outputs and final states of every segment");
}

template <typename DT>
bool describe_prefill(const PrefillPlan& plan, int N, int H, int dk, int dv, bool packed, std::string& out)
{
#define KDA_PF(DKV, DVV)                                                                                   \
    if (dk == DKV && dv == DVV) {                                                                          \
        describe_prefill_t<DT, DKV, DVV>(plan, N, H, packed, out);                                         \
        return true;                                                                                       \
    }
    if constexpr (DT::is_bf16) {
        KDA_PF(32, 32) KDA_PF(32, 64) KDA_PF(32, 128)
        KDA_PF(64, 32) KDA_PF(64, 64) KDA_PF(64, 128)
        KDA_PF(128, 32) KDA_PF(128, 64) KDA_PF(128, 128)
    } else {
        KDA_PF(32, 32) KDA_PF(32, 64)
    }
#undef KDA_PF
    return false;
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
