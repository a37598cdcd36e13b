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
template <typename DT>
struct Op;
template <>
struct Op<BF16> {
    using T = uint16_t;  // LDS operand element
    using Frag = bf16x8;
    static __device__ __forceinline__ Frag make(const float (&x)[8])
    {
        u32x4 w;
        w[0] = pack_bf16x2(x[0], x[1]);
        w[1] = pack_bf16x2(x[2], x[3]);
        w[2] = pack_bf16x2(x[4], x[5]);
        w[3] = pack_bf16x2(x[6], x[7]);
        return __builtin_bit_cast(Frag, w);
    }
    static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b)
    {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ T to_op(float x) { return f32_to_bf16(x); }
    static __device__ __forceinline__ float from_op(T x) { return bf16_to_f32(x); }
    // 4 consecutive LDS elements -> 4 floats
    static __device__ __forceinline__ void ld4(const T* p, float* x)
    {
        const u32x2 w = *reinterpret_cast<const u32x2*>(p);
        x[0] = bf16_lo(w[0]);
        x[1] = bf16_hi(w[0]);
        x[2] = bf16_lo(w[1]);
        x[3] = bf16_hi(w[1]);
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
    static __device__ __forceinline__ Frag make(const float (&x)[8])
    {
        Frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f.v[i] = x[i];
        return f;
    }
    static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b)
    {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
    }
    static __device__ __forceinline__ T to_op(float x) { return x; }
    static __device__ __forceinline__ float from_op(T x) { return x; }
    static __device__ __forceinline__ void ld4(const T* p, float* x)
    {
        const f32x4 w = *reinterpret_cast<const f32x4*>(p);
        x[0] = w[0];
        x[1] = w[1];
        x[2] = w[2];
        x[3] = w[3];
    }
    static __device__ __forceinline__ void st4(T* p, const f32x4& v)
    {
        *reinterpret_cast<f32x4*>(p) = v;
    }
};

// K-block of 32 with the permuted index k(q, e) = 16*(e/4) + 4q + (e%4): lane
// group q supplies elements e = 0..7.  The same permutation is used for both
// operands of every product, so the sum over k is unchanged; it lets a pair of
// 16x16 accumulator tiles (rows 4q..4q+3 of each) serve directly as an operand.
__device__ __forceinline__ int kperm(int q, int e) { return ((e >> 2) << 4) + (q << 2) + (e & 3); }

// fragment of a row-major LDS tile: row `row`, K-block starting at column kc
template <typename DT>
__device__ __forceinline__ void lds_row_frag(const typename Op<DT>::T* tile, int stride, int row,
                                             int kc, int q, float (&x)[8])
{
    const typename Op<DT>::T* p = tile + row * stride + kc + 4 * q;
    Op<DT>::ld4(p, x);
    Op<DT>::ld4(p + 16, x + 4);
}

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
    static constexpr int NCW = NCOL / 32;                 // chain waves
    static constexpr int NW0 = NCW > DK / 64 ? NCW : DK / 64;
    static constexpr int NW = NW0 <= 1 ? 1 : NW0 <= 2 ? 2 : NW0 <= 4 ? 4 : 8;
    static constexpr int NT = NW * 64;
    static constexpr int PARTS = NT / DK;     // threads per key channel (elementwise phase)
    static constexpr int TPT = CH / PARTS;    // tokens per thread
    static constexpr int SL = TPT < 16 ? TPT : 16;
    static constexpr int NSLOT = CH / SL;
    using OT = typename Op<DT>::T;
    static constexpr int ES = sizeof(OT);
    static constexpr int SK = DK + 8;  // row strides (elements) of the padded tiles
    static constexpr int SV = DV + 8;
    static constexpr int ST = CH + 8;
    static constexpr int SA = CH + 4;  // fp32 solve tiles
    // LDS layout (bytes)
    static constexpr int O_Q = 0;                      // q -> QE
    static constexpr int O_K = O_Q + CH * SK * ES;     // k -> KE
    static constexpr int O_G = O_K + CH * SK * ES;     // g -> KF
    static constexpr int O_V = O_G + CH * SK * ES;     // v
    static constexpr int O_T = O_V + CH * SV * ES;     // T
    static constexpr int O_P = O_T + CH * ST * ES;     // P
    static constexpr int O_A = O_P + CH * ST * ES;     // A (fp32)
    static constexpr int O_X = O_A + CH * SA * 4;      // (I+A)^-1 (fp32)
    static constexpr int O_Y = O_X + CH * SA * 4;      // solve scratch, 3 x 16x16 fp32
    static constexpr int O_VEC = O_Y + 3 * 256 * 4;    // 16 x DK fp32 channel vectors
    static constexpr int O_SIG = O_VEC + 16 * DK * 4;  // NSLOT x DK fp32
    static constexpr int O_B = O_SIG + NSLOT * DK * 4; // beta[64]
    static constexpr int LDS = O_B + CH * 4;
    // raw tile loading: 16-byte units
    static constexpr int UPR_K = DK * ES / 16;  // units per row
    static constexpr int UPR_V = DV * ES / 16;
    static constexpr int U_K = CH * UPR_K;      // units per q/k/g tile
    static constexpr int U_V = CH * UPR_V;
    static constexpr int U_ALL = 3 * U_K + U_V;
    static constexpr int UPT = (U_ALL + NT - 1) / NT;  // units per thread
    static_assert(LDS <= 160 * 1024, "LDS budget exceeded");
    static_assert(PARTS >= 1 && CH % PARTS == 0, "bad elementwise split");
    static_assert((TPT % 16 == 0) || (16 % TPT == 0), "sub-tile alignment");
};

// channel-vector slots
enum { V_ER = 0, V_FY = 4, V_FX = 8, V_EL = 11, V_GC = 15 };

template <typename DT, int DK, int DV, bool SUMMARY>
__global__ void __launch_bounds__((ChunkCfg<DT, DK, DV, SUMMARY>::NT))
prefill_chunk_kernel(PrefillDev p)
{
    using C = ChunkCfg<DT, DK, DV, SUMMARY>;
    using O = Op<DT>;
    using OT = typename O::T;
    using Frag = typename O::Frag;
    using ST = typename DT::storage;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    OT* sQ = reinterpret_cast<OT*>(smem + C::O_Q);
    OT* sK = reinterpret_cast<OT*>(smem + C::O_K);
    OT* sG = reinterpret_cast<OT*>(smem + C::O_G);
    OT* sV = reinterpret_cast<OT*>(smem + C::O_V);
    OT* sT = reinterpret_cast<OT*>(smem + C::O_T);
    OT* sP = reinterpret_cast<OT*>(smem + C::O_P);
    float* sA = reinterpret_cast<float*>(smem + C::O_A);
    float* sX = reinterpret_cast<float*>(smem + C::O_X);
    float* sY = reinterpret_cast<float*>(smem + C::O_Y);
    float* sVec = reinterpret_cast<float*>(smem + C::O_VEC);
    float* sSig = reinterpret_cast<float*>(smem + C::O_SIG);
    float* sB = reinterpret_cast<float*>(smem + C::O_B);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;

    // ---- work item
    const int H = p.H;
    const int item = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int32_t* cuc = p.tab;
    const int32_t* seg_off = p.tab + (p.N + 1);
    const int32_t* p1_off = p.tab + 2 * (p.N + 1);
    const int32_t* off = SUMMARY ? p1_off : seg_off;
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

    // ---- chain registers: wave owns columns [32*wave, 32*wave+32) of the extended state
    constexpr int RT = DK / 16;  // state row tiles
    const bool chain = wave < C::NCW;
    const int colbase = 32 * wave;
    const bool mcols = SUMMARY && colbase >= DV;
    f32x4 S[RT][2];
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
            for (int ct = 0; ct < 2; ++ct)
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

    // zero the strictly-upper 16x16 blocks of T and P once: only lower blocks are rewritten
    for (int e = tid; e < CH * CH; e += C::NT) {
        const int r = e / CH, c = e % CH;
        if ((c >> 4) > (r >> 4)) {
            sT[r * C::ST + c] = O::to_op(0.f);
            sP[r * C::ST + c] = O::to_op(0.f);
        }
    }

    // identity fragments (exact in bf16) for X = V I
    Frag Iden[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (kperm(q4, e) == ct * 16 + l16) ? 1.f : 0.f;
        Iden[ct] = O::make(x);
    }

    // ---- raw tile prefetch (registers) and commit (LDS)
    u32x4 pre[C::UPT];
    float preb = 0.f;
    auto prefetch = [&](int64_t c0, int len) {
#pragma unroll
        for (int i = 0; i < C::UPT; ++i) {
            const int u = tid + i * C::NT;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (u < C::U_ALL) {
                const ST* base;
                int row, cu8, D;
                if (u < 3 * C::U_K) {
                    const int tsel = u / C::U_K, uu = u % C::U_K;
                    row = uu / C::UPR_K;
                    cu8 = uu % C::UPR_K;
                    base = tsel == 0 ? gq : tsel == 1 ? gk : gg;
                    D = DK;
                } else {
                    const int uu = u - 3 * C::U_K;
                    row = uu / C::UPR_V;
                    cu8 = uu % C::UPR_V;
                    base = gv;
                    D = DV;
                }
                if (row < len) {
                    const ST* ptr = base + ((c0 + row) * H + h) * D + cu8 * (16 / C::ES);
                    w = *reinterpret_cast<const u32x4*>(ptr);
                }
            }
            pre[i] = w;
        }
        preb = (tid < len) ? load_elem<DT>(gb, (c0 + tid) * H + h) : 0.f;
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < C::UPT; ++i) {
            const int u = tid + i * C::NT;
            if (u < C::U_ALL) {
                OT* dst;
                if (u < 3 * C::U_K) {
                    const int tsel = u / C::U_K, uu = u % C::U_K;
                    const int row = uu / C::UPR_K, cu8 = uu % C::UPR_K;
                    OT* t = tsel == 0 ? sQ : tsel == 1 ? sK : sG;
                    dst = t + row * C::SK + cu8 * (16 / C::ES);
                } else {
                    const int uu = u - 3 * C::U_K;
                    const int row = uu / C::UPR_V, cu8 = uu % C::UPR_V;
                    dst = sV + row * C::SV + cu8 * (16 / C::ES);
                }
                *reinterpret_cast<u32x4*>(dst) = pre[i];
            }
        }
        if (tid < CH) sB[tid] = preb;
    };

    const int64_t nchunks = (t_end - t_begin + CH - 1) / CH;
    if (nchunks > 0) prefetch(t_begin, int(t_end - t_begin < CH ? t_end - t_begin : CH));

    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t c0 = t_begin + ci * CH;
        const int len = int(t_end - c0 < CH ? t_end - c0 : CH);
        __syncthreads();  // previous chunk's operands are no longer read
        commit();
        __syncthreads();

        // ---- elementwise phase A: per-slot sums of g (per key channel)
        const int ch = tid % DK;
        const int part = tid / DK;
        const int tok0 = part * C::TPT;
        {
#pragma unroll
            for (int sl = 0; sl < C::TPT / C::SL; ++sl) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < C::SL; ++i)
                    acc += O::from_op(sG[(tok0 + sl * C::SL + i) * C::SK + ch]);
                sSig[((tok0 / C::SL) + sl) * DK + ch] = acc;
            }
        }
        __syncthreads();
        // ---- elementwise phase B: decayed operands, in place, and channel vectors
        {
            float R[5];
            R[0] = 0.f;
            float run = 0.f;
#pragma unroll
            for (int sl = 0; sl < C::NSLOT; ++sl) {
                run += sSig[sl * DK + ch];
                if (((sl + 1) * C::SL) % 16 == 0) R[((sl + 1) * C::SL) / 16] = run;
            }
            float G = 0.f;
            for (int sl = 0; sl < tok0 / C::SL; ++sl) G += sSig[sl * DK + ch];
#pragma unroll 4
            for (int i = 0; i < C::TPT; ++i) {
                const int r = tok0 + i;
                const int a = r >> 4;
                const float gr = O::from_op(sG[r * C::SK + ch]);
                G += gr;
                const float ra = a == 0 ? R[0] : a == 1 ? R[1] : a == 2 ? R[2] : R[3];
                const float e1 = __expf(G - ra);
                const float e2 = __expf(ra - G);
                const float kv = O::from_op(sK[r * C::SK + ch]);
                const float qv = O::from_op(sQ[r * C::SK + ch]);
                sQ[r * C::SK + ch] = O::to_op(qv * e1);
                sK[r * C::SK + ch] = O::to_op(kv * e1);
                sG[r * C::SK + ch] = O::to_op(kv * e2);
            }
            if (part == 0) {
                float* vv = sVec;
#pragma unroll
                for (int a = 0; a < 4; ++a) vv[(V_ER + a) * DK + ch] = __expf(R[a]);
#pragma unroll
                for (int b = 0; b < 4; ++b) vv[(V_FY + b) * DK + ch] = __expf(R[b + 1] - R[b]);
                vv[(V_FX + 0) * DK + ch] = __expf(R[2] - R[1]);  // (a,b) = (2,0)
                vv[(V_FX + 1) * DK + ch] = __expf(R[3] - R[1]);  // (3,0)
                vv[(V_FX + 2) * DK + ch] = __expf(R[3] - R[2]);  // (3,1)
#pragma unroll
                for (int b = 0; b < 4; ++b) vv[(V_EL + b) * DK + ch] = __expf(R[4] - R[b + 1]);
                vv[V_GC * DK + ch] = __expf(R[4]);
            }
        }
        __syncthreads();

        // ---- products: A (strictly lower, x beta_r, fp32) and P (lower incl. diagonal)
        for (int task = wave; task < 20; task += C::NW) {
            const bool isP = task >= 10;
            int bi = isP ? task - 10 : task;
            int a = 0;
            while (bi > a) { bi -= a + 1; ++a; }
            const int b = bi;  // 0 <= b <= a
            const OT* X = isP ? sQ : sK;
            const int fx = (a >= b + 2) ? (a == 2 ? 0 : (b == 0 ? 1 : 2)) : -1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                float y[8], x[8];
                lds_row_frag<DT>(sG, C::SK, b * 16 + l16, kb * 32, q4, y);
                lds_row_frag<DT>(X, C::SK, a * 16 + l16, kb * 32, q4, x);
                if (b < a) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] *= sVec[(V_FY + b) * DK + kb * 32 + kperm(q4, e)];
                }
                if (fx >= 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] *= sVec[(V_FX + fx) * DK + kb * 32 + kperm(q4, e)];
                }
                O::mma(acc, O::make(y), O::make(x));
            }
            // acc: lane (col r = 16a + l16, rows i = 16b + 4*q4 + j)
            const int r = a * 16 + l16;
            const int i0 = b * 16 + 4 * q4;
            if (isP) {
                f32x4 v4;
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[j] = (i0 + j <= r) ? acc[j] : 0.f;
                O::st4(sP + r * C::ST + i0, v4);
            } else {
                const float br = sB[r];
                f32x4 v4;
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[j] = (i0 + j < r) ? br * acc[j] : 0.f;
                *reinterpret_cast<f32x4*>(sA + r * C::SA + i0) = v4;
            }
        }
        __syncthreads();

        // ---- solve X = (I + A)^{-1}: diagonal 16x16 blocks by forward substitution
        if (tid < 64) {
            const int a = tid >> 4, j = tid & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == j) ? 1.f : 0.f;
                const float* arow = sA + (a * 16 + r) * C::SA + a * 16;
#pragma unroll
                for (int i = 0; i < r; ++i) acc -= arow[i] * x[i];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sX[(a * 16 + r) * C::SA + a * 16 + j] = x[r];
        }
        __syncthreads();
        // off-diagonal blocks, by distance d = a - b:  X_ab = -X_aa sum_{m=b}^{a-1} A_am X_mb
#pragma unroll
        for (int d = 1; d <= 3; ++d) {
            const int nb = 4 - d;
            for (int e = tid; e < nb * 256; e += C::NT) {
                const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
                const int a = d + blk, b = blk;
                float acc = 0.f;
                for (int m = b; m < a; ++m) {
                    const float* arow = sA + (a * 16 + rr) * C::SA + m * 16;
                    const float* xcol = sX + (m * 16) * C::SA + b * 16 + cc;
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc += arow[i] * xcol[i * C::SA];
                }
                sY[blk * 256 + rr * 16 + cc] = acc;
            }
            __syncthreads();
            for (int e = tid; e < nb * 256; e += C::NT) {
                const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
                const int a = d + blk, b = blk;
                const float* xrow = sX + (a * 16 + rr) * C::SA + a * 16;
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (i <= rr) acc += xrow[i] * sY[blk * 256 + i * 16 + cc];
                sX[(a * 16 + rr) * C::SA + b * 16 + cc] = -acc;
            }
            __syncthreads();
        }
        // T = X Diag(beta) on the lower blocks (diagonal blocks: upper part zero)
        for (int e = tid; e < CH * CH; e += C::NT) {
            const int r = e / CH, c = e % CH;
            if ((c >> 4) <= (r >> 4)) {
                const float x = (c <= r) ? sX[r * C::SA + c] * sB[c] : 0.f;
                sT[r * C::ST + c] = O::to_op(x);
            }
        }
        __syncthreads();

        // ---- prefetch the next chunk while the chain runs
        if (ci + 1 < nchunks) {
            const int64_t n0 = c0 + CH;
            prefetch(n0, int(t_end - n0 < CH ? t_end - n0 : CH));
        }

        if (chain) {
            // packed state operands (rows = key channels), reused by X and O
            Frag Sb[DK / 32][2];
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) Sb[kb][ct] = acc_frag<DT>(S[2 * kb][ct], S[2 * kb + 1][ct]);

            // X = V - (K . e^G) S       (rows = tokens, 4 row tiles x 2 col tiles)
            f32x4 Xt[4][2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) Xt[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!mcols) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    float x[8];
                    lds_row_frag<DT>(sV, C::SV, rt * 16 + l16, colbase, q4, x);
                    const Frag vf = O::make(x);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) O::mma(Xt[rt][ct], vf, Iden[ct]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    float x[8];
                    lds_row_frag<DT>(sK, C::SK, rt * 16 + l16, kb * 32, q4, x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] *= -sVec[(V_ER + rt) * DK + kb * 32 + kperm(q4, e)];
                    const Frag af = O::make(x);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) O::mma(Xt[rt][ct], af, Sb[kb][ct]);
                }

            // U = T X      (T lower triangular: row tile rt needs token blocks kbt <= rt/2)
            Frag Xb[2][2];
#pragma unroll
            for (int kbt = 0; kbt < 2; ++kbt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) Xb[kbt][ct] = acc_frag<DT>(Xt[2 * kbt][ct], Xt[2 * kbt + 1][ct]);
            f32x4 Ut[4][2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) Ut[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kbt = 0; kbt <= rt / 2; ++kbt) {
                    float x[8];
                    lds_row_frag<DT>(sT, C::ST, rt * 16 + l16, kbt * 32, q4, x);
                    const Frag tf = O::make(x);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) O::mma(Ut[rt][ct], tf, Xb[kbt][ct]);
                }
            }
            Frag Ub[2][2];
#pragma unroll
            for (int kbt = 0; kbt < 2; ++kbt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) Ub[kbt][ct] = acc_frag<DT>(Ut[2 * kbt][ct], Ut[2 * kbt + 1][ct]);

            if (!SUMMARY) {
                // O = (Q . e^G) S + P U
                ST* go = static_cast<ST*>(p.o);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f32x4 Ot[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                    for (int kb = 0; kb < DK / 32; ++kb) {
                        float x[8];
                        lds_row_frag<DT>(sQ, C::SK, rt * 16 + l16, kb * 32, q4, x);
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[e] *= sVec[(V_ER + rt) * DK + kb * 32 + kperm(q4, e)];
                        const Frag af = O::make(x);
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct) O::mma(Ot[ct], af, Sb[kb][ct]);
                    }
#pragma unroll
                    for (int kbt = 0; kbt <= rt / 2; ++kbt) {
                        float x[8];
                        lds_row_frag<DT>(sP, C::ST, rt * 16 + l16, kbt * 32, q4, x);
                        const Frag pf = O::make(x);
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct) O::mma(Ot[ct], pf, Ub[kbt][ct]);
                    }
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int row = rt * 16 + 4 * q4 + j;
                            if (row < len)
                                store_elem<DT>(go, ((c0 + row) * H + h) * DV + colbase + ct * 16 + l16,
                                               Ot[ct][j]);
                        }
                }
            }

            // S <- Diag(e^{G_last}) S + (K . e^{G_last - G})^T U
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float gc = sVec[V_GC * DK + rt * 16 + 4 * q4 + j];
                    S[rt][0][j] *= gc;
                    S[rt][1][j] *= gc;
                }
                const int c = rt * 16 + l16;  // key channel of this lane's operand row
#pragma unroll
                for (int kbt = 0; kbt < 2; ++kbt) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tok = kbt * 32 + kperm(q4, e);
                        const int b = tok >> 4;
                        x[e] = O::from_op(sG[tok * C::SK + c]) * sVec[(V_FY + b) * DK + c] *
                               sVec[(V_EL + b) * DK + c];
                    }
                    const Frag kf = O::make(x);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) O::mma(S[rt][ct], kf, Ub[kbt][ct]);
                }
            }
        }
    }

    // ---- write the segment result
    if (chain) {
        float* dst = nullptr;
        int ld = DV, cofs = 0;
        if (SUMMARY) {
            dst = p.ms + (int64_t(item) * H + h) * DK * (DK + DV);
            ld = DK + DV;
        } else if (last_seg && p.fin) {
            dst = p.fin + (int64_t(n) * H + h) * DK * DV;
        }
        if (dst) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        dst[(rt * 16 + 4 * q4 + j) * ld + cofs + colbase + ct * 16 + l16] = S[rt][ct][j];
        }
    }
}

// ------------------------------------------------------------- scan kernel
// Per (sequence, head, 32-column block): S_in(s+1) = M_s S_in(s) + S~_s.
template <int DK, int DV>
__global__ void __launch_bounds__(256) scan_kernel(PrefillDev p)
{
    constexpr int NB = DV / 32;
    __shared__ float sS[DK][33];
    const int H = p.H;
    const int jb = blockIdx.x % NB;
    const int h = (blockIdx.x / NB) % H;
    const int n = blockIdx.x / (NB * H);
    const int32_t* seg_off = p.tab + (p.N + 1);
    const int32_t* p1_off = p.tab + 2 * (p.N + 1);
    const int nseg = seg_off[n + 1] - seg_off[n];
    if (nseg <= 1) return;
    const int tid = threadIdx.x;
    // thread -> (row c, 32/(256/DK) columns)
    constexpr int TPR = 256 / DK;       // threads per row
    constexpr int CPT = 32 / TPR;       // columns per thread
    const int c = tid / TPR;
    const int j0 = (tid % TPR) * CPT;
    for (int e = tid; e < DK * 32; e += 256) {
        const int r = e / 32, cc = e % 32;
        float x = 0.f;
        if (p.init) x = p.init[(int64_t(n) * H + h) * DK * DV + r * DV + jb * 32 + cc];
        sS[r][cc] = x;
    }
    __syncthreads();
    for (int s = 0; s + 1 < nseg; ++s) {
        const float* ms = p.ms + (int64_t(p1_off[n] + s) * H + h) * DK * (DK + DV);
        float acc[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) acc[j] = ms[c * (DK + DV) + jb * 32 + j0 + j];
        const float* mrow = ms + c * (DK + DV) + DV;
        for (int cc = 0; cc < DK; ++cc) {
            const float m = mrow[cc];
#pragma unroll
            for (int j = 0; j < CPT; ++j) acc[j] += m * sS[cc][j0 + j];
        }
        __syncthreads();
        float* out = p.sin + (int64_t(seg_off[n] + s + 1) * H + h) * DK * DV;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            sS[c][j0 + j] = acc[j];
            out[c * DV + jb * 32 + j0 + j] = acc[j];
        }
        __syncthreads();
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
        hipLaunchKernelGGL((scan_kernel<DK, DV>), dim3(unsigned(a.N * a.H * (DV / 32))), dim3(256), 0,
                           stream, d);
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
        KDA_PF(32, 32) KDA_PF(32, 64) KDA_PF(64, 32) KDA_PF(64, 64)
    }
#undef KDA_PF
    return hipErrorInvalidValue;
}

}  // namespace kda
