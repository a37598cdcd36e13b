// kda_backward: the pieces of the backward shared by its kernels (arguments,
// segment lookup, the segment scan and the planner); the kernels that run the
// chunks are in kda_bwd_chunk.hpp.
//
// Sources: "NLP——技术报告解读-Kimi-K3", Model Architecture / Kimi Delta
// Attention (KDA) (the state update and read-out; the pages give no backward,
// so it is the chain rule applied to that step), and Infrastructure / KDA
// algorithm-system co-design (FlashKDA serves training as well as inference;
// one sequence split across the compute units, each segment's transition
// computed independently and composed exactly).
//
// For L = sum_t <dO_t, o_t> + <dS_fin, S_T>, the state gradient evolves as
// dS_prev = F^T (dS + q dO^T), F = (I - beta k k^T) Diag(e^g) the forward
// transition: affine in dS and free of the forward state.  So a segment maps
// dS_start = M^T dS_end + C, with M the segment's forward transition and C
// the segment's own contribution (dS_end = 0).  Every segment but a
// sequence's last first takes its dS_end from a window of `warm` tokens after
// it: the state-free step run backwards from dS = 0 at the window's far end
// beside the window's M^T (columns starting at I).  When the computed M^T is
// exactly zero (its entries underflow within about a hundred tokens of the
// gate's bounded decay) dS_end is the window's C; a window that reaches the
// sequence end starts from the final state's gradient and is exact.  Chains
// where a window's M^T is not zero are flagged, and for them a summary pass
// computes [C | M^T] per (segment, head) and a scan takes dS_start = M^T
// dS_end + C backwards over the segments.  The full pass then runs every
// segment from its dS_end, in parallel.
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
    const float* ckpt;      // the forward's checkpoints every ckpt_interval tokens, or null
    int64_t ckpt_cap;
    int64_t ckpt_interval;  // a positive multiple of BWD_CHUNK
    const void* d_o;        // [T, H, dv] or null
    const float* d_fin;     // [N, H, dk, dv] or null
    float *dq, *dk, *dv, *dg, *dbeta, *d_init;
    float* scratch;         // per workgroup: the states at a chunk's sub-chunk starts, and dS'
    int64_t Lseg;           // tokens per segment (a multiple of BWD_CHUNK)
    float* cm;              // per (segment, head): C [dk][dv] then M^T [dk][dk], fp32
    float* dsend;           // per (segment, head): dS at the segment's end [dk][dv], fp32
    int32_t* flags = nullptr;  // per (segment, head): 1 where the window's M^T was not zero
    int64_t warm = 0;          // window tokens (a multiple of 16); 0: summary pass and scan for every chain
    int64_t segs_cap = 0;      // the plan's segment count (bounds checks)
};

// Whether the chain (sequence of segments seg0 .. seg0+nseg-1, head h) goes
// through the summary pass and the scan: always without windows (no flags),
// else when any of its segments was flagged; uniform across the workgroup.
__device__ __forceinline__ bool bwd_chain_flagged(const BackwardArgs& a, int seg0, int nseg, int h)
{
    if (a.flags == nullptr) return true;
    // lane j reads segment j's flag, all at once (see the prefill's chain_flagged)
    const int lane = threadIdx.x & 63;
    bool any = false;
    for (int j0 = 0; j0 < nseg; j0 += 64) {
        const int j = j0 + lane;
        const bool f = j < nseg && a.flags[int64_t(seg0 + j) * a.H + h] != 0;
        any = any || __ballot(f) != 0;
    }
    return any;
}

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
        ck += (x - prev) / a.ckpt_interval;
        prev = x;
    }
    return L;
}

// Scan: one workgroup of 256 threads per (sequence, head, 16 columns of dS).
// Backwards over the sequence's segments: dS_end of segment s is dS_start of
// segment s + 1, and dS_start(s) = M_s^T dS_end(s) + C_s, in fp32.  M_s^T is
// staged in LDS (the next one is loaded into registers while the current
// product runs); each thread owns DK/16 rows of one column.  Writes every
// segment's dS_end for the full pass.
constexpr int BWD_SCAN_COLS = 16;
template <int DK>
struct BwdScanCfg {
    static constexpr int RG = 256 / BWD_SCAN_COLS;  // row groups
    static constexpr int RPT = DK / RG;             // rows per thread
    static constexpr int SM = DK + 4;               // padded row stride of M^T in LDS
    static constexpr int NV = DK * DK / 4 / 256;    // float4 of M^T per thread
    static constexpr int LDS = (DK * SM + DK * (BWD_SCAN_COLS + 1)) * 4;
};

template <int DK, int DV>
__global__ void __launch_bounds__(256) bwd_scan_kernel(BackwardArgs a)
{
    using C = BwdScanCfg<DK>;
    constexpr int NSL = DV / BWD_SCAN_COLS;
    extern __shared__ __attribute__((aligned(16))) float ssm[];
    float* sM = ssm;                 // [DK][SM]
    float* sd = ssm + DK * C::SM;    // [DK][BWD_SCAN_COLS + 1]
    constexpr int SD = BWD_SCAN_COLS + 1;
    const int H = a.H;
    const int slice = blockIdx.x % NSL, unit = blockIdx.x / NSL;
    const int n = unit / H, h = unit % H;
    const int t = threadIdx.x, jj = t % BWD_SCAN_COLS, rgp = t / BWD_SCAN_COLS;
    const int col = slice * BWD_SCAN_COLS + jj;
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
    KDA_CHECK(n < a.N, CK_SEQ);
    KDA_CHECK(seg0 + nseg <= a.segs_cap, CK_WS);
    if (!bwd_chain_flagged(a, seg0, nseg, h)) return;  // the windows gave every dS_end
    auto cm_of = [&](int s) { return a.cm + (int64_t(seg0 + s) * H + h) * (DK * DV + DK * DK); };
    auto dsend_of = [&](int s) { return a.dsend + (int64_t(seg0 + s) * H + h) * DK * DV; };
    // the last segment ends at the final state: its dS_end is the final state's gradient
    for (int r = rgp; r < DK; r += C::RG) {
        dsend_of(nseg - 1)[r * DV + col] = a.d_fin ? a.d_fin[unit * int64_t(DK) * DV + r * DV + col] : 0.f;
        if (nseg > 1) sd[r * SD + jj] = cm_of(nseg - 1)[r * DV + col];  // dS_start of the last segment
    }
    f32x4 pre[C::NV];
    auto load_m = [&](int s) {
        const f32x4* src = reinterpret_cast<const f32x4*>(cm_of(s) + DK * DV);
#pragma unroll
        for (int i = 0; i < C::NV; ++i) pre[i] = src[t + 256 * i];
    };
    if (nseg >= 3) load_m(nseg - 2);
    __syncthreads();
    // dS_start of segment 0 is the full pass's (the initial state's gradient),
    // so the composition stops at segment 1 and segment 0's summary is not read
    for (int s = nseg - 2; s >= 1; --s) {
#pragma unroll
        for (int i = 0; i < C::NV; ++i) {
            const int e = 4 * (t + 256 * i), r = e / DK, c = e % DK;
            *reinterpret_cast<f32x4*>(sM + r * C::SM + c) = pre[i];
        }
        const float* Cs = cm_of(s);
        float acc[C::RPT];
#pragma unroll
        for (int i = 0; i < C::RPT; ++i) acc[i] = Cs[(rgp * C::RPT + i) * DV + col];
        __syncthreads();  // M_s^T staged
        if (s >= 2) load_m(s - 1);
        for (int c = 0; c < DK; c += 4) {
            const float d0 = sd[c * SD + jj], d1 = sd[(c + 1) * SD + jj];
            const float d2 = sd[(c + 2) * SD + jj], d3 = sd[(c + 3) * SD + jj];
#pragma unroll
            for (int i = 0; i < C::RPT; ++i) {
                const f32x4 m = *reinterpret_cast<const f32x4*>(sM + (rgp * C::RPT + i) * C::SM + c);
                acc[i] += m[0] * d0 + m[1] * d1 + m[2] * d2 + m[3] * d3;
            }
        }
        for (int r = rgp; r < DK; r += C::RG) dsend_of(s)[r * DV + col] = sd[r * SD + jj];
        __syncthreads();  // every thread has read dS_end(s) and M_s^T
#pragma unroll
        for (int i = 0; i < C::RPT; ++i) sd[(rgp * C::RPT + i) * SD + jj] = acc[i];
        __syncthreads();
    }
    if (nseg >= 2)
        for (int r = rgp; r < DK; r += C::RG) dsend_of(0)[r * DV + col] = sd[r * SD + jj];
}

struct BwdPlan {
    int64_t Lseg = 0, segs_max = 0, warm = 0;
    int grid = 0;
    size_t off_scratch = 0, off_cm = 0, off_dsend = 0, off_flags = 0, bytes = 0;
};

constexpr int64_t BWD_WARM_DEFAULT = 128;  // tokens

// Segment length: enough (segment, head) items to cover the compute units
// about once (each runs its chunks in series), at least one 64-token chunk.
// force_tokens > 0 fixes it instead (rounded up to whole chunks); warm_req
// < 0 takes the default window, 0 turns the windows off, > 0 sets them (a
// multiple of 16 tokens).
inline BwdPlan backward_plan(int64_t T_total, int N, int H, int dk, int dv, int64_t force_tokens = 0,
                             int64_t warm_req = -1)
{
    BwdPlan p;
    p.warm = warm_req < 0 ? BWD_WARM_DEFAULT : warm_req;
    const int64_t T = T_total > 0 ? T_total : 1;
    if (int64_t(N) * H >= BWD_MAX_WG / 2) {
        p.Lseg = (T + BWD_CHUNK - 1) / BWD_CHUNK * BWD_CHUNK;  // one segment per sequence
    } else {
        const int64_t per = (T * H + int64_t(BWD_MAX_WG) * BWD_CHUNK - 1) / (int64_t(BWD_MAX_WG) * BWD_CHUNK);
        p.Lseg = BWD_CHUNK * (per > 0 ? per : 1);
    }
    if (force_tokens > 0) p.Lseg = (force_tokens + BWD_CHUNK - 1) / BWD_CHUNK * BWD_CHUNK;
    // >= the sum over sequences of max(1, ceil(len / Lseg)); exact for one sequence
    p.segs_max = N == 1 ? (T + p.Lseg - 1) / p.Lseg : T / p.Lseg + 1 + N;
    const int64_t items = p.segs_max * H;
    p.grid = int(items < BWD_MAX_WG ? items : BWD_MAX_WG);
    size_t off = 0;
    p.off_scratch = off;
    // per workgroup: the states at the four 16-token sub-chunk starts of a chunk
    // (in two layouts), and one more for dS'
    off = align256(off + size_t(p.grid) * (2 * (BWD_CHUNK / 16) + 1) * size_t(dk) * dv * sizeof(float));
    p.off_cm = off;
    off = align256(off + size_t(items) * (size_t(dk) * dv + size_t(dk) * dk) * sizeof(float));
    p.off_dsend = off;
    off = align256(off + size_t(items) * dk * dv * sizeof(float));
    p.off_flags = off;
    off = align256(off + size_t(items) * sizeof(int32_t));
    p.bytes = off;
    return p;
}

}  // namespace kda
