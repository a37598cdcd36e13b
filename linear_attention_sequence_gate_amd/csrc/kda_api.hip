// libkda C ABI: argument validation, planning and kernel launches.
// Every check runs on the host before anything is enqueued; see include/kda.h
// for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <mutex>

#include "kda.h"
#include "kda_decode.hpp"
#include "kda_gate.hpp"
#include "kda_prefill.hpp"
#include "kda_serial.hpp"
#include "kda_spec.hpp"
#include "kda_step.hpp"
#include "kda_backward.hpp"
#include "kda_bwd_chunk.hpp"

namespace {

thread_local char g_err[512] = "";

kda_status_t fail(kda_status_t s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

kda_status_t ok()
{
    g_err[0] = '\0';
    return KDA_OK;
}

kda_status_t from_hip(hipError_t e, const char* what)
{
    if (e == hipSuccess) return ok();
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
bool dtype_ok(kda_dtype_t t) { return t == KDA_F32 || t == KDA_BF16; }
size_t dsize(kda_dtype_t t) { return t == KDA_BF16 ? 2 : 4; }

// true when [a, a+na) and [b, b+nb) overlap (byte ranges)
bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status_t s)
{
    switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    default: break;  // the int-range enumerators and unknown codes
    }
    return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_err; }

int kda_version(void) { return 100; }

kda_status_t kda_gate(const void* z, const float* A, void* g, int64_t n_tokens, int H, int d_k,
                      kda_dtype_t dtype, float g_min, void* stream)
{
    if (n_tokens < 0 || H < 1 || d_k < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: bad sizes n_tokens=%lld H=%d d_k=%d",
                    (long long)n_tokens, H, d_k);
    if (!dtype_ok(dtype)) return fail(KDA_ERR_UNSUPPORTED, "kda_gate: unknown dtype %d", (int)dtype);
    // the prefill and the backward factor decay ratios per 16-token sub-tile
    // and need g >= -5 to keep every factor inside the fp32 range
    if (!std::isfinite(g_min) || !(g_min < 0.f) || g_min < -5.f)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: g_min must lie in [-5, 0)");
    if (n_tokens == 0) return ok();
    if (!z || !A || !g) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: null pointer");
    const size_t bytes = size_t(n_tokens) * H * d_k * dsize(dtype);
    if (z != g && overlap(z, bytes, g, bytes))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: g partially overlaps z");
    if (overlap(A, sizeof(float) * H, g, bytes))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: g overlaps A");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = dtype == KDA_BF16 ? kda::launch_gate<kda::BF16>(z, A, g, n_tokens, H, d_k, g_min, s)
                                     : kda::launch_gate<kda::F32>(z, A, g, n_tokens, H, d_k, g_min, s);
    return from_hip(e, "kda_gate launch");
}

// the one-wave step kernels take 16-byte aligned token tensors and one
// workgroup per 32-column slice of each (b, h) state; otherwise the
// workgroup-per-state kernels run (scalar token loads)
static bool step_wave_ok(const void* q, const void* k, const void* v, const void* g, const void* o, int B, int H,
                         int d_v)
{
    return kda::step_wave_aligned(q, k, v, g, o) && int64_t(B) * H * (d_v / 32) <= 0x7fffffff;
}

static kda_status_t decode_impl(const char* who, const void* q, const void* k, const void* v, const void* g,
                               const void* beta, float* state, void* o, int B, int H, int d_k, int d_v,
                               kda_dtype_t dtype, void* stream, const float* gate_A = nullptr, float g_min = -5.f)
{
    if (B < 0 || H < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: bad sizes B=%d H=%d", who, B, H);
    if (!dtype_ok(dtype))
        return fail(KDA_ERR_UNSUPPORTED, "%s: unknown dtype %d", who, (int)dtype);
    if (!dim_ok(d_k) || !dim_ok(d_v))
        return fail(KDA_ERR_UNSUPPORTED, "%s: d_k=%d d_v=%d not in {32,64,128}", who, d_k, d_v);
    if (B == 0) return ok();
    if (!q || !k || !v || !g || !beta || !state || !o)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null pointer", who);
    if ((reinterpret_cast<uintptr_t>(state) & 15) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state must be 16-byte aligned", who);
    if (int64_t(B) * H > 0x7fffffff)
        return fail(KDA_ERR_UNSUPPORTED, "%s: B*H too large", who);
    const size_t es = dsize(dtype);
    const size_t nk = size_t(B) * H * d_k * es, nv = size_t(B) * H * d_v * es;
    const size_t nb = size_t(B) * H * es, ns = size_t(B) * H * d_k * d_v * sizeof(float);
    const void* ins[6] = {q, k, v, g, beta, gate_A};
    const size_t insz[6] = {nk, nk, nv, nk, nb, gate_A ? size_t(H) * sizeof(float) : 0};
    for (int i = 0; i < 6; ++i) {
        if (overlap(o, nv, ins[i], insz[i]))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: o aliases an input", who);
        if (overlap(state, ns, ins[i], insz[i]))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state aliases an input", who);
    }
    if (overlap(o, nv, state, ns))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: o aliases the state", who);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (step_wave_ok(q, k, v, g, o, B, H, d_v))
        e = dtype == KDA_BF16 ? kda::launch_step_wave<kda::BF16>(0, q, k, v, g, beta, nullptr, state, o, B, 1, H,
                                                                 d_k, d_v, s, gate_A, g_min)
                              : kda::launch_step_wave<kda::F32>(0, q, k, v, g, beta, nullptr, state, o, B, 1, H,
                                                                d_k, d_v, s, gate_A, g_min);
    else
        e = dtype == KDA_BF16
                ? kda::launch_decode<kda::BF16>(q, k, v, g, beta, state, o, B * H, d_k, d_v, s, H, gate_A, g_min)
                : kda::launch_decode<kda::F32>(q, k, v, g, beta, state, o, B * H, d_k, d_v, s, H, gate_A, g_min);
    return from_hip(e, "decode launch");
}

kda_status_t kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, float* state, void* o, int B, int H, int d_k,
                             int d_v, kda_dtype_t dtype, void* stream)
{
    return decode_impl("kda_decode_step", q, k, v, g, beta, state, o, B, H, d_k, d_v, dtype, stream);
}

kda_status_t kda_decode_step_gated(const void* q, const void* k, const void* v, const void* z, const float* A,
                                   float g_min, const void* beta, float* state, void* o, int B, int H, int d_k,
                                   int d_v, kda_dtype_t dtype, void* stream)
{
    if (!std::isfinite(g_min) || !(g_min < 0.f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode_step_gated: g_min must be finite and negative");
    if (B > 0 && !A) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode_step_gated: null A");
    return decode_impl("kda_decode_step_gated", q, k, v, z, beta, state, o, B, H, d_k, d_v, dtype, stream, A,
                       g_min);
}

// shared checks of kda_verify / kda_commit; returns KDA_OK with *noop set for B == 0
static kda_status_t spec_check(const char* who, bool commit, const void* q, const void* k, const void* v,
                               const void* g, const void* beta, const void* n_accept, const float* state,
                               const void* o, int B, int K, int H, int d_k, int d_v, kda_dtype_t dtype,
                               bool* noop)
{
    *noop = false;
    if (B < 0 || H < 1 || K < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: bad sizes B=%d K=%d H=%d", who, B, K, H);
    if (K > KDA_MAX_DRAFT) return fail(KDA_ERR_UNSUPPORTED, "%s: K=%d > %d", who, K, KDA_MAX_DRAFT);
    if (!dtype_ok(dtype)) return fail(KDA_ERR_UNSUPPORTED, "%s: unknown dtype %d", who, (int)dtype);
    if (!dim_ok(d_k) || !dim_ok(d_v))
        return fail(KDA_ERR_UNSUPPORTED, "%s: d_k=%d d_v=%d not in {32,64,128}", who, d_k, d_v);
    if (B == 0) {
        *noop = true;
        return ok();
    }
    if ((!commit && (!q || !o)) || !k || !v || !g || !beta || !state || (commit && !n_accept))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null pointer", who);
    if ((reinterpret_cast<uintptr_t>(state) & 15) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state must be 16-byte aligned", who);
    if (int64_t(B) * H > 0x7fffffff || int64_t(B) * K * H * 128 > (int64_t(1) << 40))
        return fail(KDA_ERR_UNSUPPORTED, "%s: B*K*H too large", who);
    const size_t es = dsize(dtype);
    const size_t nt = size_t(B) * K * H;
    const size_t nk = nt * d_k * es, nv = nt * d_v * es, nb = nt * es;
    const size_t ns = size_t(B) * H * d_k * d_v * sizeof(float);
    const void* ins[6] = {q, k, v, g, beta, n_accept};
    const size_t insz[6] = {commit ? 0 : nk, nk, nv, nk, nb, commit ? size_t(B) * sizeof(int32_t) : 0};
    for (int i = 0; i < 6; ++i) {
        if (!commit && overlap(o, nv, ins[i], insz[i]))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: o aliases an input", who);
        if (overlap(state, ns, ins[i], insz[i]))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state aliases an input", who);
    }
    if (!commit && overlap(o, nv, state, ns))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: o aliases the state", who);
    return ok();
}

kda_status_t kda_verify(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        const float* state, void* o, int B, int K, int H, int d_k, int d_v,
                        kda_dtype_t dtype, void* stream)
{
    bool noop;
    kda_status_t st = spec_check("kda_verify", false, q, k, v, g, beta, nullptr, state, o, B, K, H, d_k, d_v,
                                 dtype, &noop);
    if (st != KDA_OK || noop) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* S = const_cast<float*>(state);  // read only in verify mode
    hipError_t e;
    if (step_wave_ok(q, k, v, g, o, B, H, d_v))
        e = dtype == KDA_BF16
                ? kda::launch_step_wave<kda::BF16>(1, q, k, v, g, beta, nullptr, S, o, B, K, H, d_k, d_v, s)
                : kda::launch_step_wave<kda::F32>(1, q, k, v, g, beta, nullptr, S, o, B, K, H, d_k, d_v, s);
    else
        e = dtype == KDA_BF16
                ? kda::launch_spec<kda::BF16>(q, k, v, g, beta, nullptr, S, o, B, K, H, d_k, d_v, false, s)
                : kda::launch_spec<kda::F32>(q, k, v, g, beta, nullptr, S, o, B, K, H, d_k, d_v, false, s);
    return from_hip(e, "kda_verify launch");
}

kda_status_t kda_commit(const void* k, const void* v, const void* g, const void* beta,
                        const int32_t* n_accept, float* state, int B, int K, int H, int d_k, int d_v,
                        kda_dtype_t dtype, void* stream)
{
    bool noop;
    kda_status_t st = spec_check("kda_commit", true, nullptr, k, v, g, beta, n_accept, state, nullptr, B, K, H,
                                 d_k, d_v, dtype, &noop);
    if (st != KDA_OK || noop) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (step_wave_ok(nullptr, k, v, g, nullptr, B, H, d_v))
        e = dtype == KDA_BF16 ? kda::launch_step_wave<kda::BF16>(2, nullptr, k, v, g, beta, n_accept, state,
                                                                 nullptr, B, K, H, d_k, d_v, s)
                              : kda::launch_step_wave<kda::F32>(2, nullptr, k, v, g, beta, n_accept, state,
                                                                nullptr, B, K, H, d_k, d_v, s);
    else
        e = dtype == KDA_BF16 ? kda::launch_spec<kda::BF16>(nullptr, k, v, g, beta, n_accept, state, nullptr, B,
                                                            K, H, d_k, d_v, true, s)
                              : kda::launch_spec<kda::F32>(nullptr, k, v, g, beta, n_accept, state, nullptr, B, K,
                                                           H, d_k, d_v, true, s);
    return from_hip(e, "kda_commit launch");
}

// the shapes the block kernels are built for
static bool prefill_shape_ok(int64_t T_total, int N, int H, int d_k, int d_v, int chunk, kda_dtype_t dtype)
{
    return T_total >= 0 && T_total <= int64_t(0x7fffffff) && N >= 1 && H >= 1 && H <= KDA_MAX_HEADS &&
           dim_ok(d_k) && dim_ok(d_v) && chunk == 64 && dtype_ok(dtype);
}

// fp32 head shapes without a chunk kernel run token by token
static bool serial_path(int d_k, int d_v, kda_dtype_t dtype)
{
    return dtype == KDA_F32 && kda::serial_shape_f32(d_k, d_v);
}

static kda::PrefillPlan plan_for(int64_t T_total, int N, int H, int d_k, int d_v, kda_dtype_t dtype,
                                 int force_L = 0, int warm_req = -1)
{
    if (serial_path(d_k, d_v, dtype)) return kda::serial_plan(T_total, N, H, d_k, d_v, force_L, warm_req);
    return kda::prefill_plan(T_total, N, H, d_k, d_v, force_L, warm_req);
}

size_t kda_prefill_workspace_size(int64_t T_total, int N, int H, int d_k, int d_v, int chunk,
                                  kda_dtype_t dtype)
{
    if (!prefill_shape_ok(T_total, N, H, d_k, d_v, chunk, dtype)) return 0;
    return plan_for(T_total, N, H, d_k, d_v, dtype).workspace_bytes;
}

// force_L > 0 fixes the segment length in chunks; warm_req < 0 takes the
// planner's warm-up, 0 turns it off, > 0 sets it (both only from the test
// entry point)
static kda_status_t prefill_impl(const char* who, const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total, int H,
                                 int d_k, int d_v, int chunk, const float* initial_state, float* final_state,
                                 void* o, kda_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                 int ckpt_interval, float* ckpt_states, int64_t ckpt_capacity, void* stream,
                                 const float* gate_A = nullptr, float g_min = -5.f, int force_L = 0,
                                 int warm_req = -1)
{
    if (N < 1 || T_total < 0 || H < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: bad sizes N=%d T_total=%lld H=%d", who, N,
                    (long long)T_total, H);
    if (H > KDA_MAX_HEADS) return fail(KDA_ERR_UNSUPPORTED, "%s: H=%d > %d", who, H, KDA_MAX_HEADS);
    if (!cu_seqlens && N != 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is NULL but N=%d", who, N);
    if (!dtype_ok(dtype))
        return fail(KDA_ERR_UNSUPPORTED, "%s: unknown dtype %d", who, (int)dtype);
    if (!dim_ok(d_k) || !dim_ok(d_v))
        return fail(KDA_ERR_UNSUPPORTED, "%s: d_k=%d d_v=%d not in {32,64,128}", who, d_k, d_v);
    if (chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "%s: chunk=%d (only 64)", who, chunk);
    if (T_total > int64_t(0x7fffffff))  // token offsets are int32, as cu_seqlens
        return fail(KDA_ERR_UNSUPPORTED, "%s: T_total > 2^31 - 1", who);
    if (T_total > 0 && (!q || !k || !v || !g || !beta || !o))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null token tensor", who);
    if (gate_A) {
        // the block kernels bound every decay factor through g >= -5 per token
        if (!std::isfinite(g_min) || !(g_min < 0.f) || g_min < -5.f)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: g_min must lie in [-5, 0)", who);
        const size_t na = size_t(H) * sizeof(float);
        if (overlap(o, size_t(T_total) * H * d_v * dsize(dtype), gate_A, na) ||
            overlap(final_state, final_state ? size_t(N) * H * d_k * d_v * sizeof(float) : 0, gate_A, na) ||
            overlap(workspace, plan_for(T_total, N, H, d_k, d_v, dtype, force_L, warm_req).workspace_bytes,
                    gate_A, na))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: A overlaps an output buffer", who);
    }
    const kda::PrefillPlan plan = plan_for(T_total, N, H, d_k, d_v, dtype, force_L, warm_req);
    const size_t ws_need = plan.workspace_bytes;
    if (ws_need > 0 && (!workspace || workspace_bytes < ws_need))
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < %zu needed", who,
                    workspace_bytes, ws_need);
    const size_t es = dsize(dtype);
    const size_t nk = size_t(T_total) * H * d_k * es, nv = size_t(T_total) * H * d_v * es;
    const size_t nb = size_t(T_total) * H * es;
    const size_t ns = size_t(N) * H * d_k * d_v * sizeof(float);
    const void* ins[6] = {q, k, v, g, beta, initial_state};
    const size_t insz[6] = {nk, nk, nv, nk, nb, initial_state ? ns : 0};
    for (int i = 0; i < 6; ++i) {
        if (overlap(o, nv, ins[i], insz[i]))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: o aliases an input", who);
        if (i < 5 && overlap(final_state, final_state ? ns : 0, ins[i], insz[i]))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: final_state aliases a token input", who);
        if (overlap(workspace, ws_need, ins[i], insz[i]))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: workspace aliases an input", who);
    }
    if (final_state && initial_state && final_state != initial_state &&
        overlap(final_state, ns, initial_state, ns))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: final_state partially overlaps initial_state", who);
    if (overlap(o, nv, final_state, final_state ? ns : 0) ||
        overlap(workspace, ws_need, o, nv) ||
        overlap(workspace, ws_need, final_state, final_state ? ns : 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: output buffers overlap", who);
    if (ckpt_interval < 0 || (ckpt_interval > 0 && ckpt_interval % kda::CH != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: checkpoint interval %d is not a positive multiple of %d", who,
                    ckpt_interval, kda::CH);
    if (ckpt_interval > 0 && T_total / ckpt_interval > 0x7fffffff)
        return fail(KDA_ERR_UNSUPPORTED, "%s: too many checkpoints", who);
    if (ckpt_interval > 0 && ckpt_capacity > 0) {
        if (!ckpt_states) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null checkpoint buffer", who);
        if ((reinterpret_cast<uintptr_t>(ckpt_states) & 3) != 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: checkpoint buffer not 4-byte aligned", who);
        const size_t nc = size_t(ckpt_capacity) * H * d_k * d_v * sizeof(float);
        const void* all[9] = {q, k, v, g, beta, initial_state, final_state, o, workspace};
        const size_t allsz[9] = {size_t(T_total) * H * d_k * dsize(dtype), size_t(T_total) * H * d_k * dsize(dtype),
                                 size_t(T_total) * H * d_v * dsize(dtype), size_t(T_total) * H * d_k * dsize(dtype),
                                 size_t(T_total) * H * dsize(dtype),
                                 initial_state ? size_t(N) * H * d_k * d_v * sizeof(float) : 0,
                                 final_state ? size_t(N) * H * d_k * d_v * sizeof(float) : 0,
                                 size_t(T_total) * H * d_v * dsize(dtype), ws_need};
        for (int i = 0; i < 9; ++i)
            if (overlap(ckpt_states, nc, all[i], allsz[i]))
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s: checkpoint buffer overlaps another buffer", who);
    }
    if (!final_state && T_total == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    kda::PrefillArgs a{q, k, v, g, beta, cu_seqlens, N, T_total, H, d_k, d_v,
                       initial_state, final_state, o, workspace};
    if (ckpt_interval > 0 && ckpt_capacity > 0) {
        a.ckpt = ckpt_states;
        a.ckpt_interval = ckpt_interval;
        a.ckpt_cap = ckpt_capacity;
    }
    a.gate_A = gate_A;
    a.g_min = g_min;
    a.init_snap = (initial_state && initial_state == final_state) ? 1 : 0;
    const hipError_t e = serial_path(d_k, d_v, dtype) ? kda::launch_serial(a, plan, s)
                         : dtype == KDA_BF16         ? kda::launch_prefill<kda::BF16>(a, plan, s)
                                                     : kda::launch_prefill<kda::F32>(a, plan, s);
    return from_hip(e, "kda_prefill launch");
}

kda_status_t kda_prefill(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total,
                         int H, int d_k, int d_v, int chunk, const float* initial_state,
                         float* final_state, void* o, kda_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    return prefill_impl("kda_prefill", q, k, v, g, beta, cu_seqlens, N, T_total, H, d_k, d_v, chunk,
                        initial_state, final_state, o, dtype, workspace, workspace_bytes, 0, nullptr, 0, stream);
}

kda_status_t kda_prefill_ckpt(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total,
                              int H, int d_k, int d_v, int chunk, const float* initial_state,
                              float* final_state, void* o, kda_dtype_t dtype, void* workspace,
                              size_t workspace_bytes, int ckpt_interval, float* ckpt_states,
                              int64_t ckpt_capacity, void* stream)
{
    if (ckpt_interval <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_ckpt: checkpoint interval %d", ckpt_interval);
    if (ckpt_capacity < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_ckpt: negative checkpoint capacity");
    return prefill_impl("kda_prefill_ckpt", q, k, v, g, beta, cu_seqlens, N, T_total, H, d_k, d_v, chunk,
                        initial_state, final_state, o, dtype, workspace, workspace_bytes, ckpt_interval,
                        ckpt_states, ckpt_capacity, stream);
}

kda_status_t kda_prefill_gated(const void* q, const void* k, const void* v, const void* z, const float* A,
                               float g_min, const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total,
                               int H, int d_k, int d_v, int chunk, const float* initial_state, float* final_state,
                               void* o, kda_dtype_t dtype, void* workspace, size_t workspace_bytes,
                               int ckpt_interval, float* ckpt_states, int64_t ckpt_capacity, void* stream)
{
    if (!std::isfinite(g_min) || !(g_min < 0.f) || g_min < -5.f)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_gated: g_min must lie in [-5, 0)");
    if (T_total > 0 && !A) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_gated: null A");
    if (ckpt_interval < 0 || ckpt_capacity < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_gated: negative checkpoint interval or capacity");
    // with no tokens nothing reads A (the state is only copied through)
    return prefill_impl("kda_prefill_gated", q, k, v, z, beta, cu_seqlens, N, T_total, H, d_k, d_v, chunk,
                        initial_state, final_state, o, dtype, workspace, workspace_bytes, ckpt_interval,
                        ckpt_states, ckpt_capacity, stream, T_total > 0 ? A : nullptr, g_min);
}

// ---- the prefill without a workspace argument, for callers that cannot
// allocate.  Its workspace is this array: each GPU the library runs on holds
// one copy until the process ends.  Host code must use the address that
// hipGetSymbolAddress returns for the current device, never the array's name
// (on the host that is a stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; null with *err set on failure.
static void* scratch_address(hipError_t* err)
{
    constexpr int MAX_DEV = 64;
    static std::mutex mu;
    static void* addr[MAX_DEV] = {};
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= MAX_DEV) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

kda_status_t kda_prefill_gated_noalloc(const void* q, const void* k, const void* v, const void* z, const float* A,
                                       float g_min, const void* beta, const int32_t* cu_seqlens, int N,
                                       int64_t T_total, int H, int d_k, int d_v, int chunk,
                                       const float* initial_state, float* final_state, void* o, kda_dtype_t dtype,
                                       int ckpt_interval, float* ckpt_states, int64_t ckpt_capacity, void* stream)
{
    const char* who = "kda_prefill_gated_noalloc";
    if (!prefill_shape_ok(T_total, N, H, d_k, d_v, chunk, dtype))
        return fail(KDA_ERR_UNSUPPORTED, "%s: shape outside the supported set (see kda_prefill)", who);
    const size_t need = plan_for(T_total, N, H, d_k, d_v, dtype).workspace_bytes;
    if (need > KDA_NOALLOC_SCRATCH_BYTES)
        return fail(KDA_ERR_UNSUPPORTED, "%s: this call needs %zu bytes of workspace, more than the %zu-byte "
                    "static scratch; use kda_prefill_gated with a workspace", who, need,
                    size_t(KDA_NOALLOC_SCRATCH_BYTES));
    hipError_t e = hipSuccess;
    void* ws = need > 0 ? scratch_address(&e) : nullptr;
    if (need > 0 && !ws) return from_hip(e, "kda_prefill_gated_noalloc: scratch address");
    return kda_prefill_gated(q, k, v, z, A, g_min, beta, cu_seqlens, N, T_total, H, d_k, d_v, chunk, initial_state,
                             final_state, o, dtype, ws, need, ckpt_interval, ckpt_states, ckpt_capacity, stream);
}

// ---- test-only entry points: the planner's choices made explicit
static bool test_plan_ok(int seg_chunks, int warm_tokens)
{
    return seg_chunks >= 0 && (warm_tokens == -1 || (warm_tokens >= 0 && warm_tokens % kda::BC == 0));
}

size_t kda_test_prefill_workspace_size(int64_t T_total, int N, int H, int d_k, int d_v, kda_dtype_t dtype,
                                       int seg_chunks, int warm_tokens)
{
    if (!prefill_shape_ok(T_total, N, H, d_k, d_v, 64, dtype) || !test_plan_ok(seg_chunks, warm_tokens)) return 0;
    return plan_for(T_total, N, H, d_k, d_v, dtype, seg_chunks, warm_tokens).workspace_bytes;
}

int64_t kda_test_prefill_flags(int64_t T_total, int N, int H, int d_k, int d_v, kda_dtype_t dtype, int seg_chunks,
                               int warm_tokens, size_t* offset_bytes)
{
    if (!prefill_shape_ok(T_total, N, H, d_k, d_v, 64, dtype) || !test_plan_ok(seg_chunks, warm_tokens) ||
        !offset_bytes)
        return -1;
    const kda::PrefillPlan p = plan_for(T_total, N, H, d_k, d_v, dtype, seg_chunks, warm_tokens);
    *offset_bytes = p.off_flags;
    return p.warm > 0 ? p.nseg_max * H : 0;
}

kda_status_t kda_test_prefill(const void* q, const void* k, const void* v, const void* g_or_z, const float* A,
                              float g_min, const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total,
                              int H, int d_k, int d_v, const float* initial_state, float* final_state, void* o,
                              kda_dtype_t dtype, void* workspace, size_t workspace_bytes, int ckpt_interval,
                              float* ckpt_states, int64_t ckpt_capacity, int seg_chunks, int warm_tokens,
                              void* stream)
{
    if (!test_plan_ok(seg_chunks, warm_tokens))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_test_prefill: seg_chunks=%d warm_tokens=%d", seg_chunks,
                    warm_tokens);
    if (ckpt_interval < 0 || ckpt_capacity < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_test_prefill: negative checkpoint interval or capacity");
    if (A && (!std::isfinite(g_min) || !(g_min < 0.f) || g_min < -5.f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_test_prefill: g_min must lie in [-5, 0)");
    return prefill_impl("kda_test_prefill", q, k, v, g_or_z, beta, cu_seqlens, N, T_total, H, d_k, d_v, 64,
                        initial_state, final_state, o, dtype, workspace, workspace_bytes, ckpt_interval, ckpt_states,
                        ckpt_capacity, stream, T_total > 0 ? A : nullptr, g_min, seg_chunks, warm_tokens);
}

size_t kda_backward_workspace_size(int64_t T_total, int N, int H, int d_k, int d_v)
{
    if (T_total < 0 || T_total > int64_t(0x7fffffff) || N < 1 || H < 1 || H > KDA_MAX_HEADS || !dim_ok(d_k) ||
        !dim_ok(d_v))
        return 0;
    return kda::backward_plan(T_total, N, H, d_k, d_v).bytes;
}

// ---- plan descriptions (host only)
static int64_t emit_text(const std::string& text, char* buf, size_t cap)
{
    if (buf && cap > 0) {
        const size_t n = text.size() < cap - 1 ? text.size() : cap - 1;
        memcpy(buf, text.data(), n);
        buf[n] = '\0';
    }
    return int64_t(text.size());
}

int64_t kda_describe_prefill_plan(int64_t T_total, int N, int H, int d_k, int d_v, kda_dtype_t dtype, int packed,
                                  char* buf, size_t cap)
{
    if (!prefill_shape_ok(T_total, N, H, d_k, d_v, 64, dtype) || (!packed && N != 1) || (!buf && cap > 0)) return -1;
    if (serial_path(d_k, d_v, dtype)) {
        const kda::PrefillPlan p = kda::serial_plan(T_total, N, H, d_k, d_v);
        char head[512];
        snprintf(head, sizeof(head),
                 "kda_prefill plan: T_total=%lld N=%d H=%d d_k=%d d_v=%d dtype=f32%s\n"
                 "token-serial fp32 path (no chunk kernel for this fp32 head shape)\n"
                 "segments: %d chunks of 64 tokens (%lld tokens) each; at most %lld segments\n"
                 "warm-up window: %d tokens\nworkspace: %zu bytes\n",
                 (long long)T_total, N, H, d_k, d_v, packed ? " (packed, cu_seqlens given)" : "", p.seg_chunks,
                 (long long)p.seg_chunks * 64, (long long)p.nseg_max, p.warm, p.workspace_bytes);
        std::string text = head;
        kda::describe_serial(p, N, H, d_k, d_v, packed != 0, text);
        return emit_text(text, buf, cap);
    }
    const kda::PrefillPlan p = kda::prefill_plan(T_total, N, H, d_k, d_v);
    char head[512];
    snprintf(head, sizeof(head),
             "kda_prefill plan: T_total=%lld N=%d H=%d d_k=%d d_v=%d dtype=%s%s\n"
             "segments: %d chunks of 64 tokens (%lld tokens) each; at most %lld segments, %lld of them "
             "non-final\nwarm-up window: %d tokens%s\nworkspace: %zu bytes\n",
             (long long)T_total, N, H, d_k, d_v, dtype == KDA_BF16 ? "bf16" : "f32",
             packed ? " (packed, cu_seqlens given)" : "", p.seg_chunks, (long long)p.seg_chunks * 64,
             (long long)p.nseg_max, (long long)p.np1_max, p.warm,
             p.warm > 0 ? "" : " (none: the exact passes run for every chain)", p.workspace_bytes);
    std::string text = head;
    const bool ok = dtype == KDA_BF16 ? kda::describe_prefill<kda::BF16>(p, N, H, d_k, d_v, packed != 0, text)
                                      : kda::describe_prefill<kda::F32>(p, N, H, d_k, d_v, packed != 0, text);
    if (!ok) return -1;
    return emit_text(text, buf, cap);
}

int64_t kda_describe_backward_plan(int64_t T_total, int N, int H, int d_k, int d_v, kda_dtype_t dtype, char* buf,
                                   size_t cap)
{
    if (T_total < 0 || T_total > int64_t(0x7fffffff) || N < 1 || H < 1 || H > KDA_MAX_HEADS || !dim_ok(d_k) ||
        !dim_ok(d_v) || !dtype_ok(dtype) || (!buf && cap > 0))
        return -1;
    const kda::BwdPlan p = kda::backward_plan(T_total, N, H, d_k, d_v);
    char head[512];
    snprintf(head, sizeof(head),
             "kda_backward plan: T_total=%lld N=%d H=%d d_k=%d d_v=%d dtype=%s\n"
             "segments: %lld tokens each; at most %lld segments; window %lld tokens; full pass %d workgroups\n"
             "workspace: %zu bytes\n",
             (long long)T_total, N, H, d_k, d_v, dtype == KDA_BF16 ? "bf16" : "f32", (long long)p.Lseg,
             (long long)p.segs_max, (long long)p.warm, p.grid, p.bytes);
    std::string text = head;
    const bool ok = dtype == KDA_BF16 ? kda::describe_backward<kda::BF16>(p, T_total, N, H, d_k, d_v, text)
                                      : kda::describe_backward<kda::F32>(p, T_total, N, H, d_k, d_v, text);
    if (!ok) return -1;
    return emit_text(text, buf, cap);
}

// seg_tokens > 0 fixes the segment length (the test entry point only)
static kda_status_t backward_impl(const char* who, const void* q, const void* k, const void* v, const void* g,
                                  const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total, int H,
                                  int d_k, int d_v, const float* initial_state, const float* ckpt_states,
                                  int64_t ckpt_capacity, int ckpt_interval, const void* d_o,
                                  const float* d_final_state, float* dq, float* dk, float* dv, float* dg,
                                  float* dbeta, float* d_initial_state, kda_dtype_t dtype, void* workspace,
                                  size_t workspace_bytes, void* stream, int64_t seg_tokens,
                                  int64_t warm_tokens = -1)
{
    if (N < 1 || T_total < 0 || H < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: bad sizes N=%d T_total=%lld H=%d", who, N, (long long)T_total, H);
    if (H > KDA_MAX_HEADS) return fail(KDA_ERR_UNSUPPORTED, "%s: H=%d > %d", who, H, KDA_MAX_HEADS);
    if (T_total > int64_t(0x7fffffff)) return fail(KDA_ERR_UNSUPPORTED, "%s: T_total > 2^31 - 1", who);
    if (!cu_seqlens && N != 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is NULL but N=%d", who, N);
    if (!dtype_ok(dtype)) return fail(KDA_ERR_UNSUPPORTED, "%s: unknown dtype %d", who, (int)dtype);
    if (!dim_ok(d_k) || !dim_ok(d_v))
        return fail(KDA_ERR_UNSUPPORTED, "%s: d_k=%d d_v=%d not in {32,64,128}", who, d_k, d_v);
    if (T_total > 0 && (!q || !k || !v || !g || !beta || !dq || !dk || !dv || !dg || !dbeta))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null token tensor", who);
    if (!d_initial_state) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null d_initial_state", who);
    if (ckpt_capacity < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: negative checkpoint capacity", who);
    const bool have_ck = ckpt_states && ckpt_capacity > 0;
    if (have_ck && (ckpt_interval <= 0 || ckpt_interval % kda::BWD_CHUNK != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: checkpoint interval %d is not a positive multiple of %d", who,
                    ckpt_interval, kda::BWD_CHUNK);
    // without checkpoints every 64-token chunk rebuilds its state from the
    // sequence start: quadratic in the length, so long inputs are refused
    if (!have_ck && T_total > KDA_BWD_MAX_TOKENS_WITHOUT_CKPT)
        return fail(KDA_ERR_UNSUPPORTED, "%s: %lld tokens without checkpoints (at most %d); pass the forward's "
                    "checkpoints (kda_prefill_ckpt or kda_prefill_gated, interval 64 for the fast path)", who,
                    (long long)T_total, KDA_BWD_MAX_TOKENS_WITHOUT_CKPT);
    const kda::BwdPlan plan = kda::backward_plan(T_total, N, H, d_k, d_v, seg_tokens, warm_tokens);
    const size_t need = plan.bytes;
    if (!workspace || workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < %zu needed", who, workspace_bytes, need);
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (!al16(initial_state) || !al16(ckpt_states) || !al16(d_final_state) || !al16(d_initial_state) ||
        !al16(dv) || !al16(workspace))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: states, dv and the workspace must be 16-byte aligned", who);
    const size_t es = dsize(dtype), T = size_t(T_total);
    const size_t nk = T * H * d_k * es, nv = T * H * d_v * es, nb = T * H * es;
    const size_t ns = size_t(N) * H * d_k * d_v * sizeof(float);
    const size_t nck = ckpt_states ? size_t(ckpt_capacity) * H * d_k * d_v * sizeof(float) : 0;
    const void* ins[9] = {q, k, v, g, beta, initial_state, ckpt_states, d_o, d_final_state};
    const size_t insz[9] = {nk, nk, nv, nk, nb, initial_state ? ns : 0, nck, d_o ? nv : 0, d_final_state ? ns : 0};
    void* outs[7] = {dq, dk, dv, dg, dbeta, d_initial_state, workspace};
    const size_t fk = T * H * d_k * sizeof(float);
    const size_t outsz[7] = {fk, fk, T * H * d_v * sizeof(float), fk, T * H * sizeof(float), ns, need};
    for (int i = 0; i < 7; ++i) {
        for (int j = 0; j < 9; ++j)
            if (overlap(outs[i], outsz[i], ins[j], insz[j]))
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s: an output overlaps an input", who);
        for (int j = i + 1; j < 7; ++j)
            if (overlap(outs[i], outsz[i], outs[j], outsz[j]))
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s: two outputs overlap", who);
    }
    kda::BackwardArgs a{q, k, v, g, beta, cu_seqlens, N, T_total, H, initial_state,
                        have_ck ? ckpt_states : nullptr, have_ck ? ckpt_capacity : 0,
                        have_ck ? int64_t(ckpt_interval) : int64_t(kda::BWD_CHUNK), d_o, d_final_state,
                        dq, dk, dv, dg, dbeta, d_initial_state, static_cast<float*>(workspace), 0, nullptr,
                        nullptr};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == KDA_BF16 ? kda::launch_backward<kda::BF16>(a, plan, d_k, d_v, s)
                                           : kda::launch_backward<kda::F32>(a, plan, d_k, d_v, s);
    return from_hip(e, "kda_backward launch");
}

kda_status_t kda_backward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const int32_t* cu_seqlens, int N, int64_t T_total, int H, int d_k, int d_v,
                          const float* initial_state, const float* ckpt_states, int64_t ckpt_capacity,
                          int ckpt_interval, const void* d_o, const float* d_final_state, float* dq, float* dk,
                          float* dv, float* dg, float* dbeta, float* d_initial_state, kda_dtype_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream)
{
    return backward_impl("kda_backward", q, k, v, g, beta, cu_seqlens, N, T_total, H, d_k, d_v, initial_state,
                         ckpt_states, ckpt_capacity, ckpt_interval, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                         d_initial_state, dtype, workspace, workspace_bytes, stream, 0);
}

size_t kda_test_backward_workspace_size(int64_t T_total, int N, int H, int d_k, int d_v, int64_t seg_tokens)
{
    if (seg_tokens < 0 || T_total < 0 || T_total > int64_t(0x7fffffff) || N < 1 || H < 1 || H > KDA_MAX_HEADS ||
        !dim_ok(d_k) || !dim_ok(d_v))
        return 0;
    return kda::backward_plan(T_total, N, H, d_k, d_v, seg_tokens).bytes;
}

kda_status_t kda_test_backward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                               const int32_t* cu_seqlens, int N, int64_t T_total, int H, int d_k, int d_v,
                               const float* initial_state, const float* ckpt_states, int64_t ckpt_capacity,
                               int ckpt_interval, const void* d_o, const float* d_final_state, float* dq, float* dk,
                               float* dv, float* dg, float* dbeta, float* d_initial_state, kda_dtype_t dtype,
                               void* workspace, size_t workspace_bytes, int64_t seg_tokens, int64_t warm_tokens,
                               void* stream)
{
    if (seg_tokens < 0 || warm_tokens < -1 || (warm_tokens > 0 && warm_tokens % 16 != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_test_backward: seg_tokens=%lld warm_tokens=%lld",
                    (long long)seg_tokens, (long long)warm_tokens);
    return backward_impl("kda_test_backward", q, k, v, g, beta, cu_seqlens, N, T_total, H, d_k, d_v, initial_state,
                         ckpt_states, ckpt_capacity, ckpt_interval, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                         d_initial_state, dtype, workspace, workspace_bytes, stream, seg_tokens, warm_tokens);
}

int64_t kda_checkpoint_count(const int32_t* cu_seqlens_host, int N, int64_t T_total, int ckpt_interval)
{
    if (N < 1 || T_total < 0 || ckpt_interval <= 0) return -1;
    int64_t total = 0, prev = 0;
    for (int n = 0; n < N; ++n) {
        int64_t x = cu_seqlens_host ? int64_t(cu_seqlens_host[n + 1]) : T_total;
        x = x < 0 ? 0 : (x > T_total ? T_total : x);
        if (x < prev) x = prev;  // the same clamping the device planner applies
        total += (x - prev) / ckpt_interval;
        prev = x;
    }
    return total;
}

}  // extern "C"

#ifdef KDA_DEVICE_CHECKS
// The device-side check bits of the checked build (see include/kda.h).
extern "C" kda_status_t kda_debug_check_bits(unsigned int* bits, int reset)
{
    if (!bits) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_debug_check_bits: null pointer");
    hipError_t e = hipMemcpyFromSymbol(bits, HIP_SYMBOL(kda::kda_check_bits), sizeof(unsigned int), 0,
                                       hipMemcpyDeviceToHost);
    if (e == hipSuccess && reset) {
        const unsigned int zero = 0;
        e = hipMemcpyToSymbol(HIP_SYMBOL(kda::kda_check_bits), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
    }
    return from_hip(e, "kda_debug_check_bits");
}
#endif

#ifdef KDA_PHASE_TIMING
// Copy the per-workgroup phase cycle counters of the last chunk-kernel launch.
extern "C" int kda_phase_cycles_read(unsigned long long* host, int n)
{
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(kda::kda_phase_cycles),
                                    sizeof(unsigned long long) * size_t(n), 0, hipMemcpyDeviceToHost);
}
#endif
