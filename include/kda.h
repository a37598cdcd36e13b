/*
 * libkda — Kimi Delta Attention (KDA) forward pass on AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *   [K3-notes]  "NLP——技术报告解读-Kimi-K3" (joezjh.github.io),
 *               Model Architecture / Kimi Delta Attention (KDA):
 *                 S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *                 o_t = S_t^T q_t,   alpha_t = exp(g_t) in (0, 1]^{d_k},
 *                 g_t^h = g_min * Sigmoid(exp(A_h) * z_t^h),  g_min = -5.
 *               Infrastructure / KDA algorithm-system co-design: chunkwise
 *               kernels for prefill, intra-device context parallelism
 *               (segments of one sequence composed exactly), and the KCP
 *               identity S = S~ + M S_in.
 *   [K3-plain]  "Kimi K3 技术报告 · 大白话版" (aicoding.csdn.net), §2.1.1
 *               (decay, then delta correction, then read; at most 99.33%
 *               forgotten per step) and §5.4 (the decode state is updated in
 *               place token by token).
 *   [LateTalk]  "详解Kimi K3：强到冲击Anthropic估值的模型什么样？"
 *               (latetalk.qiaomu.ai), section on the hybrid 3:1 layout: the
 *               recurrent state has a fixed size and is overwritten by every
 *               token.
 *
 * Conventions for every call:
 *   - All tensor arguments are DEVICE pointers (memory of the current HIP
 *     device), row-major, densely packed, owned by the caller.  The library
 *     allocates no device memory, creates no streams or events and keeps no
 *     state between calls: everything a call needs is in its arguments.
 *     Everything a call enqueues goes onto `stream`, in order.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work and return; completion and asynchronous HIP
 *     faults are observed by the caller synchronising the stream.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns an error status and enqueues nothing.
 *     kda_last_error() then describes the failure (thread-local string).
 *   - dtype selects the storage type of the token tensors (q, k, v, g, z,
 *     beta, o).  States are always fp32.  Arithmetic is fp32 with fp32
 *     accumulation; bf16 tensors feed the matrix cores as bf16.
 *   - The library does not normalise q or k, does not scale q, and applies
 *     no output gate: it returns o_t exactly as defined above.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums are int-sized with every int value representable (the two
 * range enumerators are never returned or accepted), so a caller may pass any
 * int: the library rejects the ones it does not know. */
typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,    /* null pointer, negative size, bad cu_seqlens ... */
    KDA_ERR_UNSUPPORTED = 2,         /* a dimension / dtype / chunk outside the built set */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3, /* prefill workspace smaller than the queried size */
    KDA_ERR_HIP = 4,                 /* a HIP runtime call or launch failed */
    KDA_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
    KDA_STATUS_RANGE_MAX_ = 0x7fffffff
} kda_status_t;

typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1,
    KDA_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
    KDA_DTYPE_RANGE_MAX_ = 0x7fffffff
} kda_dtype_t;

/* Largest head count kda_prefill accepts (token rows stay below 2^24 bytes). */
#define KDA_MAX_HEADS 16384

/* Human-readable name of a status code (static string). */
const char* kda_status_string(kda_status_t s);

/* Description of the most recent failure on the calling thread ("" if none). */
const char* kda_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int kda_version(void);

/*
 * kda_gate — the lower-bounded log-decay gate ([K3-notes], KDA, lower-bounded
 * decay; [K3-plain] §2.1.1):
 *     g[t,h,c] = g_min * sigmoid(exp(A[h]) * z[t,h,c])
 * z, g : [n_tokens, H, d_k] in `dtype` (g may alias z: in-place is allowed).
 * A    : [H] fp32 device pointer.
 * g_min: the lower bound, in [-5, 0) (the pages use -5).  kda_prefill and
 *        kda_backward need every g >= -5 (they factor decay ratios per
 *        16-token sub-tile and keep each factor inside the fp32 range), so a
 *        lower bound below -5 is refused.
 * Computed in fp32 and rounded once to dtype.  n_tokens == 0 is a no-op.
 * Errors: KDA_ERR_INVALID_ARGUMENT for null pointers / negative sizes / bad
 * g_min, KDA_ERR_UNSUPPORTED for an unknown dtype, KDA_ERR_HIP on launch failure.
 */
kda_status_t kda_gate(const void* z, const float* A, void* g, int64_t n_tokens, int H,
                      int d_k, kda_dtype_t dtype, float g_min, void* stream);

/*
 * Workspace bytes kda_prefill needs for this problem shape (0 on invalid
 * arguments).  The value depends only on the arguments listed.
 */
size_t kda_prefill_workspace_size(int64_t T_total, int N, int H, int d_k, int d_v, int chunk,
                                  kda_dtype_t dtype);

/*
 * kda_prefill — chunkwise KDA forward over packed sequences ([K3-notes], KDA
 * recurrence; Infrastructure: chunkwise kernel, intra-device CP, KCP).
 *   q, k, g : [T_total, H, d_k]   (g = log-decay, as produced by kda_gate)
 *   v, o    : [T_total, H, d_v]
 *   beta    : [T_total, H]
 *   all in `dtype`.
 *   cu_seqlens : int32 [N + 1] DEVICE array of token offsets, cu[0] = 0,
 *                non-decreasing, cu[N] = T_total.  NULL means one sequence
 *                (then N must be 1).  Sequences of length 0 are allowed.
 *                The device copy cannot be checked on the host: the kernels
 *                clamp every offset into [0, T_total] so malformed offsets
 *                cannot cause out-of-bounds access, but the results are then
 *                unspecified.
 *   initial_state : fp32 [N, H, d_k, d_v] or NULL (zero initial states).
 *   final_state   : fp32 [N, H, d_k, d_v] or NULL (not written).  May alias
 *                   initial_state exactly (in-place hand-off); no other
 *                   aliasing is allowed between any two buffers.  In place,
 *                   a segment whose warm-up holds may write the final state
 *                   before the passes that compose other segments exactly have
 *                   read the initial state, so the first pass keeps a copy of
 *                   the initial states in the workspace for them.
 *   chunk   : 64, the granularity (in tokens) at which long sequences are
 *             cut into segments; inside a segment the recurrence advances
 *             in blocks of 32 tokens.
 *   H       : 1 .. KDA_MAX_HEADS.
 *   g       : every value in [-5, 0] (the range kda_gate produces); the
 *             kernels factor decay ratios per 16-token sub-tile and rely on
 *             this bound to keep every factor inside the fp32 range.
 *   d_k, d_v: each one of 32, 64, 128, for both dtypes.  fp32 heads with
 *             d_k = 32 and d_v <= 64 take the chunk kernels; the other fp32
 *             shapes (whose fp32 operand tiles do not fit one CU's LDS) run
 *             token by token in fp32 with the state in registers, in the
 *             same segments and warm-up windows as the chunk kernels (chains
 *             whose windows fail are rerun from their start, token by
 *             token); the same results, about ten times the bf16 time.
 *   workspace : device buffer of at least kda_prefill_workspace_size(...) bytes
 *               (may be NULL when that size is 0); its contents on entry do
 *               not matter and are clobbered.
 * Chunks restart at every sequence start; the last chunk of a sequence may be
 * short.  Long sequences are split into segments that run in parallel.  For
 * d_k <= d_v each segment takes its incoming state from the 128 tokens before
 * it, run from a zero state beside their transition M: once the computed M is
 * exactly zero (all its entries underflow, as they do within about a hundred
 * tokens under the bounded decay) the incoming state is the window's state.
 * Chains (sequence, head) where M is not zero, and every chain when d_k > d_v,
 * are composed exactly through S_end = S~ + M S_in (summary pass, scan,
 * output pass).  Both routes enqueue the same launches on `stream`; the second
 * route's kernels end at once for chains that do not need them.
 * Errors: KDA_ERR_INVALID_ARGUMENT (null required pointer, N < 1, T_total < 0,
 * N != 1 without cu_seqlens, forbidden aliasing), KDA_ERR_UNSUPPORTED (d_k,
 * d_v, chunk, H or dtype outside the supported set, T_total > 2^31 - 1:
 * token offsets are int32 like cu_seqlens),
 * KDA_ERR_WORKSPACE_TOO_SMALL, KDA_ERR_HIP.
 */
kda_status_t kda_prefill(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total,
                         int H, int d_k, int d_v, int chunk, const float* initial_state,
                         float* final_state, void* o, kda_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * kda_prefill_ckpt — kda_prefill that also emits state checkpoints for a
 * prefix cache ([K3-notes] Infrastructure / 推理与在线服务, KDA-aware prefix
 * cache: hashes over 512-token blocks; KDA states kept only at sparse
 * boundaries, so a hit can sit at any multiple of the block size).
 * Every argument of kda_prefill, plus:
 *   ckpt_interval : tokens between checkpoints, a positive multiple of 64
 *                   (512 matches the pages' block).
 *   ckpt_states   : fp32 [ckpt_capacity, H, d_k, d_v] DEVICE buffer.  For
 *                   sequence n of length len_n the state after its first
 *                   j * ckpt_interval tokens (j = 1 .. len_n / ckpt_interval)
 *                   goes to row ckpt_off[n] + j - 1, with ckpt_off the running
 *                   sum of len_m / ckpt_interval over the sequences m < n
 *                   (lengths as clamped by the planner; see kda_prefill).
 *   ckpt_capacity : rows the buffer holds; checkpoints past it are skipped.
 *                   kda_checkpoint_count gives the number needed.
 * Errors: as kda_prefill, plus KDA_ERR_INVALID_ARGUMENT for a bad interval,
 * a null buffer with a positive capacity, or a buffer overlapping another.
 */
kda_status_t kda_prefill_ckpt(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total,
                              int H, int d_k, int d_v, int chunk, const float* initial_state,
                              float* final_state, void* o, kda_dtype_t dtype, void* workspace,
                              size_t workspace_bytes, int ckpt_interval, float* ckpt_states,
                              int64_t ckpt_capacity, void* stream);

/*
 * kda_prefill_gated — kda_prefill whose decay comes straight from the gate's
 * input: g = g_min * sigmoid(exp(A[h]) * z) ("NLP——技术报告解读-Kimi-K3",
 * Model Architecture / Kimi Delta Attention (KDA), lower-bounded decay; the
 * same map as kda_gate) is computed in fp32 inside the prefill's decay stage
 * and never written out, so one call covers the gate and the prefill.
 * Arguments as kda_prefill and kda_prefill_ckpt, except:
 *   z      : [T_total, H, d_k] DEVICE, the input dtype (in place of g).
 *   A      : fp32 [H] DEVICE, read only (may be NULL when T_total = 0).
 *   g_min  : in [-5, 0) (-5 on the pages); the block kernels bound every decay
 *            factor through g >= -5.
 *   ckpt_interval : 0 for no checkpoints, else as in kda_prefill_ckpt.
 * Results equal kda_gate followed by kda_prefill up to the rounding of g to
 * the input dtype, which this path skips.
 * Errors: as kda_prefill_ckpt, plus KDA_ERR_INVALID_ARGUMENT for a null A, a
 * g_min outside [-5, 0), or A overlapping an output buffer.
 */
kda_status_t kda_prefill_gated(const void* q, const void* k, const void* v, const void* z, const float* A,
                               float g_min, const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total,
                               int H, int d_k, int d_v, int chunk, const float* initial_state, float* final_state,
                               void* o, kda_dtype_t dtype, void* workspace, size_t workspace_bytes,
                               int ckpt_interval, float* ckpt_states, int64_t ckpt_capacity, void* stream);

/* Bytes of the static scratch kda_prefill_gated_noalloc takes its workspace from. */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * kda_prefill_gated_noalloc — kda_prefill_gated without a workspace argument,
 * for callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation).  It takes its
 * workspace from a static device array of KDA_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (its device
 * address is looked up on the first call on each device), and calls no
 * allocating routine.  Arguments, results and errors are those of
 * kda_prefill_gated, plus KDA_ERR_UNSUPPORTED when the call would need more
 * workspace than the scratch holds (kda_prefill_workspace_size gives the
 * amount; a single sequence at d_k = d_v = 128 needs about 50 MB at most).
 * Every call on a GPU shares that GPU's scratch, which keeps the last call's
 * contents (nothing in it must start at zero): calls that overlap in time on
 * one GPU, on different streams or threads, race and give wrong results;
 * serialize them.
 */
kda_status_t kda_prefill_gated_noalloc(const void* q, const void* k, const void* v, const void* z, const float* A,
                                       float g_min, const void* beta, const int32_t* cu_seqlens, int N,
                                       int64_t T_total, int H, int d_k, int d_v, int chunk,
                                       const float* initial_state, float* final_state, void* o, kda_dtype_t dtype,
                                       int ckpt_interval, float* ckpt_states, int64_t ckpt_capacity, void* stream);

/*
 * Plan descriptions — what kda_prefill (and its gated and checkpointing
 * forms, which plan alike) and kda_backward would launch for these sizes, as
 * text: the segment length, the warm-up window, the workspace bytes and one
 * line per kernel launch with its grid, workgroup size, LDS bytes and role.
 * Host only: no device call, no state; the plan depends only on the
 * arguments.  packed: cu_seqlens will be given (it must be when N > 1).
 * Writes at most cap bytes including the terminating NUL into buf (buf may
 * be NULL when cap is 0) and returns the length of the whole description,
 * as snprintf does; -1 for a shape the call would reject.
 */
int64_t kda_describe_prefill_plan(int64_t T_total, int N, int H, int d_k, int d_v, kda_dtype_t dtype, int packed,
                                  char* buf, size_t cap);
int64_t kda_describe_backward_plan(int64_t T_total, int N, int H, int d_k, int d_v, kda_dtype_t dtype, char* buf,
                                   size_t cap);

/*
 * TEST ONLY — the prefill with the planner's two choices given as arguments,
 * so tests can force segment boundaries and either route (kda_prefill).
 *   g_or_z, A   : with A NULL, g_or_z is the log-decay g (as kda_prefill);
 *                 else it is the gate's input z (as kda_prefill_gated, with
 *                 g_min in [-5, 0)).
 *   seg_chunks  : segment length in 64-token chunks, or 0 for the planner's.
 *   warm_tokens : the warm-up window before each segment, a positive multiple
 *                 of 32 tokens; 0 = no warm-up (every chain through the
 *                 summary pass, scan and output pass); -1 = the planner's.
 * Other arguments as kda_prefill_gated; chunk is 64.  The workspace size for
 * the same choices is kda_test_prefill_workspace_size (0 on bad arguments).
 * kda_test_prefill_flags returns how many int32 warm-up flags ([segments][H],
 * 1 = that segment's window left M non-zero, so its chain went through the
 * exact passes) the workspace holds, and at *offset_bytes where; 0 without a
 * warm-up pass, -1 on bad arguments.  Only rows of real segments are written.
 */
kda_status_t kda_test_prefill(const void* q, const void* k, const void* v, const void* g_or_z, const float* A,
                              float g_min, const void* beta, const int32_t* cu_seqlens, int N, int64_t T_total,
                              int H, int d_k, int d_v, const float* initial_state, float* final_state, void* o,
                              kda_dtype_t dtype, void* workspace, size_t workspace_bytes, int ckpt_interval,
                              float* ckpt_states, int64_t ckpt_capacity, int seg_chunks, int warm_tokens,
                              void* stream);
size_t kda_test_prefill_workspace_size(int64_t T_total, int N, int H, int d_k, int d_v, kda_dtype_t dtype,
                                       int seg_chunks, int warm_tokens);
int64_t kda_test_prefill_flags(int64_t T_total, int N, int H, int d_k, int d_v, kda_dtype_t dtype, int seg_chunks,
                               int warm_tokens, size_t* offset_bytes);

/*
 * kda_backward — gradients for training ([K3-notes] Model Architecture / KDA:
 * the state update and read-out, differentiated; Infrastructure / KDA
 * algorithm-system co-design: FlashKDA serves training as well as inference).
 * For the loss L = sum_t <d_o[t], o[t]> + <d_final_state, S_T> of the prefill
 * with the same arguments (kda_prefill), returns, all fp32:
 *   dq, dk, dg : [T_total, H, d_k]   dv : [T_total, H, d_v]   dbeta : [T_total, H]
 *   d_initial_state : [N, H, d_k, d_v]
 * Inputs as kda_prefill (q, k, v, g, beta in `dtype`; g is the log-decay), plus:
 *   d_o            : [T_total, H, d_v] (dtype) or NULL (no output gradient).
 *   d_final_state  : fp32 [N, H, d_k, d_v] or NULL (zero).
 *   initial_state  : the forward's, or NULL (zero).
 *   ckpt_states    : the forward's checkpoints (kda_prefill_ckpt or
 *                    kda_prefill_gated with the same inputs and initial state)
 *                    at ckpt_interval tokens, ckpt_capacity rows, laid out as
 *                    kda_prefill_ckpt writes them; may be NULL.  Each 64-token
 *                    chunk rebuilds its forward state from the nearest
 *                    checkpoint at or before its start that the buffer holds
 *                    (interval 64: the chunk's own row, nothing to rebuild),
 *                    else from the initial state.  Without checkpoints that
 *                    rebuild is quadratic in the sequence length, so T_total
 *                    is then limited to KDA_BWD_MAX_TOKENS_WITHOUT_CKPT.
 *   ckpt_interval  : a positive multiple of 64 when ckpt_states is given
 *                    (ignored otherwise).
 *   workspace      : at least kda_backward_workspace_size(T_total, N, H, d_k,
 *                    d_v) bytes: per workgroup slot, the states at the four
 *                    16-token sub-chunk starts of a 64-token chunk (in up to
 *                    two layouts) and one staging state; per (segment, head) the segment's
 *                    gradient summary, its end-of-segment state gradient and
 *                    a flag (segments of a sequence run in parallel).
 * Segments of one sequence run in parallel.  Each takes the state gradient at
 * its end from the 128 tokens after it, run backwards from zero beside the
 * window's transposed transition; where that transition is not exactly zero
 * (slow decay), the chain's segments are composed exactly through a summary
 * pass and a scan instead, whose launches end at once for the other chains.
 * The products run on the matrix cores with operands in `dtype` (bf16
 * operands and fp32 accumulation for KDA_BF16, as in the prefill).
 * State buffers, dv and the workspace must be 16-byte aligned; no output may
 * overlap an input or another output.  d_k, d_v each one of 32, 64, 128.
 * The gradient with respect to z and A of the gate follows from dg by the
 * chain rule of kda_gate's formula and is left to the caller.
 * Errors: KDA_ERR_INVALID_ARGUMENT (also a bad ckpt_interval with
 * checkpoints), KDA_ERR_UNSUPPORTED (also T_total above
 * KDA_BWD_MAX_TOKENS_WITHOUT_CKPT without checkpoints),
 * KDA_ERR_WORKSPACE_TOO_SMALL, KDA_ERR_HIP.
 */
#define KDA_BWD_MAX_TOKENS_WITHOUT_CKPT 4096
size_t kda_backward_workspace_size(int64_t T_total, int N, int H, int d_k, int d_v);
kda_status_t kda_backward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const int32_t* cu_seqlens, int N, int64_t T_total, int H, int d_k, int d_v,
                          const float* initial_state, const float* ckpt_states, int64_t ckpt_capacity,
                          int ckpt_interval, const void* d_o, const float* d_final_state, float* dq, float* dk,
                          float* dv, float* dg, float* dbeta, float* d_initial_state, kda_dtype_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * TEST ONLY — kda_backward with the planner's two choices given: seg_tokens >
 * 0 cuts every sequence into segments of that many tokens (rounded up to whole
 * 64-token chunks), 0 takes the planner's; warm_tokens is the window after each
 * segment that gives its end-of-segment state gradient (a positive multiple of
 * 16), 0 sends every chain through the summary pass and the scan, -1 takes the
 * planner's.  kda_test_backward_workspace_size is the workspace for the same
 * segment length (it does not depend on the window).
 */
kda_status_t kda_test_backward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                               const int32_t* cu_seqlens, int N, int64_t T_total, int H, int d_k, int d_v,
                               const float* initial_state, const float* ckpt_states, int64_t ckpt_capacity,
                               int ckpt_interval, const void* d_o, const float* d_final_state, float* dq, float* dk,
                               float* dv, float* dg, float* dbeta, float* d_initial_state, kda_dtype_t dtype,
                               void* workspace, size_t workspace_bytes, int64_t seg_tokens, int64_t warm_tokens,
                               void* stream);
size_t kda_test_backward_workspace_size(int64_t T_total, int N, int H, int d_k, int d_v, int64_t seg_tokens);

/*
 * Number of checkpoints kda_prefill_ckpt writes for these HOST cu_seqlens
 * (NULL: one sequence of T_total tokens), with the planner's clamping; -1 on
 * invalid arguments (N < 1, T_total < 0, ckpt_interval <= 0).  Host only.
 */
int64_t kda_checkpoint_count(const int32_t* cu_seqlens_host, int N, int64_t T_total, int ckpt_interval);

/*
 * kda_decode_step — one token per sequence against a resident fp32 state,
 * updated IN PLACE ([K3-notes] KDA recurrence; [K3-plain] §5.4; [LateTalk]
 * fixed-size state overwritten by every token):
 *     S <- (I - beta k k^T) Diag(exp(g)) S + beta k v^T ;   o = S^T q
 *   q, k, g : [B, H, d_k]   v, o : [B, H, d_v]   beta : [B, H]   (dtype)
 *   state   : fp32 [B, H, d_k, d_v], read and overwritten.
 *   d_k, d_v: each one of 32, 64, 128.  B == 0 is a no-op.
 * `o` must not alias any input or the state.
 * Errors: KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP.
 */
kda_status_t kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, float* state, void* o, int B, int H, int d_k,
                             int d_v, kda_dtype_t dtype, void* stream);

/*
 * kda_decode_step_gated — kda_decode_step taking the gate's input: the decay
 * is g = g_min * sigmoid(exp(A[h]) * z) ([K3-notes] KDA, lower-bounded decay;
 * the map kda_gate computes), evaluated in fp32 inside the step, so one call
 * covers the gate and the decode step.
 *   z     : [B, H, d_k] (dtype), in place of g.
 *   A     : fp32 [H] DEVICE, read only (may be NULL when B == 0).
 *   g_min : finite and negative (-5 on the pages).
 * Other arguments as kda_decode_step.  Results equal kda_gate followed by
 * kda_decode_step up to the rounding of g to the input dtype, which this path
 * skips.
 * Errors: as kda_decode_step, plus KDA_ERR_INVALID_ARGUMENT for a null A, a
 * bad g_min, or A overlapping o or the state.
 */
kda_status_t kda_decode_step_gated(const void* q, const void* k, const void* v, const void* z, const float* A,
                                   float g_min, const void* beta, float* state, void* o, int B, int H, int d_k,
                                   int d_v, kda_dtype_t dtype, void* stream);

/* Largest number of draft tokens per sequence kda_verify / kda_commit accept. */
#define KDA_MAX_DRAFT 64

/*
 * kda_verify — speculative multi-token decode: K draft tokens per sequence run
 * through the recurrence from the resident state, which is NOT modified
 * ([K3-notes] Infrastructure / 推理与在线服务, KDA decoding under MTP
 * speculative decoding: cache the projected inputs, not states; [K3-plain]
 * §5.4: a wrong guess cannot be undone on an in-place state, so inputs are
 * kept and replayed; [LateTalk] section 先分后合，和一条没有开源的流水线).
 *   q, k, g : [B, K, H, d_k]   v, o : [B, K, H, d_v]   beta : [B, K, H]  (dtype)
 *   state   : fp32 [B, H, d_k, d_v], read only.
 *   o[b, i] is what kda_decode_step would return for draft token i after the
 *   tokens 0..i-1 of the same sequence.
 *   1 <= K <= KDA_MAX_DRAFT; d_k, d_v each one of 32, 64, 128; B == 0 is a no-op.
 *   The caller keeps q, k, v, g, beta (the projected inputs) for kda_commit.
 * `o` must not alias any input or the state.
 * Errors: KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP.
 */
kda_status_t kda_verify(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        const float* state, void* o, int B, int K, int H, int d_k, int d_v,
                        kda_dtype_t dtype, void* stream);

/*
 * kda_commit — roll forward by replay: the first n_accept[b] of the K cached
 * draft tokens of sequence b (the tensors passed to kda_verify) are applied to
 * the state IN PLACE; the rejected rest leave no trace.  Same sources as
 * kda_verify.
 *   k, g : [B, K, H, d_k]   v : [B, K, H, d_v]   beta : [B, K, H]  (dtype)
 *   n_accept : int32 [B] DEVICE array; each value is clamped to [0, K]
 *              (0 leaves that sequence's state untouched).
 *   state    : fp32 [B, H, d_k, d_v], read and overwritten.
 *   No output is written (the outputs of accepted tokens are those kda_verify
 *   returned).  Sizes as for kda_verify.
 * Errors: KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP.
 */
kda_status_t kda_commit(const void* k, const void* v, const void* g, const void* beta,
                        const int32_t* n_accept, float* state, int B, int K, int H, int d_k, int d_v,
                        kda_dtype_t dtype, void* stream);

/*
 * kda_debug_check_bits — exported only by the checked build of the library
 * (libkda_checked.so, compiled with -DKDA_DEVICE_CHECKS; a debugging aid, not
 * a method step).  In that build every kernel checks, where it sets up its
 * work item, that the token ranges, sequence and state indices, workspace
 * indices, checkpoint rows and block lengths its accesses are derived from
 * lie inside the buffers' extents, and sets one bit per kind of failure in a
 * device word (bit 0 token range, 1 sequence or state index, 2 workspace
 * index, 3 checkpoint row, 4 block length); kernels carry on either way.
 *   bits  : host pointer; receives the word of the current device.  The call
 *           synchronises with the device (a blocking copy).
 *   reset : non-zero clears the word after reading it.
 * Errors: KDA_ERR_INVALID_ARGUMENT (null bits), KDA_ERR_HIP.
 */
kda_status_t kda_debug_check_bits(unsigned int* bits, int reset);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
