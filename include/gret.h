/*
 * gret.h -- C ABI of libgret, multi-head gated retention (gRet) on AMD gfx950.
 *
 * The method is the Self-Decoder mixer described on the page
 * "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次":
 *   section "路线二：Multi-Head Gated Retention" -- per head, a dk x dv matrix
 *     state is scaled by one data-dependent scalar gate per position and
 *     receives the key/value outer product; the output is the query times the
 *     updated state:  S_n = g_n S_{n-1} + k_n^T v_n,  o_n = q_n S_n;
 *   section "Prefill 与 Decode 为什么使用两种计算形态" -- prompts are processed
 *     in the chunkwise form (decayed causal attention inside a chunk, the
 *     carried state for everything before it), decode steps in the recurrent
 *     form; both are the same formula, the chunk size is only a tuning knob;
 *   section "Prefill 的实现骨架" -- a prompt that is not a multiple of the chunk
 *     size is masked at its tail, and the state at the end of prefill is kept
 *     for the decode steps that follow;
 *   section "单 token Decode 的实现骨架" -- a decode step multiplies the old
 *     state by the exponential of the gate value and adds the key/value outer
 *     product, which is why this ABI takes the log of the gate.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers. Every tensor pointer is a device pointer owned by the caller. The
 *   library never allocates device memory, never frees or retains a pointer
 *   after the call returns, keeps no global state and is reentrant -- with one
 *   exception, gret_prefill_noalloc, which uses a fixed device array of the
 *   library's own in place of the caller's workspace (see there).
 * Layouts (contiguous, row-major, head-major as [batch, head, position, dim]):
 *   prefill  q, k [B,H,N,dk]; v, out [B,H,N,dv]; log_gamma [B,H,N]
 *   decode   q, k [B,H,dk];   v, out [B,H,dv];   log_gamma [B,H]
 *   state    [B,H,dk,dv], element [i][j] pairs key dim i with value dim j
 * Types. q, k, v and out use `dtype` (GRET_DTYPE_BF16 or GRET_DTYPE_F32);
 *   log_gamma and the state are always fp32. bf16 outputs are rounded to
 *   nearest-even. The bf16 path computes contractions on bf16 matrix cores
 *   with fp32 accumulation and an fp32 state carry; the fp32 path computes
 *   everything in fp32.
 * Gates. log_gamma holds log(gamma) per position; it must lie in [-inf, 0]
 *   (gamma in [0, 1], as the page's sigmoid gate always gives). Kernels clamp
 *   it to [GRET_LOG_GAMMA_FLOOR, 0]; the floor stands in for gamma = 0, whose
 *   log (-inf) would make the chunkwise form compute -inf - (-inf). NaN or
 *   positive values give unspecified (but finite-time, in-bounds) results.
 * Scaling. There is no scale argument: keys are expected to arrive already
 *   multiplied by dk^(-1/2), as the page's implementation does before the
 *   update. There is no position argument: gRet has no positional term.
 * Errors. Arguments are validated synchronously; on any failure the call
 *   returns a nonzero gret_status_t and launches nothing. On success the work
 *   is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *   returns GRET_OK without synchronising. A launch failure is reported as
 *   GRET_ERR_HIP; any HIP error already pending on the calling thread is
 *   cleared before the launch. No C++ exception crosses this ABI.
 */
#ifndef GRET_H
#define GRET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GRET_DTYPE_F32 = 0,
    GRET_DTYPE_BF16 = 1
} gret_dtype_t;

typedef enum {
    GRET_OK = 0,
    GRET_ERR_NULL = 1,        /* a required pointer is NULL                   */
    GRET_ERR_SHAPE = 2,       /* B, H or N < 1, sizes overflow, or a launch
                                 would need more than 2^31 - 1 workgroups
                                 (limits stated per entry point)             */
    GRET_ERR_UNSUPPORTED = 3, /* dk, dv, chunk or dtype outside the set below,
                                 or a tensor pointer not 16-byte aligned      */
    GRET_ERR_ALIAS = 4,       /* out overlaps an input, or states overlap
                                 without being identical                      */
    GRET_ERR_HIP = 5,         /* a HIP runtime call or launch failed          */
    GRET_ERR_WORKSPACE = 6,   /* workspace missing, too small or misaligned   */
    GRET_ERR_VALUE = 7,       /* a scalar argument out of range (eps, scale)  */
    GRET_ERR_SCRATCH = 8      /* gret_prefill_noalloc: the sizes need more than
                                 its fixed device scratch                     */
} gret_status_t;

/* Log-gate floor used in place of -inf (gamma ~ 1.8e-35). */
#define GRET_LOG_GAMMA_FLOOR (-80.0f)

/* Supported head sizes: dk, dv in {64, 128} (any pairing).
   Supported prefill chunk sizes: 64, 128, 256. */

/*
 * gret_prefill_workspace_bytes -- device scratch that gret_prefill needs.
 *
 * Prefill splits each head's sequence into segments that run at the same time
 * and are chained afterwards (the chunkwise form of section "Prefill 与 Decode
 * 为什么使用两种计算形态", applied at two levels). The partial states live in a
 * caller-owned workspace whose size depends only on the arguments below (not
 * on the device). Writes the size to *bytes (0 when none is needed).
 * Returns GRET_OK or a validation error (GRET_ERR_NULL if bytes is NULL).
 */
int gret_prefill_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                                 int64_t chunk, int dtype, size_t* bytes);

/*
 * gret_prefill -- chunkwise gated retention over a whole prompt.
 *
 * For each (b,h): starting from state_in[b,h] (zero when state_in is NULL),
 * computes out[b,h,n,:] = q_n S_n for n = 0..N-1 with
 * S_n = exp(log_gamma[b,h,n]) S_{n-1} + k_n^T v_n, and writes S_{N-1} to
 * state_out[b,h] unless state_out is NULL (sections "路线二：Multi-Head Gated
 * Retention", "Prefill 与 Decode 为什么使用两种计算形态", "Prefill 的实现骨架").
 *
 *   q, k, v, log_gamma  inputs (layouts above), required
 *   state_in            fp32 [B,H,dk,dv] or NULL (zero initial state)
 *   out                 output [B,H,N,dv] in dtype, required; must not overlap
 *                       any input, state_out or the workspace
 *   state_out           fp32 [B,H,dk,dv] or NULL; may be identical to state_in
 *                       (in place); any other overlap is GRET_ERR_ALIAS
 *   B, H, N             >= 1; N need not be a multiple of chunk (the tail chunk
 *                       is masked and state_out is exactly S_{N-1});
 *                       B*H <= 2^27 - 1 (also for the decode step). With dtype
 *                       BF16 the head's length is not limited as such: each
 *                       workgroup addresses the rows of its own piece of a
 *                       head with 32-bit offsets, so ceil(B*H*ceil(N/chunk) /
 *                       G) + 2 chunks (G = the launch's workgroups, one per
 *                       compute unit, at most 1024) must fit 2^31 bytes of
 *                       rows of max(dk, dv) bf16 -- about B*H*N <= 2^31 on a
 *                       256-CU device -- else GRET_ERR_SHAPE (checked after
 *                       the device's CU count is read, before any launch)
 *   dk, dv              64 or 128
 *   chunk               64, 128 or 256 -- the chunk length of the chunkwise form
 *   dtype               gret_dtype_t of q, k, v, out
 *   workspace           device scratch of at least
 *                       gret_prefill_workspace_bytes(...) bytes, 256-byte
 *                       aligned; may be NULL when that size is 0. Its contents
 *                       on entry do not matter; calls that share a workspace
 *                       must be ordered on one stream.
 *   stream              hipStream_t to enqueue on (NULL = null stream)
 */
int gret_prefill(const void* q, const void* k, const void* v, const float* log_gamma,
                 const float* state_in, void* out, float* state_out, int64_t B, int64_t H,
                 int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * gret_prefill_noalloc -- gret_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, semantics and results as gret_prefill,
 * without the workspace: the bf16 path keeps its partial segment states in a
 * device array of GRET_NOALLOC_SCRATCH_BYTES owned by the library, one per GPU,
 * created when the library's code is loaded on that GPU and held until the
 * process ends. The call allocates nothing (no hipMalloc, no allocating
 * library routine); on its first call on a GPU it looks up that GPU's array
 * with hipGetSymbolAddress (the caller's device must be current).
 *
 * Limit: the scratch must hold this device's segment plan, i.e. the number
 * of bytes gret_prefill_workspace_bytes would give for the device's own number
 * of workgroups (one per compute unit) instead of its device-independent cap.
 * At dk = dv = 128 that is 64 KiB per segment; 24 heads of any length need
 * about 19 MB on a 256-CU GPU. Larger requests return GRET_ERR_SCRATCH (before
 * anything is enqueued, after a device-attribute query). fp32 calls need no
 * scratch.
 *
 * Every call on one GPU shares that GPU's array, whose contents the kernels
 * fully rewrite before reading (nothing needs clearing). Calls that overlap in
 * time on one GPU -- on different streams, or from different threads without
 * ordering -- race on it and give undefined results: order them on one stream.
 */
#define GRET_NOALLOC_SCRATCH_BYTES (64u << 20)
int gret_prefill_noalloc(const void* q, const void* k, const void* v, const float* log_gamma,
                         const float* state_in, void* out, float* state_out, int64_t B, int64_t H,
                         int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype,
                         void* stream);

/*
 * gret_decode_step -- one recurrent step for B*H independent heads.
 *
 * state_out[b,h] = exp(log_gamma[b,h]) state_in[b,h] + k[b,h]^T v[b,h] and
 * out[b,h,:] = q[b,h] state_out[b,h] (the output reads the updated state;
 * section "单 token Decode 的实现骨架").
 *
 *   q, k [B,H,dk], v [B,H,dv] in dtype; log_gamma [B,H] fp32 -- required
 *   state_in   fp32 [B,H,dk,dv] or NULL (zero state)
 *   state_out  fp32 [B,H,dk,dv], required; may be identical to state_in (the
 *              usual in-place update); any other overlap is GRET_ERR_ALIAS
 *   out        [B,H,dv] in dtype, required; must not overlap any other buffer
 *   dk, dv     64 or 128;  B, H >= 1
 * The state streams through HBM once per step (read + write), so this is the
 * bandwidth-bound half of the method.
 */
int gret_decode_step(const void* q, const void* k, const void* v, const float* log_gamma,
                     const float* state_in, void* out, float* state_out, int64_t B, int64_t H,
                     int64_t dk, int64_t dv, int dtype, void* stream);

/*
 * Output epilogue of the gated entry points below (page "YOCO 完全拆解：
 * Decoder-Decoder 架构如何让 KV Cache 只存一次", section "路线二：Multi-Head Gated
 * Retention", the per-head normalisation and output gate of the multi-head
 * output). For every (batch, head, position), with o the head's dv retention
 * outputs at that position:
 *   mean = sum(o) / dv,  var = sum((o - mean)^2) / dv
 *   z[j] = (o[j] - mean) / sqrt(var + norm_eps) * w[h][j] + b[h][j]
 *   y[j] = swish(gate[j]) * z[j],  swish(x) = x / (1 + exp(-x))
 * i.e. GroupNorm with one group per head over the H*dv channels, an optional
 * per-channel affine (w = 1 when norm_weight is NULL, b = 0 when norm_bias is
 * NULL), and the element-wise gate swish(X W_G); y is written to out. The
 * projection X W_G happens before the call: gate holds its result.
 *
 *   gate         same dtype and layout as out ([B,H,N,dv] for prefill, [B,H,dv]
 *                for decode), required, 16-byte aligned; read only
 *   norm_weight  fp32 [H,dv] or NULL;  norm_bias  fp32 [H,dv] or NULL
 *   norm_eps     finite and >= 0, else GRET_ERR_VALUE (torch's GroupNorm
 *                default is 1e-5); with norm_eps = 0 a constant row divides
 *                0 by 0
 * out must not overlap gate, norm_weight or norm_bias (GRET_ERR_ALIAS); every
 * other argument and rule is that of the plain entry point. The statistics are
 * computed in fp32: from the fp32 retention output in the decode step, and in
 * prefill from the output rounded to dtype (what the plain entry point would
 * store). In the bf16 prefill with chunk 64 the prefill kernels apply the
 * epilogue in their output store; with chunk 128 or 256, and in fp32, the
 * plain output is stored and a second pass rewrites out in place. Both give
 * the same values.
 */
int gret_prefill_gated(const void* q, const void* k, const void* v, const float* log_gamma,
                       const float* state_in, const void* gate, const float* norm_weight,
                       const float* norm_bias, float norm_eps, void* out, float* state_out,
                       int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream);

int gret_decode_step_gated(const void* q, const void* k, const void* v, const float* log_gamma,
                           const float* state_in, const void* gate, const float* norm_weight,
                           const float* norm_bias, float norm_eps, void* out, float* state_out,
                           int64_t B, int64_t H, int64_t dk, int64_t dv, int dtype, void* stream);

/*
 * Cross-Decoder decode attention over the shared global KV cache (page "YOCO
 * 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次", sections "增量生成时究竟
 * 追加什么" and "接入推理引擎时的四个关键点": at a decode step each Cross-Decoder
 * layer's query for the new token attends over the one global cache of keys
 * and values; with GQA, groups of G = Hq / Hkv query heads share one KV head).
 * For every sequence b and query head h, with g = h / G:
 *   out[b,h,:] = softmax_t(scale * q[b,h,:] . k_cache[b,g,t,:]) v_cache[b,g,t,:]
 * over t < lengths[b] (or t < L when lengths is NULL). Rotary position terms
 * are applied to q and the cached keys before the call.
 *
 *   q          [B,Hq,d] bf16;  out [B,Hq,d] bf16
 *   k_cache, v_cache  [B,Hkv,L,d] bf16 (L = allocated positions per sequence)
 *   lengths    device int32 [B] with 1 <= lengths[b] <= L, or NULL (all L);
 *              values outside that range give unspecified results (memory
 *              accesses stay inside the caches)
 *   scale      finite (usually d^-1/2), else GRET_ERR_VALUE
 *   dtype      GRET_DTYPE_BF16 only (else GRET_ERR_UNSUPPORTED)
 *   d          64 or 128;  Hq a multiple of Hkv with Hq / Hkv <= 16;
 *              B*Hq <= 2^30 - 1;  B*Hkv*L*128 <= 2^50;  L needs no other
 *              bound until the plan would need more than 1024 ranges per
 *              sequence and KV head (L above about 2^33 at d = 128): each
 *              range addresses its positions with 32-bit offsets from its
 *              own first position
 *   workspace  at least gret_cross_attention_workspace_bytes(...) bytes,
 *              256-byte aligned (per-range partial results); calls that share
 *              a workspace must be ordered on one stream
 * Pointers are 16-byte aligned device pointers (lengths 4-byte); out must not
 * overlap any other buffer, nor the workspace any input (GRET_ERR_ALIAS).
 */
int gret_cross_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                         int64_t d, size_t* bytes);

int gret_cross_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* lengths, void* out, int64_t B, int64_t Hq,
                                int64_t Hkv, int64_t L, int64_t d, float scale, int dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Key and log-gate projection with the key scaling and the gate's temperature
 * applied in the product's epilogue (page "YOCO 完全拆解：Decoder-Decoder 架构
 * 如何让 KV Cache 只存一次", section "路线二：Multi-Head Gated Retention": each
 * head projects a position's hidden state to its key and to a gate
 * sigmoid(X W_gamma)^(1/tau); section "单 token Decode 的实现骨架": the key is
 * scaled by d_h^-1/2 and the gate's log divided by 16). For token m = b*N + n:
 *   k_out[b,h,n,c]     = key_scale * sum_d x[m,d] * w_key[h*dk + c, d]
 *   log_gamma[b,h,n]   = log(sigmoid(sum_d x[m,d] * w_gamma[h,d])) / temperature
 * which are the key and log-gate layouts gret_prefill and gret_decode_step
 * take. With w_gamma and log_gamma NULL it is a plain head-major projection
 * (queries, values or the output gate, with key_scale 1 or any other scale).
 *
 *   x            [B*N, D] bf16, token-major (row m = hidden state of token m)
 *   w_key        [H*dk, D] bf16 (row j = weights of output channel j)
 *   w_gamma      [H, D] bf16, or NULL together with log_gamma
 *   key_scale    finite; temperature finite and > 0 (else GRET_ERR_VALUE)
 *   k_out        [B,H,N,dk] bf16 (fp32 accumulation, round to nearest even)
 *   log_gamma    [B,H,N] fp32
 *   dtype        GRET_DTYPE_BF16 only (else GRET_ERR_UNSUPPORTED)
 *   D a multiple of 128 up to 65536; dk a multiple of 16 up to 256; H <= 256
 *   when the gate is computed (else GRET_ERR_UNSUPPORTED)
 * Pointers are 16-byte aligned device pointers; k_out and log_gamma must not
 * overlap each other or any input (GRET_ERR_ALIAS). No workspace.
 */
int gret_head_projection(const void* x, const void* w_key, const void* w_gamma, float key_scale,
                         float temperature, void* k_out, float* log_gamma, int64_t B, int64_t N,
                         int64_t D, int64_t H, int64_t dk, int dtype, void* stream);

/*
 * Sliding-window-attention Self-Decoder mixer (page "YOCO 完全拆解：Decoder-
 * Decoder 架构如何让 KV Cache 只存一次", section "路线一：滑动窗口注意力":
 * position i attends only to the most recent `window` positions, the causal
 * window mask admitting j in [i - window + 1, i]; decoding keeps only those
 * keys and values, overwriting the oldest, in a ring (slot p mod window);
 * section "Prefill 的实现骨架": the prefill leaves the last `window` keys and
 * values in that fixed buffer). With g = h / (Hq / Hkv):
 *   out[b,h,i,:] = softmax_j(scale * q[b,h,i,:] . k[b,g,j,:]) v[b,g,j,:]
 * over max(0, i - window + 1) <= j <= i. Rotary position terms are applied
 * to q and k before the call.
 *
 * gret_swa_prefill:
 *   q            [B,Hq,N,d] bf16;  out [B,Hq,N,d] bf16 (fp32 softmax)
 *   k, v         [B,Hkv,N,d] bf16
 *   k_ring, v_ring  [B,Hkv,window,d] bf16, or both NULL: when given, slot
 *                p mod window receives position p for the last min(N, window)
 *                positions (other slots are left as they are)
 *   N            >= 1 (each workgroup addresses its query tile and its window
 *                of keys from their own first rows, so the prompt's length
 *                is limited only by the sizes below)
 *   window       1 .. 2^23;  d 64 or 128;  Hq a multiple of Hkv;  B*Hq*max(N,
 *                window)*d <= 2^50 and each launch <= 2^31 - 1 workgroups
 *                (B*Hq*ceil(N/256) for the attention)
 *   scale        finite (usually d^-1/2), else GRET_ERR_VALUE
 *   dtype        GRET_DTYPE_BF16 only (else GRET_ERR_UNSUPPORTED)
 * out and the rings must not overlap each other or an input (GRET_ERR_ALIAS).
 *
 * gret_swa_decode_step: one new token per sequence at position positions[b]
 * (device int32 [B], >= 0; the ring must hold positions
 * max(0, p - window + 1) .. p - 1 of that sequence, as left by the prefill and
 * earlier steps). Writes k_new, v_new [B,Hkv,d] into slot p mod window of the
 * rings (in place), then
 *   out[b,h,:] = attention of q[b,h,:] over the min(p + 1, window) valid slots.
 *   q, out       [B,Hq,d] bf16;  Hq / Hkv <= 16;  window <= 2^23
 *   workspace    at least gret_swa_decode_workspace_bytes(...) bytes, 256-byte
 *                aligned (valid-slot counts and per-range partial results);
 *                calls that share a workspace or rings must be ordered on one
 *                stream
 * Negative positions give unspecified results; every access stays inside the
 * rings. Pointers are 16-byte aligned device pointers (positions 4-byte); out,
 * the workspace and the rings must not overlap any other buffer.
 */
int gret_swa_prefill(const void* q, const void* k, const void* v, void* out, void* k_ring,
                     void* v_ring, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                     int64_t window, float scale, int dtype, void* stream);

int gret_swa_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t window, int64_t d,
                                    size_t* bytes);

int gret_swa_decode_step(const void* q, const void* k_new, const void* v_new, void* k_ring,
                         void* v_ring, const int32_t* positions, void* out, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t window, int64_t d, float scale, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable text for a gret_status_t value (never NULL). */
const char* gret_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GRET_H */
