// gret_internal.h -- launch entry points shared between the C ABI layer and
// the kernel translation units. Not part of the public interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gret_segments.h"

namespace gret {

// Log-gate clamp range applied by every kernel (see GRET_LOG_GAMMA_FLOOR).
constexpr float kLogGammaFloor = -80.0f;

// A segment's incoming state S_in reaches output n of the segment as
// exp(B_n) q_n S_in, B_n the log-decay accumulated since the segment start.
// Once B_n < -20 (exp(-20) ~ 2.1e-9 ~ 2^-28.9) that term is below
// 2^-28 |q_n|_1 max|S_in|: about 19 bits under the bf16 rounding of a stored
// output on the incoming state's own scale, and of the bf16 state operand the
// cross-chunk product itself uses. From there on a segment's outputs come from
// its zero-state pass; its leading chunks are recomputed from S_in.
constexpr float kSurvivalDropLog = -20.0f;

// Rows of one head that a bf16 prefill pass (a segment, or the recomputed
// leading chunks of one) may span: it addresses them through buffer ranges
// with 32-bit byte offsets taken from its own first row, formed in 32-bit
// arithmetic, so 2^31 bytes of the widest rows.
constexpr int64_t prefill_pass_rows(int64_t dk, int64_t dv) {
    return (int64_t(1) << 31) / (2 * (dk > dv ? dk : dv));
}

// Workgroups one launch may have (a single grid dimension). The C ABI checks
// every launch of a call against it before anything is enqueued.
constexpr int64_t kMaxGridGroups = 0x7fffffff;

// Output epilogue (per-head GroupNorm + swish gate); gate == nullptr means none.
struct OutputGate {
    const void* gate = nullptr;
    const float* weight = nullptr;  // [H][dv] or null
    const float* bias = nullptr;    // [H][dv] or null
    float eps = 0.0f;
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_gamma;
    const float* state_in;  // may be null
    void* out;
    float* state_out;       // may be null
    int64_t B, H, N, dk, dv, chunk;
    void* workspace;
    size_t workspace_bytes;
    hipStream_t stream;
    OutputGate epi;  // applied by the chunk-64 bf16 kernels in their output store
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_gamma;
    const float* state_in;  // may be null
    void* out;
    float* state_out;
    int64_t B, H, dk, dv;
    OutputGate epi;
    hipStream_t stream;
};

// The epilogue applied in place to a stored output: rows = B*H*N rows of dv
// values each, head of row r = (r / N) % H.
struct EpilogueArgs {
    void* out;
    OutputGate epi;
    int64_t rows, H, N, dv;
    hipStream_t stream;
};

// Workspace layout of the bf16 (matrix-core) prefill path for a plan.
struct PrefillWorkspace {
    size_t state_off;  // float [BH][max_seg][dk*dv]
    size_t meta_off;   // float2 [BH][max_seg]: (total log-decay, prefix chunks)
    size_t bytes;
};

PrefillWorkspace bf16_workspace_layout(const SegPlan& p, int64_t dk, int64_t dv);

// Each returns a hipError_t from the launch (hipSuccess when enqueued).
hipError_t launch_decode_f32(const DecodeArgs& a);
hipError_t launch_decode_bf16(const DecodeArgs& a);
hipError_t launch_prefill_f32(const PrefillArgs& a);
hipError_t launch_prefill_bf16(const PrefillArgs& a, const SegPlan& plan);

// Workgroups per CU the bf16 prefill kernel can keep resident (0 on error).
int prefill_bf16_blocks_per_cu(int64_t dk, int64_t dv, int64_t chunk);

// Cross-Decoder decode attention over the global KV cache (gret_xattn.hip).
struct XAttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* lengths;  // [B] or null (all L)
    void* out;
    int64_t B, Hq, Hkv, L, d;
    float scale;
    void* workspace;
    hipStream_t stream;
};
// Position ranges per (sequence, KV head) and the workspace they need; the plan
// depends only on the shapes (not on the device).
constexpr int64_t kXAttnTargetGroups = 1024;
// Cached positions one range of the cross-attention plan may span (with the
// tile a wavefront loads past its end): its buffer ranges take 32-bit byte
// offsets from the range's first position, 2^31 bytes of rows of d bf16.
constexpr int64_t xattn_range_rows(int64_t d) { return (int64_t(1) << 31) / (2 * d); }
struct XAttnPlan {
    int64_t S = 1, SL = 0;
    size_t acc_off = 0, bytes = 0;
};
XAttnPlan xattn_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d);
hipError_t launch_xattn_decode(const XAttnArgs& a);

hipError_t launch_output_gate_f32(const EpilogueArgs& a);
hipError_t launch_output_gate_bf16(const EpilogueArgs& a);
// Workgroups of the epilogue launch for `rows` rows of heads of N positions.
int64_t output_gate_groups(int64_t rows, int64_t N);

// Key and log-gate projection (gret_proj.hip): x [B*N, D] bf16, weights as
// rows; keys head-major [B,H,N,dk] bf16 times key_scale, log-gates [B,H,N].
struct ProjArgs {
    const void* x;
    const void* w_key;
    const void* w_gamma;  // [H, D] or null (no gate)
    void* k_out;
    float* log_gamma;     // null iff w_gamma is null
    int64_t B, N, D, H, dk;
    float key_scale, inv_temperature;
    hipStream_t stream;
};
hipError_t launch_head_projection(const ProjArgs& a);

// Sliding-window attention Self-Decoder (gret_swa.hip): prefill over the
// prompt (and the ring buffers it leaves), decode-step append into the rings.
struct SwaArgs {
    const void* q;   // [B,Hq,N,d]
    const void* k;   // [B,Hkv,N,d]
    const void* v;
    void* out;       // [B,Hq,N,d]
    void* k_ring;    // [B,Hkv,window,d] or null (then v_ring is null too)
    void* v_ring;
    int64_t B, Hq, Hkv, N, d, window;
    float scale;
    hipStream_t stream;
};
hipError_t launch_swa_prefill(const SwaArgs& a);
// Workgroups of the larger of the prefill's two launches (attention, ring fill).
int64_t swa_prefill_groups(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                           int64_t window, bool ring);
struct SwaDecodeArgs {
    const void* k_new;  // [B,Hkv,d]
    const void* v_new;
    void* k_ring;       // [B,Hkv,window,d]
    void* v_ring;
    const int32_t* positions;  // [B]
    int64_t B, Hkv, d, window;
    hipStream_t stream;
};
hipError_t launch_swa_append(const SwaDecodeArgs& a, int32_t* lengths);

// The chunk-64 bf16 prefill (gret_prefill_c64.hip), dispatched by the two above.
hipError_t launch_prefill_bf16_c64(const PrefillArgs& a, const SegPlan& plan);
int prefill_bf16_c64_blocks_per_cu(int64_t dk, int64_t dv);

}  // namespace gret
