// gret_api.cpp -- the C ABI of libgret: argument validation, aliasing rules,
// prefill planning and dispatch to the kernels. Validation never touches the
// HIP runtime (gret_prefill_noalloc's scratch-size check follows a device
// attribute query), so a rejected call has no side effect at all.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/gret.h"
#include "gret_internal.h"

// Device scratch of gret_prefill_noalloc: one array per GPU, created when the
// library's code object is loaded on that device and held until the process
// ends. Host code never uses the array's name as an address (on the host it is
// only a stand-in for the symbol); kernels get the per-device address found by
// hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[GRET_NOALLOC_SCRATCH_BYTES];

namespace {

using gret::SegPlan;

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (the current device), looked up
// once per device; nullptr if the lookup fails.
void* scratch_on(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

constexpr int64_t kMaxElems = int64_t(1) << 50;  // guards size arithmetic

struct Span {
    uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Span span_of(const void* p, int64_t bytes) {
    Span s;
    if (p && bytes > 0) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + static_cast<uintptr_t>(bytes);
    }
    return s;
}

bool overlaps(const Span& a, const Span& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool head_dim_ok(int64_t d) { return d == 64 || d == 128; }

int check_common(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int dtype) {
    if (dtype != GRET_DTYPE_F32 && dtype != GRET_DTYPE_BF16) return GRET_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || N < 1) return GRET_ERR_SHAPE;
    if (B > kMaxElems || H > kMaxElems / B || N > kMaxElems / (B * H)) return GRET_ERR_SHAPE;
    if (B * H * N > kMaxElems / 128) return GRET_ERR_SHAPE;
    // Launches that scale with B*H: the decode step (B*H workgroups), the fp32
    // prefill (B*H*dv/32) and the bf16 prefill's combine (B*H*dk*dv/1024, at
    // most 16 per head); the bf16 prefill's other launches have <= 1024.
    if (B * H > gret::kMaxGridGroups / 16) return GRET_ERR_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GRET_ERR_UNSUPPORTED;
    return GRET_OK;
}

// Plan used for both workspace sizing (G at its cap) and launching (G chosen
// from the device).
SegPlan make_plan(int64_t B, int64_t H, int64_t N, int64_t chunk, int64_t G) {
    SegPlan p;
    p.BH = B * H;
    p.nc = (N + chunk - 1) / chunk;
    p.T = p.BH * p.nc;
    p.G = G < 1 ? 1 : (G > p.T ? p.T : G);
    p.max_seg = gret::seg_max_per_head(p.BH, p.nc, p.G);
    return p;
}

size_t workspace_need(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                      int dtype) {
    if (dtype != GRET_DTYPE_BF16) return 0;
    const SegPlan cap = make_plan(B, H, N, chunk, gret::kMaxPrefillGroups);
    return gret::bf16_workspace_layout(cap, dk, dv).bytes;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GRET_OK : GRET_ERR_HIP; }

// Checks the output-epilogue arguments; spans of the read-only epilogue
// tensors go to *sg, *sw, *sb.
int check_epilogue(const void* gate, const float* w, const float* b, float eps, int64_t rows,
                   int64_t H, int64_t dv, int64_t esz, Span* sg, Span* sw, Span* sb) {
    if (!gate) return GRET_ERR_NULL;
    if (!aligned(gate, 16)) return GRET_ERR_UNSUPPORTED;
    if ((w && !aligned(w, 4)) || (b && !aligned(b, 4))) return GRET_ERR_UNSUPPORTED;
    if (!isfinite(eps) || eps < 0.0f) return GRET_ERR_VALUE;
    *sg = span_of(gate, rows * dv * esz);
    *sw = span_of(w, H * dv * 4);
    *sb = span_of(b, H * dv * 4);
    return GRET_OK;
}

int prefill_impl(const void* q, const void* k, const void* v, const float* log_gamma,
                 const float* state_in, const gret::OutputGate* epi, void* out, float* state_out,
                 int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                 int dtype, void* workspace, size_t workspace_bytes, bool use_scratch,
                 void* stream);
int decode_impl(const void* q, const void* k, const void* v, const float* log_gamma,
                const float* state_in, const gret::OutputGate* epi, void* out, float* state_out,
                int64_t B, int64_t H, int64_t dk, int64_t dv, int dtype, void* stream);

}  // namespace

namespace gret {

PrefillWorkspace bf16_workspace_layout(const SegPlan& p, int64_t dk, int64_t dv) {
    PrefillWorkspace w;
    const size_t slots = static_cast<size_t>(p.BH) * static_cast<size_t>(p.max_seg);
    w.state_off = 0;
    w.meta_off = slots * static_cast<size_t>(dk * dv) * sizeof(float);
    w.bytes = w.meta_off + slots * 2 * sizeof(float);
    w.bytes = (w.bytes + 255) & ~size_t(255);
    return w;
}

}  // namespace gret

namespace {

int prefill_impl(const void* q, const void* k, const void* v, const float* log_gamma,
                 const float* state_in, const gret::OutputGate* epi, void* out, float* state_out,
                 int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                 int dtype, void* workspace, size_t workspace_bytes, bool use_scratch,
                 void* stream) {
    if (!q || !k || !v || !log_gamma || !out) return GRET_ERR_NULL;
    int st = check_common(B, H, N, dk, dv, dtype);
    if (st != GRET_OK) return st;
    if (chunk != 64 && chunk != 128 && chunk != 256) return GRET_ERR_UNSUPPORTED;
    for (const void* p : {q, k, v, (const void*)out, (const void*)state_in, (const void*)state_out})
        if (p && !aligned(p, 16)) return GRET_ERR_UNSUPPORTED;
    if (!aligned(log_gamma, 4)) return GRET_ERR_UNSUPPORTED;

    const int64_t esz = dtype == GRET_DTYPE_BF16 ? 2 : 4;
    const int64_t BHN = B * H * N;
    Span sg, sgw, sgb;
    if (epi) {
        st = check_epilogue(epi->gate, epi->weight, epi->bias, epi->eps, BHN, H, dv, esz, &sg,
                            &sgw, &sgb);
        if (st != GRET_OK) return st;
    }
    if (epi && gret::output_gate_groups(BHN, N) > gret::kMaxGridGroups) return GRET_ERR_SHAPE;
    if (use_scratch) {
        workspace = nullptr;  // the library's own scratch replaces it (below)
        workspace_bytes = 0;
    }
    const size_t need = use_scratch ? 0 : workspace_need(B, H, N, dk, dv, chunk, dtype);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return GRET_ERR_WORKSPACE;

    const Span sq = span_of(q, BHN * dk * esz), sk = span_of(k, BHN * dk * esz),
               sv = span_of(v, BHN * dv * esz), sl = span_of(log_gamma, BHN * 4),
               so = span_of(out, BHN * dv * esz),
               si = span_of(state_in, B * H * dk * dv * 4),
               ss = span_of(state_out, B * H * dk * dv * 4),
               sw = span_of(workspace, need > 0 ? (int64_t)need : 0);
    for (const Span& x : {sq, sk, sv, sl, si, ss, sw})
        if (overlaps(so, x)) return GRET_ERR_ALIAS;
    for (const Span& x : {sq, sk, sv, sl, sw})
        if (overlaps(ss, x)) return GRET_ERR_ALIAS;
    if (overlaps(ss, si) && state_out != state_in) return GRET_ERR_ALIAS;
    for (const Span& x : {sq, sk, sv, sl, si})
        if (overlaps(sw, x)) return GRET_ERR_ALIAS;
    for (const Span& x : {sg, sgw, sgb})
        if (overlaps(so, x) || overlaps(ss, x) || overlaps(sw, x)) return GRET_ERR_ALIAS;

    gret::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_gamma = log_gamma;
    a.state_in = state_in;
    a.out = out;
    a.state_out = state_out;
    a.B = B;
    a.H = H;
    a.N = N;
    a.dk = dk;
    a.dv = dv;
    a.chunk = chunk;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    a.stream = reinterpret_cast<hipStream_t>(stream);

    (void)hipGetLastError();  // clear anything pending from unrelated calls
    gret::EpilogueArgs ea;
    if (epi) {
        ea.out = out;
        ea.epi = *epi;
        ea.rows = BHN;
        ea.H = H;
        ea.N = N;
        ea.dv = dv;
        ea.stream = a.stream;
    }
    if (dtype == GRET_DTYPE_F32) {
        st = hip_status(gret::launch_prefill_f32(a));
        if (st != GRET_OK || !epi) return st;
        return hip_status(gret::launch_output_gate_f32(ea));
    }

    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GRET_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return GRET_ERR_HIP;
    const int per_cu = gret::prefill_bf16_blocks_per_cu(dk, dv, chunk);
    if (per_cu <= 0 || cus <= 0) return GRET_ERR_HIP;
    int64_t G = static_cast<int64_t>(cus) * per_cu;
    if (G > gret::kMaxPrefillGroups) G = gret::kMaxPrefillGroups;
    const SegPlan plan = make_plan(B, H, N, chunk, G);
    // a pass issues loads up to two chunks past its last one
    if ((gret::seg_max_piece_chunks(plan) + 2) * chunk > gret::prefill_pass_rows(dk, dv))
        return GRET_ERR_SHAPE;
    if (use_scratch) {
        // the scratch holds the workspace of this device's plan (its number of
        // workgroups), not of the device-independent cap
        if (gret::bf16_workspace_layout(plan, dk, dv).bytes > GRET_NOALLOC_SCRATCH_BYTES)
            return GRET_ERR_SCRATCH;
        a.workspace = scratch_on(dev);
        a.workspace_bytes = GRET_NOALLOC_SCRATCH_BYTES;
        if (!a.workspace) return GRET_ERR_HIP;
    }
    // chunk 64: the kernels apply the epilogue in their output store; the
    // other chunk sizes store the plain output and a pass rewrites it
    const bool fused = epi && chunk == 64;
    if (fused) a.epi = *epi;
    st = hip_status(gret::launch_prefill_bf16(a, plan));
    if (st != GRET_OK || !epi || fused) return st;
    return hip_status(gret::launch_output_gate_bf16(ea));
}

int decode_impl(const void* q, const void* k, const void* v, const float* log_gamma,
                const float* state_in, const gret::OutputGate* epi, void* out, float* state_out,
                int64_t B, int64_t H, int64_t dk, int64_t dv, int dtype, void* stream) {
    if (!q || !k || !v || !log_gamma || !out || !state_out) return GRET_ERR_NULL;
    int st = check_common(B, H, 1, dk, dv, dtype);
    if (st != GRET_OK) return st;
    for (const void* p : {q, k, v, (const void*)out, (const void*)state_in, (const void*)state_out})
        if (p && !aligned(p, 16)) return GRET_ERR_UNSUPPORTED;
    if (!aligned(log_gamma, 4)) return GRET_ERR_UNSUPPORTED;

    const int64_t esz = dtype == GRET_DTYPE_BF16 ? 2 : 4;
    const int64_t BH = B * H;
    Span sg, sgw, sgb;
    if (epi) {
        st = check_epilogue(epi->gate, epi->weight, epi->bias, epi->eps, BH, H, dv, esz, &sg,
                            &sgw, &sgb);
        if (st != GRET_OK) return st;
    }
    const Span sq = span_of(q, BH * dk * esz), sk = span_of(k, BH * dk * esz),
               sv = span_of(v, BH * dv * esz), sl = span_of(log_gamma, BH * 4),
               so = span_of(out, BH * dv * esz), si = span_of(state_in, BH * dk * dv * 4),
               ss = span_of(state_out, BH * dk * dv * 4);
    for (const Span& x : {sq, sk, sv, sl, si, ss})
        if (overlaps(so, x)) return GRET_ERR_ALIAS;
    for (const Span& x : {sq, sk, sv, sl})
        if (overlaps(ss, x)) return GRET_ERR_ALIAS;
    if (overlaps(ss, si) && state_out != state_in) return GRET_ERR_ALIAS;
    for (const Span& x : {sg, sgw, sgb})
        if (overlaps(so, x) || overlaps(ss, x)) return GRET_ERR_ALIAS;

    gret::DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_gamma = log_gamma;
    a.state_in = state_in;
    a.out = out;
    a.state_out = state_out;
    a.B = B;
    a.H = H;
    a.dk = dk;
    a.dv = dv;
    if (epi) a.epi = *epi;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return hip_status(dtype == GRET_DTYPE_BF16 ? gret::launch_decode_bf16(a)
                                               : gret::launch_decode_f32(a));
}

}  // namespace

extern "C" {

const char* gret_status_string(int status) {
    switch (status) {
        case GRET_OK: return "GRET_OK: success";
        case GRET_ERR_NULL: return "GRET_ERR_NULL: a required pointer is NULL";
        case GRET_ERR_SHAPE:
            return "GRET_ERR_SHAPE: B, H or N is < 1, the sizes overflow, or a launch would need "
                   "more than 2^31 - 1 workgroups";
        case GRET_ERR_UNSUPPORTED:
            return "GRET_ERR_UNSUPPORTED: dk/dv not in {64,128}, chunk not in {64,128,256}, "
                   "unknown dtype, or a tensor pointer not 16-byte aligned";
        case GRET_ERR_ALIAS:
            return "GRET_ERR_ALIAS: out overlaps another buffer, or the states overlap without "
                   "being identical";
        case GRET_ERR_HIP: return "GRET_ERR_HIP: a HIP runtime call or kernel launch failed";
        case GRET_ERR_WORKSPACE:
            return "GRET_ERR_WORKSPACE: workspace missing, smaller than "
                   "gret_prefill_workspace_bytes() or not 256-byte aligned";
        case GRET_ERR_VALUE:
            return "GRET_ERR_VALUE: norm_eps is negative or not finite, or scale is not finite";
        case GRET_ERR_SCRATCH:
            return "GRET_ERR_SCRATCH: gret_prefill_noalloc needs more than its fixed device "
                   "scratch (GRET_NOALLOC_SCRATCH_BYTES) for these sizes; use gret_prefill "
                   "with a workspace";
        default: return "unknown gret status";
    }
}

int gret_prefill_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                                 int64_t chunk, int dtype, size_t* bytes) {
    if (!bytes) return GRET_ERR_NULL;
    int st = check_common(B, H, N, dk, dv, dtype);
    if (st != GRET_OK) return st;
    if (chunk != 64 && chunk != 128 && chunk != 256) return GRET_ERR_UNSUPPORTED;
    *bytes = workspace_need(B, H, N, dk, dv, chunk, dtype);
    return GRET_OK;
}

int gret_prefill(const void* q, const void* k, const void* v, const float* log_gamma,
                 const float* state_in, void* out, float* state_out, int64_t B, int64_t H,
                 int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, log_gamma, state_in, nullptr, out, state_out, B, H, N, dk, dv,
                        chunk, dtype, workspace, workspace_bytes, false, stream);
}

int gret_prefill_noalloc(const void* q, const void* k, const void* v, const float* log_gamma,
                         const float* state_in, void* out, float* state_out, int64_t B, int64_t H,
                         int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype,
                         void* stream) {
    return prefill_impl(q, k, v, log_gamma, state_in, nullptr, out, state_out, B, H, N, dk, dv,
                        chunk, dtype, nullptr, 0, true, stream);
}

int gret_prefill_gated(const void* q, const void* k, const void* v, const float* log_gamma,
                       const float* state_in, const void* gate, const float* norm_weight,
                       const float* norm_bias, float norm_eps, void* out, float* state_out,
                       int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    gret::OutputGate epi;
    epi.gate = gate;
    epi.weight = norm_weight;
    epi.bias = norm_bias;
    epi.eps = norm_eps;
    if (!gate) return GRET_ERR_NULL;
    return prefill_impl(q, k, v, log_gamma, state_in, &epi, out, state_out, B, H, N, dk, dv,
                        chunk, dtype, workspace, workspace_bytes, false, stream);
}

int gret_decode_step(const void* q, const void* k, const void* v, const float* log_gamma,
                     const float* state_in, void* out, float* state_out, int64_t B, int64_t H,
                     int64_t dk, int64_t dv, int dtype, void* stream) {
    return decode_impl(q, k, v, log_gamma, state_in, nullptr, out, state_out, B, H, dk, dv,
                       dtype, stream);
}

int gret_decode_step_gated(const void* q, const void* k, const void* v, const float* log_gamma,
                           const float* state_in, const void* gate, const float* norm_weight,
                           const float* norm_bias, float norm_eps, void* out, float* state_out,
                           int64_t B, int64_t H, int64_t dk, int64_t dv, int dtype, void* stream) {
    gret::OutputGate epi;
    epi.gate = gate;
    epi.weight = norm_weight;
    epi.bias = norm_bias;
    epi.eps = norm_eps;
    if (!gate) return GRET_ERR_NULL;
    return decode_impl(q, k, v, log_gamma, state_in, &epi, out, state_out, B, H, dk, dv, dtype,
                       stream);
}

}  // extern "C"

namespace {

int check_xattn(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || L < 1) return GRET_ERR_SHAPE;
    if (B > kMaxElems || Hq > kMaxElems / B) return GRET_ERR_SHAPE;
    if (B * Hkv > kMaxElems / L / 128 || B * Hq > kMaxElems / 128) return GRET_ERR_SHAPE;
    // the combine launch has B*Hq workgroups, the split launch B*Hkv*S (S
    // ranges per sequence and KV head: about 1024 workgroups in all, or one
    // per sequence and KV head, or as many as a very long cache needs)
    if (B * Hq > gret::kMaxGridGroups / 2) return GRET_ERR_SHAPE;
    if (d != 64 && d != 128) return GRET_ERR_UNSUPPORTED;
    if (Hq % Hkv != 0 || Hq / Hkv > 16) return GRET_ERR_UNSUPPORTED;
    // the combine merges at most kXAttnTargetGroups ranges per head
    const gret::XAttnPlan plan = gret::xattn_plan(B, Hq, Hkv, L, d);
    if (plan.S > gret::kXAttnTargetGroups || B * Hkv * plan.S > gret::kMaxGridGroups)
        return GRET_ERR_SHAPE;
    return GRET_OK;
}

}  // namespace

extern "C" {

int gret_cross_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                         int64_t d, size_t* bytes) {
    if (!bytes) return GRET_ERR_NULL;
    const int st = check_xattn(B, Hq, Hkv, L, d);
    if (st != GRET_OK) return st;
    *bytes = gret::xattn_plan(B, Hq, Hkv, L, d).bytes;
    return GRET_OK;
}

int gret_cross_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* lengths, void* out, int64_t B, int64_t Hq,
                                int64_t Hkv, int64_t L, int64_t d, float scale, int dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k_cache || !v_cache || !out) return GRET_ERR_NULL;
    int st = check_xattn(B, Hq, Hkv, L, d);
    if (st != GRET_OK) return st;
    if (dtype != GRET_DTYPE_BF16) return GRET_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return GRET_ERR_VALUE;
    for (const void* p : {q, k_cache, v_cache, (const void*)out})
        if (!aligned(p, 16)) return GRET_ERR_UNSUPPORTED;
    if (lengths && !aligned(lengths, 4)) return GRET_ERR_UNSUPPORTED;
    const gret::XAttnPlan plan = gret::xattn_plan(B, Hq, Hkv, L, d);
    if (!workspace || workspace_bytes < plan.bytes || !aligned(workspace, 256))
        return GRET_ERR_WORKSPACE;
    const Span sq = span_of(q, B * Hq * d * 2), sk = span_of(k_cache, B * Hkv * L * d * 2),
               sv = span_of(v_cache, B * Hkv * L * d * 2), sl = span_of(lengths, B * 4),
               so = span_of(out, B * Hq * d * 2),
               sw = span_of(workspace, static_cast<int64_t>(plan.bytes));
    for (const Span& x : {sq, sk, sv, sl, sw})
        if (overlaps(so, x)) return GRET_ERR_ALIAS;
    for (const Span& x : {sq, sk, sv, sl})
        if (overlaps(sw, x)) return GRET_ERR_ALIAS;

    gret::XAttnArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.lengths = lengths;
    a.out = out;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.L = L;
    a.d = d;
    a.scale = scale;
    a.workspace = workspace;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return hip_status(gret::launch_xattn_decode(a));
}

int gret_head_projection(const void* x, const void* w_key, const void* w_gamma, float key_scale,
                         float temperature, void* k_out, float* log_gamma, int64_t B, int64_t N,
                         int64_t D, int64_t H, int64_t dk, int dtype, void* stream) {
    if (!x || !w_key || !k_out) return GRET_ERR_NULL;
    if ((w_gamma == nullptr) != (log_gamma == nullptr)) return GRET_ERR_NULL;
    if (B < 1 || N < 1 || D < 1 || H < 1 || dk < 1) return GRET_ERR_SHAPE;
    if (B > kMaxElems / N || H > kMaxElems / dk) return GRET_ERR_SHAPE;
    const int64_t M = B * N, J = H * dk;
    if (D > 65536 || M > kMaxElems / D || M > kMaxElems / J) return GRET_ERR_SHAPE;
    if (dtype != GRET_DTYPE_BF16) return GRET_ERR_UNSUPPORTED;
    if (D % 128 != 0 || dk % 16 != 0 || dk > 256) return GRET_ERR_UNSUPPORTED;
    if (w_gamma && H > 256) return GRET_ERR_UNSUPPORTED;
    if ((M + 255) / 256 * ((J + 255) / 256 + 1) > 0x7fffffff) return GRET_ERR_SHAPE;
    if (!isfinite(key_scale) || !isfinite(temperature) || !(temperature > 0.0f))
        return GRET_ERR_VALUE;
    for (const void* p : {x, w_key, w_gamma, (const void*)k_out, (const void*)log_gamma})
        if (p && !aligned(p, 16)) return GRET_ERR_UNSUPPORTED;
    const Span sx = span_of(x, M * D * 2), swk = span_of(w_key, J * D * 2),
               swg = span_of(w_gamma, H * D * 2), sk = span_of(k_out, M * J * 2),
               sl = span_of(log_gamma, M * H * 4);
    for (const Span& s : {sx, swk, swg, sl})
        if (overlaps(sk, s)) return GRET_ERR_ALIAS;
    for (const Span& s : {sx, swk, swg})
        if (overlaps(sl, s)) return GRET_ERR_ALIAS;

    gret::ProjArgs a;
    a.x = x;
    a.w_key = w_key;
    a.w_gamma = w_gamma;
    a.k_out = k_out;
    a.log_gamma = log_gamma;
    a.B = B;
    a.N = N;
    a.D = D;
    a.H = H;
    a.dk = dk;
    a.key_scale = key_scale;
    a.inv_temperature = static_cast<float>(1.0 / static_cast<double>(temperature));
    a.stream = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return hip_status(gret::launch_head_projection(a));
}

}  // extern "C"

namespace {
constexpr int64_t kSwaMaxN = int64_t(1) << 23;

int check_swa(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t window, int dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || window < 1) return GRET_ERR_SHAPE;
    if (B > kMaxElems / Hq || window > kSwaMaxN) return GRET_ERR_SHAPE;
    if (!head_dim_ok(d) || Hq % Hkv != 0) return GRET_ERR_UNSUPPORTED;
    if (dtype != GRET_DTYPE_BF16) return GRET_ERR_UNSUPPORTED;
    return GRET_OK;
}

size_t swa_lengths_bytes(int64_t B) { return (static_cast<size_t>(B) * 4 + 255) / 256 * 256; }
}  // namespace

extern "C" {

int gret_swa_prefill(const void* q, const void* k, const void* v, void* out, void* k_ring,
                     void* v_ring, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                     int64_t window, float scale, int dtype, void* stream) {
    if (!q || !k || !v || !out) return GRET_ERR_NULL;
    if ((k_ring == nullptr) != (v_ring == nullptr)) return GRET_ERR_NULL;
    int st = check_swa(B, Hq, Hkv, d, window, dtype);
    if (st != GRET_OK) return st;
    if (N < 1) return GRET_ERR_SHAPE;
    const int64_t span_rows = N > window ? N : window;  // positions of q/k/v/out, of the rings
    if (B * Hq > kMaxElems / (span_rows * d)) return GRET_ERR_SHAPE;
    if (gret::swa_prefill_groups(B, Hq, Hkv, N, d, window, k_ring != nullptr) >
        gret::kMaxGridGroups)
        return GRET_ERR_SHAPE;
    if (!isfinite(scale)) return GRET_ERR_VALUE;
    for (const void* p : {q, k, v, (const void*)out, (const void*)k_ring, (const void*)v_ring})
        if (p && !aligned(p, 16)) return GRET_ERR_UNSUPPORTED;
    const Span sq = span_of(q, B * Hq * N * d * 2), sk = span_of(k, B * Hkv * N * d * 2),
               sv = span_of(v, B * Hkv * N * d * 2), so = span_of(out, B * Hq * N * d * 2),
               srk = span_of(k_ring, B * Hkv * window * d * 2),
               srv = span_of(v_ring, B * Hkv * window * d * 2);
    for (const Span& x : {sq, sk, sv, srk, srv})
        if (overlaps(so, x)) return GRET_ERR_ALIAS;
    for (const Span& x : {sq, sk, sv, srv})
        if (overlaps(srk, x)) return GRET_ERR_ALIAS;
    for (const Span& x : {sq, sk, sv})
        if (overlaps(srv, x)) return GRET_ERR_ALIAS;

    gret::SwaArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.k_ring = k_ring;
    a.v_ring = v_ring;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.window = window;
    a.scale = scale;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return hip_status(gret::launch_swa_prefill(a));
}

int gret_swa_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t window, int64_t d,
                                    size_t* bytes) {
    if (!bytes) return GRET_ERR_NULL;
    int st = check_swa(B, Hq, Hkv, d, window, GRET_DTYPE_BF16);
    if (st != GRET_OK) return st;
    st = check_xattn(B, Hq, Hkv, window, d);
    if (st != GRET_OK) return st;
    *bytes = swa_lengths_bytes(B) + gret::xattn_plan(B, Hq, Hkv, window, d).bytes;
    return GRET_OK;
}

int gret_swa_decode_step(const void* q, const void* k_new, const void* v_new, void* k_ring,
                         void* v_ring, const int32_t* positions, void* out, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t window, int64_t d, float scale, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k_new || !v_new || !k_ring || !v_ring || !positions || !out) return GRET_ERR_NULL;
    int st = check_swa(B, Hq, Hkv, d, window, dtype);
    if (st != GRET_OK) return st;
    st = check_xattn(B, Hq, Hkv, window, d);
    if (st != GRET_OK) return st;
    if (!isfinite(scale)) return GRET_ERR_VALUE;
    for (const void* p : {q, k_new, v_new, (const void*)k_ring, (const void*)v_ring,
                          (const void*)out})
        if (!aligned(p, 16)) return GRET_ERR_UNSUPPORTED;
    if (!aligned(positions, 4)) return GRET_ERR_UNSUPPORTED;
    const size_t lbytes = swa_lengths_bytes(B);
    const gret::XAttnPlan plan = gret::xattn_plan(B, Hq, Hkv, window, d);
    if (!workspace || workspace_bytes < lbytes + plan.bytes || !aligned(workspace, 256))
        return GRET_ERR_WORKSPACE;
    const Span sq = span_of(q, B * Hq * d * 2), skn = span_of(k_new, B * Hkv * d * 2),
               svn = span_of(v_new, B * Hkv * d * 2),
               srk = span_of(k_ring, B * Hkv * window * d * 2),
               srv = span_of(v_ring, B * Hkv * window * d * 2), sp = span_of(positions, B * 4),
               so = span_of(out, B * Hq * d * 2),
               sw = span_of(workspace, static_cast<int64_t>(lbytes + plan.bytes));
    for (const Span& x : {sq, skn, svn, srk, srv, sp, sw})
        if (overlaps(so, x)) return GRET_ERR_ALIAS;
    for (const Span& x : {sq, skn, svn, srk, srv, sp})
        if (overlaps(sw, x)) return GRET_ERR_ALIAS;
    for (const Span& x : {sq, skn, svn, srv, sp})
        if (overlaps(srk, x)) return GRET_ERR_ALIAS;
    for (const Span& x : {sq, skn, svn, sp})
        if (overlaps(srv, x)) return GRET_ERR_ALIAS;

    gret::SwaDecodeArgs da;
    da.k_new = k_new;
    da.v_new = v_new;
    da.k_ring = k_ring;
    da.v_ring = v_ring;
    da.positions = positions;
    da.B = B;
    da.Hkv = Hkv;
    da.d = d;
    da.window = window;
    da.stream = reinterpret_cast<hipStream_t>(stream);
    int32_t* lengths = static_cast<int32_t*>(workspace);
    (void)hipGetLastError();
    st = hip_status(gret::launch_swa_append(da, lengths));
    if (st != GRET_OK) return st;
    gret::XAttnArgs a;
    a.q = q;
    a.k = k_ring;
    a.v = v_ring;
    a.lengths = lengths;
    a.out = out;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.L = window;
    a.d = d;
    a.scale = scale;
    a.workspace = static_cast<char*>(workspace) + lbytes;
    a.stream = da.stream;
    return hip_status(gret::launch_xattn_decode(a));
}

}  // extern "C"
