// gret_decode.hip -- recurrent decode step of gated retention on gfx950.
//
// One step per (batch, head): S <- gamma S + k^T v, o = q S with the updated
// state (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次",
// sections "路线二：Multi-Head Gated Retention" and "单 token Decode 的实现骨架").
//
// The state is fp32 [dk][dv] per head and is read and written once per step,
// so the kernel is bound by HBM bandwidth (about 0.6 flop per byte). Design:
//   * one 256-thread workgroup per head; thread t owns 4 consecutive value
//     columns (a float4) of every RG-th key row, so a wavefront reads whole
//     512-byte state rows and every access is a coalesced 16-byte vector;
//   * all of a thread's state loads are issued before any arithmetic
//     (RPT = 16 outstanding 16-byte loads per lane at dk = dv = 128);
//   * the loads use the default cache policy and the stores the nontemporal
//     one: the line just read is rewritten in full. (Nontemporal loads
//     measured 1.17x slower at 256 x 24 heads, default stores 1.3x slower.)
//   * the update is fused with the output contraction: each updated float4 is
//     stored and immediately accumulated into q_i * S[i][:];
//   * the column sums are reduced across the lanes of a wavefront with
//     cross-lane shuffles and across the four wavefronts through LDS;
//   * with an output gate (same page and section: per-head normalisation,
//     then the element-wise gate swish(X W_G)), the dv outputs of the head,
//     held in fp32 by the first dv/4 lanes, are normalised (two-pass mean and
//     variance over those lanes), scaled, gated and then stored.
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kDecodeThreads = 256;

template <typename T, int DK, int DV, bool GATED>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_gamma, const float* state_in, T* __restrict__ out,
    float* state_out, const T* __restrict__ gate, const float* __restrict__ norm_weight,
    const float* __restrict__ norm_bias, float norm_eps, int64_t H) {
    constexpr int CG = DV / 4;                 // float4 column groups
    constexpr int RG = kDecodeThreads / CG;    // row groups
    constexpr int RPT = DK / RG;               // rows per thread
    constexpr int WAVES = kDecodeThreads / 64;
    static_assert(RG * CG == kDecodeThreads && RPT * RG == DK, "tiling");
    static_assert(CG <= 64 && 64 % CG == 0, "a row group must fit in a wavefront");

    __shared__ float s_q[DK];
    __shared__ float s_k[DK];
    __shared__ f32x4 s_red[WAVES][CG];

    const int64_t head = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;

    // The state loads go out first: the token's q, k, v and gate are small and
    // their latency then overlaps the state's.
    const int64_t base = head * DK * DV;
    f32x4 s[RPT];
    if (state_in) {
        const f32x4* src = reinterpret_cast<const f32x4*>(state_in + base);
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            s[r] = src[(rg + r * RG) * CG + cg];
    } else {
#pragma unroll
        for (int r = 0; r < RPT; ++r) s[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float gamma = __expf(clamp_log_gamma(log_gamma[head], kLogGammaFloor));
    f32x4 vv;
    vv[0] = load_as_float(v, head * DV + 4 * cg + 0);
    vv[1] = load_as_float(v, head * DV + 4 * cg + 1);
    vv[2] = load_as_float(v, head * DV + 4 * cg + 2);
    vv[3] = load_as_float(v, head * DV + 4 * cg + 3);
    for (int i = tid; i < DK; i += kDecodeThreads) {
        s_q[i] = load_as_float(q, head * DK + i);
        s_k[i] = load_as_float(k, head * DK + i);
    }
    __syncthreads();  // s_q, s_k ready

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    f32x4* dst = reinterpret_cast<f32x4*>(state_out + base);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int i = rg + r * RG;
        const float ki = s_k[i];
        const float qi = s_q[i];
        f32x4 t;
        t[0] = fmaf(gamma, s[r][0], ki * vv[0]);
        t[1] = fmaf(gamma, s[r][1], ki * vv[1]);
        t[2] = fmaf(gamma, s[r][2], ki * vv[2]);
        t[3] = fmaf(gamma, s[r][3], ki * vv[3]);
        __builtin_nontemporal_store(t, dst + i * CG + cg);
        acc[0] = fmaf(qi, t[0], acc[0]);
        acc[1] = fmaf(qi, t[1], acc[1]);
        acc[2] = fmaf(qi, t[2], acc[2]);
        acc[3] = fmaf(qi, t[3], acc[3]);
    }

    // Lanes cg, cg + CG, ... of a wavefront hold the same columns.
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
        acc[0] += __shfl_xor(acc[0], off);
        acc[1] += __shfl_xor(acc[1], off);
        acc[2] += __shfl_xor(acc[2], off);
        acc[3] += __shfl_xor(acc[3], off);
    }
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (lane < CG) s_red[wave][lane] = acc;
    __syncthreads();
    if (tid < CG) {
        f32x4 o = s_red[0][tid];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            o[0] += s_red[w][tid][0];
            o[1] += s_red[w][tid][1];
            o[2] += s_red[w][tid][2];
            o[3] += s_red[w][tid][3];
        }
        if constexpr (GATED) {
            // lanes 0..CG-1 of wavefront 0 hold the head's dv outputs
            float sum = o[0] + o[1] + o[2] + o[3];
#pragma unroll
            for (int off = 1; off < CG; off <<= 1) sum += __shfl_xor(sum, off);
            const float mean = sum * (1.0f / DV);
            float sq = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) sq += (o[i] - mean) * (o[i] - mean);
#pragma unroll
            for (int off = 1; off < CG; off <<= 1) sq += __shfl_xor(sq, off);
            const float rstd = rsqrtf(sq * (1.0f / DV) + norm_eps);
            const int64_t h = head % H;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * tid + i;
                float z = (o[i] - mean) * rstd;
                if (norm_weight) z *= norm_weight[h * DV + j];
                if (norm_bias) z += norm_bias[h * DV + j];
                o[i] = swish(load_as_float(gate, head * DV + j)) * z;
            }
        }
        store_from_float(out, head * DV + 4 * tid + 0, o[0]);
        store_from_float(out, head * DV + 4 * tid + 1, o[1]);
        store_from_float(out, head * DV + 4 * tid + 2, o[2]);
        store_from_float(out, head * DV + 4 * tid + 3, o[3]);
    }
}

template <typename T>
hipError_t launch_decode_t(const DecodeArgs& a) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H));
    const dim3 block(kDecodeThreads);
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    T* out = static_cast<T*>(a.out);
    const T* gate = static_cast<const T*>(a.epi.gate);
#define GRET_DECODE_CASE(DK_, DV_)                                                             \
    if (a.dk == DK_ && a.dv == DV_) {                                                          \
        if (gate)                                                                              \
            hipLaunchKernelGGL((decode_step_kernel<T, DK_, DV_, true>), grid, block, 0,        \
                               a.stream, q, k, v, a.log_gamma, a.state_in, out, a.state_out,   \
                               gate, a.epi.weight, a.epi.bias, a.epi.eps, a.H);                \
        else                                                                                   \
            hipLaunchKernelGGL((decode_step_kernel<T, DK_, DV_, false>), grid, block, 0,       \
                               a.stream, q, k, v, a.log_gamma, a.state_in, out, a.state_out,   \
                               nullptr, nullptr, nullptr, 0.0f, a.H);                          \
        return hipGetLastError();                                                              \
    }
    GRET_DECODE_CASE(64, 64)
    GRET_DECODE_CASE(64, 128)
    GRET_DECODE_CASE(128, 64)
    GRET_DECODE_CASE(128, 128)
#undef GRET_DECODE_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_f32(const DecodeArgs& a) { return launch_decode_t<float>(a); }
hipError_t launch_decode_bf16(const DecodeArgs& a) { return launch_decode_t<bf16_t>(a); }

}  // namespace gret
