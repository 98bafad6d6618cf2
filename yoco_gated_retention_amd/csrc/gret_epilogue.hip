// gret_epilogue.hip -- output epilogue of gated retention on gfx950, applied in
// place to a stored retention output (the fp32 prefill and the bf16 prefill at
// chunk 128 and 256; at chunk 64 the prefill kernels apply it in their output
// store).
//
// Page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次", section
// "路线二：Multi-Head Gated Retention": the multi-head output is normalised per
// head (GroupNorm: one group per head over its dv channels) and multiplied
// element by element by the output gate swish(X W_G). Per (batch, head,
// position) row of dv values:
//   z = (o - mean) / sqrt(var + eps) * w[h] + b[h],   y = swish(gate) * z.
//
// The kernel is a streaming pass (read the row and its gate, write the row),
// bound by HBM bandwidth: 3 * dv * sizeof(T) bytes per row. A workgroup takes
// 128 consecutive rows of one head, so the head's affine for a lane's channels
// is loaded once; each lane owns one 16-byte piece of a row, a row is spread
// over dv * sizeof(T) / 16 adjacent lanes, and a wavefront issues the loads of
// all its rows (8 row pieces and their gates per lane at dv = 128 in bf16)
// before any arithmetic. The gate is read once and loaded nontemporal; the
// rows keep the default policy, since the line just read is rewritten. Rows past N are handled by range-checked
// buffer accesses (loads read 0, stores are dropped), so no branch sits between
// the loads and they all stay in flight together. Mean and variance (two
// passes over registers, fp32) are reduced with cross-lane exchanges inside a
// row's lanes.
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kEpiThreads = 256;

// Cache policy of a load: 0 default, 2 nontemporal.
template <int POL>
__device__ inline i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL);
}
constexpr int kLoadDefault = 0, kLoadStream = 2;
__device__ inline void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, i32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

template <typename T>
struct Piece;  // one 16-byte piece of a row, widened to fp32
template <>
struct Piece<float> {
    static constexpr int N = 4;
    static __device__ inline void unpack(i32x4 raw, float (&x)[N]) {
        const f32x4 v = __builtin_bit_cast(f32x4, raw);
        x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
    }
    static __device__ inline i32x4 pack(const float (&x)[N]) {
        return __builtin_bit_cast(i32x4, f32x4{x[0], x[1], x[2], x[3]});
    }
};
template <>
struct Piece<bf16_t> {
    static constexpr int N = 8;
    static __device__ inline void unpack(i32x4 raw, float (&x)[N]) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = from_bf16(v[i]);
    }
    static __device__ inline i32x4 pack(const float (&x)[N]) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = to_bf16(x[i]);
        return __builtin_bit_cast(i32x4, v);
    }
};

constexpr int kRowsPerGroup = 128;  // 64 and 256 measured slower, 96 and 192 too

template <typename T, int DV>
__global__ __launch_bounds__(kEpiThreads) void output_gate_kernel(
    T* out, const T* __restrict__ gate, const float* __restrict__ weight,
    const float* __restrict__ bias, float eps, int64_t N, int64_t H, int64_t blocks_per_head) {
    constexpr int VPL = Piece<T>::N;                // values per lane
    constexpr int LPR = DV / VPL;                   // lanes per row
    constexpr int RPW = 64 / LPR;                   // rows per wavefront and step
    constexpr int WAVES = kEpiThreads / 64;
    constexpr int STEPS = kRowsPerGroup / (RPW * WAVES);
    static_assert(LPR * VPL == DV && LPR <= 64 && 64 % LPR == 0, "row split");
    static_assert(STEPS * RPW * WAVES == kRowsPerGroup, "rows per workgroup");
    const int64_t bh = blockIdx.x / blocks_per_head;
    const int64_t n0 = (blockIdx.x - bh * blocks_per_head) * kRowsPerGroup;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = (lane % LPR) * VPL;
    const int64_t h = bh % H;
    // this workgroup's rows of the head, as one range-checked buffer each
    const int64_t rows = N - n0 < kRowsPerGroup ? N - n0 : kRowsPerGroup;
    const uint32_t bytes = static_cast<uint32_t>(rows * DV * sizeof(T));
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + (bh * N + n0) * DV, bytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gate + (bh * N + n0) * DV, bytes);
    i32x4 xr[STEPS], gr[STEPS];
    uint32_t off[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int r = (s * WAVES + wave) * RPW + lane / LPR;
        off[s] = static_cast<uint32_t>((r * DV + c0) * sizeof(T));
        xr[s] = buf_load16<kLoadDefault>(ro, off[s]);
        gr[s] = buf_load16<kLoadStream>(rg, off[s]);
    }
    float w[VPL], b[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        w[i] = weight ? weight[h * DV + c0 + i] : 1.0f;
        b[i] = bias ? bias[h * DV + c0 + i] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        float x[VPL], g[VPL];
        Piece<T>::unpack(xr[s], x);
        Piece<T>::unpack(gr[s], g);
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) sum += x[i];
        const float mean = group_sum<LPR>(sum) * (1.0f / DV);
        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) sq += (x[i] - mean) * (x[i] - mean);
        const float rstd = rsqrtf(group_sum<LPR>(sq) * (1.0f / DV) + eps);
#pragma unroll
        for (int i = 0; i < VPL; ++i) x[i] = swish(g[i]) * ((x[i] - mean) * rstd * w[i] + b[i]);
        buf_store16(ro, off[s], Piece<T>::pack(x));
    }
}

template <typename T>
hipError_t launch_t(const EpilogueArgs& a) {
    const int64_t per_head = (a.N + kRowsPerGroup - 1) / kRowsPerGroup;
    const int64_t blocks = output_gate_groups(a.rows, a.N);
    if (blocks < 1 || blocks > kMaxGridGroups) return hipErrorInvalidValue;
    T* out = static_cast<T*>(a.out);
    const T* gate = static_cast<const T*>(a.epi.gate);
    if (a.dv == 64)
        hipLaunchKernelGGL((output_gate_kernel<T, 64>), dim3(static_cast<unsigned>(blocks)),
                           dim3(kEpiThreads), 0, a.stream, out, gate, a.epi.weight, a.epi.bias,
                           a.epi.eps, a.N, a.H, per_head);
    else if (a.dv == 128)
        hipLaunchKernelGGL((output_gate_kernel<T, 128>), dim3(static_cast<unsigned>(blocks)),
                           dim3(kEpiThreads), 0, a.stream, out, gate, a.epi.weight, a.epi.bias,
                           a.epi.eps, a.N, a.H, per_head);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

int64_t output_gate_groups(int64_t rows, int64_t N) {
    return rows / N * ((N + kRowsPerGroup - 1) / kRowsPerGroup);
}

hipError_t launch_output_gate_f32(const EpilogueArgs& a) { return launch_t<float>(a); }
hipError_t launch_output_gate_bf16(const EpilogueArgs& a) { return launch_t<bf16_t>(a); }

}  // namespace gret
