// gret_epilogue.hip -- output epilogue of gated retention on gfx950, applied in
// place to a stored retention output.
//
// Page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次", section
// "路线二：Multi-Head Gated Retention": the multi-head output is normalised per
// head (GroupNorm: one group per head over its dv channels) and multiplied
// element by element by the output gate swish(X W_G). Per (batch, head,
// position) row of dv values:
//   z = (o - mean) / sqrt(var + eps) * w[h] + b[h],   y = swish(gate) * z.
//
// The kernel is a streaming pass (read the row and its gate, write the row),
// bound by HBM bandwidth: 3 * dv * sizeof(T) bytes per row. Each lane owns one
// 16-byte piece of a row, a row is spread over dv * sizeof(T) / 16 adjacent
// lanes, and its mean and variance (two passes over registers, fp32) are
// reduced with cross-lane exchanges inside that lane group. Wavefronts stride
// over the rows.
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kEpiThreads = 256;

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ inline float swish(float x) { return x / (1.0f + __expf(-x)); }

template <typename T>
struct Piece;  // one 16-byte piece of a row, widened to fp32
template <>
struct Piece<float> {
    static constexpr int N = 4;
    static __device__ inline void load(const float* p, float (&x)[N]) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p);
        x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
    }
    static __device__ inline void store(float* p, const float (&x)[N]) {
        *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    }
};
template <>
struct Piece<bf16_t> {
    static constexpr int N = 8;
    static __device__ inline void load(const bf16_t* p, float (&x)[N]) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = from_bf16(v[i]);
    }
    static __device__ inline void store(bf16_t* p, const float (&x)[N]) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = to_bf16(x[i]);
        *reinterpret_cast<bf16x8*>(p) = v;
    }
};

template <typename T, int DV>
__global__ __launch_bounds__(kEpiThreads) void output_gate_kernel(
    T* out, const T* __restrict__ gate, const float* __restrict__ weight,
    const float* __restrict__ bias, float eps, int64_t rows, int64_t H, int64_t N) {
    constexpr int VPL = Piece<T>::N;  // values per lane
    constexpr int LPR = DV / VPL;     // lanes per row
    constexpr int RPW = 64 / LPR;     // rows per wavefront and step
    static_assert(LPR * VPL == DV && LPR <= 64 && 64 % LPR == 0, "row split");
    const int lane = threadIdx.x & 63;
    const int sub = lane / LPR;
    const int c0 = (lane % LPR) * VPL;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kEpiThreads + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kEpiThreads) >> 6;
    for (int64_t r0 = wave * RPW; r0 < rows; r0 += nwaves * RPW) {
        const int64_t r = r0 + sub;
        const bool ok = r < rows;  // the same for all lanes of a row
        float x[VPL], g[VPL];
        if (ok) {
            Piece<T>::load(out + r * DV + c0, x);
            Piece<T>::load(gate + r * DV + c0, g);
        } else {
#pragma unroll
            for (int i = 0; i < VPL; ++i) x[i] = g[i] = 0.0f;
        }
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) s += x[i];
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off);
        const float mean = s * (1.0f / DV);
        float q = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) q += (x[i] - mean) * (x[i] - mean);
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) q += __shfl_xor(q, off);
        const float rstd = rsqrtf(q * (1.0f / DV) + eps);
        if (ok) {
            const int64_t h = (r / N) % H;
            const float* wr = weight ? weight + h * DV + c0 : nullptr;
            const float* br = bias ? bias + h * DV + c0 : nullptr;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                float z = (x[i] - mean) * rstd;
                if (wr) z *= wr[i];
                if (br) z += br[i];
                x[i] = swish(g[i]) * z;
            }
            Piece<T>::store(out + r * DV + c0, x);
        }
    }
}

template <typename T>
hipError_t launch_t(const EpilogueArgs& a) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
    const int64_t rpw = 64 / (a.dv / Piece<T>::N);
    const int64_t waves_needed = (a.rows + rpw - 1) / rpw;
    int64_t blocks = (waves_needed + kEpiThreads / 64 - 1) / (kEpiThreads / 64);
    const int64_t cap = static_cast<int64_t>(cus > 0 ? cus : 1) * 8;
    if (blocks > cap) blocks = cap;
    T* out = static_cast<T*>(a.out);
    const T* gate = static_cast<const T*>(a.epi.gate);
    if (a.dv == 64)
        hipLaunchKernelGGL((output_gate_kernel<T, 64>), dim3(blocks), dim3(kEpiThreads), 0,
                           a.stream, out, gate, a.epi.weight, a.epi.bias, a.epi.eps, a.rows, a.H,
                           a.N);
    else if (a.dv == 128)
        hipLaunchKernelGGL((output_gate_kernel<T, 128>), dim3(blocks), dim3(kEpiThreads), 0,
                           a.stream, out, gate, a.epi.weight, a.epi.bias, a.epi.eps, a.rows, a.H,
                           a.N);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_output_gate_f32(const EpilogueArgs& a) { return launch_t<float>(a); }
hipError_t launch_output_gate_bf16(const EpilogueArgs& a) { return launch_t<bf16_t>(a); }

}  // namespace gret
