// gret_prefill_f32.hip -- chunkwise gated-retention prefill, fp32 throughout.
//
// This is the precision path (fp32 inputs and outputs, fp32 arithmetic on the
// vector ALUs). It evaluates the chunkwise form of the page "YOCO 完全拆解：
// Decoder-Decoder 架构如何让 KV Cache 只存一次", section "Prefill 与 Decode 为什么
// 使用两种计算形态": for a chunk starting at position a with chunk-local
// inclusive log-decay sums beta_j,
//   out[a+j] = exp(beta_j) q_{a+j} S + sum_{l<=j} exp(beta_j - beta_l)
//              (q_{a+j} . k_{a+l}) v_{a+l}
//   S       <- exp(beta_last) S + sum_l exp(beta_last - beta_l) k_{a+l}^T v_{a+l}
// Only differences of log-decays are exponentiated inside a chunk, so every
// factor is <= 1 and nothing overflows. A tail chunk shorter than the chunk
// size simply has fewer rows (the padding of section "Prefill 的实现骨架" never
// materialises), so the final state is exactly S_{N-1}.
//
// Work split: one 256-thread workgroup per (batch*head, 32-column slice of
// dv); the state slice [dk][32] lives in LDS for the whole sequence. This path
// targets small fp32 problems and is not tuned for bandwidth.
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kF32Threads = 256;
constexpr int kSlice = 32;   // value columns per workgroup
constexpr int kRowBlk = 16;  // output rows per intra-chunk block

template <int DK, int DV, int C>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ log_gamma, const float* state_in, float* __restrict__ out,
    float* state_out, int64_t N) {
    __shared__ float s_state[DK][kSlice];
    __shared__ float s_beta[C];
    __shared__ float s_p[kRowBlk][C];

    constexpr int kSlices = DV / kSlice;
    const int64_t head = blockIdx.x / kSlices;
    const int c0 = (blockIdx.x % kSlices) * kSlice;
    const int tid = threadIdx.x;

    const float* qh = q + head * N * DK;
    const float* kh = k + head * N * DK;
    const float* vh = v + head * N * DV;
    const float* lh = log_gamma + head * N;
    float* oh = out + head * N * DV;

    for (int e = tid; e < DK * kSlice; e += kF32Threads) {
        const int i = e / kSlice, c = e % kSlice;
        s_state[i][c] = state_in ? state_in[head * DK * DV + i * DV + c0 + c] : 0.0f;
    }

    for (int64_t a = 0; a < N; a += C) {
        const int n = static_cast<int>(N - a < C ? N - a : C);
        __syncthreads();  // previous chunk's state update complete
        if (tid == 0) {
            float acc = 0.0f;
            for (int j = 0; j < n; ++j) {
                acc += clamp_log_gamma(lh[a + j], kLogGammaFloor);
                s_beta[j] = acc;
            }
        }
        __syncthreads();
        const float g = s_beta[n - 1];

        for (int j0 = 0; j0 < n; j0 += kRowBlk) {
            // decayed causal scores for rows j0 .. j0+15
            for (int e = tid; e < kRowBlk * C; e += kF32Threads) {
                const int jj = e / C, l = e % C, j = j0 + jj;
                float p = 0.0f;
                if (j < n && l <= j) {
                    const float* qr = qh + (a + j) * DK;
                    const float* kr = kh + (a + l) * DK;
                    for (int i = 0; i < DK; ++i) p = fmaf(qr[i], kr[i], p);
                    p *= __expf(s_beta[j] - s_beta[l]);
                }
                s_p[jj][l] = p;
            }
            __syncthreads();
            for (int e = tid; e < kRowBlk * kSlice; e += kF32Threads) {
                const int jj = e / kSlice, c = e % kSlice, j = j0 + jj;
                if (j < n) {
                    const float* qr = qh + (a + j) * DK;
                    float cross = 0.0f;
                    for (int i = 0; i < DK; ++i) cross = fmaf(qr[i], s_state[i][c], cross);
                    float intra = 0.0f;
                    for (int l = 0; l <= j; ++l) intra = fmaf(s_p[jj][l], vh[(a + l) * DV + c0 + c], intra);
                    oh[(a + j) * DV + c0 + c] = fmaf(__expf(s_beta[j]), cross, intra);
                }
            }
            __syncthreads();
        }

        // state update
        const float eg = __expf(g);
        for (int e = tid; e < DK * kSlice; e += kF32Threads) {
            const int i = e / kSlice, c = e % kSlice;
            float acc = 0.0f;
            for (int l = 0; l < n; ++l)
                acc = fmaf(__expf(g - s_beta[l]) * kh[(a + l) * DK + i], vh[(a + l) * DV + c0 + c], acc);
            s_state[i][c] = fmaf(eg, s_state[i][c], acc);
        }
    }
    __syncthreads();
    if (state_out) {
        for (int e = tid; e < DK * kSlice; e += kF32Threads) {
            const int i = e / kSlice, c = e % kSlice;
            state_out[head * DK * DV + i * DV + c0 + c] = s_state[i][c];
        }
    }
}

template <int DK, int DV>
hipError_t launch_f32_dims(const PrefillArgs& a) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * (DV / kSlice)));
    const dim3 block(kF32Threads);
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    float* out = static_cast<float*>(a.out);
    switch (a.chunk) {
        case 64:
            hipLaunchKernelGGL((prefill_f32_kernel<DK, DV, 64>), grid, block, 0, a.stream, q, k, v,
                               a.log_gamma, a.state_in, out, a.state_out, a.N);
            break;
        case 128:
            hipLaunchKernelGGL((prefill_f32_kernel<DK, DV, 128>), grid, block, 0, a.stream, q, k,
                               v, a.log_gamma, a.state_in, out, a.state_out, a.N);
            break;
        case 256:
            hipLaunchKernelGGL((prefill_f32_kernel<DK, DV, 256>), grid, block, 0, a.stream, q, k,
                               v, a.log_gamma, a.state_in, out, a.state_out, a.N);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a) {
    if (a.dk == 64 && a.dv == 64) return launch_f32_dims<64, 64>(a);
    if (a.dk == 64 && a.dv == 128) return launch_f32_dims<64, 128>(a);
    if (a.dk == 128 && a.dv == 64) return launch_f32_dims<128, 64>(a);
    if (a.dk == 128 && a.dv == 128) return launch_f32_dims<128, 128>(a);
    return hipErrorInvalidValue;
}

}  // namespace gret
