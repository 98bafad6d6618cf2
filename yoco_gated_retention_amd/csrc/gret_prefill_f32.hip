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
// dv); the state slice [dk][32] lives in LDS for the whole sequence. A chunk
// is processed in sub-chunks of 64 positions staged in LDS (queries, keys and
// the value slice, all fp32): the log-decay scan of the whole chunk (wavefront
// scans with DPP row operations, then the wavefront totals), the decayed
// scores of each pair of a query sub-chunk and an earlier-or-equal key
// sub-chunk (4 x 4 register tiles per thread), the cross-chunk term from the
// state, and the state update accumulated in registers over the key
// sub-chunks. This path serves the fp32 tolerance tier on small problems.
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kF32Threads = 256;
constexpr int kSlice = 32;  // value columns per workgroup
constexpr int kSub = 64;    // positions per staged sub-chunk

template <int CTRL, int ROW_MASK>
__device__ inline float dpp_or_zero(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, ROW_MASK, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wavefront: shifts by 1, 2, 4 and 8
// lanes inside each 16-lane row, then the row totals carried across rows by the
// row broadcasts of lanes 15 and 31. Lanes with no source add 0.
__device__ inline float wave_inclusive_sum(float x) {
    constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
    x += dpp_or_zero<kRowShr | 1, 0xF>(x);
    x += dpp_or_zero<kRowShr | 2, 0xF>(x);
    x += dpp_or_zero<kRowShr | 4, 0xF>(x);
    x += dpp_or_zero<kRowShr | 8, 0xF>(x);
    x += dpp_or_zero<kRowBcast15, 0xA>(x);
    x += dpp_or_zero<kRowBcast31, 0xC>(x);
    return x;
}

template <int DK>
struct F32Lds {
    static constexpr int QP = DK + 4;  // padded row pitch of the query / key tiles
    static constexpr int PP = kSub + 4;
    float s[DK][kSlice];     // state slice
    float q[kSub][QP];       // query sub-chunk
    float k[kSub][QP];       // key sub-chunk
    float v[kSub][kSlice];   // value sub-chunk, this workgroup's columns
    float p[kSub][PP];       // decayed scores of one (query, key) sub-chunk pair
    float beta[256];         // chunk-local inclusive log-decay (up to chunk 256)
    float wsum[4];           // wavefront totals of the scan
};

// rows [r0, r0 + kSub) of a head's [N, D] matrix into LDS (rows past n read 0)
template <int D, int PITCH>
__device__ inline void stage_rows(float (*dst)[PITCH], const float* src, int n, int r0) {
    constexpr int V4 = D / 4;  // float4 per row
    for (int e = threadIdx.x; e < kSub * V4; e += kF32Threads) {
        const int r = e / V4, c4 = e % V4;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r0 + r < n) x = reinterpret_cast<const float4*>(src + static_cast<int64_t>(r0 + r) * D)[c4];
        *reinterpret_cast<float4*>(&dst[r][4 * c4]) = x;
    }
}

// value columns [c0, c0 + 32) of rows [r0, r0 + kSub)
template <int DV>
__device__ inline void stage_values(float (*dst)[kSlice], const float* src, int n, int r0, int c0) {
    for (int e = threadIdx.x; e < kSub * (kSlice / 4); e += kF32Threads) {
        const int r = e / (kSlice / 4), c4 = e % (kSlice / 4);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r0 + r < n)
            x = reinterpret_cast<const float4*>(src + static_cast<int64_t>(r0 + r) * DV + c0)[c4];
        *reinterpret_cast<float4*>(&dst[r][4 * c4]) = x;
    }
}

template <int DK, int DV, int C>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ log_gamma, const float* state_in, float* __restrict__ out,
    float* state_out, int64_t N) {
    static_assert(C % kSub == 0 && C <= 256, "chunk");
    using LdsT = F32Lds<DK>;
    __shared__ __attribute__((aligned(16))) LdsT L;
    constexpr int kSlices = DV / kSlice;
    constexpr int SUBS = C / kSub;
    // state-update ownership: row i of the slice, TC consecutive columns
    constexpr int TPR = kF32Threads / DK;  // threads per state row (2 or 4)
    constexpr int TC = kSlice / TPR;       // columns per thread (16 or 8)
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
        L.s[i][c] = state_in ? state_in[head * DK * DV + i * DV + c0 + c] : 0.0f;
    }

    for (int64_t a = 0; a < N; a += C) {
        const int n = static_cast<int>(N - a < C ? N - a : C);
        const float* qa = qh + a * DK;
        const float* ka = kh + a * DK;
        const float* va = vh + a * DV;
        // 1. chunk-local inclusive log-decay (positions past n add 0)
        {
            const int w = tid >> 6;
            float x = tid < n ? clamp_log_gamma(lh[a + tid], kLogGammaFloor) : 0.0f;
            x = wave_inclusive_sum(x);
            if ((tid & 63) == 63) L.wsum[w] = x;
            __syncthreads();  // also: the previous chunk's state update is complete
            for (int u = 0; u < w; ++u) x += L.wsum[u];
            if (tid < C) L.beta[tid] = x;
        }
        __syncthreads();
        const float g = L.beta[C - 1];  // = beta of the last real position

        // 2. outputs, one query sub-chunk at a time
        for (int r = 0; r < SUBS && r * kSub < n; ++r) {
            __syncthreads();  // previous users of the query tile are done
            stage_rows<DK, LdsT::QP>(L.q, qa, n, r * kSub);
            // this thread's outputs: row j, columns cj .. cj + 7
            const int j = tid >> 2, cj = (tid & 3) * 8;
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
            for (int sb = 0; sb <= r; ++sb) {
                __syncthreads();  // query tile staged; previous key / score users done
                stage_rows<DK, LdsT::QP>(L.k, ka, n, sb * kSub);
                stage_values<DV>(L.v, va, n, sb * kSub, c0);
                __syncthreads();
                // scores: a 4 x 4 tile per thread, rows 4 (tid / 16) .., columns 4 (tid % 16) ..
                {
                    const int jr = 4 * (tid >> 4), lc = 4 * (tid & 15);
                    float pt[4][4] = {};
                    for (int i = 0; i < DK; i += 4) {
                        float4 qq[4], kk[4];
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            qq[x] = *reinterpret_cast<const float4*>(&L.q[jr + x][i]);
                            kk[x] = *reinterpret_cast<const float4*>(&L.k[lc + x][i]);
                        }
#pragma unroll
                        for (int x = 0; x < 4; ++x)
#pragma unroll
                            for (int y = 0; y < 4; ++y) {
                                pt[x][y] = fmaf(qq[x].x, kk[y].x, pt[x][y]);
                                pt[x][y] = fmaf(qq[x].y, kk[y].y, pt[x][y]);
                                pt[x][y] = fmaf(qq[x].z, kk[y].z, pt[x][y]);
                                pt[x][y] = fmaf(qq[x].w, kk[y].w, pt[x][y]);
                            }
                    }
#pragma unroll
                    for (int x = 0; x < 4; ++x)
#pragma unroll
                        for (int y = 0; y < 4; ++y) {
                            const int jj = r * kSub + jr + x, ll = sb * kSub + lc + y;
                            L.p[jr + x][lc + y] =
                                ll <= jj ? pt[x][y] * __expf(L.beta[jj] - L.beta[ll]) : 0.0f;
                        }
                }
                __syncthreads();
                // intra-chunk part: scores of row j times the value slice
                for (int l = 0; l < kSub; ++l) {
                    const float pj = L.p[j][l];
                    const float4 v0 = *reinterpret_cast<const float4*>(&L.v[l][cj]);
                    const float4 v1 = *reinterpret_cast<const float4*>(&L.v[l][cj + 4]);
                    acc[0] = fmaf(pj, v0.x, acc[0]);
                    acc[1] = fmaf(pj, v0.y, acc[1]);
                    acc[2] = fmaf(pj, v0.z, acc[2]);
                    acc[3] = fmaf(pj, v0.w, acc[3]);
                    acc[4] = fmaf(pj, v1.x, acc[4]);
                    acc[5] = fmaf(pj, v1.y, acc[5]);
                    acc[6] = fmaf(pj, v1.z, acc[6]);
                    acc[7] = fmaf(pj, v1.w, acc[7]);
                }
            }
            // cross-chunk part exp(beta_j) q_j S (the state before this chunk)
            float cr[8] = {};
            for (int i = 0; i < DK; ++i) {
                const float qv = L.q[j][i];
                const float4 s0 = *reinterpret_cast<const float4*>(&L.s[i][cj]);
                const float4 s1 = *reinterpret_cast<const float4*>(&L.s[i][cj + 4]);
                cr[0] = fmaf(qv, s0.x, cr[0]);
                cr[1] = fmaf(qv, s0.y, cr[1]);
                cr[2] = fmaf(qv, s0.z, cr[2]);
                cr[3] = fmaf(qv, s0.w, cr[3]);
                cr[4] = fmaf(qv, s1.x, cr[4]);
                cr[5] = fmaf(qv, s1.y, cr[5]);
                cr[6] = fmaf(qv, s1.z, cr[6]);
                cr[7] = fmaf(qv, s1.w, cr[7]);
            }
            const int jj = r * kSub + j;
            if (jj < n) {
                const float f = __expf(L.beta[jj]);
                float4 o0, o1;
                o0.x = fmaf(f, cr[0], acc[0]);
                o0.y = fmaf(f, cr[1], acc[1]);
                o0.z = fmaf(f, cr[2], acc[2]);
                o0.w = fmaf(f, cr[3], acc[3]);
                o1.x = fmaf(f, cr[4], acc[4]);
                o1.y = fmaf(f, cr[5], acc[5]);
                o1.z = fmaf(f, cr[6], acc[6]);
                o1.w = fmaf(f, cr[7], acc[7]);
                float* dst = oh + (a + jj) * DV + c0 + cj;
                reinterpret_cast<float4*>(dst)[0] = o0;
                reinterpret_cast<float4*>(dst)[1] = o1;
            }
        }

        // 3. state update: S <- exp(g) S + sum_l exp(g - beta_l) k_l^T v_l
        const int si = tid / TPR, sc = (tid % TPR) * TC;
        float upd[TC];
#pragma unroll
        for (int e = 0; e < TC; ++e) upd[e] = 0.0f;
        for (int sb = 0; sb < SUBS && sb * kSub < n; ++sb) {
            __syncthreads();  // previous users of the key / value tiles are done
            stage_rows<DK, LdsT::QP>(L.k, ka, n, sb * kSub);
            stage_values<DV>(L.v, va, n, sb * kSub, c0);
            __syncthreads();
            for (int l = 0; l < kSub; ++l) {
                const int ll = sb * kSub + l;
                const float kv = ll < n ? __expf(g - L.beta[ll]) * L.k[l][si] : 0.0f;
#pragma unroll
                for (int e = 0; e < TC; e += 4) {
                    const float4 vv = *reinterpret_cast<const float4*>(&L.v[l][sc + e]);
                    upd[e] = fmaf(kv, vv.x, upd[e]);
                    upd[e + 1] = fmaf(kv, vv.y, upd[e + 1]);
                    upd[e + 2] = fmaf(kv, vv.z, upd[e + 2]);
                    upd[e + 3] = fmaf(kv, vv.w, upd[e + 3]);
                }
            }
        }
        __syncthreads();  // every thread's cross term has read the old state
        const float eg = __expf(g);
#pragma unroll
        for (int e = 0; e < TC; ++e) L.s[si][sc + e] = fmaf(eg, L.s[si][sc + e], upd[e]);
    }
    __syncthreads();
    if (state_out) {
        for (int e = tid; e < DK * kSlice; e += kF32Threads) {
            const int i = e / kSlice, c = e % kSlice;
            state_out[head * DK * DV + i * DV + c0 + c] = L.s[i][c];
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
