// gret_prefill_common.h -- device pieces shared by the two bf16 prefill
// translation units (chunks of 64 positions in gret_prefill_c64.hip, chunks
// of 128 and 256 in gret_prefill_bf16.hip): matrix-core and LDS primitives,
// the swizzled tile layout, range-checked buffer access, kernel parameters and
// the segment-combine kernel. Everything is internal to each translation unit.
#pragma once
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kTile = 64;  // positions per tile
constexpr int kPadP = 8;   // bf16 padding per row of the score tile


// Range-checked buffer access (CDNA buffer resources). A descriptor covers one
// head's rows; a load past its end returns zeros and a store past it is
// dropped by the hardware, which is exactly the tail masking the chunkwise form
// needs (padded positions carry zero K and V and log-gate 0, and their outputs
// are not written), without a branch on the hot path.
__device__ inline bf16x8 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    return __builtin_bit_cast(bf16x8, v);
}
__device__ inline float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ inline void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, const bf16x4& v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), r, byte_off, 0, 0);
}

struct Params {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const float* log_gamma;
    const float* state_in;
    bf16_t* out;
    float* state_out;
    float* ws_state;  // [BH][max_seg][DK*DV]
    float2* ws_meta;  // [BH][max_seg]: (total log-decay, leading chunks)
    SegPlan plan;
    int64_t N;
    // output epilogue applied in the kernel's output store (chunk 64 only):
    // gate [BH][N][DV] and the per-head affine [H][DV] (null: 1 and 0)
    const bf16_t* gate;
    const float* gate_w;
    const float* gate_b;
    float eps;
    int64_t H;
};

inline Params make_params(const PrefillArgs& a, const SegPlan& plan, int64_t dk, int64_t dv) {
    Params p;
    p.q = static_cast<const bf16_t*>(a.q);
    p.k = static_cast<const bf16_t*>(a.k);
    p.v = static_cast<const bf16_t*>(a.v);
    p.log_gamma = a.log_gamma;
    p.state_in = a.state_in;
    p.out = static_cast<bf16_t*>(a.out);
    p.state_out = a.state_out;
    const PrefillWorkspace lay = bf16_workspace_layout(plan, dk, dv);
    p.ws_state = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + lay.state_off);
    p.ws_meta = reinterpret_cast<float2*>(static_cast<char*>(a.workspace) + lay.meta_off);
    p.plan = plan;
    p.N = a.N;
    p.gate = static_cast<const bf16_t*>(a.epi.gate);
    p.gate_w = a.epi.weight;
    p.gate_b = a.epi.bias;
    p.eps = a.epi.eps;
    p.H = a.H;
    return p;
}

// Per-head views of the prefill tensors.
struct HeadRsrc {
    __amdgpu_buffer_rsrc_t q, k, v, lg, out;
};

template <int DK, int DV>
constexpr int64_t kRsrcRows = prefill_pass_rows(DK, DV);

// Buffer ranges over the rows of head x from row0 on (to the head's end, at
// most kRsrcRows rows): a pass addresses its rows relative to its own first
// row, so no limit applies to the head's length, only to one pass's span.
// Rows past the range read as zero and stores there are dropped.
template <int DK, int DV>
__device__ inline HeadRsrc head_rsrc(const Params& p, int64_t x, int64_t row0) {
    const int64_t N = p.N;
    const int64_t left = N - row0;
    const int64_t rows = left < kRsrcRows<DK, DV> ? left : kRsrcRows<DK, DV>;
    const int64_t r0 = x * N + row0;
    HeadRsrc hr;
    hr.q = make_rsrc(p.q + r0 * DK, static_cast<uint32_t>(rows * DK * 2));
    hr.k = make_rsrc(p.k + r0 * DK, static_cast<uint32_t>(rows * DK * 2));
    hr.v = make_rsrc(p.v + r0 * DV, static_cast<uint32_t>(rows * DV * 2));
    hr.lg = make_rsrc(p.log_gamma + r0, static_cast<uint32_t>(rows * 4));
    hr.out = make_rsrc(p.out + r0 * DV, static_cast<uint32_t>(rows * DV * 2));
    return hr;
}

// XOR swizzle of the 16-byte chunks of a row-major tile row. The LDS serves
// 16 lanes x 16 bytes per cycle, so 16 consecutive rows read at one chunk must
// land in 16 different chunk slots; and one 16-lane group of a transposing
// read touches 4 consecutive rows x 2 adjacent chunks (an even chunk and the
// next), at rows t0..t0+3 and t0+8..t0+11 for the two groups served together.
// For 16-chunk rows (128 columns) the slot is c ^ (4 (r % 4) + (r / 4) % 4):
// a bijection on 16 rows, and its bits 1..3 (which decide the 32-byte pair of
// an even/odd chunk) take 8 different values over each such set of 8 rows.
// 8-chunk rows (64 columns) use c ^ (2 (r % 4) + (r / 4) % 2).
template <int D>
__device__ inline int swz(int row) {
    if constexpr (D / 8 >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    return 2 * (row & 3) + ((row >> 2) & 1);
}

// Element offset of (row, col) in a swizzled row-major tile with D columns.
template <int D>
__device__ inline int toff(int row, int col) {
    return row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
}

// 8 consecutive positions t0..t0+7 of column col0 + l (l = this lane's index
// in its 16-lane group) from a row-major swizzled tile with D columns: the
// MFMA operand for a contraction over positions.
template <int D>
__device__ inline bf16x8 read_cols8(const bf16_t* tile, int t0, int col0) {
    const int s = threadIdx.x & 15;
    const int row = t0 + (s >> 2);
    const int col = col0 + 4 * (s & 3);
    const bf16x4 a = lds_read_tr4(tile + toff<D>(row, col));
    const bf16x4 b = lds_read_tr4(tile + toff<D>(row + 4, col));
    return cat44(a, b);
}

// The 10 16x16 blocks on or below the diagonal of a 64x64 score tile, largest
// rows first: (3,3) (3,2) (2,2) (3,1) (2,1) (1,1) (3,0) (2,0) (1,0) (0,0),
// packed as 4-bit (4 jb + b) entries of an immediate (a table in memory would
// be a global load that the compiler waits for together with the prefetches).
constexpr uint64_t kCausalBlocks = 0xFull | 0xEull << 4 | 0xAull << 8 | 0xDull << 12 |
                                   0x9ull << 16 | 0x5ull << 20 | 0xCull << 24 | 0x8ull << 28 |
                                   0x4ull << 32 | 0x0ull << 36;

// Chains the segment maps of each head: S_in(s) = S_end(s-1),
// S_end(s) = exp(G_s) S_in(s) + S_loc(s). Leaves S_in(s) in slot s and writes
// the final state.
constexpr int kCombineThreads = 256;

template <int DK, int DV>
__global__ __launch_bounds__(kCombineThreads) void prefill_combine_kernel(Params p) {
    const SegPlan& pl = p.plan;
    constexpr int PER_BLOCK = kCombineThreads * 4;
    constexpr int BLOCKS_PER_HEAD = DK * DV / PER_BLOCK;
    const int64_t x = blockIdx.x / BLOCKS_PER_HEAD;
    const int64_t e0 = (blockIdx.x % BLOCKS_PER_HEAD) * PER_BLOCK + threadIdx.x * 4;
    const int64_t nseg = seg_count(pl, x);
    float* base = p.ws_state + x * pl.max_seg * (int64_t)(DK * DV) + e0;
    f32x4 s = *reinterpret_cast<const f32x4*>(base);
    for (int64_t sI = 1; sI < nseg; ++sI) {
        float* slot = base + sI * (int64_t)(DK * DV);
        const float eg = __expf(p.ws_meta[x * pl.max_seg + sI].x);
        const f32x4 loc = *reinterpret_cast<const f32x4*>(slot);
        *reinterpret_cast<f32x4*>(slot) = s;
        s[0] = fmaf(eg, s[0], loc[0]);
        s[1] = fmaf(eg, s[1], loc[1]);
        s[2] = fmaf(eg, s[2], loc[2]);
        s[3] = fmaf(eg, s[3], loc[3]);
    }
    if (p.state_out) *reinterpret_cast<f32x4*>(p.state_out + x * DK * DV + e0) = s;
}

template <int DK, int DV>
hipError_t launch_combine(const Params& p, hipStream_t stream) {
    const int per_head = DK * DV / (kCombineThreads * 4);
    hipLaunchKernelGGL((prefill_combine_kernel<DK, DV>), dim3(p.plan.BH * per_head),
                       dim3(kCombineThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace
}  // namespace gret
