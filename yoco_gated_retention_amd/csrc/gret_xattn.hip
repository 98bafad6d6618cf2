// gret_xattn.hip -- Cross-Decoder decode attention over the shared global KV
// cache on gfx950 (bf16 operands on matrix cores, fp32 softmax and sums).
//
// Page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次", sections
// "增量生成时究竟追加什么" and "接入推理引擎时的四个关键点": at a decode step every
// Cross-Decoder layer's query for the new token attends over the single global
// cache of keys and values; with GQA, G = Hq / Hkv query heads share one KV
// head. Reading the whole cache every step makes this the bandwidth hotspot
// of decode: 2 * d * 2 bytes per cached position and KV head.
//
//   out[b, h] = softmax(scale * q[b, h] K[b, g]^T) V[b, g],  g = h / G,
//   over the first length[b] cached positions.
//
// Split-K schedule (flash decoding): one workgroup per (sequence, KV head,
// range of positions). Its 4 wavefronts stream their own 32-position tiles of
// K and V from HBM into per-wavefront LDS buffers (buffer_load ... lds,
// double-buffered; no workgroup barrier in the loop) and keep an online
// softmax per query head:
//   * scores S^T = K Q^T (16x16x32 bf16 MFMA; the group's G <= 16 query heads
//     are the B-operand columns, so every K/V byte is read once per step);
//   * running max / sum in fp32, probabilities rounded to bf16;
//   * O^T += V^T P^T with V read by the transposing LDS load; the positions of
//     the V^T operand are permuted to match the score layout, so P never
//     leaves the registers.
// The wavefronts merge through LDS, the workgroup writes its partial (max,
// sum, unnormalised output) per head, and a second kernel merges the ranges
// with log-sum-exp weights. When the plan has one range per (sequence, KV
// head) -- many short caches, such as the sliding-window rings -- the
// workgroup writes the normalised output itself and the second launch is
// skipped.
#include <hip/hip_runtime.h>
#include <math.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kXTile = 32;     // positions per tile
constexpr int kXWaves = 4;     // wavefronts per workgroup
template <int D>
constexpr int64_t kXRangeRows = xattn_range_rows(D);
constexpr int kXThreads = 64 * kXWaves;


// Tile layouts (row-major, 16-byte chunks of row r permuted by c ^ sigma(r));
// K is read as 16-byte row fragments, V with the transposing load.
template <int D, bool IS_V>
__device__ inline int xswz(int r) {
    if constexpr (D == 128) {
        if constexpr (IS_V) return ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3);
        return ((r & 1) << 2) | ((r >> 1) & 3) | (((r >> 3) & 1) << 3);
    } else {
        return r & 7;
    }
}
template <int D, bool IS_V>
__device__ inline int xoff(int row, int col) {
    return row * D + (((col >> 3) ^ xswz<D, IS_V>(row)) << 3) + (col & 7);
}


// One 1 KB DMA instruction of a tile with D columns (lane i -> LDS byte 16 i of
// block blk = row (512/D) blk + i / (D/8), slot i % (D/8)).
template <int D, bool IS_V>
__device__ inline void dma_block(__amdgpu_buffer_rsrc_t r, bf16_t* tile, int blk, uint32_t pos0) {
    constexpr int RPI = 512 / D;
    constexpr int SPR = D / 8;
    const int lane = threadIdx.x & 63;
    const int row = RPI * blk + lane / SPR;
    const int chunk = (lane % SPR) ^ xswz<D, IS_V>(row);
    const uint32_t voff = ((pos0 + row) * D + chunk * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + blk * 512), 16, voff, 0, 0,
                                             2 /* nontemporal: streamed once per step */);
}

template <int D>
struct XCfg {
    static constexpr int KS = D / 32;                 // k-steps of the score product
    static constexpr int VT = D / 16;                 // 16-column tiles of the output
    static constexpr int BLK = kXTile * D * 2 / 1024; // 1 KB DMA blocks per tile and tensor
    static constexpr int DMA = 2 * BLK;               // DMA instructions per tile
    static constexpr int TILE = kXTile * D;           // elements per tile buffer
};

struct XParams {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const int32_t* lengths;
    bf16_t* out;
    float2* part_ml;  // [B][Hkv][S][G]: (max, sum)
    float* part_acc;  // [B][Hkv][S][G][D]
    int64_t B, Hq, Hkv, L, S, SL;
    int G;
    float scale;
};

// One 32-position tile of this wavefront: scores, online softmax, P V.
template <int D, int BUF>
__device__ inline void x_tile(const bf16_t* kt, const bf16_t* vt, const bf16x8 (&qf)[XCfg<D>::KS],
                              uint32_t pos0, uint32_t hi, float scale, float& m_run, float& l_run,
                              f32x4 (&acc)[XCfg<D>::VT]) {
    using c = XCfg<D>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4, s = lane & 15;
    float sc[2][4];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < c::KS; ++ks)
            a = mfma16(lds_read8(kt + xoff<D, false>(16 * pt + li, 32 * ks + 8 * g)), qf[ks], a);
        // a[i] = q[head li] . k[pos0 + 16 pt + 4 g + i]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t pos = pos0 + 16 * pt + 4 * g + i;
            sc[pt][i] = pos < hi ? a[i] * scale : -INFINITY;
        }
    }
    float mt = sc[0][0];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[pt][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);  // finite: the tile holds a valid position
    const float corr = __expf(m_run - m_new);
    bf16x8 pf;
    float psum = 0.0f;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = __expf(sc[pt][i] - m_new);
            psum += p;
            pf[4 * pt + i] = to_bf16(p);
        }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < c::VT; ++t) {
        acc[t][0] *= corr;
        acc[t][1] *= corr;
        acc[t][2] *= corr;
        acc[t][3] *= corr;
        const int col = 16 * t + 4 * (s & 3);
        const bf16x8 vf = cat44(lds_read_tr4(vt + xoff<D, true>(4 * g + (s >> 2), col)),
                                lds_read_tr4(vt + xoff<D, true>(16 + 4 * g + (s >> 2), col)));
        acc[t] = mfma16(vf, pf, acc[t]);
    }
}

template <int D>
__global__ __launch_bounds__(kXThreads) void xattn_split_kernel(XParams p) {
    using c = XCfg<D>;
    // per-wavefront double buffers, one LDS object per buffer index
    __shared__ __attribute__((aligned(16))) bf16_t k0_[kXWaves * c::TILE], k1_[kXWaves * c::TILE];
    __shared__ __attribute__((aligned(16))) bf16_t v0_[kXWaves * c::TILE], v1_[kXWaves * c::TILE];
    __shared__ float s_ml[kXWaves][16][2];
    static_assert(16 * D * sizeof(float) <= c::TILE * sizeof(bf16_t), "partials fit a tile buffer");

    const int64_t blk = blockIdx.x;
    const int64_t split = blk % p.S;
    const int64_t bg = blk / p.S;
    const int64_t b = bg / p.Hkv, kvh = bg % p.Hkv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    int64_t len = p.lengths ? p.lengths[b] : p.L;
    len = len < 0 ? 0 : (len > p.L ? p.L : len);  // keeps every access inside the cache
    const int64_t lo = split * p.SL;
    const int64_t hi64 = lo + p.SL < len ? lo + p.SL : len;
    float2* ml = p.part_ml + (bg * p.S + split) * p.G;
    float* pacc = p.part_acc + (bg * p.S + split) * p.G * D;
    if (lo >= hi64) {  // nothing of this sequence in the range
        for (int i = threadIdx.x; i < p.G * D; i += kXThreads) pacc[i] = 0.0f;
        if (threadIdx.x < p.G) ml[threadIdx.x] = make_float2(-INFINITY, 0.0f);
        return;
    }
    const uint32_t hi = static_cast<uint32_t>(hi64 - lo);
    const int64_t head0 = kvh * p.G;
    bf16x8 qf[c::KS];
#pragma unroll
    for (int ks = 0; ks < c::KS; ++ks) {
        if (li < p.G)
            qf[ks] = *reinterpret_cast<const bf16x8*>(p.q + ((b * p.Hq + head0 + li) * D +
                                                             32 * ks + 8 * g));
        else
            qf[ks] = bf16x8{};
    }
    // buffer ranges start at this range's first position (32-bit offsets: a
    // range of the plan spans at most kXRangeRows rows), so positions below
    // are relative to lo
    const int64_t kv_base = (bg * p.L + lo) * D;
    const int64_t rows = p.L - lo < kXRangeRows<D> ? p.L - lo : kXRangeRows<D>;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(p.k + kv_base, static_cast<uint32_t>(rows * D * 2));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(p.v + kv_base, static_cast<uint32_t>(rows * D * 2));

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 acc[c::VT];
#pragma unroll
    for (int t = 0; t < c::VT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int buf, uint32_t pos0) {
#pragma unroll
        for (int i = 0; i < c::BLK; ++i) {
            if (buf == 0) {
                dma_block<D, false>(kr, k0_ + w * c::TILE, i, pos0);
                dma_block<D, true>(vr, v0_ + w * c::TILE, i, pos0);
            } else {
                dma_block<D, false>(kr, k1_ + w * c::TILE, i, pos0);
                dma_block<D, true>(vr, v1_ + w * c::TILE, i, pos0);
            }
        }
    };
    const uint32_t step = kXTile * kXWaves;
    uint32_t pos = kXTile * w;
    if (pos < hi) issue(0, pos);
    // unrolled by two so that every access's buffer is a compile-time fact
    while (pos < hi) {
        const uint32_t nxt = pos + step;
        if (nxt < hi) {
            issue(1, nxt);
            wait_vm<c::DMA>();
        } else {
            wait_vm<0>();
        }
        x_tile<D, 0>(k0_ + w * c::TILE, v0_ + w * c::TILE, qf, pos, hi, p.scale, m_run, l_run, acc);
        __builtin_amdgcn_s_waitcnt(kLgkmWaitZero);  // reads of buffer 0 done before it refills
        pos = nxt;
        if (pos >= hi) break;
        const uint32_t nxt2 = pos + step;
        if (nxt2 < hi) {
            issue(0, nxt2);
            wait_vm<c::DMA>();
        } else {
            wait_vm<0>();
        }
        x_tile<D, 1>(k1_ + w * c::TILE, v1_ + w * c::TILE, qf, pos, hi, p.scale, m_run, l_run, acc);
        __builtin_amdgcn_s_waitcnt(kLgkmWaitZero);
        pos = nxt2;
    }
    wait_vm<0>();

    // wavefront partials: l summed over the four lanes of a head column
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (g == 0) {
        s_ml[w][li][0] = m_run;
        s_ml[w][li][1] = l_run;
    }
    // this wavefront's output partials go to its own (now idle) K buffer 0
    float* my_acc = reinterpret_cast<float*>(k0_ + w * c::TILE);
#pragma unroll
    for (int t = 0; t < c::VT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) my_acc[li * D + 16 * t + 4 * g + i] = acc[t][i];
    __syncthreads();
    // merge the wavefronts (a wavefront with no tile has max -inf, sum 0)
    for (int e = threadIdx.x; e < p.G * D; e += kXThreads) {
        const int h = e / D, j = e % D;
        float M = s_ml[0][h][0];
#pragma unroll
        for (int ww = 1; ww < kXWaves; ++ww) M = fmaxf(M, s_ml[ww][h][0]);
        float lsum = 0.0f, a = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kXWaves; ++ww) {
            const float f = s_ml[ww][h][0] == -INFINITY ? 0.0f : __expf(s_ml[ww][h][0] - M);
            lsum += f * s_ml[ww][h][1];
            a += f * reinterpret_cast<const float*>(k0_ + ww * c::TILE)[h * D + j];
        }
        if (p.S == 1) {
            // one range per (sequence, KV head): this is the whole softmax, and
            // the output is what the merge of a single range would give
            p.out[(b * p.Hq + head0 + h) * D + j] = to_bf16(a / lsum);
        } else {
            pacc[e] = a;
            if (j == 0) ml[h] = make_float2(M, lsum);
        }
    }
}

// Merges the ranges of every (sequence, query head): out = sum_s e^(m_s - M) a_s
// / sum_s e^(m_s - M) l_s. The range weights are computed once into LDS (block
// reductions for the max and the sum); then every thread accumulates one output
// value over a share of the ranges, with coalesced, unrolled loads.
constexpr int kXCombineThreads = 256;
constexpr int kXMaxRanges = static_cast<int>(kXAttnTargetGroups);

__device__ inline float block_reduce(float v, float* red, bool is_max) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(v, off);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    __syncthreads();  // red is free
    if (lane == 0) red[w] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int i = 1; i < kXCombineThreads / 64; ++i) v = is_max ? fmaxf(v, red[i]) : v + red[i];
    return v;
}

template <int D>
__global__ __launch_bounds__(kXCombineThreads) void xattn_combine_kernel(XParams p) {
    constexpr int PER = kXCombineThreads / D;  // threads per output value
    __shared__ float sw[kXMaxRanges];
    __shared__ float red[kXCombineThreads / 64];
    __shared__ float part[kXCombineThreads];
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.Hq, h = bh % p.Hq;
    const int64_t kvh = h / p.G;
    const int gi = static_cast<int>(h % p.G);
    const int64_t base = (b * p.Hkv + kvh) * p.S;
    const int S = static_cast<int>(p.S);
    float M = -INFINITY;
    for (int s = threadIdx.x; s < S; s += kXCombineThreads)
        M = fmaxf(M, p.part_ml[(base + s) * p.G + gi].x);
    M = block_reduce(M, red, true);
    float lsum = 0.0f;
    for (int s = threadIdx.x; s < S; s += kXCombineThreads) {
        const float2 ml = p.part_ml[(base + s) * p.G + gi];
        const float f = ml.x == -INFINITY ? 0.0f : __expf(ml.x - M);
        sw[s] = f;
        lsum += f * ml.y;
    }
    lsum = block_reduce(lsum, red, false);  // its barriers also publish sw
    const int j = threadIdx.x % D, r = threadIdx.x / D;
    const float* acc = p.part_acc + (base * p.G + gi) * D + j;
    const int64_t stride = static_cast<int64_t>(p.G) * D;
    float a = 0.0f;
#pragma unroll 8
    for (int s = r; s < S; s += PER) a += sw[s] * acc[s * stride];
    part[threadIdx.x] = a;
    __syncthreads();
    if (r == 0) {
#pragma unroll
        for (int k = 1; k < PER; ++k) a += part[k * D + j];
        p.out[bh * D + j] = to_bf16(a / lsum);
    }
}

template <int D>
hipError_t launch_d(const XAttnArgs& a) {
    XParams p;
    p.q = static_cast<const bf16_t*>(a.q);
    p.k = static_cast<const bf16_t*>(a.k);
    p.v = static_cast<const bf16_t*>(a.v);
    p.lengths = a.lengths;
    p.out = static_cast<bf16_t*>(a.out);
    const XAttnPlan plan = xattn_plan(a.B, a.Hq, a.Hkv, a.L, a.d);
    p.part_ml = reinterpret_cast<float2*>(a.workspace);
    p.part_acc = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + plan.acc_off);
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.L = a.L;
    p.S = plan.S;
    p.SL = plan.SL;
    p.G = static_cast<int>(a.Hq / a.Hkv);
    p.scale = a.scale;
    hipLaunchKernelGGL((xattn_split_kernel<D>), dim3(static_cast<unsigned>(a.B * a.Hkv * plan.S)),
                       dim3(kXThreads), 0, a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.S == 1) return e;  // one range: the split kernel wrote out
    hipLaunchKernelGGL((xattn_combine_kernel<D>), dim3(static_cast<unsigned>(a.B * a.Hq)),
                       dim3(kXCombineThreads), 0, a.stream, p);
    return hipGetLastError();
}

}  // namespace

XAttnPlan xattn_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d) {
    XAttnPlan pl;
    const int64_t G = Hq / Hkv;
    // about kXAttnTargetGroups workgroups, ranges of at least 512 positions,
    // each a multiple of the 4 x 32 positions a workgroup takes per round
    const int64_t bg = B * Hkv;
    int64_t S = (kXAttnTargetGroups + bg - 1) / bg;
    const int64_t max_s = (L + 511) / 512;
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    const int64_t round = static_cast<int64_t>(kXTile) * kXWaves;
    // a range (plus the tile a wavefront may load past it) must fit the 32-bit
    // offsets of its buffer ranges
    const int64_t max_sl = (xattn_range_rows(d) - round) / round * round;
    const int64_t min_s = (L + max_sl - round - 1) / (max_sl - round);
    if (S < min_s) S = min_s;
    int64_t SL = (L + S - 1) / S;
    SL = (SL + round - 1) / round * round;
    S = (L + SL - 1) / SL;
    pl.S = S;
    pl.SL = SL;
    const size_t parts = static_cast<size_t>(bg) * static_cast<size_t>(S) * static_cast<size_t>(G);
    pl.acc_off = (parts * sizeof(float) * 2 + 255) & ~size_t(255);
    pl.bytes = pl.acc_off + parts * static_cast<size_t>(d) * sizeof(float);
    pl.bytes = (pl.bytes + 255) & ~size_t(255);
    return pl;
}

hipError_t launch_xattn_decode(const XAttnArgs& a) {
    if (a.d == 64) return launch_d<64>(a);
    if (a.d == 128) return launch_d<128>(a);
    return hipErrorInvalidValue;
}

}  // namespace gret
