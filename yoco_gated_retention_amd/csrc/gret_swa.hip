// gret_swa.hip -- the sliding-window-attention Self-Decoder mixer on gfx950:
// windowed causal prefill on the matrix cores, the ring buffer a prefill
// leaves, and the decode-step append into that ring (the decode attention
// itself runs on the cross-attention kernels over the ring).
//
// Page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次", section
// "路线一：滑动窗口注意力": position i attends to the most recent W positions
// only (causal window mask admitting j in [i - W + 1, i]); decoding keeps just
// those W keys and values per layer, overwriting the oldest (ring slot p mod W;
// W = 1024 in the paper's runs). Section "Prefill 的实现骨架": the prefill
// leaves each layer's last W keys and values in a fixed buffer.
//
// Prefill, per (sequence, query head, 256-query tile): 8 wavefronts own 32
// queries each. Keys and values stream through LDS in two stages of 128
// positions (two 64-key blocks each) over the tile's joint window: a stage is
// refilled by direct buffer-to-LDS loads as soon as every wavefront has
// consumed it, so the loads run one stage (two blocks) ahead with one
// workgroup barrier per 128 keys. A wavefront computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (Q^T stays in registers), so each lane holds 16
// scores of one query and the other half-wave the other 16 of the 32 keys:
// the online softmax needs one cross-lane exchange per block. The
// probabilities stay in registers as the B operand of O^T += V^T P^T, whose
// V^T operand comes from transposing LDS reads in the same key order.
// Workgroups are ordered so that one XCD runs consecutive query tiles of one
// head together and their overlapping windows hit in its L2.
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kSWaves = 8;
constexpr int kSThreads = 64 * kSWaves;
constexpr int kSQ = 32 * kSWaves;  // queries per workgroup
constexpr int kSK = 64;            // keys per block (one softmax update)
constexpr int kSBlocks = 2;        // blocks per LDS stage; two stages, refilled one stage ahead
constexpr int kXcds = 8;


// Tile layouts: row-major, the 16-byte chunks of row r permuted by c ^ sw(r).
// K is read as 16-byte row pieces of 8 consecutive rows (any 8 aligned rows
// land in 8 different 16-byte slots of a 128-byte bank period); V with the
// transposing read, 4 consecutive rows x 32 bytes per 16-lane group, the two
// half-wavefronts 4 rows apart. Measured on the kernel's own addresses (bytes
// per clock and CU, 128-column tiles): K 227 with its layout; V 163 with
// sw = 4 (r % 4) + (r / 4) % 4, against 116 with the K/V layout of the
// chunk-64 prefill, whose rows r and r + 4 share a 32-byte slot pair.
template <int D>
__device__ inline int kswz(int r) {
    if constexpr (D == 128) return ((r & 1) << 2) | ((r >> 1) & 3) | (((r >> 3) & 1) << 3);
    return r & 7;
}
template <int D>
__device__ inline int vswz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    return ((r & 3) << 1) | ((r >> 2) & 1);
}
template <int D, bool IS_V>
__device__ inline int soff(int row, int col) {
    const int sw = IS_V ? vswz<D>(row) : kswz<D>(row);
    return row * D + (((col >> 3) ^ sw) << 3) + (col & 7);
}

template <int D>
struct SCfg {
    static constexpr int KS = D / 16;               // k-steps of S^T = K Q^T
    static constexpr int CB = D / 32;               // 32-channel blocks of O^T
    static constexpr int TILE = kSBlocks * kSK * D;  // elements per K or V stage
    static constexpr int BLK = TILE * 2 / 1024;     // 1 KB loads per K or V stage
    static constexpr int PER_WAVE = BLK / kSWaves;  // of each, per wavefront
    static constexpr int DMA = 2 * PER_WAVE;        // loads per wavefront and stage
};

// One 1 KB direct load of a stage of kSBlocks * 64 positions: lane i fills LDS byte 16 i of
// block blk = row (512 / D) blk + i / (D / 8), slot i % (D / 8), from the
// global chunk slot ^ swizzle of that position.
template <int D, bool IS_V>
__device__ inline void dma_block(__amdgpu_buffer_rsrc_t r, bf16_t* tile, int blk, uint32_t key0) {
    constexpr int RPI = 512 / D;
    constexpr int SPR = D / 8;
    const int lane = threadIdx.x & 63;
    const int row = RPI * blk + lane / SPR;
    const int chunk = (lane % SPR) ^ (IS_V ? vswz<D>(row) : kswz<D>(row));
    const uint32_t voff = ((key0 + row) * D + chunk * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + blk * 512), 16, voff, 0, 0, 0);
}

template <int D>
__device__ inline void dma_stage(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, bf16_t* kt,
                                 bf16_t* vt, uint32_t key0) {
    using c = SCfg<D>;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < c::PER_WAVE; ++i) dma_block<D, false>(kr, kt, w * c::PER_WAVE + i, key0);
#pragma unroll
    for (int i = 0; i < c::PER_WAVE; ++i) dma_block<D, true>(vr, vt, w * c::PER_WAVE + i, key0);
}

// The key/value stages in LDS (file scope, so that every helper names
// the object it touches and the compiler can tell the stages apart when it
// orders LDS reads after the direct loads into other stages); sized for d = 128.
__shared__ __attribute__((aligned(1024))) bf16_t swa_k0[kSBlocks * kSK * 128];
__shared__ __attribute__((aligned(1024))) bf16_t swa_v0[kSBlocks * kSK * 128];
__shared__ __attribute__((aligned(1024))) bf16_t swa_k1[kSBlocks * kSK * 128];
__shared__ __attribute__((aligned(1024))) bf16_t swa_v1[kSBlocks * kSK * 128];
template <int X>
__device__ inline bf16_t* swa_kst() {
    if constexpr (X == 0) return swa_k0;
    return swa_k1;
}
template <int X>
__device__ inline bf16_t* swa_vst() {
    if constexpr (X == 0) return swa_v0;
    return swa_v1;
}

struct SwaParams {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    bf16_t* out;
    int64_t B, Hq, Hkv, N, W;
    int G, q_tiles;
    float scale_log2;  // scale * log2(e)
};

// 2^x with the hardware instruction (results below 2^-126 flush to 0, which
// for softmax weights is below the bf16 resolution of the output anyway).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// How far (log2 units) a score may exceed the softmax reference before the
// reference moves and the output is rescaled.
constexpr float kLazyLog2 = 8.0f;

// Running softmax state and output of one wavefront's 32 queries.
template <int D>
struct SwaAcc {
    f32x16 o[SCfg<D>::CB];
    float m, l;
};

// One 64-key block (keys key0 ..) against this wavefront's queries.
template <int D>
__device__ inline void swa_block(const bf16_t* kt, const bf16_t* vt, const bf16x8 (&qf)[SCfg<D>::KS],
                                 int64_t key0, int64_t qi, int64_t W, bool need_mask, float cl,
                                 SwaAcc<D>& st) {
    using c = SCfg<D>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 31, hh = lane >> 5;
    f32x16 s[2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[half][r] = 0.0f;
    // the two halves are independent accumulation chains: interleave them,
    // with the LDS reads of K two k-steps ahead of the products
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < c::KS; ++ks)
#pragma unroll
        for (int half = 0; half < 2; ++half)
            s[half] = mfma32(lds_read8(kt + soff<D, false>(32 * half + li, 16 * ks + 8 * hh)),
                             qf[ks], s[half]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int g = 0; g < c::KS - 2; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    // s[half][r] = q[qi] . k[key0 + 32 half + 8 (r / 4) + 4 hh + r % 4]
    if (need_mask) {
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t j = key0 + 32 * half + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (!(j <= qi && j > qi - W)) s[half][r] = -INFINITY;
            }
    }
    float mt = s[0][0];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[half][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // st.m is the reference the weights are taken against, not the running
    // maximum: it moves only when a score exceeds it by more than kLazyLog2
    // (in log2 units), so the weights stay <= 2^kLazyLog2 and the output is
    // rescaled rarely; the final division by l makes the reference cancel.
    const bool grow = (mt - st.m) * cl > kLazyLog2;
    const float m_new = grow ? mt : st.m;
    // while a query has seen no admitted key yet its reference is -inf:
    // subtract 0 instead, so masked scores give exactly 0 and nothing is NaN
    const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = grow ? fast_exp2((st.m - m_ref) * cl) : 1.0f;
    const float mc = m_ref * cl;
    bf16x8 pb[2][2];
    float psum = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = fast_exp2(fmaf(s[half][r], cl, -mc));
            psum += pr;
            pb[half][r >> 3][r & 7] = to_bf16(pr);
        }
    st.l = st.l * corr + psum;
    st.m = m_new;
    if (__any(corr != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < c::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.o[cb][r] *= corr;
    }
    // O^T[channel][query] += sum over keys V^T P^T; element e of k-step k2
    // of half `half` is key 32 half + 16 k2 + 8 (e / 4) + 4 hh + e % 4 on
    // both operands.
    const int s16 = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int row = 32 * half + 16 * k2 + 4 * hh + (s16 >> 2);
#pragma unroll
            for (int cb = 0; cb < c::CB; ++cb) {
                const int col = 32 * cb + 16 * g1 + 4 * (s16 & 3);
                const bf16x8 a = cat44(lds_read_tr4(vt + soff<D, true>(row, col)),
                                       lds_read_tr4(vt + soff<D, true>(row + 8, col)));
                st.o[cb] = mfma32(a, pb[half][k2], st.o[cb]);
            }
        }
}

// One pipeline step over stage t (LDS stage X = t % 2, blocks 2t and 2t + 1
// of n): wait for its loads, then, once every wavefront has finished the
// stage before, refill that stage's buffers with stage t + 1 and compute.
// Loads are issued unconditionally so that the compiler's own waits stay out
// of the loop: with the refill under a branch it made the reads of one stage
// wait for all loads in flight. Blocks past the window are loaded too (rows
// past the head read zeros) and never used.
template <int D, int X>
__device__ inline void swa_step(int t, int n, int64_t kb0, __amdgpu_buffer_rsrc_t kr,
                                __amdgpu_buffer_rsrc_t vr, const bf16x8 (&qf)[SCfg<D>::KS],
                                int64_t qi, int64_t qw0, int64_t W, float cl, SwaAcc<D>& st) {
    wait_vm<0>();
    lds_barrier();
    // kr and vr start at key block kb0
    dma_stage<D>(kr, vr, swa_kst<X ^ 1>(), swa_vst<X ^ 1>(),
                 static_cast<uint32_t>(kSBlocks * (t + 1) * kSK));
#pragma unroll
    for (int hb = 0; hb < kSBlocks; ++hb) {
        const int i = kSBlocks * t + hb;
        const int64_t key0 = (kb0 + i) * kSK;
        // this wavefront's queries qw0 .. qw0 + 31 see keys qw0 - W + 1 .. qw0 + 31
        const bool active = i < n && key0 + kSK > qw0 - W + 1 && key0 <= qw0 + 31;
        if (active) {
            const bool inside = key0 + kSK - 1 <= qw0 && key0 >= qw0 + 31 - W + 1;
            swa_block<D>(swa_kst<X>() + hb * kSK * D, swa_vst<X>() + hb * kSK * D, qf, key0, qi, W,
                         !inside, cl, st);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D>
__global__ __launch_bounds__(kSThreads) void swa_prefill_kernel(SwaParams p) {
    using c = SCfg<D>;

    // Workgroup ids reach the XCDs round-robin; give XCD x a contiguous range
    // of the (head, query tile) order.
    const uint32_t nblk = gridDim.x, bid = blockIdx.x;
    const uint32_t xcd = bid % kXcds, local = bid / kXcds;
    const uint32_t per = nblk / kXcds, rem = nblk % kXcds;
    const uint32_t work = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int64_t bh = work / p.q_tiles, qt = work % p.q_tiles;
    const int64_t b = bh / p.Hq, h = bh % p.Hq, g = h / p.G;
    const int64_t N = p.N, W = p.W;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 31, hh = lane >> 5;
    const int64_t q0 = qt * kSQ, qw0 = q0 + 32 * w, qi = qw0 + li;

    // Buffer ranges start at this tile's first query and its first key block
    // (32-bit offsets: a range spans at most 2^31 bytes, and a tile addresses
    // fewer than W + 512 rows of it), so the prompt's length is not limited.
    constexpr int64_t kRows = (int64_t(1) << 31) / (2 * D);
    const int64_t q_rows = N - q0 < kRows ? N - q0 : kRows;
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc(p.q + (bh * N + q0) * D, static_cast<uint32_t>(q_rows * D * 2));
    bf16x8 qf[c::KS];
#pragma unroll
    for (int ks = 0; ks < c::KS; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                qr, static_cast<uint32_t>(((qi - q0) * D + 16 * ks + 8 * hh) * 2),
                                                0, 0));
    const int64_t kvh = b * p.Hkv + g;
    const int64_t jlo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
    const int64_t jhi = q0 + kSQ < N ? q0 + kSQ : N;
    const int64_t kb0 = jlo / kSK, kb1 = (jhi + kSK - 1) / kSK;
    const int n = static_cast<int>(kb1 - kb0);
    const int64_t k_rows = N - kb0 * kSK < kRows ? N - kb0 * kSK : kRows;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(p.k + (kvh * N + kb0 * kSK) * D,
                                                static_cast<uint32_t>(k_rows * D * 2));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(p.v + (kvh * N + kb0 * kSK) * D,
                                                static_cast<uint32_t>(k_rows * D * 2));

    SwaAcc<D> st;
#pragma unroll
    for (int cb = 0; cb < c::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[cb][r] = 0.0f;
    st.m = -INFINITY;
    st.l = 0.0f;
    const float cl = p.scale_log2;

    dma_stage<D>(kr, vr, swa_kst<0>(), swa_vst<0>(), 0);
    const int stages = (n + kSBlocks - 1) / kSBlocks;
    int t = 0;
    for (; t + 2 <= stages; t += 2) {
        swa_step<D, 0>(t, n, kb0, kr, vr, qf, qi, qw0, W, cl, st);
        swa_step<D, 1>(t + 1, n, kb0, kr, vr, qf, qi, qw0, W, cl, st);
    }
    if (t < stages) swa_step<D, 0>(t, n, kb0, kr, vr, qf, qi, qw0, W, cl, st);
    wait_vm<0>();  // the loads past the window have landed before the LDS is released

    if (qi >= N) return;
    const float l = st.l + __shfl_xor(st.l, 32);
    const float inv = 1.0f / l;
    bf16_t* o = p.out + (bh * N + qi) * D;
#pragma unroll
    for (int cb = 0; cb < c::CB; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = to_bf16(st.o[cb][4 * g4 + e] * inv);
            *reinterpret_cast<bf16x4*>(o + 32 * cb + 8 * g4 + 4 * hh) = v;
        }
}

// Copies the last min(N, W) positions of every KV head into its ring
// (slot p mod W), 16 bytes per thread.
constexpr int kCopyThreads = 256;
__global__ __launch_bounds__(kCopyThreads) void swa_ring_fill_kernel(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, bf16_t* rk, bf16_t* rv, int64_t N,
    int64_t W, int64_t D, int64_t blocks_per_head) {
    const int64_t kvh = blockIdx.x / blocks_per_head;
    const int64_t piece = (blockIdx.x % blocks_per_head) * kCopyThreads + threadIdx.x;
    const int64_t keep = N < W ? N : W;
    const int64_t per_pos = D / 8;
    if (piece >= keep * per_pos) return;
    const int64_t pos = N - keep + piece / per_pos, col = (piece % per_pos) * 8;
    const int64_t src = (kvh * N + pos) * D + col, dst = (kvh * W + pos % W) * D + col;
    *reinterpret_cast<bf16x8*>(rk + dst) = *reinterpret_cast<const bf16x8*>(k + src);
    *reinterpret_cast<bf16x8*>(rv + dst) = *reinterpret_cast<const bf16x8*>(v + src);
}

// Decode append: the new token's key and value go to ring slot pos mod W of
// every KV head; the number of valid slots min(pos + 1, W) goes to lengths.
__global__ __launch_bounds__(64) void swa_append_kernel(
    const bf16_t* __restrict__ k_new, const bf16_t* __restrict__ v_new, bf16_t* rk, bf16_t* rv,
    const int32_t* __restrict__ positions, int32_t* lengths, int64_t Hkv, int64_t W, int64_t D) {
    const int64_t b = blockIdx.x;
    int64_t pos = positions[b];
    pos = pos < 0 ? 0 : pos;  // out-of-contract positions still write inside the ring
    const int64_t slot = pos % W;
    const int64_t per_head = D / 8;
    for (int64_t t = threadIdx.x; t < Hkv * per_head; t += 64) {
        const int64_t g = t / per_head, col = (t % per_head) * 8;
        const int64_t src = (b * Hkv + g) * D + col, dst = ((b * Hkv + g) * W + slot) * D + col;
        *reinterpret_cast<bf16x8*>(rk + dst) = *reinterpret_cast<const bf16x8*>(k_new + src);
        *reinterpret_cast<bf16x8*>(rv + dst) = *reinterpret_cast<const bf16x8*>(v_new + src);
    }
    if (threadIdx.x == 0) lengths[b] = static_cast<int32_t>(pos + 1 < W ? pos + 1 : W);
}

}  // namespace

namespace {
// Workgroups per KV head of the ring fill: the last min(N, window) rows, d / 8
// 16-byte pieces each, one piece per thread.
int64_t ring_fill_groups_per_head(int64_t N, int64_t d, int64_t window) {
    const int64_t keep = N < window ? N : window;
    return (keep * (d / 8) + kCopyThreads - 1) / kCopyThreads;
}
}  // namespace

int64_t swa_prefill_groups(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                           int64_t window, bool ring) {
    const int64_t attn = B * Hq * ((N + kSQ - 1) / kSQ);
    const int64_t fill = ring ? B * Hkv * ring_fill_groups_per_head(N, d, window) : 0;
    return attn > fill ? attn : fill;
}

hipError_t launch_swa_prefill(const SwaArgs& a) {
    SwaParams p;
    p.q = static_cast<const bf16_t*>(a.q);
    p.k = static_cast<const bf16_t*>(a.k);
    p.v = static_cast<const bf16_t*>(a.v);
    p.out = static_cast<bf16_t*>(a.out);
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.N = a.N;
    p.W = a.window;
    p.G = static_cast<int>(a.Hq / a.Hkv);
    const int64_t qt = (a.N + kSQ - 1) / kSQ;
    const int64_t blocks = a.B * a.Hq * qt;
    const int64_t most = swa_prefill_groups(a.B, a.Hq, a.Hkv, a.N, a.d, a.window, a.k_ring != nullptr);
    if (blocks < 1 || most > kMaxGridGroups) return hipErrorInvalidValue;
    p.q_tiles = static_cast<int>(qt);
    p.scale_log2 = a.scale * 1.4426950408889634f;
    if (a.d == 128)
        hipLaunchKernelGGL(swa_prefill_kernel<128>, dim3(static_cast<unsigned>(blocks)),
                           dim3(kSThreads), 0, a.stream, p);
    else if (a.d == 64)
        hipLaunchKernelGGL(swa_prefill_kernel<64>, dim3(static_cast<unsigned>(blocks)),
                           dim3(kSThreads), 0, a.stream, p);
    else
        return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.k_ring) return e;
    const int64_t per_head = ring_fill_groups_per_head(a.N, a.d, a.window);
    hipLaunchKernelGGL(swa_ring_fill_kernel, dim3(static_cast<unsigned>(a.B * a.Hkv * per_head)),
                       dim3(kCopyThreads), 0, a.stream, p.k, p.v,
                       static_cast<bf16_t*>(a.k_ring), static_cast<bf16_t*>(a.v_ring), a.N,
                       a.window, a.d, per_head);
    return hipGetLastError();
}

hipError_t launch_swa_append(const SwaDecodeArgs& a, int32_t* lengths) {
    hipLaunchKernelGGL(swa_append_kernel, dim3(static_cast<unsigned>(a.B)), dim3(64), 0, a.stream,
                       static_cast<const bf16_t*>(a.k_new), static_cast<const bf16_t*>(a.v_new),
                       static_cast<bf16_t*>(a.k_ring), static_cast<bf16_t*>(a.v_ring), a.positions,
                       lengths, a.Hkv, a.window, a.d);
    return hipGetLastError();
}

}  // namespace gret
