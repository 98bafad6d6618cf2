// gret_proj.hip -- key and log-gate projection of gated retention on gfx950,
// with the key scaling and the gate's log-sigmoid over its temperature applied
// in the matrix product's epilogue.
//
// Page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次": section
// "路线二：Multi-Head Gated Retention" projects each position's hidden state to
// the key of every head and to a head-wise gate sigmoid(X W_gamma)^(1/tau);
// section "单 token Decode 的实现骨架" has the key scaled by d_h^-1/2 and the
// gate's log divided by 16. For tokens m = (b, n) of x [B*N, D] and weights
// stored as rows ([H*dk, D] for keys, [H, D] for the gate):
//   k_out[b,h,n,c]  = key_scale * <x[m,:], W_K[h*dk + c,:]>        (bf16)
//   log_gamma[b,h,n] = log sigmoid(<x[m,:], W_gamma[h,:]>) / tau    (fp32)
//
// One bf16 matrix-core product C^T = W x^T per 256-channel x 256-token tile,
// four wavefronts of 128 x 128 (fp32 accumulators in the accumulation
// registers). The hidden dimension advances 32 features per pipeline stage:
// four stages of LDS are filled by direct buffer-to-LDS loads up to four
// stages ahead, and the operands of the next stage are read from LDS into a
// second register set while the matrix cores work on the current one, so one
// workgroup barrier per stage is the only synchronisation. Computing the
// transpose leaves each lane with 4 consecutive channels of one token, which
// are stored as one 8-byte piece straight into the head-major key layout. The
// gate is one extra tile (weight rows past H read as zeros) spread over all
// four wavefronts by tokens. The key tile's results leave through LDS (the
// stage buffers, free once the last operands are read) so that every store
// writes whole 16-byte pieces, 256 contiguous bytes per token and head. Workgroups are ordered so that the tiles running
// together on one XCD share token tiles (x rows) and channel tiles (weight
// rows) in that XCD's L2.
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kPM = 256;        // tokens per tile
constexpr int kPN = 256;        // output channels per tile
constexpr int kPK = 32;         // hidden features per pipeline stage (D: a multiple of 4 kPK)
constexpr int kPThreads = 256;  // 4 wavefronts: 2 along channels x 2 along tokens
constexpr int kPWave = 128;     // channels and tokens per wavefront
constexpr int kPStage = (kPN + kPM) * kPK;  // bf16 per stage: weight rows, then x rows
constexpr int kPGroupM = 6;     // token tiles per group of the workgroup order
constexpr int kXcds = 8;


// Stage layout: rows of 32 bf16 (four 16-byte chunks); chunk c of row r sits
// in slot c ^ ((r >> 1) & 3). Eight lanes reading one chunk of rows r0..r0+7
// (r0 a multiple of 8) then cover the 8 distinct 16-byte slots of a 128-byte
// bank period.
__device__ inline int pswz(int row) { return (row >> 1) & 3; }
__device__ inline int poff(int row, int chunk) { return row * kPK + ((chunk ^ pswz(row)) << 3); }

// One 1 KB direct load of 16 rows (block blk of a 256-row operand): lane l
// fills LDS slot l % 4 of row 16 blk + l / 4 from global chunk slot ^ swizzle.
__device__ inline void dma_rows(__amdgpu_buffer_rsrc_t r, bf16_t* part, int blk, int64_t D,
                                int k0) {
    const int lane = threadIdx.x & 63;
    const int row = 16 * blk + (lane >> 2);
    const int chunk = (lane & 3) ^ pswz(row);
    const uint32_t voff = static_cast<uint32_t>((row * D + k0 + chunk * 8) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(part + blk * 512), 16, voff, 0, 0, 0);
}

// log(sigmoid(u)) = min(u, 0) - log1p(e^-|u|), no exponential overflows. The
// log1p of t in (0, 1] uses log(w) t / (w - 1) with w = 1 + t rounded, which
// cancels the rounding of w (Goldberg's correction; exact t when w == 1).
__device__ inline float log_sigmoid(float u) {
    const float t = __expf(-fabsf(u));
    const float w = 1.0f + t;
    const float l1p = w == 1.0f ? t : __logf(w) * t * __builtin_amdgcn_rcpf(w - 1.0f);
    return fminf(u, 0.0f) - l1p;
}

struct ProjParams {
    const bf16_t* x;
    const bf16_t* w_key;
    const bf16_t* w_gamma;
    bf16_t* k_out;
    float* log_gamma;
    int64_t M, N, D, H, dk;
    int key_tiles, col_tiles, token_tiles;
    float key_scale, inv_temperature;
};

// The four pipeline stages in LDS (file scope, so that every helper names the
// object it touches and the compiler can tell the stages apart when it orders
// LDS reads after the direct loads into other stages).
__shared__ __attribute__((aligned(1024))) bf16_t proj_s0[kPStage];
__shared__ __attribute__((aligned(1024))) bf16_t proj_s1[kPStage];
__shared__ __attribute__((aligned(1024))) bf16_t proj_s2[kPStage];
__shared__ __attribute__((aligned(1024))) bf16_t proj_s3[kPStage];
template <int X>
__device__ inline bf16_t* proj_slot() {
    if constexpr (X == 0) return proj_s0;
    if constexpr (X == 1) return proj_s1;
    if constexpr (X == 2) return proj_s2;
    return proj_s3;
}

// The 8 direct loads of one stage issued by this wavefront (4 weight blocks,
// 4 x blocks; 4 wavefronts cover the 16 + 16 blocks of 16 rows).
__device__ inline void dma_stage(bf16_t* st, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx,
                                 int wave, int64_t D, int t) {
    const int k0 = t * kPK;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_rows(rw, st, 4 * wave + i, D, k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_rows(rx, st + kPN * kPK, 4 * wave + i, D, k0);
}

// Wait until this wavefront's loads of stage s have landed while the loads of
// up to `later` (0..3) further stages stay in flight.
__device__ inline void wait_dma(int later) {
    if (later >= 3)
        wait_vm<24>();
    else if (later == 2)
        wait_vm<16>();
    else if (later == 1)
        wait_vm<8>();
    else
        wait_vm<0>();
}

// Matrix-core operands of one stage for NA channel blocks (weight rows
// a_row + 16 i) and NB token blocks (x rows b_row + 16 j).
template <int NA, int NB>
struct Ops {
    bf16x8 a[NA], b[NB];
};

template <int NA, int NB>
__device__ inline void read_ops(const bf16_t* st, int a_row, int b_row, Ops<NA, NB>& o) {
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, c = lane >> 4;
#pragma unroll
    for (int i = 0; i < NA; ++i)
        o.a[i] = *reinterpret_cast<const bf16x8*>(st + poff(a_row + 16 * i + li, c));
#pragma unroll
    for (int j = 0; j < NB; ++j)
        o.b[j] = *reinterpret_cast<const bf16x8*>(st + kPN * kPK + poff(b_row + 16 * j + li, c));
}

template <int NA, int NB>
__device__ inline void mma_ops(const Ops<NA, NB>& o, f32x4 (&acc)[NA][NB]) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma16(o.a[i], o.b[j], acc[i][j]);
}

// One stage t (in LDS slot X = t % 4): make stage t + 1 visible (NEXT),
// refill slot X with stage t + 4 (DMA), read stage t + 1's operands into the
// other register set and run stage t's products. `later`: stages after t + 1
// whose loads may stay in flight.
template <int X, bool DMA, bool NEXT, int NA, int NB>
__device__ inline void pipe_step(int t, int later, int a_row, int b_row,
                                 __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx, int wave,
                                 int64_t D, Ops<NA, NB>& r0, Ops<NA, NB>& r1,
                                 f32x4 (&acc)[NA][NB]) {
    Ops<NA, NB>& cur = (X & 1) ? r1 : r0;
    Ops<NA, NB>& nxt = (X & 1) ? r0 : r1;
    if constexpr (NEXT) {
        wait_dma(later);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DMA) dma_stage(proj_slot<X>(), rw, rx, wave, D, t + 4);
        read_ops<NA, NB>(proj_slot<(X + 1) & 3>(), a_row, b_row, nxt);
    }
    mma_ops<NA, NB>(cur, acc);
    if constexpr (NEXT) {
        // issue order: the direct loads, then one LDS read per NB products,
        // so that the reads for the next stage are in flight early and the
        // matrix cores never wait for them
        constexpr int kDsGroups = NA + NB;
        constexpr int kPerGroup = NA * NB / kDsGroups;
        if constexpr (DMA) __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
#pragma unroll
        for (int g = 0; g < kDsGroups; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, kPerGroup, 0);
        }
    }
    // keep the next stage's products out of this stage: they would wait for
    // the LDS reads just issued
    __builtin_amdgcn_sched_barrier(0);
}

// The hidden-dimension loop of one tile: acc[i][j] += the products of channel
// block i and token block j over all D features (KT = D / 32 stages, a
// multiple of 4).
template <int NA, int NB>
__device__ inline void tile_loop(int KT, int a_row, int b_row, __amdgpu_buffer_rsrc_t rw,
                                 __amdgpu_buffer_rsrc_t rx, int64_t D, f32x4 (&acc)[NA][NB]) {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    dma_stage(proj_slot<0>(), rw, rx, wave, D, 0);
    dma_stage(proj_slot<1>(), rw, rx, wave, D, 1);
    dma_stage(proj_slot<2>(), rw, rx, wave, D, 2);
    dma_stage(proj_slot<3>(), rw, rx, wave, D, 3);
    wait_dma(3);
    lds_barrier();
    Ops<NA, NB> r0, r1;
    read_ops<NA, NB>(proj_slot<0>(), a_row, b_row, r0);
    int t = 0;
    for (; t + 4 < KT; t += 4) {  // stages t + 4 .. t + 7 exist
        pipe_step<0, true, true>(t, 2, a_row, b_row, rw, rx, wave, D, r0, r1, acc);
        pipe_step<1, true, true>(t + 1, 2, a_row, b_row, rw, rx, wave, D, r0, r1, acc);
        pipe_step<2, true, true>(t + 2, 2, a_row, b_row, rw, rx, wave, D, r0, r1, acc);
        pipe_step<3, true, true>(t + 3, 2, a_row, b_row, rw, rx, wave, D, r0, r1, acc);
    }
    pipe_step<0, false, true>(t, 2, a_row, b_row, rw, rx, wave, D, r0, r1, acc);
    pipe_step<1, false, true>(t + 1, 1, a_row, b_row, rw, rx, wave, D, r0, r1, acc);
    pipe_step<2, false, true>(t + 2, 0, a_row, b_row, rw, rx, wave, D, r0, r1, acc);
    pipe_step<3, false, false>(t + 3, 0, a_row, b_row, rw, rx, wave, D, r0, r1, acc);
}

// Token index -> (sequence, position) for the 16 tokens of a block.
struct TokenMap {
    int64_t b, n;
    bool ok;
};
__device__ inline TokenMap token_at(const ProjParams& p, int64_t m) {
    TokenMap t;
    t.ok = m < p.M;
    t.b = m / p.N;
    t.n = m - t.b * p.N;
    return t;
}

// A key tile: channels ct*256 + wn*128 + 16 i + 4 (lane / 16) .. +3 of tokens
// m0 + wm*128 + 16 j + lane % 16.
__device__ inline void key_tile(const ProjParams& p, int64_t m0, int ct) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t D = p.D, J = p.H * p.dk;
    const int64_t rows_x = p.M - m0 < kPM ? p.M - m0 : kPM;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x + m0 * D, static_cast<uint32_t>(rows_x * D * 2));
    const int64_t j0 = static_cast<int64_t>(ct) * kPN;
    const int64_t rows_w = J - j0 < kPN ? J - j0 : kPN;
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(p.w_key + j0 * D, static_cast<uint32_t>(rows_w * D * 2));
    f32x4 acc[8][8];
    tile_loop<8, 8>(static_cast<int>(D / kPK), wn * kPWave, wm * kPWave, rw, rx, D, acc);

    // Epilogue through LDS. Once every wavefront has read its last operands
    // the four stage buffers are free: wavefront w stages its scaled bf16
    // 128 x 128 tile token-major in buffer w (row t = 128 channels; 16-byte
    // piece c of row t at slot c ^ (t % 16), so the 16 tokens of one product
    // block land in 16 different slots), then stores whole 16-byte pieces:
    // 16 lanes cover the 256 bytes of one token's channels.
    lds_barrier();
    bf16_t* st = wave == 0 ? proj_s0 : wave == 1 ? proj_s1 : wave == 2 ? proj_s2 : proj_s3;
    const int li = lane & 15, cq = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = to_bf16(acc[i][j][e] * p.key_scale);
            const int t = 16 * j + li, ch = 16 * i + cq;
            *reinterpret_cast<bf16x4*>(st + t * kPWave + (((ch >> 3) ^ li) << 3) + (ch & 7)) = v;
        }
    const int c16 = lane & 15;
    const int64_t jc = j0 + wn * kPWave + 8 * c16;  // first of this lane's 8 channels
    const int64_t h = jc / p.dk, c = jc - h * p.dk;  // dk % 8 == 0: one head
    const int64_t tw = m0 + wm * kPWave + (lane >> 4);
    int64_t b = tw / p.N, n = tw - b * p.N;
    bf16_t* dst_h = p.k_out + h * p.N * p.dk + c;
    for (int s4 = 0; s4 < kPWave / 4; ++s4) {
        const int t = 4 * s4 + (lane >> 4);
        const bf16x8 val = *reinterpret_cast<const bf16x8*>(st + t * kPWave + ((c16 ^ (t & 15)) << 3));
        if (tw + 4 * s4 < p.M && jc < J)
            *reinterpret_cast<bf16x8*>(dst_h + (b * p.H * p.N + n) * p.dk) = val;
        n += 4;
        while (n >= p.N) {
            n -= p.N;
            ++b;
        }
    }
}

// The gate tile: NA = ceil(H / 16) channel blocks (gate heads) of 64 tokens
// per wavefront (m0 + 64 wave + 16 j + lane % 16).
template <int NA>
__device__ inline void gate_tile(const ProjParams& p, int64_t m0) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t D = p.D;
    const int64_t rows_x = p.M - m0 < kPM ? p.M - m0 : kPM;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x + m0 * D, static_cast<uint32_t>(rows_x * D * 2));
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w_gamma, static_cast<uint32_t>(p.H * D * 2));
    f32x4 acc[NA][4];
    tile_loop<NA, 4>(static_cast<int>(D / kPK), 0, 64 * wave, rw, rx, D, acc);

    const int li = lane & 15, cq = 4 * (lane >> 4);
    TokenMap tok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tok[j] = token_at(p, m0 + 64 * wave + 16 * j + li);
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t h = 16 * i + cq + e;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float ls = log_sigmoid(acc[i][j][e]);
                if (h < p.H && tok[j].ok)
                    p.log_gamma[(tok[j].b * p.H + h) * p.N + tok[j].n] = ls * p.inv_temperature;
            }
        }
}

__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void proj_kernel(ProjParams p) {
    // Workgroup ids reach the XCDs round-robin; give XCD x a contiguous range
    // of the work order, grouped by kPGroupM token tiles.
    const uint32_t nblk = gridDim.x, bid = blockIdx.x;
    const uint32_t xcd = bid % kXcds, local = bid / kXcds;
    const uint32_t per = nblk / kXcds, rem = nblk % kXcds;
    const uint32_t work = xcd * per + (xcd < rem ? xcd : rem) + local;
    const uint32_t CT = static_cast<uint32_t>(p.col_tiles);
    const uint32_t TT = static_cast<uint32_t>(p.token_tiles);
    const uint32_t group = kPGroupM * CT;
    const uint32_t first = (work / group) * kPGroupM;
    const uint32_t gm = TT - first < kPGroupM ? TT - first : kPGroupM;
    const uint32_t in_group = work % group;
    const uint32_t tt = first + in_group % gm;
    const int ct = static_cast<int>(in_group / gm);
    const int64_t m0 = static_cast<int64_t>(tt) * kPM;
    // the gate column (when there is one) comes first in each group, next to
    // the first key tiles of the same token tiles, while their x rows are in L2
    const int kt = p.col_tiles > p.key_tiles ? ct - 1 : ct;
    if (kt >= 0)
        key_tile(p, m0, kt);
    else if (p.H <= 32)
        gate_tile<2>(p, m0);
    else if (p.H <= 64)
        gate_tile<4>(p, m0);
    else if (p.H <= 128)
        gate_tile<8>(p, m0);
    else
        gate_tile<16>(p, m0);
}

}  // namespace

hipError_t launch_head_projection(const ProjArgs& a) {
    ProjParams p;
    p.x = static_cast<const bf16_t*>(a.x);
    p.w_key = static_cast<const bf16_t*>(a.w_key);
    p.w_gamma = static_cast<const bf16_t*>(a.w_gamma);
    p.k_out = static_cast<bf16_t*>(a.k_out);
    p.log_gamma = a.log_gamma;
    p.M = a.B * a.N;
    p.N = a.N;
    p.D = a.D;
    p.H = a.H;
    p.dk = a.dk;
    const int64_t J = a.H * a.dk;
    const int64_t key_tiles = (J + kPN - 1) / kPN;
    const int64_t col_tiles = key_tiles + (a.w_gamma ? 1 : 0);
    const int64_t token_tiles = (p.M + kPM - 1) / kPM;
    const int64_t blocks = token_tiles * col_tiles;
    if (a.D % (4 * kPK) != 0 || blocks < 1 || blocks > 0x7fffffff) return hipErrorInvalidValue;
    p.key_tiles = static_cast<int>(key_tiles);
    p.col_tiles = static_cast<int>(col_tiles);
    p.token_tiles = static_cast<int>(token_tiles);
    p.key_scale = a.key_scale;
    p.inv_temperature = a.inv_temperature;
    hipLaunchKernelGGL(proj_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kPThreads), 0,
                       a.stream, p);
    return hipGetLastError();
}

}  // namespace gret
