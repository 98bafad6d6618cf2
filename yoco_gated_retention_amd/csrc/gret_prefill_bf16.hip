// gret_prefill_bf16.hip -- chunkwise gated-retention prefill on gfx950 matrix
// cores (bf16 operands, fp32 accumulation, fp32 state carry).
//
// Method (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次",
// sections "路线二：Multi-Head Gated Retention" and "Prefill 与 Decode 为什么使用
// 两种计算形态"): inside a chunk of C positions starting at a, with beta_j the
// chunk-local inclusive sum of log-gates,
//   out[a+j] = exp(beta_j) q_{a+j} S + sum_{l<=j} exp(beta_j - beta_l) (q_{a+j}.k_{a+l}) v_{a+l}
//   S       <- exp(beta_last) S + sum_l exp(beta_last - beta_l) k_{a+l}^T v_{a+l}
// Only differences of log-decays inside a chunk are exponentiated, so every
// factor is at most 1. The head-wise scalar gate keeps every contraction a
// plain matrix product, which is what makes the matrix cores usable (same
// section, on head-wise versus element-wise decay).
//
// Parallel schedule. The chunk-to-chunk state carry is the only serial
// dependence. Carrying a state is the affine map S -> exp(G) S + S_loc, so each
// head's chunk sequence is cut into segments that run concurrently (segment
// bookkeeping in gret_segments.h), in three launches:
//   1. main:    every segment runs from a zero state (the first segment of a
//               head from the caller's state) and writes its end state and its
//               total log-decay to the workspace. A non-first segment first
//               runs only the state update over its leading chunks, until the
//               running log-decay from the segment start drops below
//               kSurvivalDropLog (the incoming state's survival factor is then
//               below the smallest normal fp32 number), and from there on
//               stores outputs too. Log-gates are <= 0, so the running sum only
//               decreases and every later output has a smaller factor.
//   2. combine: per head, chain the segment maps in order, leaving each
//               segment's incoming state in its workspace slot; the last one
//               is the final state.
//   3. prefix:  every non-first segment recomputes its leading chunks, now
//               from its incoming state, and writes their outputs.
// Each output is written exactly once and inputs are read about once (the
// leading chunks twice).
//
// Workgroup layout: DV/16 wavefronts (8 at dv = 128, two per SIMD); wave w
// owns value columns [16w, 16w+16) of the state and of the output. Per
// 64-position tile:
//   global -> registers (prefetched one tile ahead, range-checked buffer
//   loads) -> LDS, Q, K and V row-major with an XOR swizzle of 16-byte chunks.
//   Operands whose contraction runs over positions (K^T, V^T) are read with
//   the gfx950 transposing LDS load ds_read_b64_tr_b16, so no transposed copy
//   is ever made. The state stays in registers as fp32 accumulator tiles.
//   * scores   P^T = K Q^T per 16x16 tile (16x16x32 bf16 MFMA), decay mask
//              exp(beta_j - beta_l) in fp32, cast to bf16 into LDS;
//   * output   O^T = S^T Q^T (S straight from the accumulator registers)
//              scaled by exp(beta_j), plus V^T P~^T; each lane ends with 4
//              consecutive output columns of one row and stores 8 bytes;
//   * state    S = exp(g) S + K^T (Gamma V) with Gamma_l = exp(g - beta_l).
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kTile = 64;  // positions per tile
constexpr int kPadP = 8;   // bf16 padding per row of the score tile

__device__ inline f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline bf16x8 lds_read8(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ inline bf16x4 lds_read4(const bf16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }

// Transposing LDS read: within each 16-lane group, lane l receives element
// (l % 4) of the 8-byte pieces addressed by lanes 4e + l/4 (e = 0..3). With
// lane s pointing at row t0 + s/4, column n0 + 4(s % 4) of a row-major tile,
// lane l gets column n0 + l of rows t0..t0+3.
__device__ inline bf16x4 lds_read_tr4(const bf16_t* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ inline bf16x8 cat44(const bf16x4& a, const bf16x4& b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Range-checked buffer access (CDNA buffer resources). A descriptor covers one
// head's rows; a load past its end returns zeros and a store past it is
// dropped by the hardware, which is exactly the tail masking the chunkwise form
// needs (padded positions carry zero K and V and log-gate 0, and their outputs
// are not written), without a branch on the hot path.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, gfx9-family data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferWord3);
}
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
};

// Per-head views of the prefill tensors.
struct HeadRsrc {
    __amdgpu_buffer_rsrc_t q, k, v, lg, out;
};

template <int DK, int DV, int R>
struct Cfg {
    static constexpr int C = kTile * R;
    static constexpr int NW = DV / 16;      // wavefronts; wave w owns value columns 16w..16w+15
    static constexpr int NT = 64 * NW;      // threads per workgroup
    static constexpr int TK = DK / 16;      // 16-row key tiles of the state
    static constexpr int KS = DK / 32;      // k-steps over dk
    static constexpr int QCH = DK / 8;      // 16-byte chunks per Q/K row
    static constexpr int VCH = DV / 8;      // 16-byte chunks per V row
    static constexpr int QLD = kTile * QCH / NT;  // staged chunks per thread
    static constexpr int VLD = kTile * VCH / NT;
    static constexpr int PP = kTile + kPadP;  // row pitch (elements) of the score tile
    static constexpr int BSTEP = NW / 4;      // score tiles: waves per query block
    static_assert(QLD >= 1 && QLD * NT == kTile * QCH, "Q/K staging");
    static_assert(VLD >= 1 && VLD * NT == kTile * VCH, "V staging");
    static_assert(QCH >= 8 && VCH >= 8, "swizzle spans 8 chunks");
    static_assert(NW == 4 || NW == 8, "waves");
    static_assert(NT == DV * 4, "threads");
};

// Threads per workgroup for a value width (one wavefront per 16 columns).
template <int DV>
constexpr int kThreadsFor = DV * 4;

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

// One staged tile and the per-chunk tables derived from its log-gates.
template <int DK, int DV, int R>
struct __attribute__((aligned(16))) TileBuf {
    using c = Cfg<DK, DV, R>;
    bf16_t qs[kTile * DK];
    bf16_t ks[kTile * DK];
    bf16_t vs[kTile * DV];
    float beta[c::C];  // chunk-local inclusive log-decay
    float gam[c::C];   // exp(beta_last - beta_l): weight of position l in the state update
    float fexp[c::C];  // exp(beta_j): weight of the incoming state in output j
};

// Chunks of 64 double-buffer the staged tile (the next chunk is written while
// slower wavefronts still read the current one), which saves a barrier.
template <int DK, int DV, int R>
struct __attribute__((aligned(16))) Smem {
    using c = Cfg<DK, DV, R>;
    static constexpr int NB = R == 1 ? 2 : 1;
    TileBuf<DK, DV, R> buf[NB];
    bf16_t ps[kTile * c::PP];
    bf16_t os[R == 1 ? kTile * DV : 8];  // output tile staged for full-row stores
};

template <int DK, int DV>
struct __attribute__((aligned(16))) Smem2 {  // earlier tiles of the chunk (chunks > 64)
    bf16_t ks[kTile * DK];
    bf16_t vs[kTile * DV];
};

// All LDS of one workgroup; the restaging buffers exist only for chunks > 64.
template <int DK, int DV, int R>
struct SmemAll {
    Smem<DK, DV, R> m;
    Smem2<DK, DV> e;
    __device__ Smem2<DK, DV>* extra() { return &e; }
};
template <int DK, int DV>
struct SmemAll<DK, DV, 1> {
    Smem<DK, DV, 1> m;
    __device__ Smem2<DK, DV>* extra() { return nullptr; }
};

// Registers that hold one tile of global data between its load and its LDS write.
template <int DK, int DV, int R>
struct TileRegs {
    using c = Cfg<DK, DV, R>;
    bf16x8 q[c::QLD];
    bf16x8 k[c::QLD];
    bf16x8 v[c::VLD];
    float ell[R];  // log-gates of the chunk (lane holds R consecutive)
};

// Loads tile `tile_pos` of a head (Q only when WITH_Q) plus the log-gates of
// the chunk starting at chunk_pos. Positions past the end read as zero.
template <int DK, int DV, int R, bool WITH_Q = true>
__device__ inline void load_tile(const HeadRsrc& hr, uint32_t tile_pos, uint32_t chunk_pos,
                                 TileRegs<DK, DV, R>& t) {
    using c = Cfg<DK, DV, R>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < c::QLD; ++i) {
        const int id = tid + i * c::NT;
        const uint32_t off = ((tile_pos + id / c::QCH) * DK + (id % c::QCH) * 8) * 2;
        if constexpr (WITH_Q) t.q[i] = buf_load8(hr.q, off);
        t.k[i] = buf_load8(hr.k, off);
    }
#pragma unroll
    for (int i = 0; i < c::VLD; ++i) {
        const int id = tid + i * c::NT;
        t.v[i] = buf_load8(hr.v, ((tile_pos + id / c::VCH) * DV + (id % c::VCH) * 8) * 2);
    }
    const uint32_t lane = tid & 63;
#pragma unroll
    for (int i = 0; i < R; ++i) t.ell[i] = buf_load_f32(hr.lg, (chunk_pos + lane * R + i) * 4);
}

template <int DK, int DV, int R, bool WITH_Q = true>
__device__ inline void write_tile(const TileRegs<DK, DV, R>& t, bf16_t* qs, bf16_t* ks,
                                  bf16_t* vs) {
    using c = Cfg<DK, DV, R>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < c::QLD; ++i) {
        const int id = tid + i * c::NT;
        const int o = toff<DK>(id / c::QCH, (id % c::QCH) * 8);
        if constexpr (WITH_Q) *reinterpret_cast<bf16x8*>(qs + o) = t.q[i];
        *reinterpret_cast<bf16x8*>(ks + o) = t.k[i];
    }
#pragma unroll
    for (int i = 0; i < c::VLD; ++i) {
        const int id = tid + i * c::NT;
        *reinterpret_cast<bf16x8*>(vs + toff<DV>(id / c::VCH, (id % c::VCH) * 8)) = t.v[i];
    }
}

// Wave 0: chunk-local inclusive prefix sum of the clamped log-gates
// (positions past the end read as log-gate 0) and the two exponential tables
// of the chunk.
template <int DK, int DV, int R>
__device__ inline void make_tables(const TileRegs<DK, DV, R>& t, TileBuf<DK, DV, R>& tb) {
    const int tid = threadIdx.x;
    if (tid >= 64) return;
    float loc[R];
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        run += clamp_log_gamma(t.ell[i], kLogGammaFloor);
        loc[i] = run;
    }
    float tot = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(tot, off);
        if (tid >= off) tot += o;
    }
    const float gc = __shfl(tot, 63);
    const float excl = tot - run;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const float b = excl + loc[i];
        tb.beta[tid * R + i] = b;
        tb.gam[tid * R + i] = __expf(gc - b);
        tb.fexp[tid * R + i] = __expf(b);
    }
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

// Per-thread state of one segment's pass.
template <int DK, int DV, int R>
struct Acc {
    using c = Cfg<DK, DV, R>;
    f32x4 s[c::TK];                    // S[16tk + 4g + i][16w + li]
    f32x4 ds[R > 1 ? c::TK : 1];       // chunk increment (chunks > 64)
};

// Stages K and V of an earlier tile of the current chunk into s2.
template <int DK, int DV, int R>
__device__ inline void restage(const HeadRsrc& hr, uint32_t pos, Smem2<DK, DV>& s2) {
    TileRegs<DK, DV, R> t;
    load_tile<DK, DV, R, false>(hr, pos, pos, t);
    write_tile<DK, DV, R, false>(t, nullptr, s2.ks, s2.vs);
}

// Cross-chunk term O^T = S^T Q^T for the 64 rows of the tile, then row j scaled
// by exp(beta_j). The state tile pair (2m, 2m+1) gives each lane
// dk = 32m + {4g..4g+3, 16+4g..16+4g+3}; the Q operand is read with the same
// permutation of dk, so the contraction pairs matching indices.
template <int DK, int DV, int R, class TB>
__device__ inline void cross_term(const TB& tb, const Acc<DK, DV, R>& a, int r,
                                  f32x4 (&o)[4]) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) o[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < c::KS; ++m) {
        const f32x4 lo4 = a.s[2 * m], hi4 = a.s[2 * m + 1];
        const bf16x8 sf = {to_bf16(lo4[0]), to_bf16(lo4[1]), to_bf16(lo4[2]), to_bf16(lo4[3]),
                           to_bf16(hi4[0]), to_bf16(hi4[1]), to_bf16(hi4[2]), to_bf16(hi4[3])};
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const int row = 16 * jt + li;
            const bf16x8 qf = cat44(lds_read4(tb.qs + toff<DK>(row, 32 * m + 4 * g)),
                                    lds_read4(tb.qs + toff<DK>(row, 32 * m + 16 + 4 * g)));
            o[jt] = mfma16(sf, qf, o[jt]);
        }
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const float f = tb.fexp[kTile * r + 16 * jt + li];
        o[jt][0] *= f;
        o[jt][1] *= f;
        o[jt][2] *= f;
        o[jt][3] *= f;
    }
}

// Decayed score block (jb, b): rows 16jb.. of query tile r against columns
// 16b.. of key tile t, written as bf16 to ps[j][l]. With diag, entries above
// the diagonal are zero.
template <int DK, int DV, int R, class TB>
__device__ inline void score_block(const TB& tb, bf16_t* ps, const bf16_t* ksrc,
                                   int r, int t, int jb, int b, bool diag) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int jrow = 16 * jb + li;
    const float bj = tb.beta[kTile * r + jrow];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < c::KS; ++ks) {
        const bf16x8 qf = lds_read8(tb.qs + toff<DK>(jrow, 32 * ks + 8 * g));
        const bf16x8 kf = lds_read8(ksrc + toff<DK>(16 * b + li, 32 * ks + 8 * g));
        acc = mfma16(kf, qf, acc);
    }
    // acc[i] = P^T[l = 16b + 4g + i][j = jrow]
    bf16x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int l = 16 * b + 4 * g + i;
        float val = 0.0f;
        if (!diag || l <= jrow) val = acc[i] * __expf(bj - tb.beta[kTile * t + l]);
        pk[i] = to_bf16(val);
    }
    *reinterpret_cast<bf16x4*>(ps + jrow * c::PP + 16 * b + 4 * g) = pk;
}

// The 10 blocks on or below the diagonal of a 64x64 score tile, largest rows
// first: (3,3) (3,2) (2,2) (3,1) (2,1) (1,1) (3,0) (2,0) (1,0) (0,0), packed as
// 4-bit (4 jb + b) entries of an immediate (a table in memory would be a
// global load that the compiler waits for together with the prefetches).
constexpr uint64_t kCausalBlocks = 0xFull | 0xEull << 4 | 0xAull << 8 | 0xDull << 12 |
                                   0x9ull << 16 | 0x5ull << 20 | 0xCull << 24 | 0x8ull << 28 |
                                   0x4ull << 32 | 0x0ull << 36;

// Wave w computes entries w, w + NW, ...
template <int DK, int DV, int R, class TB>
__device__ inline void scores_diag(const TB& tb, bf16_t* ps, int r) {
    using c = Cfg<DK, DV, R>;
    const int w = threadIdx.x >> 6;
    for (int i = w; i < 10; i += c::NW) {
        const int e = static_cast<int>((kCausalBlocks >> (4 * i)) & 0xF);
        score_block<DK, DV, R>(tb, ps, tb.ks, r, r, e >> 2, e & 3, true);
    }
}

template <int DK, int DV, int R, class TB>
__device__ inline void scores_full(const TB& tb, bf16_t* ps, const bf16_t* ksrc,
                                   int r, int t) {
    using c = Cfg<DK, DV, R>;
    const int w = threadIdx.x >> 6;
    for (int i = w; i < 16; i += c::NW)
        score_block<DK, DV, R>(tb, ps, ksrc, r, t, i >> 2, i & 3, false);
}

// Blocks (0,1) and (2,3) lie above the diagonal but inside 32-position steps
// that the diagonal product uses; they hold zeros.
template <int DK, int DV, int R>
__device__ inline void zero_upper_blocks(bf16_t* ps) {
    using c = Cfg<DK, DV, R>;
    for (int e = threadIdx.x; e < 2 * 16 * 4; e += c::NT) {
        const int blk = e / 64, rem = e % 64;
        const int jb = blk == 0 ? 0 : 2, b = jb + 1;
        const int row = 16 * jb + rem / 4, col = 16 * b + 4 * (rem % 4);
        *reinterpret_cast<bf16x4*>(ps + row * c::PP + col) = bf16x4{};
    }
}

// O^T[cols][rows] += V_t^T P~^T over the positions of tile t (V read transposed).
template <int DK, int DV, int R>
__device__ inline void apply_scores(const bf16_t* ps, const bf16_t* vsrc, bool diag,
                                    f32x4 (&o)[4]) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 vf = read_cols8<DV>(vsrc, 32 * ks + 8 * g, 16 * w);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (diag && 2 * ks > jt) continue;  // whole 32-position step is above the diagonal
            const bf16x8 pf = lds_read8(ps + (16 * jt + li) * c::PP + 32 * ks + 8 * g);
            o[jt] = mfma16(vf, pf, o[jt]);
        }
    }
}

template <int DK, int DV, int R>
__device__ inline void store_out(const __amdgpu_buffer_rsrc_t& out, uint32_t tile_pos,
                                 const f32x4 (&o)[4]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const uint32_t pos = tile_pos + 16 * jt + li;
        const bf16x4 pk = {to_bf16(o[jt][0]), to_bf16(o[jt][1]), to_bf16(o[jt][2]),
                           to_bf16(o[jt][3])};
        buf_store4(out, (pos * DV + 16 * w + 4 * g) * 2, pk);
    }
}

// Output through LDS: each lane's fragment (4 consecutive columns of one row)
// goes to a swizzled row-major tile, and whole rows then leave with 16-byte
// stores, so every store instruction of a wavefront covers 4 complete 256-byte
// rows instead of sixteen 32-byte pieces.
template <int DK, int DV, int R>
__device__ inline void out_to_lds(bf16_t* os, const f32x4 (&o)[4]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const bf16x4 pk = {to_bf16(o[jt][0]), to_bf16(o[jt][1]), to_bf16(o[jt][2]),
                           to_bf16(o[jt][3])};
        *reinterpret_cast<bf16x4*>(os + toff<DV>(16 * jt + li, 16 * w + 4 * g)) = pk;
    }
}

template <int DK, int DV, int R>
__device__ inline void flush_out(const bf16_t* os, const __amdgpu_buffer_rsrc_t& out,
                                 uint32_t tile_pos) {
    using c = Cfg<DK, DV, R>;
    constexpr int PER = kTile * c::VCH / c::NT;  // 16-byte pieces per thread
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int id = threadIdx.x + i * c::NT;
        const int row = id / c::VCH, ch = id % c::VCH;
        const bf16x8 v = lds_read8(os + toff<DV>(row, 8 * ch));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), out,
                                               ((tile_pos + row) * DV + 8 * ch) * 2, 0, 0);
    }
}

// acc += K^T (Gamma V) over tile r of the chunk, Gamma_l = exp(g - beta_l)
// from the chunk table; K and V are read transposed so that positions are the
// contraction index.
template <int DK, int DV, int R, class TB>
__device__ inline void state_update(const TB& tb, int r,
                                    f32x4 (&acc)[Cfg<DK, DV, R>::TK]) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int t0 = 32 * ks + 8 * g;
        const bf16x8 vf = read_cols8<DV>(tb.vs, t0, 16 * w);
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(tb.gam + kTile * r + t0);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(tb.gam + kTile * r + t0 + 4);
        const bf16x8 bf = {to_bf16(from_bf16(vf[0]) * g0[0]), to_bf16(from_bf16(vf[1]) * g0[1]),
                           to_bf16(from_bf16(vf[2]) * g0[2]), to_bf16(from_bf16(vf[3]) * g0[3]),
                           to_bf16(from_bf16(vf[4]) * g1[0]), to_bf16(from_bf16(vf[5]) * g1[1]),
                           to_bf16(from_bf16(vf[6]) * g1[2]), to_bf16(from_bf16(vf[7]) * g1[3])};
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk) {
            const bf16x8 kf = read_cols8<DK>(tb.ks, t0, 16 * tk);
            acc[tk] = mfma16(kf, bf, acc[tk]);
        }
    }
}

template <int DK, int DV, int R>
__device__ inline HeadRsrc head_rsrc(const Params& p, int64_t x) {
    const int64_t N = p.N;
    HeadRsrc hr;
    hr.q = make_rsrc(p.q + x * N * DK, static_cast<uint32_t>(N * DK * 2));
    hr.k = make_rsrc(p.k + x * N * DK, static_cast<uint32_t>(N * DK * 2));
    hr.v = make_rsrc(p.v + x * N * DV, static_cast<uint32_t>(N * DV * 2));
    hr.lg = make_rsrc(p.log_gamma + x * N, static_cast<uint32_t>(N * 4));
    hr.out = make_rsrc(p.out + x * N * DV, static_cast<uint32_t>(N * DV * 2));
    return hr;
}

template <int DK, int DV, int R>
__device__ inline void scale_state(Acc<DK, DV, R>& a, float eg) {
    using c = Cfg<DK, DV, R>;
#pragma unroll
    for (int tk = 0; tk < c::TK; ++tk) {
        a.s[tk][0] *= eg;
        a.s[tk][1] *= eg;
        a.s[tk][2] *= eg;
        a.s[tk][3] *= eg;
    }
}

// One chunk of 64 positions from the staged buffer `cur`. It first stores the
// previous chunk's output tile (staged in LDS, `prev_out` / `prev_pos`), then
// computes this chunk, leaves its output tile in LDS, stages the next chunk
// (already in `stage`) into the other buffer and refills `stage` with the chunk
// three ahead. Returns the chunk's total log-decay.
template <int DK, int DV, int R>
__device__ inline float chunk_c64(const HeadRsrc& hr, const __amdgpu_buffer_rsrc_t& prev_out,
                                  uint32_t prev_pos, Smem<DK, DV, R>& sm, int cur, uint32_t pos,
                                  Acc<DK, DV, R>& a, TileRegs<DK, DV, R>& stage) {
    const TileBuf<DK, DV, R>& tb = sm.buf[cur];
    flush_out<DK, DV, R>(sm.os, prev_out, prev_pos);
    f32x4 o[4];
    cross_term<DK, DV, R>(tb, a, 0, o);
    scores_diag<DK, DV, R>(tb, sm.ps, 0);
    __syncthreads();
    apply_scores<DK, DV, R>(sm.ps, tb.vs, true, o);
    out_to_lds<DK, DV, R>(sm.os, o);
    const float gc = tb.beta[kTile - 1];
    scale_state<DK, DV, R>(a, __expf(gc));
    state_update<DK, DV, R>(tb, 0, a.s);
    TileBuf<DK, DV, R>& nb = sm.buf[cur ^ 1];
    make_tables<DK, DV, R>(stage, nb);
    write_tile<DK, DV, R>(stage, nb.qs, nb.ks, nb.vs);
    load_tile<DK, DV, R>(hr, pos + 3 * kTile, pos + 3 * kTile, stage);
    __syncthreads();
    return gc;
}

// Chunks of 64 positions (one tile per chunk): a branch-free steady-state
// loop over double-buffered LDS tiles with two barriers per chunk, fed by two
// register sets so that every tile's loads are issued two chunks before they
// are staged (about 100 KB in flight per CU). Reads past the head's end return
// zeros, and in state-only mode the outputs are still computed but stored
// through a zero-length descriptor, so the hardware drops them. Every
// iteration therefore issues the same memory operations in the same order,
// which lets the compiler wait only for the loads it stages while younger
// loads and the output stores stay in flight.
template <int DK, int DV, int R>
__device__ float run_chunks_c64(const Params& p, Smem<DK, DV, R>& sm, int64_t x, int64_t cb,
                                int64_t ce, bool full_from_start, Acc<DK, DV, R>& a,
                                int64_t* lead) {
    static_assert(R == 1, "one tile per chunk");
    bool full = full_from_start;
    float total = 0.0f;
    *lead = full ? 0 : (ce - cb);
    const HeadRsrc hr = head_rsrc<DK, DV, R>(p, x);
    const __amdgpu_buffer_rsrc_t drop = make_rsrc(p.out, 0);
    TileRegs<DK, DV, R> ta, tb;
    uint32_t pos = static_cast<uint32_t>(cb * kTile);
    load_tile<DK, DV, R>(hr, pos, pos, ta);
    load_tile<DK, DV, R>(hr, pos + kTile, pos + kTile, tb);
    __syncthreads();  // the previous segment of this workgroup is done with the LDS tiles
    flush_out<DK, DV, R>(sm.os, drop, 0);  // same store pattern as the loop, all dropped
    make_tables<DK, DV, R>(ta, sm.buf[0]);
    write_tile<DK, DV, R>(ta, sm.buf[0].qs, sm.buf[0].ks, sm.buf[0].vs);
    load_tile<DK, DV, R>(hr, pos + 2 * kTile, pos + 2 * kTile, ta);
    __syncthreads();
    __amdgpu_buffer_rsrc_t prev_out = drop;
    uint32_t prev_pos = 0;
    for (int64_t ch = cb; ch < ce; ch += 2, pos += 2 * kTile) {
        float gc = chunk_c64<DK, DV, R>(hr, prev_out, prev_pos, sm, 0, pos, a, tb);
        prev_out = full ? hr.out : drop;
        prev_pos = pos;
        total += gc;
        if (!full && total < kSurvivalDropLog) {
            full = true;
            *lead = ch + 1 - cb;
        }
        if (ch + 1 >= ce) break;
        gc = chunk_c64<DK, DV, R>(hr, prev_out, prev_pos, sm, 1, pos + kTile, a, ta);
        prev_out = full ? hr.out : drop;
        prev_pos = pos + kTile;
        total += gc;
        if (!full && total < kSurvivalDropLog) {
            full = true;
            *lead = ch + 2 - cb;
        }
    }
    flush_out<DK, DV, R>(sm.os, prev_out, prev_pos);  // the last chunk's output tile
    return total;
}

// ---------------------------------------------------------------------------
// Chunk-64 path fed by LDS DMA.
//
// Tiles go from HBM straight into LDS with buffer_load ... lds (no registers
// involved), into three buffer sets, so that while chunk n is computed the
// tiles of chunks n+1 and n+2 are in flight. The compiler tracks LDS DMA per
// LDS object, so each set is a distinct __shared__ array and the loop is
// unrolled by three to keep every access's target set a compile-time fact.
// Publication of a tile to the other wavefronts is explicit: each wavefront
// waits for its own DMA writes of that tile (s_waitcnt vmcnt with the number
// of its younger memory operations, which the loop keeps constant), then all
// meet at a barrier. Barriers here carry no release fence, so they do not
// drain the loads still in flight for the next tiles.

typedef __attribute__((address_space(3))) void lds_void;

struct TileView {
    const bf16_t* qs;
    const bf16_t* ks;
    const bf16_t* vs;
    const float* beta;
    const float* gam;
    const float* fexp;
};

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wavefront are outstanding (gfx9 encoding; expcnt and lgkmcnt left alone).
constexpr int vm_wait_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kLgkmWaitZero = 0xC07F;  // lgkmcnt(0) only

template <int N>
__device__ inline void wait_vm() {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(N));
}

// Workgroup barrier for LDS data: this wavefront's LDS writes complete, then
// s_barrier; compiler-only fences keep memory accesses on their side.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(kLgkmWaitZero);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Cache policy of the streamed q/k/v/log-gate loads: nontemporal (each byte is
// read once). The output stores keep the default write-back policy: with the
// nontemporal bit they measured 1.5x slower.
constexpr int kStreamLoad = 2;

// One 1 KB DMA instruction of a swizzled row-major tile with D columns: lane i
// lands at LDS byte 16 i of block blk, i.e. row (512/D) blk + i / (D/8), slot
// i % (D/8), so it fetches the global 16-byte chunk slot ^ swz(row) of that row.
template <int D>
__device__ inline void dma_block(__amdgpu_buffer_rsrc_t r, bf16_t* tile, int blk,
                                 uint32_t tile_pos) {
    constexpr int RPI = 512 / D;  // rows per instruction
    constexpr int SPR = D / 8;    // 16-byte slots per row
    const int lane = threadIdx.x & 63;
    const int row = RPI * blk + lane / SPR;
    const int chunk = (lane % SPR) ^ swz<D>(row);
    const uint32_t voff = ((tile_pos + row) * D + chunk * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + blk * 512), 16, voff, 0, 0,
                                             kStreamLoad);
}

template <int DK, int DV>
struct C64Lds {
    bf16_t* q[3];
    bf16_t* k[3];
    bf16_t* v[3];
    float* ell[3];
    float* tab[3];  // beta[64] | gam[64] | fexp[64]
    bf16_t* ps;
};

template <int DK, int DV>
struct C64Counts {
    static constexpr int NW = DV / 16;
    static constexpr int QB = DK / 8 / NW;  // DMA blocks of Q (and of K) per wavefront
    static constexpr int VB = DV / 8 / NW;  // DMA blocks of V per wavefront
    static constexpr int DMA = 2 * QB + VB; // per wavefront and tile (+1 log-gate DMA on wave 0)
    static constexpr int ST = 4;            // output stores per wavefront and chunk
    static_assert(QB * NW * 8 == DK && VB * NW * 8 == DV, "DMA split");
};

// Issues this wavefront's share of the DMA of the tile at tile_pos into set X.
template <int DK, int DV, int X>
__device__ inline void dma_tile(const C64Lds<DK, DV>& L, const HeadRsrc& hr, uint32_t tile_pos) {
    using n = C64Counts<DK, DV>;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < n::QB; ++i) dma_block<DK>(hr.q, L.q[X], w * n::QB + i, tile_pos);
#pragma unroll
    for (int i = 0; i < n::QB; ++i) dma_block<DK>(hr.k, L.k[X], w * n::QB + i, tile_pos);
#pragma unroll
    for (int i = 0; i < n::VB; ++i) dma_block<DV>(hr.v, L.v[X], w * n::VB + i, tile_pos);
    if (w == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(hr.lg, (lds_void*)L.ell[X], 4,
                                                 (tile_pos + (threadIdx.x & 63)) * 4, 0, 0, kStreamLoad);
}

// Waits until this wavefront's DMA writes of the tile used by the k-th chunk of
// the pass are complete. Younger operations of the wavefront: the next tile's
// DMA (from chunk k-1) and the output stores of chunks k-2 and k-1.
template <int DK, int DV>
__device__ inline void wait_tile(int k) {
    using n = C64Counts<DK, DV>;
    const bool w0 = threadIdx.x < 64;
    if (k == 0) {
        if (w0) wait_vm<n::DMA + 1>(); else wait_vm<n::DMA>();
    } else if (k == 1) {
        if (w0) wait_vm<n::DMA + 1 + n::ST>(); else wait_vm<n::DMA + n::ST>();
    } else {
        if (w0) wait_vm<n::DMA + 1 + 2 * n::ST>(); else wait_vm<n::DMA + 2 * n::ST>();
    }
}

// Wave 0: chunk tables from the DMA'd log-gates (past the end they read 0).
__device__ inline void tables_from_lds(const float* ell, float* tab) {
    const int lane = threadIdx.x;
    float b = clamp_log_gamma(ell[lane], kLogGammaFloor);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(b, off);
        if (lane >= off) b += o;
    }
    const float gc = __shfl(b, 63);
    tab[lane] = b;
    tab[64 + lane] = __expf(gc - b);
    tab[128 + lane] = __expf(b);
}

template <int DK, int DV, int X>
__device__ inline float chunk_dma(const C64Lds<DK, DV>& L, const HeadRsrc& hr,
                                  const __amdgpu_buffer_rsrc_t& out, int k, uint32_t pos,
                                  Acc<DK, DV, 1>& a) {
    wait_tile<DK, DV>(k);
    if (threadIdx.x < 64) tables_from_lds(L.ell[X], L.tab[X]);
    lds_barrier();
    dma_tile<DK, DV, (X + 2) % 3>(L, hr, pos + 2 * kTile);
    const TileView tv{L.q[X], L.k[X], L.v[X], L.tab[X], L.tab[X] + 64, L.tab[X] + 128};
    f32x4 o[4];
    cross_term<DK, DV, 1>(tv, a, 0, o);
    scores_diag<DK, DV, 1>(tv, L.ps, 0);
    lds_barrier();
    apply_scores<DK, DV, 1>(L.ps, tv.vs, true, o);
    store_out<DK, DV, 1>(out, pos, o);
    const float gc = tv.beta[kTile - 1];
    scale_state<DK, DV, 1>(a, __expf(gc));
    state_update<DK, DV, 1>(tv, 0, a.s);
    return gc;
}

// Runs chunks [cb, ce) of head x through the DMA pipeline (same contract as
// run_chunks).
template <int DK, int DV>
__device__ float run_chunks_dma(const Params& p, const C64Lds<DK, DV>& L, int64_t x, int64_t cb,
                                int64_t ce, bool full_from_start, Acc<DK, DV, 1>& a,
                                int64_t* lead) {
    bool full = full_from_start;
    float total = 0.0f;
    *lead = full ? 0 : (ce - cb);
    const HeadRsrc hr = head_rsrc<DK, DV, 1>(p, x);
    const __amdgpu_buffer_rsrc_t drop = make_rsrc(p.out, 0);
    const int nch = static_cast<int>(ce - cb);
    uint32_t pos = static_cast<uint32_t>(cb * kTile);
    // earlier passes of this workgroup: drain their DMA, and let every
    // wavefront finish reading the buffers
    wait_vm<0>();
    lds_barrier();
    dma_tile<DK, DV, 0>(L, hr, pos);
    dma_tile<DK, DV, 1>(L, hr, pos + kTile);
    auto account = [&](float gc, int k) {
        total += gc;
        if (!full && total < kSurvivalDropLog) {
            full = true;
            *lead = k + 1;
        }
    };
    for (int k = 0;; k += 3, pos += 3 * kTile) {
        if (k >= nch) break;
        account(chunk_dma<DK, DV, 0>(L, hr, full ? hr.out : drop, k, pos, a), k);
        if (k + 1 >= nch) break;
        account(chunk_dma<DK, DV, 1>(L, hr, full ? hr.out : drop, k + 1, pos + kTile, a), k + 1);
        if (k + 2 >= nch) break;
        account(chunk_dma<DK, DV, 2>(L, hr, full ? hr.out : drop, k + 2, pos + 2 * kTile, a), k + 2);
    }
    wait_vm<0>();  // no DMA into this workgroup's LDS may outlive the pass
    return total;
}

// LDS of the chunk-64 kernels: three buffer sets, each array its own object.
#define GRET_C64_LDS(DK, DV)                                                              \
    __shared__ __attribute__((aligned(16))) bf16_t q0_[kTile * DK], q1_[kTile * DK],      \
        q2_[kTile * DK];                                                                  \
    __shared__ __attribute__((aligned(16))) bf16_t k0_[kTile * DK], k1_[kTile * DK],      \
        k2_[kTile * DK];                                                                  \
    __shared__ __attribute__((aligned(16))) bf16_t v0_[kTile * DV], v1_[kTile * DV],      \
        v2_[kTile * DV];                                                                  \
    __shared__ __attribute__((aligned(16))) float l0_[kTile], l1_[kTile], l2_[kTile];    \
    __shared__ __attribute__((aligned(16))) float t0_[3 * kTile], t1_[3 * kTile],        \
        t2_[3 * kTile];                                                                   \
    __shared__ __attribute__((aligned(16))) bf16_t ps_[kTile * (kTile + kPadP)];          \
    const C64Lds<DK, DV> L{{q0_, q1_, q2_}, {k0_, k1_, k2_}, {v0_, v1_, v2_},             \
                           {l0_, l1_, l2_}, {t0_, t1_, t2_}, ps_};

template <int DK, int DV>
__global__ __launch_bounds__(kThreadsFor<DV>) void prefill_main_c64_kernel(Params p) {
    GRET_C64_LDS(DK, DV)
    zero_upper_blocks<DK, DV, 1>(L.ps);  // never rewritten
    const SegPlan& pl = p.plan;
    const int64_t gidx = blockIdx.x;
    const int64_t hi = seg_lo(pl, gidx + 1);
    int64_t t = seg_lo(pl, gidx);
    Acc<DK, DV, 1> a;
    while (t < hi) {
        const int64_t x = t / pl.nc;
        const int64_t cb = t - x * pl.nc;
        const int64_t ce = (hi - x * pl.nc) < pl.nc ? (hi - x * pl.nc) : pl.nc;
        const bool initial = cb == 0;
        const int64_t slot = initial ? 0 : gidx - seg_first_inner(pl, x) + 1;
        load_state<DK, DV, 1>(a, initial && p.state_in ? p.state_in + x * DK * DV : nullptr);
        int64_t lead = 0;
        const float total = run_chunks_dma<DK, DV>(p, L, x, cb, ce, initial, a, &lead);
        float* dst = p.ws_state + (x * pl.max_seg + slot) * (int64_t)(DK * DV);
        save_state<DK, DV, 1>(a, dst);
        if (threadIdx.x == 0) p.ws_meta[x * pl.max_seg + slot] = make_float2(total, (float)lead);
        t = x * pl.nc + ce;
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreadsFor<DV>) void prefill_prefix_c64_kernel(Params p) {
    GRET_C64_LDS(DK, DV)
    const SegPlan& pl = p.plan;
    const int64_t gidx = blockIdx.x;
    const int64_t lo = seg_lo(pl, gidx);
    const int64_t x = lo / pl.nc;
    const int64_t cb = lo - x * pl.nc;
    if (cb == 0) return;  // this workgroup starts at a head boundary: nothing to redo
    const int64_t slot = gidx - seg_first_inner(pl, x) + 1;
    const int64_t lead = static_cast<int64_t>(p.ws_meta[x * pl.max_seg + slot].y);
    if (lead <= 0) return;
    zero_upper_blocks<DK, DV, 1>(L.ps);
    Acc<DK, DV, 1> a;
    load_state<DK, DV, 1>(a, p.ws_state + (x * pl.max_seg + slot) * (int64_t)(DK * DV));
    int64_t unused = 0;
    run_chunks_dma<DK, DV>(p, L, x, cb, cb + lead, true, a, &unused);
}
#undef GRET_C64_LDS

// Runs chunks [cb, ce) of head x. With full_from_start the pass computes
// outputs from the first chunk; otherwise only the state until the running
// log-decay drops below kSurvivalDropLog (then outputs too). Returns the total
// log-decay; *lead receives the number of state-only chunks.
template <int DK, int DV, int R>
__device__ float run_chunks(const Params& p, Smem<DK, DV, R>& sm, Smem2<DK, DV>* s2, int64_t x,
                            int64_t cb, int64_t ce, bool full_from_start, Acc<DK, DV, R>& a,
                            int64_t* lead) {
    if constexpr (R == 1) {
        (void)s2;
        return run_chunks_c64<DK, DV, R>(p, sm, x, cb, ce, full_from_start, a, lead);
    } else {
        using c = Cfg<DK, DV, R>;
        bool full = full_from_start;
        float total = 0.0f;
        *lead = full ? 0 : (ce - cb);
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk) a.ds[tk] = f32x4{0.f, 0.f, 0.f, 0.f};
        const HeadRsrc hr = head_rsrc<DK, DV, R>(p, x);
        TileRegs<DK, DV, R> tr;
        load_tile<DK, DV, R>(hr, static_cast<uint32_t>(cb * c::C),
                             static_cast<uint32_t>(cb * c::C), tr);
        for (int64_t ch = cb; ch < ce; ++ch) {
            const int64_t cpos = ch * c::C;
            const int64_t nvalid = p.N - cpos < c::C ? p.N - cpos : c::C;
            const int rv = static_cast<int>((nvalid + kTile - 1) / kTile);
            for (int r = 0; r < rv; ++r) {
                const uint32_t tpos = static_cast<uint32_t>(cpos + kTile * r);
                TileBuf<DK, DV, R>& tb = sm.buf[0];
                if (r == 0) make_tables<DK, DV, R>(tr, tb);
                write_tile<DK, DV, R>(tr, tb.qs, tb.ks, tb.vs);
                __syncthreads();
                const float gc = tb.beta[c::C - 1];
                if (r + 1 < rv) {
                    load_tile<DK, DV, R>(hr, tpos + kTile, static_cast<uint32_t>(cpos), tr);
                } else if (ch + 1 < ce) {
                    load_tile<DK, DV, R>(hr, static_cast<uint32_t>(cpos + c::C),
                                         static_cast<uint32_t>(cpos + c::C), tr);
                }
                if (full) {
                    f32x4 o[4];
                    cross_term<DK, DV, R>(tb, a, r, o);
                    for (int t = 0; t < r; ++t) {
                        restage<DK, DV, R>(hr, static_cast<uint32_t>(cpos + kTile * t), *s2);
                        __syncthreads();
                        scores_full<DK, DV, R>(tb, sm.ps, s2->ks, r, t);
                        __syncthreads();
                        apply_scores<DK, DV, R>(sm.ps, s2->vs, false, o);
                        __syncthreads();
                    }
                    zero_upper_blocks<DK, DV, R>(sm.ps);
                    scores_diag<DK, DV, R>(tb, sm.ps, r);
                    __syncthreads();
                    apply_scores<DK, DV, R>(sm.ps, tb.vs, true, o);
                    store_out<DK, DV, R>(hr.out, tpos, o);
                }
                state_update<DK, DV, R>(tb, r, a.ds);
                if (r == rv - 1) {
                    const float eg = __expf(gc);
#pragma unroll
                    for (int tk = 0; tk < c::TK; ++tk) {
                        f32x4& sv = a.s[tk];
                        f32x4& dv = a.ds[tk];
                        sv[0] = fmaf(eg, sv[0], dv[0]);
                        sv[1] = fmaf(eg, sv[1], dv[1]);
                        sv[2] = fmaf(eg, sv[2], dv[2]);
                        sv[3] = fmaf(eg, sv[3], dv[3]);
                        dv = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                    total += gc;
                    if (!full && total < kSurvivalDropLog) {
                        full = true;
                        *lead = ch + 1 - cb;
                    }
                }
                __syncthreads();  // LDS tiles are rewritten next iteration
            }
        }
        return total;
    }
}

template <int DK, int DV, int R>
__device__ inline void load_state(Acc<DK, DV, R>& a, const float* src) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    if (!src) {
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk) a.s[tk] = f32x4{0.f, 0.f, 0.f, 0.f};
        return;
    }
#pragma unroll
    for (int tk = 0; tk < c::TK; ++tk)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.s[tk][i] = src[(16 * tk + 4 * g + i) * DV + 16 * w + li];
}

template <int DK, int DV, int R>
__device__ inline void save_state(const Acc<DK, DV, R>& a, float* dst) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tk = 0; tk < c::TK; ++tk)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * tk + 4 * g + i) * DV + 16 * w + li] = a.s[tk][i];
}

template <int DK, int DV, int R>
__global__ __launch_bounds__(kThreadsFor<DV>) void prefill_main_kernel(Params p) {
    __shared__ SmemAll<DK, DV, R> all;
    Smem<DK, DV, R>& sm = all.m;
    Smem2<DK, DV>* s2 = all.extra();
    if constexpr (R == 1) zero_upper_blocks<DK, DV, R>(sm.ps);  // never rewritten
    const SegPlan& pl = p.plan;
    const int64_t gidx = blockIdx.x;
    const int64_t hi = seg_lo(pl, gidx + 1);
    int64_t t = seg_lo(pl, gidx);
    Acc<DK, DV, R> a;
    while (t < hi) {
        const int64_t x = t / pl.nc;
        const int64_t cb = t - x * pl.nc;
        const int64_t ce = (hi - x * pl.nc) < pl.nc ? (hi - x * pl.nc) : pl.nc;
        const bool initial = cb == 0;
        const int64_t slot = initial ? 0 : gidx - seg_first_inner(pl, x) + 1;
        load_state<DK, DV, R>(a, initial && p.state_in ? p.state_in + x * DK * DV : nullptr);
        int64_t lead = 0;
        const float total = run_chunks<DK, DV, R>(p, sm, s2, x, cb, ce, initial, a, &lead);
        float* dst = p.ws_state + (x * pl.max_seg + slot) * (int64_t)(DK * DV);
        save_state<DK, DV, R>(a, dst);
        if (threadIdx.x == 0) p.ws_meta[x * pl.max_seg + slot] = make_float2(total, (float)lead);
        t = x * pl.nc + ce;
    }
}

template <int DK, int DV, int R>
__global__ __launch_bounds__(kThreadsFor<DV>) void prefill_prefix_kernel(Params p) {
    __shared__ SmemAll<DK, DV, R> all;
    Smem<DK, DV, R>& sm = all.m;
    Smem2<DK, DV>* s2 = all.extra();
    const SegPlan& pl = p.plan;
    const int64_t gidx = blockIdx.x;
    const int64_t lo = seg_lo(pl, gidx);
    const int64_t x = lo / pl.nc;
    const int64_t cb = lo - x * pl.nc;
    if (cb == 0) return;  // this workgroup starts at a head boundary: nothing to redo
    const int64_t slot = gidx - seg_first_inner(pl, x) + 1;
    const int64_t lead = static_cast<int64_t>(p.ws_meta[x * pl.max_seg + slot].y);
    if (lead <= 0) return;
    if constexpr (R == 1) zero_upper_blocks<DK, DV, R>(sm.ps);  // never rewritten
    Acc<DK, DV, R> a;
    load_state<DK, DV, R>(a, p.ws_state + (x * pl.max_seg + slot) * (int64_t)(DK * DV));
    int64_t unused = 0;
    run_chunks<DK, DV, R>(p, sm, s2, x, cb, cb + lead, true, a, &unused);
}

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

template <int DK, int DV, int R>
hipError_t launch_rc(const PrefillArgs& a, const SegPlan& plan) {
    Params p;
    p.q = static_cast<const bf16_t*>(a.q);
    p.k = static_cast<const bf16_t*>(a.k);
    p.v = static_cast<const bf16_t*>(a.v);
    p.log_gamma = a.log_gamma;
    p.state_in = a.state_in;
    p.out = static_cast<bf16_t*>(a.out);
    p.state_out = a.state_out;
    const PrefillWorkspace lay = bf16_workspace_layout(plan, DK, DV);
    p.ws_state = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + lay.state_off);
    p.ws_meta = reinterpret_cast<float2*>(static_cast<char*>(a.workspace) + lay.meta_off);
    p.plan = plan;
    p.N = a.N;
    const dim3 block(Cfg<DK, DV, R>::NT);
    if constexpr (R == 1)
        hipLaunchKernelGGL((prefill_main_c64_kernel<DK, DV>), dim3(plan.G), block, 0, a.stream, p);
    else
        hipLaunchKernelGGL((prefill_main_kernel<DK, DV, R>), dim3(plan.G), block, 0, a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int per_head = DK * DV / (kCombineThreads * 4);
    hipLaunchKernelGGL((prefill_combine_kernel<DK, DV>), dim3(plan.BH * per_head),
                       dim3(kCombineThreads), 0, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (R == 1)
        hipLaunchKernelGGL((prefill_prefix_c64_kernel<DK, DV>), dim3(plan.G), block, 0, a.stream, p);
    else
        hipLaunchKernelGGL((prefill_prefix_kernel<DK, DV, R>), dim3(plan.G), block, 0, a.stream, p);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const PrefillArgs& a, const SegPlan& plan) {
    switch (a.chunk) {
        case 64: return launch_rc<DK, DV, 1>(a, plan);
        case 128: return launch_rc<DK, DV, 2>(a, plan);
        case 256: return launch_rc<DK, DV, 4>(a, plan);
        default: return hipErrorInvalidValue;
    }
}

template <int DK, int DV, int R>
int blocks_per_cu_rc() {
    int n = 0;
    hipError_t e;
    if constexpr (R == 1)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_main_c64_kernel<DK, DV>,
                                                         Cfg<DK, DV, R>::NT, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_main_kernel<DK, DV, R>,
                                                         Cfg<DK, DV, R>::NT, 0);
    return e == hipSuccess ? n : 0;
}

template <int DK, int DV>
int blocks_per_cu_dims(int64_t chunk) {
    switch (chunk) {
        case 64: return blocks_per_cu_rc<DK, DV, 1>();
        case 128: return blocks_per_cu_rc<DK, DV, 2>();
        case 256: return blocks_per_cu_rc<DK, DV, 4>();
        default: return 0;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, const SegPlan& plan) {
    if (a.dk == 64 && a.dv == 64) return launch_dims<64, 64>(a, plan);
    if (a.dk == 64 && a.dv == 128) return launch_dims<64, 128>(a, plan);
    if (a.dk == 128 && a.dv == 64) return launch_dims<128, 64>(a, plan);
    if (a.dk == 128 && a.dv == 128) return launch_dims<128, 128>(a, plan);
    return hipErrorInvalidValue;
}

int prefill_bf16_blocks_per_cu(int64_t dk, int64_t dv, int64_t chunk) {
    if (dk == 64 && dv == 64) return blocks_per_cu_dims<64, 64>(chunk);
    if (dk == 64 && dv == 128) return blocks_per_cu_dims<64, 128>(chunk);
    if (dk == 128 && dv == 64) return blocks_per_cu_dims<128, 64>(chunk);
    if (dk == 128 && dv == 128) return blocks_per_cu_dims<128, 128>(chunk);
    return 0;
}

}  // namespace gret
