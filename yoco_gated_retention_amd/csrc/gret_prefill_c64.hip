// gret_prefill_c64.hip -- chunkwise gated-retention prefill in chunks of 64
// positions on gfx950 matrix cores (bf16 operands, fp32 accumulation, fp32
// state carry). This is the default and fastest chunk size.
//
// Method (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次",
// sections "路线二：Multi-Head Gated Retention" and "Prefill 与 Decode 为什么使用
// 两种计算形态"): inside a chunk of 64 positions starting at a, with beta_j the
// chunk-local inclusive sum of log-gates,
//   out[a+j] = exp(beta_j) q_{a+j} S + sum_{l<=j} exp(beta_j - beta_l) (q_{a+j}.k_{a+l}) v_{a+l}
//   S       <- exp(beta_63) S + sum_l exp(beta_63 - beta_l) k_{a+l}^T v_{a+l}
// Only differences of log-decays inside a chunk are exponentiated, so every
// factor is at most 1. The head-wise scalar gate keeps every contraction a
// plain matrix product (same section, on head-wise versus element-wise decay).
//
// Parallel schedule: segments of each head's chunk sequence run concurrently
// (gret_segments.h), in three launches: main (every segment from a zero state,
// non-first segments output-free until the incoming state's survival factor
// is below fp32 resolution), combine (chains the affine segment maps), prefix
// (recomputes the leading chunks of non-first segments from their incoming
// state).
//
// Workgroup: DV/16 wavefronts (8 at dv = 128, two per SIMD); wavefront w owns
// value columns [16w, 16w + 16) of the state (fp32 accumulator registers for
// the whole segment) and of the output. Every wavefront contracts the whole Q
// tile (cross term) and K tile (state update) against its own columns.
//
// Per chunk, tiles of Q, K, V and the log-gates go from HBM straight into LDS
// with buffer_load ... lds into one of three buffer sets, two chunks ahead of
// the one being computed. Tiles are row-major with an XOR swizzle of 16-byte
// chunks; operands contracted over positions (K^T, V^T) are read with the
// transposing LDS load ds_read_b64_tr_b16.
//   * cross    O^T = S^T Q^T (S straight from the accumulators), row j scaled
//              by exp(beta_j);
//   * scores   P^T = K Q^T on the 10 causal 16x16 blocks, decay mask
//              exp(beta_j - beta_l) in fp32, rounded to bf16 into LDS;
//   * output   O^T += V^T P~^T; the output tile is staged in the chunk's own V
//              buffer (each wavefront overwrites only its own value columns,
//              which only it reads) and leaves with full-row 16-byte stores
//              one chunk later;
//   * state    S = exp(g) S + K^T (Gamma V), Gamma_l = exp(g - beta_l).
//
// Gated kernels (template flag): the output epilogue of the same page and
// section (per-head GroupNorm, then the swish output gate) is applied as each
// output tile leaves LDS. The gate tile streams into an LDS buffer of its own,
// one chunk ahead; the queries are double-buffered to make room for it. The
// output rows are normalised from the bf16 tile, the values the plain kernel
// stores, so the result equals the plain prefill followed by the epilogue pass.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gret_prefill_common.h"

namespace gret {
namespace {

// 16-column tiles of the state per wavefront. Two (4 wavefronts at dv = 128,
// one per SIMD) halve the LDS reads of Q and K but leave every LDS and matrix
// latency exposed; it measured 1.37x slower than one (8 wavefronts, two per
// SIMD).
constexpr int kColTiles = 1;

template <int DK, int DV>
struct C64 {
    static constexpr int CT = kColTiles;       // 16-column tiles per wavefront
    static constexpr int NW = DV / (16 * CT);  // wavefronts
    static constexpr int NT = 64 * NW;         // threads per workgroup
    static constexpr int TK = DK / 16;         // 16-row key tiles of the state
    static constexpr int KS = DK / 32;         // 32-wide k-steps over dk
    static constexpr int PP = kTile + kPadP;   // row pitch (elements) of the score tile
    static constexpr int QB = DK / 8 / NW;     // 1 KB DMA blocks of Q (and of K) per wavefront
    static constexpr int VB = DV / 8 / NW;     // 1 KB DMA blocks of V per wavefront
    static constexpr int DMA = 2 * QB + VB + 1;  // DMA instructions per wavefront and tile
    static constexpr int ST = VB;              // output stores per wavefront and chunk
    static_assert(NW == 4 || NW == 8, "wavefronts");
    static_assert(QB * NW * 8 == DK && VB * NW * 8 == DV, "DMA split");
    static_assert(DK / 8 >= 8 && DV / 8 >= 8, "swizzle spans 8 chunks");
};

template <int DV>
constexpr int kThreadsFor = 64 * (DV / (16 * kColTiles));

// LDS tile layout. Tiles are row-major with the 16-byte chunks of row r
// permuted by c -> c ^ sigma(r). On gfx950 the LDS banks repeat every 128
// bytes for 8- and 16-byte accesses, and each tile has its own access mix, so
// each gets its own sigma (measured per access pattern, bytes per clock and
// CU, 128-column tiles):
//   Q: 8-byte row-fragment reads (cross term) and 16-byte row-fragment reads
//      (scores): sigma = 4 (r % 2) + (r / 2) % 4 + 8 ((r / 8) % 2), 216 and 229;
//   K: 16-byte row fragments (scores) and transposing reads (state update),
//   V: transposing reads and 8-byte fragment writes (output staging):
//      sigma = 2 (r % 4) + (r / 4) % 2 + 8 ((r / 8) % 2), 124 / 173 / 210.
// (The layout used by the chunk-128/256 kernels gives 117 / 165 / 195.)
// 64-column tiles use sigma = r % 8 for all three (226 / 117 / 122).
enum TileKind { kTileQ = 0, kTileK = 1, kTileV = 2 };

template <int D, int T>
__device__ inline int tswz(int r) {
    if constexpr (D == 128) {
        if constexpr (T == kTileQ) return ((r & 1) << 2) | ((r >> 1) & 3) | (((r >> 3) & 1) << 3);
        return ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3);
    } else {
        static_assert(D == 64, "tile width");
        return r & 7;
    }
}

// Element offset of (row, col) in a tile of kind T with D columns.
template <int D, int T>
__device__ inline int toff_t(int row, int col) {
    return row * D + (((col >> 3) ^ tswz<D, T>(row)) << 3) + (col & 7);
}

// A per-lane LDS offset that the compiler may neither move out of the chunk
// loop nor merge with another:
//  * hoisted, base + offset is one register per buffer of a kind and per
//    offset for the whole loop (three copies of every Q, K and V operand
//    address); kept in the loop, the buffer's base folds into the
//    instruction's offset field and one register per offset serves every
//    buffer. That frees the registers that the gated kernels' epilogue needs
//    (without it they spill 71 registers);
//  * two 8-byte accesses a constant distance apart would otherwise become one
//    ds_read2st64_b64 / ds_write2st64_b64, which measured at a third of the
//    throughput of the two separate accesses.
__device__ inline int pinned(int off) {
    asm volatile("" : "+v"(off));
    return off;
}

// The plain kernels keep the hoisted addresses (they fit, and measured about
// 1 % faster) and only block the merging of 8-byte accesses (sep).
template <bool PIN>
__device__ inline int loff(int off) {
    if constexpr (PIN) return pinned(off);
    return off;
}
template <bool PIN>
__device__ inline int sep(int off) {
    if constexpr (PIN) return pinned(off);
    asm("" : "+v"(off));
    return off;
}

// 8 consecutive positions t0..t0+7 of column col0 + l (l = this lane's index
// in its 16-lane group) of a tile: the MFMA operand for a contraction over
// positions, read with the transposing LDS load.
template <int D, int T, bool PIN>
__device__ inline bf16x8 read_cols8_t(const bf16_t* tile, int t0, int col0) {
    const int s = threadIdx.x & 15;
    const int row = t0 + (s >> 2);
    const int col = col0 + 4 * (s & 3);
    const bf16x4 a = lds_read_tr4(tile + loff<PIN>(toff_t<D, T>(row, col)));
    const bf16x4 b = lds_read_tr4(tile + loff<PIN>(toff_t<D, T>(row + 4, col)));
    return cat44(a, b);
}

// First value column of column tile ct of this wavefront.
template <int DK, int DV>
__device__ inline int col0(int ct) {
    return 16 * (C64<DK, DV>::CT * (static_cast<int>(threadIdx.x) >> 6) + ct);
}

// State of one segment's pass: s[ct][tk][i] = S[16 tk + 4 g + i][col0(ct) + li]
// (li = lane % 16, g = lane / 16).
template <int DK, int DV>
struct Acc {
    f32x4 s[C64<DK, DV>::CT][C64<DK, DV>::TK];
};

template <int DK, int DV>
__device__ inline void load_state(Acc<DK, DV>& a, const float* src) {
    using c = C64<DK, DV>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < c::CT; ++ct)
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.s[ct][tk][i] = src ? src[(16 * tk + 4 * g + i) * DV + col0<DK, DV>(ct) + li] : 0.f;
}

template <int DK, int DV>
__device__ inline void save_state(const Acc<DK, DV>& a, float* dst) {
    using c = C64<DK, DV>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < c::CT; ++ct)
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[(16 * tk + 4 * g + i) * DV + col0<DK, DV>(ct) + li] = a.s[ct][tk][i];
}

template <int DK, int DV>
__device__ inline void scale_state(Acc<DK, DV>& a, float eg) {
    using c = C64<DK, DV>;
#pragma unroll
    for (int ct = 0; ct < c::CT; ++ct)
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk) {
            a.s[ct][tk][0] *= eg;
            a.s[ct][tk][1] *= eg;
            a.s[ct][tk][2] *= eg;
            a.s[ct][tk][3] *= eg;
        }
}

// LDS views of one chunk: its tiles and its tables.
struct TileView {
    const bf16_t* qs;
    const bf16_t* ks;
    bf16_t* vs;
    const float* beta;  // chunk-local inclusive log-decay
    const float* gam;   // exp(beta_63 - beta_l): weight of position l in the state update
    const float* fexp;  // exp(beta_j): weight of the incoming state in output j
};

// Cross-chunk term O^T = S^T Q^T for the 64 rows, then row j scaled by
// exp(beta_j). The state tile pair (2m, 2m+1) gives each lane
// dk = 32m + {4g..4g+3, 16+4g..16+4g+3}; the Q operand is read with the same
// permutation of dk, so the contraction pairs matching indices. Each Q
// fragment serves all column tiles of the wavefront.
template <int DK, int DV, bool PIN>
__device__ inline void cross_term(const TileView& tv, const Acc<DK, DV>& a,
                                  f32x4 (&o)[C64<DK, DV>::CT][4]) {
    using c = C64<DK, DV>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < c::CT; ++ct)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) o[ct][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < c::KS; ++m) {
        bf16x8 sf[c::CT];
#pragma unroll
        for (int ct = 0; ct < c::CT; ++ct) {
            const f32x4 lo4 = a.s[ct][2 * m], hi4 = a.s[ct][2 * m + 1];
            sf[ct] = bf16x8{to_bf16(lo4[0]), to_bf16(lo4[1]), to_bf16(lo4[2]), to_bf16(lo4[3]),
                            to_bf16(hi4[0]), to_bf16(hi4[1]), to_bf16(hi4[2]), to_bf16(hi4[3])};
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const int row = 16 * jt + li;
            const bf16x8 qf =
                cat44(lds_read4(tv.qs + sep<PIN>(toff_t<DK, kTileQ>(row, 32 * m + 4 * g))),
                      lds_read4(tv.qs + sep<PIN>(toff_t<DK, kTileQ>(row, 32 * m + 16 + 4 * g))));
#pragma unroll
            for (int ct = 0; ct < c::CT; ++ct) o[ct][jt] = mfma16(sf[ct], qf, o[ct][jt]);
        }
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const float f = tv.fexp[16 * jt + li];
#pragma unroll
        for (int ct = 0; ct < c::CT; ++ct) {
            o[ct][jt][0] *= f;
            o[ct][jt][1] *= f;
            o[ct][jt][2] *= f;
            o[ct][jt][3] *= f;
        }
    }
}

// Decayed score block (jb, b): query rows 16jb.. against key positions 16b..,
// written as bf16 to ps[j][l]; entries above the diagonal are zero.
template <int DK, int DV, bool PIN>
__device__ inline void score_block(const TileView& tv, bf16_t* ps, int jb, int b) {
    using c = C64<DK, DV>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int jrow = 16 * jb + li;
    const float bj = tv.beta[jrow];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < c::KS; ++ks) {
        const bf16x8 qf = lds_read8(tv.qs + loff<PIN>(toff_t<DK, kTileQ>(jrow, 32 * ks + 8 * g)));
        const bf16x8 kf = lds_read8(tv.ks + loff<PIN>(toff_t<DK, kTileK>(16 * b + li, 32 * ks + 8 * g)));
        acc = mfma16(kf, qf, acc);
    }
    // acc[i] = P^T[l = 16b + 4g + i][j = jrow]
    bf16x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int l = 16 * b + 4 * g + i;
        const float val = l <= jrow ? acc[i] * __expf(bj - tv.beta[l]) : 0.0f;
        pk[i] = to_bf16(val);
    }
    *reinterpret_cast<bf16x4*>(ps + jrow * c::PP + 16 * b + 4 * g) = pk;
}

// Wavefront w computes causal blocks w, w + NW, ...
template <int DK, int DV, bool PIN>
__device__ inline void scores_diag(const TileView& tv, bf16_t* ps) {
    const int w = threadIdx.x >> 6;
    for (int i = w; i < 10; i += C64<DK, DV>::NW) {
        const int e = static_cast<int>((kCausalBlocks >> (4 * i)) & 0xF);
        score_block<DK, DV, PIN>(tv, ps, e >> 2, e & 3);
    }
}

// Blocks (0,1) and (2,3) lie above the diagonal but inside 32-position steps
// that the diagonal product uses; they hold zeros and are never rewritten.
template <int DK, int DV>
__device__ inline void zero_upper_blocks(bf16_t* ps) {
    using c = C64<DK, DV>;
    for (int e = threadIdx.x; e < 2 * 16 * 4; e += c::NT) {
        const int blk = e / 64, rem = e % 64;
        const int jb = blk == 0 ? 0 : 2, b = jb + 1;
        const int row = 16 * jb + rem / 4, col = 16 * b + 4 * (rem % 4);
        *reinterpret_cast<bf16x4*>(ps + row * c::PP + col) = bf16x4{};
    }
}

// O^T[cols][rows] += V^T P~^T (V read transposed); 32-position steps wholly
// above the diagonal are skipped. Each P~ fragment serves all column tiles.
template <int DK, int DV, bool PIN>
__device__ inline void apply_scores(const bf16_t* ps, const bf16_t* vs,
                                    f32x4 (&o)[C64<DK, DV>::CT][4]) {
    using c = C64<DK, DV>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        bf16x8 vf[c::CT];
#pragma unroll
        for (int ct = 0; ct < c::CT; ++ct) vf[ct] = read_cols8_t<DV, kTileV, PIN>(vs, 32 * ks + 8 * g, col0<DK, DV>(ct));
#pragma unroll
        for (int jt = 2 * ks; jt < 4; ++jt) {
            const bf16x8 pf = lds_read8(ps + (16 * jt + li) * c::PP + 32 * ks + 8 * g);
#pragma unroll
            for (int ct = 0; ct < c::CT; ++ct) o[ct][jt] = mfma16(vf[ct], pf, o[ct][jt]);
        }
    }
}

// S += K^T (Gamma V) over the chunk; K and V are read transposed so that
// positions are the contraction index. Each K fragment serves all column
// tiles.
template <int DK, int DV, bool PIN>
__device__ inline void state_update(const TileView& tv, Acc<DK, DV>& a) {
    using c = C64<DK, DV>;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int t0 = 32 * ks + 8 * g;
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(tv.gam + t0);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(tv.gam + t0 + 4);
        bf16x8 bf[c::CT];
#pragma unroll
        for (int ct = 0; ct < c::CT; ++ct) {
            const bf16x8 vf = read_cols8_t<DV, kTileV, PIN>(tv.vs, t0, col0<DK, DV>(ct));
            bf[ct] = bf16x8{to_bf16(from_bf16(vf[0]) * g0[0]), to_bf16(from_bf16(vf[1]) * g0[1]),
                            to_bf16(from_bf16(vf[2]) * g0[2]), to_bf16(from_bf16(vf[3]) * g0[3]),
                            to_bf16(from_bf16(vf[4]) * g1[0]), to_bf16(from_bf16(vf[5]) * g1[1]),
                            to_bf16(from_bf16(vf[6]) * g1[2]), to_bf16(from_bf16(vf[7]) * g1[3])};
        }
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk) {
            const bf16x8 kf = read_cols8_t<DK, kTileK, PIN>(tv.ks, t0, 16 * tk);
#pragma unroll
            for (int ct = 0; ct < c::CT; ++ct) a.s[ct][tk] = mfma16(kf, bf[ct], a.s[ct][tk]);
        }
    }
}

// The chunk's output into its own V buffer (swizzled row-major, bf16): each
// lane's fragment is 4 consecutive columns of one row.
template <int DK, int DV, bool PIN>
__device__ inline void out_to_lds(bf16_t* vs, const f32x4 (&o)[C64<DK, DV>::CT][4]) {
    using c = C64<DK, DV>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < c::CT; ++ct)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const bf16x4 pk = {to_bf16(o[ct][jt][0]), to_bf16(o[ct][jt][1]),
                               to_bf16(o[ct][jt][2]), to_bf16(o[ct][jt][3])};
            *reinterpret_cast<bf16x4*>(
                vs + sep<PIN>(toff_t<DV, kTileV>(16 * jt + li, col0<DK, DV>(ct) + 4 * g))) = pk;
        }
}

// Inclusive prefix sum over the 64 lanes of a wavefront: shifts by 1, 2, 4 and 8
// lanes inside each 16-lane row, then the row totals carried across rows by the
// row broadcasts of lanes 15 and 31 (DPP moves: no LDS crossbar round trips).
// Lanes with no source add the identity 0.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_or_zero(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, ROW_MASK, 0xF, false));
}

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

// Wavefront 0: chunk tables from the log-gates in LDS (past the end they read 0).
__device__ inline void tables_from_lds(const float* ell, float* tab) {
    const int lane = threadIdx.x;
    const float b = wave_inclusive_sum(clamp_log_gamma(ell[lane], kLogGammaFloor));
    const float gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, b), 63));
    tab[lane] = b;
    tab[64 + lane] = __expf(gc - b);
    tab[128 + lane] = __expf(b);
}


// Cache policy of the streamed q/k/v/log-gate loads: nontemporal (each byte is
// read once). The output stores keep the default write-back policy: with the
// nontemporal bit they measured 1.5x slower.
constexpr int kStreamLoad = 2;

// One 1 KB DMA instruction of a swizzled row-major tile with D columns: lane i
// lands at LDS byte 16 i of block blk, i.e. row (512/D) blk + i / (D/8), slot
// i % (D/8), so it fetches the global 16-byte chunk slot ^ swz(row) of that row.
template <int D, int T>
__device__ inline void dma_block(__amdgpu_buffer_rsrc_t r, bf16_t* tile, int blk,
                                 uint32_t tile_pos) {
    constexpr int RPI = 512 / D;  // rows per instruction
    constexpr int SPR = D / 8;    // 16-byte slots per row
    const int lane = threadIdx.x & 63;
    const int row = RPI * blk + lane / SPR;
    const int chunk = (lane % SPR) ^ tswz<D, T>(row);
    const uint32_t voff = ((tile_pos + row) * D + chunk * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + blk * 512), 16, voff, 0, 0,
                                             kStreamLoad);
}

// The inverse of dma_block: lane i reads LDS byte 16 i of block blk of a
// swizzled output tile and stores it to its place in global memory, so one
// instruction writes 512/D complete, consecutive rows (1 KB contiguous).
template <int D, int T>
__device__ inline void flush_block(__amdgpu_buffer_rsrc_t r, const bf16_t* tile, int blk,
                                   uint32_t tile_pos) {
    constexpr int RPI = 512 / D;
    constexpr int SPR = D / 8;
    const int lane = threadIdx.x & 63;
    const int row = RPI * blk + lane / SPR;
    const int chunk = (lane % SPR) ^ tswz<D, T>(row);
    const bf16x8 val = lds_read8(tile + blk * 512 + 8 * lane);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, val), r,
                                           ((tile_pos + row) * D + chunk * 8) * 2, 0, 0);
}

template <int DK, int DV>
struct Lds {
    bf16_t* q[3];
    bf16_t* k[3];
    bf16_t* v[3];
    float* ell[3];
    float* tab[3];  // beta[64] | gam[64] | fexp[64]
    bf16_t* ps;
    float* sink;    // target of the log-gate DMA of wavefronts other than 0
    bf16_t* gt;     // gated kernels: gate tile of the output being flushed
    float* aff;     // gated kernels: the head's norm weight[DV] | bias[DV]
};

// Issues this wavefront's share of the DMA of the tile at tile_pos into set X.
// Wavefront 0 loads the 64 log-gates; the others issue the same instruction
// through a zero-size descriptor into a sink (no data moves), so that all
// wavefronts issue the same number of memory operations. q is the head's query
// descriptor, or a zero-size one for a tile whose outputs are not computed
// (its loads then move no data but still count as operations).
template <int DK, int DV, int X>
__device__ inline void dma_q(const Lds<DK, DV>& L, const __amdgpu_buffer_rsrc_t& q,
                             uint32_t tile_pos) {
    using c = C64<DK, DV>;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < c::QB; ++i) dma_block<DK, kTileQ>(q, L.q[X], w * c::QB + i, tile_pos);
}

template <int DK, int DV, int X>
__device__ inline void dma_k(const Lds<DK, DV>& L, const HeadRsrc& hr, uint32_t tile_pos) {
    using c = C64<DK, DV>;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < c::QB; ++i) dma_block<DK, kTileK>(hr.k, L.k[X], w * c::QB + i, tile_pos);
}

template <int DK, int DV, int X>
__device__ inline void dma_v_ell(const Lds<DK, DV>& L, const HeadRsrc& hr,
                                 const __amdgpu_buffer_rsrc_t& none, uint32_t tile_pos) {
    using c = C64<DK, DV>;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < c::VB; ++i) dma_block<DV, kTileV>(hr.v, L.v[X], w * c::VB + i, tile_pos);
    const bool w0 = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) == 0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(w0 ? hr.lg : none,
                                             (lds_void*)(w0 ? L.ell[X] : L.sink), 4,
                                             (tile_pos + (threadIdx.x & 63)) * 4, 0, 0,
                                             kStreamLoad);
}

template <int DK, int DV, int X>
__device__ inline void dma_tile(const Lds<DK, DV>& L, const HeadRsrc& hr,
                                const __amdgpu_buffer_rsrc_t& q,
                                const __amdgpu_buffer_rsrc_t& none, uint32_t tile_pos) {
    dma_q<DK, DV, X>(L, q, tile_pos);
    dma_k<DK, DV, X>(L, hr, tile_pos);
    dma_v_ell<DK, DV, X>(L, hr, none, tile_pos);
}

// Stores the output tile staged in a V buffer. Each wavefront flushes exactly
// the rows that its own DMA of the next V tile overwrites, so it needs no
// barrier between the two: its LDS reads complete before its stores issue.
template <int DK, int DV>
__device__ inline void flush_tile(const bf16_t* vs, const __amdgpu_buffer_rsrc_t& out,
                                  uint32_t tile_pos) {
    using c = C64<DK, DV>;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < c::VB; ++i) flush_block<DV, kTileV>(out, vs, w * c::VB + i, tile_pos);
}

// The gate rows of the tile at tile_pos into the gate buffer, in the layout of
// a V tile: each wavefront loads the blocks whose outputs it flushes.
template <int DK, int DV>
__device__ inline void dma_gate(bf16_t* gt, const __amdgpu_buffer_rsrc_t& g, uint32_t tile_pos) {
    using c = C64<DK, DV>;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < c::VB; ++i) dma_block<DV, kTileV>(g, gt, w * c::VB + i, tile_pos);
}

// flush_tile with the output epilogue of gated retention (page "YOCO 完全拆解：
// Decoder-Decoder 架构如何让 KV Cache 只存一次", section "路线二：Multi-Head Gated
// Retention": per-head GroupNorm over the dv channels of a position, then the
// element-wise gate swish(X W_G)). Lane i holds 8 channels of one row, a row's
// DV / 8 lanes are adjacent, so mean and variance (two passes, fp32) are
// reductions inside a lane group; the gate piece sits at the same LDS offset
// in the gate buffer, the affine of the piece's channels in aff. As in
// flush_tile, the DMAs issued right after it (the next gate tile and the next
// V tile) overwrite only this wavefront's blocks, whose LDS reads have
// completed because the stores consume them.
//   y = swish(gate) * ((o - mean) / sqrt(var + eps) * w + b)
template <int DK, int DV>
__device__ inline void flush_tile_gated(const bf16_t* vs, const bf16_t* gt, const float* aff,
                                        const __amdgpu_buffer_rsrc_t& out, uint32_t tile_pos,
                                        float eps) {
    using c = C64<DK, DV>;
    constexpr int RPI = 512 / DV;
    constexpr int SPR = DV / 8;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < c::VB; ++i) {
        const int blk = w * c::VB + i;
        const int row = RPI * blk + lane / SPR;
        const int chunk = (lane % SPR) ^ tswz<DV, kTileV>(row);
        const int po = pinned(blk * 512 + 8 * lane);
        const bf16x8 xv = lds_read8(vs + po);
        const bf16x8 gv = lds_read8(gt + po);
        const int a0 = pinned(chunk * 8);
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(aff + a0);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(aff + a0 + 4);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(aff + DV + a0);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(aff + DV + a0 + 4);
        float x[8];
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = from_bf16(xv[e]);
            sum += x[e];
        }
        const float mean = group_sum<SPR>(sum) * (1.0f / DV);
        float sq = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sq += (x[e] - mean) * (x[e] - mean);
        const float rstd = rsqrtf(group_sum<SPR>(sq) * (1.0f / DV) + eps);
        bf16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float we = e < 4 ? w0[e] : w1[e - 4];
            const float be = e < 4 ? b0[e] : b1[e - 4];
            y[e] = to_bf16(swish(from_bf16(gv[e])) * ((x[e] - mean) * rstd * we + be));
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, y), out,
                                               ((tile_pos + row) * DV + chunk * 8) * 2, 0, 0);
    }
}

// Waits until this wavefront's DMA writes of the tile used by the k-th chunk of
// the pass are complete. Chunk j issues the stores of chunk j-1's output, then
// the DMA of tile j+2, so the operations younger than tile k's DMA (issued by
// chunk k-2, or before the loop for k < 2) are tile k+1's DMA and, from k = 2
// on, the stores of chunk k-2.
template <int DK, int DV>
__device__ inline void wait_tile(int k) {
    using c = C64<DK, DV>;
    if (k < 2)
        wait_vm<c::DMA>();
    else
        wait_vm<c::DMA + c::ST>();
}

// One chunk of the pipeline, buffer set X, query buffer QX. prev_out is where
// the previous chunk's output goes (the head's output, or a zero-size range
// that drops it while a segment only advances its state); it is flushed from V
// buffer (X + 2) % 3 just before the DMA of tile k + 2 reuses that set.
//
// `full` says whether this chunk's outputs are computed (its queries were
// loaded); otherwise the chunk only advances the state. The running log-decay
// `total` (through the previous chunk) is advanced by this chunk's total;
// `next_full` receives the mode of tile k + 2, whose DMA this chunk issues:
// full when the caller asked for every output, or once the running log-decay
// through this chunk is below kSurvivalDropLog.
//
// GATED: the flush applies the output epilogue, with the gate rows of the
// flushed tile in the gate buffer (loaded one chunk earlier, right after that
// chunk's flush). The queries are double-buffered (QX = k % 2) to make room
// for it, so the DMA of tile k + 2's queries waits until every wavefront is
// done with tile k's scores. Per chunk each wavefront issues: QB keys of tile
// k + 2 (before the epilogue's vector work, so that they are in flight
// early), ST stores, VB gate loads, VB values and 1 log-gate load of tile
// k + 2 (into the rows this wavefront has just flushed), then QB queries of
// tile k + 2. The wait at the chunk start leaves the values, log-gates and
// queries of the previous chunk outstanding, so the gate of tile k - 1 and all
// of tile k have landed.
template <int DK, int DV, int X, int QX, bool GATED>
__device__ inline void chunk(const Lds<DK, DV>& L, const HeadRsrc& hr,
                             const __amdgpu_buffer_rsrc_t& gate_r,
                             const __amdgpu_buffer_rsrc_t& prev_out,
                             const __amdgpu_buffer_rsrc_t& no_q, int k, uint32_t pos, bool full,
                             bool all_full, float eps, float& total, bool& next_full,
                             Acc<DK, DV>& a) {
    using c = C64<DK, DV>;
    if constexpr (GATED)
        wait_vm<c::DMA - c::QB>();
    else
        wait_tile<DK, DV>(k);
    if (threadIdx.x < 64) tables_from_lds(L.ell[X], L.tab[X]);
    lds_barrier();
    const TileView tv{L.q[QX], L.k[X], L.v[X], L.tab[X], L.tab[X] + 64, L.tab[X] + 128};
    const float gc = tv.beta[kTile - 1];
    total += gc;
    next_full = all_full || total < kSurvivalDropLog;
    // The plain kernels issue the DMA of tile k + 2 in three parts spread
    // over the chunk (queries, keys, then values and log-gates, always in that
    // order), so that the eight wavefronts' memory instructions do not queue up
    // behind each other at the start of the chunk. The gated kernels' order is
    // given above.
    constexpr int Y = (X + 2) % 3;
    if constexpr (GATED) {
        dma_k<DK, DV, Y>(L, hr, pos + 2 * kTile);
        flush_tile_gated<DK, DV>(L.v[Y], L.gt, L.aff, prev_out, pos - kTile, eps);
        dma_gate<DK, DV>(L.gt, full ? gate_r : no_q, pos);
        dma_v_ell<DK, DV, Y>(L, hr, no_q, pos + 2 * kTile);
    } else {
        if (k > 0) flush_tile<DK, DV>(L.v[Y], prev_out, pos - kTile);
        dma_q<DK, DV, Y>(L, next_full ? hr.q : no_q, pos + 2 * kTile);
    }
    f32x4 o[c::CT][4];
    if (full) cross_term<DK, DV, GATED>(tv, a, o);
    if constexpr (!GATED) dma_k<DK, DV, Y>(L, hr, pos + 2 * kTile);
    if (full) scores_diag<DK, DV, GATED>(tv, L.ps);
    if constexpr (GATED) {
        if (full) lds_barrier();
        dma_q<DK, DV, QX>(L, next_full ? hr.q : no_q, pos + 2 * kTile);
        if (full) apply_scores<DK, DV, GATED>(L.ps, tv.vs, o);
    } else {
        dma_v_ell<DK, DV, Y>(L, hr, no_q, pos + 2 * kTile);
        if (full) {
            lds_barrier();
            apply_scores<DK, DV, GATED>(L.ps, tv.vs, o);
        }
    }
    scale_state<DK, DV>(a, __expf(gc));
    state_update<DK, DV, GATED>(tv, a);
    if (full) out_to_lds<DK, DV, GATED>(L.v[X], o);
}

// Calls f(integral_constant<int, J>) for J = I .. P-1 while it returns true.
template <int I, int P, class F>
__device__ inline bool unrolled_steps(F& f) {
    if constexpr (I == P) {
        return true;
    } else {
        if (!f(std::integral_constant<int, I>{})) return false;
        return unrolled_steps<I + 1, P>(f);
    }
}

// Runs chunks [cb, ce) of head x. With full_from_start the pass computes and
// writes every output; otherwise a chunk's outputs are computed and written
// only once the running log-decay before the previous chunk has dropped below
// kSurvivalDropLog (the mode of a tile is fixed when its DMA is issued, two
// chunks ahead; earlier chunks load no queries and only advance the state).
// Returns the total log-decay; *lead receives the number of output-free
// chunks. Reads past the head's end return zeros, so the loop has no tail
// case; the loop is unrolled by the period of the buffer indices (three sets,
// times two query buffers when GATED) so that every access's buffer is a
// compile-time fact.
// ALL_FULL compiles the pass that computes every output (the prefix launch)
// without the mode bookkeeping.
template <int DK, int DV, bool GATED, bool ALL_FULL = false>
__device__ float run_chunks(const Params& p, const Lds<DK, DV>& L, int64_t x, int64_t cb,
                           int64_t ce, bool full_from_start, Acc<DK, DV>& a, int64_t* lead) {
    float total = 0.0f;
    // offsets are taken from this pass's first row (chunk cb)
    const HeadRsrc hr = head_rsrc<DK, DV>(p, x, cb * kTile);
    // a zero-size range: stores through it are dropped, loads move no data
    const __amdgpu_buffer_rsrc_t drop = make_rsrc(p.out, 0);
    __amdgpu_buffer_rsrc_t gate_r = drop;
    const int nch = static_cast<int>(ce - cb);
    const bool all = ALL_FULL || full_from_start;
    uint32_t pos = 0;
    // earlier passes of this workgroup: drain their memory operations, and let
    // every wavefront finish reading the buffers
    wait_vm<0>();
    lds_barrier();
    if constexpr (GATED) {
        const int64_t left = p.N - cb * kTile;
        const int64_t rows = left < kRsrcRows<DK, DV> ? left : kRsrcRows<DK, DV>;
        gate_r = make_rsrc(p.gate + (x * p.N + cb * kTile) * DV,
                           static_cast<uint32_t>(rows * DV * 2));
        // the head's norm affine, read by every flush of the pass (after the
        // barrier of the first chunk)
        const int64_t h = x % p.H;
        for (int e = threadIdx.x; e < 2 * DV; e += C64<DK, DV>::NT)
            L.aff[e] = e < DV ? (p.gate_w ? p.gate_w[h * DV + e] : 1.0f)
                              : (p.gate_b ? p.gate_b[h * DV + e - DV] : 0.0f);
    }
    // modes of the tiles in buffer sets 0, 1, 2
    bool f[3] = {all, all, all};
    dma_tile<DK, DV, 0>(L, hr, all ? hr.q : drop, drop, pos);
    dma_tile<DK, DV, 1>(L, hr, all ? hr.q : drop, drop, pos + kTile);
    int first_full = all ? 0 : nch;  // first chunk whose outputs are written
    __amdgpu_buffer_rsrc_t prev = drop;  // destination of the staged output
    int last = 0;                        // buffer set holding it
    int k = 0;
    auto step = [&](auto J) -> bool {
        constexpr int j = decltype(J)::value;
        constexpr int X = j % 3;
        constexpr int QX = GATED ? j % 2 : X;
        if (k + j >= nch) return false;
        if (f[X] && first_full > k + j) first_full = k + j;
        chunk<DK, DV, X, QX, GATED>(L, hr, gate_r, prev, drop, k + j, pos + j * kTile, f[X], all,
                                    p.eps, total, f[(X + 2) % 3], a);
        prev = f[X] ? hr.out : drop;
        last = X;
        return true;
    };
    constexpr int kPeriod = GATED ? 6 : 3;
    for (;; k += kPeriod, pos += kPeriod * kTile)
        if (!unrolled_steps<0, kPeriod>(step)) break;
    *lead = first_full;
    // the last chunk's output: every wavefront's columns must be staged first
    // (and, GATED, this wavefront's gate rows must have landed)
    if constexpr (GATED) wait_vm<0>();
    lds_barrier();
    const uint32_t last_pos = static_cast<uint32_t>((ce - 1 - cb) * kTile);
    const bf16_t* last_v = last == 0 ? L.v[0] : last == 1 ? L.v[1] : L.v[2];
    if constexpr (GATED)
        flush_tile_gated<DK, DV>(last_v, L.gt, L.aff, prev, last_pos, p.eps);
    else
        flush_tile<DK, DV>(last_v, prev, last_pos);
    wait_vm<0>();  // no DMA into this workgroup's LDS may outlive the pass
    return total;
}

// LDS of the kernels: three buffer sets, each array its own object (the
// compiler orders LDS reads after pending LDS DMA per object). The gated
// kernels have two query buffers, the gate buffer and the norm affine.
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
    __shared__ __attribute__((aligned(16))) bf16_t ps_[kTile * C64<DK, DV>::PP];          \
    __shared__ __attribute__((aligned(16))) float sink_[kTile];                           \
    const Lds<DK, DV> L{{q0_, q1_, q2_}, {k0_, k1_, k2_}, {v0_, v1_, v2_},                \
                        {l0_, l1_, l2_}, {t0_, t1_, t2_}, ps_, sink_, nullptr, nullptr};

#define GRET_C64_LDS_GATED(DK, DV)                                                        \
    __shared__ __attribute__((aligned(16))) bf16_t q0_[kTile * DK], q1_[kTile * DK];      \
    __shared__ __attribute__((aligned(16))) bf16_t k0_[kTile * DK], k1_[kTile * DK],      \
        k2_[kTile * DK];                                                                  \
    __shared__ __attribute__((aligned(16))) bf16_t v0_[kTile * DV], v1_[kTile * DV],      \
        v2_[kTile * DV];                                                                  \
    __shared__ __attribute__((aligned(16))) float l0_[kTile], l1_[kTile], l2_[kTile];    \
    __shared__ __attribute__((aligned(16))) float t0_[3 * kTile], t1_[3 * kTile],        \
        t2_[3 * kTile];                                                                   \
    __shared__ __attribute__((aligned(16))) bf16_t ps_[kTile * C64<DK, DV>::PP];          \
    __shared__ __attribute__((aligned(16))) float sink_[kTile];                           \
    __shared__ __attribute__((aligned(16))) bf16_t g_[kTile * DV];                        \
    __shared__ __attribute__((aligned(16))) float aff_[2 * DV];                           \
    const Lds<DK, DV> L{{q0_, q1_, nullptr}, {k0_, k1_, k2_}, {v0_, v1_, v2_},            \
                        {l0_, l1_, l2_}, {t0_, t1_, t2_}, ps_, sink_, g_, aff_};

template <int DK, int DV, bool GATED>
__device__ inline void main_pass(const Params& p, const Lds<DK, DV>& L) {
    zero_upper_blocks<DK, DV>(L.ps);
    const SegPlan& pl = p.plan;
    // each XCD streams one contiguous range of the heads' chunk sequences
    const int64_t gidx = seg_of_block(pl.G, blockIdx.x);
    const int64_t hi = seg_lo(pl, gidx + 1);
    int64_t t = seg_lo(pl, gidx);
    Acc<DK, DV> a;
    while (t < hi) {
        const int64_t x = t / pl.nc;
        const int64_t cb = t - x * pl.nc;
        const int64_t ce = (hi - x * pl.nc) < pl.nc ? (hi - x * pl.nc) : pl.nc;
        const bool initial = cb == 0;
        const int64_t slot = initial ? 0 : gidx - seg_first_inner(pl, x) + 1;
        load_state<DK, DV>(a, initial && p.state_in ? p.state_in + x * DK * DV : nullptr);
        int64_t lead = 0;
        const float total = run_chunks<DK, DV, GATED>(p, L, x, cb, ce, initial, a, &lead);
        save_state<DK, DV>(a, p.ws_state + (x * pl.max_seg + slot) * (int64_t)(DK * DV));
        if (threadIdx.x == 0) p.ws_meta[x * pl.max_seg + slot] = make_float2(total, (float)lead);
        t = x * pl.nc + ce;
    }
}

template <int DK, int DV, bool GATED>
__device__ inline void prefix_pass(const Params& p, const Lds<DK, DV>& L) {
    const SegPlan& pl = p.plan;
    const int64_t gidx = blockIdx.x;
    const int64_t lo = seg_lo(pl, gidx);
    const int64_t x = lo / pl.nc;
    const int64_t cb = lo - x * pl.nc;
    if (cb == 0) return;  // this workgroup starts at a head boundary: nothing to redo
    const int64_t slot = gidx - seg_first_inner(pl, x) + 1;
    const int64_t lead = static_cast<int64_t>(p.ws_meta[x * pl.max_seg + slot].y);
    if (lead <= 0) return;
    zero_upper_blocks<DK, DV>(L.ps);
    Acc<DK, DV> a;
    load_state<DK, DV>(a, p.ws_state + (x * pl.max_seg + slot) * (int64_t)(DK * DV));
    int64_t unused = 0;
    run_chunks<DK, DV, GATED, true>(p, L, x, cb, cb + lead, true, a, &unused);
}

template <int DK, int DV, bool GATED>
__global__ __launch_bounds__(kThreadsFor<DV>) void prefill_main_c64_kernel(Params p) {
    if constexpr (GATED) {
        GRET_C64_LDS_GATED(DK, DV)
        main_pass<DK, DV, true>(p, L);
    } else {
        GRET_C64_LDS(DK, DV)
        main_pass<DK, DV, false>(p, L);
    }
}

template <int DK, int DV, bool GATED>
__global__ __launch_bounds__(kThreadsFor<DV>) void prefill_prefix_c64_kernel(Params p) {
    if constexpr (GATED) {
        GRET_C64_LDS_GATED(DK, DV)
        prefix_pass<DK, DV, true>(p, L);
    } else {
        GRET_C64_LDS(DK, DV)
        prefix_pass<DK, DV, false>(p, L);
    }
}
#undef GRET_C64_LDS_GATED
#undef GRET_C64_LDS

template <int DK, int DV, bool GATED>
hipError_t launch_g(const PrefillArgs& a, const SegPlan& plan) {
    const Params p = make_params(a, plan, DK, DV);
    hipLaunchKernelGGL((prefill_main_c64_kernel<DK, DV, GATED>), dim3(plan.G),
                       dim3(C64<DK, DV>::NT), 0, a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_combine<DK, DV>(p, a.stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_prefix_c64_kernel<DK, DV, GATED>), dim3(plan.G),
                       dim3(C64<DK, DV>::NT), 0, a.stream, p);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch(const PrefillArgs& a, const SegPlan& plan) {
    return a.epi.gate ? launch_g<DK, DV, true>(a, plan) : launch_g<DK, DV, false>(a, plan);
}

template <int DK, int DV>
int blocks_per_cu() {
    int n = 0;
    int ng = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, prefill_main_c64_kernel<DK, DV, false>, C64<DK, DV>::NT, 0);
    const hipError_t eg = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &ng, prefill_main_c64_kernel<DK, DV, true>, C64<DK, DV>::NT, 0);
    // the plan is shared by the plain and the gated kernels
    return e == hipSuccess && eg == hipSuccess ? (n < ng ? n : ng) : 0;
}

}  // namespace

hipError_t launch_prefill_bf16_c64(const PrefillArgs& a, const SegPlan& plan) {
    if (a.dk == 64 && a.dv == 64) return launch<64, 64>(a, plan);
    if (a.dk == 64 && a.dv == 128) return launch<64, 128>(a, plan);
    if (a.dk == 128 && a.dv == 64) return launch<128, 64>(a, plan);
    if (a.dk == 128 && a.dv == 128) return launch<128, 128>(a, plan);
    return hipErrorInvalidValue;
}

int prefill_bf16_c64_blocks_per_cu(int64_t dk, int64_t dv) {
    if (dk == 64 && dv == 64) return blocks_per_cu<64, 64>();
    if (dk == 64 && dv == 128) return blocks_per_cu<64, 128>();
    if (dk == 128 && dv == 64) return blocks_per_cu<128, 64>();
    if (dk == 128 && dv == 128) return blocks_per_cu<128, 128>();
    return 0;
}

}  // namespace gret
