// gret_prefill_bf16.hip -- chunkwise gated-retention prefill in chunks of 128
// or 256 positions on gfx950 matrix cores (bf16 operands, fp32 accumulation,
// fp32 state carry), and the dispatch of every bf16 prefill (chunks of 64 run
// the pipelined kernel of gret_prefill_c64.hip).
//
// Method (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次",
// sections "路线二：Multi-Head Gated Retention" and "Prefill 与 Decode 为什么使用
// 两种计算形态"): inside a chunk of C positions starting at a, with beta_j the
// chunk-local inclusive sum of log-gates,
//   out[a+j] = exp(beta_j) q_{a+j} S + sum_{l<=j} exp(beta_j - beta_l) (q_{a+j}.k_{a+l}) v_{a+l}
//   S       <- exp(beta_last) S + sum_l exp(beta_last - beta_l) k_{a+l}^T v_{a+l}
// The page ties a chunk of 256 to its original kernel; here larger chunks are
// supported for that reason and measured slower than chunks of 64.
//
// A chunk is processed as R = C/64 tiles of 64 positions. Tile r contracts
// against its own keys (causal diagonal) and, for every earlier tile t of the
// chunk, against that tile's keys, which are re-read into a second LDS buffer;
// the state increment of the chunk is accumulated tile by tile and applied at
// the chunk end. The segment schedule (main, combine, prefix launches) is the
// one of the chunk-64 path.
//
// Workgroup layout: DV/16 wavefronts; wave w owns value columns [16w, 16w+16)
// of the state (fp32 accumulator registers) and of the output. Tiles go
// global -> registers (range-checked buffer loads, prefetched one tile ahead)
// -> LDS (row-major, XOR-swizzled 16-byte chunks); operands contracted over
// positions are read with the transposing LDS load ds_read_b64_tr_b16.
#include <hip/hip_runtime.h>

#include "gret_prefill_common.h"

namespace gret {
namespace {

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

template <int DK, int DV, int R>
struct __attribute__((aligned(16))) Smem {
    using c = Cfg<DK, DV, R>;
    TileBuf<DK, DV, R> buf;
    bf16_t ps[kTile * c::PP];
    bf16_t ks2[kTile * DK];  // an earlier tile of the chunk, restaged
    bf16_t vs2[kTile * DV];
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


// Per-thread state of one segment's pass.
template <int DK, int DV, int R>
struct Acc {
    using c = Cfg<DK, DV, R>;
    f32x4 s[c::TK];                    // S[16tk + 4g + i][16w + li]
    f32x4 ds[R > 1 ? c::TK : 1];       // chunk increment (chunks > 64)
};

// Stages K and V of an earlier tile of the current chunk into the second buffer.
template <int DK, int DV, int R>
__device__ inline void restage(const HeadRsrc& hr, uint32_t pos, Smem<DK, DV, R>& sm) {
    TileRegs<DK, DV, R> t;
    load_tile<DK, DV, R, false>(hr, pos, pos, t);
    write_tile<DK, DV, R, false>(t, nullptr, sm.ks2, sm.vs2);
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




// Runs chunks [cb, ce) of head x. With full_from_start the pass computes
// outputs from the first chunk; otherwise only the state until the running
// log-decay drops below kSurvivalDropLog (then outputs too). Returns the total
// log-decay; *lead receives the number of state-only chunks.
template <int DK, int DV, int R>
__device__ float run_chunks(const Params& p, Smem<DK, DV, R>& sm, int64_t x, int64_t cb,
                            int64_t ce, bool full_from_start, Acc<DK, DV, R>& a, int64_t* lead) {
    {
        using c = Cfg<DK, DV, R>;
        bool full = full_from_start;
        float total = 0.0f;
        *lead = full ? 0 : (ce - cb);
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk) a.ds[tk] = f32x4{0.f, 0.f, 0.f, 0.f};
        // offsets are taken from this pass's first row (chunk cb)
        const HeadRsrc hr = head_rsrc<DK, DV>(p, x, cb * c::C);
        TileRegs<DK, DV, R> tr;
        load_tile<DK, DV, R>(hr, 0, 0, tr);
        for (int64_t ch = cb; ch < ce; ++ch) {
            const int64_t cpos = (ch - cb) * c::C;
            const int64_t nvalid = p.N - ch * c::C < c::C ? p.N - ch * c::C : c::C;
            const int rv = static_cast<int>((nvalid + kTile - 1) / kTile);
            for (int r = 0; r < rv; ++r) {
                const uint32_t tpos = static_cast<uint32_t>(cpos + kTile * r);
                TileBuf<DK, DV, R>& tb = sm.buf;
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
                        restage<DK, DV, R>(hr, static_cast<uint32_t>(cpos + kTile * t), sm);
                        __syncthreads();
                        scores_full<DK, DV, R>(tb, sm.ps, sm.ks2, r, t);
                        __syncthreads();
                        apply_scores<DK, DV, R>(sm.ps, sm.vs2, false, o);
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
    __shared__ Smem<DK, DV, R> sm;
    const SegPlan& pl = p.plan;
    // each XCD streams one contiguous range of the heads' chunk sequences
    const int64_t gidx = seg_of_block(pl.G, blockIdx.x);
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
        const float total = run_chunks<DK, DV, R>(p, sm, x, cb, ce, initial, a, &lead);
        float* dst = p.ws_state + (x * pl.max_seg + slot) * (int64_t)(DK * DV);
        save_state<DK, DV, R>(a, dst);
        if (threadIdx.x == 0) p.ws_meta[x * pl.max_seg + slot] = make_float2(total, (float)lead);
        t = x * pl.nc + ce;
    }
}

template <int DK, int DV, int R>
__global__ __launch_bounds__(kThreadsFor<DV>) void prefill_prefix_kernel(Params p) {
    __shared__ Smem<DK, DV, R> sm;
    const SegPlan& pl = p.plan;
    const int64_t gidx = blockIdx.x;
    const int64_t lo = seg_lo(pl, gidx);
    const int64_t x = lo / pl.nc;
    const int64_t cb = lo - x * pl.nc;
    if (cb == 0) return;  // this workgroup starts at a head boundary: nothing to redo
    const int64_t slot = gidx - seg_first_inner(pl, x) + 1;
    const int64_t lead = static_cast<int64_t>(p.ws_meta[x * pl.max_seg + slot].y);
    if (lead <= 0) return;
    Acc<DK, DV, R> a;
    load_state<DK, DV, R>(a, p.ws_state + (x * pl.max_seg + slot) * (int64_t)(DK * DV));
    int64_t unused = 0;
    run_chunks<DK, DV, R>(p, sm, x, cb, cb + lead, true, a, &unused);
}

template <int DK, int DV, int R>
hipError_t launch_rc(const PrefillArgs& a, const SegPlan& plan) {
    const Params p = make_params(a, plan, DK, DV);
    const dim3 block(Cfg<DK, DV, R>::NT);
    hipLaunchKernelGGL((prefill_main_kernel<DK, DV, R>), dim3(plan.G), block, 0, a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_combine<DK, DV>(p, a.stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_prefix_kernel<DK, DV, R>), dim3(plan.G), block, 0, a.stream, p);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const PrefillArgs& a, const SegPlan& plan) {
    switch (a.chunk) {
        case 128: return launch_rc<DK, DV, 2>(a, plan);
        case 256: return launch_rc<DK, DV, 4>(a, plan);
        default: return hipErrorInvalidValue;
    }
}

template <int DK, int DV, int R>
int blocks_per_cu_rc() {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, prefill_main_kernel<DK, DV, R>, Cfg<DK, DV, R>::NT, 0);
    return e == hipSuccess ? n : 0;
}

template <int DK, int DV>
int blocks_per_cu_dims(int64_t chunk) {
    switch (chunk) {
        case 128: return blocks_per_cu_rc<DK, DV, 2>();
        case 256: return blocks_per_cu_rc<DK, DV, 4>();
        default: return 0;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, const SegPlan& plan) {
    if (a.chunk == 64) return launch_prefill_bf16_c64(a, plan);
    if (a.dk == 64 && a.dv == 64) return launch_dims<64, 64>(a, plan);
    if (a.dk == 64 && a.dv == 128) return launch_dims<64, 128>(a, plan);
    if (a.dk == 128 && a.dv == 64) return launch_dims<128, 64>(a, plan);
    if (a.dk == 128 && a.dv == 128) return launch_dims<128, 128>(a, plan);
    return hipErrorInvalidValue;
}

int prefill_bf16_blocks_per_cu(int64_t dk, int64_t dv, int64_t chunk) {
    if (chunk == 64) return prefill_bf16_c64_blocks_per_cu(dk, dv);
    if (dk == 64 && dv == 64) return blocks_per_cu_dims<64, 64>(chunk);
    if (dk == 64 && dv == 128) return blocks_per_cu_dims<64, 128>(chunk);
    if (dk == 128 && dv == 64) return blocks_per_cu_dims<128, 64>(chunk);
    if (dk == 128 && dv == 128) return blocks_per_cu_dims<128, 128>(chunk);
    return 0;
}

}  // namespace gret
