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
//               computes outputs too. Log-gates are <= 0, so the running sum
//               only decreases and every later output has a smaller factor.
//   2. combine: per head, chain the segment maps in order, leaving each
//               segment's incoming state in its workspace slot; the last one
//               is the final state.
//   3. prefix:  every non-first segment recomputes its leading chunks, now
//               from its incoming state, and writes their outputs.
// Each output is written exactly once and inputs are read about once (the
// leading chunks twice).
//
// Per-workgroup data flow (256 threads = 4 wavefronts, wave w owns value
// columns [w*DV/4, (w+1)*DV/4)), per 64-position tile of a chunk:
//   global -> registers (prefetched one tile ahead) -> LDS: Q and K row-major,
//   K and V transposed (dim-major) so the position index is contiguous, which
//   is what the matrix-core operand layout needs for contractions over
//   positions. The state S stays in registers as fp32 accumulator tiles;
//   wave w holds S[:, its columns].
//   * scores   P^T = K Q^T for the wave's 16 query rows (16x16x32 bf16 MFMA),
//              decay mask exp(beta_j - beta_l) in fp32, cast to bf16 into LDS;
//   * output   O^T = S^T Q^T (S taken straight from the accumulator registers)
//              scaled by exp(beta_j), plus V^T P~^T, so each lane ends with 4
//              consecutive output columns of one row and stores 8 bytes;
//   * state    S = exp(g) S + K^T (Gamma V) with Gamma_l = exp(g - beta_l).
#include <hip/hip_runtime.h>

#include "gret_device.h"
#include "gret_internal.h"

namespace gret {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;    // positions per tile
constexpr int kPadQ = 8;     // bf16 padding per row of row-major tiles (16 bytes)
constexpr int kPadT = 8;     // bf16 padding per row of transposed tiles

__device__ inline f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 lds_read8(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ inline bf16x4 lds_read4(const bf16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }

__device__ inline bf16x8 cat44(const bf16x4& a, const bf16x4& b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

struct Params {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const float* log_gamma;
    const float* state_in;
    bf16_t* out;
    float* state_out;
    float* ws_state;   // [BH][max_seg][DK*DV]
    float2* ws_meta;   // [BH][max_seg]: (total log-decay, leading chunks)
    SegPlan plan;
    int64_t N;
};

template <int DK, int DV, int R>
struct Cfg {
    static constexpr int C = kTile * R;
    static constexpr int CW = DV / 4;       // value columns per wave
    static constexpr int TC = CW / 16;      // 16-wide column tiles per wave
    static constexpr int TK = DK / 16;      // 16-row key tiles of the state
    static constexpr int KS = DK / 32;      // k-steps over dk
    static constexpr int QP = DK + kPadQ;   // row pitch (elements) of Qs / Ks
    static constexpr int TP = kTile + kPadT;  // row pitch of Kts / Vts / Ps
    static constexpr int KBLK = 16 * (DK / 8);  // 4x8 staging blocks per K tile
    static constexpr int VBLK = 16 * (DV / 8);
    static constexpr int QLD = kTile * DK / 8 / kThreads;  // 16-byte Q loads per thread
    static_assert(TC >= 1 && TK >= 1 && KS >= 1, "tile shape");
    static_assert(KBLK <= kThreads && VBLK <= kThreads, "one staging block per thread");
    static_assert(QLD >= 1 && QLD * kThreads * 8 == kTile * DK, "Q staging");
};

template <int DK, int DV, int R>
struct __attribute__((aligned(16))) Smem {
    using c = Cfg<DK, DV, R>;
    bf16_t qs[kTile * c::QP];
    bf16_t ks[kTile * c::QP];
    bf16_t kts[DK * c::TP];
    bf16_t vts[DV * c::TP];
    bf16_t ps[kTile * c::TP];
    float beta[c::C];
};

template <int DK, int DV>
struct __attribute__((aligned(16))) Smem2 {  // earlier tiles of the chunk (chunks > 64)
    bf16_t ks[kTile * (DK + kPadQ)];
    bf16_t vts[DV * (kTile + kPadT)];
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
    bf16x8 k[4];
    bf16x8 v[4];
    float ell[R];  // wave 0: log-gates of the chunk (lane holds R consecutive)
};

// Loads tile `tile_pos` (first position of the tile, < N) of head x; Q only
// when WITH_Q, the chunk's log-gates only when chunk_start.
template <int DK, int DV, int R, bool WITH_Q = true>
__device__ inline void load_tile(const Params& p, int64_t x, int64_t tile_pos, bool chunk_start,
                                 int64_t chunk_pos, TileRegs<DK, DV, R>& t) {
    using c = Cfg<DK, DV, R>;
    const int tid = threadIdx.x;
    const int64_t N = p.N;
    const bf16x8 zero = {};
    // Q: row-major, thread covers rows tid/(DK/8) + i*(256/(DK/8)), one 16-byte piece
    if (WITH_Q) {
        constexpr int PER_ROW = DK / 8;
        constexpr int ROWS_PER_PASS = kThreads / PER_ROW;
        const int col = (tid % PER_ROW) * 8;
#pragma unroll
        for (int i = 0; i < c::QLD; ++i) {
            const int row = tid / PER_ROW + i * ROWS_PER_PASS;
            const int64_t pos = tile_pos + row;
            t.q[i] = pos < N ? *reinterpret_cast<const bf16x8*>(p.q + (x * N + pos) * DK + col)
                             : zero;
        }
    }
    // K: 4 positions x 8 dims per thread (position quad fastest across lanes)
    if (tid < c::KBLK) {
        const int pq = tid % 16, c8 = tid / 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t pos = tile_pos + 4 * pq + i;
            t.k[i] = pos < N ? *reinterpret_cast<const bf16x8*>(p.k + (x * N + pos) * DK + 8 * c8)
                             : zero;
        }
    }
    if (tid < c::VBLK) {
        const int pq = tid % 16, c8 = tid / 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t pos = tile_pos + 4 * pq + i;
            t.v[i] = pos < N ? *reinterpret_cast<const bf16x8*>(p.v + (x * N + pos) * DV + 8 * c8)
                             : zero;
        }
    }
    if (chunk_start && tid < 64) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t pos = chunk_pos + tid * R + i;
            // positions past the end decay nothing (gate 1) and carry zero K, V
            t.ell[i] = pos < N ? clamp_log_gamma(p.log_gamma[x * N + pos], kLogGammaFloor) : 0.0f;
        }
    }
}

template <int DK, int DV, int R>
__device__ inline void write_kv(const TileRegs<DK, DV, R>& t, bf16_t* ks, bf16_t* kts,
                                bf16_t* vts) {
    using c = Cfg<DK, DV, R>;
    const int tid = threadIdx.x;
    if (tid < c::KBLK) {
        const int pq = tid % 16, c8 = tid / 16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<bf16x8*>(ks + (4 * pq + i) * c::QP + 8 * c8) = t.k[i];
        if (kts) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x4 col = {t.k[0][e], t.k[1][e], t.k[2][e], t.k[3][e]};
                *reinterpret_cast<bf16x4*>(kts + (8 * c8 + e) * c::TP + 4 * pq) = col;
            }
        }
    }
    if (tid < c::VBLK) {
        const int pq = tid % 16, c8 = tid / 16;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 col = {t.v[0][e], t.v[1][e], t.v[2][e], t.v[3][e]};
            *reinterpret_cast<bf16x4*>(vts + (8 * c8 + e) * c::TP + 4 * pq) = col;
        }
    }
}

template <int DK, int DV, int R>
__device__ inline void write_q(const TileRegs<DK, DV, R>& t, bf16_t* qs) {
    using c = Cfg<DK, DV, R>;
    constexpr int PER_ROW = DK / 8;
    constexpr int ROWS_PER_PASS = kThreads / PER_ROW;
    const int tid = threadIdx.x;
    const int col = (tid % PER_ROW) * 8;
#pragma unroll
    for (int i = 0; i < c::QLD; ++i) {
        const int row = tid / PER_ROW + i * ROWS_PER_PASS;
        *reinterpret_cast<bf16x8*>(qs + row * c::QP + col) = t.q[i];
    }
}

// Wave 0: chunk-local inclusive prefix sum of the log-gates into beta[C].
template <int DK, int DV, int R>
__device__ inline void scan_beta(const TileRegs<DK, DV, R>& t, float* beta) {
    const int tid = threadIdx.x;
    if (tid >= 64) return;
    float loc[R];
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        run += t.ell[i];
        loc[i] = run;
    }
    // inclusive scan of lane totals across the wavefront
    float tot = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(tot, off);
        if (tid >= off) tot += o;
    }
    const float excl = tot - run;
#pragma unroll
    for (int i = 0; i < R; ++i) beta[tid * R + i] = excl + loc[i];
}

// Per-thread state of one segment's pass.
template <int DK, int DV, int R>
struct Acc {
    using c = Cfg<DK, DV, R>;
    f32x4 s[c::TK][c::TC];   // S[16tk + 4g + i][wave cols 16tc + li]
    f32x4 ds[R > 1 ? c::TK : 1][R > 1 ? c::TC : 1];  // chunk increment (chunks > 64)
};

// Stages K (row-major) and V (transposed) of an earlier tile of the current
// chunk (positions pos..pos+63) into s2; its transposed K is never needed.
template <int DK, int DV, int R>
__device__ inline void restage(const Params& p, int64_t x, int64_t pos, Smem2<DK, DV>& s2) {
    TileRegs<DK, DV, R> t;
    load_tile<DK, DV, R, false>(p, x, pos, false, 0, t);
    write_kv<DK, DV, R>(t, s2.ks, nullptr, s2.vts);
}

// Scores for the wave's 16 query rows (j-block w) against key tile `kt` (K
// row-major in `ksrc`), decayed and written as bf16 to sm.ps[j][l].
template <int DK, int DV, int R>
__device__ inline void scores_to_lds(Smem<DK, DV, R>& sm, const bf16_t* ksrc, int r, int t,
                                     bool diag) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int jrow = 16 * w + li;                 // row within the tile
    const float bj = sm.beta[kTile * r + jrow];
    bf16x8 qf[c::KS];
#pragma unroll
    for (int ks = 0; ks < c::KS; ++ks) qf[ks] = lds_read8(sm.qs + jrow * c::QP + 32 * ks + 8 * g);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        bf16x4 pk;
        if (!diag || b <= w) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < c::KS; ++ks) {
                const bf16x8 kf = lds_read8(ksrc + (16 * b + li) * c::QP + 32 * ks + 8 * g);
                acc = mfma16(kf, qf[ks], acc);
            }
            // acc[i] = P^T[l = 16b + 4g + i][j = jrow]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int l = 16 * b + 4 * g + i;
                float val = 0.0f;
                if (!diag || l <= jrow) val = acc[i] * __expf(bj - sm.beta[kTile * t + l]);
                pk[i] = to_bf16(val);
            }
        } else {
            pk = bf16x4{};
        }
        *reinterpret_cast<bf16x4*>(sm.ps + jrow * c::TP + 16 * b + 4 * g) = pk;
    }
}

// O^T[cols][rows] += V_t^T P~^T over the positions of tile t.
template <int DK, int DV, int R>
__device__ inline void apply_scores(Smem<DK, DV, R>& sm, const bf16_t* vtsrc, bool diag,
                                    f32x4 (&o)[4][Cfg<DK, DV, R>::TC]) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        bf16x8 vf[c::TC];
#pragma unroll
        for (int tc = 0; tc < c::TC; ++tc)
            vf[tc] = lds_read8(vtsrc + (c::CW * w + 16 * tc + li) * c::TP + 32 * ks + 8 * g);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (diag && 2 * ks > jt) continue;  // whole 32-position step is above the diagonal
            const bf16x8 pf = lds_read8(sm.ps + (16 * jt + li) * c::TP + 32 * ks + 8 * g);
#pragma unroll
            for (int tc = 0; tc < c::TC; ++tc) o[jt][tc] = mfma16(vf[tc], pf, o[jt][tc]);
        }
    }
}

template <int DK, int DV, int R>
__device__ inline void store_out(const Params& p, int64_t x, int64_t tile_pos,
                                 f32x4 (&o)[4][Cfg<DK, DV, R>::TC]) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const int64_t pos = tile_pos + 16 * jt + li;
        if (pos >= p.N) continue;
#pragma unroll
        for (int tc = 0; tc < c::TC; ++tc) {
            bf16x4 pk = {to_bf16(o[jt][tc][0]), to_bf16(o[jt][tc][1]), to_bf16(o[jt][tc][2]),
                         to_bf16(o[jt][tc][3])};
            *reinterpret_cast<bf16x4*>(p.out + (x * p.N + pos) * DV + c::CW * w + 16 * tc + 4 * g) =
                pk;
        }
    }
}

// S (or dS) += K_t^T (Gamma V_t) for the current tile; Gamma_l = exp(gc - beta_l).
template <int DK, int DV, int R>
__device__ inline void state_update(Smem<DK, DV, R>& sm, int r, float gc,
                                    f32x4 (&acc)[Cfg<DK, DV, R>::TK][Cfg<DK, DV, R>::TC]) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        float gam[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) gam[e] = __expf(gc - sm.beta[kTile * r + 32 * ks + 8 * g + e]);
        bf16x8 bf[c::TC];
#pragma unroll
        for (int tc = 0; tc < c::TC; ++tc) {
            const bf16x8 vf = lds_read8(sm.vts + (c::CW * w + 16 * tc + li) * c::TP + 32 * ks + 8 * g);
#pragma unroll
            for (int e = 0; e < 8; ++e) bf[tc][e] = to_bf16(from_bf16(vf[e]) * gam[e]);
        }
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk) {
            const bf16x8 kf = lds_read8(sm.kts + (16 * tk + li) * c::TP + 32 * ks + 8 * g);
#pragma unroll
            for (int tc = 0; tc < c::TC; ++tc) acc[tk][tc] = mfma16(kf, bf[tc], acc[tk][tc]);
        }
    }
}

// Runs chunks [cb, ce) of head x. With full_from_start the pass computes
// outputs from the first chunk; otherwise only the state until the running
// log-decay drops below kSurvivalDropLog (then outputs too). Returns the total
// log-decay; *lead receives the number of state-only chunks.
template <int DK, int DV, int R>
__device__ float run_chunks(const Params& p, Smem<DK, DV, R>& sm, Smem2<DK, DV>* s2, int64_t x,
                            int64_t cb, int64_t ce, bool full_from_start, Acc<DK, DV, R>& a,
                            int64_t* lead) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    (void)w;
    bool full = full_from_start;
    float total = 0.0f;
    *lead = full ? 0 : (ce - cb);
    if constexpr (R > 1) {
#pragma unroll
        for (int tk = 0; tk < c::TK; ++tk)
#pragma unroll
            for (int tc = 0; tc < c::TC; ++tc) a.ds[tk][tc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    TileRegs<DK, DV, R> tr;
    load_tile<DK, DV, R>(p, x, cb * c::C, true, cb * c::C, tr);

    for (int64_t ch = cb; ch < ce; ++ch) {
        const int64_t cpos = ch * c::C;
        const int64_t nvalid = p.N - cpos < c::C ? p.N - cpos : c::C;
        const int rv = static_cast<int>((nvalid + kTile - 1) / kTile);
        for (int r = 0; r < rv; ++r) {
            const int64_t tpos = cpos + kTile * r;
            if (r == 0) scan_beta<DK, DV, R>(tr, sm.beta);
            write_q<DK, DV, R>(tr, sm.qs);
            write_kv<DK, DV, R>(tr, sm.ks, sm.kts, sm.vts);
            __syncthreads();
            const float gc = sm.beta[c::C - 1];

            // prefetch the next tile of this pass
            if (r + 1 < rv) {
                load_tile<DK, DV, R>(p, x, tpos + kTile, false, 0, tr);
            } else if (ch + 1 < ce) {
                load_tile<DK, DV, R>(p, x, cpos + c::C, true, cpos + c::C, tr);
            }

            if (full) {
                f32x4 o[4][c::TC];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int tc = 0; tc < c::TC; ++tc) o[jt][tc] = f32x4{0.f, 0.f, 0.f, 0.f};
                // cross-chunk term O^T = S^T Q^T. The state tile pair (2m, 2m+1)
                // gives each lane dk = 32m + {4g..4g+3, 16+4g..16+4g+3}; the Q
                // operand is read with the same permutation of dk.
#pragma unroll
                for (int m = 0; m < c::KS; ++m) {
                    bf16x8 qf[4];
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) {
                        const bf16_t* qrow = sm.qs + (16 * jt + li) * c::QP + 32 * m + 4 * g;
                        qf[jt] = cat44(lds_read4(qrow), lds_read4(qrow + 16));
                    }
#pragma unroll
                    for (int tc = 0; tc < c::TC; ++tc) {
                        const f32x4 lo4 = a.s[2 * m][tc], hi4 = a.s[2 * m + 1][tc];
                        const bf16x8 sf = {to_bf16(lo4[0]), to_bf16(lo4[1]), to_bf16(lo4[2]),
                                           to_bf16(lo4[3]), to_bf16(hi4[0]), to_bf16(hi4[1]),
                                           to_bf16(hi4[2]), to_bf16(hi4[3])};
#pragma unroll
                        for (int jt = 0; jt < 4; ++jt) o[jt][tc] = mfma16(sf, qf[jt], o[jt][tc]);
                    }
                }
                // scale output row j by exp(beta_j)
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    const float f = __expf(sm.beta[kTile * r + 16 * jt + li]);
#pragma unroll
                    for (int tc = 0; tc < c::TC; ++tc) {
                        o[jt][tc][0] *= f;
                        o[jt][tc][1] *= f;
                        o[jt][tc][2] *= f;
                        o[jt][tc][3] *= f;
                    }
                }
                // intra-chunk terms: earlier tiles of this chunk, then the diagonal tile
                if constexpr (R > 1) {
                    for (int t = 0; t < r; ++t) {
                        restage<DK, DV, R>(p, x, cpos + kTile * t, *s2);
                        __syncthreads();
                        scores_to_lds<DK, DV, R>(sm, s2->ks, r, t, false);
                        __syncthreads();
                        apply_scores<DK, DV, R>(sm, s2->vts, false, o);
                        __syncthreads();
                    }
                }
                scores_to_lds<DK, DV, R>(sm, sm.ks, r, r, true);
                __syncthreads();
                apply_scores<DK, DV, R>(sm, sm.vts, true, o);
                store_out<DK, DV, R>(p, x, tpos, o);
            }

            // state carry
            if constexpr (R == 1) {
                const float eg = __expf(gc);
#pragma unroll
                for (int tk = 0; tk < c::TK; ++tk)
#pragma unroll
                    for (int tc = 0; tc < c::TC; ++tc) {
                        a.s[tk][tc][0] *= eg;
                        a.s[tk][tc][1] *= eg;
                        a.s[tk][tc][2] *= eg;
                        a.s[tk][tc][3] *= eg;
                    }
                state_update<DK, DV, R>(sm, r, gc, a.s);
            } else {
                state_update<DK, DV, R>(sm, r, gc, a.ds);
                if (r == rv - 1) {
                    const float eg = __expf(gc);
#pragma unroll
                    for (int tk = 0; tk < c::TK; ++tk)
#pragma unroll
                        for (int tc = 0; tc < c::TC; ++tc) {
                            f32x4& sv = a.s[tk][tc];
                            f32x4& dv = a.ds[tk][tc];
                            sv[0] = fmaf(eg, sv[0], dv[0]);
                            sv[1] = fmaf(eg, sv[1], dv[1]);
                            sv[2] = fmaf(eg, sv[2], dv[2]);
                            sv[3] = fmaf(eg, sv[3], dv[3]);
                            dv = f32x4{0.f, 0.f, 0.f, 0.f};
                        }
                }
            }
            if (r == rv - 1) {
                total += gc;
                if (!full && total < kSurvivalDropLog) {
                    full = true;
                    *lead = ch + 1 - cb;
                }
            }
            __syncthreads();  // LDS tiles are rewritten next iteration
        }
    }
    (void)li;
    (void)g;
    return total;
}

template <int DK, int DV, int R>
__device__ inline void load_state(Acc<DK, DV, R>& a, const float* src) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tk = 0; tk < c::TK; ++tk)
#pragma unroll
        for (int tc = 0; tc < c::TC; ++tc)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.s[tk][tc][i] = src ? src[(16 * tk + 4 * g + i) * DV + c::CW * w + 16 * tc + li] : 0.0f;
}

template <int DK, int DV, int R>
__device__ inline void save_state(const Acc<DK, DV, R>& a, float* dst) {
    using c = Cfg<DK, DV, R>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tk = 0; tk < c::TK; ++tk)
#pragma unroll
        for (int tc = 0; tc < c::TC; ++tc)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[(16 * tk + 4 * g + i) * DV + c::CW * w + 16 * tc + li] = a.s[tk][tc][i];
}

// One workgroup per CU: the state tiles, the prefetched tile and the
// operand fragments need more than the 256 registers a lane gets at two.
template <int DK, int DV, int R>
__global__ __launch_bounds__(kThreads, 1) void prefill_main_kernel(Params p) {
    __shared__ SmemAll<DK, DV, R> all;
    Smem<DK, DV, R>& sm = all.m;
    Smem2<DK, DV>* s2 = all.extra();
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
__global__ __launch_bounds__(kThreads, 1) void prefill_prefix_kernel(Params p) {
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
    Acc<DK, DV, R> a;
    load_state<DK, DV, R>(a, p.ws_state + (x * pl.max_seg + slot) * (int64_t)(DK * DV));
    int64_t unused = 0;
    run_chunks<DK, DV, R>(p, sm, s2, x, cb, cb + lead, true, a, &unused);
}

// Chains the segment maps of each head: S_in(s) = S_end(s-1),
// S_end(s) = exp(G_s) S_in(s) + S_loc(s). Leaves S_in(s) in slot s and writes
// the final state.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void prefill_combine_kernel(Params p) {
    const SegPlan& pl = p.plan;
    constexpr int PER_BLOCK = kThreads * 4;
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
    const dim3 block(kThreads);
    hipLaunchKernelGGL((prefill_main_kernel<DK, DV, R>), dim3(plan.G), block, 0, a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int per_head = DK * DV / (kThreads * 4);
    hipLaunchKernelGGL((prefill_combine_kernel<DK, DV>), dim3(plan.BH * per_head), block, 0,
                       a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_main_kernel<DK, DV, R>, kThreads,
                                                      0) != hipSuccess)
        return 0;
    return n;
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
