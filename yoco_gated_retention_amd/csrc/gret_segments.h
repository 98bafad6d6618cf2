// gret_segments.h -- how a prefill is cut into segments that run concurrently.
//
// The chunkwise form (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache
// 只存一次", section "Prefill 与 Decode 为什么使用两种计算形态") leaves one serial
// dependence: the state carried from chunk to chunk. Carrying a state is an
// affine map, S -> exp(G) S + S_loc, so a head's chunk sequence can be split
// into segments that each run from a zero state, whose maps are then chained
// (the same re-association one level up). This header holds the bookkeeping,
// shared by host planning and device code; it contains no arithmetic of the
// method itself.
//
// Flatten all (head, chunk) pairs into t = head * nc + chunk, t in [0, T),
// T = BH * nc. Workgroup g of G owns [lo(g), lo(g+1)) with lo(g) = floor(g*T/G)
// (G <= T, so every range is non-empty). A range that crosses a head boundary
// is processed as two or more pieces. Every piece is a segment. A segment that
// starts at chunk 0 of its head is "head-initial" (slot 0): it starts from the
// caller's initial state. Any other segment starts at lo(g) strictly inside
// head x; it gets slot s = g - first_inner(x) + 1, where first_inner(x) is the
// smallest g with lo(g) > x * nc.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define GRET_HD __host__ __device__ inline
#else
#define GRET_HD inline
#endif

namespace gret {

struct SegPlan {
    int64_t BH;       // number of (batch, head) pairs
    int64_t nc;       // chunks per head = ceil(N / chunk)
    int64_t T;        // BH * nc
    int64_t G;        // workgroups (1 <= G <= T)
    int64_t max_seg;  // slots per head
};

// Hard cap on workgroups per prefill: bounds the workspace independently of
// the device it runs on.
constexpr int64_t kMaxPrefillGroups = 1024;

GRET_HD int64_t seg_lo(const SegPlan& p, int64_t g) { return (g * p.T) / p.G; }

// Smallest g with lo(g) >= t  (t in [0, T]).
GRET_HD int64_t seg_first_g_at_or_after(const SegPlan& p, int64_t t) {
    return (t * p.G + p.T - 1) / p.T;
}

// Smallest g with lo(g) > x * nc.
GRET_HD int64_t seg_first_inner(const SegPlan& p, int64_t x) {
    return seg_first_g_at_or_after(p, x * p.nc + 1);
}

// Number of segments of head x (head-initial one included).
GRET_HD int64_t seg_count(const SegPlan& p, int64_t x) {
    const int64_t a = seg_first_inner(p, x);
    const int64_t b = seg_first_g_at_or_after(p, (x + 1) * p.nc);
    return 1 + (b > a ? b - a : 0);
}

// Longest piece, in chunks: a workgroup's range has at most ceil(T / G)
// chunks, and a piece is that range cut at head boundaries (at most nc).
// A prefill pass (a segment, or the recomputed leading chunks of one) spans
// at most this many chunks.
GRET_HD int64_t seg_max_piece_chunks(const SegPlan& p) {
    const int64_t r = (p.T + p.G - 1) / p.G;
    return r < p.nc ? r : p.nc;
}

// Segment of the workgroup with launch index b. The hardware hands workgroup
// ids to the chip's XCDs round-robin (id mod kXcds), and each XCD has its own
// L2 and address-translation caches. So that XCD x works on one contiguous
// range of the (head, chunk) order, the ids that land on XCD x take segments
// start(x), start(x) + 1, ... in launch order. A bijection of [0, G) for any
// G: the ids with b mod kXcds == x number per + (x < rem), per = G / kXcds,
// rem = G mod kXcds, and XCD x's range starts at x * per + min(x, rem).
constexpr int64_t kXcds = 8;

GRET_HD int64_t seg_of_block(int64_t G, int64_t b) {
    const int64_t x = b % kXcds, local = b / kXcds;
    const int64_t per = G / kXcds, rem = G % kXcds;
    return x * per + (x < rem ? x : rem) + local;
}

// Upper bound on seg_count over all heads for a given G: one head-initial
// segment plus at most ceil(G / BH) inner starts (an open interval of G/BH
// consecutive g values), and never more than nc segments.
GRET_HD int64_t seg_max_per_head(int64_t BH, int64_t nc, int64_t G) {
    const int64_t inner = (G + BH - 1) / BH;
    const int64_t m = 1 + inner;
    return m < nc ? m : nc;
}

}  // namespace gret
