"""Host-side check of the prefill segment bookkeeping (gret_segments.h).

The header is compiled with g++ into a small driver that enumerates, for many
(heads, chunks per head, workgroups) triples, every segment the main kernel
visits and the slot it writes, and the count the combine kernel reads. They are
checked here by brute force: slots are unique, in range (below the per-head
bound that sizes the workspace), in sequence order, and every (head, chunk)
pair is covered exactly once. The map from a workgroup's launch index to its
segment (contiguous segment runs per XCD) must be a bijection, and the bound
on a piece's length that the prefill checks its 32-bit row offsets against must
hold for every piece.
"""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "yoco_gated_retention_amd", "csrc", "gret_segments.h")

DRIVER = r"""
#include <cstdio>
#include <cstdlib>
#include "gret_segments.h"
using namespace gret;
int main(int argc, char** argv) {
    SegPlan p;
    p.BH = atoll(argv[1]); p.nc = atoll(argv[2]); p.T = p.BH * p.nc;
    long long G = atoll(argv[3]); p.G = G < p.T ? G : p.T;
    p.max_seg = seg_max_per_head(p.BH, p.nc, p.G);
    printf("P %lld %lld %lld\n", (long long)p.G, (long long)p.max_seg,
           (long long)seg_max_piece_chunks(p));
    for (int64_t g = 0; g < p.G; ++g) {
        int64_t t = seg_lo(p, g), hi = seg_lo(p, g + 1);
        while (t < hi) {
            int64_t x = t / p.nc, cb = t - x * p.nc;
            int64_t ce = (hi - x * p.nc) < p.nc ? (hi - x * p.nc) : p.nc;
            int64_t slot = cb == 0 ? 0 : g - seg_first_inner(p, x) + 1;
            printf("S %lld %lld %lld %lld %lld\n", (long long)g, (long long)x, (long long)cb,
                   (long long)ce, (long long)slot);
            t = x * p.nc + ce;
        }
    }
    for (int64_t x = 0; x < p.BH; ++x) printf("C %lld %lld\n", (long long)x, (long long)seg_count(p, x));
    for (int64_t b = 0; b < p.G; ++b) printf("B %lld %lld\n", (long long)b, (long long)seg_of_block(p.G, b));
    return 0;
}
"""


@pytest.fixture(scope="module")
def driver():
    d = tempfile.mkdtemp(prefix="gret_seg_")
    src = os.path.join(d, "seg.cpp")
    exe = os.path.join(d, "seg")
    with open(src, "w") as f:
        f.write(DRIVER)
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-fsanitize=address,undefined",
                    "-I", os.path.dirname(HDR), src, "-o", exe], check=True)
    return exe


CASES = [(1, 1, 1), (1, 1, 512), (2, 8, 3), (24, 8192, 256), (24, 2048, 1024), (24, 16384, 256),
         (6144, 1, 1024), (96, 16, 1024), (3, 1000, 7), (7, 13, 50), (24, 512, 1024),
         (1, 100, 1024), (5, 3, 1024), (24, 8192, 512), (48, 7, 100)]


@pytest.mark.parametrize("BH,nc,G", CASES)
def test_segments_cover_and_slots(driver, BH, nc, G):
    out = subprocess.run([driver, str(BH), str(nc), str(G)], check=True, capture_output=True,
                         text=True).stdout.split("\n")
    Geff, max_seg, max_piece = map(int, out[0].split()[1:])
    assert Geff == min(G, BH * nc)
    covered = {}
    slots = {}
    counts = {}
    seg_of = {}
    for line in out[1:]:
        if line.startswith("S "):
            g, x, cb, ce, slot = map(int, line.split()[1:])
            assert 0 <= x < BH and 0 <= cb < ce <= nc
            assert 0 <= slot < max_seg
            # the bound the prefill's 32-bit row offsets are checked against
            assert ce - cb <= max_piece
            assert (x, slot) not in slots, "slot written twice"
            slots[(x, slot)] = (cb, ce)
            for c in range(cb, ce):
                assert (x, c) not in covered
                covered[(x, c)] = g
        elif line.startswith("C "):
            x, n = map(int, line.split()[1:])
            counts[x] = n
        elif line.startswith("B "):
            b, g = map(int, line.split()[1:])
            seg_of[b] = g
    assert len(covered) == BH * nc
    # ... and it is attained by some piece (or exceeds the longest by one)
    longest = max(ce - cb for cb, ce in slots.values())
    assert longest <= max_piece <= longest + 1
    # the launch-index -> segment map is a bijection of [0, G), and the ids
    # that share an XCD (b mod 8) take one contiguous run of segments in order
    assert sorted(seg_of) == list(range(Geff)) and sorted(seg_of.values()) == list(range(Geff))
    for xcd in range(8):
        run = [seg_of[b] for b in range(xcd, Geff, 8)]
        assert run == list(range(run[0], run[0] + len(run))) if run else True
    starts = sorted(seg_of[b] for b in range(min(8, Geff)))
    assert starts[0] == 0
    for x in range(BH):
        segs = sorted((s, cb, ce) for (xx, s), (cb, ce) in slots.items() if xx == x)
        assert counts[x] == len(segs) <= max_seg
        # slot order is sequence order and the segments tile the head
        assert [s for s, _, _ in segs] == list(range(len(segs)))
        assert segs[0][1] == 0 and segs[-1][2] == nc
        for (s0, _, e0), (s1, b1, _) in zip(segs, segs[1:]):
            assert e0 == b1
