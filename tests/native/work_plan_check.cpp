// Checks the division of a streamed box among workgroups (work_plan.h):
// xcd_remap is a bijection, every plan is well formed, and under the
// kernels' workgroup map every (tile, plane) of the box is streamed by
// exactly one workgroup, for every combination of remapping and order.
#include <cstdio>
#include <initializer_list>
#include <vector>

#include "work_plan.h"

static int bad = 0;

static void fail(const char *what, long depth, long tiles, long cap, long minl) {
    if (++bad <= 20)
        std::printf("FAIL %s: depth=%ld tiles=%ld cap=%ld min=%ld\n", what, depth, tiles, cap,
                    minl);
}

static void check_plan(long depth, long tiles, long minl, long cap, long fill) {
    const st::ChunkPlan p = st::plan_chunks(depth, tiles, minl, cap, fill);
    const long btiles = tiles - p.a_tiles;
    if (p.a_nwg != p.a_tiles || p.a_tiles < 0 || p.a_tiles > tiles)
        return fail("group A shape", depth, tiles, cap, minl);
    if (p.a_nwg > 0 && (p.a_len != depth || p.a_tiles % cap != 0 || btiles == 0))
        return fail("group A chunks", depth, tiles, cap, minl);
    if (p.nwg != p.a_nwg + btiles * p.nchunks)
        return fail("workgroup count", depth, tiles, cap, minl);
    // group B: every chunk non-empty, and balanced: the last chunk is
    // shorter than the others by less than the chunk count
    if (p.chunk_len * p.nchunks < depth || p.chunk_len * (p.nchunks - 1) >= depth ||
        p.chunk_len * p.nchunks - depth >= p.nchunks)
        return fail("group B chunks", depth, tiles, cap, minl);
    for (int remap = 0; remap < 2; ++remap)
        for (int cmaj = 0; cmaj < 2; ++cmaj) {
            std::vector<unsigned char> seen((size_t)(tiles * depth), 0);
            for (long b = 0; b < p.nwg; ++b) {
                const st::WgWork w = st::wg_work((int)b, (int)p.nwg, (int)tiles, (int)p.a_nwg,
                                                 (int)p.a_tiles, (int)p.a_len, (int)p.chunk_len,
                                                 remap != 0, cmaj != 0);
                const bool ga = b < p.a_nwg;
                if (w.tile < (ga ? 0 : p.a_tiles) || w.tile >= (ga ? p.a_tiles : tiles) ||
                    w.zoff < 0 || w.zoff >= depth || w.len <= 0)
                    return fail("workgroup outside its group", depth, tiles, cap, minl);
                const long z1 = w.zoff + w.len < depth ? w.zoff + w.len : depth;
                for (long z = w.zoff; z < z1; ++z) seen[(size_t)(w.tile * depth + z)]++;
            }
            for (unsigned char c : seen)
                if (c != 1) return fail("coverage", depth, tiles, cap, minl);
        }
}

int main() {
    // xcd_remap: a bijection on [0, n), each XCD owning a contiguous range
    for (int n = 1; n <= 3000; ++n) {
        std::vector<int> hit(n, 0);
        for (int b = 0; b < n; ++b) {
            const int l = st::xcd_remap(b, n);
            if (l < 0 || l >= n) {
                fail("xcd_remap range", n, 0, 0, 0);
                break;
            }
            hit[l]++;
            // ids of one XCD map to consecutive logical ids
            if (b >= st::kXcds && st::xcd_remap(b - st::kXcds, n) != l - 1)
                fail("xcd_remap contiguity", n, b, 0, 0);
        }
        for (int h : hit)
            if (h != 1) {
                fail("xcd_remap bijection", n, 0, 0, 0);
                break;
            }
    }
    // xcd_remap_rounds: a bijection on [0, n) that keeps every round of
    // `round` ids in place and, within a whole round, gives each XCD a
    // contiguous range of it
    long rounds = 0;
    for (int n = 1; n <= 700; n += 3)
        for (int round : {0, 1, 8, 16, 24, 64, 80, 256}) {
            std::vector<int> hit(n, 0);
            for (int b = 0; b < n; ++b) {
                const int l = st::xcd_remap_rounds(b, n, round);
                if (l < 0 || l >= n) {
                    fail("xcd_remap_rounds range", n, round, 0, 0);
                    break;
                }
                hit[l]++;
                if (round > 0 && round < n) {
                    const int r0 = b / round * round;
                    if (l < r0 || l >= r0 + round) fail("xcd_remap_rounds round", n, round, b, 0);
                    const int m = n - r0 < round ? n - r0 : round;
                    if (l != r0 + st::xcd_remap(b - r0, m))
                        fail("xcd_remap_rounds per round", n, round, b, 0);
                } else if (l != st::xcd_remap(b, n)) {
                    fail("xcd_remap_rounds whole", n, round, b, 0);
                }
            }
            for (int h : hit)
                if (h != 1) {
                    fail("xcd_remap_rounds bijection", n, round, 0, 0);
                    break;
                }
            ++rounds;
        }
    std::printf("round remaps checked: %ld\n", rounds);
    const long depths[] = {1, 2, 3, 5, 8, 13, 16, 17, 31, 64, 100, 127, 255, 512, 1016, 1024};
    const long tiles[] = {1, 2, 7, 8, 9, 63, 255, 256, 257, 300, 304, 511, 513, 700};
    const long caps[] = {80, 256, 1024};
    const long mins[] = {4, 16};
    long plans = 0, mixed = 0;
    for (long d : depths)
        for (long t : tiles)
            for (long c : caps)
                for (long m : mins) {
                    check_plan(d, t, m, c, 12);
                    mixed += st::plan_chunks(d, t, m, c, 12).a_nwg > 0;
                    ++plans;
                }
    // worked example: 304 tiles of 512 planes, 256 workgroups at once
    const st::ChunkPlan e = st::plan_chunks(512, 304, 16, 256, 12);
    std::printf("plan(512 planes, 304 tiles, cap 256, fill 12, min 16): nwg %ld, "
                "A %ld tiles x %ld, B %ld chunks of %ld\n",
                (long)e.nwg, (long)e.a_tiles, (long)e.a_len, (long)e.nchunks, (long)e.chunk_len);
    // the 25-point apply on a 520^3 grid: 64 tiles of 256 x 16 over 512
    // planes on 256 compute units -> 4 equal chunks of 128
    const st::ChunkPlan h = st::plan_chunks(512, 64, 16, 256, 13);
    std::printf("plan(512 planes, 64 tiles, cap 256): nwg %ld, %ld chunks of %ld\n", (long)h.nwg,
                (long)h.nchunks, (long)h.chunk_len);
    std::printf("checked %ld plans (%ld mixed), %d bad\n", plans, mixed, bad);
    return bad == 0 ? 0 : 1;
}
