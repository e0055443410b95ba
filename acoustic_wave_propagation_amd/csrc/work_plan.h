// work_plan.h -- how a streamed box is divided among workgroups: the (x, y)
// face is cut into tiles, and each tile's column of z planes into chunks;
// one workgroup streams one chunk of one tile.  The host picks the chunking
// (plan_chunks); the map from a workgroup id back to its tile and chunk
// (wg_work) is what the kernels run.  No HIP dependency: constexpr functions
// compile for the device as well, and a plain C++ compiler can check that
// every plan covers each (tile, plane) exactly once.
#pragma once

#include <stdint.h>

namespace st {

constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dealt round-robin

// Bijection on [0, n) from the hardware workgroup id to a logical id such
// that XCD k (which receives ids k, k+8, k+16, ...) owns one contiguous range
// of logical ids.
__attribute__((always_inline)) constexpr int xcd_remap(int b, int n) {
    const int q = n / kXcds, r = n % kXcds;
    const int xcd = b % kXcds, i = b / kXcds;
    return xcd < r ? xcd * (q + 1) + i : r * (q + 1) + (xcd - r) * q + i;
}

// xcd_remap applied to each run of `round` consecutive ids on its own (the
// workgroups that run at the same time when each of `round` compute units
// holds one), so that within every round each XCD owns a contiguous range
// of that round's logical ids.  round <= 0 or round >= n: xcd_remap over
// all of [0, n).  A bijection on [0, n) that keeps every round in place.
__attribute__((always_inline)) constexpr int xcd_remap_rounds(int b, int n, int round) {
    if (round <= 0 || round >= n) return xcd_remap(b, n);
    const int r0 = b / round * round;
    const int m = n - r0 < round ? n - r0 : round;
    return r0 + xcd_remap(b - r0, m);
}

// Chunking of one launch.  Two groups of workgroups: group A (ids below
// a_nwg) streams tiles [0, a_tiles) in chunks of a_len planes; group B (the
// other nwg - a_nwg ids) streams the remaining tiles, each in `nchunks`
// chunks of chunk_len planes.  Uniform chunking has an empty group A.
struct ChunkPlan {
    int64_t nwg;
    int64_t chunk_len, nchunks;        // group B
    int64_t a_nwg, a_tiles, a_len;     // group A
};

// Chunking of `depth` planes under `tiles` tile columns, for a device on
// which `cap` workgroups run at once.  A set of equal chunks takes
// ceil(workgroups / cap) rounds, each lasting a chunk's planes plus the
// pipeline fill `fill`; the chunk count minimising rounds * (length + fill)
// is taken, with chunks no shorter than min_len planes (roughly).  Chunks
// are as equal as the depth allows (ceil(depth / count) planes, the last
// one shorter by less than the count): the kernels run any chunk length at
// the cost of its own steps, and the longest chunk sets a round's time.
// (Rounding the 512 planes of a 520^3 grid up to whole 12-step unroll
// blocks, 132 + 132 + 132 + 116, left the workgroups of the short chunk
// idle for the last 8% of the launch.)  When the tiles fill
// whole rounds with some left over, group A instead streams the whole
// rounds' tiles through all of z and only the remaining tiles are chunked
// (e.g. 304 tiles on 256 compute units: 256 whole columns, then 48 columns
// in 5 chunks, rather than every column in 5 chunks) if that costs less.
inline ChunkPlan plan_chunks(int64_t depth, int64_t tiles, int64_t min_len, int64_t cap,
                             int64_t fill) {
    struct Chunks {
        int64_t len, nch, cost;
    };
    auto best = [&](int64_t nt) {
        // more chunks than fill a few rounds of workgroups never pay; the
        // cap keeps the search short for very tall grids
        int64_t maxch = depth / min_len > 0 ? depth / min_len : 1;
        const int64_t enough = 8 * cap / (nt > 0 ? nt : 1) + 1;
        if (maxch > enough) maxch = enough;
        Chunks b{depth, 1, -1};
        for (int64_t nch = 1; nch <= maxch; ++nch) {
            const int64_t len = (depth + nch - 1) / nch;
            const int64_t n = (depth + len - 1) / len;
            const int64_t rounds = (nt * n + cap - 1) / cap;
            const int64_t cost = rounds * (len + fill);
            if (b.cost < 0 || cost < b.cost) b = Chunks{len, n, cost};
        }
        return b;
    };
    const Chunks uni = best(tiles);
    ChunkPlan p{tiles * uni.nch, uni.len, uni.nch, 0, 0, 0};
    const int64_t full = tiles / cap * cap, rest = tiles - full;
    if (full > 0 && rest > 0) {
        const Chunks b = best(rest);
        if (full / cap * (depth + fill) + b.cost < uni.cost)
            p = ChunkPlan{full + rest * b.nch, b.len, b.nch, full, full, depth};
    }
    return p;
}

// What one workgroup streams.
struct WgWork {
    int tile;   // tile index, x fastest
    int chunk;  // chunk index within the tile's column (its parity picks the
                // streaming direction where the kernel alternates)
    int zoff;   // first plane of the chunk, relative to the box
    int len;    // planes of a whole chunk (the box's end may cut the last)
};

// The tile and chunk of workgroup `block` of a launch of `nwg` workgroups
// over `ntile` tiles, chunked as a ChunkPlan says.  Each group is remapped
// on its own (remap), so every XCD sweeps a contiguous band of its group's
// tiles; with round > 0 each round of `round` workgroups of a group is
// remapped on its own (xcd_remap_rounds), so the band is contiguous within
// every round.  Chunk-major order (cmaj) numbers the tiles fastest, so
// workgroups that run together stream the same planes; otherwise the
// chunks of one tile are neighbours.
__attribute__((always_inline)) constexpr WgWork wg_work(int block, int nwg, int ntile,
                                                        int a_nwg, int a_tiles, int a_len,
                                                        int chunk_len, bool remap, bool cmaj,
                                                        int round = 0) {
    const bool ga = block < a_nwg;
    const int gid = ga ? block : block - a_nwg;
    const int gnwg = ga ? a_nwg : nwg - a_nwg;
    const int gt0 = ga ? 0 : a_tiles;
    const int gtiles = ga ? a_tiles : ntile - a_tiles;
    const int glen = ga ? a_len : chunk_len;
    const int wg = remap ? xcd_remap_rounds(gid, gnwg, round) : gid;
    int chunk = 0, t = 0;
    if (cmaj) {
        chunk = wg / gtiles;
        t = wg - chunk * gtiles;
    } else {
        const int nch = gnwg / gtiles;
        t = wg / nch;
        chunk = wg - t * nch;
    }
    return WgWork{gt0 + t, chunk, chunk * glen, glen};
}

}  // namespace st
