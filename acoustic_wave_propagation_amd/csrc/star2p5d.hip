// star2p5d.hip -- instantiates the shipped tile configurations of the
// streaming stencil kernel (star2p5d_kernel.h) and launches them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"
#include "star2p5d_kernel.h"

namespace st {
namespace {

// Shipped configurations per element type and radius, chosen by timing
// and traffic counters on MI355X (sweeps over outputs per thread, threads
// per workgroup, prefetch depth, halo timing, LDS buffering, chunking and
// store policy).  All use 512-thread workgroups, one plane of stencil-input
// prefetch, the halo ring loaded with the window's leading plane and two LDS
// tile buffers (one barrier per z step):
//   fp32 apply, R >= 2: 4 x 2 outputs per thread, 64 x 8 threads -> 256 x 16
//                        tile, nontemporal stores
//   fp32 apply, R = 1:   4 x 4 outputs per thread (the short window leaves
//                        registers for more rows) -> 256 x 32 tile, or
//                        512 x 16 when one such tile spans and nearly
//                        fills an interior row (449..512 points; on 2 KB row
//                        pitches whole-row tiles run ~13% faster)
//   fp32 wave:           4 x 2 per thread, 32 x 16 threads -> 128 x 32 tile
//   fp64 apply:          2 x 2 per thread, 64 x 8 threads -> 128 x 16 tile,
//                        nontemporal stores
//   fp64 wave:           2 x 2 per thread, 32 x 16 threads ->  64 x 32 tile
// The wave tiles load a step's u_prev, vel2 and eta first, ahead of the
// stencil-input prefetch, so that waiting for them does not drain the
// prefetch (1032^3 fp32 step: 4.04 against 4.13 ms).
// The fp32 apply numbers its workgroups tile-major (the z chunks of a tile
// are neighbours, so each XCD streams all chunks of a band of tiles):
// 0.2040 against 0.2056 ms chunk-major on 520^3 (4 chunks of 128 planes),
// though it fetches more (the band edges' halo rows come from another XCD's
// L2 or the Infinity Cache).
using F32Apply = TileCfg<4, 2, 64, 8, 1, 0, true, 2, false, false, true, true>;
using F32ApplyR1 = TileCfg<4, 4, 64, 8, 1, 0, true, 2, false, true, true, true>;
using F32ApplyR1Wide = TileCfg<4, 4, 128, 4, 1, 0, true, 2, false, true, true, true>;
using F32Wave = TileCfg<4, 2, 32, 16, 1, 0, true, 2, false, true, true, false, false, 1, false, true>;
using F64Apply = TileCfg<2, 2, 64, 8, 1, 0, true, 2, false, true, true, true>;
using F64Wave = TileCfg<2, 2, 32, 16, 1, 0, true, 2, false, true, true, false, false, 1, false, true>;

// Tiles of the wave step's data regions (Kind::WaveRegions, with a sponge
// width): 4 x 2 (fp32) or 2 x 2 (fp64) per thread, 64 x 8 threads -> 256 x
// 16 or 128 x 16 tiles.  Every tile reads eta on as many columns as the
// sponge width (an eighth of a 256-wide tile for a 32-point sponge, a
// quarter of a 128-wide one): 1032^3 step with pml_width 32, 3.53 ms (3.70
// when each tile read the sponge width at both of its x edges, 3.92 with
// the 128 x 32 tiles, which are the faster ones when eta is read
// everywhere: 4.00 against 4.11 ms).  The PML step's data regions
// (Kind::WavePmlRegions) keep its primary tiles: on 256 x 16 its eta masks
// and rings spill registers.
using F32WaveRegions =
    TileCfg<4, 2, 64, 8, 1, 0, true, 2, false, true, true, false, false, 1, false, true>;
using F64WaveRegions =
    TileCfg<2, 2, 64, 8, 1, 0, true, 2, false, true, true, false, false, 1, false, true>;

// Narrow tiles for the thin x slabs of the wave step's sponge (32 columns):
// 4 x 2 (fp32) or 2 x 2 (fp64) per thread, 8 x 64 or 16 x 32 threads ->
// 32 x 128 or 32 x 64 tiles.  On a full 1024^3 step they run 7% slower than
// the primary tiles; on a 32-wide box they avoid three quarters idle lanes.
using F32WaveNarrow =
    TileCfg<4, 2, 8, 64, 1, 0, true, 2, false, true, true, false, false, 1, false, true>;
using F64WaveNarrow =
    TileCfg<2, 2, 16, 32, 1, 0, true, 2, false, true, true, false, false, 1, false, true>;

// fp64 PML step: the eta rings do not fit beside the halo ring of the
// window's lead, so the halo is loaded one plane ahead of its use instead
// (shorter halo and window rings).
using F64WavePml =
    TileCfg<2, 2, 32, 16, 1, 0, false, 2, false, true, true, false, false, 1, false, true>;
using F64WavePmlNarrow =
    TileCfg<2, 2, 16, 32, 1, 0, false, 2, false, true, true, false, false, 1, false, true>;

// Kernel variant of a launch: its tile configuration and template flags.
template <typename T, int R, Kind K>
struct KindCfg {
    static constexpr bool f64 = std::is_same<T, double>::value;
    static constexpr bool pml =
        K == Kind::WavePml || K == Kind::WavePmlNarrow || K == Kind::WavePmlRegions;
    static constexpr bool narrow = K == Kind::WaveNarrow || K == Kind::WavePmlNarrow;
    static constexpr bool regions = K == Kind::WaveRegions || K == Kind::WavePmlRegions;
    static constexpr bool wide = K == Kind::WaveRegions;
    static constexpr bool wave = K == Kind::Wave || K == Kind::WaveNarrow || regions || pml;
    using Apply = typename std::conditional<f64, F64Apply,
                  typename std::conditional<R == 1, F32ApplyR1, F32Apply>::type>::type;
    using Cfg = typename std::conditional<
        K == Kind::ApplyWide && R == 1 && !f64, F32ApplyR1Wide,
        typename std::conditional<
        wide, typename std::conditional<f64, F64WaveRegions, F32WaveRegions>::type,
        typename std::conditional<
            narrow && !(pml && f64),
            typename std::conditional<f64, F64WaveNarrow, F32WaveNarrow>::type,
            typename std::conditional<
                pml && f64,
                typename std::conditional<narrow, F64WavePmlNarrow, F64WavePml>::type,
                typename std::conditional<wave,
                                          typename std::conditional<f64, F64Wave, F32Wave>::type,
                                          Apply>::type>::type>::type>::type>::type;
};

// Variants that exist for radius R (the others fall back to the primary
// ones): the row-wide apply for fp32 R = 1, the narrow and wide wave and
// PML kernels for R = 4, the radius of the acoustic model with a sponge.
template <typename T, int R>
constexpr bool kind_exists(Kind k) {
    return k == Kind::Apply || k == Kind::Wave || k == Kind::WavePml ||
           (k == Kind::ApplyWide && R == 1 && std::is_same<T, float>::value) ||
           ((k == Kind::WaveNarrow || k == Kind::WavePmlNarrow || k == Kind::WaveRegions ||
             k == Kind::WavePmlRegions) &&
            R == 4);
}

template <typename T, int R, Kind K>
int launch_kind(const StarArgs<T> &a, int nwg, hipStream_t stream) {
    using KC = KindCfg<T, R, K>;
    hipLaunchKernelGGL((star2p5d_kernel<T, R, KC::wave, typename KC::Cfg, KC::pml, KC::regions>),
                       dim3(nwg), dim3(KC::Cfg::NT), 0, stream, a);
    return hipGetLastError() == hipSuccess ? ST_OK : ST_ERR_LAUNCH;
}

template <typename T, int R>
int launch_typed(const stencil3d_desc &d, const Geometry &g, const void *in, void *out,
                 const void *u_prev, const void *vel2, const void *eta, double wscale,
                 hipStream_t stream, int pw) {
    StarArgs<T> a = make_args<T, R>(d, g.box, in, out, u_prev, vel2, eta, wscale, g.tiles_x,
                                    g.tiles_y, g.chunk_len, g.nwg);
    a.pw = (g.kind == Kind::WaveRegions || g.kind == Kind::WavePmlRegions) ? pw : 0;
    a.ga_nwg = g.a_nwg;
    a.ga_tiles = g.a_tiles;
    a.ga_len = g.a_len;
    switch (g.kind) {
    case Kind::ApplyWide:
        if constexpr (kind_exists<T, R>(Kind::ApplyWide))
            return launch_kind<T, R, Kind::ApplyWide>(a, g.nwg, stream);
        break;
    case Kind::Wave: return launch_kind<T, R, Kind::Wave>(a, g.nwg, stream);
    case Kind::WaveNarrow:
        if constexpr (kind_exists<T, R>(Kind::WaveNarrow))
            return launch_kind<T, R, Kind::WaveNarrow>(a, g.nwg, stream);
        break;
    case Kind::WaveRegions:
        if constexpr (kind_exists<T, R>(Kind::WaveRegions))
            return launch_kind<T, R, Kind::WaveRegions>(a, g.nwg, stream);
        break;
    case Kind::WavePmlRegions:
        if constexpr (kind_exists<T, R>(Kind::WavePmlRegions))
            return launch_kind<T, R, Kind::WavePmlRegions>(a, g.nwg, stream);
        break;
    case Kind::WavePml: return launch_kind<T, R, Kind::WavePml>(a, g.nwg, stream);
    case Kind::WavePmlNarrow:
        if constexpr (kind_exists<T, R>(Kind::WavePmlNarrow))
            return launch_kind<T, R, Kind::WavePmlNarrow>(a, g.nwg, stream);
        break;
    default: return launch_kind<T, R, Kind::Apply>(a, g.nwg, stream);
    }
    return ST_ERR_ARG;  // the planner never picks a variant that does not exist
}

template <typename T>
int launch_r(const stencil3d_desc &d, const Geometry &g, const void *in, void *out,
             const void *u_prev, const void *vel2, const void *eta, double wscale,
             hipStream_t s, int pw) {
    switch (d.radius) {
    case 1: return launch_typed<T, 1>(d, g, in, out, u_prev, vel2, eta, wscale, s, pw);
    case 2: return launch_typed<T, 2>(d, g, in, out, u_prev, vel2, eta, wscale, s, pw);
    case 3: return launch_typed<T, 3>(d, g, in, out, u_prev, vel2, eta, wscale, s, pw);
    case 4: return launch_typed<T, 4>(d, g, in, out, u_prev, vel2, eta, wscale, s, pw);
    }
    return ST_ERR_RADIUS;
}

// Tile shape, threads and pipeline fill of a kernel variant.
struct Shape {
    int tile_x, tile_y, threads, prologue;
    bool exists;
};

template <typename T, int R, Kind K>
Shape shape_of() {
    using KC = KindCfg<T, R, K>;
    using C = typename KC::Cfg;
    using RG = Rings<R, KC::wave, C, KC::pml>;
    return Shape{C::TX, C::TY, C::NT, 2 * R + RG::D, kind_exists<T, R>(K)};
}

template <typename T, int R>
Shape shape_k(Kind k) {
    switch (k) {
    case Kind::ApplyWide: return shape_of<T, R, Kind::ApplyWide>();
    case Kind::Wave: return shape_of<T, R, Kind::Wave>();
    case Kind::WaveNarrow: return shape_of<T, R, Kind::WaveNarrow>();
    case Kind::WaveRegions: return shape_of<T, R, Kind::WaveRegions>();
    case Kind::WavePmlRegions: return shape_of<T, R, Kind::WavePmlRegions>();
    case Kind::WavePml: return shape_of<T, R, Kind::WavePml>();
    case Kind::WavePmlNarrow: return shape_of<T, R, Kind::WavePmlNarrow>();
    default: return shape_of<T, R, Kind::Apply>();
    }
}

template <typename T>
Shape shape_t(int R, Kind k) {
    switch (R) {
    case 1: return shape_k<T, 1>(k);
    case 2: return shape_k<T, 2>(k);
    case 3: return shape_k<T, 3>(k);
    default: return shape_k<T, 4>(k);
    }
}

Shape shape_for(const stencil3d_desc &d, Kind k) {
    return d.dtype == ST_F64 ? shape_t<double>(d.radius, k) : shape_t<float>(d.radius, k);
}

}  // namespace

bool kind_available(const stencil3d_desc &d, Kind k) { return shape_for(d, k).exists; }

Geometry plan_geometry(const stencil3d_desc &d, const Box &box, Kind kind, int cus) {
    const int64_t bx = box.x1 - box.x0, by = box.y1 - box.y0, bz = box.z1 - box.z0;
    if (kind == Kind::Apply) {
        // The row-wide variant (if this kernel has one) is taken when one of
        // its tiles spans a box row that needs two of the primary tiles and
        // fills at least 7/8 of it (measured: 510 and 512 wide rows gain
        // 5-13%, a 300 wide row loses a third).
        const Shape prim = shape_for(d, Kind::Apply), wide = shape_for(d, Kind::ApplyWide);
        if (wide.exists && wide.tile_x > prim.tile_x && bx > prim.tile_x &&
            8 * bx > 7 * (int64_t)wide.tile_x && bx <= wide.tile_x)
            kind = Kind::ApplyWide;
    } else if (kind == Kind::Wave || kind == Kind::WavePml) {
        // a box no wider than the narrow wave tile (the sponge's x slabs)
        const Kind nk = kind == Kind::Wave ? Kind::WaveNarrow : Kind::WavePmlNarrow;
        const Shape prim = shape_for(d, kind), nar = shape_for(d, nk);
        if (nar.exists && nar.tile_x < prim.tile_x && bx <= nar.tile_x) kind = nk;
    }
    const Shape sh = shape_for(d, kind);
    Geometry g;
    g.kind = kind;
    g.box = box;
    g.tile_x = sh.tile_x;
    g.tile_y = sh.tile_y;
    g.threads = sh.threads;
    g.tiles_x = (int)((bx + g.tile_x - 1) / g.tile_x);
    g.tiles_y = (int)((by + g.tile_y - 1) / g.tile_y);
    const int64_t tiles = (int64_t)g.tiles_x * g.tiles_y;
    // Split z into chunks.  About 512 threads run per compute unit (the
    // register window allows two waves per SIMD), so `cap` workgroups run at
    // once; chunks are no shorter than about 4R planes.
    const int R = d.radius;
    const int64_t cap = (int64_t)(cus > 0 ? cus : 256) * (g.threads >= 512 ? 1 : 512 / g.threads);
    const ChunkPlan p = plan_chunks(bz, tiles, 4 * R, cap, sh.prologue + 4);
    g.nwg = (int)p.nwg;
    g.chunk_len = (int)p.chunk_len;
    g.nchunks = (int)p.nchunks;
    g.a_nwg = (int)p.a_nwg;
    g.a_tiles = (int)p.a_tiles;
    g.a_len = (int)p.a_len;
    return g;
}

int launch_star(const stencil3d_desc &d, const Box &box, Kind kind, const void *in, void *out,
                const void *u_prev, const void *vel2, const void *eta, double wscale, int cus,
                hipStream_t stream, int pw) {
    if (box.x1 <= box.x0 || box.y1 <= box.y0 || box.z1 <= box.z0) return ST_OK;  // empty
    const Geometry g = plan_geometry(d, box, kind, cus);
    if (d.dtype == ST_F64)
        return launch_r<double>(d, g, in, out, u_prev, vel2, eta, wscale, stream, pw);
    return launch_r<float>(d, g, in, out, u_prev, vel2, eta, wscale, stream, pw);
}

int launch_shell_copy(const stencil3d_desc &d, const void *in, void *out, hipStream_t stream) {
    const int64_t R = d.radius;
    const int64_t full_rows = 2 * R * d.ny + (d.nz - 2 * R) * 2 * R;
    int64_t full_blocks = (full_rows + 3) / 4;  // 4 waves per block, one row each
    if (full_blocks > 4096) full_blocks = 4096;
    const int64_t ends = (d.ny - 2 * R) * (d.nz - 2 * R);  // one thread per interior row
    int64_t end_blocks = (ends + 255) / 256;
    if (end_blocks > 65536) end_blocks = 65536;
    if (end_blocks < 1) end_blocks = 1;
    const int64_t blocks = full_blocks + end_blocks;
    const dim3 grid((unsigned)blocks), block(256);
    if (d.dtype == ST_F64)
        hipLaunchKernelGGL(shell_copy_kernel<double>, grid, block, 0, stream,
                           static_cast<const double *>(in), static_cast<double *>(out),
                           (int)d.nx, (int)d.ny, (int)d.nz, d.radius, (int)full_blocks);
    else
        hipLaunchKernelGGL(shell_copy_kernel<float>, grid, block, 0, stream,
                           static_cast<const float *>(in), static_cast<float *>(out),
                           (int)d.nx, (int)d.ny, (int)d.nz, d.radius, (int)full_blocks);
    return hipGetLastError() == hipSuccess ? ST_OK : ST_ERR_LAUNCH;
}

int launch_add_source(const stencil3d_desc &d, void *u, int64_t idx, double value,
                      hipStream_t stream) {
    if (d.dtype == ST_F64)
        hipLaunchKernelGGL(add_source_kernel<double>, dim3(1), dim3(64), 0, stream,
                           static_cast<double *>(u), idx, value);
    else
        hipLaunchKernelGGL(add_source_kernel<float>, dim3(1), dim3(64), 0, stream,
                           static_cast<float *>(u), idx, (float)value);
    return hipGetLastError() == hipSuccess ? ST_OK : ST_ERR_LAUNCH;
}

}  // namespace st
