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
using F32Apply = TileCfg<4, 2, 64, 8, 1, 0, true, 2, false, true, true, true>;
using F32ApplyR1 = TileCfg<4, 4, 64, 8, 1, 0, true, 2, false, true, true, true>;
using F32ApplyR1Wide = TileCfg<4, 4, 128, 4, 1, 0, true, 2, false, true, true, true>;
using F32Wave = TileCfg<4, 2, 32, 16, 1, 0>;
using F64Apply = TileCfg<2, 2, 64, 8, 1, 0, true, 2, false, true, true, true>;
using F64Wave = TileCfg<2, 2, 32, 16, 1, 0>;

template <typename T, int R, bool WAVE>
struct Shipped {
    using Cfg = typename std::conditional<
        std::is_same<T, double>::value,
        typename std::conditional<WAVE, F64Wave, F64Apply>::type,
        typename std::conditional<WAVE, F32Wave,
                                  typename std::conditional<R == 1, F32ApplyR1,
                                                            F32Apply>::type>::type>::type;
    // row-wide alternative (void: none)
    using Wide = typename std::conditional<!WAVE && R == 1 && std::is_same<T, float>::value,
                                           F32ApplyR1Wide, void>::type;
};

template <typename T, int R, bool WAVE, int V>
using CfgOf = typename std::conditional<V == 1 && !std::is_void<typename Shipped<T, R, WAVE>::Wide>::value,
                                        typename Shipped<T, R, WAVE>::Wide,
                                        typename Shipped<T, R, WAVE>::Cfg>::type;

template <typename T, int R>
int launch_typed(const stencil3d_desc &d, const Geometry &g, const void *in, void *out,
                 const void *u_prev, const void *vel2, const void *eta, bool wave,
                 double wscale, hipStream_t stream) {
    const StarArgs<T> a = make_args<T, R>(d, in, out, u_prev, vel2, eta, wscale, g.tiles_x,
                                          g.tiles_y, g.chunk_len, g.nwg);
    const dim3 grid(g.nwg), block(g.threads);
    if (wave)
        hipLaunchKernelGGL((star2p5d_kernel<T, R, true, CfgOf<T, R, true, 0>>), grid, block, 0,
                           stream, a);
    else if (g.variant == 1)
        hipLaunchKernelGGL((star2p5d_kernel<T, R, false, CfgOf<T, R, false, 1>>), grid, block,
                           0, stream, a);
    else
        hipLaunchKernelGGL((star2p5d_kernel<T, R, false, CfgOf<T, R, false, 0>>), grid, block,
                           0, stream, a);
    return hipGetLastError() == hipSuccess ? ST_OK : ST_ERR_LAUNCH;
}

template <typename T>
int launch_r(const stencil3d_desc &d, const Geometry &g, const void *in, void *out,
             const void *u_prev, const void *vel2, const void *eta, bool wave, double wscale,
             hipStream_t s) {
    switch (d.radius) {
    case 1: return launch_typed<T, 1>(d, g, in, out, u_prev, vel2, eta, wave, wscale, s);
    case 2: return launch_typed<T, 2>(d, g, in, out, u_prev, vel2, eta, wave, wscale, s);
    case 3: return launch_typed<T, 3>(d, g, in, out, u_prev, vel2, eta, wave, wscale, s);
    case 4: return launch_typed<T, 4>(d, g, in, out, u_prev, vel2, eta, wave, wscale, s);
    }
    return ST_ERR_RADIUS;
}

// Tile shape, threads and z unroll of the shipped kernel for (T, R, WAVE).
struct Shape {
    int tile_x, tile_y, threads, unroll, prologue;
};

template <typename T, int R, bool WAVE, int V>
Shape shape_of() {
    using C = CfgOf<T, R, WAVE, V>;
    using RG = Rings<R, WAVE, C>;
    return Shape{C::TX, C::TY, C::NT, RG::U, 2 * R + RG::D};
}

template <typename T, bool WAVE, int V>
Shape shape_r(int R) {
    switch (R) {
    case 1: return shape_of<T, 1, WAVE, V>();
    case 2: return shape_of<T, 2, WAVE, V>();
    case 3: return shape_of<T, 3, WAVE, V>();
    default: return shape_of<T, 4, WAVE, V>();
    }
}

Shape shape_for(const stencil3d_desc &d, bool wave, int variant) {
    if (d.dtype == ST_F64)
        return wave ? shape_r<double, true, 0>(d.radius)
                    : (variant ? shape_r<double, false, 1>(d.radius)
                               : shape_r<double, false, 0>(d.radius));
    return wave ? shape_r<float, true, 0>(d.radius)
                : (variant ? shape_r<float, false, 1>(d.radius) : shape_r<float, false, 0>(d.radius));
}

}  // namespace

Geometry plan_geometry(const stencil3d_desc &d, bool wave, int cus) {
    // The row-wide variant (if this kernel has one) is taken when one of its
    // tiles spans an interior row that needs two of the primary tiles and
    // fills at least 7/8 of it (measured: 510 and 512 wide rows gain 5-13%,
    // a 300 wide row loses a third).
    const int64_t ixr = d.nx - 2 * (int64_t)d.radius;
    const Shape prim = shape_for(d, wave, 0), wide = shape_for(d, wave, 1);
    const int variant = (wide.tile_x > prim.tile_x && ixr > prim.tile_x &&
                         8 * ixr > 7 * (int64_t)wide.tile_x && ixr <= wide.tile_x);
    const Shape sh = variant ? wide : prim;
    Geometry g;
    g.variant = variant;
    g.tile_x = sh.tile_x;
    g.tile_y = sh.tile_y;
    g.threads = sh.threads;
    const int R = d.radius;
    const int64_t ix = d.nx - 2 * R, iy = d.ny - 2 * R, iz = d.nz - 2 * R;
    g.tiles_x = (int)((ix + g.tile_x - 1) / g.tile_x);
    g.tiles_y = (int)((iy + g.tile_y - 1) / g.tile_y);
    const int64_t tiles = (int64_t)g.tiles_x * g.tiles_y;
    // Split z into chunks.  About 512 threads run per compute unit (the
    // register window allows two waves per SIMD), so `cap` workgroups run at
    // once and the launch takes ceil(workgroups / cap) rounds; each round
    // lasts a chunk's planes plus its pipeline fill.  Pick the chunk count
    // that minimises rounds * (chunk + fill); never below 4R planes per
    // chunk; chunk lengths are whole blocks of the kernel's z unroll (the
    // kernel runs whole blocks).
    const int64_t cap = (int64_t)(cus > 0 ? cus : 256) * (g.threads >= 512 ? 1 : 512 / g.threads);
    const int64_t maxch = iz / (4 * R) > 0 ? iz / (4 * R) : 1;
    int64_t best_len = 0, best_nch = 1, best_cost = -1;
    for (int64_t nch = 1; nch <= maxch; ++nch) {
        int64_t len = (iz + nch - 1) / nch;
        len = (len + sh.unroll - 1) / sh.unroll * sh.unroll;
        const int64_t n = (iz + len - 1) / len;
        const int64_t rounds = (tiles * n + cap - 1) / cap;
        const int64_t cost = rounds * (len + sh.prologue + 4);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best_len = len;
            best_nch = n;
        }
    }
    g.chunk_len = (int)best_len;
    g.nchunks = (int)best_nch;
    g.nwg = (int)(tiles * best_nch);
    return g;
}

int launch_star(const stencil3d_desc &d, const void *in, void *out, const void *u_prev,
                const void *vel2, const void *eta, bool wave, double wscale, int cus,
                hipStream_t stream) {
    const Geometry g = plan_geometry(d, wave, cus);
    if (d.dtype == ST_F64)
        return launch_r<double>(d, g, in, out, u_prev, vel2, eta, wave, wscale, stream);
    return launch_r<float>(d, g, in, out, u_prev, vel2, eta, wave, wscale, stream);
}

int launch_shell_copy(const stencil3d_desc &d, const void *in, void *out, hipStream_t stream) {
    const int64_t rows = d.ny * d.nz;
    int64_t blocks = (rows + 3) / 4;
    if (blocks > 8192) blocks = 8192;
    const dim3 grid((unsigned)blocks), block(256);
    if (d.dtype == ST_F64)
        hipLaunchKernelGGL(shell_copy_kernel<double>, grid, block, 0, stream,
                           static_cast<const double *>(in), static_cast<double *>(out),
                           (int)d.nx, (int)d.ny, (int)d.nz, d.radius);
    else
        hipLaunchKernelGGL(shell_copy_kernel<float>, grid, block, 0, stream,
                           static_cast<const float *>(in), static_cast<float *>(out),
                           (int)d.nx, (int)d.ny, (int)d.nz, d.radius);
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
