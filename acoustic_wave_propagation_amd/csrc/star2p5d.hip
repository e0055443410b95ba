// star2p5d.hip -- instantiates the shipped tile configurations of the
// streaming stencil kernel (star2p5d_kernel.h) and launches them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "star2p5d_kernel.h"

namespace st {
namespace {

// Shipped configurations per element type, chosen by timing and traffic
// counters on MI355X (sweep over outputs per thread, threads per workgroup,
// prefetch depth, halo timing, LDS buffering, chunking, store policy):
//   fp32 apply: 4 x 2 outputs per thread, 64 x 8 threads  -> 256 x 16 tile,
//               nontemporal stores
//   fp32 wave:  4 x 2 outputs per thread, 32 x 16 threads -> 128 x 32 tile
//   fp64:       2 x 2 outputs per thread, 32 x 16 threads ->  64 x 32 tile
// one plane of stencil-input prefetch, halo ring loaded with the window's
// leading plane, two LDS tile buffers (one barrier per z step).
template <typename T>
struct Shipped;
template <>
struct Shipped<float> {
    using Apply = TileCfg<4, 2, 64, 8, 1, 0, true, 2, false, true, true, true>;
    using Wave = TileCfg<4, 2, 32, 16, 1, 0>;
};
template <>
struct Shipped<double> {
    using Apply = TileCfg<2, 2, 32, 16, 1, 0>;
    using Wave = TileCfg<2, 2, 32, 16, 1, 0>;
};

template <typename T, int R>
int launch_typed(const stencil3d_desc &d, const Geometry &g, const void *in, void *out,
                 const void *u_prev, const void *vel2, const void *eta, bool wave,
                 double wscale, hipStream_t stream) {
    const StarArgs<T> a = make_args<T, R>(d, in, out, u_prev, vel2, eta, wscale, g.tiles_x,
                                          g.tiles_y, g.chunk_len, g.nwg);
    const dim3 grid(g.nwg), block(g.threads);
    if (wave)
        hipLaunchKernelGGL((star2p5d_kernel<T, R, true, typename Shipped<T>::Wave>), grid,
                           block, 0, stream, a);
    else
        hipLaunchKernelGGL((star2p5d_kernel<T, R, false, typename Shipped<T>::Apply>), grid,
                           block, 0, stream, a);
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

template <class C>
void tile_of(Geometry &g) {
    g.tile_x = C::TX;
    g.tile_y = C::TY;
    g.threads = C::NT;
}

template <bool WAVE, class C>
int unroll_of(int R) {
    switch (R) {
    case 1: return Rings<1, WAVE, C>::U;
    case 2: return Rings<2, WAVE, C>::U;
    case 3: return Rings<3, WAVE, C>::U;
    default: return Rings<4, WAVE, C>::U;
    }
}

}  // namespace

Geometry plan_geometry(const stencil3d_desc &d, bool wave, int cus) {
    Geometry g;
    int unroll;
    if (d.dtype == ST_F64) {
        if (wave) {
            tile_of<Shipped<double>::Wave>(g);
            unroll = unroll_of<true, Shipped<double>::Wave>(d.radius);
        } else {
            tile_of<Shipped<double>::Apply>(g);
            unroll = unroll_of<false, Shipped<double>::Apply>(d.radius);
        }
    } else {
        if (wave) {
            tile_of<Shipped<float>::Wave>(g);
            unroll = unroll_of<true, Shipped<float>::Wave>(d.radius);
        } else {
            tile_of<Shipped<float>::Apply>(g);
            unroll = unroll_of<false, Shipped<float>::Apply>(d.radius);
        }
    }
    const int R = d.radius;
    const int64_t ix = d.nx - 2 * R, iy = d.ny - 2 * R, iz = d.nz - 2 * R;
    g.tiles_x = (int)((ix + g.tile_x - 1) / g.tile_x);
    g.tiles_y = (int)((iy + g.tile_y - 1) / g.tile_y);
    const int64_t tiles = (int64_t)g.tiles_x * g.tiles_y;
    // About 512 threads per compute unit (one 512-thread workgroup: the
    // register window allows two waves per SIMD); split z into chunks only
    // as far as needed for that, and never below 4R planes per chunk (each
    // chunk re-reads 2R planes of z halo).  Chunk lengths are whole blocks
    // of the kernel's z unroll (the kernel runs whole blocks).
    const int64_t per_cu = g.threads >= 512 ? 1 : 512 / g.threads;
    const int64_t target = per_cu * (int64_t)(cus > 0 ? cus : 256);
    int64_t nch = (target + tiles - 1) / tiles;
    const int64_t maxch = iz / (4 * R) > 0 ? iz / (4 * R) : 1;
    if (nch > maxch) nch = maxch;
    if (nch < 1) nch = 1;
    int64_t len = (iz + nch - 1) / nch;
    len = (len + unroll - 1) / unroll * unroll;
    nch = (iz + len - 1) / len;  // every chunk non-empty
    g.chunk_len = (int)len;
    g.nchunks = (int)nch;
    g.nwg = (int)(tiles * nch);
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
