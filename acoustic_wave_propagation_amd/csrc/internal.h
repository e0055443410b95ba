// internal.h -- declarations shared by the C-ABI layer (api.cpp) and the
// kernels (star2p5d.hip).  Not installed; the public surface is stencil3d.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stencil3d.h"

namespace st {

// Launch geometry of the 2.5D kernel: XY tiles of tile_x * tile_y outputs,
// each streamed through a z-chunk of chunk_len interior planes.
struct Geometry {
    int tile_x, tile_y, threads;
    int tiles_x, tiles_y, nchunks, chunk_len, nwg;
    int variant;  // 0: the primary tile shape, 1: the row-wide one
};

// Geometry the kernel for (dtype, R, op) would use on a device with `cus`
// compute units.  Host only.
Geometry plan_geometry(const stencil3d_desc &d, bool wave, int cus);

// Enqueue the streaming stencil.  wave == false: out = star(in) on the
// interior.  wave == true: out = wave update of (u_prev, in = u, vel2, eta)
// with the weights scaled by wscale = dt^2/h^2.  Arguments are validated by
// the caller.  Returns ST_OK or ST_ERR_LAUNCH.
int launch_star(const stencil3d_desc &d, const void *in, void *out,
                const void *u_prev, const void *vel2, const void *eta,
                bool wave, double wscale, int cus, hipStream_t stream);

// Largest number of sweeps one fused pass can do for d (1: no fused kernel
// for this radius and element type).
int fused_max_sweeps(const stencil3d_desc &d);

// Relative time of a pass of ns sweeps, ns = 1..fused_max_sweeps(d) (one
// single sweep = 1).
const double *fused_pass_costs(const stencil3d_desc &d);

// One pass of ns fused Jacobi sweeps (2 <= ns <= fused_max_sweeps(d)): out's
// interior = ns applications of the stencil to in, with in's non-interior
// points held fixed.  out's non-interior points are not written.  in and
// out must not overlap.  Returns ST_OK, ST_ERR_ARG (unsupported ns or
// radius) or ST_ERR_LAUNCH.
int launch_sweeps_fused(const stencil3d_desc &d, const void *in, void *out, int ns, int cus,
                        hipStream_t stream);

// out = in on every non-interior point.
int launch_shell_copy(const stencil3d_desc &d, const void *in, void *out,
                      hipStream_t stream);

// u[idx] += value (one thread).
int launch_add_source(const stencil3d_desc &d, void *u, int64_t idx,
                      double value, hipStream_t stream);

}  // namespace st
