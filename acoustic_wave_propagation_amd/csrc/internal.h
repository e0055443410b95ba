// internal.h -- declarations shared by the C-ABI layer (api.cpp) and the
// kernels (star2p5d.hip).  Not installed; the public surface is stencil3d.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stencil3d.h"

namespace st {

// An output box [x0,x1) x [y0,y1) x [z0,z1) in allocated coordinates.
struct Box {
    int64_t x0, x1, y0, y1, z0, z1;
};

// The interior of d: every point whose whole stencil lies in the array.
inline Box interior_box(const stencil3d_desc &d) {
    const int64_t R = d.radius;
    return Box{R, d.nx - R, R, d.ny - R, R, d.nz - R};
}

// Variants of the streaming kernel.  Apply: out = star(in).  Wave: the
// wave update of (u_prev, in = u, vel2, eta).  WavePml: the PML step (the
// wave update plus the eta-gradient coupling).  The planner may replace
// Apply by ApplyWide (row-wide tiles), Wave by WaveNarrow and WavePml by
// WavePmlNarrow (32-column tiles) where those fit the box better.
// WaveRegions and WavePmlRegions: the wave update and the PML step on wider
// tiles, reading eta only near the faces for a stated sponge width (the
// data-region launches).
enum class Kind {
    Apply, ApplyWide, Wave, WaveNarrow, WavePml, WavePmlNarrow, WaveRegions, WavePmlRegions
};

// Launch geometry of the 2.5D kernel: XY tiles of tile_x * tile_y outputs
// covering the output box, each streamed through z in chunks.  The first
// a_nwg workgroups (group A, possibly none) stream tiles [0, a_tiles) in
// chunks of a_len planes; the others stream the remaining tiles in
// nchunks chunks of chunk_len planes.  nwg counts both groups.
struct Geometry {
    Kind kind;
    Box box;
    int tile_x, tile_y, threads;
    int tiles_x, tiles_y, nchunks, chunk_len, nwg;
    int a_nwg, a_tiles, a_len;
};

// Whether the kernel variant is instantiated for d's type and radius.
bool kind_available(const stencil3d_desc &d, Kind k);

// Geometry of a launch of `kind` over `box` (inside d's interior) on a
// device with `cus` compute units.  Host only.
Geometry plan_geometry(const stencil3d_desc &d, const Box &box, Kind kind, int cus);

// Enqueue the streaming stencil on the output box (inside the interior;
// empty boxes enqueue nothing).  Wave variants scale the weights by wscale
// = dt^2/h^2.  Kind::WaveRegions and WavePmlRegions with pw > 0 read eta only
// within pw of an interior face (the caller guarantees it is zero
// elsewhere).  Arguments
// are validated by the caller.  Returns ST_OK, ST_ERR_ARG (variant not
// instantiated) or ST_ERR_LAUNCH.
int launch_star(const stencil3d_desc &d, const Box &box, Kind kind, const void *in, void *out,
                const void *u_prev, const void *vel2, const void *eta, double wscale, int cus,
                hipStream_t stream, int pw = 0);

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

// Point source of a two-step pass: values v0 and v1 (steps n+1 and n+2) at
// allocated coordinates (x, y, z), if `on`.
struct Wave2Source {
    bool on;
    int64_t x, y, z;
    double v0, v1;
};

// Whether a two-step pass exists for d's type and radius.
bool wave2_available(const stencil3d_desc &d);

// Two leapfrog steps in one pass: out1 = u^{n+1} and out2 = u^{n+2} on the
// interior from u_prev = u^{n-1} and u = u^n (weights scaled by wscale =
// dt^2/h^2; pml: the PML step's update, with the eta-gradient coupling).
// pw > 0 (plain step, R = 4) states that eta is 0 at every interior point
// at least pw from all interior faces, and eta is read only where it may
// not be; otherwise eta is read on the whole interior.  Non-interior points
// of the outputs are not written; u^{n+1}'s non-interior values are taken
// as u's.  out1 and out2 must not overlap each other or any input.  Returns
// ST_OK, ST_ERR_ARG (no such pass for d) or ST_ERR_LAUNCH.
int launch_wave2(const stencil3d_desc &d, int pw, const void *u_prev, const void *u, void *out1,
                 void *out2, const void *vel2, const void *eta, double wscale,
                 const Wave2Source &src, int cus, hipStream_t stream, bool pml);

// out = in on every non-interior point.
int launch_shell_copy(const stencil3d_desc &d, const void *in, void *out,
                      hipStream_t stream);

// Device address and size of this device's static workspace (the two
// fields of wave_run_blocked_noalloc), looked up on the first call per
// device.  Returns ST_OK or ST_ERR_DEVICE.
int noalloc_scratch(void **ptr, size_t *bytes);

// u[idx] += value (one thread).
int launch_add_source(const stencil3d_desc &d, void *u, int64_t idx,
                      double value, hipStream_t stream);

}  // namespace st
