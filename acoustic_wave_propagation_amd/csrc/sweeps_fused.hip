// sweeps_fused.hip -- instantiates and launches the fused-sweep (temporally
// blocked) Jacobi kernel of sweeps_fused_kernel.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"
#include "sweeps_fused_kernel.h"

namespace st {
namespace {

// R = 1 only: the extended tile grows by NS*R points per side, so larger
// radii would spend most of the work on the overlap.  The extended tile
// adds whole 16-byte groups in x and NS rows in y on each side; 4 x 2
// (fp32) or 2 x 2 (fp64) points per thread.
//  * fp32, NS = 3..5: 128 x 32 output tiles, one set of (dense) LDS tiles
//    (two barriers per z step), 646-756 threads at three or four waves per
//    SIMD (NS = 5: 168 VGPRs, 8 bytes spilled).  The taller tile cuts the
//    overlap the stages recompute (NS = 5: extended / output area 1.48
//    against 1.83 at 128 x 16).  Per 512^3 call, ms (two passes and the
//    boundary copy), 128 x 16 with two LDS sets -> 128 x 32: 10 sweeps
//    (5 + 5) 0.930 -> 0.750, 8 (4 + 4) 0.794 -> 0.653, 6 (3 + 3) 0.653 ->
//    0.592; 128 x 48 at NS = 3: 0.629.  Taller NS = 4 and 5 tiles need four
//    waves per SIMD and spill.
//  * fp32, NS = 2 and 6: 128 x 16 output tiles (NS = 6 needs 194 VGPRs, two
//    waves per SIMD: no taller tile fits), two LDS sets at NS = 2, one at 6.
//  * fp64, NS = 2..4: 64 x 32 output tiles, one LDS set, 612-720 threads
//    (NS = 4: 148 VGPRs, three waves per SIMD).  Per 512^3 call against 64
//    x 16 tiles with two LDS sets, ms: 10 sweeps (3 + 3 + 2 + 2) 2.34 ->
//    1.93, 8 (4 + 4) 1.62 -> 1.22, 6 (3 + 3) 1.33 -> 1.04, 4 (2 + 2) 1.04
//    -> 0.92.
// Time per pass on a 512^3 grid (from calls of a known plan, less the
// boundary copy, 0.018 ms fp32 and 0.024 ms fp64): fp32 NS = 3, 4, 5, 6:
// 0.287, 0.317, 0.366, 0.559 ms (one single sweep: 0.224); fp64 NS = 2, 3,
// 4: 0.450, 0.506, 0.599 (one single sweep: 0.502).  The fp64 two-sweep
// pass varies from box to box (0.45-0.57 ms on three boxes; the others
// within 1%); the table takes the first box's figures.
template <typename T, int NS>
struct FusedShipped;
template <int NS>
struct FusedShipped<float, NS> {
    static constexpr int XE = (NS + 3) / 4 * 4;
    static constexpr int TY = NS >= 3 && NS <= 5 ? 32 : 16;  // output tile rows
    using Cfg = FusedCfg<4, 2, (128 + 2 * XE) / 4, (TY + 2 * NS) / 2, 1,
                         (TY > 16 || NS > 5) ? 1 : 2>;
};
template <int NS>
struct FusedShipped<double, NS> {
    static constexpr int XE = (NS + 1) / 2 * 2;
    using Cfg = FusedCfg<2, 2, (64 + 2 * XE) / 2, (32 + 2 * NS) / 2, 1, 1>;
};

struct FusedPlan {
    int tiles_x, tiles_y, chunk_len, nwg, threads;
    int a_nwg, a_tiles, a_len;  // group A (whole-z columns), as in plan_geometry
};

template <typename T, int NS>
FusedPlan plan_fused(const stencil3d_desc &d, int cus) {
    using C = typename FusedShipped<T, NS>::Cfg;
    using FS = FusedShape<1, NS, C>;
    FusedPlan p;
    const int64_t ix = d.nx - 2, iy = d.ny - 2, iz = d.nz - 2;
    p.tiles_x = (int)((ix + FS::TX - 1) / FS::TX);
    p.tiles_y = (int)((iy + FS::TY - 1) / FS::TY);
    p.threads = C::NT;
    const int64_t tiles = (int64_t)p.tiles_x * p.tiles_y;
    // one workgroup per compute unit (LDS and registers); chunked as for
    // the single-sweep kernel, no shorter than about 4 planes per sweep
    const ChunkPlan c = plan_chunks(iz, tiles, 4 * NS, cus > 0 ? cus : 256, FS::PROLOGUE + 4);
    p.nwg = (int)c.nwg;
    p.chunk_len = (int)c.chunk_len;
    p.a_nwg = (int)c.a_nwg;
    p.a_tiles = (int)c.a_tiles;
    p.a_len = (int)c.a_len;
    return p;
}

template <typename T, int NS>
int launch_ns(const stencil3d_desc &d, const void *in, void *out, int cus, hipStream_t s) {
    using C = typename FusedShipped<T, NS>::Cfg;
    const FusedPlan p = plan_fused<T, NS>(d, cus);
    StarArgs<T> a = make_args<T, 1>(d, interior_box(d), in, out, nullptr, nullptr, nullptr, 1.0,
                                    p.tiles_x, p.tiles_y, p.chunk_len, p.nwg);
    a.ga_nwg = p.a_nwg;
    a.ga_tiles = p.a_tiles;
    a.ga_len = p.a_len;
    hipLaunchKernelGGL((sweeps_fused_kernel<T, 1, NS, C>), dim3(p.nwg), dim3(p.threads), 0, s, a);
    return hipGetLastError() == hipSuccess ? ST_OK : ST_ERR_LAUNCH;
}

int launch_f32(const stencil3d_desc &d, const void *in, void *out, int ns, int cus,
               hipStream_t s) {
    switch (ns) {
    case 2: return launch_ns<float, 2>(d, in, out, cus, s);
    case 3: return launch_ns<float, 3>(d, in, out, cus, s);
    case 4: return launch_ns<float, 4>(d, in, out, cus, s);
    case 5: return launch_ns<float, 5>(d, in, out, cus, s);
    case 6: return launch_ns<float, 6>(d, in, out, cus, s);
    }
    return ST_ERR_ARG;
}

int launch_f64(const stencil3d_desc &d, const void *in, void *out, int ns, int cus,
               hipStream_t s) {
    switch (ns) {
    case 2: return launch_ns<double, 2>(d, in, out, cus, s);
    case 3: return launch_ns<double, 3>(d, in, out, cus, s);
    case 4: return launch_ns<double, 4>(d, in, out, cus, s);
    }
    return ST_ERR_ARG;
}

}  // namespace

int fused_max_sweeps(const stencil3d_desc &d) {
    if (d.radius != 1) return 1;
    return d.dtype == ST_F64 ? 4 : 6;
}

const double *fused_pass_costs(const stencil3d_desc &d) {
    // time of a pass of ns sweeps relative to one single sweep (index ns),
    // measured on 512^3 grids (fp32 ns = 2: an older measurement, 0.30 ms,
    // scaled to the current single sweep; no call plan isolates it, and at
    // 0.67 per sweep it is the dearest fused pass)
    static const double f32[] = {0.0, 1.0, 1.34, 1.281, 1.416, 1.634, 2.496};
    static const double f64[] = {0.0, 1.0, 0.896, 1.006, 1.192};
    return d.dtype == ST_F64 ? f64 : f32;
}

int launch_sweeps_fused(const stencil3d_desc &d, const void *in, void *out, int ns, int cus,
                        hipStream_t stream) {
    if (d.radius != 1 || ns < 2 || ns > fused_max_sweeps(d)) return ST_ERR_ARG;
    if (d.dtype == ST_F64) return launch_f64(d, in, out, ns, cus, stream);
    return launch_f32(d, in, out, ns, cus, stream);
}

}  // namespace st
