// wave2.hip -- instantiates and launches the two-step wave kernel of
// wave2_kernel.h (temporal blocking of the leapfrog).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "wave2_kernel.h"

namespace st {
namespace {

// fp32, every radius (R = 4: the 25-point wave step).  One 640-thread
// workgroup per compute unit, 4 x 1 points per thread (164 VGPRs at R = 4:
// up to three waves per SIMD); the extended tile is 64 x 40, the output
// tile 56 x 32.  The halo units wait in private LDS slots (PSTAGE), which
// leaves room for the vel2/eta ring and two stage-2 tile sets; thread rows
// are paired for conflict-free LDS access where the shape allows (PAIR,
// R = 4: 80-float rows, 146 KB).  Measured on the 1032^3 run (ms per step,
// before the per-round tile order of launch_t): 64 x 32 with R+1 full
// stage-1 tile sets 3.585, 64 x 40 as shipped 3.29-3.40 (box to box), 64 x 48
// with one stage-2 set 3.352; the shipped shape with that order: 3.03-3.08.
using Wave2F32 = Wave2Cfg<4, 1, 16, 40, 3, true, true, 2, true>;
// fp64: 2 x 1 points per thread (16-byte groups), same thread layout; the
// extended tile is 32 x 40, the output tile 24 x 32 at R = 4.
using Wave2F64 = Wave2Cfg<2, 1, 16, 40, 3, true, true, 2, true>;
// PML step (eta's 7-point coupling in both stages): the eta register ring
// and the two stages' eta tiles need more registers and LDS than three waves
// per SIMD leave, so 512 threads at two waves per SIMD over a 64 x 32
// extended tile (fp32; output tile 56 x 24 at R = 4) or 32 x 32 (fp64).
using Wave2F32Pml = Wave2Cfg<4, 1, 16, 32, 2, true, true, 2, true>;
using Wave2F64Pml = Wave2Cfg<2, 1, 16, 32, 2, true, true, 2, true>;

template <typename T, int R, class C, bool E7, bool SP>
int launch_t(const stencil3d_desc &d, int pw, const void *u_prev, const void *u, void *out1,
             void *out2, const void *vel2, const void *eta, double wscale,
             const Wave2Source &src, int cus, hipStream_t s) {
    using S = Wave2Shape<R, C, E7>;
    const int64_t ix = d.nx - 2 * R, iy = d.ny - 2 * R, iz = d.nz - 2 * R;
    const int tiles_x = (int)((ix + S::TX - 1) / S::TX);
    const int tiles_y = (int)((iy + S::TY - 1) / S::TY);
    const int64_t tiles = (int64_t)tiles_x * tiles_y;
    // chunks no shorter than about 8R planes: each costs 2R fill steps and
    // re-reads 4R planes of u^n
    const ChunkPlan p = plan_chunks(iz, tiles, 8 * R, cus > 0 ? cus : 256, S::PROLOGUE + 4);
    Wave2Args<T> g;
    g.s = make_args<T, R>(d, interior_box(d), u, out1, u_prev, vel2, eta, wscale, tiles_x, tiles_y,
                          (int)p.chunk_len, (int)p.nwg);
    g.s.pw = SP ? pw : 0;
    g.s.ga_nwg = (int)p.a_nwg;
    g.s.ga_tiles = (int)p.a_tiles;
    g.s.ga_len = (int)p.a_len;
    g.out2 = static_cast<T *>(out2);
    g.sx = src.on ? (int32_t)src.x : -1;
    g.sy = src.on ? (int32_t)src.y : -1;
    g.sz = src.on ? (int32_t)src.z : -1;
    g.s0 = (T)src.v0;
    g.s1 = (T)src.v1;
    // one workgroup per compute unit: the workgroups of a round run
    // together, and each XCD takes a contiguous range of every round's
    // tiles (rows of tiles, x fastest), so the 32 tiles an XCD streams at
    // once lie next to each other and next to the other XCDs' tiles of the
    // round.  Against a remap over the whole group (each XCD's tiles
    // contiguous over all rounds, the tiles of one round scattered in
    // strips), 1032^3 run, ms per step: plain pass 3.39 -> 3.08, PML pass
    // 3.97-4.14 -> 3.94.
    g.round = cus > 0 ? cus : 256;
    hipLaunchKernelGGL((wave2_kernel<T, R, C, E7, SP>), dim3((unsigned)p.nwg), dim3(C::NT), 0, s,
                       g);
    return hipGetLastError() == hipSuccess ? ST_OK : ST_ERR_LAUNCH;
}

// Data regions (pw > 0) for the plain step at R = 4 only, as for the
// single step.
template <typename T, class C, bool E7>
int launch_r(const stencil3d_desc &d, int pw, const void *u_prev, const void *u, void *out1,
             void *out2, const void *vel2, const void *eta, double wscale,
             const Wave2Source &src, int cus, hipStream_t s) {
    switch (d.radius) {
    case 1:
        return launch_t<T, 1, C, E7, false>(d, 0, u_prev, u, out1, out2, vel2, eta, wscale, src,
                                            cus, s);
    case 2:
        return launch_t<T, 2, C, E7, false>(d, 0, u_prev, u, out1, out2, vel2, eta, wscale, src,
                                            cus, s);
    case 3:
        return launch_t<T, 3, C, E7, false>(d, 0, u_prev, u, out1, out2, vel2, eta, wscale, src,
                                            cus, s);
    }
    if constexpr (!E7)
        if (pw > 0)
            return launch_t<T, 4, C, false, true>(d, pw, u_prev, u, out1, out2, vel2, eta, wscale,
                                                  src, cus, s);
    return launch_t<T, 4, C, E7, false>(d, 0, u_prev, u, out1, out2, vel2, eta, wscale, src, cus,
                                        s);
}

}  // namespace

bool wave2_available(const stencil3d_desc &d) { return d.radius >= 1 && d.radius <= 4; }

int launch_wave2(const stencil3d_desc &d, int pw, const void *u_prev, const void *u, void *out1,
                 void *out2, const void *vel2, const void *eta, double wscale,
                 const Wave2Source &src, int cus, hipStream_t stream, bool pml) {
    if (!wave2_available(d) || pw < 0) return ST_ERR_ARG;
    if (d.dtype == ST_F64)
        return pml ? launch_r<double, Wave2F64Pml, true>(d, pw, u_prev, u, out1, out2, vel2, eta,
                                                           wscale, src, cus, stream)
                   : launch_r<double, Wave2F64, false>(d, pw, u_prev, u, out1, out2, vel2, eta,
                                                         wscale, src, cus, stream);
    return pml ? launch_r<float, Wave2F32Pml, true>(d, pw, u_prev, u, out1, out2, vel2, eta,
                                                     wscale, src, cus, stream)
               : launch_r<float, Wave2F32, false>(d, pw, u_prev, u, out1, out2, vel2, eta, wscale,
                                                   src, cus, stream);
}

}  // namespace st
