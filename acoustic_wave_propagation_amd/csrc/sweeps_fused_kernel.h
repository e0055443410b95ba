// sweeps_fused_kernel.h -- NS Jacobi sweeps of the star stencil in one pass
// over HBM (temporal blocking), for the ping-pong entry point.
//
// The semi-stencil section of "Accelerating High-Order Stencils on GPUs"
// runs its time steps concurrently; the scheme here is this library's own:
// wavefront (pipelined) blocking in z combined with overlapped tiles in x
// and y, so each plane crosses HBM once per NS sweeps:
//
//  * A workgroup owns an output tile T of TX x TY points and a z chunk.  Its
//    threads cover the extended tile E = T grown by NS*R points on each side
//    (x rounded up to whole 16-byte groups).
//  * Stage s (s = 1..NS) computes sweep s on E at plane q_s = q_1 - (s-1) R,
//    one plane per z step: stage 1 reads the input through the same register
//    window as the single-sweep kernel; stage s > 1 reads sweep s-1, which
//    stage s-1 produced in earlier steps, from a register ring of 2R+1
//    planes.  In-plane neighbours of every stage come from LDS: at the start
//    of a step each thread writes the centre plane of every stage's input
//    into that stage's LDS tile (with two sets of tiles one barrier per step
//    suffices).
//  * Values are exact only where the dependency cone stays inside E: stage s
//    on E shrunk by s*R, so the last stage is exact on T, the only part
//    stored.  Points near the edge of E read stale LDS padding; their results
//    are never used by exact points.
//  * Non-interior points (the fixed Dirichlet boundary) keep their value in
//    every sweep: each stage selects the stencil result only on interior
//    points.  Points outside the array hold whatever the loads returned
//    (zeros past the allocation); interior points never read them.
//
// Per point and sweep the arithmetic is the same sequence of operations as
// in star2p5d_kernel, so a fused pass gives bit-identical results to NS
// single sweeps.  Each chunk reads NS*R extra planes at each end and its
// first 2(NS-1)R steps fill the pipeline.
#pragma once

#include "star2p5d_kernel.h"

namespace st {

// VX x VY points per thread, LX x LY threads covering the extended tile, D
// planes of input prefetch, LB sets of LDS tiles (2: one barrier per z step;
// 1: half the LDS, a second barrier before the tiles are rewritten),
// nontemporal stores.
//
// DENSE: the LDS layout of a tile.  The thread rows here are 34 or 36
// lanes, so a half-wave spans two of them; the LDS serves a half-wave's
// 16-byte accesses from a 512-byte bank window, and with padded rows the
// gap at a row boundary puts lanes on the same banks.  Dense: tile row t
// lies in plane t mod VY at row t / VY, rows EX elements apart with no
// padding, so the lanes of any access (all at the same row offset) touch
// one contiguous run.  The columns left and right of the extended tile
// then overlap the neighbouring rows' data: only edge points, which are
// never exact, read them.  Otherwise: padded rows of an odd number of
// 16-byte groups.
template <int VX_, int VY_, int LX_, int LY_, int D_ = 1, int LB_ = 2, bool NTS_ = true,
          bool DENSE_ = true>
struct FusedCfg {
    static constexpr int VX = VX_, VY = VY_, LX = LX_, LY = LY_, D = D_, LB = LB_;
    static constexpr bool NTS = NTS_, DENSE = DENSE_;
    static constexpr int NT = LX * LY, EX = LX * VX, EY = LY * VY;
};

template <int R, int NS, class C>
struct FusedShape {
    static constexpr int XE = (NS * R + C::VX - 1) / C::VX * C::VX;  // columns added per side
    static constexpr int YE = NS * R;                                 // rows added per side
    static constexpr int TX = C::EX - 2 * XE, TY = C::EY - 2 * YE;    // output tile
    static constexpr int W0 = 2 * R + 1 + C::D;  // input window slots
    static constexpr int WS = 2 * R + 1;         // ring slots of each intermediate sweep
    static constexpr int U = clcm(clcm(W0, WS), C::LB);  // z-loop unroll
    static constexpr int FILL = 2 * (NS - 1) * R;    // steps before the first output
    static constexpr int PROLOGUE = FILL + 2 * R + C::D;
};

template <typename T, int R, int NS, class C>
__global__ void __launch_bounds__(C::NT) sweeps_fused_kernel(StarArgs<T> a) {
    using FS = FusedShape<R, NS, C>;
    constexpr int VX = C::VX, VY = C::VY, LX = C::LX, D = C::D;
    constexpr int XE = FS::XE, YE = FS::YE, TX = FS::TX, TY = FS::TY;
    constexpr int W0 = FS::W0, WS = FS::WS, U = FS::U, FILL = FS::FILL;
    constexpr int XW = (R + VX - 1) / VX;  // padding groups left and right in LDS
    constexpr int PADL = XW * VX;
    constexpr int LP = lds_pitch<T>(PADL + C::EX + XW * VX, VX);
    constexpr int LROWS = C::EY + 2 * R;
    constexpr int PLANE = LROWS / VY * C::EX + 2 * PADL;  // DENSE: one plane
    constexpr int LTILE = C::DENSE ? VY * PLANE : LROWS * LP;
    static_assert(!C::DENSE || LROWS % VY == 0, "whole rows per plane");
    constexpr uint32_t ES = sizeof(T);
    constexpr int SAUX = C::NTS ? kAuxNT : 0;
    constexpr bool DIFF = std::is_same<T, double>::value;
    static_assert(NS >= 2, "at least two fused sweeps");
    static_assert(TX > 0 && TY > 0, "extended tile too small for NS sweeps");
    static_assert(XE % VX == 0, "whole groups of columns");
    static_assert(C::LB == 1 || C::LB == 2, "one or two sets of LDS tiles");

    __shared__ __align__(16) T lds[C::LB * NS * LTILE];

    const int tid = threadIdx.x;
    const int nx = a.nx, ny = a.ny, nz = a.nz;
    // this workgroup's tile and z chunk, mapped as for star2p5d_kernel
    // (chunk-major, XCD-remapped within each group)
    const int ntile = a.tiles_x * a.tiles_y;
    const WgWork w = wg_work((int)blockIdx.x, a.nwg, ntile, a.ga_nwg, a.ga_tiles, a.ga_len,
                             a.chunk_len, true, true);
    const int tyi = w.tile / a.tiles_x, txi = w.tile - tyi * a.tiles_x;
    const int gx0 = R + txi * TX, gy0 = R + tyi * TY;  // output tile origin
    const int zs = R + w.zoff;
    const int ze = min(zs + w.len, nz - R);
    const int n = ze - zs;                    // output planes of this chunk
    const int nsteps = n + FILL;
    const int q0 = zs - (NS - 1) * R;         // plane of stage 1 at step 0
    const uint32_t pzb = (uint32_t)(a.pz * (int64_t)ES);  // plane bytes (< 2^31)
    const bool xpart = gx0 + TX > nx - R;     // ragged x edge inside this tile

    // ---- this thread's points: columns ex..ex+VX-1 on rows ey..ey+VY-1 -----
    const int lx = tid % LX, ly = tid / LX;
    const int ex = gx0 - XE + lx * VX;
    const int ey = gy0 - YE + ly * VY;
    uint32_t loff[VY];  // load offsets (rows outside the array: kOOB)
    uint32_t soff[VY];  // store offsets (points outside T or the interior: kOOB)
    bool rin[VY];
    const bool tcol = lx * VX >= XE && lx * VX < XE + TX;
#pragma unroll
    for (int j = 0; j < VY; ++j) {
        const int y = ey + j;
        const int ty = ly * VY + j;
        rin[j] = y >= R && y < ny - R;
        // A group may start left of x = 0 (reads the previous row, or zeros
        // before the array) or end past x = nx; such points are outside the
        // array and only feed points that are outside the array too.
        loff[j] = (y >= 0 && y < ny) ? (uint32_t)((int64_t)y * nx + ex) * ES : kOOB;
        soff[j] = (tcol && ty >= YE && ty < YE + TY && rin[j] && ex < nx - R)
                      ? (uint32_t)((int64_t)y * nx + ex) * ES
                      : kOOB;
    }
    bool cin[VX];
#pragma unroll
    for (int i = 0; i < VX; ++i) cin[i] = ex + i >= R && ex + i < nx - R;
    const int nvx = max(0, min(VX, nx - R - ex));  // written columns (ragged x)
    const int lcol = lx * VX;
    const int lrow0 = R + ly * VY;
    // element of this thread's first column in tile row lrow0 + jr (jr >= -R)
    auto trow = [&](int jr) -> int {
        if constexpr (C::DENSE)
            return (R + jr) % VY * PLANE + PADL + (ly + (R + jr) / VY) * C::EX + lcol;
        else
            return (lrow0 + jr) * LP + PADL + lcol;
    };

    T w0[W0][VY][VX];             // input planes q_1-R .. q_1+R plus D in flight
    T ws[NS - 1][WS][VY][VX];     // sweeps 1..NS-1, 2R+1 planes each
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
#pragma unroll
        for (int p = 0; p < WS; ++p)
#pragma unroll
            for (int j = 0; j < VY; ++j)
#pragma unroll
                for (int i = 0; i < VX; ++i) ws[s][p][j][i] = T(0);

    // input plane q; only planes this chunk's outputs depend on are read
    auto in_rsrc = [&](int q) {
        const bool need = q >= 0 && q < nz && q >= zs - NS * R && q < ze + NS * R;
        return plane_rsrc(a.in, q, nz, pzb, need);
    };
    // prologue: window slot i holds the plane at step offset i - R
    static_for<0, 2 * R + D>([&](auto sc) {
        constexpr int sl = decltype(sc)::value;
        const rsrc_t r = in_rsrc(q0 + sl - R);
#pragma unroll
        for (int j = 0; j < VY; ++j) bload<T, VX>(r, loff[j], w0[sl][j]);
    });

    zsteps<U>(nsteps, [&](auto kc, const int k0) {
            constexpr int kk = decltype(kc)::value;
            constexpr int CS = (kk + R) % W0;          // window slot of plane q_1
            constexpr int LEAD = (kk + 2 * R + D) % W0;
            constexpr int SET = (kk % C::LB) * NS;     // LDS tile set of this step
            constexpr int CC = ((kk - R) % WS + WS) % WS;  // ring slot of a stage-s>1 centre
            const int k = k0 + kk;

            // 1. prefetch the input plane R+D above stage 1's plane
            {
                const rsrc_t r = in_rsrc(q0 + k + R + D);
#pragma unroll
                for (int j = 0; j < VY; ++j) bload<T, VX>(r, loff[j], w0[LEAD][j]);
            }

            // 2. centre plane of every stage's input into its LDS tile (with
            //    one set, after every thread has read last step's tiles)
            if constexpr (C::LB == 1) __syncthreads();
            static_for<0, NS>([&](auto sc) {
                constexpr int s = decltype(sc)::value;
                T *tile = lds + (SET + s) * LTILE;
#pragma unroll
                for (int j = 0; j < VY; ++j) {
                    if constexpr (s == 0)
                        lds_store_group<T, VX>(tile + trow(j), w0[CS][j]);
                    else
                        lds_store_group<T, VX>(tile + trow(j), ws[s - 1][CC][j]);
                }
            });
            __syncthreads();

            // 3. the stages in order; stage s+1 computes sweep s+1 at plane
            //    q_1 - s R from sweep s
            static_for<0, NS>([&](auto sc) {
                constexpr int s = decltype(sc)::value;
                const T *tile = lds + (SET + s) * LTILE;
                const int q = q0 + k - s * R;
                const bool zin = q >= R && q < nz - R;
                // value of sweep s at plane offset dz from the centre, own point
                auto zv = [&](auto dzc, int j, int i) -> T {
                    constexpr int dz = decltype(dzc)::value;
                    if constexpr (s == 0)
                        return w0[((CS + dz) % W0 + W0) % W0][j][i];
                    else
                        return ws[s - 1][((CC + dz) % WS + WS) % WS][j][i];
                };
                T xs[VY][VX + 2 * R];  // row segment, columns ex-R .. ex+VX+R-1
                // With R < VX only part of each neighbouring group is needed;
                // the whole groups are still read (one conflict-free 16-byte
                // access each) and kept alive until the stage's end, where an
                // empty asm statement uses them, so the loads are not narrowed
                // to the single elements (which, at a 16-byte lane stride,
                // would make lanes collide on LDS banks).
                T lg[VY][VX], rg[VY][VX];
#pragma unroll
                for (int j = 0; j < VY; ++j) {
                    const T *row = tile + trow(j);
                    if constexpr (R <= VX) {
                        lds_load_group<T, VX>(row - VX, lg[j]);
                        lds_load_group<T, VX>(row + VX, rg[j]);
#pragma unroll
                        for (int m = 0; m < R; ++m) {
                            xs[j][m] = lg[j][VX - R + m];
                            xs[j][R + VX + m] = rg[j][m];
                        }
                    } else {
#pragma unroll
                        for (int m = 0; m < R; ++m) {
                            xs[j][m] = row[m - R];
                            xs[j][R + VX + m] = row[VX + m];
                        }
                    }
#pragma unroll
                    for (int i = 0; i < VX; ++i) xs[j][R + i] = zv(std::integral_constant<int, 0>{}, j, i);
                }
                T ys[2 * R][VX];  // rows ey-R..ey-1 and ey+VY..ey+VY+R-1
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int i = 0; i < VX; ++i) {
                        ys[r][i] = tile[trow(r - R) + i];
                        ys[R + r][i] = tile[trow(VY + r) + i];
                    }
                T res[VY][VX];
#pragma unroll
                for (int j = 0; j < VY; ++j)
#pragma unroll
                    for (int i = 0; i < VX; ++i) {
                        const T ctr = zv(std::integral_constant<int, 0>{}, j, i);
                        T acc = (DIFF ? a.ccd : a.cc) * ctr;
                        static_for<1, R + 1>([&](auto kzc) {
                            constexpr int kz = decltype(kzc)::value;
                            const T zm = zv(std::integral_constant<int, -kz>{}, j, i);
                            const T zp = zv(std::integral_constant<int, kz>{}, j, i);
                            const T xm = xs[j][R + i - kz], xp = xs[j][R + i + kz];
                            const int qm = j - kz, qp = j + kz;
                            const T ym = qm < 0 ? ys[R + qm][i] : zv(std::integral_constant<int, 0>{}, qm < 0 ? 0 : qm, i);
                            const T yp = qp >= VY ? ys[R + qp - VY][i] : zv(std::integral_constant<int, 0>{}, qp >= VY ? 0 : qp, i);
                            if constexpr (DIFF) {
                                acc = fma(a.cz[kz - 1], (zm - ctr) + (zp - ctr), acc);
                                acc = fma(a.cy[kz - 1], (ym - ctr) + (yp - ctr), acc);
                                acc = fma(a.cx[kz - 1], (xm - ctr) + (xp - ctr), acc);
                            } else {
                                acc = fma(a.cz[kz - 1], zm + zp, acc);
                                acc = fma(a.cy[kz - 1], ym + yp, acc);
                                acc = fma(a.cx[kz - 1], xm + xp, acc);
                            }
                        });
                        // the boundary keeps its value in every sweep
                        res[j][i] = (zin && rin[j] && cin[i]) ? acc : ctr;
                    }
                if constexpr (R < VX) {
#pragma unroll
                    for (int j = 0; j < VY; ++j)
#pragma unroll
                        for (int i = 0; i < VX; ++i) asm volatile("" ::"v"(lg[j][i]), "v"(rg[j][i]));
                }

                if constexpr (s < NS - 1) {
#pragma unroll
                    for (int j = 0; j < VY; ++j)
#pragma unroll
                        for (int i = 0; i < VX; ++i) ws[s][kk % WS][j][i] = res[j][i];
                } else {
                    // 4. last sweep: store T's interior points of plane q
                    const bool st = k >= FILL && k < nsteps;
                    const rsrc_t ro = plane_rsrc(a.out, q, nz, pzb, st);
                    if (!xpart) {
#pragma unroll
                        for (int j = 0; j < VY; ++j) bstore<T, VX, SAUX>(ro, soff[j], res[j]);
                    } else {
                        // whole groups in one access, the partial group of a
                        // row element by element (as in star2p5d_kernel)
#pragma unroll
                        for (int j = 0; j < VY; ++j) {
                            bstore<T, VX, SAUX>(ro, nvx == VX ? soff[j] : kOOB, res[j]);
#pragma unroll
                            for (int i = 0; i < VX - 1; ++i)
                                bstore1<T>(ro, i < nvx && nvx < VX ? soff[j] + i * ES : kOOB,
                                           res[j][i]);
                        }
                    }
                }
            });
    });
}

}  // namespace st
