// wave2_kernel.h -- two leapfrog steps of the acoustic wave update in one
// pass over HBM (temporal blocking of the wave step).
//
// The semi-stencil section of "Accelerating High-Order Stencils on GPUs"
// runs its time steps concurrently; the scheme here is this library's own:
// it pipelines two steps in z over overlapped tiles in x and y, so each
// plane crosses HBM once per two steps:
//
//  * A workgroup owns an output tile T of TX x TY points and a z chunk; its
//    threads cover the extended tile E = T grown by R points on each side
//    (x in whole 16-byte groups).
//  * Stage 1, at plane q1 = q0 + k in z step k, computes step n+1 on all of
//    E: u^n's z neighbours from a register window (as in star2p5d_kernel),
//    its in-plane neighbours from an LDS tile of E plus an R-wide halo ring.
//    The ring of each plane is loaded in the step in which the neighbouring
//    tiles load that plane as their window's leading plane (so it comes from
//    L2) and waits until its step comes: each 16-byte unit in LDS slots
//    private to the thread that loaded it, placed into a double-buffered
//    tile one step ahead (PSTAGE), or the whole ring in one of R+D tile sets.
//  * Stage 2, at plane q2 = q1 - R, computes step n+2 on E (exact on T):
//    z neighbours of u^{n+1} from a register ring that stage 1 filled over
//    the last 2R steps, in-plane neighbours from a second LDS tile.  u^n at
//    q2 is still in stage 1's window; vel2 and eta at q2 were loaded by
//    stage 1 R steps earlier and wait in an LDS ring private to each thread
//    (threads with points in T only).  Two sets of each tile leave one
//    barrier per z step.
//  * Stage 1's result is stored on T (u^{n+1}, the next pass's u_prev) and
//    stage 2's (u^{n+2}).  Both outputs go to buffers no tile reads in the
//    pass: neighbouring tiles read u^{n-1} and u^n on their extended tiles.
//  * Points outside the interior keep u^n's value in step n+1 (the halos of
//    all u fields are the same, zero for the leapfrog), so stage 2 sees the
//    halo stage 1 would have seen in the next single step.
//  * The point source of each step is added to that step's result at the
//    source point, as the run's separate source kernel does.
//
// Per point and step the arithmetic is the same sequence of operations as
// in star2p5d_kernel's wave step, so a pass gives bit-identical results to
// two single steps (not in place) with their sources.
#pragma once

#include "star2p5d_kernel.h"

namespace st {

template <typename T>
struct Wave2Args {
    StarArgs<T> s;         // in = u^n, u_prev = u^{n-1}, out = u^{n+1}; weights carry dt^2/h^2
    T *out2;               // u^{n+2}
    int32_t sx, sy, sz;    // source point (allocated coordinates); sz = -1: no source
    T s0, s1;              // source values of steps n+1 and n+2
    int32_t round;         // workgroups per round for xcd_remap_rounds (0: whole groups)
};

// VX x VY points per thread, LX x LY threads covering the extended tile,
// minimum waves per SIMD the register allocation must allow, and where
// stage 2 takes vel2 and eta from: an LDS ring that stage 1 fills (VRING)
// or a second load from memory (L2 or the Infinity Cache: the workgroup
// read those planes R steps earlier).
//
// PSTAGE: each halo unit waits its R+D steps in LDS slots private to the
// thread that loads it (16 bytes each) and is placed into a double-buffered
// stage-1 tile one step ahead, instead of waiting in R+D full tile sets.
// T2S: stage-2 tile sets (2: one barrier per z step; 1: two).
//
// PAIR: which tile rows the two 16-lane thread rows of a half-wave take.
// The LDS serves a half-wave's 16-byte accesses from a 512-byte window of
// banks (measured: 32-lane tile rows run free of bank conflicts, 16-lane
// rows 304 bytes apart lose ~40% of LDS cycles to them), so the two rows'
// 256-byte runs must lie 256 bytes apart modulo 512.  With a row pitch of
// 4 mod 8 16-byte groups that holds for rows 4 (and 36, 44) apart: output
// rows are paired 4 apart in blocks of 8, the R rows above the output tile
// with the R rows below it (whole waves, which skip stage 2), and the halo
// rows above with those below.  Shapes the pairing does not tile keep the
// plain row order.
template <int VX_, int VY_, int LX_, int LY_, int MINW_, bool VRING_ = true,
          bool PSTAGE_ = false, int T2S_ = 2, bool PAIR_ = false>
struct Wave2Cfg {
    static constexpr int VX = VX_, VY = VY_, LX = LX_, LY = LY_, MINW = MINW_;
    static constexpr bool VRING = VRING_, PSTAGE = PSTAGE_, PAIR = PAIR_;
    static constexpr int T2S = T2S_;
    static constexpr int NT = LX * LY, EX = LX * VX, EY = LY * VY;
};

template <int R, class C, bool E7 = false>
struct Wave2Shape {
    static constexpr int D = 1;                      // window prefetch (planes)
    static constexpr int XE = round_up(R, C::VX);    // columns added per side
    static constexpr int YE = R;                     // rows added per side
    static constexpr int TX = C::EX - 2 * XE, TY = C::EY - 2 * YE;  // output tile
    static constexpr int W0 = 2 * R + 1 + D;         // u^n window slots
    static constexpr int LB = R + D;                 // steps a halo ring waits: stage-1
                                                     // tile sets, or staging slots (PSTAGE)
    static constexpr int U = clcm(clcm(W0, LB), 2);  // z-loop unroll
    static constexpr int WS = ring_fit(U, 2 * R + 1);  // u^{n+1} ring slots
    static constexpr int NV = ring_fit(U, R + 1);      // vel2/eta ring slots
    static constexpr int FILL = 2 * R;               // steps before the first u^{n+2} plane
    static constexpr int PROLOGUE = FILL + 2 * R + D;
    // PML step: eta planes q1+1 down to min(q1-1, q2+1) in registers (the
    // ring padded to divide the unroll); plane q1+d sits in slot
    // (k + d + EOFF) mod NE in step k
    static constexpr int EOFF = R - 1 > 1 ? R - 1 : 1;
    static constexpr int NE = E7 ? ring_fit(U, EOFF + 2) : 1;
};

// E7: two steps of the PML kernel's update (wave_step_pml): each stage adds
// the eta-gradient coupling sum_a (eta(p+e_a) - eta(p-e_a)) (u(p+e_a) -
// u(p-e_a)) / (4 h^2) of its own step, with the operations of
// star2p5d_kernel's PML step in the same order.  eta of plane q1+1 is loaded
// in step k with the epilogue fields into a register ring of the planes
// q1+1 .. q2+1.  Stage 1 takes eta's z neighbours from that ring and its
// in-plane neighbours from an eta tile of plane q1 on E plus the 1-wide ring
// around E (loaded one step ahead; two sets).  Each step also writes eta of
// plane q2+1 on E into one of four stage-2 eta tiles, so stage 2 finds
// planes q2-1, q2 and q2+1 in LDS (T's ring lies inside E).
//
// SP (data regions, plain step): the caller guarantees eta = 0 at every
// interior point at least pw from all interior faces; stage 1 then loads
// eta of its points by the rule of star2p5d_kernel's data regions, applied
// to E's points: in every plane on rows within pw of a y face and on
// columns within pw of an x face or of a multiple of two output-tile widths
// (with E's XE extra columns per side, pw + XE of E's columns in every tile
// away from the x faces), elsewhere only in the planes within pw of a z
// face.  A load that is skipped returns the zero it would have read.
// Stage 2 takes eta from the ring stage 1 fills.
template <typename T, int R, class C, bool E7 = false, bool SP = false>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::MINW)))
    wave2_kernel(Wave2Args<T> g) {
    using S = Wave2Shape<R, C, E7>;
    const StarArgs<T> &a = g.s;
    constexpr int VX = C::VX, VY = C::VY, LX = C::LX, NT = C::NT, EX = C::EX, EY = C::EY;
    constexpr int D = S::D, XE = S::XE, YE = S::YE, TX = S::TX, TY = S::TY;
    constexpr int W0 = S::W0, LB = S::LB, U = S::U, WS = S::WS, NV = S::NV;
    constexpr int XW = (R + VX - 1) / VX;  // halo groups left and right
    constexpr int PADL = XW * VX;          // LDS column of extended-tile x = 0
    // row pairing where the shape allows it (else the plain row order)
    constexpr int PPG = pair_pitch<T>(PADL + EX + XW * VX, VX) * (int)sizeof(T) / 16;
    constexpr bool PAIR = C::PAIR && LX == 16 && VY == 1 && (2 * R) % 4 == 0 &&
                          (EY - 2 * R) % 8 == 0 && (4 * PPG) % 32 == 16 &&
                          ((EY - R) * PPG) % 32 == 16 && ((EY + R) * PPG) % 32 == 16;
    constexpr int LP = PAIR ? pair_pitch<T>(PADL + EX + XW * VX, VX)
                            : lds_pitch<T>(PADL + EX + XW * VX, VX);
    constexpr int LTILE = (EY + 2 * R) * LP;
    constexpr int NYU = 2 * R * LX;        // halo units above and below E
    constexpr int NXU = 2 * EY * XW;       // left and right of E
    constexpr int NTT = (TX / VX) * (TY / VY);  // threads whose points lie in T
    constexpr int S1 = C::PSTAGE ? 2 : LB;      // stage-1 tile sets
    constexpr int T2S = C::T2S;                 // stage-2 tile sets
    constexpr int NE = S::NE;                   // eta register ring (PML step)
    // the vel2/eta ring of stage 2 holds vel2 only in the PML step (stage 2
    // takes eta from the register ring)
    constexpr int NVF = E7 ? 1 : 2;
    constexpr int VBASE = (S1 + T2S) * LTILE;
    constexpr int SBASE = VBASE + (C::VRING ? NV * NVF * VY * NTT * VX : 0);
    constexpr int NU = NYU + NXU;               // halo units
    constexpr int LDUMMY = SBASE + (C::PSTAGE ? LB * NU * VX : 0);
    // PML step: eta tiles, rows -1 .. EY of E with u's pitch and columns
    // (2 stage-1 sets, 4 stage-2 sets), then their sink; eta ring units:
    // the rows above and below E (LX groups each) and the group left and
    // right of every row of E
    constexpr int ETILE = E7 ? (EY + 2) * LP : 0;
    constexpr int EBASE = LDUMMY + VX;
    constexpr int EDUMMY = EBASE + 6 * ETILE;
    constexpr int NEU = 2 * LX + 2 * EY;
    constexpr uint32_t ES = sizeof(T);
    constexpr bool DIFF = std::is_same<T, double>::value;
    static_assert(TX > 0 && TY > 0, "extended tile too small");
    static_assert(NYU + NXU <= NT, "one halo unit per thread at most");
    static_assert(WS >= 2 * R + 1 && NV >= R + 1 && U % WS == 0 && U % NV == 0, "rings");
    static_assert(D == 1, "the halo ring shares the window's leading load");
    static_assert(XE % VX == 0 && YE % VY == 0 && TY % VY == 0, "whole threads in T");
    static_assert(64 % LX == 0, "a wave covers whole thread rows");
    static_assert(T2S == 1 || T2S == 2, "one or two stage-2 tile sets");
    static_assert(!(SP && E7), "data regions: the plain step's pass only");
    static_assert(!E7 || (NE >= S::EOFF + 2 && U % NE == 0 && NEU <= NT && VY == 1),
                  "PML step: eta ring, one eta unit per thread, one row per thread");

    __shared__ __align__(16) T lds[E7 ? EDUMMY + VX : LDUMMY + VX];
    T *const tile2 = lds + S1 * LTILE;     // stage 2: u^{n+1} at q2

    const int tid = threadIdx.x;
    const int nx = a.nx, ny = a.ny, nz = a.nz;
    const int ntile = a.tiles_x * a.tiles_y;
    const WgWork w = wg_work((int)blockIdx.x, a.nwg, ntile, a.ga_nwg, a.ga_tiles, a.ga_len,
                             a.chunk_len, true, true, g.round);
    const int tyi = w.tile / a.tiles_x, txi = w.tile - tyi * a.tiles_x;
    const int gx0 = R + txi * TX, gy0 = R + tyi * TY;  // output tile origin
    const int zs = R + w.zoff;
    const int ze = min(zs + w.len, nz - R);
    const int n = ze - zs;                    // output planes of this chunk
    const int nsteps = n + S::FILL;
    const int q0 = zs - R;                    // stage-1 plane of step 0
    const uint32_t pzb = (uint32_t)(a.pz * (int64_t)ES);  // plane bytes (< 2^31)
    const bool xpart = gx0 + TX > nx - R;     // ragged x edge inside this tile

    // ---- this thread's points: columns ex..ex+VX-1 on rows ey..ey+VY-1 -----
    // thread row slot -> tile row (PAIR: see the configuration)
    const int slot = tid / LX;
    auto row_of = [&](int sl) -> int {
        if (!PAIR) return sl;
        if (sl < 2 * R) return (sl & 1) ? EY - R + (sl >> 1) : (sl >> 1);
        const int t = sl - 2 * R, b = t >> 3, r = t & 7;
        return R + 8 * b + (r >> 1) + (r & 1) * 4;
    };
    const int lx = tid % LX, ly = row_of(slot);
    const int ex0 = gx0 - XE, ey0 = gy0 - YE;  // extended tile origin
    const int ex = ex0 + lx * VX, ey = ey0 + ly * VY;
    auto off_of = [&](int y, int x) -> uint32_t {
        // rows outside the array: kOOB; a group left of x = 0 reads the end
        // of the previous row (or, before the array, zeros): values only
        // points outside the interior use
        return (y >= 0 && y < ny) ? (uint32_t)(((int64_t)y * nx + x) * ES) : kOOB;
    };
    uint32_t loff[VY], soff[VY];
    bool rin[VY];
    const bool tcol = lx * VX >= XE && lx * VX < XE + TX;
#pragma unroll
    for (int j = 0; j < VY; ++j) {
        const int y = ey + j, ty = ly * VY + j;
        rin[j] = y >= R && y < ny - R;
        loff[j] = off_of(y, ex);
        soff[j] = (tcol && ty >= YE && ty < YE + TY && rin[j] && ex < nx - R) ? loff[j] : kOOB;
    }
    // SP: bit j of emask says whether row j reads eta in planes away from
    // the z faces
    uint32_t emask = 0;
    const int elo = R + a.pw;  // first x (y, z) at least pw inside the interior
    if constexpr (SP) {
        const int m = (ex - R) % (2 * TX);  // interior x modulo two output tiles (if ex >= elo)
        const bool cols = ex < elo || ex + VX > nx - elo || m < a.pw || m + VX > 2 * TX - a.pw;
#pragma unroll
        for (int j = 0; j < VY; ++j)
            emask |= (cols || ey + j < elo || ey + j >= ny - elo) ? 1u << j : 0u;
    }
    bool cin[VX];
#pragma unroll
    for (int i = 0; i < VX; ++i) cin[i] = ex + i >= R && ex + i < nx - R;
    const int nvx = max(0, min(VX, nx - R - ex));  // written columns (ragged x)
    const int lcol = PADL + lx * VX;
    const int lrow0 = R + ly * VY;
    // source point among this thread's points (column and row index, or -1)
    int si = -1, sj = -1;
    if (g.sz >= 0 && g.sx >= ex && g.sx < ex + VX && g.sy >= ey && g.sy < ey + VY) {
        si = g.sx - ex;
        sj = g.sy - ey;
    }

    // ---- halo ring unit of this thread (stage-1 tile) ------------------------
    uint32_t h_off = kOOB;
    int h_l = -1;
    if (tid < NYU) {
        const int u = tid / LX, gi = tid - u * LX;
        // row of the ring: 0..R-1 above the tile, R..2R-1 below (PAIR: the
        // two rows of a half-wave are the i-th above and the i-th below)
        const int rsel = PAIR ? ((u & 1) ? R + (u >> 1) : (u >> 1)) : u;
        const int gy = rsel < R ? ey0 - R + rsel : ey0 + EY + (rsel - R);
        h_off = off_of(gy, ex0 + gi * VX);
        h_l = (rsel < R ? rsel : EY + rsel) * LP + PADL + gi * VX;
    } else if (tid < NYU + NXU) {
        const int xu = tid - NYU;
        const int side = xu / (EY * XW), rem = xu - side * (EY * XW);
        const int row = rem / XW, c = rem - row * XW;
        h_off = off_of(ey0 + row, side ? ex0 + EX + c * VX : ex0 - PADL + c * VX);
        h_l = (R + row) * LP + (side ? PADL + EX : 0) + c * VX;
    }
    T *const h_dst = h_l >= 0 ? lds + h_l : lds + LDUMMY;  // + set * LTILE (inactive: sink)
    const int h_set_stride = h_l >= 0 ? LTILE : 0;
    // private staging slot s of this thread's halo unit (PSTAGE)
    T *const h_stage = h_l >= 0 ? lds + SBASE + tid * VX : lds + LDUMMY;
    const int h_stage_stride = h_l >= 0 ? NU * VX : 0;
    // this thread's slot of the vel2/eta ring: ring slot s, field f, row j
    // (threads with points in T only)
    const bool tthr = tcol && ly * VY >= YE && ly * VY < YE + TY;
    const int tt = (PAIR ? slot - 2 * R : ly - YE / VY) * (TX / VX) + (lx - XE / VX);
    // whether this thread's wave has a row in T (uniform over the wave)
    const int wrow0 = __builtin_amdgcn_readfirstlane(tid / 64) * 64 / LX * VY;
    const bool wave_in_t = PAIR ? wrow0 + 64 / LX - 1 >= 2 * R
                                   : wrow0 < YE + TY && wrow0 + 64 / LX * VY > YE;
    auto vring = [&](int s, int f, int j) {
        return lds + VBASE + (((s * NVF + f) * VY + j) * NTT + tt) * VX;
    };
    // PML step: this thread's eta ring unit (plane q1 of the next step) and
    // its place in the stage-1 eta tile
    uint32_t eh_off = kOOB;
    int eh_l = -1;
    if (E7 && tid < NEU) {
        if (tid < 2 * LX) {
            const int side = tid / LX, gi = tid - side * LX;
            eh_off = off_of(side ? ey0 + EY : ey0 - 1, ex0 + gi * VX);
            eh_l = (side ? EY + 1 : 0) * LP + PADL + gi * VX;
        } else {
            // the group ending at column ex0-1, or starting at ex0+EX
            const int xu = tid - 2 * LX, side = xu / EY, row = xu - side * EY;
            eh_off = off_of(ey0 + row, side ? ex0 + EX : ex0 - VX);
            eh_l = (1 + row) * LP + (side ? PADL + EX : PADL - VX);
        }
    }
    T *const eh_dst = eh_l >= 0 ? lds + EBASE + eh_l : lds + EDUMMY;
    const int eh_set_stride = eh_l >= 0 ? ETILE : 0;

    T w0[W0][VY][VX];  // u^n, planes q1-R .. q1+R plus D in flight
    T ws[WS][VY][VX];  // u^{n+1}, the last WS stage-1 planes
    T up[VY][VX], v2[VY][VX], et[VY][VX];  // u^{n-1}, vel2, eta at q1
    T hs[2][VX];       // halo unit in flight
    // PML step: eta plane q1 + d in slot (k + d + EOFF) mod NE, and the eta
    // ring unit of plane q1 in slot k mod 2
    T ew[NE][VY][VX];
    T ehs[2][VX];
#pragma unroll
    for (int p = 0; p < WS; ++p)
#pragma unroll
        for (int j = 0; j < VY; ++j)
#pragma unroll
            for (int i = 0; i < VX; ++i) ws[p][j][i] = T(0);
#pragma unroll
    for (int p = 0; p < NE; ++p)
#pragma unroll
        for (int j = 0; j < VY; ++j)
#pragma unroll
            for (int i = 0; i < VX; ++i) ew[p][j][i] = T(0);

    auto prsrc = [&](const T *base, int q, bool need) {
        return plane_rsrc(base, q, nz, pzb, need && q >= 0 && q < nz);
    };
    // u^n planes this chunk depends on
    auto u_need = [&](int q) { return q >= zs - 2 * R && q < ze + 2 * R; };

    // prologue: window slot s holds the plane at step offset s - R; the halo
    // units of steps 0..LB-2 go to their tile sets (PSTAGE: step 0's to its
    // tile, the others to their private slots), step LB-1's waits in hs[1]
    // (stored in step 0)
    static_for<0, 2 * R + D>([&](auto sc) {
        constexpr int sl = decltype(sc)::value;
        const int q = q0 + sl - R;
        const rsrc_t r = prsrc(a.in, q, u_need(q));
#pragma unroll
        for (int j = 0; j < VY; ++j) bload<T, VX>(r, loff[j], w0[sl][j]);
    });
    if constexpr (E7) {
        static_for<0, 2>([&](auto dc) {
            constexpr int d = decltype(dc)::value - 1;  // planes q0-1, q0
            const rsrc_t r = prsrc(a.eta, q0 + d, true);
#pragma unroll
            for (int j = 0; j < VY; ++j) bload<T, VX>(r, loff[j], ew[(d + S::EOFF) % NE][j]);
        });
        bload<T, VX>(prsrc(a.eta, q0, true), eh_off, ehs[0]);
    }
    {
        T hp[LB - 1][VX];
        static_for<0, LB - 1>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            bload<T, VX>(prsrc(a.in, q0 + h, u_need(q0 + h)), h_off, hp[h]);
        });
        bload<T, VX>(prsrc(a.in, q0 + LB - 1, u_need(q0 + LB - 1)), h_off, hs[1]);
        static_for<0, LB - 1>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            if constexpr (C::PSTAGE) {
                // step 0's unit straight into its tile, the others staged
                if constexpr (h == 0)
                    lds_store_group<T, VX>(h_dst, hp[h]);
                else
                    lds_store_group<T, VX>(h_stage + h * h_stage_stride, hp[h]);
            } else {
                lds_store_group<T, VX>(h_dst + h * h_set_stride, hp[h]);
            }
        });
    }

    // in-plane and z sums of one stage: the same operations, in the same
    // order, as star2p5d_kernel; zv(dz, j, i) is the stage input at plane
    // offset dz of the thread's own point (j, i).  coupling(j, i, u(x-1),
    // u(x+1), u(y-1), u(y+1), u(z-1), u(z+1), acc) returns the sum with the
    // PML step's eta-gradient term added (the plain step passes acc through)
    auto laplacian = [&](const T *tile, auto zv, T (&acc_out)[VY][VX], auto coupling) {
        T xs[VY][VX + 2 * R];  // row segment, columns ex-R .. ex+VX+R-1
        T lg[VY][VX], rg[VY][VX];
#pragma unroll
        for (int j = 0; j < VY; ++j) {
            const T *row = tile + (lrow0 + j) * LP + lcol;
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
                ys[r][i] = tile[(lrow0 - R + r) * LP + lcol + i];
                ys[R + r][i] = tile[(lrow0 + VY + r) * LP + lcol + i];
            }
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
                    const T ym = qm < 0 ? ys[R + qm][i]
                                        : zv(std::integral_constant<int, 0>{}, qm < 0 ? 0 : qm, i);
                    const T yp = qp >= VY ? ys[R + qp - VY][i]
                                          : zv(std::integral_constant<int, 0>{}, qp >= VY ? 0 : qp, i);
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
                acc_out[j][i] = coupling(
                    j, i, xs[j][R + i - 1], xs[j][R + i + 1],
                    j > 0 ? zv(std::integral_constant<int, 0>{}, j > 0 ? j - 1 : 0, i) : ys[R - 1][i],
                    j + 1 < VY ? zv(std::integral_constant<int, 0>{}, j + 1 < VY ? j + 1 : 0, i)
                               : ys[R][i],
                    zv(std::integral_constant<int, -1>{}, j, i),
                    zv(std::integral_constant<int, 1>{}, j, i), acc);
            }
        if constexpr (R < VX) {
#pragma unroll
            for (int j = 0; j < VY; ++j)
#pragma unroll
                for (int i = 0; i < VX; ++i) asm volatile("" ::"v"(lg[j][i]), "v"(rg[j][i]));
        }
    };
    // T's interior points of plane q (ragged x: whole groups in one access,
    // the partial group of a row element by element)
    auto store = [&](T *base, int q, bool st, const T (&res)[VY][VX]) {
        const rsrc_t ro = prsrc(base, q, st);
        if (!xpart) {
#pragma unroll
            for (int j = 0; j < VY; ++j) bstore<T, VX>(ro, soff[j], res[j]);
        } else {
#pragma unroll
            for (int j = 0; j < VY; ++j) {
                bstore<T, VX>(ro, nvx == VX ? soff[j] : kOOB, res[j]);
#pragma unroll
                for (int i = 0; i < VX - 1; ++i)
                    bstore1<T>(ro, i < nvx && nvx < VX ? soff[j] + i * ES : kOOB, res[j][i]);
            }
        }
    };

    zsteps<U>(nsteps, [&](auto kc, const int k0) {
            constexpr int kk = decltype(kc)::value;
            constexpr int CS = (kk + R) % W0;            // window slot of plane q1
            constexpr int LEAD = (kk + 2 * R + D) % W0;  // slot the prefetch fills
            constexpr int C2 = kk % W0;                  // window slot of plane q2 = q1 - R
            constexpr int SET = kk % LB;                 // stage-1 tile set of this step
            constexpr int HSET = (kk + LB - 1) % LB;     // set whose halo is stored now
            constexpr int HLD = kk % 2, HST = (kk + 1) % 2;
            constexpr int WC = kk % WS;                  // ring slot of plane q1
            constexpr int WC2 = ((kk - R) % WS + WS) % WS;  // ring slot of plane q2
            constexpr int VW = kk % NV, VR = ((kk - R) % NV + NV) % NV;
            constexpr int T2 = kk % T2S;                 // stage-2 tile set
            constexpr int S1SET = kk % S1;               // stage-1 tile set
            constexpr int NXT = (kk + 1) % LB;           // staging slot of step k+1
            // PML step: eta ring slots of planes q1-1, q1, q1+1 and q2+1;
            // stage-1 eta tile set
            constexpr int EO = S::EOFF;
            constexpr int EM1 = (kk + EO - 1) % NE, EC1 = (kk + EO) % NE, EP1 = (kk + EO + 1) % NE;
            constexpr int EW2 = (kk + EO + 1 - R) % NE;
            constexpr int ES1 = kk % 2;
            const int k = k0 + kk;
            // stage-2 eta tile sets of planes q2+1 (written now), q2, q2-1
            T *const e2p = lds + EBASE + (2 + (k & 3)) * ETILE;
            T *const e2c = lds + EBASE + (2 + ((k + 3) & 3)) * ETILE;
            T *const e2m = lds + EBASE + (2 + ((k + 2) & 3)) * ETILE;
            const int q1 = q0 + k, q2 = q1 - R;
            const bool in1 = q1 >= R && q1 < nz - R;
            T v2b[VY][VX] = {}, etb[VY][VX] = {};  // vel2, eta at q2 (stage 2)

            // 1. stage 1's epilogue fields of plane q1 first (used at the
            //    end of this step), then the window's leading plane and the
            //    halo ring of step k + LB -- the same plane (D = 1)
            {
                const bool need = in1 && k < nsteps;
                const rsrc_t rp = prsrc(a.u_prev, q1, need), rv = prsrc(a.vel2, q1, need);
#pragma unroll
                for (int j = 0; j < VY; ++j) {
                    bload<T, VX>(rp, loff[j], up[j]);
                    bload<T, VX>(rv, loff[j], v2[j]);
                }
                if constexpr (E7) {
                    // eta of plane q1+1 (stage 1's z neighbour now, the centre
                    // next step) and its ring units (next step's eta tile)
                    const rsrc_t re = prsrc(a.eta, q1 + 1, k < nsteps);
#pragma unroll
                    for (int j = 0; j < VY; ++j) bload<T, VX>(re, loff[j], ew[EP1][j]);
                    bload<T, VX>(re, eh_off, ehs[(kk + 1) % 2]);
                } else {
                    const rsrc_t re = prsrc(a.eta, q1, need);
                    const bool zf = !SP || q1 < elo || q1 >= nz - elo;  // near a z face
#pragma unroll
                    for (int j = 0; j < VY; ++j)
                        bload<T, VX>(re, (zf || ((emask >> j) & 1u)) ? loff[j] : kOOB, et[j]);
                }
            }
            if constexpr (!C::VRING) {
                // stage 2's vel2 and eta of plane q2 (threads with points in T;
                // the PML step keeps eta in its register ring)
                const bool need = q2 >= R && q2 < nz - R;
                const rsrc_t rv = prsrc(a.vel2, q2, need), re = prsrc(a.eta, q2, need && !E7);
#pragma unroll
                for (int j = 0; j < VY; ++j) {
                    bload<T, VX>(rv, tthr ? loff[j] : kOOB, v2b[j]);
                    bload<T, VX>(re, tthr ? loff[j] : kOOB, etb[j]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            {
                const int q = q1 + R + D;
                const rsrc_t r = prsrc(a.in, q, u_need(q));
#pragma unroll
                for (int j = 0; j < VY; ++j) bload<T, VX>(r, loff[j], w0[LEAD][j]);
                bload<T, VX>(r, h_off, hs[HLD]);
            }

            // 2. centre rows of both tiles of this step (a stage-1 set is
            //    rewritten S1 steps after its last read, a stage-2 set T2S
            //    steps after; with one stage-2 set, wait for every thread)
            if constexpr (T2S == 1) __syncthreads();
#pragma unroll
            for (int j = 0; j < VY; ++j) {
                lds_store_group<T, VX>(lds + S1SET * LTILE + (lrow0 + j) * LP + lcol, w0[CS][j]);
                lds_store_group<T, VX>(tile2 + T2 * LTILE + (lrow0 + j) * LP + lcol, ws[WC2][j]);
            }
            if constexpr (E7) {
                // eta of plane q1 (own points and the ring) into stage 1's
                // eta tile, eta of plane q2+1 (own points) into a stage-2 one
#pragma unroll
                for (int j = 0; j < VY; ++j) {
                    lds_store_group<T, VX>(lds + EBASE + ES1 * ETILE + (1 + ly * VY + j) * LP + lcol,
                                           ew[EC1][j]);
                    lds_store_group<T, VX>(e2p + (1 + ly * VY + j) * LP + lcol, ew[EW2][j]);
                }
                lds_store_group<T, VX>(eh_dst + ES1 * eh_set_stride, ehs[kk % 2]);
            }
            __syncthreads();
            if constexpr (!C::PSTAGE) {
                // halo ring of step k + LB - 1 into its set, last read in
                // step k-1
                lds_store_group<T, VX>(h_dst + HSET * h_set_stride, hs[HST]);
            } else if (h_l >= 0) {
                // the halo unit of step k + LB - 1 into its private slot;
                // step k+1's from its slot into the other tile set, last
                // read in step k-1 (threads without a unit skip this: many
                // lanes reading one sink address are served one by one)
                lds_store_group<T, VX>(h_stage + HSET * h_stage_stride, hs[HST]);
                T hv[VX];
                lds_load_group<T, VX>(h_stage + NXT * h_stage_stride, hv);
                lds_store_group<T, VX>(h_dst + (S1SET ^ 1) * h_set_stride, hv);
            }

            // eta-gradient coupling of a stage (PML step): eta of the stage's
            // plane at the thread's points in ec, of the planes below and
            // above in em / ep, in-plane neighbours outside the thread's
            // points from the eta tile etl
            auto coupling = [&](const T(&ec)[VY][VX], const T(&em)[VY][VX], const T(&ep)[VY][VX],
                                const T *etl) {
                return [&, etl](int j, int i, T uxm, T uxp, T uym, T uyp, T uzm, T uzp,
                                T acc) -> T {
                    if constexpr (!E7) {
                        return acc;
                    } else {
                        const int er = 1 + ly * VY + j;
                        const T exm = i > 0 ? ec[j][i > 0 ? i - 1 : 0] : etl[er * LP + lcol - 1];
                        const T exp1 =
                            i + 1 < VX ? ec[j][i + 1 < VX ? i + 1 : 0] : etl[er * LP + lcol + VX];
                        const T eym = j > 0 ? ec[j > 0 ? j - 1 : 0][i] : etl[(er - 1) * LP + lcol + i];
                        const T eyp =
                            j + 1 < VY ? ec[j + 1 < VY ? j + 1 : 0][i] : etl[(er + 1) * LP + lcol + i];
                        T gg = (exp1 - exm) * (uxp - uxm);
                        gg = fma(eyp - eym, uyp - uym, gg);
                        gg = fma(ep[j][i] - em[j][i], uzp - uzm, gg);
                        return fma(a.gw, gg, acc);
                    }
                };
            };

            // 3. stage 1: step n+1 at plane q1 on E
            {
                T acc[VY][VX], res[VY][VX];
                laplacian(lds + S1SET * LTILE,
                          [&](auto dzc, int j, int i) -> T {
                              constexpr int dz = decltype(dzc)::value;
                              return w0[((CS + dz) % W0 + W0) % W0][j][i];
                          },
                          acc, coupling(ew[EC1], ew[EM1], ew[EP1], lds + EBASE + ES1 * ETILE));
#pragma unroll
                for (int j = 0; j < VY; ++j)
#pragma unroll
                    for (int i = 0; i < VX; ++i) {
                        const T ctr = w0[CS][j][i];
                        const T e = E7 ? ew[EC1][j][i] : et[j][i];
                        const T u1 = damp_div<T>(
                            T(2) * ctr - (T(1) - e) * up[j][i] + v2[j][i] * acc[j][i], T(1) + e);
                        res[j][i] = (in1 && rin[j] && cin[i]) ? u1 : ctr;
                    }
                if (q1 == g.sz && sj >= 0) {
#pragma unroll
                    for (int j = 0; j < VY; ++j)
#pragma unroll
                        for (int i = 0; i < VX; ++i)
                            if (j == sj && i == si) res[j][i] += g.s0;
                }
#pragma unroll
                for (int j = 0; j < VY; ++j)
#pragma unroll
                    for (int i = 0; i < VX; ++i) ws[WC][j][i] = res[j][i];
                store(a.out, q1, k >= R && k < n + R, res);
            }

            // 4. stage 2: step n+2 at plane q2 on E (exact on T); waves
            //    without a row of T skip it
            if (wave_in_t) {
                T acc[VY][VX], res[VY][VX];
                if (C::VRING && tthr) {
#pragma unroll
                    for (int j = 0; j < VY; ++j) {
                        lds_load_group<T, VX>(vring(VR, 0, j), v2b[j]);
                        if constexpr (!E7) lds_load_group<T, VX>(vring(VR, 1, j), etb[j]);
                    }
#pragma unroll
                    for (int j = 0; j < VY; ++j) {
                        lds_store_group<T, VX>(vring(VW, 0, j), v2[j]);
                        if constexpr (!E7) lds_store_group<T, VX>(vring(VW, 1, j), et[j]);
                    }
                }
                // eta of planes q2-1, q2, q2+1 at this thread's points
                T ec2[VY][VX], em2[VY][VX], ep2[VY][VX];
                if constexpr (E7) {
#pragma unroll
                    for (int j = 0; j < VY; ++j) {
                        const int o = (1 + ly * VY + j) * LP + lcol;
                        lds_load_group<T, VX>(e2c + o, ec2[j]);
                        lds_load_group<T, VX>(e2m + o, em2[j]);
                        lds_load_group<T, VX>(e2p + o, ep2[j]);
                    }
                }
                laplacian(tile2 + T2 * LTILE,
                          [&](auto dzc, int j, int i) -> T {
                              constexpr int dz = decltype(dzc)::value;
                              return ws[((WC2 + dz) % WS + WS) % WS][j][i];
                          },
                          acc, coupling(ec2, em2, ep2, e2c));
#pragma unroll
                for (int j = 0; j < VY; ++j)
#pragma unroll
                    for (int i = 0; i < VX; ++i) {
                        const T ctr = ws[WC2][j][i];
                        const T e = E7 ? ec2[j][i] : etb[j][i];
                        res[j][i] = damp_div<T>(
                            T(2) * ctr - (T(1) - e) * w0[C2][j][i] + v2b[j][i] * acc[j][i],
                            T(1) + e);
                    }
                if (q2 == g.sz && sj >= 0) {
#pragma unroll
                    for (int j = 0; j < VY; ++j)
#pragma unroll
                        for (int i = 0; i < VX; ++i)
                            if (j == sj && i == si) res[j][i] += g.s1;
                }
                store(g.out2, q2, k >= 2 * R && k < n + 2 * R, res);
            }
    });
}

}  // namespace st
