// star2p5d_kernel.h -- device code of the 3D star stencil and the acoustic
// wave step for gfx950.  Included by star2p5d.hip, which instantiates the
// shipped tile configurations and launches them.
//
// Design (2.5D streaming, "Accelerating High-Order Stencils on GPUs",
// st_reg_fixed description; "3D Stencil: Rotate the Depth Window Through
// Registers"): a workgroup owns an XY tile of TX x TY outputs and walks it
// through a chunk of z planes.  Each thread owns VX consecutive x outputs
// on VY consecutive rows and keeps, for each of them, the values of its z
// column in a register window: planes z-R..z+R plus D planes in flight.
// Per z step:
//   1. issue the loads of plane z+R+D (own columns, into the window slot
//      that plane z-R-1 has just freed) and of the same plane's R-wide halo
//      ring, and (wave step) of plane z+DE's u_prev, vel2 and eta;
//   2. write plane z's own values (from the window, not re-read from HBM)
//      and its halo ring into one of two LDS tile buffers; barrier (the
//      other buffer lets the next step write while this one is read);
//   3. read the in-plane neighbours from LDS and the z neighbours from the
//      window, evaluate, and store.
// Each interior plane is read from HBM once per chunk; a tile's halo ring
// is loaded in the same step in which the neighbouring tiles (same XCD)
// load those rows as their own window, so the ring is served from L2.
// The loads of the next D planes (halo: R+D) stay in flight per thread,
// which covers the HBM latency at the two waves per SIMD this register
// budget allows.
//
// The window, halo and epilogue rings are indexed with compile-time slot
// numbers: the z loop is unrolled by the least common multiple of the ring
// sizes, so rotation costs no register moves (the index-rotation idea of
// st_reg_fixed, expressed with templates).  All loads are issued through
// buffer resources, unconditionally, so that the hardware wait counters
// track exactly the loads a step depends on.
//
// gfx950 specifics: wave64; each row access of a wave is one coalesced
// 16-byte-per-lane (dwordx4) access; LDS tile rows are padded so a group's
// columns are 16-byte aligned (ds_read_b128 / ds_write_b128) and rows land
// in different bank groups; workgroup ids are remapped so each XCD (own L2)
// sweeps one contiguous band of tiles.  No MFMA: the stencil is not a
// dense contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "internal.h"
#include "stencil3d.h"
#include "work_plan.h"

namespace st {

template <typename T>
struct StarArgs {
    const T *in;      // stencil input (u for the wave step)
    T *out;           // output (u_next for the wave step); may alias u_prev
    const T *u_prev;  // wave step only
    const T *vel2;
    const T *eta;
    int64_t pz;       // plane pitch in elements (nx * ny)
    int32_t nx, ny, nz;
    int32_t tiles_x, tiles_y, chunk_len, nwg;
    // Two workgroup groups: the first ga_nwg workgroups (group A) stream
    // tiles [0, ga_tiles) in z chunks of ga_len planes; the rest stream the
    // other tiles in chunks of chunk_len.  Uniform chunking: ga_nwg = 0.
    int32_t ga_nwg, ga_tiles, ga_len;
    // output box [bx0,bx1) x [by0,by1) x [bz0,bz1): inside the interior; the
    // tiles and z chunks cover it, and only its points are written
    int32_t bx0, bx1, by0, by1, bz0, bz1;
    // wave step with eta: the caller guarantees eta = 0 at every interior
    // point at least pw from all interior faces (0: no claim, eta read
    // everywhere)
    int32_t pw;
    T cc;             // centre weight, plain form
    T ccd;            // centre weight of the difference form
    T gw;             // weight of the eta-gradient coupling (PML step)
    T cx[ST_MAX_R], cy[ST_MAX_R], cz[ST_MAX_R];  // weight of offsets +-(k+1)
};

// Tile configuration: VX x VY outputs per thread, LX x LY threads per
// workgroup, D planes of stencil-input prefetch, DE planes of wave-epilogue
// prefetch (0: loaded in the step that uses them), halo ring loaded in the
// same step as the window's leading load of that plane (HLA) or D steps
// ahead of its use, LB LDS tile buffers (2: one barrier per z step),
// alternating z direction of neighbouring chunks, chunk-major (vs
// tile-major) order of the logical workgroup id, XCD remap, nontemporal
// stores, nontemporal epilogue loads, minimum waves per SIMD the register
// allocation must allow, nontemporal stencil-input loads, and whether a
// step issues its epilogue loads before (EF) or after the stencil-input
// prefetch.  The shipped choices are in star2p5d.hip; the others are kept
// for measurement.
template <int VX_, int VY_, int LX_, int LY_, int D_, int DE_, bool HLA_ = true, int LB_ = 2,
          bool ALT_ = false, bool CMAJ_ = true, bool XCD_ = true, bool NTS_ = false,
          bool NTL_ = false, int MINW_ = 1, bool NTI_ = false, bool EF_ = false>
struct TileCfg {
    static constexpr int VX = VX_, VY = VY_, LX = LX_, LY = LY_, D = D_, DE = DE_, LB = LB_;
    static constexpr int MINW = MINW_;  // register budget for >= MINW waves per SIMD
    static constexpr bool NTI = NTI_;      // nontemporal stencil-input loads
    static constexpr bool EF = EF_;        // epilogue loads first in a step
    static constexpr bool HLA = HLA_, ALT = ALT_, CMAJ = CMAJ_, XCD = XCD_, NTS = NTS_,
                          NTL = NTL_;
    static constexpr int NT = LX * LY, TX = LX * VX, TY = LY * VY;
};

constexpr int cgcd(int a, int b) { return b == 0 ? a : cgcd(b, a % b); }
constexpr int clcm(int a, int b) { return a / cgcd(a, b) * b; }
constexpr int round_up(int a, int b) { return (a + b - 1) / b * b; }
// smallest ring size >= lo that divides the unroll u (u itself if none)
constexpr int ring_fit(int u, int lo) {
    for (int r = lo; r < u; ++r)
        if (u % r == 0) return r;
    return u > lo ? u : lo;
}

// LDS row pitch: at least `need` elements, a multiple of the group width,
// and an odd multiple of 16 bytes so that the 16-byte accesses of lanes on
// consecutive rows fall in different bank groups.
template <typename T>
constexpr int lds_pitch(int need, int vx) {
    int p = round_up(need, vx);
    while ((p * (int)sizeof(T)) % 16 != 0 || ((p * (int)sizeof(T)) / 16) % 2 == 0) p += vx;
    return p;
}

// LDS row pitch of 4 mod 8 16-byte groups (at least `need` elements, a
// multiple of the group width): rows 4, 36 or 44 apart start 256 bytes
// apart modulo 512.
template <typename T>
constexpr int pair_pitch(int need, int vx) {
    int p = round_up(need, vx);
    while ((p * (int)sizeof(T)) % 16 != 0 || ((p * (int)sizeof(T)) / 16) % 8 != 4) p += vx;
    return p;
}

// num / d for the damping denominator d = 1 + eta of the wave update (d in
// [1, 2) for the sponge's eta in [0, 1)).  In fp32 it multiplies by the
// hardware reciprocal (v_rcp_f32: within 1 ulp, exact for d = 1, so
// wherever eta = 0 the result is the IEEE quotient's) instead of the
// ten-instruction IEEE division; fp64 divides.  Every wave kernel, single
// step and two-step pass, plain update and PML step, uses this form, so
// they round alike.  Measured on the 1032^3 run (ms per step, IEEE
// division against the reciprocal): plain two-step pass 3.05 -> 2.95, PML
// two-step pass 4.27 -> 4.07 (before its tile order), single steps
// unchanged (4.00 / 3.99).
template <typename T>
__device__ __forceinline__ T damp_div(T num, T d) {
    if constexpr (std::is_same<T, float>::value)
        return num * __builtin_amdgcn_rcpf(d);
    else
        return num / d;
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(std::forward<F>(f));
    }
}

// The z loop of the streaming kernels: step(kc, k0) for the steps k = k0 +
// kc in [0, n), kc a compile-time constant in [0, U).  Whole blocks of U
// steps run without any condition (the instruction stream is the same in
// every block, so the compiler's wait counts only cover loads that are at
// least a step old); the final partial block skips each step past n.  n is
// the same for every thread of the workgroup, so the barriers inside a step
// stay matched, and a chunk of any length costs its own steps only.
template <int U, typename F>
__device__ __forceinline__ void zsteps(int n, F &&step) {
    int k0 = 0;
    for (; k0 + U <= n; k0 += U) static_for<0, U>([&](auto kc) { step(kc, k0); });
    if (k0 < n)
        static_for<0, U>([&](auto kc) {
            if (decltype(kc)::value == 0 || k0 + decltype(kc)::value < n) step(kc, k0);
        });
}

// ---- buffer addressing -----------------------------------------------------
// Every plane is addressed through a buffer resource (V#) whose base is the
// plane start (uniform, scalar registers) and whose num_records ends 16
// bytes past the plane (a 16-byte group on the plane's last row may
// straddle its end), or at the plane's end on the array's last plane.
// Lanes carry 32-bit byte offsets that stay fixed over the whole z sweep,
// so a load or store costs no vector address arithmetic.  The hardware
// range check makes any access at or past num_records return zeros (loads)
// or do nothing (stores): lanes whose data is not needed use the offset
// kOOB, and loads past the plane (rows of a ragged tile beyond the array)
// read zeros that only points outside the interior use.
using rsrc_t = __amdgpu_buffer_rsrc_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 family: 32-bit raw data
constexpr uint32_t kOOB = 0x80000000u;        // >= every num_records we build
constexpr int kAuxNT = 2;                     // cache policy: nontemporal

// Plane z of an array of nz planes of pzb bytes each (pzb < 2^31, which
// validation guarantees; z in [0, nz) wherever needed is true).  A plane
// that is not needed gets num_records = 0: its accesses are still issued
// (so the instruction stream, and the wait counts the compiler derives from
// it, do not depend on the chunk length) but touch no memory.  32-bit
// arithmetic apart from the base address, so the resources of every
// unrolled step stay cheap in scalar registers.
__device__ __forceinline__ rsrc_t plane_rsrc(const void *base, int z, int nz, uint32_t pzb,
                                             bool needed) {
    const uint32_t mid = pzb + 16u < 0x7fffffffu ? pzb + 16u : 0x7fffffffu;
    const uint32_t n = !needed ? 0u : (z < nz - 1 ? mid : pzb);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(base)) + (uint64_t)(uint32_t)z * pzb, 0,
        (int)n, kRsrcWord3);
}

// N consecutive elements at byte offset off (any element-aligned offset).
template <typename T, int N, int AUX = 0>
__device__ __forceinline__ void bload(rsrc_t r, uint32_t off, T (&v)[N]) {
    constexpr int B = N * (int)sizeof(T);
    static_assert(B % 4 == 0, "whole dwords");
    uint32_t w[B / 4];
    static_for<0, B / 16>([&](auto c) {
        constexpr int k = decltype(c)::value;
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * k, 0, AUX);
        w[4 * k] = q.x, w[4 * k + 1] = q.y, w[4 * k + 2] = q.z, w[4 * k + 3] = q.w;
    });
    constexpr int done = B / 16 * 16, rem = B - done;
    if constexpr (rem == 12) {
        const u32x3 q = __builtin_amdgcn_raw_buffer_load_b96(r, off + done, 0, AUX);
        w[done / 4] = q.x, w[done / 4 + 1] = q.y, w[done / 4 + 2] = q.z;
    } else if constexpr (rem == 8) {
        const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(r, off + done, 0, AUX);
        w[done / 4] = q.x, w[done / 4 + 1] = q.y;
    } else if constexpr (rem == 4) {
        w[done / 4] = __builtin_amdgcn_raw_buffer_load_b32(r, off + done, 0, AUX);
    }
    __builtin_memcpy(v, w, B);
}

// N consecutive elements to byte offset off.
template <typename T, int N, int AUX = 0>
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, const T (&v)[N]) {
    constexpr int B = N * (int)sizeof(T);
    uint32_t w[B / 4];
    __builtin_memcpy(w, v, B);
    static_for<0, B / 16>([&](auto c) {
        constexpr int k = decltype(c)::value;
        const u32x4 q = {w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(q, r, off + 16 * k, 0, AUX);
    });
    constexpr int done = B / 16 * 16, rem = B - done;
    if constexpr (rem == 12) {
        const u32x3 q = {w[done / 4], w[done / 4 + 1], w[done / 4 + 2]};
        __builtin_amdgcn_raw_buffer_store_b96(q, r, off + done, 0, AUX);
    } else if constexpr (rem == 8) {
        const u32x2 q = {w[done / 4], w[done / 4 + 1]};
        __builtin_amdgcn_raw_buffer_store_b64(q, r, off + done, 0, AUX);
    } else if constexpr (rem == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(w[done / 4], r, off + done, 0, AUX);
    }
}

template <typename T>
__device__ __forceinline__ void bstore1(rsrc_t r, uint32_t off, T v) {
    T a[1] = {v};
    bstore<T, 1>(r, off, a);
}

// ---- LDS group access --------------------------------------------------------
// A group of N elements (16 bytes for the shipped tiles) at a 16-byte aligned
// LDS address, moved as one access (ds_read_b128 / ds_write_b128).  Lanes of
// a wave touch consecutive 16-byte groups, which the LDS serves without bank
// conflicts; element-wise (or pairwise) accesses at that lane stride make
// several lanes hit the same bank.
template <typename T, int N>
__device__ __forceinline__ void lds_load_group(const T *p, T (&v)[N]) {
    static_assert(N * sizeof(T) % 16 == 0, "whole 16-byte groups");
    const T *q = static_cast<const T *>(__builtin_assume_aligned(p, 16));
    __builtin_memcpy(v, q, N * sizeof(T));
}

template <typename T, int N>
__device__ __forceinline__ void lds_store_group(T *p, const T (&v)[N]) {
    static_assert(N * sizeof(T) % 16 == 0, "whole 16-byte groups");
    T *q = static_cast<T *>(__builtin_assume_aligned(p, 16));
    __builtin_memcpy(q, v, N * sizeof(T));
}

// Ring sizes of the kernel below, shared with the host so that z chunks can
// be sized in whole unrolled blocks.  E7: the PML step's eta planes.
template <int R, bool WAVE, class C, bool E7 = false>
struct Rings {
    static constexpr int D = C::D;                     // stencil-input prefetch depth
    static constexpr int DE = WAVE ? C::DE : 0;        // epilogue prefetch depth
    // Halo lead: steps between loading a plane's halo ring and staging it.
    // R + D loads it together with the window's leading load of the same
    // plane -- the step in which the neighbouring tiles load that plane's
    // rows as their own window -- so the ring is served from L2.
    static constexpr int HL = C::HLA ? R + D : D;
    static constexpr int H = HL + 1;                   // halo ring slots
    // window slots: planes z-R..z+R plus D in flight, padded to a multiple
    // of H so that the unroll stays short
    static constexpr int W = round_up(2 * R + 1 + D, H);
    static constexpr int E = DE + 1;                   // epilogue slots
    static constexpr int U0 = clcm(clcm(clcm(W, H), E), C::LB);
    // PML step: eta planes z-1..z+1 in registers (the ring padded to divide
    // the unroll), and the next plane's 1-wide eta halo ring (2 slots)
    static constexpr int NE = E7 ? ring_fit(U0, 3) : 1;
    static constexpr int HE = E7 ? 2 : 1;
    static constexpr int U = clcm(clcm(U0, NE), HE);   // z-loop unroll
};

// WAVE: fused wave epilogue.  E7 (wave): the PML step, which adds the
// eta-gradient coupling sum_a (eta(p+e_a) - eta(p-e_a)) (u(p+e_a) -
// u(p-e_a)) / (4 h^2) to the Laplacian -- eta's 7-point stencil of halo 1
// ("Accelerating High-Order Stencils on GPUs", smem_eta description).  As
// in smem_eta, each plane of eta is staged in LDS with its 1-wide ring; its
// z neighbours stay in a 3-plane register ring, as u's do.  SP (wave): eta
// read only near the faces for the sponge width a.pw (data regions).
template <typename T, int R, bool WAVE, class C, bool E7 = false, bool SP = false>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::MINW)))
star2p5d_kernel(StarArgs<T> a) {
    static_assert(!E7 || WAVE, "the eta stencil belongs to the wave update");
    constexpr int VX = C::VX, VY = C::VY, LX = C::LX;
    constexpr int NT = C::NT, TX = C::TX, TY = C::TY;
    using RG = Rings<R, WAVE, C, E7>;
    constexpr int D = RG::D, DE = RG::DE, HL = RG::HL, H = RG::H, W = RG::W, E = RG::E,
                  U = RG::U, NE = RG::NE, HE = RG::HE;
    // Halo ring in units of VX elements: R rows above and below the tile,
    // and XW units (XW*VX >= R columns) left and right of each tile row.
    constexpr int XW = (R + VX - 1) / VX;
    constexpr int PADL = XW * VX;               // LDS column of tile x = 0
    constexpr int LP = lds_pitch<T>(PADL + TX + XW * VX, VX);
    constexpr int LROWS = TY + 2 * R;
    constexpr int LTILE = LROWS * LP;           // one LDS tile buffer
    constexpr int LDUMMY = C::LB * LTILE;       // sink for inactive halo lanes
    constexpr int GX = TX / VX;                 // groups per tile row
    constexpr int NYU = 2 * R * GX;             // y-halo units
    constexpr int NXU = 2 * TY * XW;            // x-halo units
    constexpr int KH = (NYU + NXU + NT - 1) / NT;  // halo units per thread
    constexpr uint32_t ES = sizeof(T);
    constexpr int LAUX = C::NTL ? kAuxNT : 0, SAUX = C::NTS ? kAuxNT : 0;
    constexpr int IAUX = C::NTI ? kAuxNT : 0;
    // fp64: accumulate neighbour differences (u(p+-k) - u(p)), which keeps
    // the rounding of smooth fields far below the fp64 tolerance.
    constexpr bool DIFF = std::is_same<T, double>::value;
    static_assert(D >= 1, "at least one plane in flight");
    static_assert(C::LB == 1 || C::LB == 2, "one or two LDS tile buffers");
    // PML step: eta tile of rows gy0-1 .. gy0+TY with u's pitch and columns,
    // LB buffers after u's sink, then its own sink; eta halo units are the
    // two rows above and below (GX groups each) and the group left and right
    // of every tile row that holds the column next to the tile.
    constexpr int ETILE = E7 ? (TY + 2) * LP : 0;
    constexpr int EBASE = LDUMMY + VX;
    constexpr int EDUMMY = EBASE + C::LB * ETILE;
    constexpr int NYE = 2 * GX, NXE = 2 * TY;
    constexpr int KHE = E7 ? (NYE + NXE + NT - 1) / NT : 1;

    __shared__ __align__(16) T lds[E7 ? EDUMMY + VX : LDUMMY + VX];

    const int tid = threadIdx.x;
    const int nx = a.nx, ny = a.ny;
    // this workgroup's tile and z chunk (group A / B, XCD-remapped within
    // each group)
    const int ntile = a.tiles_x * a.tiles_y;
    const WgWork w = wg_work((int)blockIdx.x, a.nwg, ntile, a.ga_nwg, a.ga_tiles, a.ga_len,
                             a.chunk_len, C::XCD, C::CMAJ);
    const int chunk = w.chunk;
    const int tyi = w.tile / a.tiles_x;
    const int txi = w.tile - tyi * a.tiles_x;
    const int gx0 = a.bx0 + txi * TX;
    const int gy0 = a.by0 + tyi * TY;
    const int zs = a.bz0 + w.zoff;
    const int ze = min(zs + w.len, a.bz1);
    const int n = ze - zs;                      // planes of this chunk
    // Odd chunks stream downwards, so two neighbouring chunks reach their
    // shared boundary planes at the same time (both at their start, or both
    // at their end) and the second read of those planes hits in cache.  The
    // sums are symmetric in +-k, so the result does not depend on direction.
    const int dir = (C::ALT && (chunk & 1)) ? -1 : 1;
    const int z0 = dir > 0 ? zs : ze - 1;       // plane of step 0
    const uint32_t pzb = (uint32_t)(a.pz * (int64_t)ES);  // plane bytes (< 2^31)
    // some columns of this tile lie outside the box (ragged x edge)
    const bool xpart = gx0 + TX > a.bx1;

    // ---- own outputs: columns ox..ox+VX-1 on rows oy0..oy0+VY-1 ----------
    const int lx = tid % LX, ly = tid / LX;
    const int ox = gx0 + lx * VX;
    const int oy0 = gy0 + ly * VY;
    uint32_t ooff[VY];   // byte offset of (ox, oy0+j) in a plane
    uint32_t soff[VY];   // same, or kOOB where row j is not written
#pragma unroll
    for (int j = 0; j < VY; ++j) {
        ooff[j] = ((uint32_t)(oy0 + j) * (uint32_t)nx + (uint32_t)ox) * ES;
        soff[j] = (oy0 + j < a.by1 && ox < a.bx1) ? ooff[j] : kOOB;
    }
    const int nvx = max(0, min(VX, a.bx1 - ox));  // written columns (ragged x)
    // eta with data regions (a.pw > 0; eta is zero at every point at least
    // pw from all interior faces): a lane reads eta in every plane on its
    // rows within pw of an interior face in y, and on all its rows if its
    // columns lie within pw of an interior face in x or in the band of
    // columns within pw of a multiple of two tile widths (interior x); its
    // other loads read eta only in the planes within pw of a z face.
    // Elsewhere the load takes the out-of-range offset: no memory traffic,
    // and it returns that zero.  The band gives every tile the same number
    // of eta columns (even tiles their left pw columns, odd tiles their
    // right pw, which include the x sponges where the row of tiles is
    // whole), so the tiles move the same bytes per plane and stream in step
    // (their halo rows come from each other's loads in L2); tiles that read
    // eta on more columns than others drift apart and lose that reuse.  The
    // PML step's eta ring follows the same rule point by point, and its
    // units left and right of the tile are always read.
    // Bit j of emask: row j reads eta in every plane; bit VY + q: the eta
    // ring unit q does (set for every point without SP).
    const int elo = R + a.pw;  // first x (y, z) at least pw inside the interior
    auto eta_cols = [&](int x) {  // a group at x lies in the x band
        const int m = (x - R) % (2 * TX);  // interior x modulo two tiles (x >= R)
        return !SP || x < elo || x + VX > nx - elo || m < a.pw || m + VX > 2 * TX - a.pw;
    };
    auto eta_row = [&](int y) { return y < elo || y >= ny - elo; };
    auto eta_plane = [&](int k, int j) {
        const int z = z0 + dir * (k + j);
        return !SP || z < elo || z >= a.nz - elo;
    };
    uint32_t emask = 0;
#pragma unroll
    for (int j = 0; j < VY; ++j) emask |= (eta_cols(ox) || eta_row(oy0 + j)) ? 1u << j : 0u;
    // eta offset of row j (or ring unit j - VY) in a plane where zs says
    // whether the plane lies near a z face
    auto eta_off = [&](uint32_t off, int j, bool zs) {
        return (!SP || zs || ((emask >> j) & 1u)) ? off : kOOB;
    };
    const int lcol = PADL + lx * VX;
    const int lrow0 = R + ly * VY;

    // ---- halo ring units of this thread ----------------------------------
    // unit u: [0, NYU) rows above/below, [NYU, NYU+NXU) left/right columns,
    // beyond: inactive (offset kOOB, LDS sink)
    uint32_t h_off[KH];
    int h_l[KH];
#pragma unroll
    for (int q = 0; q < KH; ++q) {
        const int u = tid + q * NT;
        if (u < NYU) {
            const int rsel = u / GX, g = u - rsel * GX;
            const int gy = rsel < R ? gy0 - R + rsel : gy0 + TY + (rsel - R);
            h_off[q] = ((uint32_t)gy * (uint32_t)nx + (uint32_t)(gx0 + g * VX)) * ES;
            h_l[q] = (rsel < R ? rsel : TY + rsel) * LP + PADL + g * VX;
        } else if (u < NYU + NXU) {
            const int xu = u - NYU;
            const int side = xu / (TY * XW), rem = xu - side * (TY * XW);
            const int row = rem / XW, c = rem - row * XW;
            // left units start PADL >= R columns before the tile (columns
            // left of x = 0 land in LDS columns nothing reads)
            const int gx = side ? gx0 + TX + c * VX : gx0 - PADL + c * VX;
            h_off[q] = ((uint32_t)(gy0 + row) * (uint32_t)nx + (uint32_t)gx) * ES;
            h_l[q] = (R + row) * LP + (side ? PADL + TX : 0) + c * VX;
        } else {
            h_off[q] = kOOB;
            h_l[q] = -1;
        }
    }

    // eta halo units of this thread (PML step)
    uint32_t eh_off[KHE];
    int eh_l[KHE];
#pragma unroll
    for (int q = 0; q < KHE; ++q) {
        const int u = E7 ? tid + q * NT : NYE + NXE;
        if (u < NYE) {
            const int side = u / GX, g = u - side * GX;
            const int gy = side ? gy0 + TY : gy0 - 1;
            eh_off[q] = ((uint32_t)gy * (uint32_t)nx + (uint32_t)(gx0 + g * VX)) * ES;
            emask |= (eta_cols(gx0 + g * VX) || eta_row(gy)) ? 1u << (VY + q) : 0u;
            eh_l[q] = (side ? TY + 1 : 0) * LP + PADL + g * VX;
        } else if (u < NYE + NXE) {
            // the group ending at gx0-1 (it may start in the previous row,
            // whose values land in LDS columns nothing reads) or starting
            // at gx0+TX
            const int xu = u - NYE, side = xu / TY, row = xu - side * TY;
            const int gx = side ? gx0 + TX : gx0 - VX;
            eh_off[q] = ((uint32_t)(gy0 + row) * (uint32_t)nx + (uint32_t)gx) * ES;
            emask |= 1u << (VY + q);
            eh_l[q] = (1 + row) * LP + (side ? PADL + TX : PADL - VX);
        } else {
            eh_off[q] = kOOB;
            eh_l[q] = -1;
        }
    }

    T win[W][VY][VX];
    T hs[H][KH][VX];
    T up[E][VY][VX], v2[E][VY][VX], et[E][VY][VX];
    T ew[NE][VY][VX];    // PML step: eta plane at step offset s-1 (mod NE) in slot s
    T ehs[HE][KHE][VX];  // PML step: eta halo ring of the plane of step k in slot k % HE

    // resource of the plane at step offset j from step k (empty if unneeded)
    auto rsrc_at = [&](const T *base, int k, int j, bool needed) {
        const int z = z0 + dir * (k + j);
        return plane_rsrc(base, z, a.nz, pzb, needed);
    };
    // window slot s holds the plane at step offset s - R of the block start
    auto load_window = [&](int k, int j, bool needed, auto slot_c) {
        constexpr int s = decltype(slot_c)::value;
        const rsrc_t r = rsrc_at(a.in, k, j, needed);
#pragma unroll
        for (int jj = 0; jj < VY; ++jj) bload<T, VX, IAUX>(r, ooff[jj], win[s][jj]);
    };
    auto load_halo = [&](int k, bool needed, auto slot_c) {
        constexpr int h = decltype(slot_c)::value;
        const rsrc_t r = rsrc_at(a.in, k, 0, needed);
#pragma unroll
        for (int q = 0; q < KH; ++q) bload<T, VX, IAUX>(r, h_off[q], hs[h][q]);
    };
    auto load_epilogue = [&](int k, bool needed, auto slot_c) {
        constexpr int e = decltype(slot_c)::value;
        const rsrc_t rp = rsrc_at(a.u_prev, k, 0, needed), rv = rsrc_at(a.vel2, k, 0, needed);
#pragma unroll
        for (int jj = 0; jj < VY; ++jj) {
            bload<T, VX, LAUX>(rp, ooff[jj], up[e][jj]);
            bload<T, VX, LAUX>(rv, ooff[jj], v2[e][jj]);
        }
        if constexpr (!E7) {
            const rsrc_t re = rsrc_at(a.eta, k, 0, needed);
            const bool zs = eta_plane(k, 0);
#pragma unroll
            for (int jj = 0; jj < VY; ++jj)
                bload<T, VX, LAUX>(re, eta_off(ooff[jj], jj, zs), et[e][jj]);
        }
    };
    auto load_eta = [&](int k, int j, bool needed, auto slot_c) {
        constexpr int s = decltype(slot_c)::value;
        const rsrc_t r = rsrc_at(a.eta, k, j, needed);
        const bool zs = eta_plane(k, j);
#pragma unroll
        for (int jj = 0; jj < VY; ++jj) bload<T, VX, LAUX>(r, eta_off(ooff[jj], jj, zs), ew[s][jj]);
    };
    auto load_eta_halo = [&](int k, bool needed, auto slot_c) {
        constexpr int h = decltype(slot_c)::value;
        const rsrc_t r = rsrc_at(a.eta, k, 0, needed);
        const bool zs = eta_plane(k, 0);
#pragma unroll
        for (int q = 0; q < KHE; ++q)
            bload<T, VX, LAUX>(r, eta_off(eh_off[q], VY + q, zs), ehs[h][q]);
    };

    // prologue: window planes at step offsets -R .. R+D-1 into slots
    // 0..2R+D-1, halo rings of steps 0..HL-1, epilogue fields of steps
    // 0..DE-1 (planes past the chunk's needs get an empty resource)
    static_for<0, 2 * R + D>([&](auto s) {
        constexpr int sv = decltype(s)::value;
        load_window(0, sv - R, sv - R < n + R, s);
    });
    static_for<0, HL>([&](auto h) {
        constexpr int hv = decltype(h)::value;
        load_halo(hv, hv < n, h);
    });
    if constexpr (WAVE)
        static_for<0, DE>([&](auto e) {
            constexpr int ev = decltype(e)::value;
            load_epilogue(ev, ev < n, e);
        });
    // PML step: eta planes of step offsets -1 and 0 (a chunk has n >= 1
    // planes, and the planes next to it lie inside the array), and the eta
    // halo ring of step 0
    if constexpr (E7) {
        load_eta(0, -1, true, std::integral_constant<int, 0>{});
        load_eta(0, 0, true, std::integral_constant<int, 1>{});
        load_eta_halo(0, true, std::integral_constant<int, 0>{});
    }

    // Steps of the chunk (zsteps: whole blocks of U, then a partial one).
    // Loads of planes past the chunk's needs get empty resources (no memory
    // traffic).
    zsteps<U>(n, [&](auto kc, const int k0) {
            constexpr int kk = decltype(kc)::value;
            constexpr int CS = (kk + R) % W;           // window slot of step k
            constexpr int LEAD = (kk + 2 * R + D) % W;  // slot of offset R+D
            constexpr int HC = kk % H, HN = (kk + HL) % H;
            constexpr int EC = kk % E, EN = (kk + DE) % E;
            constexpr int LB0 = (kk % C::LB) * LTILE;  // LDS buffer of this step
            // PML step: eta slots of planes k-1, k, k+1; halo slots of k, k+1
            constexpr int EM = kk % NE, EC7 = (kk + 1) % NE, EP = (kk + 2) % NE;
            constexpr int EHC = kk % HE, EHN = (kk + 1) % HE;
            const int k = k0 + kk;
            T *tile = lds + LB0;
            T *etile = lds + EBASE + (kk % C::LB) * ETILE;

            // 1. prefetch (always issued; empty resource past the chunk).
            //    The load counter drains in issue order, so a wait for a
            //    load also waits for every load issued before it: with EF
            //    the epilogue loads go first (pinned there by a scheduling
            //    barrier) and waiting for them leaves the stencil-input
            //    prefetch in flight.
            //    The PML step's eta loads (plane k+1 and its halo ring) go
            //    with the epilogue's.
            auto load_step_epilogue = [&]() {
                load_epilogue(k + DE, k + DE < n, std::integral_constant<int, EN>{});
                if constexpr (E7) {
                    load_eta(k, 1, k + 1 <= n, std::integral_constant<int, EP>{});
                    load_eta_halo(k + 1, k + 1 < n, std::integral_constant<int, EHN>{});
                }
            };
            if constexpr (WAVE && C::EF) {
                load_step_epilogue();
                __builtin_amdgcn_sched_barrier(0);
            }
            load_window(k, R + D, k + D < n, std::integral_constant<int, LEAD>{});
            load_halo(k + HL, k + HL < n, std::integral_constant<int, HN>{});
            if constexpr (WAVE && !C::EF) load_step_epilogue();

            // 2. stage plane k in LDS: own values from the window, halo ring
            //    from registers (inactive halo lanes write the sink).  With
            //    one buffer, wait until last step's readers are done; with
            //    two, the previous barrier already ordered them.
            if constexpr (C::LB == 1) __syncthreads();
#pragma unroll
            for (int j = 0; j < VY; ++j) lds_store_group<T, VX>(tile + (lrow0 + j) * LP + lcol, win[CS][j]);
            // (ring units and the sink are whole 16-byte groups: one
            // ds_write_b128 each)
#pragma unroll
            for (int q = 0; q < KH; ++q)
                lds_store_group<T, VX>(h_l[q] >= 0 ? tile + h_l[q] : lds + LDUMMY, hs[HC][q]);
            if constexpr (E7) {
#pragma unroll
                for (int j = 0; j < VY; ++j)
                    lds_store_group<T, VX>(etile + (1 + ly * VY + j) * LP + lcol, ew[EC7][j]);
#pragma unroll
                for (int q = 0; q < KHE; ++q)
                    lds_store_group<T, VX>(eh_l[q] >= 0 ? etile + eh_l[q] : lds + EDUMMY,
                                           ehs[EHC][q]);
            }
            __syncthreads();

            // 3. in-plane neighbours from LDS
            T xs[VY][VX + 2 * R];  // row segment, columns ox-R .. ox+VX+R-1
#pragma unroll
            for (int j = 0; j < VY; ++j) {
                const T *row = tile + (lrow0 + j) * LP + lcol;
#pragma unroll
                for (int m = 0; m < R; ++m) {
                    xs[j][m] = row[m - R];
                    xs[j][R + VX + m] = row[VX + m];
                }
#pragma unroll
                for (int i = 0; i < VX; ++i) xs[j][R + i] = win[CS][j][i];
            }
            T ys[2 * R][VX];  // rows oy0-R..oy0-1 and oy0+VY..oy0+VY+R-1
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < VX; ++i) {
                    ys[r][i] = tile[(lrow0 - R + r) * LP + lcol + i];
                    ys[R + r][i] = tile[(lrow0 + VY + r) * LP + lcol + i];
                }

            // PML step: eta's in-plane neighbours outside this thread's
            // own VX x VY block, from the eta tile
            T eL[VY], eR[VY], eT[VX], eB[VX];
            if constexpr (E7) {
                const int er0 = 1 + ly * VY;
#pragma unroll
                for (int j = 0; j < VY; ++j) {
                    eL[j] = etile[(er0 + j) * LP + lcol - 1];
                    eR[j] = etile[(er0 + j) * LP + lcol + VX];
                }
                lds_load_group<T, VX>(etile + (er0 - 1) * LP + lcol, eT);
                lds_load_group<T, VX>(etile + (er0 + VY) * LP + lcol, eB);
            }

            T res[VY][VX];
#pragma unroll
            for (int j = 0; j < VY; ++j)
#pragma unroll
                for (int i = 0; i < VX; ++i) {
                    const T ctr = win[CS][j][i];
                    T acc = (DIFF ? a.ccd : a.cc) * ctr;
#pragma unroll
                    for (int kz = 1; kz <= R; ++kz) {
                        const T zm = win[(CS + W - kz) % W][j][i];
                        const T zp = win[(CS + kz) % W][j][i];
                        const T xm = xs[j][R + i - kz], xp = xs[j][R + i + kz];
                        const int qm = j - kz, qp = j + kz;
                        const T ym = qm < 0 ? ys[R + qm][i] : win[CS][qm][i];
                        const T yp = qp >= VY ? ys[R + qp - VY][i] : win[CS][qp][i];
                        if constexpr (DIFF) {
                            acc = fma(a.cz[kz - 1], (zm - ctr) + (zp - ctr), acc);
                            acc = fma(a.cy[kz - 1], (ym - ctr) + (yp - ctr), acc);
                            acc = fma(a.cx[kz - 1], (xm - ctr) + (xp - ctr), acc);
                        } else {
                            acc = fma(a.cz[kz - 1], zm + zp, acc);
                            acc = fma(a.cy[kz - 1], ym + yp, acc);
                            acc = fma(a.cx[kz - 1], xm + xp, acc);
                        }
                    }
                    if constexpr (E7) {
                        // + dt^2/(4h^2) sum_a (eta(+a) - eta(-a)) (u(+a) - u(-a))
                        const T exm = i > 0 ? ew[EC7][j][i - 1] : eL[j];
                        const T exp1 = i + 1 < VX ? ew[EC7][j][i + 1] : eR[j];
                        const T eym = j > 0 ? ew[EC7][j - 1][i] : eT[i];
                        const T eyp = j + 1 < VY ? ew[EC7][j + 1][i] : eB[i];
                        const T uym = j > 0 ? win[CS][j - 1][i] : ys[R - 1][i];
                        const T uyp = j + 1 < VY ? win[CS][j + 1][i] : ys[R][i];
                        T g = (exp1 - exm) * (xs[j][R + i + 1] - xs[j][R + i - 1]);
                        g = fma(eyp - eym, uyp - uym, g);
                        g = fma(ew[EP][j][i] - ew[EM][j][i],
                                win[(CS + 1) % W][j][i] - win[(CS + W - 1) % W][j][i], g);
                        acc = fma(a.gw, g, acc);
                    }
                    if constexpr (WAVE) {
                        // the weights carry dt^2/h^2: acc = dt^2 * Lap(u)
                        // (PML step: plus dt^2 times the coupling)
                        const T e = E7 ? ew[EC7][j][i] : et[EC][j][i];
                        acc = damp_div<T>(
                            T(2) * ctr - (T(1) - e) * up[EC][j][i] + v2[EC][j][i] * acc,
                            T(1) + e);
                    }
                    res[j][i] = acc;
                }

            // 4. store the written part: rows outside the box carry kOOB.  In
            //    a tile on the ragged x edge of the box, lanes whose group is
            //    whole store it in one access and the (at most one) partial
            //    group of a row is stored element by element; the other
            //    lanes' accesses of each kind are dropped (kOOB), so no lane
            //    branches and every wave issues the same instructions.
            const rsrc_t ro = rsrc_at(a.out, k, 0, k < n);
            if (!xpart) {
#pragma unroll
                for (int j = 0; j < VY; ++j) bstore<T, VX, SAUX>(ro, soff[j], res[j]);
            } else {
#pragma unroll
                for (int j = 0; j < VY; ++j) {
                    bstore<T, VX, SAUX>(ro, nvx == VX ? soff[j] : kOOB, res[j]);
#pragma unroll
                    for (int i = 0; i < VX - 1; ++i)
                        bstore1<T>(ro, i < nvx && nvx < VX ? soff[j] + i * ES : kOOB, res[j][i]);
                }
            }
    });
}

// out = in on every non-interior point.  The non-interior points are the
// whole rows (y, z) with z or y in the R-wide shell -- 2R ny rows in the
// shell planes plus 2R (nz - 2R) rows of the other planes -- and the R
// points at each end of every other row.  Blocks [0, full_blocks) copy the
// whole rows, one wave per row; the remaining blocks copy the row ends, one
// thread per interior row (both parts grid-stride).
template <typename T>
__global__ void __launch_bounds__(256)
    shell_copy_kernel(const T *__restrict__ in, T *__restrict__ out, int nx, int ny, int nz,
                      int R, int full_blocks) {
    const int64_t iy = ny - 2 * R, iz = nz - 2 * R;
    if ((int)blockIdx.x < full_blocks) {
        const int lane = threadIdx.x & 63;
        const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
        const int64_t nwaves = ((int64_t)full_blocks * blockDim.x) >> 6;
        const int64_t zrows = 2 * (int64_t)R * ny;   // rows of the 2R shell planes
        const int64_t rows = zrows + iz * 2 * R;     // plus y-shell rows of the others
        for (int64_t r = wave; r < rows; r += nwaves) {
            int64_t z, y;
            if (r < zrows) {
                const int64_t p = r / ny;
                z = p < R ? p : nz - 2 * R + p;
                y = r - p * ny;
            } else {
                const int64_t q = r - zrows, p = q / (2 * R), k = q - p * (2 * R);
                z = R + p;
                y = k < R ? k : ny - 2 * R + k;
            }
            const int64_t base = (z * ny + y) * nx;
            for (int x = lane; x < nx; x += 64) out[base + x] = in[base + x];
        }
    } else {
        const int64_t stride = ((int64_t)gridDim.x - full_blocks) * blockDim.x;
        for (int64_t t = ((int64_t)blockIdx.x - full_blocks) * blockDim.x + threadIdx.x;
             t < iy * iz; t += stride) {
            const int64_t z = R + t / iy, y = R + t % iy;
            const int64_t base = (z * ny + y) * nx;
            for (int k = 0; k < R; ++k) {
                out[base + k] = in[base + k];
                out[base + nx - 1 - k] = in[base + nx - 1 - k];
            }
        }
    }
}

template <typename T>
__global__ void add_source_kernel(T *u, int64_t idx, T value) {
    if (threadIdx.x == 0 && blockIdx.x == 0) u[idx] += value;
}

// Fill StarArgs from a descriptor: weights combined in fp64, scaled by
// wscale (1, or dt^2/h^2 for the wave step) and rounded once to T.
template <typename T, int R>
StarArgs<T> make_args(const stencil3d_desc &d, const Box &b, const void *in, void *out,
                      const void *u_prev, const void *vel2, const void *eta, double wscale,
                      int tiles_x, int tiles_y, int chunk_len, int nwg) {
    StarArgs<T> a;
    a.in = static_cast<const T *>(in);
    a.out = static_cast<T *>(out);
    a.u_prev = static_cast<const T *>(u_prev);
    a.vel2 = static_cast<const T *>(vel2);
    a.eta = static_cast<const T *>(eta);
    a.pz = d.nx * d.ny;
    a.nx = (int32_t)d.nx;
    a.ny = (int32_t)d.ny;
    a.nz = (int32_t)d.nz;
    a.tiles_x = tiles_x;
    a.tiles_y = tiles_y;
    a.chunk_len = chunk_len;
    a.nwg = nwg;
    a.ga_nwg = 0;
    a.ga_tiles = 0;
    a.ga_len = 0;
    a.bx0 = (int32_t)b.x0;
    a.bx1 = (int32_t)b.x1;
    a.by0 = (int32_t)b.y0;
    a.by1 = (int32_t)b.y1;
    a.bz0 = (int32_t)b.z0;
    a.bz1 = (int32_t)b.z1;
    a.pw = 0;
    a.gw = (T)(wscale * 0.25);
    const double cc = d.cx[0] + d.cy[0] + d.cz[0];
    double ksum = 0.0;
    for (int k = 1; k <= R; ++k) ksum += d.cx[k] + d.cy[k] + d.cz[k];
    a.cc = (T)(wscale * cc);
    a.ccd = (T)(wscale * (cc + 2.0 * ksum));
    for (int k = 0; k < ST_MAX_R; ++k) {
        const bool on = k < R;
        a.cx[k] = on ? (T)(wscale * d.cx[k + 1]) : T(0);
        a.cy[k] = on ? (T)(wscale * d.cy[k + 1]) : T(0);
        a.cz[k] = on ? (T)(wscale * d.cz[k + 1]) : T(0);
    }
    return a;
}

}  // namespace st
