// star2p5d.hip -- gfx950 kernels of the 3D star stencil and the acoustic
// wave step.
//
// Design (2.5D streaming, "Accelerating High-Order Stencils on GPUs",
// st_reg_fixed description; "3D Stencil: Rotate the Depth Window Through
// Registers"): a workgroup owns an XY tile of TX x TY outputs and walks it
// through a chunk of z planes.  Each thread owns VX consecutive x outputs
// on VY consecutive rows and keeps, for each of them, the 2R+1 values of
// its z column (planes z-R..z+R) in registers, plus one slot for the plane
// in flight.  Per z step:
//   1. issue the loads of the leading plane z+R+1 (own columns, into the
//      free window slot) and of the R-wide halo ring of plane z+1;
//   2. barrier; write plane z's own values (from the window, not re-read
//      from HBM) and its halo ring into the one LDS tile; barrier;
//   3. read the in-plane neighbours from LDS, the z neighbours from the
//      window, evaluate, and store with a streaming (nontemporal) store.
// Each interior plane is read from HBM once per chunk; the halo ring comes
// from L2 / the Infinity Cache where a neighbouring tile has fetched it.
//
// The window is indexed by compile-time slot numbers: the z loop is
// unrolled by the slot count NW = 2R+2, so rotation costs no register
// moves (the index-rotation idea of st_reg_fixed, expressed with
// templates).
//
// gfx950 specifics: wave64; lanes of a wave cover 16 (fp32) or 32 (fp64)
// consecutive x groups of 16 bytes, so every global access of a row is one
// coalesced dwordx4 per lane; LDS tile rows are padded so that a group's
// columns are 16-byte aligned (ds_read_b128 / ds_write_b128); workgroup
// ids are remapped so that each XCD (own L2) sweeps a contiguous band of
// tiles and the halo rows shared by neighbouring tiles hit in its L2.
// No MFMA: the stencil is not a dense contraction.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "internal.h"

namespace st {
namespace {

constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dealt round-robin

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
    T cc;             // centre weight, plain form
    T ccd;            // centre weight of the difference form
    T cx[ST_MAX_R], cy[ST_MAX_R], cz[ST_MAX_R];  // weight of offsets +-(k+1)
};

// Tile shapes: VX x VY outputs per thread, LX x LY threads per workgroup.
template <typename T>
struct Tile;
template <>
struct Tile<float> {
    static constexpr int VX = 4, VY = 2, LX = 16, LY = 16;
};
template <>
struct Tile<double> {
    static constexpr int VX = 2, VY = 2, LX = 32, LY = 8;
};

// Bijection from the hardware workgroup id to a logical tile id such that
// XCD k (which receives ids k, k+8, k+16, ...) owns one contiguous range of
// logical ids.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int q = n / kXcds, r = n % kXcds;
    const int xcd = b % kXcds, i = b / kXcds;
    return xcd < r ? xcd * (q + 1) + i : r * (q + 1) + (xcd - r) * q + i;
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(std::forward<F>(f));
    }
}

// N consecutive elements of one row starting at column x.  Fully inside
// the row: one vector access.  Straddling the row end (ragged edge tiles
// only): element-wise, with columns clamped to the row; the clamped values
// are never used by a written output.
template <typename T, int N>
__device__ __forceinline__ void load_group(const T *__restrict__ plane,
                                           uint32_t ro, int x, int nx,
                                           T (&v)[N]) {
    if (x + N <= nx) {
        const T *p = plane + ro + (uint32_t)x;
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = p[i];
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] = plane[ro + (uint32_t)min(x + i, nx - 1)];
    }
}

template <typename T, int N>
__device__ __forceinline__ void load_group_nt(const T *__restrict__ plane,
                                              uint32_t ro, int x, int nx,
                                              T (&v)[N]) {
    if (x + N <= nx) {
        const T *p = plane + ro + (uint32_t)x;
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = __builtin_nontemporal_load(p + i);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] = plane[ro + (uint32_t)min(x + i, nx - 1)];
    }
}

constexpr int round_up(int a, int b) { return (a + b - 1) / b * b; }

// LDS row pitch: at least `need` elements, a multiple of the group width,
// and an odd multiple of 16 bytes so that the 16-byte accesses of lanes on
// consecutive rows fall in different bank groups.
template <typename T>
constexpr int lds_pitch(int need, int vx) {
    int p = round_up(need, vx);
    while (((p * (int)sizeof(T)) / 16) % 2 == 0 ||
           (p * (int)sizeof(T)) % 16 != 0)
        p += vx;
    return p;
}

template <typename T, int R, bool WAVE>
__global__ void __launch_bounds__(Tile<T>::LX *Tile<T>::LY)
    star2p5d_kernel(StarArgs<T> a) {
    constexpr int VX = Tile<T>::VX, VY = Tile<T>::VY;
    constexpr int LX = Tile<T>::LX, LY = Tile<T>::LY;
    constexpr int NT = LX * LY;
    constexpr int TX = LX * VX, TY = LY * VY;
    constexpr int PADL = round_up(R, VX);       // LDS column of interior x=0
    constexpr int LP = lds_pitch<T>(PADL + TX + R, VX);
    constexpr int LROWS = TY + 2 * R;
    constexpr int NW = 2 * R + 2;               // window slots (even)
    constexpr int GX = TX / VX;                 // groups per tile row
    constexpr int NYU = 2 * R * GX;             // y-halo units, VX wide
    constexpr int NXU = 2 * TY;                 // x-halo units, R wide
    constexpr int KY = (NYU + NT - 1) / NT;
    constexpr int KX = (NXU + NT - 1) / NT;
    // fp64: accumulate neighbour differences (u(p+-k) - u(p)), which keeps
    // the rounding of smooth fields far below the fp64 tolerance.
    constexpr bool DIFF = std::is_same<T, double>::value;

    __shared__ __align__(16) T lds[LROWS * LP];

    const int tid = threadIdx.x;
    const int nx = a.nx, ny = a.ny;
    const int wg = xcd_remap(blockIdx.x, a.nwg);
    const int ntile = a.tiles_x * a.tiles_y;
    const int chunk = wg / ntile;
    const int trem = wg - chunk * ntile;
    const int tyi = trem / a.tiles_x;
    const int txi = trem - tyi * a.tiles_x;
    const int gx0 = R + txi * TX;
    const int gy0 = R + tyi * TY;
    const int zs = R + chunk * a.chunk_len;
    const int ze = min(zs + a.chunk_len, a.nz - R);

    // ---- own outputs: columns ox..ox+VX-1 on rows oy0..oy0+VY-1 ----------
    const int lx = tid % LX, ly = tid / LX;
    const int ox = gx0 + lx * VX;
    const int oy0 = gy0 + ly * VY;
    uint32_t orow[VY];
#pragma unroll
    for (int j = 0; j < VY; ++j) orow[j] = (uint32_t)min(oy0 + j, ny - 1) * nx;
    const int nvx = max(0, min(VX, nx - R - ox));  // written columns
    const int nvy = max(0, min(VY, ny - R - oy0));  // written rows
    const int lcol = PADL + lx * VX;
    const int lrow0 = R + ly * VY;

    // ---- halo ring units of this thread ----------------------------------
    uint32_t hy_ro[KY];
    int hy_x[KY], hy_l[KY];
    bool hy_on[KY];
#pragma unroll
    for (int q = 0; q < KY; ++q) {
        const int u = tid + q * NT;
        hy_on[q] = u < NYU;
        const int uu = hy_on[q] ? u : 0;
        const int rsel = uu / GX, g = uu - rsel * GX;
        const int gy = rsel < R ? gy0 - R + rsel : gy0 + TY + (rsel - R);
        hy_ro[q] = (uint32_t)min(gy, ny - 1) * nx;
        hy_x[q] = gx0 + g * VX;
        hy_l[q] = (rsel < R ? rsel : TY + rsel) * LP + PADL + g * VX;
    }
    uint32_t hx_ro[KX];
    int hx_x[KX], hx_l[KX];
    bool hx_on[KX];
    const int ux0 = (tid - (NYU % NT) + NT) % NT;  // x units start after y
#pragma unroll
    for (int q = 0; q < KX; ++q) {
        const int u = ux0 + q * NT;
        hx_on[q] = u < NXU;
        const int uu = hx_on[q] ? u : 0;
        const int side = uu / TY, row = uu - side * TY;
        hx_ro[q] = (uint32_t)min(gy0 + row, ny - 1) * nx;
        hx_x[q] = side ? gx0 + TX : gx0 - R;
        hx_l[q] = (R + row) * LP + (side ? PADL + TX : PADL - R);
    }

    T win[NW][VY][VX];
    T hys[2][KY][VX];
    T hxs[2][KX][R];

    auto load_window = [&](int z, auto slot_c) {
        constexpr int s = decltype(slot_c)::value;
        const T *pl = a.in + (int64_t)z * a.pz;
#pragma unroll
        for (int j = 0; j < VY; ++j) load_group<T, VX>(pl, orow[j], ox, nx, win[s][j]);
    };
    auto load_halo = [&](int z, auto slot_c) {
        constexpr int h = decltype(slot_c)::value;
        const T *pl = a.in + (int64_t)z * a.pz;
#pragma unroll
        for (int q = 0; q < KY; ++q)
            if (hy_on[q]) load_group<T, VX>(pl, hy_ro[q], hy_x[q], nx, hys[h][q]);
#pragma unroll
        for (int q = 0; q < KX; ++q)
            if (hx_on[q]) load_group<T, R>(pl, hx_ro[q], hx_x[q], nx, hxs[h][q]);
    };

    // prologue: planes zs-R..zs+R into slots 0..2R, halo of zs into slot 0
    static_for<0, 2 * R + 1>([&](auto s) { load_window(zs - R + decltype(s)::value, s); });
    load_halo(zs, std::integral_constant<int, 0>{});

    bool done = false;
    for (int k0 = 0; !done; k0 += NW) {
        static_for<0, NW>([&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            constexpr int C = (kk + R) % NW;           // slot of plane z
            constexpr int LEAD = (kk + 2 * R + 1) % NW;  // slot for plane z+R+1
            constexpr int HC = kk & 1, HN = (kk + 1) & 1;
            if (done) return;
            const int z = zs + k0 + kk;
            if (z >= ze) {
                done = true;
                return;
            }
            // 1. prefetch: leading plane and next plane's halo ring
            if (z + R + 1 < ze + R) load_window(z + R + 1, std::integral_constant<int, LEAD>{});
            if (z + 1 < ze) load_halo(z + 1, std::integral_constant<int, HN>{});

            T up[VY][VX], v2[VY][VX], et[VY][VX];
            if constexpr (WAVE) {
                const int64_t po = (int64_t)z * a.pz;
#pragma unroll
                for (int j = 0; j < VY; ++j) {
                    load_group_nt<T, VX>(a.u_prev + po, orow[j], ox, nx, up[j]);
                    load_group_nt<T, VX>(a.vel2 + po, orow[j], ox, nx, v2[j]);
                    load_group_nt<T, VX>(a.eta + po, orow[j], ox, nx, et[j]);
                }
            }

            // 2. stage plane z in LDS: own values from the window, halo ring
            //    from registers
            __syncthreads();
#pragma unroll
            for (int j = 0; j < VY; ++j)
#pragma unroll
                for (int i = 0; i < VX; ++i) lds[(lrow0 + j) * LP + lcol + i] = win[C][j][i];
#pragma unroll
            for (int q = 0; q < KY; ++q)
                if (hy_on[q])
#pragma unroll
                    for (int i = 0; i < VX; ++i) lds[hy_l[q] + i] = hys[HC][q][i];
#pragma unroll
            for (int q = 0; q < KX; ++q)
                if (hx_on[q])
#pragma unroll
                    for (int i = 0; i < R; ++i) lds[hx_l[q] + i] = hxs[HC][q][i];
            __syncthreads();

            // 3. in-plane neighbours from LDS
            T xs[VY][VX + 2 * R];  // row segment, columns ox-R .. ox+VX+R-1
#pragma unroll
            for (int j = 0; j < VY; ++j) {
                const T *row = lds + (lrow0 + j) * LP + lcol;
#pragma unroll
                for (int m = 0; m < R; ++m) {
                    xs[j][m] = row[m - R];
                    xs[j][R + VX + m] = row[VX + m];
                }
#pragma unroll
                for (int i = 0; i < VX; ++i) xs[j][R + i] = win[C][j][i];
            }
            T ys[2 * R][VX];  // rows oy0-R..oy0-1 and oy0+VY..oy0+VY+R-1
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < VX; ++i) {
                    ys[r][i] = lds[(lrow0 - R + r) * LP + lcol + i];
                    ys[R + r][i] = lds[(lrow0 + VY + r) * LP + lcol + i];
                }

            T res[VY][VX];
#pragma unroll
            for (int j = 0; j < VY; ++j)
#pragma unroll
                for (int i = 0; i < VX; ++i) {
                    const T ctr = win[C][j][i];
                    T acc = (DIFF ? a.ccd : a.cc) * ctr;
#pragma unroll
                    for (int k = 1; k <= R; ++k) {
                        const T zm = win[(C + NW - k) % NW][j][i];
                        const T zp = win[(C + k) % NW][j][i];
                        const T xm = xs[j][R + i - k], xp = xs[j][R + i + k];
                        const int qm = j - k, qp = j + k;
                        const T ym = qm < 0 ? ys[R + qm][i] : win[C][qm][i];
                        const T yp = qp >= VY ? ys[R + qp - VY][i] : win[C][qp][i];
                        if constexpr (DIFF) {
                            acc = fma(a.cz[k - 1], (zm - ctr) + (zp - ctr), acc);
                            acc = fma(a.cy[k - 1], (ym - ctr) + (yp - ctr), acc);
                            acc = fma(a.cx[k - 1], (xm - ctr) + (xp - ctr), acc);
                        } else {
                            acc = fma(a.cz[k - 1], zm + zp, acc);
                            acc = fma(a.cy[k - 1], ym + yp, acc);
                            acc = fma(a.cx[k - 1], xm + xp, acc);
                        }
                    }
                    if constexpr (WAVE) {
                        // weights carry dt^2/h^2: acc = dt^2 * Lap(u)
                        const T e = et[j][i];
                        acc = (T(2) * ctr - (T(1) - e) * up[j][i] + v2[j][i] * acc) / (T(1) + e);
                    }
                    res[j][i] = acc;
                }

            // 4. store the written part of the group (streaming stores)
            T *po = a.out + (int64_t)z * a.pz;
#pragma unroll
            for (int j = 0; j < VY; ++j) {
                if (j < nvy) {
                    T *p = po + orow[j] + (uint32_t)ox;
                    if (nvx == VX) {
#pragma unroll
                        for (int i = 0; i < VX; ++i) __builtin_nontemporal_store(res[j][i], p + i);
                    } else {
#pragma unroll
                        for (int i = 0; i < VX; ++i)
                            if (i < nvx) __builtin_nontemporal_store(res[j][i], p + i);
                    }
                }
            }
        });
    }
}

// out = in on every non-interior point; one wave per (y, z) row.
template <typename T>
__global__ void __launch_bounds__(256)
    shell_copy_kernel(const T *__restrict__ in, T *__restrict__ out, int nx,
                      int ny, int nz, int R) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int64_t rows = (int64_t)ny * nz;
    for (int64_t row = wave; row < rows; row += nwaves) {
        const int z = (int)(row / ny), y = (int)(row - (int64_t)z * ny);
        const T *s = in + row * nx;
        T *d = out + row * nx;
        if (z < R || z >= nz - R || y < R || y >= ny - R) {
            for (int x = lane; x < nx; x += 64) d[x] = s[x];
        } else if (lane < 2 * R) {
            const int x = lane < R ? lane : nx - 2 * R + lane;
            d[x] = s[x];
        }
    }
}

template <typename T>
__global__ void add_source_kernel(T *u, int64_t idx, T value) {
    if (threadIdx.x == 0 && blockIdx.x == 0) u[idx] += value;
}

template <typename T>
void tile_of(int &tx, int &ty, int &nt) {
    tx = Tile<T>::LX * Tile<T>::VX;
    ty = Tile<T>::LY * Tile<T>::VY;
    nt = Tile<T>::LX * Tile<T>::LY;
}

template <typename T, int R>
int launch_typed(const stencil3d_desc &d, const Geometry &g, const void *in,
                 void *out, const void *u_prev, const void *vel2,
                 const void *eta, bool wave, double wscale,
                 hipStream_t stream) {
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
    a.tiles_x = g.tiles_x;
    a.tiles_y = g.tiles_y;
    a.chunk_len = g.chunk_len;
    a.nwg = g.nwg;
    // Weights are combined in fp64 and rounded once to T.
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
    const dim3 grid(g.nwg), block(g.threads);
    if (wave)
        hipLaunchKernelGGL((star2p5d_kernel<T, R, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((star2p5d_kernel<T, R, false>), grid, block, 0, stream, a);
    return hipGetLastError() == hipSuccess ? ST_OK : ST_ERR_LAUNCH;
}

template <typename T>
int launch_r(const stencil3d_desc &d, const Geometry &g, const void *in,
             void *out, const void *u_prev, const void *vel2, const void *eta,
             bool wave, double wscale, hipStream_t s) {
    switch (d.radius) {
    case 1: return launch_typed<T, 1>(d, g, in, out, u_prev, vel2, eta, wave, wscale, s);
    case 2: return launch_typed<T, 2>(d, g, in, out, u_prev, vel2, eta, wave, wscale, s);
    case 3: return launch_typed<T, 3>(d, g, in, out, u_prev, vel2, eta, wave, wscale, s);
    case 4: return launch_typed<T, 4>(d, g, in, out, u_prev, vel2, eta, wave, wscale, s);
    }
    return ST_ERR_RADIUS;
}

}  // namespace

Geometry plan_geometry(const stencil3d_desc &d, int cus) {
    Geometry g;
    if (d.dtype == ST_F64)
        tile_of<double>(g.tile_x, g.tile_y, g.threads);
    else
        tile_of<float>(g.tile_x, g.tile_y, g.threads);
    const int R = d.radius;
    const int64_t ix = d.nx - 2 * R, iy = d.ny - 2 * R, iz = d.nz - 2 * R;
    g.tiles_x = (int)((ix + g.tile_x - 1) / g.tile_x);
    g.tiles_y = (int)((iy + g.tile_y - 1) / g.tile_y);
    const int64_t tiles = (int64_t)g.tiles_x * g.tiles_y;
    // Enough workgroups for two per compute unit; split z into chunks only
    // as far as needed for that, and never below 4R planes per chunk (each
    // chunk re-reads 2R planes of z halo).
    const int64_t target = 2 * (int64_t)(cus > 0 ? cus : 256);
    int64_t nch = (target + tiles - 1) / tiles;
    const int64_t maxch = iz / (4 * R) > 0 ? iz / (4 * R) : 1;
    if (nch > maxch) nch = maxch;
    if (nch < 1) nch = 1;
    int64_t len = (iz + nch - 1) / nch;
    nch = (iz + len - 1) / len;  // every chunk non-empty
    g.chunk_len = (int)len;
    g.nchunks = (int)nch;
    g.nwg = (int)(tiles * nch);
    return g;
}

int launch_star(const stencil3d_desc &d, const void *in, void *out,
                const void *u_prev, const void *vel2, const void *eta,
                bool wave, double wscale, int cus, hipStream_t stream) {
    const Geometry g = plan_geometry(d, cus);
    if (d.dtype == ST_F64)
        return launch_r<double>(d, g, in, out, u_prev, vel2, eta, wave, wscale, stream);
    return launch_r<float>(d, g, in, out, u_prev, vel2, eta, wave, wscale, stream);
}

int launch_shell_copy(const stencil3d_desc &d, const void *in, void *out,
                      hipStream_t stream) {
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

int launch_add_source(const stencil3d_desc &d, void *u, int64_t idx,
                      double value, hipStream_t stream) {
    if (d.dtype == ST_F64)
        hipLaunchKernelGGL(add_source_kernel<double>, dim3(1), dim3(64), 0, stream,
                           static_cast<double *>(u), idx, value);
    else
        hipLaunchKernelGGL(add_source_kernel<float>, dim3(1), dim3(64), 0, stream,
                           static_cast<float *>(u), idx, (float)value);
    return hipGetLastError() == hipSuccess ? ST_OK : ST_ERR_LAUNCH;
}

}  // namespace st
