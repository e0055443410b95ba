/*
 * oracle.c -- plain, slow CPU reference for the 3D star stencil and the
 * acoustic wave step.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark call this; the product
 * library never links, loads or calls it, and it shares no source, header,
 * table or helper with the HIP path.
 *
 * Layout (as in "Accelerating High-Order Stencils on GPUs", gmem kernel
 * description): the grid is one flat array with x innermost, element
 * (x, y, z) at index x + nx*(y + ny*z).  nx, ny, nz are the allocated
 * extents, halo included.
 *
 * Precision: inputs are fp32 or fp64 arrays (fp32 is widened exactly), the
 * weights are fp64, and every sum is accumulated in long double (x87 80-bit
 * on x86-64) so that the oracle's own rounding sits well below the fp64
 * tolerance it is compared at.  Results are written as fp64.
 *
 * Parallelism: one OpenMP "parallel for" over z planes, nothing else -- no
 * tiling, no blocking, no reordering of the sum beyond the definition.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <omp.h>

/* Read element i of an fp32 (is_f64 == 0) or fp64 array as long double. */
static inline long double rd(const void *p, int is_f64, int64_t i)
{
    if (is_f64)
        return (long double)((const double *)p)[i];
    return (long double)((const float *)p)[i];
}

int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Threads the loops below use from now on (n >= 1). */
void oracle_set_num_threads(int n)
{
    if (n >= 1)
        omp_set_num_threads(n);
}

/*
 * The star stencil of radius R at one interior point.
 *
 * "Accelerating High-Order Stencils on GPUs" (gmem kernel description): the
 * point itself plus R neighbours along each direction of each axis, 6R+1
 * points in all (25 at R = 4).  The weights are given per axis: w[0] is
 * that axis' share of the centre weight, w[k] (k = 1..R) multiplies the two
 * points at offsets +k and -k on that axis.  The 7-point rule of the
 * "Thread Coarsening and Register Tiling" notes (Fig 8.10) is the R = 1
 * case: centre plus the six face neighbours.
 *
 * Written as a literal sum over the list of 6R+1 offsets.
 */
static long double star_at(const void *u, int is_f64, int64_t nx, int64_t ny,
                           int64_t x, int64_t y, int64_t z, int R,
                           const double *cx, const double *cy,
                           const double *cz)
{
    const int64_t sx = 1, sy = nx, sz = nx * ny;
    const int64_t c = x * sx + y * sy + z * sz;
    long double acc = ((long double)cx[0] + (long double)cy[0] +
                       (long double)cz[0]) * rd(u, is_f64, c);
    for (int k = 1; k <= R; ++k) {
        acc += (long double)cx[k] * rd(u, is_f64, c + k * sx);
        acc += (long double)cx[k] * rd(u, is_f64, c - k * sx);
        acc += (long double)cy[k] * rd(u, is_f64, c + k * sy);
        acc += (long double)cy[k] * rd(u, is_f64, c - k * sy);
        acc += (long double)cz[k] * rd(u, is_f64, c + k * sz);
        acc += (long double)cz[k] * rd(u, is_f64, c - k * sz);
    }
    return acc;
}

/*
 * One application of the star stencil.
 *
 * Interior = points whose whole stencil lies inside the allocation:
 * x in [R, nx-R), y in [R, ny-R), z in [R, nz-R) (the interior guard of the
 * Fig 8.10 kernel in the register-tiling notes, generalised to radius R).
 *
 * boundary == 0 ("halo untouched"): only interior points of out are
 *   written; every other element keeps whatever the caller put there.
 * boundary == 1 ("Dirichlet copy"): every non-interior point of out is set
 *   to the input value, as the starter kernel of "3D Stencil: Rotate the
 *   Depth Window Through Registers" copies boundary points unchanged.
 */
void oracle_star_apply(const void *in, int in_is_f64, double *out,
                       int64_t nx, int64_t ny, int64_t nz, int R,
                       const double *cx, const double *cy, const double *cz,
                       int boundary)
{
    int64_t z;
#pragma omp parallel for schedule(static)
    for (z = 0; z < nz; ++z) {
        for (int64_t y = 0; y < ny; ++y) {
            for (int64_t x = 0; x < nx; ++x) {
                const int64_t i = x + nx * (y + ny * z);
                const int interior = x >= R && x < nx - R && y >= R &&
                                     y < ny - R && z >= R && z < nz - R;
                if (interior)
                    out[i] = (double)star_at(in, in_is_f64, nx, ny, x, y, z,
                                             R, cx, cy, cz);
                else if (boundary == 1)
                    out[i] = (double)rd(in, in_is_f64, i);
            }
        }
    }
}

/*
 * One time step of the acoustic isotropic wave equation with a damping
 * sponge, at every interior point (non-interior points of u_next are not
 * written):
 *
 *   L      = star(u) / h^2                       (R = 4: 8th-order Laplacian)
 *   u_next = (2 u - (1 - eta) u_prev + vel2 dt^2 L) / (1 + eta)
 *
 * "Accelerating High-Order Stencils on GPUs" names the acoustic isotropic
 * model, its R = 4 stencil on u (smem_u description) and the eta array of
 * its absorbing layer (smem_eta description) but prints no update formula;
 * this is the standard second-order-in-time leapfrog with a pointwise
 * damping term, the reading recorded in the design notes.  All five fields
 * share one layout; each input's element type is given by its own flag
 * (0 = fp32, 1 = fp64) so that an fp64 state can run on fp32 material
 * fields.
 */
void oracle_wave_step(const void *u_prev, int up_f64, const void *u,
                      int u_f64, const void *vel2, int v_f64,
                      const void *eta, int e_f64, double *u_next,
                      int64_t nx, int64_t ny, int64_t nz, int R,
                      const double *cx, const double *cy, const double *cz,
                      double dt, double h)
{
    const long double dt2 = (long double)dt * (long double)dt;
    const long double h2 = (long double)h * (long double)h;
    int64_t z;
#pragma omp parallel for schedule(static)
    for (z = R; z < nz - R; ++z) {
        for (int64_t y = R; y < ny - R; ++y) {
            for (int64_t x = R; x < nx - R; ++x) {
                const int64_t i = x + nx * (y + ny * z);
                const long double L =
                    star_at(u, u_f64, nx, ny, x, y, z, R, cx, cy, cz) / h2;
                const long double e = rd(eta, e_f64, i);
                const long double un = rd(u, u_f64, i);
                const long double up = rd(u_prev, up_f64, i);
                const long double v2 = rd(vel2, v_f64, i);
                u_next[i] =
                    (double)((2.0L * un - (1.0L - e) * up + v2 * dt2 * L) /
                             (1.0L + e));
            }
        }
    }
}

/*
 * The eta-gradient coupling at one interior point, without the 1/h^2:
 *
 *   G = sum over the axes a of (eta(p+e_a) - eta(p-e_a)) (u(p+e_a) - u(p-e_a)) / 4
 *
 * i.e. grad(eta) . grad(u) with both gradients by second-order central
 * differences.  "Accelerating High-Order Stencils on GPUs" (smem_eta
 * description) states that the PML kernel reads eta through a low-order
 * 7-point stencil, halo 1, next to the 25-point stencil on u, but prints no
 * formula; this term -- the six face neighbours of eta paired with the
 * same six neighbours of u, which with the centre value that the damping
 * reads makes the 7-point stencil -- is the reading recorded in the design
 * notes.
 */
static long double eta_coupling_at(const void *u, int u_f64, const void *eta,
                                   int e_f64, int64_t nx, int64_t ny,
                                   int64_t x, int64_t y, int64_t z)
{
    const int64_t c = x + nx * (y + ny * z);
    const int64_t stride[3] = {1, nx, nx * ny};
    long double acc = 0.0L;
    for (int a = 0; a < 3; ++a) {
        const int64_t s = stride[a];
        const long double deta = rd(eta, e_f64, c + s) - rd(eta, e_f64, c - s);
        const long double du = rd(u, u_f64, c + s) - rd(u, u_f64, c - s);
        acc += deta * du;
    }
    return acc / 4.0L;
}

/*
 * One wave step of the PML kernel: the update of oracle_wave_step with the
 * eta-gradient coupling added to the Laplacian term,
 *
 *   L      = star(u) / h^2
 *   G      = eta_coupling(u, eta) / h^2
 *   u_next = (2 u - (1 - eta) u_prev + vel2 dt^2 (L + G)) / (1 + eta)
 *
 * on every interior point (non-interior points of u_next are not written).
 * Where eta is constant over a point's six face neighbours, G = 0 and the
 * step is that of oracle_wave_step.
 */
void oracle_wave_step_pml(const void *u_prev, int up_f64, const void *u,
                          int u_f64, const void *vel2, int v_f64,
                          const void *eta, int e_f64, double *u_next,
                          int64_t nx, int64_t ny, int64_t nz, int R,
                          const double *cx, const double *cy,
                          const double *cz, double dt, double h)
{
    const long double dt2 = (long double)dt * (long double)dt;
    const long double h2 = (long double)h * (long double)h;
    int64_t z;
#pragma omp parallel for schedule(static)
    for (z = R; z < nz - R; ++z) {
        for (int64_t y = R; y < ny - R; ++y) {
            for (int64_t x = R; x < nx - R; ++x) {
                const int64_t i = x + nx * (y + ny * z);
                const long double L =
                    star_at(u, u_f64, nx, ny, x, y, z, R, cx, cy, cz) / h2;
                const long double G =
                    eta_coupling_at(u, u_f64, eta, e_f64, nx, ny, x, y, z) / h2;
                const long double e = rd(eta, e_f64, i);
                const long double un = rd(u, u_f64, i);
                const long double up = rd(u_prev, up_f64, i);
                const long double v2 = rd(vel2, v_f64, i);
                u_next[i] = (double)((2.0L * un - (1.0L - e) * up +
                                      v2 * dt2 * (L + G)) / (1.0L + e));
            }
        }
    }
}
