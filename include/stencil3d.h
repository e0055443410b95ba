/*
 * stencil3d.h -- C ABI of libstencil3d.so: the 3D star stencil of radius R
 * and the acoustic isotropic wave step on MI355X (gfx950).
 *
 * Grid layout ("Accelerating High-Order Stencils on GPUs", gmem kernel
 * description): one dense flat array per field, x innermost, element
 * (x, y, z) at index x + nx*(y + ny*z).  nx, ny, nz are the ALLOCATED
 * extents, halo included; the written region ("interior") is
 * x in [R, nx-R), y in [R, ny-R), z in [R, nz-R), the points whose whole
 * stencil lies inside the array.
 *
 * Conventions shared by every entry point:
 *  - Pointers named in/out/u/... are DEVICE pointers (hipMalloc or torch
 *    allocations), aligned to the element size, owned by the caller.  The
 *    library allocates no device memory and keeps no pointer after return
 *    (wave_run_blocked_noalloc uses a static device array of the library's
 *    own instead).
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it and the call returns without synchronising.
 *  - Return value: ST_OK (0) or a negative ST_ERR_* code.  Every argument
 *    is validated before anything is enqueued, so a failed call leaves no
 *    partial work; no C++ exception crosses this boundary.  ST_ERR_LAUNCH
 *    reports a HIP error seen right after the launch.
 *  - Thread safety: calls may come from any host thread; the library holds
 *    no mutable state besides per-device caches (compute-unit count, the
 *    static workspace's address).  Overlapping wave_run_blocked_noalloc
 *    calls on one GPU race on its workspace.
 *  - Graph capture: a call only enqueues kernel launches on stream (no
 *    allocation, synchronisation, memset or copy), so it may be captured
 *    into a HIP graph and replayed.  Host arguments are read when the call
 *    is made: a captured wave_run replays the source values it was given.
 */
#ifndef STENCIL3D_H
#define STENCIL3D_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ST_ABI_VERSION 6
#define ST_MAX_R 4

/* element types */
#define ST_F32 0
#define ST_F64 1

/* boundary modes */
#define ST_BC_HALO_UNTOUCHED 0  /* write the interior only                  */
#define ST_BC_DIRICHLET_COPY 1  /* also copy every non-interior point in->out */

/* status codes */
#define ST_OK 0
#define ST_ERR_NULL (-1)        /* a required pointer is NULL                */
#define ST_ERR_STRUCT_SIZE (-2) /* desc->struct_size != sizeof(stencil3d_desc) */
#define ST_ERR_DTYPE (-3)       /* dtype not ST_F32 / ST_F64                 */
#define ST_ERR_RADIUS (-4)      /* radius outside 1..ST_MAX_R                */
#define ST_ERR_DIMS (-5)        /* an extent < 2R+1, or a plane too large    */
#define ST_ERR_BOUNDARY (-6)    /* unknown boundary mode                     */
#define ST_ERR_ALIAS (-7)       /* buffers overlap where they must not       */
#define ST_ERR_BAD_INDEX (-8)   /* source point outside the interior         */
#define ST_ERR_COEFF (-9)       /* a weight is NaN or infinite               */
#define ST_ERR_ARG (-10)        /* bad scalar argument (dt, h, counts)       */
#define ST_ERR_ALIGN (-11)      /* pointer not aligned to the element size   */
#define ST_ERR_LAUNCH (-12)     /* HIP reported an error at launch           */
#define ST_ERR_DEVICE (-13)     /* no usable HIP device                      */
#define ST_ERR_WORKSPACE (-14)  /* field too large for the static workspace  */

/* Largest field (nx*ny*nz*element size, bytes) that
 * wave_run_blocked_noalloc accepts: its two work fields live in a static
 * device array of twice this size (64 MiB per GPU). */
#define ST_NOALLOC_FIELD_BYTES_MAX (32u << 20)

/*
 * Problem descriptor.  cx/cy/cz hold the per-axis weights: index 0 is that
 * axis' share of the centre weight (the 3D centre weight is
 * cx[0]+cy[0]+cz[0]), index k = 1..R the weight of the two points at
 * offsets +k and -k on that axis.  Entries above R are ignored.
 *
 * pml_width describes the data regions of the wave step ("Accelerating
 * High-Order Stencils on GPUs": one kernel for the inner region, another
 * for the PML region, where only the latter reads eta).  If pml_width > 0
 * the caller guarantees that eta is exactly 0 at every interior point whose
 * distance (in points, along any axis) from the nearest interior face is
 * at least pml_width.  For R = 4 the single wave and PML steps then read
 * eta only near the faces: the rows within pml_width of a y face as two
 * launches of their own; in the other rows on the columns near the x
 * faces, in the planes near the z faces, and on as many columns of every
 * tile (which keeps the tiles streaming in step).  The two-step passes of
 * wave_run_blocked apply the same rule in one launch (see there).  The
 * results are bit-identical to pml_width = 0 under that guarantee, and
 * wrong where it does not hold.
 * On MI355X a 1024^3 wave step with a 32-point sponge takes 3.53 ms with
 * pml_width = 32 and 4.0 ms with 0 (eta read everywhere in one launch);
 * the PML step 3.73 and 3.98 ms.
 * Ignored by the plain stencil.  168 bytes, naturally aligned.
 */
typedef struct stencil3d_desc {
    uint32_t struct_size; /* = sizeof(stencil3d_desc)                    */
    int32_t dtype;        /* ST_F32 | ST_F64                              */
    int64_t nx, ny, nz;   /* allocated extents incl. halo; x innermost    */
    int32_t radius;       /* R, 1..ST_MAX_R                               */
    int32_t boundary;     /* ST_BC_*                                      */
    double cx[ST_MAX_R + 1];
    double cy[ST_MAX_R + 1];
    double cz[ST_MAX_R + 1];
    int64_t pml_width;    /* eta is zero this far inside; 0 = no claim    */
} stencil3d_desc;

/* ST_ABI_VERSION of the built library. */
int stencil3d_abi_version(void);

/* Static description of a status code (never NULL). */
const char *stencil3d_strerror(int code);

/*
 * Fill *d for a grid of the given extents with the standard order-2R
 * central second-difference weights on every axis (unit spacing), so the
 * stencil is the discrete Laplacian: R = 1 gives the 7-point rule of the
 * "Thread Coarsening and Register Tiling" notes (Fig 8.10) with centre -6;
 * R = 4 the 25-point rule of the acoustic isotropic kernels in
 * "Accelerating High-Order Stencils on GPUs".  Host only; validates the
 * result.
 */
int stencil3d_desc_init(stencil3d_desc *d, int dtype, int64_t nx,
                        int64_t ny, int64_t nz, int radius, int boundary);

/*
 * Check a descriptor without touching the GPU: struct size, dtype, radius,
 * boundary mode, extents (each >= 2R+1; nx*ny*elem < 2^31 bytes so that
 * in-plane offsets fit 32 bits), finite weights and pml_width >= 0
 * (ST_ERR_ARG).
 */
int stencil3d_desc_validate(const stencil3d_desc *d);

/*
 * One application of the star stencil ("Accelerating High-Order Stencils
 * on GPUs": each output reads its point and R neighbours along each
 * direction of each axis, 2.5D streaming of XY tiles through z):
 *
 *   out(p) = (cx0+cy0+cz0) in(p)
 *            + sum_{k=1..R} [ cx_k (in(p+k ex) + in(p-k ex))
 *                           + cy_k (in(p+k ey) + in(p-k ey))
 *                           + cz_k (in(p+k ez) + in(p-k ez)) ]
 *
 * on every interior point.  ST_BC_HALO_UNTOUCHED leaves the rest of out as
 * it was; ST_BC_DIRICHLET_COPY sets it to in (the boundary copy of the
 * starter kernel in "3D Stencil: Rotate the Depth Window Through
 * Registers").  in and out have d's extents and element type and must not
 * overlap (ST_ERR_ALIAS).
 */
int stencil3d_apply(const stencil3d_desc *d, const void *in, void *out,
                    void *stream);

/*
 * Jacobi ping-pong: `sweeps` applications of the stencil with a fixed
 * Dirichlet boundary (the iterated application of the starter kernel in
 * "3D Stencil: Rotate the Depth Window Through Registers"): buf1's
 * non-interior points are first set from buf0, then the sweeps alternate
 * between the buffers, writing interiors only.  The result is in buf0 if
 * sweeps is even, else in buf1 -- bit-identical to one stencil3d_apply
 * (ST_BC_DIRICHLET_COPY) per sweep.  For R = 1 the library fuses up to 6
 * (fp32) or 4 (fp64) sweeps into one pass over HBM (temporal blocking: the
 * semi-stencil section of "Accelerating High-Order Stencils on GPUs" runs
 * its time steps concurrently; the scheme here, a wavefront in z over
 * overlapped XY tiles, is this library's own design).  The buffer that does
 * not hold the result then holds an earlier sweep, not necessarily
 * sweeps-1.
 * d->boundary is ignored.  sweeps >= 0 (ST_ERR_ARG); buffers must not
 * overlap.
 */
int stencil3d_jacobi(const stencil3d_desc *d, void *buf0, void *buf1,
                     int sweeps, void *stream);

/*
 * The passes stencil3d_jacobi makes for d and `sweeps`, without running
 * them (host only: no device call, no allocation): *passes = the number of
 * passes over memory, each one kernel launch after the boundary copy;
 * ns[0 .. min(*passes, max) - 1] = the sweeps each pass fuses, in launch
 * order (ns may be NULL when max is 0).  Errors: those of
 * stencil3d_desc_validate, ST_ERR_NULL (passes, or ns with max > 0),
 * ST_ERR_ARG (sweeps or max negative).
 */
int stencil3d_jacobi_plan(const stencil3d_desc *d, int sweeps, int64_t *passes,
                          int *ns, int max);

/*
 * One time step of the acoustic isotropic wave equation with a damping
 * sponge (the acoustic isotropic model with an absorbing eta layer of
 * "Accelerating High-Order Stencils on GPUs", smem_u / smem_eta
 * descriptions; the update formula is the standard leapfrog reading):
 *
 *   L      = star_d(u) / h^2
 *   u_next = (2 u - (1 - eta) u_prev + vel2 dt^2 L) / (1 + eta)
 *
 * on every interior point; non-interior points of u_next are not written.
 * star_d is the stencil of d with d's weights (the Laplacian with unit
 * spacing from stencil3d_desc_init).  vel2 is in m^2/s^2, dt in s, h in m,
 * eta dimensionless; all five arrays share d's extents and element type.
 * In fp32 the division is a multiplication by the hardware reciprocal of
 * 1 + eta (within 1 ulp; exact where eta = 0); fp64 divides.
 * u_next may be the same buffer as u_prev (each point reads u_prev only at
 * itself), but must not overlap u, vel2 or eta.  dt, h finite, h > 0.
 * With d->pml_width > 0 (R = 4), eta is read only where it may be non-zero
 * (three launches: two y slabs and the rows between them).
 */
int wave_step(const stencil3d_desc *d, const void *u_prev, const void *u,
              void *u_next, const void *vel2, const void *eta, double dt,
              double h, void *stream);

/*
 * One time step of the PML kernel: the update of wave_step with the
 * coupling of eta's and u's central-difference gradients added to the
 * Laplacian term ("Accelerating High-Order Stencils on GPUs", smem_eta
 * description: eta enters the PML region through a low-order 7-point
 * stencil of halo 1 beside the 25-point stencil on u; the pages print no
 * formula, this is the reading taken):
 *
 *   L      = star_d(u) / h^2
 *   G      = sum_{a = x,y,z} (eta(p+e_a) - eta(p-e_a)) (u(p+e_a) - u(p-e_a)) / (4 h^2)
 *   u_next = (2 u - (1 - eta) u_prev + vel2 dt^2 (L + G)) / (1 + eta)
 *
 * on every interior point; non-interior points of u_next are not written.
 * eta is read at the interior points and their face neighbours (which may
 * lie in the halo).  Where eta is the same on a point's six face neighbours
 * G = 0 and the result is wave_step's.  Same arrays, layout, aliasing and
 * argument rules as wave_step.  With d->pml_width > 0 (R = 4) eta is read
 * only where it may be non-zero, in the launches of wave_step (same bits:
 * an eta value not read enters as the zero it is guaranteed to be).
 */
int wave_step_pml(const stencil3d_desc *d, const void *u_prev,
                  const void *u, void *u_next, const void *vel2,
                  const void *eta, double dt, double h, void *stream);

/*
 * Point source: u[ix, iy, iz] += value (rounded to d's element type), one
 * device thread.  (ix, iy, iz) are allocated coordinates and must be
 * interior (ST_ERR_BAD_INDEX).
 */
int wave_add_source(const stencil3d_desc *d, void *u, int64_t ix,
                    int64_t iy, int64_t iz, double value, void *stream);

/*
 * Two-buffer leapfrog time loop: for n = 0..nsteps-1,
 *   wave_step(u_prev -> u_prev as u_next); wave_add_source(u_prev,
 *   src_trace[n]); swap roles of the two buffers.
 * On return the newest field is in `u` if nsteps is even, else in `u_prev`
 * (the other buffer holds the field one step older).  src_trace is a HOST
 * array of nsteps values, or NULL for no source.  Same argument rules as
 * wave_step and wave_add_source.
 */
int wave_run(const stencil3d_desc *d, void *u_prev, void *u,
             const void *vel2, const void *eta, double dt, double h,
             int nsteps, int64_t src_x, int64_t src_y, int64_t src_z,
             const double *src_trace, void *stream);

/*
 * wave_run with the PML kernel's step (wave_step_pml) in place of
 * wave_step; same arguments, buffers and result placement.
 */
int wave_run_pml(const stencil3d_desc *d, void *u_prev, void *u,
                 const void *vel2, const void *eta, double dt, double h,
                 int nsteps, int64_t src_x, int64_t src_y, int64_t src_z,
                 const double *src_trace, void *stream);

/*
 * Time-blocked leapfrog: the wave_step time loop of wave_run, two steps per
 * pass over memory (two-step kernels for both element types and every
 * radius), single steps otherwise and for an odd last step.  The
 * semi-stencil section of "Accelerating High-Order Stencils on GPUs" runs
 * its time steps concurrently; the two-step wavefront over overlapped XY
 * tiles is this library's own design.  Four caller-owned fields of d's
 * shape rotate: with
 * b = {u_prev, u, work0, work1}, the field of time level k (u_prev holds
 * level 0, u level 1) lives in b[k mod 4].  A two-step pass reads levels
 * k-1 and k and writes k+1 and k+2 into the two other buffers (its tiles
 * overlap, so no level can be overwritten in place).  On return the newest
 * field (level nsteps + 1) is in b[(nsteps + 1) mod 4] and the one before
 * it in b[nsteps mod 4]; for a multiple of 4 steps that is u and u_prev,
 * as wave_run leaves them for an even count.  work0 and work1 need no
 * initial values: for nsteps > 0 the call first sets their non-interior
 * points from u (two copy kernels on stream), then writes their interiors
 * as levels are computed; nsteps = 0 enqueues nothing.
 *
 * Results are bit-identical to single steps with their sources
 * (wave_step(b[k-1], b[k] -> b[k+1]), then wave_add_source), with these
 * conditions: outside the interior u_prev and u must hold the same values
 * (zero, as a leapfrog from zero halos keeps them), since a pass takes
 * level k+1's non-interior points to be level k's.  With d->pml_width > 0
 * (R = 4) each pass reads eta only where it may be non-zero, in one launch:
 * its tiles on rows within pml_width of a y face read eta on every column,
 * the others as wave_step's data regions do (columns near the x faces and
 * the same number on every tile, planes near the z faces); the same bits
 * under the pml_width guarantee.  On MI355X the 1024^3 R = 4 run with a
 * 32-point sponge takes 2.87 ms per step with pml_width = 32 and 2.94 ms
 * with 0, against 3.53 and 4.0 ms for wave_run.
 * Same arguments as wave_run otherwise.  Errors: those of wave_run, plus
 * ST_ERR_NULL / ST_ERR_ALIGN for work0 or work1 and ST_ERR_ALIAS where any
 * two of the four u buffers, vel2 and eta overlap (vel2 and eta may be the
 * same buffer).
 */
int wave_run_blocked(const stencil3d_desc *d, void *u_prev, void *u,
                     void *work0, void *work1, const void *vel2,
                     const void *eta, double dt, double h, int nsteps,
                     int64_t src_x, int64_t src_y, int64_t src_z,
                     const double *src_trace, void *stream);

/*
 * The time-blocked run of the PML kernel's step: wave_run_blocked with
 * wave_step_pml's update (eta's 7-point coupling beside the 25-point stencil
 * on u, "Accelerating High-Order Stencils on GPUs", smem_eta description;
 * the coupling formula is the reading documented at wave_step_pml) in both
 * steps of every two-step pass, and single wave_step_pml steps for an odd
 * last step.  Same arguments, buffer rotation, result placement, workspace
 * handling and conditions as wave_run_blocked; the results are bit-identical
 * to single wave_step_pml steps with their sources (up to the sign of a zero
 * result where d->pml_width makes the single steps skip eta; the passes
 * read eta on the whole interior).  On MI355X the 1024^3 R = 4 workload
 * takes 3.76 ms per step, against 3.98 for wave_run_pml and 3.73 for
 * wave_run_pml with pml_width = 32: eta's register ring and tiles leave
 * room for only two waves per SIMD on a smaller extended tile.
 */
int wave_run_pml_blocked(const stencil3d_desc *d, void *u_prev, void *u,
                         void *work0, void *work1, const void *vel2,
                         const void *eta, double dt, double h, int nsteps,
                         int64_t src_x, int64_t src_y, int64_t src_z,
                         const double *src_trace, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * time-blocked leapfrog of wave_run_blocked with its two work fields taken
 * from a static device array inside the library (2 x
 * ST_NOALLOC_FIELD_BYTES_MAX bytes, held by each GPU the library runs on
 * until the process ends) instead of from the caller.  The call allocates
 * nothing: no hipMalloc, no hipFree, no allocating library routine.  The
 * array's device address is looked up once per device on its first call.
 *
 * Arguments, rules and results are wave_run's: the newest field ends in u
 * for an even nsteps, else in u_prev, the other buffer holding the level
 * before it, bit-identical to wave_run (and to wave_run_blocked) under
 * wave_run_blocked's condition that u_prev and u hold the same
 * non-interior values.  Internally: two-step passes for the first
 * 4*floor(nsteps/4) steps (which leave the levels in u_prev and u), then
 * the remaining steps as in-place single steps.
 *
 * Errors: those of wave_run, plus ST_ERR_WORKSPACE (before anything is
 * enqueued) if one field exceeds ST_NOALLOC_FIELD_BYTES_MAX.
 *
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents (each call first sets the non-interior points it reads and
 * writes every interior point before reading it, so no state leaks from
 * one call into the next).  Calls that overlap in time on one GPU -- from
 * two streams, or two host threads -- race on the array and give wrong
 * results; serialise them.
 */
int wave_run_blocked_noalloc(const stencil3d_desc *d, void *u_prev, void *u,
                             const void *vel2, const void *eta, double dt,
                             double h, int nsteps, int64_t src_x,
                             int64_t src_y, int64_t src_z,
                             const double *src_trace, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* STENCIL3D_H */
