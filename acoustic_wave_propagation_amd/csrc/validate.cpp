// validate.cpp -- argument validation of the C ABI (see validate.h).  Plain
// C++ with no HIP header: every rule can be checked on a host without the
// HIP runtime.

#include "validate.h"

#include <math.h>
#include <string.h>

namespace st {
namespace check {
namespace {

// Order-2R central second-difference weights per axis (unit spacing):
// index 0 the centre, index k the weight of offsets +-k.
const double *second_difference(int R) {
    static const double w1[] = {-2.0, 1.0};
    static const double w2[] = {-5.0 / 2.0, 4.0 / 3.0, -1.0 / 12.0};
    static const double w3[] = {-49.0 / 18.0, 3.0 / 2.0, -3.0 / 20.0, 1.0 / 90.0};
    static const double w4[] = {-205.0 / 72.0, 8.0 / 5.0, -1.0 / 5.0, 8.0 / 315.0,
                                -1.0 / 560.0};
    switch (R) {
    case 1: return w1;
    case 2: return w2;
    case 3: return w3;
    case 4: return w4;
    }
    return nullptr;
}

size_t field_bytes(const stencil3d_desc *d) {
    return (size_t)d->nx * (size_t)d->ny * (size_t)d->nz * elem_size(d);
}

int pointer(const stencil3d_desc *d, const void *p) {
    if (!p) return ST_ERR_NULL;
    if ((uintptr_t)p % elem_size(d)) return ST_ERR_ALIGN;
    return ST_OK;
}

bool overlap(const stencil3d_desc *d, const void *a, const void *b) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b, n = field_bytes(d);
    return x < y + n && y < x + n;
}

bool interior_index(const stencil3d_desc *d, int64_t ix, int64_t iy, int64_t iz) {
    const int64_t R = d->radius;
    return ix >= R && ix < d->nx - R && iy >= R && iy < d->ny - R && iz >= R && iz < d->nz - R;
}

}  // namespace

size_t elem_size(const stencil3d_desc *d) { return d->dtype == ST_F64 ? 8 : 4; }

const char *message(int code) {
    switch (code) {
    case ST_OK: return "ok";
    case ST_ERR_NULL: return "required pointer is NULL";
    case ST_ERR_STRUCT_SIZE: return "descriptor struct_size does not match this library";
    case ST_ERR_DTYPE: return "unknown element type";
    case ST_ERR_RADIUS: return "radius outside 1..ST_MAX_R";
    case ST_ERR_DIMS: return "grid extents too small (< 2R+1) or plane too large";
    case ST_ERR_BOUNDARY: return "unknown boundary mode";
    case ST_ERR_ALIAS: return "buffers overlap where they must not";
    case ST_ERR_BAD_INDEX: return "source point outside the interior";
    case ST_ERR_COEFF: return "non-finite stencil weight";
    case ST_ERR_ARG: return "bad scalar argument";
    case ST_ERR_ALIGN: return "pointer not aligned to the element size";
    case ST_ERR_LAUNCH: return "HIP kernel launch failed";
    case ST_ERR_DEVICE: return "no usable HIP device";
    case ST_ERR_WORKSPACE:
        return "field larger than the static workspace of wave_run_blocked_noalloc";
    }
    return "unknown status code";
}

int desc(const stencil3d_desc *d) {
    if (!d) return ST_ERR_NULL;
    if (d->struct_size != sizeof(stencil3d_desc)) return ST_ERR_STRUCT_SIZE;
    if (d->dtype != ST_F32 && d->dtype != ST_F64) return ST_ERR_DTYPE;
    if (d->radius < 1 || d->radius > ST_MAX_R) return ST_ERR_RADIUS;
    if (d->boundary != ST_BC_HALO_UNTOUCHED && d->boundary != ST_BC_DIRICHLET_COPY)
        return ST_ERR_BOUNDARY;
    const int64_t m = 2 * (int64_t)d->radius + 1;
    if (d->nx < m || d->ny < m || d->nz < m) return ST_ERR_DIMS;
    const int64_t lim = (int64_t)1 << 31;
    if (d->nx >= lim || d->ny >= lim || d->nz >= lim) return ST_ERR_DIMS;
    if (d->nx * d->ny * (int64_t)elem_size(d) >= lim) return ST_ERR_DIMS;
    for (int k = 0; k <= d->radius; ++k)
        if (!isfinite(d->cx[k]) || !isfinite(d->cy[k]) || !isfinite(d->cz[k]))
            return ST_ERR_COEFF;
    if (d->pml_width < 0) return ST_ERR_ARG;
    return ST_OK;
}

int init(stencil3d_desc *d, int dtype, int64_t nx, int64_t ny, int64_t nz, int radius,
         int boundary) {
    if (!d) return ST_ERR_NULL;
    memset(d, 0, sizeof(*d));
    d->struct_size = sizeof(stencil3d_desc);
    d->dtype = dtype;
    d->nx = nx;
    d->ny = ny;
    d->nz = nz;
    d->radius = radius;
    d->boundary = boundary;
    const double *w = second_difference(radius);
    if (!w) return ST_ERR_RADIUS;
    for (int k = 0; k <= radius; ++k) d->cx[k] = d->cy[k] = d->cz[k] = w[k];
    return desc(d);
}

int apply_args(const stencil3d_desc *d, const void *in, const void *out) {
    int st = desc(d);
    if (st) return st;
    if ((st = pointer(d, in)) || (st = pointer(d, out))) return st;
    if (overlap(d, in, out)) return ST_ERR_ALIAS;
    return ST_OK;
}

int jacobi_args(const stencil3d_desc *d, const void *buf0, const void *buf1, int sweeps) {
    int st = desc(d);
    if (st) return st;
    if ((st = pointer(d, buf0)) || (st = pointer(d, buf1))) return st;
    if (sweeps < 0) return ST_ERR_ARG;
    if (overlap(d, buf0, buf1)) return ST_ERR_ALIAS;
    return ST_OK;
}

int wave_args(const stencil3d_desc *d, const void *u_prev, const void *u, const void *u_next,
              const void *vel2, const void *eta, double dt, double h) {
    int st = desc(d);
    if (st) return st;
    if ((st = pointer(d, u_prev)) || (st = pointer(d, u)) || (st = pointer(d, u_next)) ||
        (st = pointer(d, vel2)) || (st = pointer(d, eta)))
        return st;
    if (!isfinite(dt) || !isfinite(h) || !(h > 0.0)) return ST_ERR_ARG;
    // u_next may be u_prev exactly (in-place leapfrog) but not a shifted
    // overlap of it, and must not overlap any other input.
    if (overlap(d, u_next, u) || overlap(d, u_next, vel2) || overlap(d, u_next, eta))
        return ST_ERR_ALIAS;
    if (u_next != u_prev && overlap(d, u_next, u_prev)) return ST_ERR_ALIAS;
    return ST_OK;
}

int source_args(const stencil3d_desc *d, const void *u, int64_t ix, int64_t iy, int64_t iz,
                double value) {
    int st = desc(d);
    if (st) return st;
    if ((st = pointer(d, u))) return st;
    if (!interior_index(d, ix, iy, iz)) return ST_ERR_BAD_INDEX;
    if (!isfinite(value)) return ST_ERR_ARG;
    return ST_OK;
}

int run_args(const stencil3d_desc *d, const void *u_prev, const void *u, const void *vel2,
             const void *eta, double dt, double h, int nsteps, int64_t sx, int64_t sy,
             int64_t sz, const double *src_trace) {
    int st = wave_args(d, u_prev, u, u_prev, vel2, eta, dt, h);
    if (st) return st;
    // both buffers are written in turn
    if (overlap(d, u_prev, u) || overlap(d, u, vel2) || overlap(d, u, eta)) return ST_ERR_ALIAS;
    if (nsteps < 0) return ST_ERR_ARG;
    if (src_trace) {
        if (!interior_index(d, sx, sy, sz)) return ST_ERR_BAD_INDEX;
        for (int n = 0; n < nsteps; ++n)
            if (!isfinite(src_trace[n])) return ST_ERR_ARG;
    }
    return ST_OK;
}

int blocked_args(const stencil3d_desc *d, const void *u_prev, const void *u, const void *work0,
                 const void *work1, const void *vel2, const void *eta, double dt, double h,
                 int nsteps, int64_t sx, int64_t sy, int64_t sz, const double *src_trace) {
    int st = run_args(d, u_prev, u, vel2, eta, dt, h, nsteps, sx, sy, sz, src_trace);
    if (st) return st;
    if ((st = pointer(d, work0)) || (st = pointer(d, work1))) return st;
    // all four u buffers are written in turn: no overlap among them or with
    // vel2 and eta
    const void *others[] = {u_prev, u, vel2, eta};
    for (const void *o : others)
        if (overlap(d, work0, o) || overlap(d, work1, o)) return ST_ERR_ALIAS;
    if (overlap(d, work0, work1)) return ST_ERR_ALIAS;
    return ST_OK;
}

int noalloc_args(const stencil3d_desc *d, const void *u_prev, const void *u, const void *vel2,
                 const void *eta, double dt, double h, int nsteps, int64_t sx, int64_t sy,
                 int64_t sz, const double *src_trace) {
    int st = run_args(d, u_prev, u, vel2, eta, dt, h, nsteps, sx, sy, sz, src_trace);
    if (st) return st;
    if (field_bytes(d) > (size_t)ST_NOALLOC_FIELD_BYTES_MAX) return ST_ERR_WORKSPACE;
    return ST_OK;
}

}  // namespace check
}  // namespace st
