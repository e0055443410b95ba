// validate.h -- argument validation of the C ABI, free of HIP: descriptor
// checks, pointer alignment and aliasing rules, scalar arguments, and the
// Laplacian weight table.  Compiled into libstencil3d.so and, on its own,
// into a host-only test program.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "stencil3d.h"

namespace st {
namespace check {

size_t elem_size(const stencil3d_desc *d);

// ST_OK or the ST_ERR_* code of the first rule a call breaks.
int desc(const stencil3d_desc *d);
int init(stencil3d_desc *d, int dtype, int64_t nx, int64_t ny, int64_t nz, int radius,
         int boundary);
const char *message(int code);

int apply_args(const stencil3d_desc *d, const void *in, const void *out);
int jacobi_args(const stencil3d_desc *d, const void *buf0, const void *buf1, int sweeps);
int wave_args(const stencil3d_desc *d, const void *u_prev, const void *u, const void *u_next,
              const void *vel2, const void *eta, double dt, double h);
int source_args(const stencil3d_desc *d, const void *u, int64_t ix, int64_t iy, int64_t iz,
                double value);
int run_args(const stencil3d_desc *d, const void *u_prev, const void *u, const void *vel2,
             const void *eta, double dt, double h, int nsteps, int64_t sx, int64_t sy,
             int64_t sz, const double *src_trace);
int blocked_args(const stencil3d_desc *d, const void *u_prev, const void *u, const void *work0,
                 const void *work1, const void *vel2, const void *eta, double dt, double h,
                 int nsteps, int64_t sx, int64_t sy, int64_t sz, const double *src_trace);

// run_args, plus: one field fits the static workspace (ST_ERR_WORKSPACE).
int noalloc_args(const stencil3d_desc *d, const void *u_prev, const void *u, const void *vel2,
                 const void *eta, double dt, double h, int nsteps, int64_t sx, int64_t sy,
                 int64_t sz, const double *src_trace);

}  // namespace check
}  // namespace st
