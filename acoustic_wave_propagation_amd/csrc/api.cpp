// api.cpp -- the extern "C" surface of libstencil3d.so (include/stencil3d.h).
//
// Everything here runs on the host: argument validation (complete before
// anything is enqueued), the Laplacian weight table, geometry planning via
// the kernel layer, and the native Jacobi and leapfrog loops.  No exception
// leaves this file; every entry point returns an ST_* status.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "internal.h"
#include "pass_plan.h"
#include "stencil3d.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not yet queried

// Compute units of the current device (cached per device).  0 on failure.
int current_cus(int *status) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        *status = ST_ERR_DEVICE;
        return 0;
    }
    if (dev < kMaxDevices) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        *status = ST_ERR_DEVICE;
        return 0;
    }
    if (dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

size_t elem_size(const stencil3d_desc *d) { return d->dtype == ST_F64 ? 8 : 4; }

size_t field_bytes(const stencil3d_desc *d) {
    return (size_t)d->nx * (size_t)d->ny * (size_t)d->nz * elem_size(d);
}

int check_ptr(const stencil3d_desc *d, const void *p) {
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

// The wave update on the interior (pml: the PML step, with the
// eta-gradient coupling).  When the descriptor states a sponge width p
// (eta = 0 at least p points inside every interior face) and the eta-free
// kernel exists, the interior is launched as data regions -- an inner box
// that does not read eta, and six slabs that do ("Accelerating High-Order
// Stencils on GPUs": one kernel for the inner region, another for the PML
// region).  The inner box keeps distance p from every face, p + 1 for the
// PML step, whose coupling reads eta one point further out; there eta and
// its differences are zero.  Every point is written by exactly one launch
// with the same arithmetic, so the result is bit-identical to one launch
// over the interior (for the PML step: up to the sign of a zero result).
int launch_wave(const stencil3d_desc &d, const void *u, void *u_next, const void *u_prev,
                const void *vel2, const void *eta, double wscale, int cus, hipStream_t s,
                bool pml) {
    const st::Box in = st::interior_box(d);
    const st::Kind kind = pml ? st::Kind::WavePml : st::Kind::Wave;
    // (extents are below 2^31: a width from 2^30 up never fits, and clamping
    // it keeps p + 1 and 2 p from overflowing)
    const int64_t pw = d.pml_width < ((int64_t)1 << 30) ? d.pml_width : (int64_t)1 << 30;
    const int64_t p = pw > 0 ? pw + (pml ? 1 : 0) : 0;
    auto fits = [p](int64_t lo, int64_t hi) { return p < hi - lo && 2 * p < hi - lo; };
    const bool split = p > 0 && st::kind_available(d, st::Kind::WaveNoEta) &&
                       fits(in.x0, in.x1) && fits(in.y0, in.y1) && fits(in.z0, in.z1);
    if (!split)
        return st::launch_star(d, in, kind, u, u_next, u_prev, vel2, eta, wscale, cus, s);
    const st::Box c{in.x0 + p, in.x1 - p, in.y0 + p, in.y1 - p, in.z0 + p, in.z1 - p};
    const st::Box slabs[6] = {
        {in.x0, in.x1, in.y0, in.y1, in.z0, c.z0},  // below the inner box in z
        {in.x0, in.x1, in.y0, in.y1, c.z1, in.z1},  // above
        {in.x0, in.x1, in.y0, c.y0, c.z0, c.z1},    // in its z range: y < inner
        {in.x0, in.x1, c.y1, in.y1, c.z0, c.z1},    // y > inner
        {in.x0, c.x0, c.y0, c.y1, c.z0, c.z1},      // inner y, z: x < inner
        {c.x1, in.x1, c.y0, c.y1, c.z0, c.z1},      // x > inner
    };
    int st = st::launch_star(d, c, st::Kind::WaveNoEta, u, u_next, u_prev, vel2, eta, wscale,
                             cus, s);
    for (int i = 0; i < 6 && st == ST_OK; ++i)
        st = st::launch_star(d, slabs[i], kind, u, u_next, u_prev, vel2, eta, wscale, cus, s);
    return st;
}

int wave_checks(const stencil3d_desc *d, double dt, double h) {
    if (!isfinite(dt) || !isfinite(h) || !(h > 0.0)) return ST_ERR_ARG;
    (void)d;
    return ST_OK;
}

}  // namespace

// The library is built with hidden symbols; only the functions of
// stencil3d.h are exported.
#define ST_EXPORT __attribute__((visibility("default")))

extern "C" {

ST_EXPORT int stencil3d_abi_version(void) { return ST_ABI_VERSION; }

ST_EXPORT const char *stencil3d_strerror(int code) {
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
    }
    return "unknown status code";
}

ST_EXPORT int stencil3d_desc_validate(const stencil3d_desc *d) {
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

ST_EXPORT int stencil3d_desc_init(stencil3d_desc *d, int dtype, int64_t nx, int64_t ny, int64_t nz,
                        int radius, int boundary) {
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
    return stencil3d_desc_validate(d);
}

ST_EXPORT int stencil3d_apply(const stencil3d_desc *d, const void *in, void *out, void *stream) {
    int st = stencil3d_desc_validate(d);
    if (st) return st;
    if ((st = check_ptr(d, in)) || (st = check_ptr(d, out))) return st;
    if (overlap(d, in, out)) return ST_ERR_ALIAS;
    st = ST_OK;
    const int cus = current_cus(&st);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = st::launch_star(*d, st::interior_box(*d), st::Kind::Apply, in, out, nullptr, nullptr,
                         nullptr, 1.0, cus, s);
    if (st == ST_OK && d->boundary == ST_BC_DIRICHLET_COPY)
        st = st::launch_shell_copy(*d, in, out, s);
    return st;
}

ST_EXPORT int stencil3d_jacobi(const stencil3d_desc *d, void *buf0, void *buf1, int sweeps,
                     void *stream) {
    int st = stencil3d_desc_validate(d);
    if (st) return st;
    if ((st = check_ptr(d, buf0)) || (st = check_ptr(d, buf1))) return st;
    if (sweeps < 0) return ST_ERR_ARG;
    if (overlap(d, buf0, buf1)) return ST_ERR_ALIAS;
    st = ST_OK;
    const int cus = current_cus(&st);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    stencil3d_desc di = *d;
    di.boundary = ST_BC_HALO_UNTOUCHED;
    if ((st = st::launch_shell_copy(di, buf0, buf1, s))) return st;
    // Passes of several fused sweeps (temporal blocking) where a fused
    // kernel exists; each pass reads one buffer and writes the other's
    // interior.  Bit-identical to one sweep per pass.
    const int maxns = st::fused_max_sweeps(di);
    const st::PassPlan plan = st::plan_passes(sweeps, maxns, st::fused_pass_costs(di));
    void *b[2] = {buf0, buf1};
    int cur = 0;
    auto pass = [&](int ns) {
        const int r = ns == 1 ? st::launch_star(di, st::interior_box(di), st::Kind::Apply, b[cur],
                                                b[cur ^ 1], nullptr, nullptr, nullptr, 1.0, cus, s)
                              : st::launch_sweeps_fused(di, b[cur], b[cur ^ 1], ns, cus, s);
        cur ^= 1;
        return r;
    };
    for (int64_t k = 0; k < plan.bulk; ++k)
        if ((st = pass(plan.bulk_ns))) return st;
    for (int k = 0; k < plan.ntail; ++k)
        if ((st = pass(plan.tail[k]))) return st;
    return ST_OK;
}

static int wave_validate(const stencil3d_desc *d, const void *u_prev, const void *u,
                         const void *u_next, const void *vel2, const void *eta, double dt,
                         double h) {
    int st = stencil3d_desc_validate(d);
    if (st) return st;
    if ((st = check_ptr(d, u_prev)) || (st = check_ptr(d, u)) || (st = check_ptr(d, u_next)) ||
        (st = check_ptr(d, vel2)) || (st = check_ptr(d, eta)))
        return st;
    if ((st = wave_checks(d, dt, h))) return st;
    // u_next may be u_prev exactly (in-place leapfrog) but not a shifted
    // overlap of it, and must not overlap any other input.
    if (overlap(d, u_next, u) || overlap(d, u_next, vel2) || overlap(d, u_next, eta))
        return ST_ERR_ALIAS;
    if (u_next != u_prev && overlap(d, u_next, u_prev)) return ST_ERR_ALIAS;
    return ST_OK;
}

static int step_common(const stencil3d_desc *d, const void *u_prev, const void *u, void *u_next,
                       const void *vel2, const void *eta, double dt, double h, void *stream,
                       bool pml) {
    int st = wave_validate(d, u_prev, u, u_next, vel2, eta, dt, h);
    if (st) return st;
    const int cus = current_cus(&st);
    if (st) return st;
    return launch_wave(*d, u, u_next, u_prev, vel2, eta, (dt * dt) / (h * h), cus,
                       static_cast<hipStream_t>(stream), pml);
}

ST_EXPORT int wave_step(const stencil3d_desc *d, const void *u_prev, const void *u, void *u_next,
              const void *vel2, const void *eta, double dt, double h, void *stream) {
    return step_common(d, u_prev, u, u_next, vel2, eta, dt, h, stream, false);
}

ST_EXPORT int wave_step_pml(const stencil3d_desc *d, const void *u_prev, const void *u,
                            void *u_next, const void *vel2, const void *eta, double dt, double h,
                            void *stream) {
    return step_common(d, u_prev, u, u_next, vel2, eta, dt, h, stream, true);
}

ST_EXPORT int wave_add_source(const stencil3d_desc *d, void *u, int64_t ix, int64_t iy, int64_t iz,
                    double value, void *stream) {
    int st = stencil3d_desc_validate(d);
    if (st) return st;
    if ((st = check_ptr(d, u))) return st;
    if (!interior_index(d, ix, iy, iz)) return ST_ERR_BAD_INDEX;
    if (!isfinite(value)) return ST_ERR_ARG;
    const int64_t idx = ix + d->nx * (iy + d->ny * iz);
    return st::launch_add_source(*d, u, idx, value, static_cast<hipStream_t>(stream));
}

static int run_common(const stencil3d_desc *d, void *u_prev, void *u, const void *vel2,
                      const void *eta, double dt, double h, int nsteps, int64_t src_x,
                      int64_t src_y, int64_t src_z, const double *src_trace, void *stream,
                      bool pml) {
    int st = wave_validate(d, u_prev, u, u_prev, vel2, eta, dt, h);
    if (st) return st;
    if (overlap(d, u_prev, u)) return ST_ERR_ALIAS;
    if (nsteps < 0) return ST_ERR_ARG;
    if (src_trace) {
        if (!interior_index(d, src_x, src_y, src_z)) return ST_ERR_BAD_INDEX;
        for (int n = 0; n < nsteps; ++n)
            if (!isfinite(src_trace[n])) return ST_ERR_ARG;
    }
    const int cus = current_cus(&st);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const double wscale = (dt * dt) / (h * h);
    const int64_t idx = src_x + d->nx * (src_y + d->ny * src_z);
    void *a = u_prev, *b = u;  // a: older, b: newer
    for (int n = 0; n < nsteps; ++n) {
        st = launch_wave(*d, b, a, a, vel2, eta, wscale, cus, s, pml);
        if (st) return st;
        if (src_trace && (st = st::launch_add_source(*d, a, idx, src_trace[n], s))) return st;
        void *t = a;
        a = b;
        b = t;
    }
    return ST_OK;
}

ST_EXPORT int wave_run(const stencil3d_desc *d, void *u_prev, void *u, const void *vel2,
                       const void *eta, double dt, double h, int nsteps, int64_t src_x,
                       int64_t src_y, int64_t src_z, const double *src_trace, void *stream) {
    return run_common(d, u_prev, u, vel2, eta, dt, h, nsteps, src_x, src_y, src_z, src_trace,
                      stream, false);
}

ST_EXPORT int wave_run_pml(const stencil3d_desc *d, void *u_prev, void *u, const void *vel2,
                           const void *eta, double dt, double h, int nsteps, int64_t src_x,
                           int64_t src_y, int64_t src_z, const double *src_trace,
                           void *stream) {
    return run_common(d, u_prev, u, vel2, eta, dt, h, nsteps, src_x, src_y, src_z, src_trace,
                      stream, true);
}

}  // extern "C"
