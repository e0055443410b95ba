// api.cpp -- the extern "C" surface of libstencil3d.so (include/stencil3d.h).
//
// Everything here runs on the host: argument validation (validate.cpp,
// complete before anything is enqueued), geometry planning via the kernel
// layer, and the native Jacobi and leapfrog loops.  No exception leaves
// this file; every entry point returns an ST_* status.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "internal.h"
#include "pass_plan.h"
#include "stencil3d.h"
#include "validate.h"

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

// The wave update on the interior (pml: the PML step, with the
// eta-gradient coupling).  When the descriptor states a sponge width p
// (eta = 0 at least p points inside every interior face), the update reads
// eta only near the faces ("Accelerating High-Order Stencils on GPUs": one
// kernel for the inner region, another for the PML region, where only the
// latter reads eta).  The rows within p of a y face go to two launches of
// their own (slabs that read eta everywhere); the launch over the other
// rows reads eta on the columns within p of an x face or of a multiple of
// two tile widths (p columns of every tile: the left ones of even tiles,
// the right ones of odd tiles), and elsewhere only in the planes within p
// of a z face (the PML step's eta ring by the same rule, point by point).
// Every tile of that launch moves the same bytes per plane, so its tiles
// stream in step.
// Every point is written by exactly one launch with the same arithmetic
// (eta = 0 where it is not read), so the result is bit-identical to one
// launch over the interior.
int launch_wave(const stencil3d_desc &d, const void *u, void *u_next, const void *u_prev,
                const void *vel2, const void *eta, double wscale, int cus, hipStream_t s,
                bool pml) {
    const st::Box in = st::interior_box(d);
    // (extents are below 2^31: clamping the width keeps 2 p from overflowing)
    const int64_t p = d.pml_width < ((int64_t)1 << 30) ? d.pml_width : (int64_t)1 << 30;
    if (p <= 0 || d.radius != 4)
        return st::launch_star(d, in, pml ? st::Kind::WavePml : st::Kind::Wave, u, u_next,
                               u_prev, vel2, eta, wscale, cus, s);
    const st::Kind wide = pml ? st::Kind::WavePmlRegions : st::Kind::WaveRegions;
    const int pi = (int)p;
    if (2 * p >= in.y1 - in.y0)  // every row lies within p of a y face
        return st::launch_star(d, in, wide, u, u_next, u_prev, vel2, eta, wscale, cus, s, pi);
    const st::Box rows[3] = {
        {in.x0, in.x1, in.y0 + p, in.y1 - p, in.z0, in.z1},  // x and z sponges only
        {in.x0, in.x1, in.y0, in.y0 + p, in.z0, in.z1},      // y < inner
        {in.x0, in.x1, in.y1 - p, in.y1, in.z0, in.z1},      // y > inner
    };
    int st = ST_OK;
    for (int i = 0; i < 3 && st == ST_OK; ++i)
        st = st::launch_star(d, rows[i], wide, u, u_next, u_prev, vel2, eta, wscale, cus, s, pi);
    return st;
}

}  // namespace

// The library is built with hidden symbols; only the functions of
// stencil3d.h are exported.
#define ST_EXPORT __attribute__((visibility("default")))

extern "C" {

ST_EXPORT int stencil3d_abi_version(void) { return ST_ABI_VERSION; }

ST_EXPORT const char *stencil3d_strerror(int code) { return st::check::message(code); }

ST_EXPORT int stencil3d_desc_validate(const stencil3d_desc *d) { return st::check::desc(d); }

ST_EXPORT int stencil3d_desc_init(stencil3d_desc *d, int dtype, int64_t nx, int64_t ny, int64_t nz,
                                  int radius, int boundary) {
    return st::check::init(d, dtype, nx, ny, nz, radius, boundary);
}

ST_EXPORT int stencil3d_apply(const stencil3d_desc *d, const void *in, void *out, void *stream) {
    int st = st::check::apply_args(d, in, out);
    if (st) return st;
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
    int st = st::check::jacobi_args(d, buf0, buf1, sweeps);
    if (st) return st;
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

ST_EXPORT int stencil3d_jacobi_plan(const stencil3d_desc *d, int sweeps, int64_t *passes,
                                   int *ns, int max) {
    int st = st::check::desc(d);
    if (st) return st;
    if (!passes || (max > 0 && !ns)) return ST_ERR_NULL;
    if (sweeps < 0 || max < 0) return ST_ERR_ARG;
    // the plan stencil3d_jacobi follows (the boundary mode does not enter it)
    const st::PassPlan plan =
        st::plan_passes(sweeps, st::fused_max_sweeps(*d), st::fused_pass_costs(*d));
    *passes = plan.bulk + plan.ntail;
    int64_t k = 0;
    for (; k < plan.bulk && k < max; ++k) ns[k] = plan.bulk_ns;
    for (int t = 0; t < plan.ntail && k < max; ++t, ++k) ns[k] = plan.tail[t];
    return ST_OK;
}

static int step_common(const stencil3d_desc *d, const void *u_prev, const void *u, void *u_next,
                       const void *vel2, const void *eta, double dt, double h, void *stream,
                       bool pml) {
    int st = st::check::wave_args(d, u_prev, u, u_next, vel2, eta, dt, h);
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
    const int st = st::check::source_args(d, u, ix, iy, iz, value);
    if (st) return st;
    const int64_t idx = ix + d->nx * (iy + d->ny * iz);
    return st::launch_add_source(*d, u, idx, value, static_cast<hipStream_t>(stream));
}

// The two-buffer leapfrog for steps n0 .. n1-1: a holds the older level,
// b the newer; each step writes the next level over the older one in place
// and adds its source, then the roles swap.
static int leapfrog(const stencil3d_desc &d, void *a, void *b, const void *vel2,
                    const void *eta, double wscale, int n0, int n1, int64_t idx,
                    const double *src_trace, int cus, hipStream_t s, bool pml) {
    for (int n = n0; n < n1; ++n) {
        int st = launch_wave(d, b, a, a, vel2, eta, wscale, cus, s, pml);
        if (st) return st;
        if (src_trace && (st = st::launch_add_source(d, a, idx, src_trace[n], s))) return st;
        void *t = a;
        a = b;
        b = t;
    }
    return ST_OK;
}

static int run_common(const stencil3d_desc *d, void *u_prev, void *u, const void *vel2,
                      const void *eta, double dt, double h, int nsteps, int64_t src_x,
                      int64_t src_y, int64_t src_z, const double *src_trace, void *stream,
                      bool pml) {
    int st = st::check::run_args(d, u_prev, u, vel2, eta, dt, h, nsteps, src_x, src_y, src_z,
                                 src_trace);
    if (st) return st;
    const int cus = current_cus(&st);
    if (st) return st;
    const int64_t idx = src_x + d->nx * (src_y + d->ny * src_z);
    return leapfrog(*d, u_prev, u, vel2, eta, (dt * dt) / (h * h), 0, nsteps, idx, src_trace,
                    cus, static_cast<hipStream_t>(stream), pml);
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

// Two steps in one pass (launch_wave2).  With a sponge width p (plain step,
// R = 4) the pass reads eta only where it may be nonzero, in one launch:
// split into launch_wave's three row launches it measured slower (1032^3,
// ms per step: one launch reading eta everywhere 2.930, three launches
// 2.906, one launch 2.866), since the pass is bound by on-chip work more
// than by its bytes and the two y-slab launches fill the chip poorly.
static int launch_pass(const stencil3d_desc &d, const void *u_prev, const void *u, void *o1,
                       void *o2, const void *vel2, const void *eta, double wscale,
                       const st::Wave2Source &src, int cus, hipStream_t s, bool pml) {
    // (extents are below 2^31: clamping keeps the width in an int)
    const int64_t p = d.pml_width < ((int64_t)1 << 30) ? d.pml_width : (int64_t)1 << 30;
    const int pw = (pml || d.radius != 4) ? 0 : (int)p;
    return st::launch_wave2(d, pw, u_prev, u, o1, o2, vel2, eta, wscale, src, cus, s, pml);
}

// Time-blocked leapfrog over four buffers: u^k lives in b[k mod 4], so two
// steps at a time read (u^{k-1}, u^k) and write (u^{k+1}, u^{k+2}) into
// the other two buffers, which no tile of the pass reads.  A pass reads
// its inputs' non-interior points too, and the levels it writes keep u's
// there, so the work buffers' non-interior points are first set from u
// (two copy kernels: graph-safe, and whatever the buffers held before is
// never read).
static int blocked_loop(const stencil3d_desc &d, void *u_prev, void *u, void *work0, void *work1,
                        const void *vel2, const void *eta, double wscale, int nsteps,
                        int64_t src_x, int64_t src_y, int64_t src_z, const double *src_trace,
                        int cus, hipStream_t s, bool pml) {
    if (nsteps <= 0) return ST_OK;
    int st = st::launch_shell_copy(d, u, work0, s);
    if (!st) st = st::launch_shell_copy(d, u, work1, s);
    if (st) return st;
    const int64_t idx = src_x + d.nx * (src_y + d.ny * src_z);
    void *b[4] = {u_prev, u, work0, work1};
    const bool two = st::wave2_available(d);
    for (int n = 0; n < nsteps;) {
        void *p = b[n % 4], *c = b[(n + 1) % 4], *o1 = b[(n + 2) % 4], *o2 = b[(n + 3) % 4];
        if (two && nsteps - n >= 2) {
            const st::Wave2Source src{src_trace != nullptr, src_x, src_y, src_z,
                                      src_trace ? src_trace[n] : 0.0,
                                      src_trace ? src_trace[n + 1] : 0.0};
            st = launch_pass(d, p, c, o1, o2, vel2, eta, wscale, src, cus, s, pml);
            n += 2;
        } else {
            st = launch_wave(d, c, o1, p, vel2, eta, wscale, cus, s, pml);
            if (!st && src_trace) st = st::launch_add_source(d, o1, idx, src_trace[n], s);
            n += 1;
        }
        if (st) return st;
    }
    return ST_OK;
}

static int blocked_common(const stencil3d_desc *d, void *u_prev, void *u, void *work0,
                          void *work1, const void *vel2, const void *eta, double dt, double h,
                          int nsteps, int64_t src_x, int64_t src_y, int64_t src_z,
                          const double *src_trace, void *stream, bool pml) {
    int st = st::check::blocked_args(d, u_prev, u, work0, work1, vel2, eta, dt, h, nsteps, src_x,
                                     src_y, src_z, src_trace);
    if (st) return st;
    const int cus = current_cus(&st);
    if (st) return st;
    return blocked_loop(*d, u_prev, u, work0, work1, vel2, eta, (dt * dt) / (h * h), nsteps,
                        src_x, src_y, src_z, src_trace, cus, static_cast<hipStream_t>(stream),
                        pml);
}

ST_EXPORT int wave_run_blocked(const stencil3d_desc *d, void *u_prev, void *u, void *work0,
                               void *work1, const void *vel2, const void *eta, double dt,
                               double h, int nsteps, int64_t src_x, int64_t src_y,
                               int64_t src_z, const double *src_trace, void *stream) {
    return blocked_common(d, u_prev, u, work0, work1, vel2, eta, dt, h, nsteps, src_x, src_y,
                          src_z, src_trace, stream, false);
}

ST_EXPORT int wave_run_pml_blocked(const stencil3d_desc *d, void *u_prev, void *u, void *work0,
                                   void *work1, const void *vel2, const void *eta, double dt,
                                   double h, int nsteps, int64_t src_x, int64_t src_y,
                                   int64_t src_z, const double *src_trace, void *stream) {
    return blocked_common(d, u_prev, u, work0, work1, vel2, eta, dt, h, nsteps, src_x, src_y,
                          src_z, src_trace, stream, true);
}

// wave_run_blocked with the two work fields in the library's static
// workspace: two-step passes for the first 4 * floor(nsteps / 4) steps
// (after which the levels are back in u_prev and u), then the remaining
// steps as in-place single steps, so the result sits where wave_run leaves
// it.  Calls no allocating routine.
ST_EXPORT int wave_run_blocked_noalloc(const stencil3d_desc *d, void *u_prev, void *u,
                                       const void *vel2, const void *eta, double dt, double h,
                                       int nsteps, int64_t src_x, int64_t src_y, int64_t src_z,
                                       const double *src_trace, void *stream) {
    int st = st::check::noalloc_args(d, u_prev, u, vel2, eta, dt, h, nsteps, src_x, src_y,
                                     src_z, src_trace);
    if (st) return st;
    const int cus = current_cus(&st);
    if (st) return st;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if ((st = st::noalloc_scratch(&ws, &ws_bytes))) return st;
    const size_t fb = (size_t)d->nx * d->ny * d->nz * st::check::elem_size(d);
    const size_t stride = (fb + 255) / 256 * 256;
    if (2 * stride > ws_bytes) return ST_ERR_WORKSPACE;
    void *work0 = ws, *work1 = static_cast<char *>(ws) + stride;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const double wscale = (dt * dt) / (h * h);
    const int bulk = nsteps / 4 * 4;
    st = blocked_loop(*d, u_prev, u, work0, work1, vel2, eta, wscale, bulk, src_x, src_y, src_z,
                      src_trace, cus, s, false);
    if (st) return st;
    const int64_t idx = src_x + d->nx * (src_y + d->ny * src_z);
    return leapfrog(*d, u_prev, u, vel2, eta, wscale, bulk, nsteps, idx, src_trace, cus, s,
                    false);
}

}  // extern "C"
