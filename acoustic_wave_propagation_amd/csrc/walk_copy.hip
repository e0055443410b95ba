// walk_copy.hip -- copy kernels that move memory the way the streaming
// stencil does, without its arithmetic: the measured ceiling of its access
// pattern (libwalkcopy.so, timed by bench.py --ceilings).  Not part of the
// stencil library.
//
// Both copy the interior of a cubic fp32 grid of extent n (halo R) from in
// to out, 16 bytes per lane access:
//  * walk_copy_zmarch: workgroups of 512 threads own a TX x TY tile of the
//    interior (4 x 2 points per thread) and stream a chunk of its z planes,
//    one plane of loads in flight and one barrier per step, tiles numbered
//    tile-major and remapped so each XCD streams a contiguous band -- the
//    walk of the shipped R = 4 apply.
//  * walk_copy_rows: one-shot, one 128-lane half workgroup per interior row.
// Store modes: 0 writes each interior row where it lies (it starts 4R bytes
// into its row, so the first and last 32-byte sectors of the row are
// written in part); 1 writes each row shifted to the start of its
// allocated row (whole 32-byte sectors, the bytes of a copy that needs no
// halo left untouched); 2 (rows only) as 0 plus the R halo elements at each
// end of the row, rewritten with out's own values (whole sectors again).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "work_plan.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

// (store modes are template arguments so that each variant has a kernel
// name of its own in profiler output)
template <int LX, int LY, int SHIFT>
__global__ void __launch_bounds__(LX *LY)
    zmarch_kernel(const float *__restrict__ in, float *__restrict__ out, int n, int R,
                  int chunk, int nch) {
    constexpr int VY = 2, TX = 4 * LX, TY = LY * VY;
    const int ni = n - 2 * R;
    const int tx = ni / TX, ntile = tx * (ni / TY);
    const int wg = st::xcd_remap((int)blockIdx.x, ntile * nch);
    const int tile = wg / nch, ck = wg - tile * nch;
    const int lx = threadIdx.x % LX, ly = threadIdx.x / LX;
    const int ox = R + (tile % tx) * TX + 4 * lx;
    const int oy = R + (tile / tx) * TY + VY * ly;
    const int z0 = R + ck * chunk;
    const int64_t pl = (int64_t)n * n;
    const int sh = SHIFT ? R : 0;
    f4 cur[VY], nxt[VY];
#pragma unroll
    for (int j = 0; j < VY; ++j)
        cur[j] = *(const f4 *)(in + (int64_t)z0 * pl + (int64_t)(oy + j) * n + ox);
    for (int k = 0; k < chunk; ++k) {
        const int64_t z = z0 + k;
#pragma unroll
        for (int j = 0; j < VY; ++j)
            nxt[j] = k + 1 < chunk ? *(const f4 *)(in + (z + 1) * pl + (int64_t)(oy + j) * n + ox)
                                   : cur[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < VY; ++j)
            __builtin_nontemporal_store(cur[j], (f4 *)(out + z * pl + (int64_t)(oy + j) * n + ox - sh));
#pragma unroll
        for (int j = 0; j < VY; ++j) cur[j] = nxt[j];
    }
}

template <int MODE>
__global__ void __launch_bounds__(256)
    rows_kernel(const float *__restrict__ in, float *__restrict__ out, int n, int R) {
    const int ni = n - 2 * R;
    const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
    const int l = threadIdx.x & 127;
    if (row >= (int64_t)ni * ni) return;
    const int64_t y = R + row % ni, z = R + row / ni;
    const int64_t base = (z * n + y) * n;
    for (int x = R + 4 * l; x < n - R; x += 512) {
        const f4 v = __builtin_nontemporal_load((const f4 *)(in + base + x));
        __builtin_nontemporal_store(v, (f4 *)(out + base + x - (MODE == 1 ? R : 0)));
    }
    if (MODE == 2 && l < R) {
        // the row's halo, rewritten in place with its own values
        volatile float *vo = out;
        vo[base + l] = vo[base + l];
        vo[base + n - 1 - l] = vo[base + n - 1 - l];
    }
}

}  // namespace

#define WC_EXPORT extern "C" __attribute__((visibility("default")))

// 0, or -1 if the shape does not fit the walk (interior not a multiple of
// the tile or of the chunk count, R not 4, rows not 16-byte aligned),
// -2 on a launch error.  tile_w: 256 (256 x 16 tiles) or 512 (512 x 8).
WC_EXPORT int walk_copy_zmarch(const float *in, float *out, int n, int R, int tile_w,
                               int chunks, int shift, void *stream) {
    const int ni = n - 2 * R;
    const int tw = tile_w == 512 ? 512 : 256, th = tile_w == 512 ? 8 : 16;
    if (R != 4 || n % 4 != 0 || chunks < 1 || ni % tw || ni % th || ni % chunks) return -1;
    const int nwg = (ni / tw) * (ni / th) * chunks;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int len = ni / chunks;
    if (tw == 512 && shift)
        hipLaunchKernelGGL((zmarch_kernel<128, 4, 1>), dim3(nwg), dim3(512), 0, s, in, out, n, R,
                           len, chunks);
    else if (tw == 512)
        hipLaunchKernelGGL((zmarch_kernel<128, 4, 0>), dim3(nwg), dim3(512), 0, s, in, out, n, R,
                           len, chunks);
    else if (shift)
        hipLaunchKernelGGL((zmarch_kernel<64, 8, 1>), dim3(nwg), dim3(512), 0, s, in, out, n, R,
                           len, chunks);
    else
        hipLaunchKernelGGL((zmarch_kernel<64, 8, 0>), dim3(nwg), dim3(512), 0, s, in, out, n, R,
                           len, chunks);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

WC_EXPORT int walk_copy_rows(const float *in, float *out, int n, int R, int mode,
                             void *stream) {
    const int ni = n - 2 * R;
    if (R != 4 || n % 4 != 0 || mode < 0 || mode > 2 || ni < 1) return -1;
    const int64_t rows = (int64_t)ni * ni;
    const dim3 grid((unsigned)((rows + 1) / 2)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mode == 0)
        hipLaunchKernelGGL(rows_kernel<0>, grid, block, 0, s, in, out, n, R);
    else if (mode == 1)
        hipLaunchKernelGGL(rows_kernel<1>, grid, block, 0, s, in, out, n, R);
    else
        hipLaunchKernelGGL(rows_kernel<2>, grid, block, 0, s, in, out, n, R);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
