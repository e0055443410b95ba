/*
 * A plain C99 consumer of libstencil3d.so: no Python, no torch.  Device
 * memory comes from the HIP runtime's C API.
 *
 *   abi_consumer cpu            argument validation only (no device needed)
 *   abi_consumer gpu OUT.bin    one R = 2 fp32 apply on a 19x23x41 grid;
 *                               writes the input and output arrays to OUT.bin
 *                               (raw float32, input first) for comparison
 *                               with the oracle
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "stencil3d.h"

#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);  \
            return 1;                                                        \
        }                                                                    \
    } while (0)

static int cpu_checks(void) {
    stencil3d_desc d;
    EXPECT(stencil3d_abi_version() == ST_ABI_VERSION);
    EXPECT(strcmp(stencil3d_strerror(ST_OK), "ok") == 0);
    EXPECT(stencil3d_desc_init(&d, ST_F32, 41, 23, 19, 2, ST_BC_HALO_UNTOUCHED) == ST_OK);
    EXPECT(d.struct_size == sizeof(stencil3d_desc) && d.nx == 41 && d.nz == 19);
    EXPECT(stencil3d_desc_validate(&d) == ST_OK);
    d.radius = 7;
    EXPECT(stencil3d_desc_validate(&d) == ST_ERR_RADIUS);
    d.radius = 2;
    /* every entry point rejects before touching a device */
    EXPECT(stencil3d_apply(&d, NULL, NULL, NULL) == ST_ERR_NULL);
    EXPECT(stencil3d_apply(NULL, NULL, NULL, NULL) == ST_ERR_NULL);
    EXPECT(stencil3d_jacobi(&d, (void *)64, (void *)64, 1, NULL) == ST_ERR_ALIAS);
    EXPECT(wave_step(&d, (void *)64, (void *)1000000, (void *)2000000,
                     (void *)3000000, (void *)4000000, 1e-3, 0.0, NULL) == ST_ERR_ARG);
    EXPECT(wave_step_pml(&d, (void *)64, (void *)1000000, (void *)2000000,
                         (void *)3000000, (void *)4000000, 1e-3, 0.0, NULL) == ST_ERR_ARG);
    EXPECT(wave_run_pml(&d, (void *)64, (void *)1000000, (void *)3000000, (void *)4000000,
                        1e-3, 10.0, -1, 10, 10, 10, NULL, NULL) == ST_ERR_ARG);
    EXPECT(wave_add_source(&d, (void *)64, 0, 5, 5, 1.0, NULL) == ST_ERR_BAD_INDEX);
    EXPECT(wave_run_blocked(&d, (void *)64, (void *)1000000, (void *)2000000, (void *)2000000,
                            (void *)3000000, (void *)4000000, 1e-3, 10.0, 2, 10, 10, 10, NULL,
                            NULL) == ST_ERR_ALIAS);
    {
        /* the Jacobi pass plan, a host-only query: R = 1 fp32, 10 sweeps
           as two passes of five */
        stencil3d_desc j;
        int64_t passes = -1;
        int ns[4] = {0, 0, 0, 0};
        EXPECT(stencil3d_desc_init(&j, ST_F32, 40, 40, 40, 1, ST_BC_DIRICHLET_COPY) == ST_OK);
        EXPECT(stencil3d_jacobi_plan(&j, 10, &passes, ns, 4) == ST_OK);
        EXPECT(passes == 2 && ns[0] == 5 && ns[1] == 5 && ns[2] == 0);
        EXPECT(stencil3d_jacobi_plan(&j, 10, NULL, NULL, 0) == ST_ERR_NULL);
    }
    printf("cpu checks ok\n");
    return 0;
}

static int gpu_run(const char *path) {
    const int64_t nx = 41, ny = 23, nz = 19;
    const size_t n = (size_t)(nx * ny * nz), bytes = n * sizeof(float);
    float *h_in = (float *)malloc(bytes), *h_out = (float *)malloc(bytes);
    void *d_in = NULL, *d_out = NULL;
    stencil3d_desc d;
    uint32_t s = 12345u;
    EXPECT(h_in && h_out);
    for (size_t i = 0; i < n; ++i) { /* an LCG in [-1, 1) */
        s = s * 1664525u + 1013904223u;
        h_in[i] = (float)((double)(s >> 8) / 8388608.0 - 1.0);
    }
    EXPECT(hipMalloc(&d_in, bytes) == hipSuccess);
    EXPECT(hipMalloc(&d_out, bytes) == hipSuccess);
    EXPECT(hipMemcpy(d_in, h_in, bytes, hipMemcpyHostToDevice) == hipSuccess);
    EXPECT(hipMemset(d_out, 0, bytes) == hipSuccess);
    EXPECT(stencil3d_desc_init(&d, ST_F32, nx, ny, nz, 2, ST_BC_HALO_UNTOUCHED) == ST_OK);
    EXPECT(stencil3d_apply(&d, d_in, d_out, NULL) == ST_OK);
    EXPECT(hipDeviceSynchronize() == hipSuccess);
    EXPECT(hipMemcpy(h_out, d_out, bytes, hipMemcpyDeviceToHost) == hipSuccess);
    FILE *f = fopen(path, "wb");
    EXPECT(f != NULL);
    EXPECT(fwrite(h_in, 1, bytes, f) == bytes && fwrite(h_out, 1, bytes, f) == bytes);
    fclose(f);
    hipFree(d_in);
    hipFree(d_out);
    free(h_in);
    free(h_out);
    printf("gpu apply ok\n");
    return 0;
}

/* Two leapfrog steps through wave_run_blocked (R = 4, fp32): u_prev and u
 * random on the interior, zero halos; vel2 and eta random; a point source.
 * Writes u_prev, u, vel2, eta, work0 (level 2) and work1 (level 3). */
static int gpu_blocked(const char *path) {
    const int64_t nx = 41, ny = 23, nz = 19, R = 4;
    const size_t n = (size_t)(nx * ny * nz), bytes = n * sizeof(float);
    float *h[6];
    void *dv[6] = {NULL, NULL, NULL, NULL, NULL, NULL};
    stencil3d_desc d;
    uint32_t s = 777u;
    for (int f = 0; f < 6; ++f) {
        h[f] = (float *)calloc(n, sizeof(float));
        EXPECT(h[f] != NULL);
    }
    for (int64_t z = 0; z < nz; ++z)
        for (int64_t y = 0; y < ny; ++y)
            for (int64_t x = 0; x < nx; ++x) {
                const size_t i = (size_t)((z * ny + y) * nx + x);
                const int in = x >= R && x < nx - R && y >= R && y < ny - R && z >= R && z < nz - R;
                for (int f = 0; f < 4; ++f) { /* LCG in [0, 1) */
                    s = s * 1664525u + 1013904223u;
                    const double r = (double)(s >> 8) / 16777216.0;
                    if (f < 2) h[f][i] = in ? (float)(2.0 * r - 1.0) : 0.0f;  /* u_prev, u */
                    else if (f == 2) h[f][i] = (float)(2.25e6 + r * (2.025e7 - 2.25e6));
                    else h[f][i] = (float)(0.1 * r);
                }
            }
    for (int f = 0; f < 6; ++f) {
        EXPECT(hipMalloc(&dv[f], bytes) == hipSuccess);
        EXPECT(hipMemcpy(dv[f], h[f], bytes, hipMemcpyHostToDevice) == hipSuccess);
    }
    const double trace[2] = {0.5, -0.25};
    EXPECT(stencil3d_desc_init(&d, ST_F32, nx, ny, nz, (int)R, ST_BC_HALO_UNTOUCHED) == ST_OK);
    EXPECT(wave_run_blocked(&d, dv[0], dv[1], dv[4], dv[5], dv[2], dv[3], 1e-3, 10.0, 2, 20, 11,
                            9, trace, NULL) == ST_OK);
    EXPECT(hipDeviceSynchronize() == hipSuccess);
    FILE *fp = fopen(path, "wb");
    EXPECT(fp != NULL);
    for (int f = 0; f < 6; ++f) {
        if (f >= 4) EXPECT(hipMemcpy(h[f], dv[f], bytes, hipMemcpyDeviceToHost) == hipSuccess);
        EXPECT(fwrite(h[f], 1, bytes, fp) == bytes);
        hipFree(dv[f]);
    }
    fclose(fp);
    for (int f = 0; f < 6; ++f) free(h[f]);
    printf("gpu blocked run ok\n");
    return 0;
}

int main(int argc, char **argv) {
    if (argc >= 2 && strcmp(argv[1], "cpu") == 0) return cpu_checks();
    if (argc >= 3 && strcmp(argv[1], "gpu") == 0) return gpu_run(argv[2]);
    if (argc >= 3 && strcmp(argv[1], "blocked") == 0) return gpu_blocked(argv[2]);
    fprintf(stderr, "usage: %s cpu | gpu OUT.bin | blocked OUT.bin\n", argv[0]);
    return 2;
}
