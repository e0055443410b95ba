// Host-only check of the C ABI's argument validation: validate.cpp compiled
// with the system C++ compiler and no HIP header.  Prints "validate ok" and
// exits 0 when every rule gives the documented status.
#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "stencil3d.h"
#include "validate.h"

using namespace st::check;

static int failures = 0;
#define EXPECT(cond)                                                     \
    do {                                                                 \
        if (!(cond)) {                                                   \
            printf("FAILED line %d: %s\n", __LINE__, #cond);             \
            ++failures;                                                  \
        }                                                                \
    } while (0)

int main() {
    stencil3d_desc d;
    // descriptor
    EXPECT(init(&d, ST_F32, 20, 21, 22, 4, ST_BC_HALO_UNTOUCHED) == ST_OK);
    EXPECT(d.struct_size == sizeof(stencil3d_desc) && d.radius == 4);
    EXPECT(d.cx[0] == -205.0 / 72.0 && d.cz[4] == -1.0 / 560.0 && d.pml_width == 0);
    EXPECT(desc(nullptr) == ST_ERR_NULL);
    EXPECT(init(nullptr, ST_F32, 9, 9, 9, 1, 0) == ST_ERR_NULL);
    EXPECT(init(&d, ST_F32, 9, 9, 9, 5, 0) == ST_ERR_RADIUS);
    EXPECT(init(&d, 7, 9, 9, 9, 1, 0) == ST_ERR_DTYPE);
    EXPECT(init(&d, ST_F32, 9, 9, 9, 1, 2) == ST_ERR_BOUNDARY);
    EXPECT(init(&d, ST_F32, 2, 9, 9, 1, 0) == ST_ERR_DIMS);       // < 2R+1
    EXPECT(init(&d, ST_F32, 3, 3, 3, 1, 0) == ST_OK);             // == 2R+1
    EXPECT(init(&d, ST_F32, 1L << 31, 3, 3, 1, 0) == ST_ERR_DIMS);
    EXPECT(init(&d, ST_F64, 1L << 14, 1L << 14, 3, 1, 0) == ST_ERR_DIMS);  // 2 GiB plane
    EXPECT(init(&d, ST_F32, 1L << 14, 1L << 14, 3, 1, 0) == ST_OK);        // 1 GiB plane
    init(&d, ST_F32, 9, 9, 9, 1, 0);
    d.struct_size = 8;
    EXPECT(desc(&d) == ST_ERR_STRUCT_SIZE);
    init(&d, ST_F32, 9, 9, 9, 1, 0);
    d.cy[1] = NAN;
    EXPECT(desc(&d) == ST_ERR_COEFF);
    d.cy[1] = 1.0;
    d.cz[3] = NAN;  // above R: ignored
    EXPECT(desc(&d) == ST_OK);
    d.pml_width = -1;
    EXPECT(desc(&d) == ST_ERR_ARG);
    d.pml_width = INT64_MAX;
    EXPECT(desc(&d) == ST_OK);
    EXPECT(elem_size(&d) == 4);

    // pointers: fields of 9^3 fp32 = 2916 bytes, placed 4096 apart
    init(&d, ST_F32, 9, 9, 9, 1, 0);
    const char *base = (const char *)0x10000000;
    const void *A = base, *B = base + 4096, *C = base + 8192, *D = base + 12288,
               *E = base + 16384;
    EXPECT(apply_args(&d, A, B) == ST_OK);
    EXPECT(apply_args(&d, nullptr, B) == ST_ERR_NULL);
    EXPECT(apply_args(&d, base + 2, B) == ST_ERR_ALIGN);
    EXPECT(apply_args(&d, A, A) == ST_ERR_ALIAS);
    EXPECT(apply_args(&d, A, base + 2912) == ST_ERR_ALIAS);        // last element shared
    EXPECT(apply_args(&d, A, base + 2916) == ST_OK);               // adjacent
    EXPECT(jacobi_args(&d, A, B, 0) == ST_OK);
    EXPECT(jacobi_args(&d, A, B, -1) == ST_ERR_ARG);
    EXPECT(jacobi_args(&d, A, base + 4, 3) == ST_ERR_ALIAS);

    // wave step: u_next may be u_prev itself, nothing else
    EXPECT(wave_args(&d, A, B, C, D, E, 1e-3, 10.0) == ST_OK);
    EXPECT(wave_args(&d, A, B, A, D, E, 1e-3, 10.0) == ST_OK);
    EXPECT(wave_args(&d, A, B, base + 64, D, E, 1e-3, 10.0) == ST_ERR_ALIAS);
    EXPECT(wave_args(&d, A, B, B, D, E, 1e-3, 10.0) == ST_ERR_ALIAS);
    EXPECT(wave_args(&d, A, B, C, C, E, 1e-3, 10.0) == ST_ERR_ALIAS);
    EXPECT(wave_args(&d, A, B, C, D, C, 1e-3, 10.0) == ST_ERR_ALIAS);
    EXPECT(wave_args(&d, A, B, C, B, B, 1e-3, 10.0) == ST_OK);     // inputs may share
    EXPECT(wave_args(&d, A, B, C, D, E, NAN, 10.0) == ST_ERR_ARG);
    EXPECT(wave_args(&d, A, B, C, D, E, 1e-3, 0.0) == ST_ERR_ARG);
    EXPECT(wave_args(&d, A, B, C, D, E, 1e-3, -1.0) == ST_ERR_ARG);
    EXPECT(wave_args(&d, A, B, C, D, E, 1e-3, INFINITY) == ST_ERR_ARG);
    EXPECT(wave_args(&d, A, B, C, D, nullptr, 1e-3, 10.0) == ST_ERR_NULL);

    // source and time loop
    EXPECT(source_args(&d, A, 1, 1, 1, 1.0) == ST_OK);
    EXPECT(source_args(&d, A, 7, 7, 7, 1.0) == ST_OK);
    EXPECT(source_args(&d, A, 0, 1, 1, 1.0) == ST_ERR_BAD_INDEX);
    EXPECT(source_args(&d, A, 1, 8, 1, 1.0) == ST_ERR_BAD_INDEX);
    EXPECT(source_args(&d, A, 1, 1, 1, NAN) == ST_ERR_ARG);
    const double tr[3] = {0.1, 0.2, 0.3}, bad[3] = {0.1, 0.2, NAN};
    EXPECT(run_args(&d, A, B, D, E, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_OK);
    EXPECT(run_args(&d, A, B, D, E, 1e-3, 10.0, 3, 4, 4, 4, nullptr) == ST_OK);
    EXPECT(run_args(&d, A, B, D, E, 1e-3, 10.0, -1, 4, 4, 4, tr) == ST_ERR_ARG);
    EXPECT(run_args(&d, A, B, D, E, 1e-3, 10.0, 3, 4, 4, 4, bad) == ST_ERR_ARG);
    EXPECT(run_args(&d, A, B, D, E, 1e-3, 10.0, 2, 4, 4, 4, bad) == ST_OK);  // reads n only
    EXPECT(run_args(&d, A, B, D, E, 1e-3, 10.0, 3, 0, 4, 4, tr) == ST_ERR_BAD_INDEX);
    EXPECT(run_args(&d, A, base + 8, D, E, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_ERR_ALIAS);
    EXPECT(run_args(&d, A, B, A, E, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_ERR_ALIAS);
    // u is written in every other step: no overlap with vel2 or eta
    EXPECT(run_args(&d, A, B, B, E, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_ERR_ALIAS);
    EXPECT(run_args(&d, A, B, D, base + 4100, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_ERR_ALIAS);

    // time-blocked run: four u buffers written in turn, vel2 and eta
    const void *F = base + 20480, *G = base + 24576;
    EXPECT(blocked_args(&d, A, B, C, F, D, E, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_OK);
    EXPECT(blocked_args(&d, A, B, C, F, D, D, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_OK);
    EXPECT(blocked_args(&d, A, B, C, F, D, E, 1e-3, 10.0, -1, 4, 4, 4, tr) == ST_ERR_ARG);
    EXPECT(blocked_args(&d, A, B, C, F, D, E, 1e-3, 10.0, 3, 0, 4, 4, tr) == ST_ERR_BAD_INDEX);
    EXPECT(blocked_args(&d, A, B, nullptr, F, D, E, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_ERR_NULL);
    EXPECT(blocked_args(&d, A, B, C, base + 20482, D, E, 1e-3, 10.0, 3, 4, 4, 4, tr) ==
           ST_ERR_ALIGN);
    const void *bufs[6] = {A, B, C, F, D, E};
    for (int i = 0; i < 4; ++i)        // a u buffer ...
        for (int j = 0; j < 6; ++j) {  // ... on any other buffer, exact or shifted
            if (i == j) continue;
            for (int shift = 0; shift <= 4; shift += 4) {
                const void *p[6] = {bufs[0], bufs[1], bufs[2], bufs[3], bufs[4], bufs[5]};
                p[i] = (const char *)bufs[j] + shift;
                EXPECT(blocked_args(&d, p[0], p[1], p[2], p[3], p[4], p[5], 1e-3, 10.0, 3, 4, 4,
                                    4, tr) == ST_ERR_ALIAS);
            }
        }
    EXPECT(blocked_args(&d, A, B, C, G, D, E, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_OK);

    // no-allocation run: run_args plus the workspace limit
    EXPECT(noalloc_args(&d, A, B, D, E, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_OK);
    EXPECT(noalloc_args(&d, A, B, D, E, 1e-3, 10.0, -1, 4, 4, 4, tr) == ST_ERR_ARG);
    EXPECT(noalloc_args(&d, A, B, B, E, 1e-3, 10.0, 3, 4, 4, 4, tr) == ST_ERR_ALIAS);
    {
        stencil3d_desc big;
        // 128 x 128 x 512 fp32 = 32 MiB: the limit itself; one plane more is over
        EXPECT(init(&big, ST_F32, 128, 128, 512, 4, 0) == ST_OK);
        const char *far = (const char *)0x100000000;
        const void *P = far, *Q = far + (64 << 20), *S = far + (128 << 20),
                   *T = far + (192 << 20);
        EXPECT(noalloc_args(&big, P, Q, S, T, 1e-3, 10.0, 3, 8, 8, 8, tr) == ST_OK);
        big.nz = 513;
        EXPECT(noalloc_args(&big, P, Q, S, T, 1e-3, 10.0, 3, 8, 8, 8, tr) == ST_ERR_WORKSPACE);
        big.nz = 256;
        big.dtype = ST_F64;  // 128 x 128 x 256 fp64 = 32 MiB
        EXPECT(noalloc_args(&big, P, Q, S, T, 1e-3, 10.0, 3, 8, 8, 8, tr) == ST_OK);
        big.nz = 257;
        EXPECT(noalloc_args(&big, P, Q, S, T, 1e-3, 10.0, 3, 8, 8, 8, tr) == ST_ERR_WORKSPACE);
    }

    // messages
    EXPECT(strcmp(message(ST_OK), "ok") == 0);
    for (int c = ST_ERR_WORKSPACE; c < 0; ++c)  // every code has its own message
        EXPECT(strcmp(message(c), message(-99)) != 0);
    EXPECT(strcmp(message(-99), "unknown status code") == 0);

    if (failures) return 1;
    printf("validate ok\n");
    return 0;
}
