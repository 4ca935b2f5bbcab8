/* A plain C99 caller of libulysses.so through include/ulysses.h.
 *
 *   abi_c_check host   plan calls and error paths only (no GPU needed)
 *   abi_c_check gpu    mode 0 then mode 1 of a W=3 uneven bf16 geometry on
 *                      the device; the round trip must return the input
 *
 * Prints "OK ..." and exits 0, or prints the failure and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ulysses.h"

#define FAIL(...)                         \
    do {                                  \
        fprintf(stderr, "FAIL: ");        \
        fprintf(stderr, __VA_ARGS__);     \
        fprintf(stderr, "\n");            \
        return 1;                         \
    } while (0)

static int host_checks(void) {
    const int64_t seq[3] = {5, 0, 7}, head[3] = {2, 3, 1};
    ulysses_plan *plan = NULL;
    int64_t shape[4];
    if (ulysses_plan_create(&plan, 3, 2, 64, seq, head, ULYSSES_BF16, 0) != ULYSSES_OK)
        FAIL("plan_create: %s", ulysses_last_error());
    if (ulysses_plan_shape(plan, 0, 0, 1, shape) != ULYSSES_OK || shape[0] != 2 ||
        shape[1] != 12 || shape[2] != 2 || shape[3] != 64)
        FAIL("mode-0 output shape of rank 0");
    if (ulysses_plan_shape(plan, 1, 2, 1, shape) != ULYSSES_OK || shape[1] != 7 || shape[2] != 6)
        FAIL("mode-1 output shape of rank 2");
    if (ulysses_plan_window_bytes(plan, 0) != 12 * 3 * 64 * 2) FAIL("window bytes");
    if (ulysses_plan_bytes(plan, 1) != 2LL * 2 * 12 * 6 * 64 * 2) FAIL("plan bytes");
    if (ulysses_plan_shape(plan, 2, 0, 0, shape) != ULYSSES_EINVAL) FAIL("bad mode accepted");
    if (ulysses_a2a_4d(plan, 0, NULL, NULL, 0) != ULYSSES_EINVAL) FAIL("null arrays accepted");
    if (strlen(ulysses_last_error()) == 0) FAIL("no error message");
    ulysses_plan_destroy(plan);
    if (ulysses_plan_create(&plan, 3, 1, 12, seq, head, ULYSSES_BF16, 0) != ULYSSES_EALIGN)
        FAIL("24-byte rows accepted");
    if (plan != NULL) FAIL("plan set on error");
    ulysses_plan_destroy(NULL);
    return 0;
}

static int gpu_checks(void) {
    const int world = 3;
    const int64_t b = 2, d = 128, seq[3] = {70, 1, 33}, head[3] = {3, 2, 4};
    ulysses_plan *plan = NULL;
    void *x[3], *y[3], *z[3];
    uint16_t *host[3], *back;
    size_t nbytes[3];
    int r, rc = 0;
    if (ulysses_plan_create(&plan, world, b, d, seq, head, ULYSSES_BF16, 0) != ULYSSES_OK)
        FAIL("plan_create: %s", ulysses_last_error());
    for (r = 0; r < world; ++r) {
        int64_t in[4], mid[4];
        size_t i, n;
        ulysses_plan_shape(plan, 0, r, 0, in);
        ulysses_plan_shape(plan, 0, r, 1, mid);
        n = (size_t)(in[0] * in[1] * in[2] * in[3]);
        nbytes[r] = n * 2;
        host[r] = (uint16_t *)malloc(nbytes[r]);
        for (i = 0; i < n; ++i) host[r][i] = (uint16_t)(i * 2654435761u >> 7) ^ (uint16_t)r;
        if (hipMalloc(&x[r], nbytes[r]) != hipSuccess ||
            hipMalloc(&y[r], (size_t)(mid[0] * mid[1] * mid[2] * mid[3]) * 2) != hipSuccess ||
            hipMalloc(&z[r], nbytes[r]) != hipSuccess)
            FAIL("hipMalloc");
        if (hipMemcpy(x[r], host[r], nbytes[r], hipMemcpyHostToDevice) != hipSuccess)
            FAIL("hipMemcpy to device");
    }
    if (ulysses_a2a_4d(plan, 0, (const void *const *)x, y, 0) != ULYSSES_OK)
        FAIL("mode 0: %s", ulysses_last_error());
    if (ulysses_a2a_4d(plan, 1, (const void *const *)y, z, 0) != ULYSSES_OK)
        FAIL("mode 1: %s", ulysses_last_error());
    if (hipDeviceSynchronize() != hipSuccess) FAIL("synchronize");
    for (r = 0; r < world; ++r) {
        back = (uint16_t *)malloc(nbytes[r]);
        if (hipMemcpy(back, z[r], nbytes[r], hipMemcpyDeviceToHost) != hipSuccess)
            FAIL("hipMemcpy to host");
        if (memcmp(back, host[r], nbytes[r]) != 0) rc = 1;
        free(back);
        free(host[r]);
        hipFree(x[r]);
        hipFree(y[r]);
        hipFree(z[r]);
    }
    ulysses_plan_destroy(plan);
    if (rc) FAIL("mode 1 after mode 0 did not return the input");
    return 0;
}

int main(int argc, char **argv) {
    int rc;
    if (argc != 2) FAIL("usage: abi_c_check host|gpu");
    rc = strcmp(argv[1], "gpu") == 0 ? gpu_checks() : host_checks();
    if (rc == 0) printf("OK %s\n", argv[1]);
    return rc;
}
