/*
 * abi_smoke.c — libtpshard.so used from plain C through include/tpshard.h.
 *
 *   abi_smoke host ndim d_0 .. d_{ndim-1} elem_bytes n_axes s_0 .. mask_0 ..
 *       host-only calls: tp_version, tp_shard_shape on the given tensor and
 *       mesh (prints "shape l_0 .. bytes B total T" or "status S"), a
 *       workspace query, and an argument the library must refuse.
 *   abi_smoke gpu N k n
 *       Y = X W (bf16 out) and P = X W (fp32 out) on device buffers from
 *       hipMalloc, inputs small integers, against the exact products
 *       computed here (Y rounded to bf16, nearest even). Prints "ok" or the
 *       first mismatch.
 * Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tpshard.h"

static uint16_t bf16_of(float x) {  /* round to nearest even (finite x) */
    uint32_t b;
    memcpy(&b, &x, 4);
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

static float f32_of_bf16(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float x;
    memcpy(&x, &b, 4);
    return x;
}

static int host_mode(int argc, char** argv) {
    int i = 2;
    if (argc < 4) return 2;
    const int32_t ndim = atoi(argv[i++]);
    int64_t shape[8], sizes[32], local[8], bytes = 0, total = 0;
    uint32_t mask[8];
    if (ndim < 1 || ndim > 8) return 2;
    for (int d = 0; d < ndim; ++d) shape[d] = atoll(argv[i++]);
    const int32_t elem = atoi(argv[i++]);
    const int32_t n_axes = atoi(argv[i++]);
    if (n_axes < 0 || n_axes > 32 || argc < i + n_axes + ndim) return 2;
    for (int a = 0; a < n_axes; ++a) sizes[a] = atoll(argv[i++]);
    for (int d = 0; d < ndim; ++d) mask[d] = (uint32_t)strtoul(argv[i++], NULL, 10);
    printf("version %d\n", tp_version());
    const tp_status st = tp_shard_shape(ndim, shape, elem, n_axes, sizes, mask, local, &bytes, &total);
    if (st == TP_OK) {
        printf("shape");
        for (int d = 0; d < ndim; ++d) printf(" %lld", (long long)local[d]);
        printf(" bytes %lld total %lld\n", (long long)bytes, (long long)total);
    } else {
        printf("status %d %s\n", (int)st, tp_last_error());
    }
    size_t ws = 0;
    if (tp_col_linear_workspace_size(16, 8192, 1280, TP_ACT_NONE, &ws) != TP_OK) return 1;
    printf("workspace %zu\n", ws);
    /* k = 100 is not a multiple of 64: refused before anything is enqueued */
    const tp_status bad = tp_col_linear(NULL, NULL, NULL, 4, 100, 64, TP_ACT_NONE, NULL, NULL, 0, NULL);
    printf("refused %d %s\n", (int)bad, tp_last_error());
    return bad == TP_ERR_UNSUPPORTED ? 0 : 1;
}

#define HIP_OK(x)                                                                     \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            printf("hip error %s at line %d\n", hipGetErrorString(e_), __LINE__);     \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

static int gpu_mode(int argc, char** argv) {
    if (argc < 5) return 2;
    const int64_t N = atoll(argv[2]), k = atoll(argv[3]), n = atoll(argv[4]);
    if (N < 1 || k < 64 || n < 64 || N * k > (1 << 26) || k * n > (1 << 26)) return 2;
    uint16_t* X = malloc(sizeof(uint16_t) * N * k);
    uint16_t* W = malloc(sizeof(uint16_t) * k * n);
    uint16_t* Y = malloc(sizeof(uint16_t) * N * n);
    float* P = malloc(sizeof(float) * N * n);
    int64_t* exact = malloc(sizeof(int64_t) * N * n);
    if (!X || !W || !Y || !P || !exact) return 1;
    uint32_t s = 2024u;  /* small integers in [-2, 2] */
    for (int64_t i = 0; i < N * k; ++i) { s = s * 1664525u + 1013904223u; X[i] = bf16_of((float)((int)(s >> 28) % 5 - 2)); }
    for (int64_t i = 0; i < k * n; ++i) { s = s * 1664525u + 1013904223u; W[i] = bf16_of((float)((int)(s >> 28) % 5 - 2)); }
    for (int64_t r = 0; r < N; ++r)
        for (int64_t c = 0; c < n; ++c) {
            int64_t acc = 0;
            for (int64_t j = 0; j < k; ++j) acc += (int64_t)f32_of_bf16(X[r * k + j]) * (int64_t)f32_of_bf16(W[j * n + c]);
            exact[r * n + c] = acc;
        }
    void *dX, *dW, *dY, *dP, *dws = NULL;
    size_t ws_col = 0, ws_row = 0;
    if (tp_col_linear_workspace_size(N, k, n, TP_ACT_NONE, &ws_col) != TP_OK) return 1;
    if (tp_row_linear_partial_workspace_size(N, k, n, &ws_row) != TP_OK) return 1;
    const size_t ws = ws_col > ws_row ? ws_col : ws_row;
    HIP_OK(hipMalloc(&dX, sizeof(uint16_t) * N * k));
    HIP_OK(hipMalloc(&dW, sizeof(uint16_t) * k * n));
    HIP_OK(hipMalloc(&dY, sizeof(uint16_t) * N * n));
    HIP_OK(hipMalloc(&dP, sizeof(float) * N * n));
    if (ws) HIP_OK(hipMalloc(&dws, ws));
    HIP_OK(hipMemcpy(dX, X, sizeof(uint16_t) * N * k, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dW, W, sizeof(uint16_t) * k * n, hipMemcpyHostToDevice));
    tp_status st = tp_col_linear(dX, dW, dY, N, k, n, TP_ACT_NONE, NULL, dws, ws, NULL);
    if (st != TP_OK) { printf("tp_col_linear: %d %s\n", (int)st, tp_last_error()); return 1; }
    st = tp_row_linear_partial(dX, dW, (float*)dP, N, k, n, 0, dws, ws, NULL);
    if (st != TP_OK) { printf("tp_row_linear_partial: %d %s\n", (int)st, tp_last_error()); return 1; }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(Y, dY, sizeof(uint16_t) * N * n, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(P, dP, sizeof(float) * N * n, hipMemcpyDeviceToHost));
    int bad = 0;
    for (int64_t i = 0; i < N * n && !bad; ++i) {
        if (Y[i] != bf16_of((float)exact[i])) {
            printf("Y mismatch at %lld: %04x, want %04x\n", (long long)i, Y[i], bf16_of((float)exact[i]));
            bad = 1;
        } else if (P[i] != (float)exact[i]) {
            printf("P mismatch at %lld: %g, want %lld\n", (long long)i, P[i], (long long)exact[i]);
            bad = 1;
        }
    }
    HIP_OK(hipFree(dX));
    HIP_OK(hipFree(dW));
    HIP_OK(hipFree(dY));
    HIP_OK(hipFree(dP));
    if (dws) HIP_OK(hipFree(dws));
    free(X); free(W); free(Y); free(P); free(exact);
    if (!bad) printf("ok %lld x %lld x %lld, workspace %zu\n", (long long)N, (long long)k, (long long)n, ws);
    return bad;
}

int main(int argc, char** argv) {
    if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_mode(argc, argv);
    if (argc >= 2 && strcmp(argv[1], "gpu") == 0) return gpu_mode(argc, argv);
    fprintf(stderr, "usage: abi_smoke host ... | abi_smoke gpu N k n\n");
    return 2;
}
