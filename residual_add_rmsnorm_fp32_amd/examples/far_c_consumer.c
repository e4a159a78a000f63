/*
 * far_c_consumer.c -- a plain C caller of the fused add + RMSNorm (+ fp8) library.
 *
 * Uses only include/far.h, libfar.so and the HIP runtime's C API: it fills P bf16
 * partials, a residual and gamma with small exactly representable values, runs the
 * epilogue with dynamic per-token fp8 quantisation and the new residual written in
 * place into the residual buffer, and prints every output as hexadecimal codes, one
 * JSON object per line, for a test to compare with the CPU oracle.
 *
 * Inputs (bf16 = the top 16 bits of the float, exact for these values):
 *   partial p [t][h] = ((7 t + 3 h + 5 p) mod 17 - 8) / 8
 *   residual  [t][h] = ((11 t + h) mod 13 - 6) / 4
 *   gamma     [h]    = 1 + ((h mod 9) - 4) / 16
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "far.h"

enum { P = 3, T = 5, H = 520 };

static uint16_t bf16_of(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    return (uint16_t)(u >> 16); /* exact: every value here has <= 8 significant bits */
}

#define HIP_OK(x)                                                          \
    do {                                                                   \
        hipError_t e_ = (x);                                               \
        if (e_ != hipSuccess) {                                            \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
            return 2;                                                      \
        }                                                                  \
    } while (0)

static void print_u16(const char *name, const uint16_t *a, int n) {
    printf("{\"%s\": [", name);
    for (int i = 0; i < n; ++i) printf("%s%u", i ? "," : "", a[i]);
    printf("]}\n");
}

int main(void) {
    static uint16_t hp[P][T * H], hr[T * H], hg[H], out_res[T * H];
    static uint8_t hq[T * H];
    static float hs[T];
    for (int p = 0; p < P; ++p)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h)
                hp[p][t * H + h] = bf16_of((float)((7 * t + 3 * h + 5 * p) % 17 - 8) / 8.0f);
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) hr[t * H + h] = bf16_of((float)((11 * t + h) % 13 - 6) / 4.0f);
    for (int h = 0; h < H; ++h) hg[h] = bf16_of(1.0f + (float)((h % 9) - 4) / 16.0f);

    void *dp[P], *dr, *dg, *dq;
    float *ds;
    for (int p = 0; p < P; ++p) {
        HIP_OK(hipMalloc(&dp[p], sizeof(hp[p])));
        HIP_OK(hipMemcpy(dp[p], hp[p], sizeof(hp[p]), hipMemcpyHostToDevice));
    }
    HIP_OK(hipMalloc(&dr, sizeof(hr)));
    HIP_OK(hipMemcpy(dr, hr, sizeof(hr), hipMemcpyHostToDevice));
    HIP_OK(hipMalloc(&dg, sizeof(hg)));
    HIP_OK(hipMemcpy(dg, hg, sizeof(hg), hipMemcpyHostToDevice));
    HIP_OK(hipMalloc(&dq, sizeof(hq)));
    HIP_OK(hipMalloc((void **)&ds, sizeof(hs)));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    const void *parts[P] = {dp[0], dp[1], dp[2]};
    /* in place: the new residual overwrites the residual buffer */
    far_status_t st = far_fused_add_rmsnorm(parts, P, dr, dg, T, H, FAR_DTYPE_BF16, 1e-6f, 0.0f,
                                            FAR_QUANT_FP8_DYNAMIC_TOKEN, NULL, NULL, dr, dq, ds,
                                            (far_stream_t)stream);
    if (st != FAR_OK) {
        fprintf(stderr, "far_fused_add_rmsnorm: %s\n", far_status_string(st));
        return 1;
    }
    /* an argument error is reported, not silently ignored */
    far_status_t bad = far_fused_add_rmsnorm(parts, P, dr, dg, T, H, FAR_DTYPE_BF16, 1e-6f, 0.0f,
                                             FAR_QUANT_FP8_DYNAMIC_TOKEN, NULL, NULL, dr, dq, NULL,
                                             (far_stream_t)stream);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(out_res, dr, sizeof(out_res), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hq, dq, sizeof(hq), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hs, ds, sizeof(hs), hipMemcpyDeviceToHost));

    printf("{\"P\": %d, \"T\": %d, \"H\": %d, \"version\": %d, \"missing_scale_out_status\": %d}\n", P, T,
           H, far_version(), (int)bad);
    print_u16("new_residual", out_res, T * H);
    printf("{\"quant_out\": [");
    for (int i = 0; i < T * H; ++i) printf("%s%u", i ? "," : "", hq[i]);
    printf("]}\n{\"scale_out\": [");
    for (int t = 0; t < T; ++t) printf("%s%.9e", t ? "," : "", (double)hs[t]);
    printf("]}\n");

    for (int p = 0; p < P; ++p) hipFree(dp[p]);
    hipFree(dr);
    hipFree(dg);
    hipFree(dq);
    hipFree(ds);
    hipStreamDestroy(stream);
    return 0;
}
