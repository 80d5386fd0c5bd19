/* Drives the host half of the C ABI (include/mxgemm.h) under
 * AddressSanitizer and UndefinedBehaviorSanitizer, linked against a build
 * of the library without device code (hipcc --offload-host-only): argument
 * validation, configuration choice, split-K part counts and workspace
 * sizes, name and status queries.  Calls that pass validation stop at the
 * device check (no GPU, or no kernel image in this build: MXG_ERR_DEVICE
 * or MXG_ERR_HIP), so no kernel ever starts on the fake addresses used
 * here.  Built and run by tests/test_sanitize_host.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/mxgemm.h"

#define CHECK(cond)                                                    \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                                  \
        }                                                              \
    } while (0)

#define STOPPED(rc) ((rc) == MXG_ERR_DEVICE || (rc) == MXG_ERR_HIP)

static const char *A = (const char *)0x10000;   /* aligned, never dereferenced on the host */

static int variant_named(const char *name)
{
    for (int v = 0; v < mx_num_variants(); ++v)
        if (strcmp(mx_variant_name(v), name) == 0)
            return v;
    return -1;
}

int main(void)
{
    void *a = (void *)A;
    CHECK(mx_abi_version() == MXGEMM_ABI_VERSION);
    for (int s = -12; s <= 1; ++s)
        CHECK(mx_status_string(s) != NULL);
    for (int v = -1; v <= mx_num_variants(); ++v)
        CHECK((mx_variant_name(v) != NULL) == (v >= 0 && v < mx_num_variants()));
    /* the default configuration and its workspace over a grid of shapes */
    const int64_t Ms[] = {1, 5, 16, 31, 32, 33, 64, 100, 128, 200, 256, 512, 2048, 8192};
    const int64_t Ns[] = {1, 7, 256, 4096, 14336, 25600, 28672};
    const int64_t Ks[] = {128, 256, 640, 4096, 5120, 8192, 14336, 1 << 20};
    for (int f = 0; f < 2; ++f)
        for (size_t i = 0; i < sizeof Ms / sizeof Ms[0]; ++i)
            for (size_t j = 0; j < sizeof Ns / sizeof Ns[0]; ++j)
                for (size_t k = 0; k < sizeof Ks / sizeof Ks[0]; ++k) {
                    int sp = 0;
                    const int v = mx_default_config(f, Ms[i], Ns[j], Ks[k], 1, &sp);
                    CHECK(v >= 0 && v < mx_num_variants() && sp >= 1);
                    CHECK(Ks[k] <= mx_variant_max_k(v, f) * sp);
                    const size_t need = mx_scaled_mm_workspace_bytes(f, Ms[i], Ns[j], Ks[k]);
                    CHECK(need == mx_config_workspace_bytes(v, sp, Ms[i], Ns[j]));
                    int sp0 = 0;
                    CHECK(mx_default_config(f, Ms[i], Ns[j], Ks[k], 0, &sp0) >= 0 && sp0 == 1);
                }
    /* valid calls get as far as the device */
    int rc = mx_scaled_mm_fp4(a, a, a, a, a, 512, 4096, 4096, MXG_OUT_BF16, NULL, 0, NULL);
    CHECK(STOPPED(rc));
    rc = mx_scaled_mm_fp8(a, a, a, a, a, 64, 4096, 4096, MXG_OUT_F32, a, 1, NULL);
    CHECK(STOPPED(rc));
    const int tile = variant_named("tile_128x128"), dec = variant_named("decode_32x64");
    CHECK(tile >= 0 && dec >= 0);
    const size_t need = mx_config_workspace_bytes(tile, 2, 512, 4096);
    CHECK(need > 0);
    rc = mx_scaled_mm_config(1, a, a, a, a, a, 512, 4096, 4096, 0, tile, 2, a, need, NULL);
    CHECK(STOPPED(rc));
    rc = mx_scaled_mm_config(1, a, a, a, a, a, 512, 4096, 4096, 0, tile, 8, a, (size_t)1 << 40, NULL);
    CHECK(STOPPED(rc));
    CHECK(mx_scaled_mm_config(1, a, a, a, a, a, 32, 14336, 4096, 0, dec, 2, a, (size_t)1 << 40, NULL) ==
          MXG_ERR_CONFIG);
    rc = mx_empty_like(1, 32, 256, 256, NULL);
    CHECK(STOPPED(rc));
    /* the allocation-free entry point: validation, then the device */
    CHECK(mx_noalloc_scratch_bytes() >= mx_scaled_mm_workspace_bytes(1, 512, 4096, 14336));
    CHECK(STOPPED(mx_scaled_mm_noalloc(1, a, a, a, a, a, 512, 4096, 14336, 0, NULL)));
    CHECK(STOPPED(mx_scaled_mm_noalloc(0, a, a, a, a, a, 64, 4096, 4096, 2, NULL)));
    CHECK(mx_scaled_mm_noalloc(1, a, a, a, a, NULL, 8, 8, 128, 0, NULL) == MXG_ERR_NULL);
    CHECK(mx_scaled_mm_noalloc(1, a, a, a, a, a, 8, 8, 100, 0, NULL) == MXG_ERR_K_ALIGN);
    /* rejected calls */
    CHECK(mx_scaled_mm_config(1, a, a, a, a, a, 512, 4096, 4096, 0, tile, 2, a, need - 1, NULL) ==
          MXG_ERR_WORKSPACE);
    CHECK(mx_scaled_mm_config(1, a, a, a, a, a, 512, 4096, 4096, 0, tile, 9, a, (size_t)1 << 40, NULL) ==
          MXG_ERR_CONFIG);
    CHECK(mx_scaled_mm_fp4(NULL, a, a, a, a, 8, 8, 128, 0, NULL, 0, NULL) == MXG_ERR_NULL);
    CHECK(mx_scaled_mm_fp4(a, a, a, a, a, 8, 8, 100, 0, NULL, 0, NULL) == MXG_ERR_K_ALIGN);
    CHECK(mx_quantize_bf16(a, a, a, 4, 48, 1, NULL) == MXG_ERR_K_ALIGN);
    CHECK(mx_grouped_mm_fp8(a, a, a, a, a, NULL, 4, 64, 8, 128, 0, NULL) == MXG_ERR_NULL);
    CHECK(mx_scaled_mm_fused(1, a, a, a, a, NULL, 9, a, NULL, 8, 64, 128, 0, -1, NULL) == MXG_ERR_CONFIG);
    CHECK(mx_dense_gemm(2, 0, 0, a, a, a, 8, 8, 8, 0, NULL) == MXG_ERR_DTYPE);
    puts("abi sanitizer run ok");
    return 0;
}
