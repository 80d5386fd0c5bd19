// mxgemm.hip -- host side of the NT MX block-scaled GEMM library: argument
// validation, configuration choice, kernel launch and the C ABI declared in
// include/mxgemm.h.
//
// Contract ("PyTorch 接上 FlyDSL", 5ulink.com, section "支持边界"): A
// row-major, B column-major, K a multiple of 128, MXFP8/MXFP4 inputs with
// one E8M0 scale per 32 values, FP32 accumulation, FP16/BF16 output; any
// unsupported combination is reported so the caller can fall back.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/mxgemm.h"
#include "mx_direct.hpp"

using namespace mxg;

namespace {

thread_local int g_last_hip_error = 0;

// ------------------------------------------------------------------ variants
typedef void (*KernelFn)(GemmArgs);

struct Variant {
    const char *name;
    int tile_m, tile_n;   // workgroup output tile
    int threads;
    // [fmt][out][split]
    KernelFn fn[2][3][2];
};

#define MXG_FN(F, WM, WN, AM, AN, D, O, S) (&mx_gemm_direct<F, WM, WN, AM, AN, D, O, S>)
#define MXG_OUTS(F, WM, WN, AM, AN, D)                                                        \
    {{MXG_FN(F, WM, WN, AM, AN, D, OUT_BF16, false), MXG_FN(F, WM, WN, AM, AN, D, OUT_BF16, true)}, \
     {MXG_FN(F, WM, WN, AM, AN, D, OUT_F16, false), MXG_FN(F, WM, WN, AM, AN, D, OUT_F16, true)},   \
     {MXG_FN(F, WM, WN, AM, AN, D, OUT_F32, false), MXG_FN(F, WM, WN, AM, AN, D, OUT_F32, true)}}
#define MXG_VARIANT(NAME, WM, WN, AM, AN, D8, D4)                                              \
    {NAME, WM * AM * 16, WN * AN * 16, 64 * AM * AN,                                           \
     {MXG_OUTS(FMT_FP8, WM, WN, AM, AN, D8), MXG_OUTS(FMT_FP4, WM, WN, AM, AN, D4)}}

const Variant kVariants[] = {
    MXG_VARIANT("direct_16x64_w1x4", 1, 1, 1, 4, 8, 8),
    MXG_VARIANT("direct_32x64_w1x4", 2, 1, 1, 4, 4, 8),
    MXG_VARIANT("direct_64x64_w1x4", 4, 1, 1, 4, 4, 8),
    MXG_VARIANT("direct_64x64_w2x2", 2, 2, 2, 2, 4, 4),
    MXG_VARIANT("direct_128x128_w2x2", 4, 4, 2, 2, 2, 2),
};
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

// ---------------------------------------------------------------- validation
int validate(const void *a, const void *b, const void *sa, const void *sb, const void *c,
             int64_t M, int64_t N, int64_t K, int out_dtype)
{
    if (!a || !b || !sa || !sb || !c)
        return MXG_ERR_NULL;
    if (M < 1 || N < 1 || K < 1)
        return MXG_ERR_SHAPE;
    if (K % 128 != 0)
        return MXG_ERR_K_ALIGN;
    // kernels index rows with int and steps with int; sizes in size_t
    if (M > INT32_MAX || N > INT32_MAX || K / 128 > INT32_MAX / 4)
        return MXG_ERR_SHAPE;
    if (M > INT64_MAX / N || M > INT64_MAX / K || N > INT64_MAX / K)
        return MXG_ERR_SHAPE;
    if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 15u)
        return MXG_ERR_PTR_ALIGN;
    if (((uintptr_t)sa | (uintptr_t)sb) & 3u)
        return MXG_ERR_PTR_ALIGN;
    if (out_dtype < MXG_OUT_BF16 || out_dtype > MXG_OUT_F32)
        return MXG_ERR_DTYPE;
    return MXG_OK;
}

// gfx950 check, once per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 ok, 2 not gfx950

int check_device()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXG_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return MXG_ERR_DEVICE;
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            g_last_hip_error = (int)e;
            return MXG_ERR_HIP;
        }
        st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? MXG_OK : MXG_ERR_DEVICE;
}

// ------------------------------------------------------------ configuration
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_for(int variant, int split_k, int64_t M, int64_t N)
{
    if (split_k <= 1)
        return 0;
    const Variant &v = kVariants[variant];
    size_t tiles = (size_t)cdiv(M, v.tile_m) * (size_t)cdiv(N, v.tile_n);
    return align256(tiles * sizeof(unsigned)) + (size_t)split_k * (size_t)M * (size_t)N * sizeof(float);
}

int pick_variant(int64_t M)
{
    if (M <= 16) return 0;
    if (M <= 32) return 1;
    if (M <= 64) return 2;
    if (M <= 256) return 3;
    return 4;
}

// Enough workgroups to give every SIMD of the 256 CUs about two waves; each
// split keeps at least four 128-deep steps.
int pick_splits(int variant, int64_t M, int64_t N, int64_t K)
{
    const Variant &v = kVariants[variant];
    int64_t tiles = cdiv(M, v.tile_m) * cdiv(N, v.tile_n);
    int64_t waves_per_wg = v.threads / 64;
    int64_t target_wgs = (256 * 4 * 2 + waves_per_wg - 1) / waves_per_wg;
    int64_t s = cdiv(target_wgs, tiles);
    int64_t max_s = (K / 128) / 4;
    if (s > max_s) s = max_s;
    if (s > 16) s = 16;
    if (s < 1) s = 1;
    return (int)s;
}

int launch(int is_fp4, const void *a, const void *b, const void *sa, const void *sb, void *c,
           int64_t M, int64_t N, int64_t K, int out_dtype, int variant, int split_k,
           void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const Variant &v = kVariants[variant];
    GemmArgs p;
    p.a = (const uint8_t *)a;
    p.b = (const uint8_t *)b;
    p.sa = (const uint8_t *)sa;
    p.sb = (const uint8_t *)sb;
    p.c = c;
    p.M = (int)M;
    p.N = (int)N;
    p.ksteps = (int)(K / 128);
    p.splits = split_k;
    p.part = nullptr;
    p.cnt = nullptr;
    const int64_t gx = cdiv(N, v.tile_n), gy = cdiv(M, v.tile_m);
    if (gx > INT32_MAX || gy > 65535)
        return MXG_ERR_SHAPE;
    if (split_k > 1) {
        size_t need = workspace_for(variant, split_k, M, N);
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
            return MXG_ERR_WORKSPACE;
        size_t tiles = (size_t)gx * (size_t)gy;
        p.cnt = (unsigned *)workspace;
        p.part = (float *)((char *)workspace + align256(tiles * sizeof(unsigned)));
    }
    KernelFn fn = v.fn[is_fp4 ? 1 : 0][out_dtype][split_k > 1 ? 1 : 0];
    dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)split_k);
    hipLaunchKernelGGL(fn, grid, dim3(v.threads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXG_ERR_HIP;
    }
    return MXG_OK;
}

int run_default(int is_fp4, const void *a, const void *b, const void *sa, const void *sb, void *c,
                int64_t M, int64_t N, int64_t K, int out_dtype, void *workspace,
                size_t workspace_bytes, hipStream_t stream)
{
    int rc = validate(a, b, sa, sb, c, M, N, K, out_dtype);
    if (rc)
        return rc;
    int variant = pick_variant(M);
    int s = pick_splits(variant, M, N, K);
    if (s > 1 && (!workspace || workspace_bytes < workspace_for(variant, s, M, N) ||
                  ((uintptr_t)workspace & 255u)))
        s = 1;
    rc = check_device();
    if (rc)
        return rc;
    return launch(is_fp4, a, b, sa, sb, c, M, N, K, out_dtype, variant, s, workspace,
                  workspace_bytes, stream);
}

}  // namespace

extern "C" {

int mx_scaled_mm_fp4(const void *a, const void *b, const void *a_scale, const void *b_scale,
                     void *c, int64_t M, int64_t N, int64_t K, int out_dtype, void *workspace,
                     size_t workspace_bytes, mxg_stream_t stream)
{
    return run_default(1, a, b, a_scale, b_scale, c, M, N, K, out_dtype, workspace,
                       workspace_bytes, (hipStream_t)stream);
}

int mx_scaled_mm_fp8(const void *a, const void *b, const void *a_scale, const void *b_scale,
                     void *c, int64_t M, int64_t N, int64_t K, int out_dtype, void *workspace,
                     size_t workspace_bytes, mxg_stream_t stream)
{
    return run_default(0, a, b, a_scale, b_scale, c, M, N, K, out_dtype, workspace,
                       workspace_bytes, (hipStream_t)stream);
}

size_t mx_scaled_mm_workspace_bytes(int is_fp4, int64_t M, int64_t N, int64_t K)
{
    (void)is_fp4;
    if (M < 1 || N < 1 || K < 128 || K % 128)
        return 0;
    int variant = pick_variant(M);
    return workspace_for(variant, pick_splits(variant, M, N, K), M, N);
}

int mx_default_config(int is_fp4, int64_t M, int64_t N, int64_t K, size_t workspace_bytes,
                      int *variant, int *split_k)
{
    (void)is_fp4;
    if (!variant || !split_k)
        return MXG_ERR_NULL;
    if (M < 1 || N < 1 || K < 1)
        return MXG_ERR_SHAPE;
    if (K % 128)
        return MXG_ERR_K_ALIGN;
    int v = pick_variant(M);
    int s = pick_splits(v, M, N, K);
    if (s > 1 && workspace_bytes < workspace_for(v, s, M, N))
        s = 1;
    *variant = v;
    *split_k = s;
    return MXG_OK;
}

int mx_scaled_mm_config(int is_fp4, const void *a, const void *b, const void *a_scale,
                        const void *b_scale, void *c, int64_t M, int64_t N, int64_t K,
                        int out_dtype, int variant, int split_k, void *workspace,
                        size_t workspace_bytes, mxg_stream_t stream)
{
    int rc = validate(a, b, a_scale, b_scale, c, M, N, K, out_dtype);
    if (rc)
        return rc;
    if (variant < 0 || variant >= kNumVariants || split_k < 1 || split_k > K / 128 ||
        split_k > 65535)
        return MXG_ERR_CONFIG;
    if (split_k > 1 && (!workspace || workspace_bytes < workspace_for(variant, split_k, M, N) ||
                        ((uintptr_t)workspace & 255u)))
        return MXG_ERR_WORKSPACE;
    rc = check_device();
    if (rc)
        return rc;
    return launch(is_fp4, a, b, a_scale, b_scale, c, M, N, K, out_dtype, variant, split_k,
                  workspace, workspace_bytes, (hipStream_t)stream);
}

size_t mx_config_workspace_bytes(int variant, int split_k, int64_t M, int64_t N)
{
    if (variant < 0 || variant >= kNumVariants || M < 1 || N < 1)
        return 0;
    return workspace_for(variant, split_k, M, N);
}

int mx_num_variants(void) { return kNumVariants; }

const char *mx_variant_name(int variant)
{
    if (variant < 0 || variant >= kNumVariants)
        return nullptr;
    return kVariants[variant].name;
}

const char *mx_status_string(int status)
{
    switch (status) {
    case MXG_OK: return "ok";
    case MXG_ERR_NULL: return "null pointer argument";
    case MXG_ERR_SHAPE: return "invalid shape (M, N, K must be >= 1 and fit the kernels' index range)";
    case MXG_ERR_K_ALIGN: return "K is not a multiple of 128";
    case MXG_ERR_PTR_ALIGN: return "misaligned pointer (operands and C need 16 bytes, scales 4 bytes)";
    case MXG_ERR_DTYPE: return "unknown output dtype";
    case MXG_ERR_WORKSPACE: return "workspace missing, misaligned or too small for the requested split-K";
    case MXG_ERR_DEVICE: return "current device is not gfx950";
    case MXG_ERR_HIP: return "HIP runtime error";
    case MXG_ERR_CONFIG: return "invalid kernel variant or split count";
    default: return "unknown status";
    }
}

int mx_last_hip_error(void) { return g_last_hip_error; }

int mx_abi_version(void) { return MXGEMM_ABI_VERSION; }

}  // extern "C"
