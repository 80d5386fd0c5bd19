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
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/mxgemm.h"
#include "mx_decode.hpp"
#include "mx_dense.hpp"
#include "mx_quant.hpp"
#include "mx_stream.hpp"
#include "mx_tile.hpp"

using namespace mxg;

namespace {

thread_local int g_last_hip_error = 0;

// ------------------------------------------------------------------ variants
typedef void (*KernelFn)(GemmArgs);

struct Variant {
    const char *name;
    int bm, bn;              // workgroup output tile
    int threads;
    KernelFn fn[2][3];       // [fmt][out]
    int kmax[2];             // largest K per format (0: any K); with split-K, of one K part
    int linear;              // 1: one-dimensional grid, the kernel maps blocks to tiles
    int split;               // 1: the kernel takes split-K across workgroups (mx_splitk.hpp)
};

// Ring depth of the register-streaming kernel (groups in flight per wave)
// from a register budget: a ring slot holds 4 steps of every A and B
// subtile plus their scale codes.
constexpr int ring_depth(int fmt, int mt, int wn)
{
    return (mt + wn) * (fmt == FMT_FP4 ? 20 : 36) <= 80 ? 2 : 1;
}

#define MXG_SFN(F, MT, WN, KW, O) (&mx_gemm_stream<F, MT, WN, KW, ring_depth(F, MT, WN), O>)
#define MXG_SOUTS(F, MT, WN, KW) \
    {MXG_SFN(F, MT, WN, KW, OUT_BF16), MXG_SFN(F, MT, WN, KW, OUT_F16), MXG_SFN(F, MT, WN, KW, OUT_F32)}
// (split-K across workgroups only with KW > 1: its reduction runs on the
// workgroup's LDS-summed tile)
#define MXG_STREAM(MT, WN, KW)                                                        \
    {"stream_" #MT "x" #WN "_k" #KW, 16 * MT, 16 * WN, 64 * KW,                        \
     {MXG_SOUTS(FMT_FP8, MT, WN, KW), MXG_SOUTS(FMT_FP4, MT, WN, KW)}, {0, 0}, 0, (KW) > 1}

// Decode kernel: A tile of MT subtiles and all scale codes resident in LDS
// (K up to K8 / K4 for FP8 / FP4), NW groups of 16 B rows, each streamed by
// KS waves (one K part each) through private rings of G 256-byte stages,
// held in LDS slots that the loads write directly (DMA = 1) or in registers.
#define MXG_DFN(F, MT, NW, KM, G, O, KS, DMA) (&mx_gemm_decode<F, MT, NW, KM, G, O, KS, 0, DMA>)
#define MXG_DOUTS(F, MT, NW, KM, G, KS, DMA)                                                     \
    {MXG_DFN(F, MT, NW, KM, G, OUT_BF16, KS, DMA), MXG_DFN(F, MT, NW, KM, G, OUT_F16, KS, DMA),   \
     MXG_DFN(F, MT, NW, KM, G, OUT_F32, KS, DMA)}
#define MXG_DECODE(NAME, MT, NW, G, KS, K4, K8, DMA)                                           \
    {NAME, 16 * (MT), 16 * (NW), 64 * (NW) * (KS),                                             \
     {MXG_DOUTS(FMT_FP8, MT, NW, K8, G, KS, DMA), MXG_DOUTS(FMT_FP4, MT, NW, K4, G, KS, DMA)},   \
     {K8, K4}, 0, 0}

// Tiles on the 32x32x64 instruction, loaded straight into LDS: NS code
// slots of 128 bytes per row (four slots: three super-stages of prefetch).
#define MXG_TFN(F, MT, NT, NS, O) (&mx_gemm_tile<F, MT, NT, O, 0, 0, NS>)
#define MXG_TOUTS(F, MT, NT, NS) \
    {MXG_TFN(F, MT, NT, NS, OUT_BF16), MXG_TFN(F, MT, NT, NS, OUT_F16), MXG_TFN(F, MT, NT, NS, OUT_F32)}
#define MXG_TILE(NAME, MT, NT, NS)          \
    {NAME, 64 * (MT), 64 * (NT), 256,       \
     {MXG_TOUTS(FMT_FP8, MT, NT, NS), MXG_TOUTS(FMT_FP4, MT, NT, NS)}, {0, 0}, 1, 1}

const Variant kVariants[] = {
    MXG_STREAM(1, 1, 4),
    MXG_STREAM(1, 1, 16),
    MXG_STREAM(1, 2, 4),
    MXG_STREAM(2, 1, 4),
    MXG_STREAM(2, 2, 4),
    MXG_STREAM(2, 4, 8),
    MXG_STREAM(4, 2, 8),
    MXG_STREAM(2, 1, 1),
    MXG_STREAM(2, 1, 2),
    MXG_STREAM(1, 1, 1),
    MXG_STREAM(1, 1, 2),
    //          name              MT NW G  KS K4    K8    DMA
    MXG_DECODE("decode_32x64",    2, 4, 3, 1, 4096, 2048, 1),
    MXG_DECODE("decode_16x64",    1, 4, 3, 1, 4096, 2048, 1),
    MXG_DECODE("decode_32x64_k2", 2, 4, 2, 2, 4096, 2048, 0),
    // the same with room for a longer A tile (more LDS: 1-2% slower at K <= 4096)
    MXG_DECODE("decode_32x64_k2_long", 2, 4, 2, 2, 5120, 2048, 0),
    MXG_DECODE("decode_16x64_k2_long", 1, 4, 2, 2, 8192, 2048, 0),
    //        name               MT NT NS
    MXG_TILE("tile_256x256",     4, 4, 2),
    MXG_TILE("tile_256x128",     4, 2, 2),
    MXG_TILE("tile_128x256",     2, 4, 2),
    MXG_TILE("tile_128x128",     2, 2, 2),
    MXG_TILE("tile_128x128_r4",  2, 2, 4),
    MXG_TILE("tile_64x64_r4",    1, 1, 4),
};
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

// Grouped products: the same kernels with the group lookup at the start.
#define MXG_GSFN(F, MT, WN, KW, O) (&mx_gemm_stream<F, MT, WN, KW, ring_depth(F, MT, WN), O, 1>)
#define MXG_GSOUTS(F, MT, WN, KW) \
    {MXG_GSFN(F, MT, WN, KW, OUT_BF16), MXG_GSFN(F, MT, WN, KW, OUT_F16), MXG_GSFN(F, MT, WN, KW, OUT_F32)}
#define MXG_GSTREAM(MT, WN, KW)                                                       \
    {"gstream_" #MT "x" #WN "_k" #KW, 16 * MT, 16 * WN, 64 * KW,                       \
     {MXG_GSOUTS(FMT_FP8, MT, WN, KW), MXG_GSOUTS(FMT_FP4, MT, WN, KW)}, {0, 0}, 0, 0}
#define MXG_GTFN(F, MT, NT, O) (&mx_gemm_tile<F, MT, NT, O, 1>)
#define MXG_GTOUTS(F, MT, NT) \
    {MXG_GTFN(F, MT, NT, OUT_BF16), MXG_GTFN(F, MT, NT, OUT_F16), MXG_GTFN(F, MT, NT, OUT_F32)}
#define MXG_GTILE(NAME, MT, NT)                                                     \
    {NAME, 64 * (MT), 64 * (NT), 256,                                               \
     {MXG_GTOUTS(FMT_FP8, MT, NT), MXG_GTOUTS(FMT_FP4, MT, NT)}, {0, 0}, 1, 0}

const Variant kGroupVariants[] = {
    MXG_GSTREAM(1, 2, 4),
    MXG_GSTREAM(2, 4, 8),
    MXG_GTILE("gtile_128x128", 2, 2),
    MXG_GTILE("gtile_256x128", 4, 2),
    MXG_GTILE("gtile_256x256", 4, 4),
};
constexpr int kNumGroupVariants = (int)(sizeof(kGroupVariants) / sizeof(kGroupVariants[0]));
constexpr int64_t kMaxGroups = 1 << 16;

// Fused-epilogue products: the same kernels with bias / activation and the
// MX output kinds in the epilogue.
struct FusedVariant {
    const char *name;
    int bm, bn;
    int threads;
    KernelFn fn[2][5];       // [fmt][out kind]
    int linear;
    int kmax[2];             // largest K per format (0: any K)
};
#define MXG_FSFN(F, MT, WN, KW, O) (&mx_gemm_stream<F, MT, WN, KW, ring_depth(F, MT, WN), O, 0, 1>)
#define MXG_FSOUTS(F, MT, WN, KW)                                                                  \
    {MXG_FSFN(F, MT, WN, KW, OUT_BF16), MXG_FSFN(F, MT, WN, KW, OUT_F16),                          \
     MXG_FSFN(F, MT, WN, KW, OUT_F32), MXG_FSFN(F, MT, WN, KW, OUT_MX8), MXG_FSFN(F, MT, WN, KW, OUT_MX4)}
#define MXG_FSTREAM(MT, WN, KW)                                                                    \
    {"fstream_" #MT "x" #WN "_k" #KW, 16 * MT, 16 * WN, 64 * KW,                                   \
     {MXG_FSOUTS(FMT_FP8, MT, WN, KW), MXG_FSOUTS(FMT_FP4, MT, WN, KW)}, 0, {0, 0}}
#define MXG_FDFN(F, MT, NW, KM, G, KS, O) (&mx_gemm_decode<F, MT, NW, KM, G, O, KS, 1>)
#define MXG_FDOUTS(F, MT, NW, KM, G, KS)                                                           \
    {MXG_FDFN(F, MT, NW, KM, G, KS, OUT_BF16), MXG_FDFN(F, MT, NW, KM, G, KS, OUT_F16),            \
     MXG_FDFN(F, MT, NW, KM, G, KS, OUT_F32), MXG_FDFN(F, MT, NW, KM, G, KS, OUT_MX8),             \
     MXG_FDFN(F, MT, NW, KM, G, KS, OUT_MX4)}
#define MXG_FDECODE(NAME, MT, NW, G, KS, K4, K8)                                                   \
    {NAME, 16 * (MT), 16 * (NW), 64 * (NW) * (KS),                                                 \
     {MXG_FDOUTS(FMT_FP8, MT, NW, K8, G, KS), MXG_FDOUTS(FMT_FP4, MT, NW, K4, G, KS)}, 0, {K8, K4}}
#define MXG_FTFN(F, MT, NT, NS, O) (&mx_gemm_tile<F, MT, NT, O, 0, 1, NS>)
#define MXG_FTOUTS(F, MT, NT, NS)                                                                  \
    {MXG_FTFN(F, MT, NT, NS, OUT_BF16), MXG_FTFN(F, MT, NT, NS, OUT_F16),                          \
     MXG_FTFN(F, MT, NT, NS, OUT_F32), MXG_FTFN(F, MT, NT, NS, OUT_MX8),                            \
     MXG_FTFN(F, MT, NT, NS, OUT_MX4)}
#define MXG_FTILE(NAME, MT, NT, NS)                                                                \
    {NAME, 64 * (MT), 64 * (NT), 256, {MXG_FTOUTS(FMT_FP8, MT, NT, NS), MXG_FTOUTS(FMT_FP4, MT, NT, NS)}, 1, {0, 0}}

const FusedVariant kFusedVariants[] = {
    MXG_FSTREAM(1, 2, 4),
    MXG_FSTREAM(2, 4, 8),
    MXG_FTILE("ftile_128x128", 2, 2, 2),
    MXG_FTILE("ftile_256x128", 4, 2, 2),
    MXG_FTILE("ftile_256x256", 4, 4, 2),
    MXG_FDECODE("fdecode_16x64_k2", 1, 4, 2, 2, 4096, 2048),
    MXG_FDECODE("fdecode_32x64_k2", 2, 4, 2, 2, 4096, 2048),
    MXG_FTILE("ftile_128x256", 2, 4, 2),
    MXG_FDECODE("fdecode_16x64_k2_long", 1, 4, 2, 2, 8192, 2048),
    MXG_FDECODE("fdecode_32x64_k2_long", 2, 4, 2, 2, 5120, 2048),
    MXG_FTILE("ftile_64x64_r4", 1, 1, 4),
};
constexpr int kNumFusedVariants = (int)(sizeof(kFusedVariants) / sizeof(kFusedVariants[0]));

// ---------------------------------------------------------------- validation
// Largest K: every per-workgroup buffer range (at most 256 rows) must stay
// below 2^31 bytes.
constexpr int64_t kMaxK = (int64_t)1 << 22;
static_assert(256 * kMaxK < ((int64_t)1 << 31), "per-workgroup buffer range");

int validate(const void *a, const void *b, const void *sa, const void *sb, const void *c,
             int64_t M, int64_t N, int64_t K, int out_dtype)
{
    if (!a || !b || !sa || !sb || !c)
        return MXG_ERR_NULL;
    if (M < 1 || N < 1 || K < 1)
        return MXG_ERR_SHAPE;
    if (K % 128 != 0)
        return MXG_ERR_K_ALIGN;
    // kernels index rows and columns with int
    if (M > INT32_MAX || N > INT32_MAX || K > kMaxK)
        return MXG_ERR_SHAPE;
    if (M > INT64_MAX / N)
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

int find_variant(const char *name)
{
    for (int i = 0; i < kNumVariants; ++i)
        if (strcmp(kVariants[i].name, name) == 0)
            return i;
    return 0;
}

// ------------------------------------------------------------ split-K
// Largest number of K parts, and the K granularity of a part (128-K steps:
// the kernels' scale codes come four steps per 16-byte row piece).
constexpr int kMaxSplits = 64;
constexpr int kSplitGran = 4;

inline int64_t tiles_of(const Variant &v, int64_t M, int64_t N) { return cdiv(M, v.bm) * cdiv(N, v.bn); }

// Floats of one partial tile in the workspace: every thread's four-float
// pieces (the stream kernels give each thread whole pieces even where the
// tile has fewer groups of four columns than threads).
inline int64_t tile_floats(const Variant &v)
{
    return cdiv((int64_t)v.bm * v.bn / 4, v.threads) * v.threads * 4;
}

// Workspace of `splits` K parts: a fixed region of kSplitCounters arrival
// counters (the same for every configuration, so that one workspace serves
// any sequence of calls) and then tiles x splits partial tiles of FP32.
constexpr size_t kCounterBytes = (size_t)kSplitCounters * 4;

inline size_t splitk_bytes(const Variant &v, int splits, int64_t M, int64_t N)
{
    if (splits <= 1)
        return 0;
    const int64_t tiles = tiles_of(v, M, N);
    return kCounterBytes + (size_t)(tiles * splits * tile_floats(v) * 4);
}

// The largest K part of `splits` parts: whole units of kSplitGran steps.
inline int64_t part_k(int64_t K, int splits)
{
    const int64_t units = cdiv(K / 128, kSplitGran);
    return std::min(K, cdiv(units, splits) * kSplitGran * 128);
}

// Whether variant v can run K in `splits` parts (every part non-empty and
// within the variant's K limit).
int check_split(const Variant &v, int is_fp4, int64_t M, int64_t N, int64_t K, int splits)
{
    if (splits < 1 || splits > kMaxSplits)
        return MXG_ERR_CONFIG;
    if (splits > 1 && (!v.split || splits > cdiv(K / 128, kSplitGran) || tiles_of(v, M, N) > kSplitCounters))
        return MXG_ERR_CONFIG;
    const int kmax = v.kmax[is_fp4 ? 1 : 0];
    if (kmax && part_k(K, splits) > kmax)
        return MXG_ERR_CONFIG;
    return MXG_OK;
}

// Default tile choice, from measured sweeps on MI355X.  Up to 64 rows of A
// the product is a B stream: for E2M1 with 5-32 rows and wide N the
// whole-row decode kernel (A and the scales read once per workgroup), else
// the register-streaming kernel (at 33-64 rows and wide N the 64 x 64
// four-slot tile); beyond that the tile kernels take over, with the largest
// tile that still gives every compute unit work (per-CU traffic is
// proportional to tile rows + tile columns, so bigger tiles move fewer bytes
// per FLOP).
int pick_variant(int is_fp4, int64_t M, int64_t N, int64_t K)
{
    // E2M1, 5-32 rows, wide N, A tile fits LDS (K up to 8192 for 16 rows,
    // 5120 for 32): the whole-row decode kernel, at K <= 4096 with one wave
    // per row group and its B ring in LDS (32 x 14336 x 4096: 8.6 us against
    // 9.0-9.4 with two waves and register rings, 10.6 for stream_2x4_k8;
    // 8 x 14336 x 4096: 7.7 against 7.9-8.3), above with two waves and
    // register rings, whose smaller LDS footprint leaves room for the A tile
    // (32 x 25600 x 5120: 18.8 against 23.5 for stream_2x4_k8; 16 x 14336 x
    // 8192: 13.4 against 19.7 for stream_1x1_k4); at 1-4 rows the narrow
    // stream tile is faster
    if (is_fp4 && M > 4 && M <= 32 && N >= 8192 && K <= (M <= 16 ? 8192 : 5120)) {
        if (K <= 4096)
            return find_variant(M <= 16 ? "decode_16x64" : "decode_32x64");
        return find_variant(M <= 16 ? "decode_16x64_k2_long" : "decode_32x64_k2_long");
    }
    // long K splits over sixteen waves (8 x 4096 x 14336 E2M1: 8.4 us against
    // 10.3 with four)
    // (on wide N the 64 x 64 four-slot tile: 1 x 14336 x 8192 15.4 us against
    // 22.7 on sixteen waves, 16 x 14336 x 10240 19.2 against 27.5, 4 x 25600
    // x 8192 27.2 against 37.2)
    if (M <= 16 && is_fp4 && K >= 8192)
        return find_variant(N >= 8192 ? "tile_64x64_r4" : "stream_1x1_k16");
    // 1-16 rows on narrow N: one wave per K up to K = 1024, two up to 2048
    // (E2M1) / 4096 (E4M3), else four (E2M1 8 x 256 x 512: 2.72 us against
    // 3.48 with four waves, 8 x 256 x 2048: 3.34 against 3.57, 8 x 4096 x
    // 4096: 4.47 with four against 4.76 with two; E4M3 8 x 4096 x 512: 3.17
    // against 3.96, 8 x 4096 x 4096: 5.77 with two against 6.30)
    if (M <= 16) {
        // (E4M3 at K >= 8192: the 64 x 64 four-slot tile, 16 x 14336 x 8192
        // 25.0 us against 28.7, 8 x 14336 x 8192 26.4 against 27.2)
        if (N >= 8192)
            return find_variant(is_fp4 ? "stream_1x1_k4" : K >= 8192 ? "tile_64x64_r4" : "stream_1x2_k4");
        return find_variant(K <= 1024 ? "stream_1x1_k1"
                            : K <= (is_fp4 ? 2048 : 4096) ? "stream_1x1_k2" : "stream_1x1_k4");
    }
    // 17-32 rows on narrow N: as many waves splitting K as the row is long
    // (one up to 256 bytes per row, two up to 1024, else four; E2M1
    // 32 x 256 x 256: 3.14 us against 3.58 with four, 32 x 1024 x 2048:
    // 4.10 against 4.58; E4M3 32 x 4096 x 512: 3.68 against 4.15, at
    // 32 x 1024 x 2048 four waves stay ahead, 5.04 against 5.34)
    // 17-32 rows on wide N that the decode kernel does not take (E4M3, or
    // E2M1 past its K limit): the 64 x 64 four-slot tile (E4M3 32 x 14336 x
    // 4096: 15.8 us against 19.9 on stream_2x4_k8, 32 x 25600 x 5120: 34.4
    // against 44.7; E2M1 32 x 14336 x 8192: 16.7 against 18.3, 32 x 25600 x
    // 8192: 29.2 against 32.4; two K parts slower on each)
    if (M <= 32) {
        const int64_t rb = is_fp4 ? K / 2 : K;
        return find_variant(N >= 8192 ? "tile_64x64_r4"
                            : rb <= 256 ? "stream_2x1_k1" : rb <= 1024 ? "stream_2x1_k2" : "stream_2x1_k4");
    }
    // 33-64 rows on wide N: the 64 x 64 four-slot tile (64 x 14336 x 4096:
    // 11.7 us against 14.9 on a 64 x 64 split-K tile of register rings,
    // 64 x 25600 x 5120 24.8 against 32.7, E4M3 48 x 28672 x 4096 29.4
    // against 40.8); on narrow N the 32 x 32 stream tile (E4M3 64 x 4096 x
    // 4096: 9.5 us against 14.6 on 64 x 64 tiles, 10.5 with four K parts)
    if (M <= 64)
        return find_variant(N >= 8192 ? "tile_64x64_r4" : "stream_2x2_k4");
    // 65-128 rows on narrow N give the tile kernels too few output tiles
    // (128 x 4096 x 4096 E2M1: 17.3 us on tile_128x128, 7.9 on the decode
    // kernel; 128 x 4096 x 14336: 56.8 against 21.5 on stream_4x2_k8)
    if (M <= 128 && cdiv(M, 128) * cdiv(N, 128) < 64)
        return find_variant(!is_fp4 || K > 5120 ? "stream_4x2_k8"
                            : K <= 4096 ? "decode_32x64_k2" : "decode_32x64_k2_long");
    // and up to 256 rows with at most 64 such tiles: 64 x 64 tiles with four
    // code slots (256 x 4096 x 4096: 9.75 us against 12.2 on stream_4x4_k4
    // and 17.3 on tile_128x128; 256 x 4096 x 14336: 25.9 against 33.3;
    // E4M3 256 x 4096 x 4096: 14.3 against 15.9; 256 x 4096 x 1024: 5.4
    // against 6.8)
    if (M <= 256 && cdiv(M, 128) * cdiv(N, 128) <= 64)
        return find_variant("tile_64x64_r4");
    // tiles of 256 rows only above 128 rows, where they are not half empty
    // (128 x 25600 x 5120 E2M1: 29.1 us on 128 x 128, 32.7 on 256 x 128);
    // 256 x 256 from 192 tiles (512 x 25600 x 5120: 55.5 us, against 71.8 on
    // 128 x 256; at 112 tiles, 512 x 14336 x 4096, 128 x 256 wins: 31.0
    // against 37.8)
    if (M > 128 && cdiv(M, 256) * cdiv(N, 256) >= 192)
        return find_variant("tile_256x256");
    // from 256 rows the 128 x 256 tile (256 x 28672 x 8192: 47.9 us E2M1 and
    // 77.5 us E4M3, against 50.6 and 80.5 for 256 x 128)
    if (M >= 256 && cdiv(M, 128) * cdiv(N, 256) >= 192)
        return find_variant("tile_128x256");
    if (M > 128 && cdiv(M, 256) * cdiv(N, 128) >= 192)
        return find_variant("tile_256x128");
    // up to 128 tiles of 128 x 128 and K <= 4096: four times the workgroups
    // on 64 x 64 tiles (512 x 4096 x 4096: 15.2 us against 16.9 on
    // tile_128x128_r4, E4M3 21.9 against 24.4; 512 x 4096 x 2048: 9.6
    // against 12.5; E4M3 512 x 2048 x 2048: 8.6 against 18.8; at 160 tiles,
    // 640 x 4096 x 4096, 20.4 against 17.2, and at K = 14336 the 128 x 128
    // tile in two K parts is faster)
    if (cdiv(M, 128) * cdiv(N, 128) <= 128 && K <= 4096)
        return find_variant("tile_64x64_r4");
    // the 128 x 128 tile's super-stage is little MFMA work: over a long K a
    // ring of four code slots keeps its loads in flight across three of
    // them (128 x 25600 x 5120 E2M1: 32.3 -> 26.6 us; 512 x 4096 x 4096
    // E4M3: 25.2 -> 21.9), at short K the two-slot ring starts sooner
    // (333 x 517 x 1152: 9.0 against 10.1)
    return find_variant(K >= 4096 ? "tile_128x128_r4" : "tile_128x128");
}

struct Config {
    int variant, splits;
};

// Default configuration.  Without a workspace: pick_variant, whole K per
// workgroup.  With one: the same, except where too few output tiles leave
// compute units idle over a long K and split-K across workgroups measured
// faster on MI355X (E2M1; every part count also measured slower on c2,
// c3, c4 and the K = 4096 cells):
//   * a tile kernel launch of at most 128 tiles with K >= 8192: two K parts
//     (512 x 4096 x 14336: 53.0 -> 39.2 us on tile_128x128; at K = 4096 the
//     parts' extra round trip costs more than the idle half of the chip:
//     18.0 -> 20.2 us);
//   * 17-32 rows of E2M1 on narrow N (the whole-row decode kernel does not
//     apply) with K >= 12288: the 32 x 64 stream tile in four K parts
//     (32 x 4096 x 14336: 14.5 us on stream_2x1_k4 -> 12.7);
//   * 65-128 rows on narrow N that would run the 64 x 128 stream tile: the
//     64 x 64 four-slot tile in two K parts (below).
// Environment overrides of the default path, read once per process:
//   MXG_CONFIG=<variant>[:<K parts>]  the default path runs that
//     configuration instead of its own choice, for every shape (tuning; a
//     configuration that does not apply to a call's shape returns
//     MXG_ERR_CONFIG, one that needs more workspace than the call has
//     MXG_ERR_WORKSPACE, an unknown variant name MXG_ERR_CONFIG);
//   MXG_LOG=1  every default-path call prints its format, shape and
//     configuration to stderr.
struct EnvOverrides {
    int variant = -1;   // -1: none
    int splits = 1;
    bool bad = false;   // MXG_CONFIG set but not a variant name / part count
    bool log = false;
};

const EnvOverrides &env_overrides()
{
    static const EnvOverrides env = [] {
        EnvOverrides o;
        const char *lg = getenv("MXG_LOG");
        o.log = lg && *lg && strcmp(lg, "0") != 0;
        const char *cfg = getenv("MXG_CONFIG");
        if (!cfg || !*cfg)
            return o;
        const char *colon = strchr(cfg, ':');
        const size_t len = colon ? (size_t)(colon - cfg) : strlen(cfg);
        for (int v = 0; v < kNumVariants; ++v)
            if (strlen(kVariants[v].name) == len && strncmp(kVariants[v].name, cfg, len) == 0)
                o.variant = v;
        if (colon) {
            char *end = nullptr;
            const long parts = strtol(colon + 1, &end, 10);
            if (end == colon + 1 || *end || parts < 1 || parts > kMaxSplits)
                o.bad = true;
            else
                o.splits = (int)parts;
        }
        if (o.variant < 0)
            o.bad = true;
        return o;
    }();
    return env;
}

Config pick_config(int is_fp4, int64_t M, int64_t N, int64_t K, bool with_ws)
{
    const EnvOverrides &env = env_overrides();
    if (env.variant >= 0)
        return Config{env.variant, with_ws ? env.splits : 1};
    Config cf{pick_variant(is_fp4, M, N, K), 1};
    if (!with_ws)
        return cf;
    const Variant &v = kVariants[cf.variant];
    const int64_t units = cdiv(K / 128, kSplitGran);
    if (v.linear && tiles_of(v, M, N) <= 128 && K >= 8192 && units >= 2)
        return Config{cf.variant, 2};
    if (is_fp4 && M > 16 && M <= 32 && N < 8192 && K >= 12288 && units >= 4)
        return Config{find_variant("stream_2x4_k8"), 4};
    // 65-128 rows on narrow N where the stream tile would run (E4M3, or
    // E2M1 with K > 5120): 64 x 64 tiles with four code slots in two K
    // parts (128 x 4096 x 14336: 22.0 -> 18.1 us; E4M3 128 x 4096 x 8192:
    // 27.8 -> 18.3; E4M3 128 x 4096 x 4096: 13.9 -> 11.9; whole K on 64 x 64
    // tiles is no faster than the stream tile at long K)
    if (cf.variant == find_variant("stream_4x2_k8") && units >= 2)
        return Config{find_variant("tile_64x64_r4"), 2};
    return cf;
}

// Kernel arguments of a plain product over the whole K range.
GemmArgs make_args(int is_fp4, const void *a, const void *b, const void *sa, const void *sb, void *c,
                   int64_t M, int64_t N, int64_t K)
{
    GemmArgs p;
    memset(&p, 0, sizeof(p));
    p.a = (const uint8_t *)a;
    p.b = (const uint8_t *)b;
    p.sa = (const uint8_t *)sa;
    p.sb = (const uint8_t *)sb;
    p.c = c;
    p.M = (int)M;
    p.N = (int)N;
    p.nsteps = (int)(K / 128);
    p.row_bytes = (unsigned)(is_fp4 ? K / 2 : K);
    p.srow_bytes = (unsigned)(K / 32);
    p.kbytes = p.row_bytes;
    p.splits = 1;
    return p;
}

int launch(int is_fp4, const void *a, const void *b, const void *sa, const void *sb, void *c,
           int64_t M, int64_t N, int64_t K, int out_dtype, int variant, int splits, void *ws,
           hipStream_t stream)
{
    const Variant &v = kVariants[variant];
    GemmArgs p = make_args(is_fp4, a, b, sa, sb, c, M, N, K);
    const int64_t gx = cdiv(N, v.bn), gy = cdiv(M, v.bm);
    dim3 grid;
    if (v.linear) {
        if (gx * gy > INT32_MAX)
            return MXG_ERR_SHAPE;
        grid = dim3((unsigned)(gx * gy));
    } else {
        if (gx > INT32_MAX || gy > 65535)
            return MXG_ERR_SHAPE;
        grid = dim3((unsigned)gx, (unsigned)gy);
    }
    if (splits > 1) {
        p.splits = splits;
        p.flags = (unsigned *)ws;
        p.ws = (float *)((char *)ws + kCounterBytes);
        grid.z = (unsigned)splits;
    }
    KernelFn fn = v.fn[is_fp4 ? 1 : 0][out_dtype];
    hipLaunchKernelGGL(fn, grid, dim3(v.threads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXG_ERR_HIP;
    }
    return MXG_OK;
}

// variant argument of the run_* helpers: a table index, or this value for
// the default choice
constexpr int kPickDefault = -1000;

// ------------------------------------------------------------ grouped
int validate_grouped(const void *a, const void *b, const void *sa, const void *sb, const void *c,
                     const int32_t *offs, int64_t groups, int64_t M, int64_t N, int64_t K,
                     int out_dtype)
{
    if (!offs)
        return MXG_ERR_NULL;
    if (groups < 1 || groups > kMaxGroups || M < 0)
        return MXG_ERR_SHAPE;
    // M = 0 computes nothing but is checked like a one-row product, except
    // that A, its scales and C (empty tensors) may be NULL
    if (M == 0) {
        a = a ? a : b;
        sa = sa ? sa : sb;
        c = c ? c : b;
    }
    int rc = validate(a, b, sa, sb, c, M > 0 ? M : 1, N, K, out_dtype);
    if (rc)
        return rc;
    if ((uintptr_t)offs & 3u)
        return MXG_ERR_PTR_ALIGN;
    if (groups > INT64_MAX / N || groups * N > INT64_MAX / K)
        return MXG_ERR_SHAPE;
    return MXG_OK;
}

// Default grouped kernel from the mean rows per group (MI355X sweeps: up to
// 16 rows a group the product is a B stream -- 256 rows over 32 experts at
// N = K = 2048 MXFP8 ran 31.9 us on gstream_1x2_k4, 40.8 on gstream_2x4_k8).
int find_group_variant(const char *name)
{
    for (int i = 0; i < kNumGroupVariants; ++i)
        if (strcmp(kGroupVariants[i].name, name) == 0)
            return i;
    return 0;
}

int pick_group_variant(int64_t groups, int64_t M, int64_t N)
{
    (void)N;
    const int64_t mean = M / groups;
    if (mean <= 16)
        return find_group_variant("gstream_1x2_k4");
    if (mean <= 48)
        return find_group_variant("gstream_2x4_k8");
    if (mean <= 192)
        return find_group_variant("gtile_128x128");
    // 8 x 1024 rows, N = K = 4096, MXFP8: 190 us against 226 for 256x128 and
    // 242 for 128x128
    return find_group_variant("gtile_256x256");
}

int launch_grouped(int is_fp4, const void *a, const void *b, const void *sa, const void *sb,
                   void *c, const int32_t *offs, int64_t groups, int64_t M, int64_t N, int64_t K,
                   int out_dtype, int variant, hipStream_t stream)
{
    const Variant &v = kGroupVariants[variant];
    // M: total rows; each workgroup narrows it to its group
    GemmArgs p = make_args(is_fp4, a, b, sa, sb, c, M, N, K);
    p.offs = offs;
    p.groups = (int)groups;
    // worst case over all splits of M rows into the groups
    const int64_t mtiles = cdiv(M, v.bm) + groups, gx = cdiv(N, v.bn);
    dim3 grid;
    if (v.linear) {
        if (mtiles * gx > INT32_MAX)
            return MXG_ERR_SHAPE;
        grid = dim3((unsigned)(mtiles * gx));
    } else {
        if (gx > INT32_MAX || mtiles > 65535)
            return MXG_ERR_SHAPE;
        grid = dim3((unsigned)gx, (unsigned)mtiles);
    }
    hipLaunchKernelGGL(v.fn[is_fp4 ? 1 : 0][out_dtype], grid, dim3(v.threads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXG_ERR_HIP;
    }
    return MXG_OK;
}

int run_grouped(int is_fp4, const void *a, const void *b, const void *sa, const void *sb, void *c,
                const int32_t *offs, int64_t groups, int64_t M, int64_t N, int64_t K,
                int out_dtype, int variant, hipStream_t stream)
{
    int rc = validate_grouped(a, b, sa, sb, c, offs, groups, M, N, K, out_dtype);
    if (rc)
        return rc;
    if (variant == kPickDefault)
        variant = pick_group_variant(groups, M, N);
    if (variant < 0 || variant >= kNumGroupVariants)
        return MXG_ERR_CONFIG;
    if (M == 0)
        return MXG_OK;
    // the worst-case grid must fit the launch (checked again in launch_grouped)
    const Variant &v = kGroupVariants[variant];
    const int64_t mtiles = cdiv(M, v.bm) + groups, gx = cdiv(N, v.bn);
    if (v.linear ? mtiles * gx > INT32_MAX : (gx > INT32_MAX || mtiles > 65535))
        return MXG_ERR_SHAPE;
    rc = check_device();
    if (rc)
        return rc;
    return launch_grouped(is_fp4, a, b, sa, sb, c, offs, groups, M, N, K, out_dtype, variant,
                          stream);
}

// ------------------------------------------------------------ fused epilogue
// Default fused kernel: the plain product's choice, among the kernels whose
// workgroup tiles cover whole 32-column blocks.
int find_fused_variant(const char *name)
{
    for (int i = 0; i < kNumFusedVariants; ++i)
        if (strcmp(kFusedVariants[i].name, name) == 0)
            return i;
    return 0;
}

int pick_fused_variant(int is_fp4, int64_t M, int64_t N, int64_t K)
{
    // the plain product's decode-width choice (see pick_variant)
    if (is_fp4 && M > 4 && M <= 32 && N >= 8192 && K <= (M <= 16 ? 8192 : 5120)) {
        if (K <= 4096)
            return find_fused_variant(M <= 16 ? "fdecode_16x64_k2" : "fdecode_32x64_k2");
        return find_fused_variant(M <= 16 ? "fdecode_16x64_k2_long" : "fdecode_32x64_k2_long");
    }
    // wide N as the plain product: the 64 x 64 four-slot tile (SiLU, bias,
    // MXFP8 out: E4M3 32 x 14336 x 4096 17.1 us against 20.8 on
    // fstream_2x4_k8, 64 x 14336 x 4096 18.6 against 30.8, 24 x 25600 x 5120
    // 33.9 against 44.0; 16 x 14336 x 8192 27.7 against 29.2 on fstream_1x2_k4)
    if (M <= 16)
        return find_fused_variant(N >= 8192 && K >= 8192 ? "ftile_64x64_r4" : "fstream_1x2_k4");
    if (M <= 64)
        return find_fused_variant(N >= 8192 ? "ftile_64x64_r4" : "fstream_2x4_k8");
    // the plain product's tile rule
    if (M > 128 && cdiv(M, 256) * cdiv(N, 256) >= 192)
        return find_fused_variant("ftile_256x256");
    if (M >= 256 && cdiv(M, 128) * cdiv(N, 256) >= 192)
        return find_fused_variant("ftile_128x256");
    if (M > 128 && cdiv(M, 256) * cdiv(N, 128) >= 192)
        return find_fused_variant("ftile_256x128");
    return find_fused_variant("ftile_128x128");
}

int run_fused(int is_fp4, const void *a, const void *b, const void *sa, const void *sb,
              const void *bias, int act, void *c, void *c_scale, int64_t M, int64_t N, int64_t K,
              int out_kind, int variant, hipStream_t stream)
{
    const bool mx_out = out_kind == MXG_OUT_MXFP8 || out_kind == MXG_OUT_MXFP4;
    if (out_kind < MXG_OUT_BF16 || out_kind > MXG_OUT_MXFP4)
        return MXG_ERR_DTYPE;
    // operand checks as for the plain product (the output dtype is checked above)
    int rc = validate(a, b, sa, sb, c, M, N, K, MXG_OUT_BF16);
    if (rc)
        return rc;
    if (act < MXG_ACT_NONE || act > MXG_ACT_GELU_TANH)
        return MXG_ERR_CONFIG;
    if ((uintptr_t)bias & 1u)
        return MXG_ERR_PTR_ALIGN;
    if (bias && N > ((int64_t)1 << 30))   // the kernels read bias through a 2N-byte buffer range
        return MXG_ERR_SHAPE;
    if (mx_out) {
        if (!c_scale)
            return MXG_ERR_NULL;
        if (N % 32)
            return MXG_ERR_SHAPE;
    }
    if (variant == kPickDefault)
        variant = pick_fused_variant(is_fp4, M, N, K);
    if (variant < 0 || variant >= kNumFusedVariants)
        return MXG_ERR_CONFIG;
    const FusedVariant &v = kFusedVariants[variant];
    if (v.kmax[is_fp4 ? 1 : 0] && K > v.kmax[is_fp4 ? 1 : 0])
        return MXG_ERR_CONFIG;
    const int64_t gx = cdiv(N, v.bn), gy = cdiv(M, v.bm);
    if (v.linear ? gx * gy > INT32_MAX : (gx > INT32_MAX || gy > 65535))
        return MXG_ERR_SHAPE;
    rc = check_device();
    if (rc)
        return rc;
    GemmArgs p = make_args(is_fp4, a, b, sa, sb, c, M, N, K);
    p.bias = (const uint16_t *)bias;
    p.act = act;
    p.c_scale = (uint8_t *)c_scale;
    const dim3 grid = v.linear ? dim3((unsigned)(gx * gy)) : dim3((unsigned)gx, (unsigned)gy);
    hipLaunchKernelGGL(v.fn[is_fp4 ? 1 : 0][out_kind], grid, dim3(v.threads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXG_ERR_HIP;
    }
    return MXG_OK;
}

// ------------------------------------------------------------ dense BF16 / FP16
typedef void (*DenseFn)(DenseArgs);
#define MXG_DFN4(T, TA, TB) \
    {&mx_dense_gemm_kernel<T, TA, TB, OUT_BF16>, &mx_dense_gemm_kernel<T, TA, TB, OUT_F16>, \
     &mx_dense_gemm_kernel<T, TA, TB, OUT_F32>}
#define MXG_DLAYOUTS(T) {{MXG_DFN4(T, 0, 0), MXG_DFN4(T, 0, 1)}, {MXG_DFN4(T, 1, 0), MXG_DFN4(T, 1, 1)}}
const DenseFn kDense[2][2][2][3] = {MXG_DLAYOUTS(DENSE_BF16), MXG_DLAYOUTS(DENSE_F16)};

// NT (both operands K-contiguous, the MFMA's own layout): the tile kernel
// with 16-bit operands (its loads, LDS slots and pipeline; no scale codes).
// [dtype][tile: 256x256, 128x256, 128x128][out]
// The other layouts: an operand contiguous along M or N gets slots of K
// rows, read with transposing LDS reads (TA: A stored [K][M]; TB: B stored
// [K][N]).  [trans_a][trans_b][dtype][tile][out]
#define MXG_D16(F, MT, NT, TB, TA)                                                               \
    {&mx_gemm_tile<F, MT, NT, OUT_BF16, 0, 0, 2, TB, TA>,                                       \
     &mx_gemm_tile<F, MT, NT, OUT_F16, 0, 0, 2, TB, TA>, &mx_gemm_tile<F, MT, NT, OUT_F32, 0, 0, 2, TB, TA>}
#define MXG_D16T(TB, TA)                                                                         \
    {{MXG_D16(FMT_BF16, 4, 4, TB, TA), MXG_D16(FMT_BF16, 2, 4, TB, TA), MXG_D16(FMT_BF16, 2, 2, TB, TA)}, \
     {MXG_D16(FMT_F16, 4, 4, TB, TA), MXG_D16(FMT_F16, 2, 4, TB, TA), MXG_D16(FMT_F16, 2, 2, TB, TA)}}
const KernelFn kDenseTile[2][2][2][3][3] = {{MXG_D16T(1, 0), MXG_D16T(0, 0)}, {MXG_D16T(1, 1), MXG_D16T(0, 1)}};

// The largest of the three tiles that still gives at least 192 workgroups
// (the same rule as the MX products'), else 128 x 128.
int dense_nt_tile(int64_t M, int64_t N)
{
    if (M > 128 && cdiv(M, 256) * cdiv(N, 256) >= 192)
        return 0;
    if (M >= 256 && cdiv(M, 128) * cdiv(N, 256) >= 192)
        return 1;
    return 2;
}

int run_dense(int dtype, int trans_a, int trans_b, const void *a, const void *b, void *c,
              int64_t M, int64_t N, int64_t K, int out_dtype, hipStream_t stream)
{
    if (!a || !b || !c)
        return MXG_ERR_NULL;
    if (dtype != 0 && dtype != 1)
        return MXG_ERR_DTYPE;
    if (out_dtype < MXG_OUT_BF16 || out_dtype > MXG_OUT_F32)
        return MXG_ERR_DTYPE;
    if (trans_a < 0 || trans_a > 1 || trans_b < 0 || trans_b > 1)
        return MXG_ERR_CONFIG;
    if (M < 1 || N < 1 || K < 1 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return MXG_ERR_SHAPE;
    // every operand below 2 GiB (one buffer range each); C indexed in size_t
    if (M * K >= ((int64_t)1 << 30) || N * K >= ((int64_t)1 << 30) || M > INT64_MAX / N)
        return MXG_ERR_SHAPE;
    // rows of both operands 16-byte aligned: the contiguous dimension % 8
    const int64_t lda = trans_a ? M : K, ldb = trans_b ? K : N;
    if (lda % 8 || ldb % 8)
        return MXG_ERR_SHAPE;
    if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 15u)
        return MXG_ERR_PTR_ALIGN;
    // the tile kernel where its 32-bit offsets into an operand stored [K][M]
    // or [K][N] cannot wrap (a super-stage's 64 K rows past a live one's
    // start, M or N columns each); else (only with K < 64 and 2^24 or more
    // columns) the transposing kernel
    const bool a_ok = !trans_a || 2 * M * (K + 64) < ((int64_t)1 << 32);
    const bool b_ok = trans_b || 2 * N * (K + 64) < ((int64_t)1 << 32);
    if (a_ok && b_ok) {
        const int t = dense_nt_tile(M, N);
        const int bm = t == 0 ? 256 : 128, bn = t == 2 ? 128 : 256;
        const int64_t tiles = cdiv(M, bm) * cdiv(N, bn);
        if (tiles > INT32_MAX)
            return MXG_ERR_SHAPE;
        int rc = check_device();
        if (rc)
            return rc;
        GemmArgs p;
        memset(&p, 0, sizeof(p));
        p.a = (const uint8_t *)a;
        p.b = (const uint8_t *)b;
        p.c = c;
        p.M = (int)M;
        p.N = (int)N;
        p.row_bytes = (unsigned)(2 * K);
        p.kbytes = p.row_bytes;
        p.splits = 1;
        hipLaunchKernelGGL(kDenseTile[trans_a][trans_b][dtype][t][out_dtype], dim3((unsigned)tiles), dim3(256), 0,
                           stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) {
            g_last_hip_error = (int)e;
            return MXG_ERR_HIP;
        }
        return MXG_OK;
    }
    const int64_t gx = cdiv(N, DenseTile::BN), gy = cdiv(M, DenseTile::BM);
    if (gx > INT32_MAX || gy > 65535)
        return MXG_ERR_SHAPE;
    int rc = check_device();
    if (rc)
        return rc;
    DenseArgs p;
    p.a = (const uint16_t *)a;
    p.b = (const uint16_t *)b;
    p.c = c;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    hipLaunchKernelGGL(kDense[dtype][trans_a][trans_b][out_dtype], dim3((unsigned)gx, (unsigned)gy),
                       dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXG_ERR_HIP;
    }
    return MXG_OK;
}

// An empty kernel (measurement support: the launch cost alone).
__global__ __launch_bounds__(1024) void mx_empty_kernel() {}

// ------------------------------------------------- allocation-free entry point
// mx_scaled_mm_noalloc runs the default configuration with the split-K
// workspace in this array instead of a caller's buffer.  Each GPU the
// library runs on holds its own copy until the process ends.  Its size
// covers every default split-K configuration (at most 64 KiB of counters
// plus 128 tiles x 2 parts x 128 x 128 FP32 = 16.06 MiB).
constexpr size_t kScratchBytes = (size_t)20 << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

// Device address of this GPU's scratch, looked up once per device with the
// device current (the array's name is not a device address on the host),
// and its counter region cleared by a fill kernel on the first call's
// stream, ahead of that call's own kernels.
__global__ __launch_bounds__(256) void mx_zero_words(unsigned *p, int n)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n)
        p[i] = 0u;
}

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_of_device(hipStream_t stream, void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXG_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return MXG_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            g_last_hip_error = (int)e;
            return MXG_ERR_HIP;
        }
        hipLaunchKernelGGL(mx_zero_words, dim3(kSplitCounters / 256), dim3(256), 0, stream, (unsigned *)ptr,
                           kSplitCounters);
        e = hipGetLastError();
        if (e != hipSuccess) {
            g_last_hip_error = (int)e;
            return MXG_ERR_HIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MXG_OK;
}

int validate_ws(const void *ws, size_t ws_bytes)
{
    if (ws && ((uintptr_t)ws & 15u))
        return MXG_ERR_PTR_ALIGN;
    (void)ws_bytes;
    return MXG_OK;
}

int run_default(int is_fp4, const void *a, const void *b, const void *sa, const void *sb, void *c,
                int64_t M, int64_t N, int64_t K, int out_dtype, void *ws, size_t ws_bytes,
                hipStream_t stream)
{
    int rc = validate(a, b, sa, sb, c, M, N, K, out_dtype);
    if (rc)
        return rc;
    rc = validate_ws(ws, ws_bytes);
    if (rc)
        return rc;
    const EnvOverrides &env = env_overrides();
    if (env.bad)
        return MXG_ERR_CONFIG;
    Config cf = pick_config(is_fp4, M, N, K, true);
    if (env.variant >= 0) {
        // a configuration forced through MXG_CONFIG: as mx_scaled_mm_config
        rc = check_split(kVariants[cf.variant], is_fp4, M, N, K, cf.splits);
        if (rc)
            return rc;
        if (cf.splits > 1 && (!ws || ws_bytes < splitk_bytes(kVariants[cf.variant], cf.splits, M, N)))
            return MXG_ERR_WORKSPACE;
    } else if (cf.splits > 1 && (!ws || ws_bytes < splitk_bytes(kVariants[cf.variant], cf.splits, M, N))) {
        // a missing or short workspace: the whole-K configuration (correct, maybe slower)
        cf = pick_config(is_fp4, M, N, K, false);
    }
    if (env.log)
        fprintf(stderr, "mxgemm: %s M=%lld N=%lld K=%lld -> %s, %d K part%s%s\n", is_fp4 ? "mxfp4" : "mxfp8",
                (long long)M, (long long)N, (long long)K, kVariants[cf.variant].name, cf.splits,
                cf.splits == 1 ? "" : "s", env.variant >= 0 ? " (MXG_CONFIG)" : "");
    rc = check_device();
    if (rc)
        return rc;
    return launch(is_fp4, a, b, sa, sb, c, M, N, K, out_dtype, cf.variant, cf.splits, ws, stream);
}

}  // namespace

extern "C" {

int mx_scaled_mm_fp4(const void *a, const void *b, const void *a_scale, const void *b_scale,
                     void *c, int64_t M, int64_t N, int64_t K, int out_dtype, void *workspace,
                     size_t workspace_bytes, mxg_stream_t stream)
{
    return run_default(1, a, b, a_scale, b_scale, c, M, N, K, out_dtype, workspace, workspace_bytes,
                       (hipStream_t)stream);
}

int mx_scaled_mm_fp8(const void *a, const void *b, const void *a_scale, const void *b_scale,
                     void *c, int64_t M, int64_t N, int64_t K, int out_dtype, void *workspace,
                     size_t workspace_bytes, mxg_stream_t stream)
{
    return run_default(0, a, b, a_scale, b_scale, c, M, N, K, out_dtype, workspace, workspace_bytes,
                       (hipStream_t)stream);
}

int mx_scaled_mm_noalloc(int is_fp4, const void *a, const void *b, const void *a_scale,
                         const void *b_scale, void *c, int64_t M, int64_t N, int64_t K, int out_dtype,
                         mxg_stream_t stream)
{
    is_fp4 = is_fp4 ? 1 : 0;
    int rc = validate(a, b, a_scale, b_scale, c, M, N, K, out_dtype);
    if (rc)
        return rc;
    const EnvOverrides &env = env_overrides();
    if (env.bad)
        return MXG_ERR_CONFIG;
    const Config cf = pick_config(is_fp4, M, N, K, true);
    if (env.variant >= 0) {
        rc = check_split(kVariants[cf.variant], is_fp4, M, N, K, cf.splits);
        if (rc)
            return rc;
    }
    if (splitk_bytes(kVariants[cf.variant], cf.splits, M, N) > kScratchBytes)
        return MXG_ERR_SCRATCH;
    rc = check_device();
    if (rc)
        return rc;
    void *ws = nullptr;
    if (cf.splits > 1) {
        rc = scratch_of_device((hipStream_t)stream, &ws);
        if (rc)
            return rc;
    }
    return launch(is_fp4, a, b, a_scale, b_scale, c, M, N, K, out_dtype, cf.variant, cf.splits, ws,
                  (hipStream_t)stream);
}

size_t mx_noalloc_scratch_bytes(void) { return kScratchBytes; }

static int check_shape(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || K < 1 || M > INT32_MAX || N > INT32_MAX || K > kMaxK)
        return MXG_ERR_SHAPE;
    if (K % 128)
        return MXG_ERR_K_ALIGN;
    return MXG_OK;
}

int mx_default_config(int is_fp4, int64_t M, int64_t N, int64_t K, int with_workspace, int *splits)
{
    const int rc = check_shape(M, N, K);
    if (rc)
        return rc;
    const EnvOverrides &env = env_overrides();
    if (env.bad)
        return MXG_ERR_CONFIG;
    const Config cf = pick_config(is_fp4 ? 1 : 0, M, N, K, with_workspace != 0);
    if (env.variant >= 0 && check_split(kVariants[cf.variant], is_fp4 ? 1 : 0, M, N, K, cf.splits))
        return MXG_ERR_CONFIG;
    if (splits)
        *splits = cf.splits;
    return cf.variant;
}

int mx_default_variant(int is_fp4, int64_t M, int64_t N, int64_t K)
{
    return mx_default_config(is_fp4, M, N, K, 1, nullptr);
}

size_t mx_scaled_mm_workspace_bytes(int is_fp4, int64_t M, int64_t N, int64_t K)
{
    if (check_shape(M, N, K))
        return 0;
    const Config cf = pick_config(is_fp4 ? 1 : 0, M, N, K, true);
    return splitk_bytes(kVariants[cf.variant], cf.splits, M, N);
}

size_t mx_config_workspace_bytes(int variant, int splits, int64_t M, int64_t N)
{
    if (variant < 0 || variant >= kNumVariants || splits < 1 || splits > kMaxSplits || M < 1 || N < 1 ||
        M > INT32_MAX || N > INT32_MAX ||
        (splits > 1 && (!kVariants[variant].split || tiles_of(kVariants[variant], M, N) > kSplitCounters)))
        return 0;
    return splitk_bytes(kVariants[variant], splits, M, N);
}

int mx_scaled_mm_config(int is_fp4, const void *a, const void *b, const void *a_scale,
                        const void *b_scale, void *c, int64_t M, int64_t N, int64_t K,
                        int out_dtype, int variant, int splits, void *workspace,
                        size_t workspace_bytes, mxg_stream_t stream)
{
    int rc = validate(a, b, a_scale, b_scale, c, M, N, K, out_dtype);
    if (rc)
        return rc;
    if (variant < 0 || variant >= kNumVariants)
        return MXG_ERR_CONFIG;
    rc = check_split(kVariants[variant], is_fp4, M, N, K, splits);
    if (rc)
        return rc;
    rc = validate_ws(workspace, workspace_bytes);
    if (rc)
        return rc;
    if (splits > 1 && (!workspace || workspace_bytes < splitk_bytes(kVariants[variant], splits, M, N)))
        return MXG_ERR_WORKSPACE;
    rc = check_device();
    if (rc)
        return rc;
    return launch(is_fp4 ? 1 : 0, a, b, a_scale, b_scale, c, M, N, K, out_dtype, variant, splits,
                  workspace, (hipStream_t)stream);
}

int mx_empty_like(int is_fp4, int64_t M, int64_t N, int64_t K, mxg_stream_t stream)
{
    int splits = 1;
    const int variant = mx_default_config(is_fp4, M, N, K, 1, &splits);
    if (variant < 0)
        return variant;
    int rc = check_device();
    if (rc)
        return rc;
    const Variant &v = kVariants[variant];
    const int64_t gx = cdiv(N, v.bn), gy = cdiv(M, v.bm);
    if (v.linear ? gx * gy > INT32_MAX : (gx > INT32_MAX || gy > 65535))
        return MXG_ERR_SHAPE;
    dim3 grid = v.linear ? dim3((unsigned)(gx * gy)) : dim3((unsigned)gx, (unsigned)gy);
    grid.z = (unsigned)splits;
    hipLaunchKernelGGL(mx_empty_kernel, grid, dim3(v.threads), 0, (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXG_ERR_HIP;
    }
    return MXG_OK;
}

int mx_num_variants(void) { return kNumVariants; }

int64_t mx_variant_max_k(int variant, int is_fp4)
{
    if (variant < 0 || variant >= kNumVariants)
        return MXG_ERR_CONFIG;
    const int km = kVariants[variant].kmax[is_fp4 ? 1 : 0];
    return km ? km : kMaxK;
}

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
    case MXG_ERR_DEVICE: return "current device is not gfx950";
    case MXG_ERR_HIP: return "HIP runtime error";
    case MXG_ERR_CONFIG: return "invalid kernel variant or K-part count";
    case MXG_ERR_WORKSPACE: return "workspace missing or too small for the requested K parts";
    case MXG_ERR_SCRATCH: return "the shape needs more split-K workspace than mx_scaled_mm_noalloc's built-in scratch holds";
    default: return "unknown status";
    }
}

int mx_quantize_bf16(const void *x, void *codes, void *scales, int64_t rows, int64_t K,
                     int is_fp4, mxg_stream_t stream)
{
    if (!x || !codes || !scales)
        return MXG_ERR_NULL;
    if (rows < 1 || K < 1 || rows > ((int64_t)1 << 40) / K)
        return MXG_ERR_SHAPE;
    if (K % 32)
        return MXG_ERR_K_ALIGN;
    if (((uintptr_t)x & 15) || ((uintptr_t)codes & 15))
        return MXG_ERR_PTR_ALIGN;
    int rc = check_device();
    if (rc)
        return rc;
    const long long nblocks = (long long)(rows * (K / 32));
    const long long tiles = (nblocks + 63) / 64;                     // one per wave
    const unsigned grid = (unsigned)std::min<long long>((tiles + 3) / 4, 16384);
    if (is_fp4)
        hipLaunchKernelGGL(mx_quantize<FMT_FP4>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                           (const uint16_t *)x, (uint8_t *)codes, (uint8_t *)scales, nblocks);
    else
        hipLaunchKernelGGL(mx_quantize<FMT_FP8>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                           (const uint16_t *)x, (uint8_t *)codes, (uint8_t *)scales, nblocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXG_ERR_HIP;
    }
    return MXG_OK;
}

int mx_grouped_mm_fp4(const void *a, const void *b, const void *a_scale, const void *b_scale,
                      void *c, const int32_t *offs, int64_t groups, int64_t M, int64_t N,
                      int64_t K, int out_dtype, mxg_stream_t stream)
{
    return run_grouped(1, a, b, a_scale, b_scale, c, offs, groups, M, N, K, out_dtype, kPickDefault,
                       (hipStream_t)stream);
}

int mx_grouped_mm_fp8(const void *a, const void *b, const void *a_scale, const void *b_scale,
                      void *c, const int32_t *offs, int64_t groups, int64_t M, int64_t N,
                      int64_t K, int out_dtype, mxg_stream_t stream)
{
    return run_grouped(0, a, b, a_scale, b_scale, c, offs, groups, M, N, K, out_dtype, kPickDefault,
                       (hipStream_t)stream);
}

int mx_grouped_mm_config(int is_fp4, const void *a, const void *b, const void *a_scale,
                         const void *b_scale, void *c, const int32_t *offs, int64_t groups,
                         int64_t M, int64_t N, int64_t K, int out_dtype, int variant,
                         mxg_stream_t stream)
{
    return run_grouped(is_fp4 ? 1 : 0, a, b, a_scale, b_scale, c, offs, groups, M, N, K,
                       out_dtype, variant, (hipStream_t)stream);
}

int mx_grouped_num_variants(void) { return kNumGroupVariants; }

const char *mx_grouped_variant_name(int variant)
{
    if (variant < 0 || variant >= kNumGroupVariants)
        return nullptr;
    return kGroupVariants[variant].name;
}

int mx_grouped_default_variant(int64_t groups, int64_t M, int64_t N)
{
    if (groups < 1 || groups > kMaxGroups || M < 0 || N < 1)
        return MXG_ERR_SHAPE;
    return pick_group_variant(groups, M, N);
}

int mx_scaled_mm_fused(int is_fp4, const void *a, const void *b, const void *a_scale,
                       const void *b_scale, const void *bias, int act, void *c, void *c_scale,
                       int64_t M, int64_t N, int64_t K, int out_kind, int variant,
                       mxg_stream_t stream)
{
    return run_fused(is_fp4 ? 1 : 0, a, b, a_scale, b_scale, bias, act, c, c_scale, M, N, K,
                     out_kind, variant < 0 ? kPickDefault : variant, (hipStream_t)stream);
}

int mx_fused_num_variants(void) { return kNumFusedVariants; }

int mx_fused_default_variant(int is_fp4, int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || K < 1 || M > INT32_MAX || N > INT32_MAX)
        return MXG_ERR_SHAPE;
    return pick_fused_variant(is_fp4 ? 1 : 0, M, N, K);
}

int64_t mx_fused_variant_max_k(int variant, int is_fp4)
{
    if (variant < 0 || variant >= kNumFusedVariants)
        return MXG_ERR_CONFIG;
    const int km = kFusedVariants[variant].kmax[is_fp4 ? 1 : 0];
    return km ? km : kMaxK;
}

const char *mx_fused_variant_name(int variant)
{
    if (variant < 0 || variant >= kNumFusedVariants)
        return nullptr;
    return kFusedVariants[variant].name;
}

int mx_dense_gemm(int dtype, int trans_a, int trans_b, const void *a, const void *b, void *c,
                  int64_t M, int64_t N, int64_t K, int out_dtype, mxg_stream_t stream)
{
    return run_dense(dtype, trans_a, trans_b, a, b, c, M, N, K, out_dtype, (hipStream_t)stream);
}

int mx_last_hip_error(void) { return g_last_hip_error; }

int mx_abi_version(void) { return MXGEMM_ABI_VERSION; }

}  // extern "C"
