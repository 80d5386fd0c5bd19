/*
 * mxgemm.h -- C ABI of the MI355X (gfx950) NT MX block-scaled GEMM library.
 *
 * The operation ("PyTorch 接上 FlyDSL", 5ulink.com, section "支持边界":
 * support-matrix row "MXFP 缩放 GEMM" and the paragraph under the table;
 * the devotd.net page, section 2, defines "NT" as left operand row-major,
 * right operand column-major):
 *
 *   C[m,n] = sum_{kb < K/32} 2^(sa[m,kb]-127) * 2^(sb[n,kb]-127)
 *                           * sum_{j<32} A[m,32kb+j] * B[n,32kb+j]
 *
 * with MXFP4 (E2M1) or MXFP8 (E4M3, OCP "FN" flavour) elements, one E8M0
 * scale per 32 consecutive K values (BlockWise1x32), FP32 accumulation and
 * BF16 or FP16 output.  K must be a multiple of 128.
 *
 * Memory layouts (all device memory, all contiguous, no leading dimensions):
 *   a        FP4: [M][K/2] bytes, element k of row m in byte m*K/2 + k/2,
 *                 low nibble when k is even, high nibble when k is odd.
 *            FP8: [M][K] bytes.
 *   b        B is K x N column-major, i.e. [N][K/2] (FP4) or [N][K] (FP8)
 *            bytes, the same packing as a.
 *   a_scale  [M][K/32] E8M0 bytes, row-major.
 *   b_scale  [N][K/32] E8M0 bytes, row-major.
 *   c        [M][N] row-major, element type given by out_dtype; every
 *            element is overwritten.  c must not overlap any input.
 *
 * Ownership and threading: the caller allocates and owns every buffer.  A
 * call validates its arguments on the host, enqueues its kernels on
 * `stream` and returns without synchronizing; buffers must stay valid until
 * that work has completed.  The library allocates no device memory in a
 * call and keeps no pointer after it returns.  Calls on different streams
 * may run concurrently.
 *
 * Errors: every function returns an mxg_status_t.  Argument checks happen
 * before any HIP call, so a rejected call touches no device state.  A
 * non-zero status means the product was not computed and the caller should
 * use another implementation (the pages' rule: unsupported combinations
 * fall back to the original implementation).  Faults inside an enqueued
 * kernel surface at the caller's next synchronization, as for any HIP work.
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t; 0 is the null stream of the current device. */
typedef struct ihipStream_t *mxg_stream_t;

typedef enum {
    MXG_OUT_BF16 = 0, /* bfloat16, round to nearest even */
    MXG_OUT_F16 = 1,  /* IEEE half, round to nearest even */
    MXG_OUT_F32 = 2,  /* the FP32 accumulator before output rounding */
    /* mx_scaled_mm_fused only: the BF16-rounded result MX-quantized along N */
    MXG_OUT_MXFP8 = 3, /* E4M3 codes [M][N] + E8M0 [M][N/32] */
    MXG_OUT_MXFP4 = 4  /* E2M1 codes [M][N/2] + E8M0 [M][N/32] */
} mxg_out_t;

/* Epilogue activations of mx_scaled_mm_fused. */
typedef enum {
    MXG_ACT_NONE = 0,
    MXG_ACT_RELU = 1,      /* max(x, 0) */
    MXG_ACT_SILU = 2,      /* x / (1 + exp(-x)) */
    MXG_ACT_GELU_TANH = 3  /* 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
} mxg_act_t;

typedef enum {
    MXG_OK = 0,
    MXG_ERR_NULL = -1,      /* a required pointer is NULL */
    MXG_ERR_SHAPE = -2,     /* M, N or K < 1, K > 2^22, M or N > 2^31-1, or M*N overflows int64 */
    MXG_ERR_K_ALIGN = -3,   /* K is not a multiple of 128 */
    MXG_ERR_PTR_ALIGN = -4, /* a, b or c is not 16-byte aligned; a scale pointer not 4-byte aligned */
    MXG_ERR_DTYPE = -5,     /* out_dtype is not an mxg_out_t */
    MXG_ERR_WORKSPACE = -6, /* an explicit split-K configuration lacks a large enough workspace */
    MXG_ERR_DEVICE = -7,    /* the current device is not gfx950 */
    MXG_ERR_HIP = -8,       /* a HIP call failed (see mx_last_hip_error) */
    MXG_ERR_CONFIG = -9,    /* an explicit kernel variant or K-part count is invalid */
    MXG_ERR_SCRATCH = -10   /* mx_scaled_mm_noalloc: the shape needs more scratch than it has */
} mxg_status_t;

/*
 * MXFP4 (E2M1) x MXFP4 NT scaled GEMM: C = A * B^T as defined above.
 *
 * a, b         packed E2M1 codes, [M][K/2] and [N][K/2] bytes, 16-byte aligned.
 * a_scale      E8M0 codes [M][K/32], 4-byte aligned.
 * b_scale      E8M0 codes [N][K/32], 4-byte aligned.
 * c            [M][N] output of type out_dtype, 16-byte aligned.
 * M, N, K      logical sizes (K counts elements, not bytes); M, N >= 1,
 *              K a positive multiple of 128 and at most 2^22.
 * out_dtype    an mxg_out_t (BF16, FP16 or FP32).
 * workspace    optional device memory for split-K across workgroups (the
 *              small-M shapes whose output tiles are too few to occupy
 *              every compute unit -- the pages' largest MXFP4 gain is such
 *              a decode shape, 32 x 14336 x 4096: "PyTorch 接上 FlyDSL",
 *              5ulink.com, section "内核级成绩"): the workgroups of one
 *              output tile each take a part of K, write FP32 partial tiles
 *              here, and the last to finish sums them in part order (so the
 *              result does not depend on timing).  Needs
 *              mx_scaled_mm_workspace_bytes(...) bytes, 16-byte aligned;
 *              its first 64 KiB (the arrival counters, at the same place
 *              for every shape and configuration) zero-filled once by the
 *              caller when it is allocated.  Every call leaves them at zero
 *              again, so one workspace serves any sequence of calls on one
 *              stream.  NULL, or fewer bytes than needed: the product runs
 *              without split-K -- same contract, possibly slower -- and the
 *              workspace is not touched.  Calls that may run at the same
 *              time (other streams) need distinct workspaces; the library
 *              keeps no pointer to it after the call's kernels complete.
 * workspace_bytes  size of workspace in bytes.
 * stream       HIP stream the work is enqueued on (0 = null stream).
 *
 * Returns MXG_OK after enqueueing, or an error status with nothing
 * enqueued (MXG_ERR_PTR_ALIGN also for a workspace not 16-byte aligned).
 *
 * Environment (read once, at the first call of the process; also honoured
 * by mx_scaled_mm_noalloc, mx_default_config and
 * mx_scaled_mm_workspace_bytes):
 *   MXG_CONFIG=<variant name>[:<K parts>]  run that configuration instead
 *     of the library's choice, for every shape (tuning; names from
 *     mx_variant_name).  A configuration that does not apply to a call's
 *     shape returns MXG_ERR_CONFIG, one whose K parts need more workspace
 *     than the call brings MXG_ERR_WORKSPACE, and a value that names no
 *     variant or part count MXG_ERR_CONFIG for every call.
 *   MXG_LOG=1  each call prints its format, M, N, K and the configuration
 *     it runs (variant, K parts) to stderr.
 */
int mx_scaled_mm_fp4(const void *a, const void *b, const void *a_scale, const void *b_scale,
                     void *c, int64_t M, int64_t N, int64_t K, int out_dtype, void *workspace,
                     size_t workspace_bytes, mxg_stream_t stream);

/* MXFP8 (E4M3) x MXFP8 NT scaled GEMM.  Same contract as mx_scaled_mm_fp4
 * except that a and b hold one E4M3 code per byte: [M][K] and [N][K]. */
int mx_scaled_mm_fp8(const void *a, const void *b, const void *a_scale, const void *b_scale,
                     void *c, int64_t M, int64_t N, int64_t K, int out_dtype, void *workspace,
                     size_t workspace_bytes, mxg_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * product as mx_scaled_mm_fp4 (is_fp4 = 1) / mx_scaled_mm_fp8 (0) with a
 * large enough workspace, whose split-K workspace is instead a static array
 * inside the library, one per GPU, of mx_noalloc_scratch_bytes() bytes (20
 * MiB, held until the process ends).  The call allocates nothing: no
 * hipMalloc or allocating library routine, here or in any call (the first
 * call on a GPU looks up the array's address and clears its counters with
 * a small kernel on `stream`).  The caller still provides a, b, the scales
 * and c as for mx_scaled_mm_fp4/fp8.  All calls on one GPU share the array:
 * calls that may overlap on one GPU (other streams, other threads) race
 * and must be serialized by the caller.  Returns the statuses of
 * mx_scaled_mm_fp4/fp8, plus MXG_ERR_SCRATCH, before anything is enqueued,
 * for a shape whose default configuration needs more workspace than the
 * array holds (none of the current ones does: at most 16.1 MiB).
 */
int mx_scaled_mm_noalloc(int is_fp4, const void *a, const void *b, const void *a_scale,
                         const void *b_scale, void *c, int64_t M, int64_t N, int64_t K, int out_dtype,
                         mxg_stream_t stream);
size_t mx_noalloc_scratch_bytes(void);

/* Workspace bytes mx_scaled_mm_fp4 (is_fp4 = 1) / mx_scaled_mm_fp8 (0)
 * use for this shape: 0 when the shape runs without split-K, or is
 * invalid.  A pure function of its arguments. */
size_t mx_scaled_mm_workspace_bytes(int is_fp4, int64_t M, int64_t N, int64_t K);

/* Explicit kernel variant and K-part count, for tests and tuning: run
 * variant `variant` (0 .. mx_num_variants()-1) with K cut into `splits`
 * parts (1: no split-K) instead of the default configuration.  is_fp4: 1
 * for MXFP4 operands, 0 for MXFP8.  Same operand contract and errors as
 * mx_scaled_mm_fp4/fp8, plus MXG_ERR_CONFIG for an unknown variant, a
 * variant without split-K asked for splits > 1, splits outside 1 .. 64 or
 * above K/512 (every part gets at least 512 K), or a K part beyond the
 * variant's limit (mx_variant_max_k); MXG_ERR_WORKSPACE when splits > 1
 * and the workspace is NULL or smaller than mx_config_workspace_bytes.
 * Every configuration computes the same product; they differ in tiling and
 * therefore in FP32 accumulation order. */
int mx_scaled_mm_config(int is_fp4, const void *a, const void *b, const void *a_scale,
                        const void *b_scale, void *c, int64_t M, int64_t N, int64_t K,
                        int out_dtype, int variant, int splits, void *workspace,
                        size_t workspace_bytes, mxg_stream_t stream);
/* Workspace bytes of an explicit configuration: 0 for splits == 1, for a
 * variant without split-K, or for invalid arguments. */
size_t mx_config_workspace_bytes(int variant, int splits, int64_t M, int64_t N);
int mx_num_variants(void);
/* Largest K a variant accepts for the format (is_fp4: 1 MXFP4, 0 MXFP8),
 * per K part under split-K; some variants keep the whole A tile of their
 * K range in LDS and so bound it.  Returns
 * MXG_ERR_CONFIG for an unknown variant.  A call with a larger K returns
 * MXG_ERR_CONFIG. */
int64_t mx_variant_max_k(int variant, int is_fp4);
/* Human-readable name of a variant (tile shape), or NULL if out of range. */
const char *mx_variant_name(int variant);

/*
 * MX quantization, the step before the GEMM ("PyTorch 接上 FlyDSL",
 * 5ulink.com, paragraph under the support matrix: one E8M0 scale per 32
 * values, BlockWise1x32).  Quantizes rows x 32-value blocks of BF16 values
 * along K, in the operand layout mx_scaled_mm_fp4/fp8 take (apply it to A
 * [M][K] and to B as [N][K]).  Per block (OCP MX v1.0 conversion; the pages
 * do not spell it out): scale code = floor(log2 amax) - emax + 127 clamped
 * to [0, 254] (emax 2 for E2M1, 8 for E4M3; 0 for an all-zero block; 0xFF
 * for a block holding a NaN or an infinity, whose element codes are 0);
 * each element |x| / 2^(code-127) rounded to the nearest E2M1/E4M3 code,
 * ties to even, saturating at the largest finite code; sign copied from x.
 *
 * x            BF16 bit patterns [rows][K], 16-byte aligned.
 * codes        output: E2M1 [rows][K/2] bytes (two codes per byte, even k in
 *              the low nibble) or E4M3 [rows][K] bytes; 16-byte aligned.
 * scales       output: E8M0 codes [rows][K/32].
 * rows, K      rows >= 1; K a positive multiple of 32.
 * is_fp4       1: E2M1 codes (MXFP4); 0: E4M3 codes (MXFP8).
 * stream       HIP stream the work is enqueued on (0 = null stream).
 *
 * Returns MXG_OK after enqueueing, or an error with nothing enqueued:
 * MXG_ERR_NULL, MXG_ERR_SHAPE (rows or K < 1, rows*K > 2^40),
 * MXG_ERR_K_ALIGN (K % 32 != 0), MXG_ERR_PTR_ALIGN, MXG_ERR_DEVICE,
 * MXG_ERR_HIP.  The caller owns all buffers; nothing is allocated.
 */
int mx_quantize_bf16(const void *x, void *codes, void *scales, int64_t rows, int64_t K,
                     int is_fp4, mxg_stream_t stream);

/*
 * Grouped (mixture-of-experts) MX GEMM ("PyTorch 接上 FlyDSL", 5ulink.com:
 * support-matrix row "Grouped GEMM" -- F.grouped_mm, the groups of A may
 * differ in length and empty groups are skipped -- and "MXFP8 Grouped GEMM"
 * among the next steps in the closing paragraph).  One call computes, for
 * every group g with rows [offs[g-1], offs[g]) of A (offs[-1] = 0):
 *
 *   C[rows of g] = A[rows of g] * B[g]^T      (the MX product above)
 *
 * a        [M][K/2] (FP4) or [M][K] (FP8): all groups' rows, in group order.
 * b        [groups][N][K/2] or [groups][N][K]: one NT operand per group.
 * a_scale  [M][K/32];  b_scale [groups][N][K/32].
 * c        [M][N] of out_dtype.  Rows in some group are overwritten; rows
 *          past the last group's end are not written.
 * offs     DEVICE memory, int32 [groups], 4-byte aligned: the end row of
 *          each group (cumulative sizes).  Read by the kernels, so no host
 *          synchronization is needed.  Entries are used as
 *          end[g] = min(M, max(0, offs[0..g])), so any content yields
 *          in-bounds rows; a group with end[g] == end[g-1] is empty and
 *          costs nothing.
 * groups   1 .. 65536.   M >= 0 (0: nothing is enqueued, and a, a_scale
 *          and c may be NULL), N >= 1, K as for mx_scaled_mm_*.
 *          groups * N * K must fit int64.
 *
 * Same alignment, ownership and error contract as mx_scaled_mm_fp4/fp8,
 * plus MXG_ERR_NULL for a NULL offs and MXG_ERR_SHAPE for a group count
 * out of range or a shape whose worst-case grid does not fit (rows per
 * group are only known on the device, so the grid covers the worst split).
 * Nothing is allocated.
 */
int mx_grouped_mm_fp4(const void *a, const void *b, const void *a_scale, const void *b_scale,
                      void *c, const int32_t *offs, int64_t groups, int64_t M, int64_t N,
                      int64_t K, int out_dtype, mxg_stream_t stream);
int mx_grouped_mm_fp8(const void *a, const void *b, const void *a_scale, const void *b_scale,
                      void *c, const int32_t *offs, int64_t groups, int64_t M, int64_t N,
                      int64_t K, int out_dtype, mxg_stream_t stream);
/* Grouped product with an explicit kernel variant, 0 .. mx_grouped_num_variants()-1
 * (names from mx_grouped_variant_name); MXG_ERR_CONFIG for an unknown one. */
int mx_grouped_mm_config(int is_fp4, const void *a, const void *b, const void *a_scale,
                         const void *b_scale, void *c, const int32_t *offs, int64_t groups,
                         int64_t M, int64_t N, int64_t K, int out_dtype, int variant,
                         mxg_stream_t stream);
int mx_grouped_num_variants(void);
const char *mx_grouped_variant_name(int variant);
/* The variant mx_grouped_mm_fp4/fp8 pick (from the mean rows per group),
 * or MXG_ERR_SHAPE. */
int mx_grouped_default_variant(int64_t groups, int64_t M, int64_t N);

/*
 * MX GEMM with a fused epilogue (the "GEMM 尾部融合" -- GEMM tail fusion --
 * of the next steps in "PyTorch 接上 FlyDSL", 5ulink.com, closing
 * paragraph; the pages do not define it further).  Per output element, in
 * FP32 inside the kernel, before the output leaves it:
 *
 *   y[m][n] = act(C[m][n] + bias[n])          (C the product above)
 *
 * is_fp4      1: MXFP4 operands, 0: MXFP8; operands and scales as for
 *             mx_scaled_mm_fp4/fp8.
 * bias        BF16 [N] (2-byte aligned; N <= 2^30), or NULL for no bias.
 * act         an mxg_act_t.
 * out_kind    MXG_OUT_BF16 / F16 / F32: y rounded to nearest even into c
 *             [M][N].  MXG_OUT_MXFP8 / MXFP4: y rounded to BF16, then
 *             MX-quantized along N exactly as mx_quantize_bf16 quantizes a
 *             BF16 [M][N] matrix: codes into c ([M][N] E4M3 or [M][N/2]
 *             E2M1), E8M0 codes into c_scale [M][N/32]; needs N % 32 == 0.
 *             The output is then the A operand of a following MX GEMM with
 *             K' = N.
 * c_scale     MX kinds only (else ignored, may be NULL).
 * variant     negative: the library's choice; else 0 .. mx_fused_num_variants()-1.
 *
 * Errors as mx_scaled_mm_fp4/fp8, plus MXG_ERR_DTYPE for an unknown
 * out_kind, MXG_ERR_CONFIG for an unknown act or variant, MXG_ERR_NULL for a
 * missing c_scale, MXG_ERR_SHAPE for an MX kind with N % 32 != 0,
 * MXG_ERR_PTR_ALIGN for an odd bias address.  Nothing is allocated.
 */
int mx_scaled_mm_fused(int is_fp4, const void *a, const void *b, const void *a_scale,
                       const void *b_scale, const void *bias, int act, void *c, void *c_scale,
                       int64_t M, int64_t N, int64_t K, int out_kind, int variant,
                       mxg_stream_t stream);
int mx_fused_num_variants(void);
const char *mx_fused_variant_name(int variant);
/* The variant mx_scaled_mm_fused picks for variant < 0 (is_fp4: 1 MXFP4,
 * 0 MXFP8), or MXG_ERR_SHAPE for M, N or K < 1. */
int mx_fused_default_variant(int is_fp4, int64_t M, int64_t N, int64_t K);
/* Largest K a fused variant accepts for the format (the decode-width
 * variants keep the A tile in LDS); MXG_ERR_CONFIG for an unknown variant.
 * A call with a larger K returns MXG_ERR_CONFIG. */
int64_t mx_fused_variant_max_k(int variant, int is_fp4);

/*
 * Dense BF16 / FP16 GEMM ("PyTorch 接上 FlyDSL", 5ulink.com, support-matrix
 * row for torch.mm: FP16/BF16, static 2-D, NN / NT / TN / TT):
 *
 *   C[M][N] = A[M][K] * B[K][N]      FP32 accumulation
 *
 * dtype      0: BF16 operands, 1: FP16 operands (bit patterns, 2 bytes each).
 * trans_a    0: a is stored [M][K] row-major; 1: a is stored [K][M].
 * trans_b    0: b is stored [K][N] row-major; 1: b is stored [N][K].
 *            (trans_a = 0, trans_b = 1 is "NT", the MFMA's own layout.)
 * c          [M][N] row-major of out_dtype (BF16 / FP16 / FP32), overwritten.
 * M, N, K    >= 1; the contiguous dimension of each stored operand (K or M
 *            for a, N or K for b) a multiple of 8; M*K and N*K below 2^30
 *            elements.
 *
 * Returns MXG_OK after enqueueing, or MXG_ERR_NULL, MXG_ERR_DTYPE (dtype or
 * out_dtype), MXG_ERR_CONFIG (trans flag not 0/1), MXG_ERR_SHAPE,
 * MXG_ERR_PTR_ALIGN (a, b, c 16-byte aligned), MXG_ERR_DEVICE, MXG_ERR_HIP.
 * Nothing is allocated; same ownership and stream contract as above.
 */
int mx_dense_gemm(int dtype, int trans_a, int trans_b, const void *a, const void *b, void *c,
                  int64_t M, int64_t N, int64_t K, int out_dtype, mxg_stream_t stream);

/* The configuration the default entry points pick for a shape: returns the
 * variant (>= 0) and stores the K-part count in *splits (if not NULL), for
 * a call given a large enough workspace (with_workspace = 1) or none (0);
 * or a negative status for an invalid shape. */
int mx_default_config(int is_fp4, int64_t M, int64_t N, int64_t K, int with_workspace, int *splits);
/* mx_default_config(is_fp4, M, N, K, 1, NULL). */
int mx_default_variant(int is_fp4, int64_t M, int64_t N, int64_t K);

/* Measurement support: enqueue an empty kernel on exactly the grid and
 * workgroup size that mx_scaled_mm_fp4/fp8 would launch for this shape, so
 * that the launch cost alone can be timed next to the product (the
 * "dispatch floor" of shapes too small to reach any bandwidth or MFMA
 * roofline).  Returns MXG_OK after enqueueing, or the status
 * mx_default_variant gives for the shape, MXG_ERR_DEVICE or MXG_ERR_HIP.
 * Touches no memory. */
int mx_empty_like(int is_fp4, int64_t M, int64_t N, int64_t K, mxg_stream_t stream);

/* Static description of a status code; never NULL. */
const char *mx_status_string(int status);

/* The last HIP error code seen by this thread (0 if none). */
int mx_last_hip_error(void);

/* ABI version of this header (bumped on incompatible changes). */
int mx_abi_version(void);
#define MXGEMM_ABI_VERSION 8

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_H */
