/*
 * bsfp8.h -- C-ABI of libbsfp8.so: block-scaled FP8 and NVFP4-style linear
 * layers on AMD MI355X (gfx950).
 *
 * Page citations use the page titles:
 *   [FG-FP8] "Transformers 中的细粒度 FP8 量化：配置、DeepGEMM 加速路径与
 *            UE8M0 缩放格式完全指南", sections 一 .. 九
 *   [HF-PT]  "FP8 de granularidade fina" (Transformers docs)
 *   [NVFP4]  "混合精度策略解析：NVIDIA Mistral-Medium-3.5-128B-NVFP4中FP8与
 *            NVFP4的协同工作", sections on NVFP4 and on the config files
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer on the current HIP device,
 *   except where a parameter says "host".  The caller allocates and owns all
 *   memory; the library allocates nothing, keeps no state between calls
 *   (apart from a per-device architecture check done once), never
 *   synchronises the device and never prints.
 * - `stream` is a hipStream_t passed as void*; NULL means the default
 *   stream.  Every call only enqueues work on that stream.
 * - Matrices are row-major and dense unless a leading dimension is given.
 *   bf16 tensors are raw 16-bit patterns (uint16_t); FP8 tensors are OCP
 *   E4M3FN bytes; UE8M0 scales are E8M0 bytes (value 2^(b-127)); fp32
 *   scales are IEEE binary32.
 * - All argument checks run on the host before any HIP call, so the error
 *   returns below are reachable without a GPU.  A zero-sized problem
 *   (M, T or R == 0) returns BSFP8_OK without launching anything.
 * - Return value: a bsfp8_status; BSFP8_EHIP means a HIP call or a kernel
 *   launch failed (the HIP error is not cleared and can be read with
 *   hipGetLastError / hipPeekAtLastError).
 * - Pointers must be 16-byte aligned and leading dimensions must keep every
 *   row 16-byte aligned (EINVAL otherwise).
 */
#ifndef BSFP8_H
#define BSFP8_H

#include <stddef.h>
#include <stdint.h>

#ifndef BSFP8_API
#define BSFP8_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSFP8_OK = 0,
  BSFP8_EINVAL = 1,   /* bad argument: enum, size, null pointer, alignment  */
  BSFP8_ENOTSUP = 2,  /* legal on the pages but not provided here, or a     */
                      /* device that is not gfx950, or a stream that       */
                      /* belongs to another device                         */
  BSFP8_ENOSPC = 3,   /* workspace smaller than bsfp8_workspace_size()      */
  BSFP8_EHIP = 4      /* HIP runtime / launch error                         */
} bsfp8_status;

/* scale_fmt: [FG-FP8] §四 allows "float" or "ue8m0"; §七 stores UE8M0 scales
   as float8_e8m0fnu bytes. */
typedef enum { BSFP8_SCALE_FLOAT = 0, BSFP8_SCALE_UE8M0 = 1 } bsfp8_scale_fmt;

/* activation_scheme: [FG-FP8] §四 allows "dynamic" or "static" (the pages
   keep static on a separate kernel path, §6.1, §6.3, and give no formula).
   Static here is one calibrated per-tensor scale supplied by the caller:
   fp8_quant_act (in x_scale[0]) and fp8_linear (through act_scale) take it
   with 128 x 128 blocks; the other entry points consume quantized operands
   and do not depend on the scheme. */
typedef enum { BSFP8_ACT_DYNAMIC = 0, BSFP8_ACT_STATIC = 1 } bsfp8_act_scheme;

/* Operation ids for bsfp8_workspace_size. */
typedef enum {
  BSFP8_OP_BLOCK_GEMM = 0,
  BSFP8_OP_LINEAR = 1,
  BSFP8_OP_GROUPED_GEMM = 2,
  BSFP8_OP_FP4_QUANT = 3,
  BSFP8_OP_FP4_GEMM = 4,
  BSFP8_OP_FP8_FP4_GEMM = 5,
  BSFP8_OP_LINEAR_B32 = 6      /* fp8_linear with (32, 32) weight blocks */
} bsfp8_op;

/* Kernels fp8_block_gemm / fp8_linear choose between (bsfp8_gemm_kernel). */
typedef enum {
  BSFP8_GEMM_NONE = 0,          /* empty problem: nothing is launched          */
  BSFP8_GEMM_RESERVED = 1,      /* not returned                                */
  BSFP8_GEMM_TILE_128x256 = 2,  /* LDS-staged MFMA kernel, 128 x 256 tiles     */
  BSFP8_GEMM_TILE_256x256 = 3,  /* LDS-staged MFMA kernel, 256 x 256 tiles     */
  BSFP8_GEMM_DECODE = 4         /* M <= 16: one-launch weight-streaming kernel */
} bsfp8_gemm_kind;

/* Library version (major * 10000 + minor * 100 + patch). */
BSFP8_API int32_t bsfp8_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
BSFP8_API const char* bsfp8_status_string(int32_t status);

/*
 * fp8_quant_act -- activation quantization in 1 x group_k groups: per-token
 * dynamic scales ([FG-FP8] §一, second bullet; [HF-PT] opening list) or one
 * static calibrated scale ([FG-FP8] §四: activation_scheme "static").
 *
 *   x        bf16 [M][ldx], read-only; only the first K columns are used.
 *   M, K     rows (tokens) and columns (input channels); K % 16 == 0.
 *   ldx      row stride of x in elements, ldx >= K, ldx % 8 == 0.
 *   group_k  group width; must equal the weight block's K size: 128, or
 *            32 for (32, 32) weight blocks ([FG-FP8] §一: the groups line
 *            up with the weight blocks; §九: (32, 32) is a tested
 *            non-default block).  STATIC takes 128 only.
 *   act_scheme  BSFP8_ACT_DYNAMIC: the scales below, per group.
 *               BSFP8_ACT_STATIC: x_scale[0] holds the calibrated
 *               per-tensor scale on entry (fp32 s > 0, or the E8M0 byte
 *               b, s = 2^(b-127)); codes = E4M3(fl32(x/s)) or
 *               E4M3(x * 2^-(b-127)), and every entry of x_scale is set to
 *               that scale, so fp8_block_gemm takes the result unchanged.
 *   scale_fmt   FLOAT: s = fl32(amax/448), codes = E4M3(fl32(x/s)).
 *               UE8M0: s = 2^e, e = ceil(log2(amax/448)) clamped to
 *               [-127,127] ([FG-FP8] §七 note: fp32 scales round *up* to
 *               UE8M0), stored as byte e+127; codes = E4M3(x * 2^-e).
 *               amax = 0 gives s = 1.  E4M3 rounding is to nearest even,
 *               saturating at +-448, sign of zero kept.
 *   xq       out, E4M3 [M][K] (dense).
 *   x_scale  out, [M][ceil(K/group_k)] fp32 (FLOAT) or uint8 (UE8M0); the
 *            dequantization multiplier of each group.
 * Errors: EINVAL (null pointers, M or K < 0, K % 16, ldx < K, ldx % 8,
 * group_k <= 0, bad enum, misalignment); ENOTSUP (group_k other than 128 or
 * 32, or 32 with STATIC).
 */
BSFP8_API int32_t fp8_quant_act(const void* x, int64_t M, int64_t K, int64_t ldx,
                      int32_t group_k, int32_t act_scheme, int32_t scale_fmt,
                      void* xq, void* x_scale, void* stream);

/*
 * fp8_quant_weight -- per 2D block weight quantization
 * (weight_block_size = (block_n, block_k), [FG-FP8] §一 first bullet; the
 * scale tensor weight_scale_inv has shape (ceil(N/bn), ceil(K/bk)),
 * [FG-FP8] §一 third paragraph).
 *
 *   w        bf16 [N][ldw] in nn.Linear orientation (out, in); read-only.
 *   N, K     output and input features; K % 16 == 0.
 *   ldw      row stride in elements, ldw >= K, ldw % 8 == 0.
 *   block_n, block_k   (128, 128) or (32, 32) ([FG-FP8] §九); other
 *            positive sizes -> ENOTSUP.
 *   scale_fmt  as for fp8_quant_act, with the amax over the whole block.
 *   wq       out, E4M3 [N][K].
 *   w_scale_inv  out, [ceil(N/bn)][ceil(K/bk)] fp32 or uint8 E8M0.
 * A partial edge block takes its amax over its in-range elements only.
 */
BSFP8_API int32_t fp8_quant_weight(const void* w, int64_t N, int64_t K, int64_t ldw,
                         int32_t block_n, int32_t block_k, int32_t scale_fmt,
                         void* wq, void* w_scale_inv, void* stream);

/*
 * fp8_block_gemm -- the block-scaled FP8 GEMM ([FG-FP8] §一: aligned act
 * groups and weight blocks let the matmul run block by block):
 *
 *   Y[m][n] = bf16_rne( sum_kb S_a[m][kb] * S_w[n/B][kb]
 *                          * sum_{k in kb} Xq[m][k] * Wq[n][k]  + bias[n] )
 *
 * with B the block edge (128, or 32), exact FP8 products, fp32
 * accumulation, the combined scale applied to the fp32 partial sum once per
 * B-wide K block, and the unquantized bias ([FG-FP8] §三: bias is not
 * quantized) added in fp32.
 *
 *   xq, x_scale       as written by fp8_quant_act (M rows).
 *   wq, w_scale_inv   as written by fp8_quant_weight (N rows).
 *   bias              bf16 [N] or NULL.
 *   y                 out, bf16 [M][N].
 *   block_n, block_k  (128, 128), or (32, 32) with 1 x 32 act groups
 *                     (a separate kernel, no workspace).
 *   workspace         device buffer of at least
 *                     bsfp8_workspace_size(BSFP8_OP_BLOCK_GEMM, M, N, K, 0)
 *                     bytes (may be NULL when that size is 0); contents on
 *                     entry are ignored, on exit undefined.
 * Errors: EINVAL (dims < 0, K % 16, N % 8, null required pointers, bad
 * enum, misalignment); ENOTSUP (other block sizes, K > 2^22); ENOSPC.
 * fp8_linear shares these limits (with (32, 32) blocks its workspace is
 * bsfp8_workspace_size(BSFP8_OP_LINEAR_B32, ...)); fp8_grouped_gemm takes
 * (128, 128) and (32, 32) blocks, fp8_grouped_gemm_silu_mul_quant
 * (128, 128) only.
 */
BSFP8_API int32_t fp8_block_gemm(const void* xq, const void* x_scale, const void* wq,
                       const void* w_scale_inv, const void* bias, void* y,
                       int64_t M, int64_t N, int64_t K, int32_t block_n,
                       int32_t block_k, int32_t scale_fmt, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * fp8_linear -- one FP8 linear layer on bf16 activations: fp8_quant_act
 * followed by fp8_block_gemm, i.e. the forward of the pages' FP8Linear
 * ([FG-FP8] §八 step 6).  Results are identical to calling the two entry
 * points in sequence.  For small M the quantization runs inside the GEMM
 * launch; otherwise the quantized activations are staged in `workspace`.
 *
 *   x          bf16 [M][ldx];  other arguments as above.
 *   act_scheme BSFP8_ACT_DYNAMIC (act_scale ignored, may be NULL) or
 *              BSFP8_ACT_STATIC: act_scale is a DEVICE pointer to the
 *              calibrated per-tensor scale (fp32 s > 0, 4-byte aligned, or
 *              the E8M0 byte), read-only; the result equals fp8_quant_act
 *              with the static scheme and that scale, then fp8_block_gemm.
 *              STATIC takes 128 x 128 blocks only (ENOTSUP otherwise);
 *              a NULL act_scale is EINVAL.
 *   workspace  >= bsfp8_workspace_size(BSFP8_OP_LINEAR, M, N, K, 0) bytes
 *              (the same for both schemes).
 */
BSFP8_API int32_t fp8_linear(const void* x, int64_t ldx, const void* wq,
                   const void* w_scale_inv, const void* bias, void* y,
                   int64_t M, int64_t N, int64_t K, int32_t block_n,
                   int32_t block_k, int32_t act_scheme, int32_t scale_fmt,
                   const void* act_scale, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Bytes of the device array that fp8_linear_noalloc takes as its workspace
   (one array per GPU the library runs on, held until the process ends). */
#define BSFP8_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * fp8_linear_noalloc -- fp8_linear for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and results as fp8_linear, without the
 * workspace: the library uses a device array of BSFP8_NOALLOC_SCRATCH_BYTES
 * of its own (looked up once per device), and calls no allocating routine.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; calls that overlap on one GPU (different streams
 *     without ordering) race and give undefined results.
 *   - Errors: those of fp8_linear, and ENOSPC when
 *     bsfp8_workspace_size(BSFP8_OP_LINEAR or BSFP8_OP_LINEAR_B32, M, N, K, 0)
 *     exceeds BSFP8_NOALLOC_SCRATCH_BYTES (use fp8_linear then).
 */
BSFP8_API int32_t fp8_linear_noalloc(const void* x, int64_t ldx, const void* wq,
                                     const void* w_scale_inv, const void* bias, void* y,
                                     int64_t M, int64_t N, int64_t K, int32_t block_n,
                                     int32_t block_k, int32_t act_scheme, int32_t scale_fmt,
                                     const void* act_scale, void* stream);

/*
 * fp8_grouped_gemm -- MoE expert GEMM over contiguous per-expert row
 * segments ([FG-FP8] §一 FP8Experts; §6.4 and §七 expert backends).  For
 * every expert e, rows [off[e], off[e+1]) of Y are the fp8_block_gemm of the
 * same rows of (xq, x_scale) with expert e's (wq[e], w_scale_inv[e]).
 *
 *   xq           E4M3 [T][K];  x_scale [T][ceil(K/B)] (fp32 | UE8M0).
 *   wq           E4M3 [E][N][K];  w_scale_inv [E][ceil(N/B)][ceil(K/B)].
 *   block_n, block_k  (B, B) = (128, 128), or (32, 32) with 1 x 32 act
 *                groups ([FG-FP8] §九); other sizes ENOTSUP.
 *   seg_offsets  DEVICE int32 [E+1]: off[0] = 0, nondecreasing, off[E] = T.
 *                This is a precondition and is not checked (checking would
 *                need a device synchronisation).
 *   E            number of experts, 1 <= E <= 1024.
 *   y            out, bf16 [T][N]; rows of empty segments do not exist.
 *   workspace    >= bsfp8_workspace_size(BSFP8_OP_GROUPED_GEMM, T, N, K, E).
 */
BSFP8_API int32_t fp8_grouped_gemm(const void* xq, const void* x_scale, const void* wq,
                         const void* w_scale_inv, const int32_t* seg_offsets,
                         int32_t E, void* y, int64_t T, int64_t N, int64_t K,
                         int32_t block_n, int32_t block_k, int32_t scale_fmt,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8_grouped_gemm_silu_mul_quant -- an MoE expert MLP's gate/up GEMM with
 * the step to the down GEMM fused into its epilogue: the gate/up/down MLP
 * of [NVFP4] (layer-wise quantization section) run as FP8 experts
 * ([FG-FP8] §一 FP8Experts, §6.4), the down projection's input quantized
 * per token in 1 x 128 groups like any activation ([FG-FP8] §一).
 * For every expert e and row t in [off[e], off[e+1]):
 *   g = (X W_e[0:I]^T)[t],  u = (X W_e[I:2I]^T)[t]   (fp32 accumulation),
 *   h = bf16(silu(g) * u),  silu(g) = g / (1 + e^-g),
 *   (hq, h_scale) = the 1 x 128 activation quantization of h (the codes
 *   and scales fp8_quant_act writes for that bf16 row), in scale_fmt.
 * The result feeds fp8_grouped_gemm (the down projection) unchanged.
 *
 *   xq, x_scale  as fp8_grouped_gemm (K input channels, 1 x 128 groups).
 *   wq           E4M3 [E][2I][K]: rows [0, I) gate, rows [I, 2I) up;
 *                w_scale_inv [E][2I/128][ceil(K/128)] (fp32 | UE8M0).
 *   seg_offsets  DEVICE int32 [E+1], the same precondition as
 *                fp8_grouped_gemm.
 *   hq           out, E4M3 [T][I] (16-byte aligned);  h_scale out,
 *                [T][I/128] fp32 | UE8M0.
 *   h_bf16       out, bf16 [T][I] (the rounded h), or NULL.
 *   I            intermediate size, a positive multiple of 128.
 * No workspace.  Errors: those of fp8_grouped_gemm with N = 2I; EINVAL for
 * I <= 0 or I % 128 != 0, a null or misaligned h_scale (4 bytes) or a
 * misaligned h_bf16 (16 bytes); ENOTSUP when one expert's weight (2 I K
 * bytes) exceeds 2^31 - 1 bytes.
 */
BSFP8_API int32_t fp8_grouped_gemm_silu_mul_quant(const void* xq, const void* x_scale,
                                        const void* wq, const void* w_scale_inv,
                                        const int32_t* seg_offsets, int32_t E, void* hq,
                                        void* h_scale, void* h_bf16, int64_t T, int64_t I,
                                        int64_t K, int32_t scale_fmt, void* stream);

/*
 * fp4_quant -- NVFP4-style quantization ([NVFP4]: 4-bit float weights and
 * input activations in 16-element groups, group_size 16): E2M1 codes with
 * an E4M3 scale per 16-element group and one fp32 scale per tensor.
 *
 *   g   = fl32(amax_tensor / 2688)  (1.0 for an all-zero tensor)
 *   sg  = E4M3(fl32(amax_group / fl32(6 g)))
 *   eff = fl32(dec(sg) * g);  codes = E2M1(fl32(x / eff)), 0 when eff == 0
 *
 *   x          bf16 [R][K], K % 32 == 0.
 *   dynamic_tscale  1: compute g from x and write it to *tscale;
 *                   0: read g from *tscale (must be > 0, finite).
 *   q4         out, uint8 [R][K/2]; element 2i in the low nibble of byte i.
 *   gscale     out, E4M3 [R][K/16].
 *   tscale     DEVICE float[1], out (dynamic) or in (static).
 *   workspace  >= bsfp8_workspace_size(BSFP8_OP_FP4_QUANT, R, 0, K, 0).
 */
BSFP8_API int32_t fp4_quant(const void* x, int64_t R, int64_t K, int32_t dynamic_tscale,
                  void* q4, void* gscale, float* tscale, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * fp4_group_gemm -- GEMM of two NVFP4-style operands (the MLP projections of
 * [NVFP4]):
 *
 *   Y[m][n] = bf16_rne( g_a g_w sum_k dec(qa[m][k]) dec(sa[m][k/16])
 *                                    * dec(qw[n][k]) dec(sw[n][k/16]) )
 *
 *   xq4, x_gscale, x_tscale   as written by fp4_quant for X (M rows).
 *   wq4, w_gscale, w_tscale   as written by fp4_quant for W (N rows).
 *   y                          out, bf16 [M][N].  K % 32 == 0.
 *   workspace  >= bsfp8_workspace_size(BSFP8_OP_FP4_GEMM, M, N, K, 0).
 * Errors: EINVAL (sizes, null pointers, misalignment), ENOTSUP (K > 2^22,
 * the bound of the FP8 GEMMs), ENOSPC (workspace).
 */
BSFP8_API int32_t fp4_group_gemm(const void* xq4, const void* x_gscale,
                       const float* x_tscale, const void* wq4,
                       const void* w_gscale, const float* w_tscale, void* y,
                       int64_t M, int64_t N, int64_t K, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * mxfp4_quant_weight -- FP4-packed weights with UE8M0 block scales, the
 * V4-style expert weights the pages' FP8-activation x FP4-weight linear
 * consumes ([FG-FP8] §一 FP4-packed experts, §6.1 deepgemm_fp8_fp4_linear;
 * UE8M0 scales §七).  Per 1 x 32 group along K of each row:
 *   e = ceil(log2(amax/6)) clamped to [-127,127] (0 for amax = 0), stored
 *   as the byte e+127;  codes = E2M1(w * 2^-e), round to nearest even.
 *
 *   w        bf16 [N][ldw], K % 32 == 0, ldw >= K, ldw % 8 == 0.
 *   wq4      out, uint8 [N][K/2]: element 2i in the low nibble of byte i.
 *   w_scale  out, E8M0 bytes [N][K/32].
 * Errors: EINVAL (sizes, null pointers, misalignment).
 */
BSFP8_API int32_t mxfp4_quant_weight(const void* w, int64_t N, int64_t K, int64_t ldw,
                                     void* wq4, void* w_scale, void* stream);

/*
 * fp8_fp4_gemm -- FP8 activations x MXFP4 weights ([FG-FP8] §6.1, the
 * FP8 x FP4 linear), on gfx950's scaled MFMA with the weights as its FP4
 * operand and their E8M0 group scales as its block scales:
 *
 *   Y[m][n] = bf16( sum_k E4M3(xq[m][k]) S_a[m][k/128]
 *                         * E2M1(wq4[n][k]) 2^(w_scale[n][k/32]-127) + bias[n] )
 *
 *   xq, x_scale  as written by fp8_quant_act (1 x 128 groups; scale_fmt
 *                FLOAT or UE8M0).
 *   wq4, w_scale as written by mxfp4_quant_weight (N rows).
 *   bias         bf16 [N] or NULL;  y out, bf16 [M][N].
 *   K % 32 == 0, N % 8 == 0, K <= 2^22.
 *   workspace    >= bsfp8_workspace_size(BSFP8_OP_FP8_FP4_GEMM, M, N, K, 0).
 * M <= 16 streams the weights in one launch (half the bytes of FP8);
 * larger M runs the LDS MFMA kernel on 128 x 256 tiles, K split as for
 * fp8_block_gemm.  Errors as fp8_block_gemm (block sizes are fixed here).
 */
BSFP8_API int32_t fp8_fp4_gemm(const void* xq, const void* x_scale, const void* wq4,
                               const void* w_scale, const void* bias, void* y, int64_t M,
                               int64_t N, int64_t K, int32_t scale_fmt, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * fp8_fp4_grouped_gemm -- MoE expert GEMM with FP4-packed expert weights
 * ([FG-FP8] §一: FP8Experts can take V4-style FP4-packed expert weights;
 * §6.1 and §6.4: the FP8 x FP4 linear and the grouped expert GEMMs of the
 * fast backend).  For every expert e, rows [off[e], off[e+1]) of Y are the
 * fp8_fp4_gemm of the same rows of (xq, x_scale) with expert e's MXFP4
 * weights (wq4[e], w_scale[e]):
 *
 *   Y[t][n] = bf16( sum_k E4M3(xq[t][k]) S_a[t][k/128]
 *                         * E2M1(wq4[e][n][k]) 2^(w_scale[e][n][k/32]-127) )
 *
 *   xq, x_scale  as written by fp8_quant_act (T rows; FLOAT or UE8M0).
 *   wq4          uint8 [E][N][K/2] (mxfp4_quant_weight per expert);
 *   w_scale      E8M0 bytes [E][N][K/32].
 *   seg_offsets  DEVICE int32 [E+1], the precondition of fp8_grouped_gemm.
 *   E            1 <= E <= 1024;  y out, bf16 [T][N].
 *   K % 32 == 0, N % 8 == 0, K <= 2^22.  No workspace.
 * Errors as fp8_grouped_gemm (block sizes are fixed here).
 */
BSFP8_API int32_t fp8_fp4_grouped_gemm(const void* xq, const void* x_scale, const void* wq4,
                                       const void* w_scale, const int32_t* seg_offsets,
                                       int32_t E, void* y, int64_t T, int64_t N, int64_t K,
                                       int32_t scale_fmt, void* stream);

/*
 * fp8_dequant_weight -- fold the block scales back into the weights, the
 * dequantize-on-load step for pre-quantized checkpoints ([FG-FP8] §五,
 * Fp8Dequantize):  W[n][k] = bf16_rne(fl32(E4M3(wq[n][k]) * S_w[n/B][k/B]))
 * for (B, B) blocks, B = 128 or 32.
 *
 *   wq           E4M3 [N][K], K % 16 == 0.
 *   w_scale_inv  [ceil(N/B)][ceil(K/B)] fp32 or UE8M0 bytes.
 *   w            out, bf16 [N][K].
 * Codes 0x7F / 0xFF (E4M3 NaN) and the E8M0 byte 0xFF are outside the
 * contract.  Errors: EINVAL (sizes, null pointers, misalignment, bad enum);
 * ENOTSUP (block sizes other than (128, 128) and (32, 32)).
 */
BSFP8_API int32_t fp8_dequant_weight(const void* wq, int64_t N, int64_t K, int32_t block_n,
                                     int32_t block_k, int32_t scale_fmt,
                                     const void* w_scale_inv, void* w, void* stream);

/*
 * fp8_scale_to_ue8m0 -- power-of-two scales stored in float32 containers to
 * the one-byte UE8M0 form the kernels read, exactly ([FG-FP8] §七: such
 * checkpoints are converted on load).  scale[i] = 2^k with -127 <= k <= 127
 * becomes the byte k + 127; any other value (not a power of two, <= 0,
 * outside that range, Inf, NaN) becomes 0xFF, the E8M0 NaN encoding, which
 * callers can test for.
 *
 *   scale  device fp32 [n];  out  device uint8 [n].
 */
BSFP8_API int32_t fp8_scale_to_ue8m0(const float* scale, int64_t n, void* out, void* stream);

/*
 * Bytes of device workspace the given operation needs for this problem
 * (0 if none).  `op` is a bsfp8_op; M is T for the grouped GEMM and R for
 * fp4_quant; E is used by the grouped GEMM only.  Returns (size_t)-1 for an
 * unknown op or negative sizes.
 */
BSFP8_API size_t bsfp8_workspace_size(int32_t op, int64_t M, int64_t N, int64_t K,
                            int32_t E);

/*
 * Which kernel (a bsfp8_gemm_kind) fp8_block_gemm and fp8_linear launch for
 * an M x N x K problem with 128 x 128 blocks (fp8_fp4_gemm follows the same
 * choice; (32, 32) blocks run their own kernel, the decode kernel up to
 * M = 16), and into how many K splits it cuts K (*splits, may
 * be NULL; 1 when K is not split: splits above 1 write fp32 partial sums to
 * the workspace and add one reduction launch).  The grouped GEMM does not
 * split K: experts with more than 128 rows run on 256 x 256 tiles and the
 * others on 64 x 256 tiles, in two launches.  Host-only, touches no device.
 * Returns -1 for negative sizes.
 */
BSFP8_API int32_t bsfp8_gemm_kernel(int64_t M, int64_t N, int64_t K, int32_t* splits);

#ifdef __cplusplus
}
#endif

#endif /* BSFP8_H */
