/*
 * bsgemm: the block-scaled low-precision linear layer of transformer
 * inference on AMD Instinct MI355X (gfx950), as a C ABI.
 *
 *   1. fp8_quant_rows   bf16 activations -> per-token e4m3fn codes + fp32 scale
 *   2. gemm_bs_fp8      Y = dequant(A) dequant(W)^T (+ bias, + tanh-GELU), W in
 *                       e4m3fn with one E8M0 scale per 32x32 block
 *   3. gemm_mxfp4_w4a8  the same with MXFP4 weights (fp4 e2m1, one E8M0 scale
 *                       per row per 32 along K)
 *   4. gemm_fp8_rowwise  e4m3 weights with one fp32 scale per output channel;
 *      fp8_quant_rows_static  quantization with a given per-tensor scale
 *   5. fp4_quant_rows, gemm_mxfp4_w4a4  MXFP4 activations x MXFP4 weights
 *   6. gemm_mxfp4_w4a8_grouped  MoE: many experts' MXFP4 weights, one launch
 *   7. add_rms_norm_quant_fp8, silu_mul_quant_fp8
 *                       fused producers: RMSNorm (with an optional residual
 *                       add) or SiLU(gate) * up, then step 1, in one kernel
 *
 * Sources (web pages bundled as the reference):
 *   - formats and scale grids: vLLM DeepSeek-V4 AMD mono runner page,
 *     AttnWeights (an e4m3 [2048, 7168] projection weight with a [64, 224]
 *     uint8 E8M0 grid, one byte per 32x32 block) and MonoLayerWeights.check
 *     (fp4x2 expert weights [.., N, K/2] with uint8 scales [N, K/32]);
 *   - per-token (q_fp8, scale) pairs feeding the W4A8 GEMM: sly-radiance
 *     README, fused norm/quant rows of its file table;
 *   - bias / bias+GELU fused into the FP8 GEMM epilogue: flash-rt
 *     groot_n17 frontend, module docstring and _fused_epilogue_enabled;
 *   - the tanh GELU: cortiq vit.rs, ACT_SRC shader, act == 2 branch;
 *   - raw device pointers + sizes + a stream, caller-owned outputs, shape
 *     checks because loads are unbounded: flash-rt groot_n17 (bf16_nn_bias
 *     call sites) and the mono runner page (_check_tensors, forward).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller. Nothing
 *     is allocated, freed or synchronized; work is enqueued on `stream`
 *     (a hipStream_t passed as void*, NULL = the null stream) and the call
 *     returns before it runs. Calls may be captured into a HIP graph.
 *   - Matrices are row-major with a leading dimension (row stride) given in
 *     elements (bytes for 8-bit and packed data). Alignment: matrices of
 *     codes, bf16 matrices, the bf16 norm weight and the outputs start on
 *     16-byte boundaries, and leading dimensions are multiples of 16 bytes;
 *     fp32 per-token scales (and the static scale) are 4-byte aligned, fp32
 *     per-channel scales 16-byte aligned, the bias 2-byte aligned; E8M0
 *     scale grids may start at any byte address.
 *   - Arguments are checked on the host before anything is launched; on
 *     error nothing is launched and outputs are untouched. The first call
 *     on a device also checks that it is a gfx950 (BS_EARCH otherwise).
 *   - Inputs must not overlap outputs.
 *   - Returns BS_OK (0) or a negative bs_status.
 */
#ifndef BSGEMM_H
#define BSGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bs_status {
    BS_OK = 0,
    BS_EINVAL = -1,      /* a size, leading dimension, epilogue or null pointer is invalid */
    BS_EALIGN = -2,      /* a pointer or leading dimension is not aligned as required */
    BS_EARCH = -3,       /* no HIP device, or the current device is not gfx950 */
    BS_EWORKSPACE = -4,  /* workspace smaller than bs_workspace_bytes() */
    BS_ELAUNCH = -5      /* the kernel launch failed (hipGetLastError) */
};

/* Largest row stride (bytes) of A and W the GEMMs accept (4 MiB): tile
 * offsets are 32-bit buffer offsets. */
#define BS_MAX_LD_BYTES ((int64_t)1 << 22)

enum bs_epilogue {
    BS_EPI_NONE = 0,            /* y = s[m] * acc                               */
    BS_EPI_BIAS = 1,            /* y = s[m] * acc + bias[n]                     */
    BS_EPI_BIAS_GELU_TANH = 2   /* y = gelu_tanh(s[m] * acc + bias[n])          */
};

/*
 * Per-token quantization to e4m3fn (the "(q_fp8, scale)" pair of the
 * sly-radiance README's fused producers). For each row m of x:
 *     amax    = max_k |x[m,k]|
 *     scale[m]= amax / 448                     (fp32, correctly rounded)
 *     q[m,k]  = e4m3fn(x[m,k] / scale[m])      (fp32 division correctly
 *               rounded, then nearest e4m3 value with ties to the even
 *               mantissa, saturating at +-448, sign kept also for zeros)
 * A row of zeros gets scale 0 and codes 0x00 / 0x80 (for -0).
 *   x_bf16  [M, K] bf16, row stride ld_x elements (ld_x >= K, 2*ld_x % 16 == 0)
 *   q_e4m3  [M, K] uint8 out, row stride ld_q bytes (ld_q >= K, ld_q % 16 == 0)
 *   scale   [M] fp32 out
 *   M >= 1, K >= 32, K % 32 == 0. NaN/Inf inputs are not supported.
 */
int fp8_quant_rows(const void *x_bf16, int64_t ld_x, void *q_e4m3, int64_t ld_q,
                   float *scale, int64_t M, int64_t K, void *stream);

/*
 * Quantization with one given (static, per-tensor) scale, for calibrated
 * activation scales (flash-rt groot_n17 frontend, fused-epilogue tier: its
 * host alphas are act_scale x w_scale per site):
 *     q[m,k] = e4m3fn(x[m,k] / scale_in[0])    (same rounding as above)
 *   scale_in   device pointer to one fp32 > 0 (finite); read by the kernel
 *   scale_out  [M] fp32 out, or NULL: every entry set to scale_in[0], so the
 *              pair (q, scale_out) feeds the GEMMs like fp8_quant_rows' does
 *   Other arguments as fp8_quant_rows. Values beyond 448 * scale saturate.
 */
int fp8_quant_rows_static(const void *x_bf16, int64_t ld_x, const float *scale_in,
                          void *q_e4m3, int64_t ld_q, float *scale_out, int64_t M, int64_t K,
                          void *stream);

/*
 * Fused producers: the row that feeds the quantizer is computed in the same
 * kernel, and the result is the "(q_fp8, scale)" pair of fp8_quant_rows
 * applied to that bf16 row (sly-radiance README, fused norm/quant rows of
 * its file table: add_rms_quant and silu_mul_quant hand (q_fp8, scale) to
 * the W4A8 GEMM; the norm and activation formulas are the cortiq dit.rs
 * page's rms_norm, silu and SwiGLU loop).
 *
 * add_rms_norm_quant_fp8, per row m (bf16 in, fp64 / fp32 as stated):
 *     r[k]  = bf16(x[m,k] + residual[m,k])     nearest-even; r = x when
 *             residual is NULL; otherwise r is written back into residual
 *     ms    = (sum_k r[k]^2) / K                fp64
 *     inv   = 1 / sqrt(ms + eps)                fp64
 *     h[k]  = bf16(fl32(fl32(r[k] * inv) * weight[k]))
 *     q[m,:], scale[m] = fp8_quant_rows of the row h
 *   x_bf16       [M, K] bf16, row stride ld_x elements
 *   residual     [M, K] bf16 in/out (updated in place), row stride ld_r
 *                elements, or NULL; must not overlap x, weight, q or scale
 *   weight_bf16  [K] bf16 norm weight
 *   eps          >= 0, finite
 *   q_e4m3, ld_q, scale: as fp8_quant_rows.
 *
 * silu_mul_quant_fp8, per row m:
 *     g = gate_up[m, k], u = gate_up[m, I + k]  (gate first, then up)
 *     a[k]  = bf16(fl32(fl32(g / (1 + exp(-g))) * u))   silu in fp64
 *     q[m,:], scale[m] = fp8_quant_rows of the row a
 *   gate_up_bf16 [M, 2I] bf16, row stride ld_gu elements (ld_gu >= 2I)
 *   q_e4m3 [M, I], scale [M] as fp8_quant_rows.
 *
 * Both: M >= 1; K (or I) >= 32, a multiple of 32 and at most 32768; the
 * alignment rules of fp8_quant_rows for every bf16 row stride. The sums of
 * squares are taken in fp64 in a different order than written above; the
 * rounding decisions that follow are the written ones unless a value lies
 * within about 1e-16 (relative) of a rounding boundary. NaN/Inf inputs are
 * not supported.
 */
int add_rms_norm_quant_fp8(const void *x_bf16, int64_t ld_x, void *residual_bf16, int64_t ld_r,
                           const void *weight_bf16, double eps, void *q_e4m3, int64_t ld_q,
                           float *scale, int64_t M, int64_t K, void *stream);

int silu_mul_quant_fp8(const void *gate_up_bf16, int64_t ld_gu, void *q_e4m3, int64_t ld_q,
                       float *scale, int64_t M, int64_t I, void *stream);

/*
 * Block-scaled e4m3 GEMM (y = x W^T form). The weight format is the mono
 * runner page's AttnWeights (an e4m3 [2048, 7168] projection weight with a
 * [64, 224] uint8 E8M0 grid: one scale byte per 32x32 block); the
 * computation is the exact dequantize-then-matmul that the sly-radiance
 * README's emulation path states, taking the per-token (q_fp8, scale) pair
 * of its fused producers; the bias and bias+GELU epilogues are the flash-rt
 * groot_n17 frontend's fused FP8 GEMM epilogue (module docstring,
 * _fused_epilogue_enabled):
 *     acc[m,n] = sum_kb 2^(w_scale[n/32][kb]-127) * sum_{k in block kb}
 *                e4m3(a[m,k]) * e4m3(w[n,k])               (fp32 accumulation)
 *     y[m,n]   = epilogue(a_scale[m] * acc[m,n] (+ bias[n]))   -> bf16, nearest-even
 *   a_e4m3   [M, K] uint8 e4m3fn, row stride ld_a bytes; a_scale [M] fp32
 *            (as produced by fp8_quant_rows)
 *   w_e4m3   [N, K] uint8 e4m3fn, row stride ld_w bytes
 *   w_scale  [N/32, K/32] uint8 E8M0, row-major, dense (row stride K/32)
 *   bias     [N] bf16, required iff epilogue != BS_EPI_NONE, else ignored
 *   y_bf16   [M, N] bf16 out, row stride ld_y elements
 *   M >= 1; N, K >= 32 and multiples of 32; ld_a, ld_w <= BS_MAX_LD_BYTES.
 *   workspace / workspace_bytes: scratch the call uses, at least
 *   bs_workspace_bytes(0, M, N, K) bytes, 16-byte aligned (may be NULL when
 *   that is 0); BS_EWORKSPACE if too small, BS_EALIGN if misaligned.
 */
int gemm_bs_fp8(const void *a_e4m3, int64_t ld_a, const float *a_scale,
                const void *w_e4m3, int64_t ld_w, const uint8_t *w_scale,
                const void *bias_bf16, int epilogue,
                void *y_bf16, int64_t ld_y,
                int64_t M, int64_t N, int64_t K,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * gemm_bs_fp8 for callers that cannot allocate: code under HIP graph capture
 * without a memory pool, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments and results as gemm_bs_fp8 without the
 * workspace: where gemm_bs_fp8 would use one (bs_workspace_bytes(0, M, N, K)
 * > 0: the split-K decode), its partial sums go to a scratch array the
 * library holds on each device (BS_NOALLOC_SCRATCH_BYTES bytes, kept until
 * the process ends). A shape that needs more returns BS_EWORKSPACE and
 * launches nothing. The call allocates and frees nothing. Every call on one
 * device shares that device's array, and its contents on entry do not
 * matter (every byte read is written first by the same call): calls that
 * overlap in time on one device (other streams, other threads) race on it
 * and must be serialized by the caller.
 */
#define BS_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int gemm_bs_fp8_noalloc(const void *a_e4m3, int64_t ld_a, const float *a_scale,
                        const void *w_e4m3, int64_t ld_w, const uint8_t *w_scale,
                        const void *bias_bf16, int epilogue,
                        void *y_bf16, int64_t ld_y,
                        int64_t M, int64_t N, int64_t K, void *stream);

/*
 * MXFP4-weight GEMM with e4m3 activations ("A8W4"): the sly-radiance
 * README's W4A8 kernels (its decode and prefill kernel rows: fp4 weights,
 * fp8 activations), on the mono runner page's MXFP4 layout
 * (MonoLayerWeights.check: fp4x2 weights [.., N, K/2] with uint8 E8M0
 * scales [N, K/32], one per row per 32 along K):
 *     w[n,k]   = e2m1(nibble k of row n) * 2^(w_scale[n][k/32]-127)
 *     y[m,n]   = epilogue(a_scale[m] * sum_k e4m3(a[m,k]) w[n,k] (+ bias[n]))
 *   w_fp4x2  [N, K/2] bytes, row stride ld_w bytes; element k of a row is in
 *            byte k/2, low nibble for even k, high nibble for odd k
 *   w_scale  [N, K/32] uint8 E8M0, row-major, dense (row stride K/32)
 *   Everything else as gemm_bs_fp8; workspace: bs_workspace_bytes(1, M, N, K).
 */
int gemm_mxfp4_w4a8(const void *a_e4m3, int64_t ld_a, const float *a_scale,
                    const void *w_fp4x2, int64_t ld_w, const uint8_t *w_scale,
                    const void *bias_bf16, int epilogue,
                    void *y_bf16, int64_t ld_y,
                    int64_t M, int64_t N, int64_t K,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * MXFP4 activations (W4A4, the sly-radiance README's base MXFP4 path that its
 * W4A8 kernel takes prefill shapes over from; the per-32 scale rule is OCP
 * MX's, the one the MXFP4 weights follow).
 *
 * fp4_quant_rows: per row m and 32-element block kb of x:
 *     scale[m,kb] = E8M0 byte of floor(log2(amax)) - 2, clamped to [0, 254]
 *                   (0 for an all-zero block)
 *     q[m,k]      = e2m1(x[m,k] / 2^(scale - 127)): nearest of
 *                   {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code,
 *                   saturating at 6, sign kept (also for zeros)
 *   x_bf16  [M, K] bf16, row stride ld_x elements
 *   q_fp4x2 [M, K/2] uint8 out (low nibble = even k), row stride ld_q bytes
 *   scale   [M, K/32] uint8 out, dense row-major
 *
 * gemm_mxfp4_w4a4:
 *     acc[m,n] = sum_kb 2^(sa[m,kb]-127) 2^(sw[n,kb]-127) sum_{k in kb} a[m,k] w[n,k]
 *     y[m,n]   = epilogue(acc (+ bias[n]))   -> bf16, nearest-even
 *   a_fp4x2 [M, K/2], row stride ld_a bytes; a_scale [M, K/32] E8M0 dense
 *   w_fp4x2 [N, K/2], w_scale [N, K/32] as gemm_mxfp4_w4a8
 *   M > 64 needs K % 64 == 0; workspace: bs_workspace_bytes(3, M, N, K)
 *   (nonzero for every M <= 64, where the small-M path may split K; wide
 *   layers with M <= 16 and 4-byte aligned scale rows do not use it).
 *   Other rules as gemm_bs_fp8.
 */
int fp4_quant_rows(const void *x_bf16, int64_t ld_x, void *q_fp4x2, int64_t ld_q,
                   uint8_t *scale, int64_t M, int64_t K, void *stream);

int gemm_mxfp4_w4a4(const void *a_fp4x2, int64_t ld_a, const uint8_t *a_scale,
                    const void *w_fp4x2, int64_t ld_w, const uint8_t *w_scale,
                    const void *bias_bf16, int epilogue,
                    void *y_bf16, int64_t ld_y,
                    int64_t M, int64_t N, int64_t K,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Grouped (MoE) W4A8 GEMM: many experts' MXFP4 weights in one launch over
 * expert-sorted token rows (mono runner page, MonoLayerWeights.check: the
 * routed experts' w13 [experts, 2 inter, hidden / 2] fp4x2 with uint8
 * scales [experts * 2 inter, hidden / 32]). For every expert e and token row
 * t in [expert_offsets[e], expert_offsets[e+1]):
 *     y[t,n] = epilogue(a_scale[t] * sum_kb 2^(S_e[n,kb]-127) sum_k a[t,k] W_e[n,k] (+ bias[e,n]))
 *   a_e4m3 [T, K], a_scale [T] fp32: the token rows, grouped by expert
 *   expert_offsets  DEVICE pointer to E + 1 int32, nondecreasing, from 0 to
 *                   at most T (read by the kernel; rows outside [0, T) are
 *                   never touched whatever they hold)
 *   max_rows_per_expert  an upper bound on any expert's rows: it picks the
 *                   kernel and its tiles (a wrong bound costs time, not
 *                   correctness)
 *   w_fp4x2  expert e's [N, K/2] at w + e * w_expert_stride bytes, row
 *            stride ld_w bytes; w_scale [E, N, K/32] E8M0 dense
 *   bias     [E, N] bf16 or NULL; y_bf16 [T, N], row stride ld_y
 *   E <= 65535. Rows of y outside every expert's range are not written.
 *   Up to 32 rows per expert (decode), each workgroup streams its 8 weight
 *   rows of one expert once per pass of up to 32 token rows. Past 32 (and
 *   K % 64 == 0), every expert is computed with the large-M tiles of the
 *   prefill GEMM (64x64 up to 64 rows, 128x128 up to 128, 160x256 up to
 *   160, 192x256 up to 192, else 256x256), experts side by side in one
 *   launch.
 */
int gemm_mxfp4_w4a8_grouped(const void *a_e4m3, int64_t ld_a, const float *a_scale,
                            const int32_t *expert_offsets, int64_t E,
                            int64_t max_rows_per_expert,
                            const void *w_fp4x2, int64_t ld_w, int64_t w_expert_stride,
                            const uint8_t *w_scale, const void *bias_bf16, int epilogue,
                            void *y_bf16, int64_t ld_y, int64_t T, int64_t N, int64_t K,
                            void *stream);

/*
 * Row-wise scaled e4m3 GEMM: one fp32 scale per token and one per output
 * channel (sly-radiance README, lm_head row of its file table: the head's
 * weight quantized to fp8 per output channel, computed as a row-wise scaled
 * GEMM with per-token fp8 activations):
 *     acc[m,n] = sum_k e4m3(a[m,k]) * e4m3(w[n,k])             (fp32 accumulation)
 *     y[m,n]   = epilogue(a_scale[m] * w_scale[n] * acc (+ bias[n]))  -> bf16
 *   w_scale  [N] fp32, 16-byte aligned
 *   Everything else as gemm_bs_fp8 (a per-tensor pair of scales is the case
 *   of constant a_scale and w_scale vectors); workspace:
 *   bs_workspace_bytes(2, M, N, K).
 */
int gemm_fp8_rowwise(const void *a_e4m3, int64_t ld_a, const float *a_scale,
                     const void *w_e4m3, int64_t ld_w, const float *w_scale,
                     const void *bias_bf16, int epilogue,
                     void *y_bf16, int64_t ld_y,
                     int64_t M, int64_t N, int64_t K,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes gemm_bs_fp8 (op 0), gemm_mxfp4_w4a8 (op 1), gemm_fp8_rowwise
 * (op 2) or gemm_mxfp4_w4a4 (op 3, every M <= 64) needs for this shape; 0
 * means none. Nonzero for
 * 8 < M <= 64, and for 2 <= M <= 8 when N * K >= 2^26, where K may be split
 * across workgroups with fp32 partial sums [S][M][N] in the workspace (S
 * depends only on N and K; from M = 9 to 16 on layers below 2^26 weights
 * the decode kernel leaves it unused). The workspace must then be 16-byte aligned;
 * its contents on entry do not matter (every byte read is written first by
 * the same call), so one buffer serves every call of a shape. Calls that
 * share a workspace must not overlap in time. */
size_t bs_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/* A static, human-readable string for a bs_status value. */
const char *bs_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BSGEMM_H */
