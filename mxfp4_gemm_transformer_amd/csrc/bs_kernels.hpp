// Host-side launchers of the gfx950 kernels. Arguments are validated by the
// C-ABI layer before these are called; each returns a hipError_t from
// hipGetLastError() after its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

hipError_t launch_quant_rows(const uint16_t *x, int64_t ld_x, uint8_t *q, int64_t ld_q,
                             float *scale, int64_t M, int64_t K, hipStream_t stream);

// Quantization with one given scale (device scalar); scale_out [M] may be NULL.
// MXFP4 (OCP MX) quantization of bf16 rows: packed [M, K/2], E8M0 [M, K/32].
hipError_t launch_quant_mxfp4_rows(const uint16_t *x, int64_t ld_x, uint8_t *q, int64_t ld_q,
                                   uint8_t *scale, int64_t M, int64_t K, hipStream_t stream);

hipError_t launch_quant_rows_static(const uint16_t *x, int64_t ld_x, const float *scale_in,
                                    uint8_t *q, int64_t ld_q, float *scale_out, int64_t M,
                                    int64_t K, hipStream_t stream);

// Fused producers (row width at most PRODUCER_MAX_K): RMSNorm with an
// optional in-place residual add, or SiLU(gate) * up, then the quantizer.
constexpr int64_t PRODUCER_MAX_K = 32768;
hipError_t launch_add_rms_quant(const uint16_t *x, int64_t ld_x, uint16_t *residual, int64_t ld_r,
                                const uint16_t *weight, double eps, uint8_t *q, int64_t ld_q,
                                float *scale, int64_t M, int64_t K, hipStream_t stream);
hipError_t launch_silu_mul_quant(const uint16_t *gate_up, int64_t ld_gu, uint8_t *q, int64_t ld_q,
                                 float *scale, int64_t M, int64_t I, hipStream_t stream);

// M <= DECODE_MAX_M: the bandwidth-bound small-M GEMM.
constexpr int64_t DECODE_MAX_M = 64;

// `ws` is the E8M0 grid, or NULL for e4m3 weights with one fp32 scale per
// output channel in `cs` (NULL otherwise): Y = s[m] cs[n] sum_k a w.
// `workspace` holds decode_workspace_bytes(M, N, K) bytes (fp32 partial sums
// of the split-K path, sized for 8 < M <= 64), 16-byte aligned; unused
// otherwise.
hipError_t launch_gemm_decode(bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                              const uint8_t *w, int64_t ldw, const uint8_t *ws, const float *cs,
                              const uint16_t *bias, int epi, uint16_t *y, int64_t ldy, int64_t M,
                              int64_t N, int64_t K, void *workspace, int num_cus,
                              hipStream_t stream);
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K);

hipError_t launch_gemm_prefill(bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                               const uint8_t *w, int64_t ldw, const uint8_t *ws, const float *cs,
                               const uint16_t *bias, int epi, uint16_t *y, int64_t ldy, int64_t M,
                               int64_t N, int64_t K, int num_cus, hipStream_t stream);

// W4A4 (fp4 activations [M, K/2] with E8M0 scales [M, K/32], MXFP4
// weights). Decode: M <= DECODE_MAX_M, split-K through the workspace
// (decode_workspace_bytes_w4a4 bytes). Prefill: M > DECODE_MAX_M,
// K % 64 == 0.
hipError_t launch_gemm_decode_w4a4(const uint8_t *a, int64_t lda, const uint8_t *a_e8m0,
                                   const uint8_t *w, int64_t ldw, const uint8_t *ws,
                                   const uint16_t *bias, int epi, uint16_t *y, int64_t ldy,
                                   int64_t M, int64_t N, int64_t K, void *workspace,
                                   int num_cus, hipStream_t stream);
size_t decode_workspace_bytes_w4a4(int64_t M, int64_t N, int64_t K);

// Grouped (MoE) GEMM over expert-sorted rows: offsets [E + 1] on the device,
// expert e's weights at w + e * w_estride ([N, K/2] fp4x2 or [N, K] e4m3)
// with scales [E, N, K/32] (fp4) or [E, N/32, K/32] (e4m3), bias [E, N].
// max_rows bounds the rows of any expert (it picks the tokens per pass).
hipError_t launch_gemm_grouped(bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                               const int32_t *offsets, int64_t E, int64_t max_rows,
                               const uint8_t *w, int64_t ldw, int64_t w_estride,
                               const uint8_t *ws, const uint16_t *bias, int epi, uint16_t *y,
                               int64_t ldy, int64_t T, int64_t N, int64_t K, hipStream_t stream);
// Its prefill-sized form (the large-M tiles per expert), MXFP4 weights only;
// launch_gemm_grouped takes it when max_rows > GROUPED_DECODE_MAX_ROWS and
// K % 64 == 0.
constexpr int64_t GROUPED_DECODE_MAX_ROWS = 32;
hipError_t launch_gemm_grouped_prefill(const uint8_t *a, int64_t lda, const float *a_scale,
                                       const int32_t *offsets, int64_t E, int64_t max_rows,
                                       const uint8_t *w, int64_t ldw, int64_t w_estride,
                                       const uint8_t *ws, const uint16_t *bias, int epi, uint16_t *y,
                                       int64_t ldy, int64_t T, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_gemm_prefill_w4a4(const uint8_t *a, int64_t lda, const uint8_t *a_e8m0,
                                    const uint8_t *w, int64_t ldw, const uint8_t *ws,
                                    const uint16_t *bias, int epi, uint16_t *y, int64_t ldy,
                                    int64_t M, int64_t N, int64_t K, int num_cus,
                                    hipStream_t stream);

}  // namespace bsg
