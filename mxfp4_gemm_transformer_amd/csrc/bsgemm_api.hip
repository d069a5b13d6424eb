// The C ABI of include/bsgemm.h: host-side argument checks, a once-per-device
// gfx950 gate, and dispatch to the kernels. Nothing here allocates or
// synchronizes. The checks mirror the mono runner page's _check_tensors
// (exact shapes and strides are validated because the kernels' loads are
// unbounded) and the flash-rt groot_n17 frontend's architecture gate (a
// mismatched device would compute garbage, so it is refused).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "bs_kernels.hpp"
#include "bsgemm.h"

namespace {

constexpr int MAX_DEVICES = 64;
// per device: 0 unknown, 1 gfx950, 2 refused; plus its CU count
std::atomic<int> g_arch_state[MAX_DEVICES];
std::atomic<int> g_num_cus[MAX_DEVICES];

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int device_check(int *num_cus) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return BS_EARCH;
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BS_EARCH;
        // gcnArchName is e.g. "gfx950:sramecc+:xnack-": compare the base target
        const char *name = prop.gcnArchName;
        const bool ok = std::strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':');
        g_num_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        st = ok ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_release);
    }
    *num_cus = g_num_cus[dev].load(std::memory_order_relaxed);
    return st == 1 ? BS_OK : BS_EARCH;
}

// Shared checks of the two GEMM entry points. `w_row_bytes` is the minimum
// row stride of W in bytes (K for e4m3, K/2 for fp4x2).
int check_gemm(const void *a, int64_t ld_a, const float *a_scale, const void *w, int64_t ld_w,
               int64_t w_row_bytes, const uint8_t *w_scale, const void *bias, int epilogue,
               const void *y, int64_t ld_y, int64_t M, int64_t N, int64_t K, size_t ws_bytes,
               size_t ws_need) {
    if (!a || !a_scale || !w || !w_scale || !y) return BS_EINVAL;
    if (M < 1 || N < 32 || K < 32 || N % 32 || K % 32) return BS_EINVAL;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return BS_EINVAL;
    if (epilogue < BS_EPI_NONE || epilogue > BS_EPI_BIAS_GELU_TANH) return BS_EINVAL;
    if (epilogue != BS_EPI_NONE && !bias) return BS_EINVAL;
    if (ld_a < K || ld_w < w_row_bytes || ld_y < N) return BS_EINVAL;
    // tile offsets (up to 256 rows of A or W plus K) are 32-bit buffer offsets
    if (ld_a > BS_MAX_LD_BYTES || ld_w > BS_MAX_LD_BYTES) return BS_EINVAL;
    if (!aligned16(a) || !aligned16(w) || !aligned16(y)) return BS_EALIGN;
    if (ld_a % 16 || ld_w % 16 || (2 * ld_y) % 16) return BS_EALIGN;
    if ((reinterpret_cast<uintptr_t>(a_scale) & 3u) != 0) return BS_EALIGN;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 1u) != 0) return BS_EALIGN;
    if (ws_bytes < ws_need) return BS_EWORKSPACE;
    return BS_OK;
}

// `w_scale` is the E8M0 grid; `chan_scale` (e4m3 weights only) replaces it
// with one fp32 scale per output channel when not NULL.
int gemm_common(bool fp4, const void *a_e4m3, int64_t ld_a, const float *a_scale, const void *w,
                int64_t ld_w, const uint8_t *w_scale, const float *chan_scale,
                const void *bias_bf16, int epilogue, void *y_bf16, int64_t ld_y, int64_t M,
                int64_t N, int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
    const int64_t w_row = fp4 ? K / 2 : K;
    const size_t ws_need = bs_workspace_bytes(fp4 ? 1 : 0, M, N, K);
    int st = check_gemm(a_e4m3, ld_a, a_scale, w, ld_w, w_row,
                        chan_scale ? reinterpret_cast<const uint8_t *>(chan_scale) : w_scale,
                        bias_bf16, epilogue, y_bf16, ld_y, M, N, K, workspace_bytes, ws_need);
    if (st != BS_OK) return st;
    if (chan_scale && !aligned16(chan_scale)) return BS_EALIGN;
    if (chan_scale) w_scale = nullptr;
    if (ws_need && (!workspace || !aligned16(workspace)))
        return workspace ? BS_EALIGN : BS_EWORKSPACE;
    int num_cus = 0;
    if ((st = device_check(&num_cus)) != BS_OK) return st;
    const auto *a = static_cast<const uint8_t *>(a_e4m3);
    const auto *wb = static_cast<const uint8_t *>(w);
    const auto *bias = static_cast<const uint16_t *>(bias_bf16);
    auto *y = static_cast<uint16_t *>(y_bf16);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (M <= bsg::DECODE_MAX_M)
        e = bsg::launch_gemm_decode(fp4, a, ld_a, a_scale, wb, ld_w, w_scale, chan_scale, bias,
                                    epilogue, y, ld_y, M, N, K, workspace, num_cus, s);
    else
        e = bsg::launch_gemm_prefill(fp4, a, ld_a, a_scale, wb, ld_w, w_scale, chan_scale, bias,
                                     epilogue, y, ld_y, M, N, K, num_cus, s);
    return e == hipSuccess ? BS_OK : BS_ELAUNCH;
}

// Scratch of gemm_bs_fp8_noalloc: the split-K partial sums of a call that
// would otherwise take them from a workspace argument. One copy per device,
// held until the process ends. In host code `scratch` names a host-side
// stand-in, never the device array: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) uint8_t scratch[BS_NOALLOC_SCRATCH_BYTES];

std::atomic<void *> g_scratch_ptr[MAX_DEVICES];

// The calling thread's current device's scratch address, looked up on the
// first call on that device (with that device current).
int scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return BS_EARCH;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BS_ELAUNCH;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return BS_OK;
}

}  // namespace

extern "C" {

int fp8_quant_rows(const void *x_bf16, int64_t ld_x, void *q_e4m3, int64_t ld_q, float *scale,
                   int64_t M, int64_t K, void *stream) {
    if (!x_bf16 || !q_e4m3 || !scale) return BS_EINVAL;
    if (M < 1 || K < 32 || K % 32 || M > INT32_MAX || K > INT32_MAX) return BS_EINVAL;
    if (ld_x < K || ld_q < K) return BS_EINVAL;
    if (!aligned16(x_bf16) || !aligned16(q_e4m3) || (2 * ld_x) % 16 || ld_q % 16)
        return BS_EALIGN;
    if ((reinterpret_cast<uintptr_t>(scale) & 3u) != 0) return BS_EALIGN;
    int num_cus = 0;
    int st = device_check(&num_cus);
    if (st != BS_OK) return st;
    hipError_t e = bsg::launch_quant_rows(static_cast<const uint16_t *>(x_bf16), ld_x,
                                          static_cast<uint8_t *>(q_e4m3), ld_q, scale, M, K,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BS_OK : BS_ELAUNCH;
}

int add_rms_norm_quant_fp8(const void *x_bf16, int64_t ld_x, void *residual_bf16, int64_t ld_r,
                           const void *weight_bf16, double eps, void *q_e4m3, int64_t ld_q,
                           float *scale, int64_t M, int64_t K, void *stream) {
    if (!x_bf16 || !weight_bf16 || !q_e4m3 || !scale) return BS_EINVAL;
    if (M < 1 || K < 32 || K % 32 || M > INT32_MAX || K > bsg::PRODUCER_MAX_K) return BS_EINVAL;
    if (ld_x < K || ld_q < K || (residual_bf16 && ld_r < K)) return BS_EINVAL;
    if (!(eps >= 0.0) || eps > 1e300) return BS_EINVAL;
    if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned16(weight_bf16) || (2 * ld_x) % 16 ||
        ld_q % 16)
        return BS_EALIGN;
    if (residual_bf16 && (!aligned16(residual_bf16) || (2 * ld_r) % 16)) return BS_EALIGN;
    if ((reinterpret_cast<uintptr_t>(scale) & 3u) != 0) return BS_EALIGN;
    int num_cus = 0;
    int st = device_check(&num_cus);
    if (st != BS_OK) return st;
    hipError_t e = bsg::launch_add_rms_quant(
        static_cast<const uint16_t *>(x_bf16), ld_x, static_cast<uint16_t *>(residual_bf16), ld_r,
        static_cast<const uint16_t *>(weight_bf16), eps, static_cast<uint8_t *>(q_e4m3), ld_q,
        scale, M, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BS_OK : BS_ELAUNCH;
}

int silu_mul_quant_fp8(const void *gate_up_bf16, int64_t ld_gu, void *q_e4m3, int64_t ld_q,
                       float *scale, int64_t M, int64_t I, void *stream) {
    if (!gate_up_bf16 || !q_e4m3 || !scale) return BS_EINVAL;
    if (M < 1 || I < 32 || I % 32 || M > INT32_MAX || I > bsg::PRODUCER_MAX_K) return BS_EINVAL;
    if (ld_gu < 2 * I || ld_q < I) return BS_EINVAL;
    if (!aligned16(gate_up_bf16) || !aligned16(q_e4m3) || (2 * ld_gu) % 16 || ld_q % 16)
        return BS_EALIGN;
    if ((reinterpret_cast<uintptr_t>(scale) & 3u) != 0) return BS_EALIGN;
    int num_cus = 0;
    int st = device_check(&num_cus);
    if (st != BS_OK) return st;
    hipError_t e = bsg::launch_silu_mul_quant(static_cast<const uint16_t *>(gate_up_bf16), ld_gu,
                                              static_cast<uint8_t *>(q_e4m3), ld_q, scale, M, I,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BS_OK : BS_ELAUNCH;
}

int gemm_bs_fp8(const void *a_e4m3, int64_t ld_a, const float *a_scale, const void *w_e4m3,
                int64_t ld_w, const uint8_t *w_scale, const void *bias_bf16, int epilogue,
                void *y_bf16, int64_t ld_y, int64_t M, int64_t N, int64_t K, void *workspace,
                size_t workspace_bytes, void *stream) {
    return gemm_common(false, a_e4m3, ld_a, a_scale, w_e4m3, ld_w, w_scale, nullptr, bias_bf16,
                       epilogue, y_bf16, ld_y, M, N, K, workspace, workspace_bytes, stream);
}

int gemm_bs_fp8_noalloc(const void *a_e4m3, int64_t ld_a, const float *a_scale,
                        const void *w_e4m3, int64_t ld_w, const uint8_t *w_scale,
                        const void *bias_bf16, int epilogue, void *y_bf16, int64_t ld_y,
                        int64_t M, int64_t N, int64_t K, void *stream) {
    if (M < 1 || N < 1 || K < 1) return BS_EINVAL;
    const size_t need = bs_workspace_bytes(0, M, N, K);
    if (need > BS_NOALLOC_SCRATCH_BYTES) return BS_EWORKSPACE;
    void *ws = nullptr;
    if (need) {
        // the device check first: the symbol lookup needs a usable device
        int num_cus = 0;
        int st = device_check(&num_cus);
        if (st != BS_OK) return st;
        if ((st = scratch_address(&ws)) != BS_OK) return st;
    }
    return gemm_common(false, a_e4m3, ld_a, a_scale, w_e4m3, ld_w, w_scale, nullptr, bias_bf16,
                       epilogue, y_bf16, ld_y, M, N, K, ws, need ? BS_NOALLOC_SCRATCH_BYTES : 0,
                       stream);
}

int gemm_mxfp4_w4a8(const void *a_e4m3, int64_t ld_a, const float *a_scale, const void *w_fp4x2,
                    int64_t ld_w, const uint8_t *w_scale, const void *bias_bf16, int epilogue,
                    void *y_bf16, int64_t ld_y, int64_t M, int64_t N, int64_t K, void *workspace,
                    size_t workspace_bytes, void *stream) {
    return gemm_common(true, a_e4m3, ld_a, a_scale, w_fp4x2, ld_w, w_scale, nullptr, bias_bf16,
                       epilogue, y_bf16, ld_y, M, N, K, workspace, workspace_bytes, stream);
}

int gemm_fp8_rowwise(const void *a_e4m3, int64_t ld_a, const float *a_scale, const void *w_e4m3,
                     int64_t ld_w, const float *w_scale, const void *bias_bf16, int epilogue,
                     void *y_bf16, int64_t ld_y, int64_t M, int64_t N, int64_t K, void *workspace,
                     size_t workspace_bytes, void *stream) {
    if (!w_scale) return BS_EINVAL;
    return gemm_common(false, a_e4m3, ld_a, a_scale, w_e4m3, ld_w, nullptr, w_scale, bias_bf16,
                       epilogue, y_bf16, ld_y, M, N, K, workspace, workspace_bytes, stream);
}

int fp8_quant_rows_static(const void *x_bf16, int64_t ld_x, const float *scale_in, void *q_e4m3,
                          int64_t ld_q, float *scale_out, int64_t M, int64_t K, void *stream) {
    if (!x_bf16 || !q_e4m3 || !scale_in) return BS_EINVAL;
    if (M < 1 || K < 32 || K % 32 || M > INT32_MAX || K > INT32_MAX) return BS_EINVAL;
    if (ld_x < K || ld_q < K) return BS_EINVAL;
    if (!aligned16(x_bf16) || !aligned16(q_e4m3) || (2 * ld_x) % 16 || ld_q % 16)
        return BS_EALIGN;
    if ((reinterpret_cast<uintptr_t>(scale_in) & 3u) != 0) return BS_EALIGN;
    if (scale_out && (reinterpret_cast<uintptr_t>(scale_out) & 3u) != 0) return BS_EALIGN;
    int num_cus = 0;
    int st = device_check(&num_cus);
    if (st != BS_OK) return st;
    hipError_t e = bsg::launch_quant_rows_static(static_cast<const uint16_t *>(x_bf16), ld_x,
                                                 scale_in, static_cast<uint8_t *>(q_e4m3), ld_q,
                                                 scale_out, M, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BS_OK : BS_ELAUNCH;
}

int fp4_quant_rows(const void *x_bf16, int64_t ld_x, void *q_fp4x2, int64_t ld_q, uint8_t *scale,
                   int64_t M, int64_t K, void *stream) {
    if (!x_bf16 || !q_fp4x2 || !scale) return BS_EINVAL;
    if (M < 1 || K < 32 || K % 32 || M > INT32_MAX || K > INT32_MAX) return BS_EINVAL;
    if (ld_x < K || ld_q < K / 2) return BS_EINVAL;
    if (!aligned16(x_bf16) || !aligned16(q_fp4x2) || (2 * ld_x) % 16 || ld_q % 16)
        return BS_EALIGN;
    int num_cus = 0;
    int st = device_check(&num_cus);
    if (st != BS_OK) return st;
    hipError_t e = bsg::launch_quant_mxfp4_rows(static_cast<const uint16_t *>(x_bf16), ld_x,
                                                static_cast<uint8_t *>(q_fp4x2), ld_q, scale, M, K,
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BS_OK : BS_ELAUNCH;
}

int gemm_mxfp4_w4a4(const void *a_fp4x2, int64_t ld_a, const uint8_t *a_scale, const void *w_fp4x2,
                    int64_t ld_w, const uint8_t *w_scale, const void *bias_bf16, int epilogue,
                    void *y_bf16, int64_t ld_y, int64_t M, int64_t N, int64_t K, void *workspace,
                    size_t workspace_bytes, void *stream) {
    if (!a_fp4x2 || !a_scale || !w_fp4x2 || !w_scale || !y_bf16) return BS_EINVAL;
    if (M < 1 || N < 32 || K < 32 || N % 32 || K % 32) return BS_EINVAL;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return BS_EINVAL;
    if (M > bsg::DECODE_MAX_M && K % 64) return BS_EINVAL;   // the prefill kernel takes whole 64-k steps
    if (epilogue < BS_EPI_NONE || epilogue > BS_EPI_BIAS_GELU_TANH) return BS_EINVAL;
    if (epilogue != BS_EPI_NONE && !bias_bf16) return BS_EINVAL;
    if (ld_a < K / 2 || ld_w < K / 2 || ld_y < N) return BS_EINVAL;
    if (ld_a > BS_MAX_LD_BYTES || ld_w > BS_MAX_LD_BYTES) return BS_EINVAL;
    if (!aligned16(a_fp4x2) || !aligned16(w_fp4x2) || !aligned16(y_bf16)) return BS_EALIGN;
    if (ld_a % 16 || ld_w % 16 || (2 * ld_y) % 16) return BS_EALIGN;
    if (bias_bf16 && (reinterpret_cast<uintptr_t>(bias_bf16) & 1u) != 0) return BS_EALIGN;
    const size_t ws_need = bs_workspace_bytes(3, M, N, K);
    if (workspace_bytes < ws_need) return BS_EWORKSPACE;
    if (ws_need && (!workspace || !aligned16(workspace))) return workspace ? BS_EALIGN : BS_EWORKSPACE;
    int num_cus = 0;
    int st = device_check(&num_cus);
    if (st != BS_OK) return st;
    const auto *a = static_cast<const uint8_t *>(a_fp4x2);
    const auto *w = static_cast<const uint8_t *>(w_fp4x2);
    const auto *bias = static_cast<const uint16_t *>(bias_bf16);
    auto *y = static_cast<uint16_t *>(y_bf16);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (M <= bsg::DECODE_MAX_M)
        e = bsg::launch_gemm_decode_w4a4(a, ld_a, a_scale, w, ld_w, w_scale, bias, epilogue, y,
                                         ld_y, M, N, K, workspace, num_cus, s);
    else
        e = bsg::launch_gemm_prefill_w4a4(a, ld_a, a_scale, w, ld_w, w_scale, bias, epilogue, y,
                                          ld_y, M, N, K, num_cus, s);
    return e == hipSuccess ? BS_OK : BS_ELAUNCH;
}

int gemm_mxfp4_w4a8_grouped(const void *a_e4m3, int64_t ld_a, const float *a_scale,
                            const int32_t *expert_offsets, int64_t E, int64_t max_rows_per_expert,
                            const void *w_fp4x2, int64_t ld_w, int64_t w_expert_stride,
                            const uint8_t *w_scale, const void *bias_bf16, int epilogue,
                            void *y_bf16, int64_t ld_y, int64_t T, int64_t N, int64_t K,
                            void *stream) {
    if (!a_e4m3 || !a_scale || !expert_offsets || !w_fp4x2 || !w_scale || !y_bf16) return BS_EINVAL;
    if (T < 1 || E < 1 || E > 65535 || N < 32 || K < 32 || N % 32 || K % 32) return BS_EINVAL;
    if (T > INT32_MAX || N > INT32_MAX || K > INT32_MAX || max_rows_per_expert < 1) return BS_EINVAL;
    if (epilogue < BS_EPI_NONE || epilogue > BS_EPI_BIAS_GELU_TANH) return BS_EINVAL;
    if (epilogue != BS_EPI_NONE && !bias_bf16) return BS_EINVAL;
    if (ld_a < K || ld_w < K / 2 || ld_y < N || w_expert_stride < N * ld_w) return BS_EINVAL;
    if (!aligned16(a_e4m3) || !aligned16(w_fp4x2) || !aligned16(y_bf16)) return BS_EALIGN;
    if (ld_a % 16 || ld_w % 16 || (2 * ld_y) % 16 || w_expert_stride % 16) return BS_EALIGN;
    if ((reinterpret_cast<uintptr_t>(a_scale) & 3u) || (reinterpret_cast<uintptr_t>(expert_offsets) & 3u))
        return BS_EALIGN;
    if (bias_bf16 && (reinterpret_cast<uintptr_t>(bias_bf16) & 1u) != 0) return BS_EALIGN;
    int num_cus = 0;
    int st = device_check(&num_cus);
    if (st != BS_OK) return st;
    hipError_t e = bsg::launch_gemm_grouped(
        true, static_cast<const uint8_t *>(a_e4m3), ld_a, a_scale, expert_offsets, E,
        max_rows_per_expert, static_cast<const uint8_t *>(w_fp4x2), ld_w, w_expert_stride, w_scale,
        static_cast<const uint16_t *>(bias_bf16), epilogue, static_cast<uint16_t *>(y_bf16), ld_y,
        T, N, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BS_OK : BS_ELAUNCH;
}

size_t bs_workspace_bytes(int op, int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || K < 1) return 0;
    if (op == 3) return bsg::decode_workspace_bytes_w4a4(M, N, K);   // W4A4: split-K decode
    return bsg::decode_workspace_bytes(M, N, K);   // split-K decode partial sums, else 0
}

const char *bs_status_string(int status) {
    switch (status) {
    case BS_OK: return "ok";
    case BS_EINVAL: return "invalid argument (size, leading dimension, epilogue or null pointer)";
    case BS_EALIGN: return "pointer or leading dimension not aligned as required";
    case BS_EARCH: return "no HIP device, or the current device is not gfx950";
    case BS_EWORKSPACE: return "workspace smaller than bs_workspace_bytes()";
    case BS_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

}  // extern "C"
