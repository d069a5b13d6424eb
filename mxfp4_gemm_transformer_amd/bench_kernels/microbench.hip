// Microbenchmarks that set the ceilings the layer's kernels are measured
// against on gfx950. They are not part of the layer: bench.py loads them
// from libbsbench.so, a library of their own, to time
//   - a plain streaming read of a buffer (the best an HBM-bound kernel of
//     that size can do in one launch),
//   - an empty kernel (the fixed cost of one launch in a graph), and
//   - back-to-back scaled MFMAs with register operands, per operand-format
//     pair (the matrix-core rate each GEMM variant can reach).
// Every entry point launches asynchronously on `stream` and returns a
// hipError_t value (0 on success).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Reads [p, p + bytes) once, 16 bytes per lane per load, `unroll` loads in
// flight per lane; each workgroup covers contiguous chunks of
// 16 * 256 * unroll bytes, grid-strided. The loaded words are folded into an
// xor that is stored only if it equals a value the data never produces
// (the buffers hold repeated non-zero bytes), so no load is dead code and
// nothing is written.
// With `shared` (s16 chunks of 16 bytes): every workgroup also reads all of
// it, as each workgroup of a decode GEMM without a split K reads every
// token's activations once.
template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                          uint32_t *__restrict__ sink,
                                                          const u32x4 *__restrict__ shared = nullptr,
                                                          int64_t s16 = 0) {
    uint32_t acc = 0;
    for (int64_t i = threadIdx.x; i < s16; i += 256) {
        const u32x4 v = shared[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    const int64_t chunk = 256 * UNROLL;
    for (int64_t base = (int64_t)blockIdx.x * chunk; base < n16; base += (int64_t)gridDim.x * chunk) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0xDEADBEEFu) sink[blockIdx.x & 255] = acc;
}

__global__ void empty_kernel() {}

// Per-CU read rate from L2: every workgroup reads its own `chunk`-byte
// region (all regions together fit the XCDs' L2) `iters` times, 16 bytes a
// lane, 8 loads in flight per wave, either into registers (DMA = false) or
// with LDS-mode buffer loads straight into a 64 KiB LDS ring (DMA = true:
// lane l's 16 bytes land at M0 + 16 l).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t m0, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <bool DMA>
__global__ __launch_bounds__(256) void l2_read_kernel(const uint8_t *__restrict__ p, int chunk, int iters,
                                                      uint32_t *__restrict__ sink) {
    __shared__ __align__(16) uint8_t lds[65536];
    const uint8_t *base = p + (int64_t)blockIdx.x * chunk;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(base), (short)0, chunk, 0x00020000);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t *)lds);
    const int per = chunk / 4096;                  // 4 KiB per round of the 4 waves
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
        for (int j0 = 0; j0 < per; j0 += 8) {
            if (DMA) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = j0 + u;
                    const uint32_t off = (uint32_t)(j * 4096 + threadIdx.x * 16);
                    const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane(
                        lds0 + (uint32_t)((j * 4096 + wave * 1024) & 65535));
                    dma16(rs, m0, j < per ? off : 0x80000000u);
                }
                asm volatile("s_waitcnt vmcnt(8)" : : : "memory");
            } else {
                uint32_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = j0 + u;
                    const auto q = __builtin_amdgcn_raw_buffer_load_b128(
                        rs, j < per ? (uint32_t)(j * 4096 + threadIdx.x * 16) : 0x80000000u, 0, 0);
                    v[u] = q[0] ^ q[1] ^ q[2] ^ q[3];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) acc ^= v[u];
            }
        }
    }
    if (DMA) {
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
        __syncthreads();
        acc = reinterpret_cast<const uint32_t *>(lds)[threadIdx.x];
    }
    if (acc == 0xDEADBEEFu) sink[blockIdx.x & 255] = acc;
}

// `iters` rounds of 4 independent scaled MFMAs per wave (4 accumulators
// hide the instruction's dependent-issue latency); operands stay in
// registers. Formats per the instruction's cbsz / blgp encoding: 0 = fp8
// e4m3, 4 = fp4 e2m1.
// RND: operands of pseudo-random bits (fp8 codes with the top exponent bit
// cleared, so none is NaN) instead of a fixed pattern of small values.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
    return x;
}

template <int FA, int FB, bool BIG, bool RND>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float *__restrict__ sink) {
    v8i a, b;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (RND) {
            const uint32_t t = (blockIdx.x * 256u + threadIdx.x) * 16u + (uint32_t)r;
            a[r] = (int)(mix32(t) & (FA == 0 ? 0xBFBFBFBFu : 0xFFFFFFFFu));
            b[r] = (int)(mix32(t + 8u) & (FB == 0 ? 0xBFBFBFBFu : 0xFFFFFFFFu));
        } else {
            a[r] = (int)(0x38383838u + threadIdx.x + r);
            b[r] = (int)(0x22222222u + threadIdx.x * 3 + r);
        }
    }
    if (BIG) {
        v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, FA, FB, 0, 127, 0, 127);
            c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, FA, FB, 0, 127, 0, 127);
            c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, FA, FB, 0, 127, 0, 127);
            c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, FA, FB, 0, 127, 0, 127);
        }
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
        if (s == 1234.5f) sink[threadIdx.x] = s;
    } else {
        v4f c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, FA, FB, 0, 127, 0, 127);
            c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c1, FA, FB, 0, 127, 0, 127);
            c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c2, FA, FB, 0, 127, 0, 127);
            c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c3, FA, FB, 0, 127, 0, 127);
        }
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
        if (s == 1234.5f) sink[threadIdx.x] = s;
    }
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16) at the 16-byte-aligned
// device address `p` on `blocks` workgroups of 256 threads with `unroll`
// (1, 2, 4, 8 or 16) loads in flight per lane. `sink` is 1 KiB of device
// memory that is never written in practice.
int bsb_stream_read(const void *p, int64_t bytes, void *sink, int blocks, int unroll, void *stream) {
    if (!p || !sink || bytes <= 0 || bytes % 16 || blocks < 1) return (int)hipErrorInvalidValue;
    const auto *q = static_cast<const u32x4 *>(p);
    auto *s = static_cast<uint32_t *>(sink);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n16 = bytes / 16;
    switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(256), 0, st, q, n16, s); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(256), 0, st, q, n16, s); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, st, q, n16, s); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, st, q, n16, s); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(blocks), dim3(256), 0, st, q, n16, s); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// As bsb_stream_read, with every workgroup also reading all `shared_bytes`
// (a multiple of 16) at the 16-byte-aligned device address `shared`.
int bsb_stream_read_shared(const void *p, int64_t bytes, const void *shared, int64_t shared_bytes,
                           void *sink, int blocks, int unroll, void *stream) {
    if (!p || !shared || !sink || bytes <= 0 || bytes % 16 || shared_bytes <= 0 || shared_bytes % 16 ||
        blocks < 1)
        return (int)hipErrorInvalidValue;
    const auto *q = static_cast<const u32x4 *>(p);
    const auto *sh = static_cast<const u32x4 *>(shared);
    auto *s = static_cast<uint32_t *>(sink);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n16 = bytes / 16, s16 = shared_bytes / 16;
    switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(256), 0, st, q, n16, s, sh, s16); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(256), 0, st, q, n16, s, sh, s16); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, st, q, n16, s, sh, s16); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, st, q, n16, s, sh, s16); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(blocks), dim3(256), 0, st, q, n16, s, sh, s16); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// `blocks` workgroups of 256 threads each read their own `chunk` bytes
// (a multiple of 32 KiB, at most 1 MiB) of the device buffer p (at least
// blocks * chunk bytes) `iters` times: into registers (dma = 0) or into LDS
// with LDS-mode loads (dma = 1). `sink`: 1 KiB, never written in practice.
int bsb_l2_read(const void *p, int chunk, int iters, int blocks, int dma, void *sink, void *stream) {
    if (!p || !sink || chunk <= 0 || chunk % 32768 || chunk > (1 << 20) || iters < 1 || blocks < 1)
        return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const auto *q = static_cast<const uint8_t *>(p);
    auto *s = static_cast<uint32_t *>(sink);
    if (dma) hipLaunchKernelGGL(l2_read_kernel<true>, dim3(blocks), dim3(256), 0, st, q, chunk, iters, s);
    else hipLaunchKernelGGL(l2_read_kernel<false>, dim3(blocks), dim3(256), 0, st, q, chunk, iters, s);
    return (int)hipGetLastError();
}

// One launch of a kernel with no body, `blocks` workgroups of 64 threads.
int bsb_empty(int blocks, void *stream) {
    if (blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(64), 0, static_cast<hipStream_t>(stream));
    return (int)hipGetLastError();
}

// `blocks` workgroups of `waves` (1..4) waves, each wave issuing 4 * iters
// scaled MFMAs on fixed-pattern operands, or on pseudo-random bits when
// random_bits != 0: shape 0 = 16x16x128, 1 = 32x32x64; formats (fa, fb) in
// {(0,0) fp8 x fp8, (0,4) fp8 x fp4, (4,0) fp4 x fp8, (4,4) fp4 x fp4}.
// FLOPs = blocks * waves * 4 * iters * (2 * 16 * 16 * 128, or 2 * 32 * 32 * 64).
// `sink` is 1 KiB of device memory that is never written in practice.
int bsb_mfma_rate(int shape, int fa, int fb, int iters, int blocks, int waves, int random_bits,
                  void *sink, void *stream) {
    if (!sink || iters < 1 || blocks < 1 || waves < 1 || waves > 4) return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    float *s = static_cast<float *>(sink);
    const dim3 grid(blocks), block(64 * waves);
#define BSB_MFMA(FA, FB)                                                                          \
    if (fa == FA && fb == FB) {                                                                   \
        if (shape && random_bits) hipLaunchKernelGGL((mfma_rate_kernel<FA, FB, true, true>), grid, block, 0, st, iters, s); \
        else if (shape) hipLaunchKernelGGL((mfma_rate_kernel<FA, FB, true, false>), grid, block, 0, st, iters, s); \
        else if (random_bits) hipLaunchKernelGGL((mfma_rate_kernel<FA, FB, false, true>), grid, block, 0, st, iters, s); \
        else hipLaunchKernelGGL((mfma_rate_kernel<FA, FB, false, false>), grid, block, 0, st, iters, s); \
        return (int)hipGetLastError();                                                            \
    }
    BSB_MFMA(0, 0)
    BSB_MFMA(0, 4)
    BSB_MFMA(4, 0)
    BSB_MFMA(4, 4)
#undef BSB_MFMA
    return (int)hipErrorInvalidValue;
}

// The current device's compute-unit count and peak engine and memory clocks
// (kHz) and memory bus width (bits), as the runtime reports them: the inputs
// of a peak derived on the box itself.
int bsb_device_info(int *cus, int *sclk_khz, int *mclk_khz, int *bus_bits) {
    if (!cus || !sclk_khz || !mclk_khz || !bus_bits) return (int)hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(sclk_khz, hipDeviceAttributeClockRate, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(mclk_khz, hipDeviceAttributeMemoryClockRate, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(bus_bits, hipDeviceAttributeMemoryBusWidth, dev);
    return (int)e;
}

}  // extern "C"
