// Per-token activation quantization to e4m3fn: one fp32 scale per row
// (amax / 448) and the row's codes, in one HBM pass over the bf16 input.
// The "(q_fp8, scale)" pair is what the sly-radiance README's fused
// producers hand to its W4A8 GEMM (fused norm/quant rows of its file table).
#include "bs_device.hpp"
#include "bs_kernels.hpp"

namespace bsg {
namespace {

constexpr int QBLOCK = 256;

// Largest |bf16| of the 8 values in a 16-byte chunk, as a magnitude bit
// pattern (for finite values, integer order of exp|mantissa = value order).
__device__ __forceinline__ uint32_t absmax8(const uint4 &c) {
    uint32_t m = 0;
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = max(m, w[i] & 0x7FFFu);
        m = max(m, (w[i] >> 16) & 0x7FFFu);
    }
    return m;
}

// The e4m3 codes of fl32(x / s) for the 8 bf16 values x of a 16-byte chunk,
// packed little-endian, without a division in the common case. With
// r = fl32(1/s), q = fl32(x * r) is within 2.5 fp32 ulps of fl32(x / s)
// (two roundings of 2^-24 relative error each, plus the 1/2 ulp of the
// exact quotient's own rounding). The e4m3 rounding of a normal value only
// changes at midpoints between codes, whose low 20 significand bits are
// exactly 0x80000, and no midpoint lies within 2^19 ulps of a binade edge;
// so if q's low 20 bits are more than 4 away from 0x80000, q and fl32(x / s)
// round to the same code. When any of the 8 products is closer, is in the
// e4m3 subnormal range (|q| < 2^-6), or 1/s overflowed (s subnormal), the
// chunk divides instead (one branch per chunk; rare for any real row).
// The rounding itself is the hardware conversion to e4m3fn after clamping
// to +-448 (round to nearest even, saturating): on gfx950 that equals the
// nearest-even saturating encode for every finite fp32 value.
template <bool HIGH>
__device__ __forceinline__ uint32_t cvt2_e4m3(float a, float b, uint32_t old) {
    const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, (int)old, HIGH);
}

__device__ __forceinline__ uint2 encode8(const uint4 &c, float s, float r, bool r_ok) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    if (s == 0.0f) {   // an all-zero row (uniform): signed zeros
        uint32_t out[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t a = w[2 * i], b = w[2 * i + 1];
            out[i] = ((a >> 8) & 0x80u) | ((a >> 16) & 0x8000u) | ((b << 8) & 0x800000u) |
                     (b & 0x80000000u);
        }
        return make_uint2(out[0], out[1]);
    }
    float xv[8], q[8];
    bool exact = r_ok;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xv[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        xv[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        q[i] = xv[i] * r;
        const uint32_t mag = __float_as_uint(q[i]) & 0x7FFFFFFFu;
        const uint32_t d = (mag & 0xFFFFFu) - 0x80000u + 4u;   // in [0, 8] near a midpoint
        exact &= (mag >= 0x3C800000u) & (d > 8u);
    }
    if (!exact) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = xv[i] / s;   // correctly rounded fp32 division
    }
    uint32_t lo = cvt2_e4m3<false>(q[0], q[1], 0u);
    lo = cvt2_e4m3<true>(q[2], q[3], lo);
    uint32_t hi = cvt2_e4m3<false>(q[4], q[5], 0u);
    hi = cvt2_e4m3<true>(q[6], q[7], hi);
    return make_uint2(lo, hi);
}

// 1/s rounded once per row, and whether it is finite (s subnormal: no)
__device__ __forceinline__ float recip_of(float s, bool &r_ok) {
    const float r = 1.0f / s;  // correctly rounded
    r_ok = (__float_as_uint(r) & 0x7FFFFFFFu) < 0x7F800000u;
    return r;
}

__device__ __forceinline__ uint32_t group_max(uint32_t v, int width) {
    for (int off = width / 2; off > 0; off >>= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

// TPR threads per row (16, 64, 256 or 1024); each holds NCH chunks of 8
// values (16 bytes) in registers between the max reduction and the encode.
// Chunk c of a row is handled by thread c % TPR, so each load instruction
// of a wave reads 64 consecutive chunks (1 KiB) and each store writes 512
// consecutive code bytes.
template <int QB, int TPR, int NCH>
__global__ __launch_bounds__(QB, (QB <= 256 && NCH <= 8) ? 4 : 1) void quant_rows_kernel(const uint16_t *__restrict__ x,
                                                            int64_t ldx, uint8_t *__restrict__ q,
                                                            int64_t ldq, float *__restrict__ scale,
                                                            int64_t M, int K) {
    constexpr int RPB = QB / TPR;
    const int tid = threadIdx.x;
    const int t = tid % TPR;
    const int64_t m = (int64_t)blockIdx.x * RPB + tid / TPR;
    const bool active = m < M;
    const int nch = K >> 3;
    const uint16_t *xr = x + (active ? m : 0) * ldx;

    uint4 v[NCH];
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = t + i * TPR;
        if (active && c < nch) {
            v[i] = ldg16(xr + 8 * c);
            amax = max(amax, absmax8(v[i]));
        } else {
            v[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    if (TPR <= 64) {
        amax = group_max(amax, TPR);
    } else {   // the TPR / 64 waves of this row meet in LDS
        __shared__ uint32_t red[QB / 64];
        amax = group_max(amax, 64);
        if ((tid & 63) == 0) red[tid >> 6] = amax;
        __syncthreads();
        const int w0 = (tid / TPR) * (TPR / 64);
        amax = red[w0];
#pragma unroll
        for (int i = 1; i < TPR / 64; ++i) amax = max(amax, red[w0 + i]);
    }
    const float s = bf16_to_f32(amax) / 448.0f;  // correctly rounded fp32 division
    if (!active) return;
    if (t == 0) scale[m] = s;
    bool r_ok;
    const float r = recip_of(s, r_ok);
    uint8_t *qr = q + m * ldq;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = t + i * TPR;
        if (c < nch) *reinterpret_cast<uint2 *>(qr + 8 * c) = encode8(v[i], s, r, r_ok);
    }
}

// Rows too long to hold in registers: a max pass, then a second read that
// encodes (the row is hot in L2 by then). One block of QBLOCK per row.
__global__ __launch_bounds__(QBLOCK) void quant_rows_long_kernel(const uint16_t *__restrict__ x,
                                                                 int64_t ldx,
                                                                 uint8_t *__restrict__ q,
                                                                 int64_t ldq,
                                                                 float *__restrict__ scale,
                                                                 int64_t M, int K) {
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int nch = K >> 3;
    const uint16_t *xr = x + m * ldx;
    uint32_t amax = 0;
    for (int c = tid; c < nch; c += QBLOCK) amax = max(amax, absmax8(ldg16(xr + 8 * c)));
    __shared__ uint32_t red[QBLOCK / 64];
    amax = group_max(amax, 64);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = red[0];
    for (int i = 1; i < QBLOCK / 64; ++i) amax = max(amax, red[i]);
    const float s = bf16_to_f32(amax) / 448.0f;
    if (tid == 0) scale[m] = s;
    bool r_ok;
    const float r = recip_of(s, r_ok);
    uint8_t *qr = q + m * ldq;
    for (int c = tid; c < nch; c += QBLOCK)
        *reinterpret_cast<uint2 *>(qr + 8 * c) = encode8(ldg16(xr + 8 * c), s, r, r_ok);
}

template <int QB, int TPR, int NCH>
void launch(const uint16_t *x, int64_t ldx, uint8_t *q, int64_t ldq, float *s, int64_t M, int K,
            hipStream_t st) {
    constexpr int RPB = QB / TPR;
    const dim3 grid((unsigned)((M + RPB - 1) / RPB));
    hipLaunchKernelGGL((quant_rows_kernel<QB, TPR, NCH>), grid, dim3(QB), 0, st, x, ldx, q, ldq, s,
                       M, K);
}

// Register budget: 1024-thread blocks get 128 VGPRs per lane, enough for 4
// chunks; 256-thread blocks hold up to 16.
template <int QB, int TPR>
bool launch_tpr(int nch_per_thread, const uint16_t *x, int64_t ldx, uint8_t *q, int64_t ldq,
                float *s, int64_t M, int K, hipStream_t st) {
    constexpr int CAP = QB > 256 ? 4 : 16;
    if (nch_per_thread <= 1) launch<QB, TPR, 1>(x, ldx, q, ldq, s, M, K, st);
    else if (nch_per_thread <= 2) launch<QB, TPR, 2>(x, ldx, q, ldq, s, M, K, st);
    else if (nch_per_thread <= 4) launch<QB, TPR, 4>(x, ldx, q, ldq, s, M, K, st);
    else if (nch_per_thread <= 8 && CAP >= 8) launch<QB, TPR, (CAP >= 8 ? 8 : 1)>(x, ldx, q, ldq, s, M, K, st);
    else if (nch_per_thread <= 16 && CAP >= 16) launch<QB, TPR, (CAP >= 16 ? 16 : 1)>(x, ldx, q, ldq, s, M, K, st);
    else return false;
    return true;
}

}  // namespace

hipError_t launch_quant_rows(const uint16_t *x, int64_t ld_x, uint8_t *q, int64_t ld_q,
                             float *scale, int64_t M, int64_t K, hipStream_t stream) {
    const int k = (int)K;
    const int nch = k / 8;
    // Many rows: a few threads per row is enough to fill the chip; few
    // rows: spread each row over a whole block (up to 1024 threads) to cut
    // the per-row latency, which is all a decode-sized call costs.
    // Many rows with long K: two waves per row keep 8 chunks a thread, few
    // enough registers for four waves per SIMD to overlap loads with the
    // (ALU-heavy) encoding.
    int tpr = M >= 512 ? (nch > 512 ? 128 : 64) : (M <= 64 ? 1024 : 256);
    if (nch <= 16) tpr = 16;
    else if (nch <= 64) tpr = 64;
    else if (nch <= 256 && tpr > 256) tpr = 256;
    const int per = (nch + tpr - 1) / tpr;
    bool ok;
    if (tpr == 16) ok = launch_tpr<QBLOCK, 16>(per, x, ld_x, q, ld_q, scale, M, k, stream);
    else if (tpr == 64) ok = launch_tpr<QBLOCK, 64>(per, x, ld_x, q, ld_q, scale, M, k, stream);
    else if (tpr == 128) ok = launch_tpr<QBLOCK, 128>(per, x, ld_x, q, ld_q, scale, M, k, stream);
    else if (tpr == 256) ok = launch_tpr<QBLOCK, 256>(per, x, ld_x, q, ld_q, scale, M, k, stream);
    else {
        ok = launch_tpr<1024, 1024>(per, x, ld_x, q, ld_q, scale, M, k, stream);
        if (!ok)   // long rows: 256 threads each hold more chunks
            ok = launch_tpr<QBLOCK, 256>((nch + 255) / 256, x, ld_x, q, ld_q, scale, M, k, stream);
    }
    if (!ok)
        hipLaunchKernelGGL(quant_rows_long_kernel, dim3((unsigned)M), dim3(QBLOCK), 0, stream, x,
                           ld_x, q, ld_q, scale, M, k);
    return hipGetLastError();
}

}  // namespace bsg
