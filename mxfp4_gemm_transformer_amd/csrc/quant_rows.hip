// Per-token activation quantization to e4m3fn: one fp32 scale per row
// (amax / 448) and the row's codes, in one HBM pass over the bf16 input.
// The "(q_fp8, scale)" pair is what the sly-radiance README's fused
// producers hand to its W4A8 GEMM (fused norm/quant rows of its file table).
//
// The same kernel, instantiated with a producer stage, is those fused
// producers: RMSNorm (with an optional residual add, the new residual
// written back) or SiLU(gate) * up computes each bf16 row in registers,
// and the quantizer runs on it without a trip through HBM.
#include "bs_device.hpp"
#include "bs_kernels.hpp"

namespace bsg {
namespace {

constexpr int QBLOCK = 256;

// Largest |bf16| of the 8 values in a 16-byte chunk, as a magnitude bit
// pattern (for finite values, integer order of exp|mantissa = value order).
// Both halves of a word at once with packed 16-bit maxima.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t absmax8(const uint4 &c) {
    const u16x2 a = __builtin_bit_cast(u16x2, c.x & 0x7FFF7FFFu);
    const u16x2 b = __builtin_bit_cast(u16x2, c.y & 0x7FFF7FFFu);
    const u16x2 d = __builtin_bit_cast(u16x2, c.z & 0x7FFF7FFFu);
    const u16x2 e = __builtin_bit_cast(u16x2, c.w & 0x7FFF7FFFu);
    const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                              __builtin_elementwise_max(d, e));
    return max((uint32_t)m.x, (uint32_t)m.y);
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xv[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        xv[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
    // Two running minima instead of a flag per value (one shift-add and
    // half a min3 per value): dmin, over (low 20 bits - 0x80000 + 4) mod
    // 2^20 moved to the top of the word, is at most 8 << 12 exactly when
    // some product's low 20 bits lie within 4 of 0x80000; qmin is the
    // smallest |product| (finite here whenever r is, so no NaN reaches it).
    uint32_t dmin = 0xFFFFFFFFu;
    float qmin = 448.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        q[i] = xv[i] * r;
        dmin = min(dmin, (__float_as_uint(q[i]) << 12) + 0x80004000u);
        qmin = fminf(qmin, fabsf(q[i]));
    }
    const bool exact = r_ok & (dmin > 0x8000u) & (qmin >= 0x1p-6f);
    if (!exact) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = xv[i] / s;   // correctly rounded fp32 division
    }
    // the low-half conversions keep whatever is in the upper half (the
    // high-half ones overwrite it), so they start from a value already in
    // a register rather than a zero of their own
    uint32_t lo = cvt2_e4m3<false>(q[0], q[1], __float_as_uint(q[0]));
    lo = cvt2_e4m3<true>(q[2], q[3], lo);
    uint32_t hi = cvt2_e4m3<false>(q[4], q[5], __float_as_uint(q[4]));
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

// ------------------------------------------------------------ producers
enum { PROD_NONE = 0, PROD_RMS = 1, PROD_ADD_RMS = 2, PROD_SILU_MUL = 3 };

struct ProdParams {
    const uint16_t *res;    // PROD_ADD_RMS: residual rows, read
    uint16_t *res_out;      // PROD_ADD_RMS: new residual rows, written (may equal res)
    int64_t ldr;
    const uint16_t *w;      // PROD_RMS / PROD_ADD_RMS: norm weight [K]
    double eps;
};

// Nearest bf16 to an fp64 value (bits), ties to even, overflow to infinity.
// Normal bf16 range: round the 52-bit fraction to 7 bits by adding
// 2^44 - 1 plus the kept LSB (a carry moves into the exponent), then rebias
// the exponent from 1023 to 127. Below 2^-126 the bf16 grid is uniform with
// step 2^-133, so the code is rint(|v| 2^133) (exact scaling; rint rounds
// to nearest even). `v` must be finite.
__device__ __forceinline__ uint32_t f64_to_bf16(double v) {
    const uint64_t bits = (uint64_t)__double_as_longlong(v);
    const uint32_t sign = (uint32_t)(bits >> 48) & 0x8000u;
    const uint64_t mag = bits & 0x7FFFFFFFFFFFFFFFull;
    uint32_t code;
    if (mag >= ((uint64_t)(1023 + 128) << 52)) {               // |v| >= 2^128
        code = 0x7F80u;
    } else if (mag < ((uint64_t)(1023 - 126) << 52)) {         // |v| < 2^-126
        code = (uint32_t)__builtin_rint(__longlong_as_double((long long)mag) * 0x1p133);
    } else {
        const uint64_t r = mag + ((1ull << 44) - 1) + ((mag >> 45) & 1ull);
        code = (uint32_t)(r >> 45) - ((1023u - 127u) << 7);    // may carry to 0x7F80
    }
    return sign | code;
}

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

// bf16(x + r) for the 8 pairs of two chunks (the fp64 sum of two bf16
// values rounds to the same bf16 as the exact sum), and the sum of the
// results' squares in fp64, in element order.
__device__ __forceinline__ uint4 add8(const uint4 &x, const uint4 &r, double &ss) {
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, rw[4] = {r.x, r.y, r.z, r.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a = f64_to_bf16((double)bf16_to_f32(lo16(xw[i])) + (double)bf16_to_f32(lo16(rw[i])));
        const uint32_t b = f64_to_bf16((double)bf16_to_f32(hi16(xw[i])) + (double)bf16_to_f32(hi16(rw[i])));
        const double da = bf16_to_f32(a), db = bf16_to_f32(b);
        ss += da * da;
        ss += db * db;
        o[i] = a | (b << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ void sumsq8(const uint4 &x, double &ss) {
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double a = bf16_to_f32(lo16(xw[i])), b = bf16_to_f32(hi16(xw[i]));
        ss += a * a;
        ss += b * b;
    }
}

// h = bf16(fl32(fl32(r * inv) * w)) for a chunk: the normalized value is
// rounded to fp32 from fp64, then multiplied by the weight in fp32.
__device__ __forceinline__ uint4 norm8(const uint4 &r, const uint4 &w, double inv) {
    const uint32_t rw[4] = {r.x, r.y, r.z, r.w}, ww[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float na = (float)((double)bf16_to_f32(lo16(rw[i])) * inv);
        const float nb = (float)((double)bf16_to_f32(hi16(rw[i])) * inv);
        o[i] = pack_bf16x2(na * bf16_to_f32(lo16(ww[i])), nb * bf16_to_f32(hi16(ww[i])));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// fl32(fl32(silu(g)) * u) (the caller rounds it to bf16), silu(g) =
// g / (1 + exp(-g)) taken in fp64 and rounded once to fp32. Fast path in fp32 for g >= -8: e = 2^(-g log2 e)
// from the hardware exp2 (the rounded argument, |arg| < 11.6, costs at most
// 6 ulps of relative error, the exp2 itself 1), then 1 + e, the hardware
// reciprocal (1 ulp), g * 1/(1 + e) and * u: the product is within about
// 10 fp32 ulps of the exact chain's product. Its bf16 rounding can only
// differ from the exact chain's when it lies within 16 fp32 ulps of a bf16
// rounding midpoint (low 16 bits near 0x8000) or is tiny; those elements,
// and gates below -8, are recomputed in fp64 (about 1 in 2000 for
// unit-scale data).
__device__ __forceinline__ float silu_mul1(uint32_t gb, uint32_t ub) {
    const float g = bf16_to_f32(gb), u = bf16_to_f32(ub);
    const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
    float a = (g * __builtin_amdgcn_rcpf(1.0f + e)) * u;
    const uint32_t ab = __float_as_uint(a);
    const bool risky = (g < -8.0f) | ((ab & 0x7FFFFFFFu) < 0x0F800000u) |     // |a| < 2^-96
                       (((ab & 0xFFFFu) - 0x8000u + 16u) <= 32u);
    if (risky) {
        const double gd = g;
        const float sg64 = (float)(gd / (1.0 + exp(-gd)));
        a = sg64 * u;
    }
    return a;
}

__device__ __forceinline__ uint4 silu_mul8(const uint4 &g, const uint4 &u) {
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2(silu_mul1(lo16(gw[i]), lo16(uw[i])), silu_mul1(hi16(gw[i]), hi16(uw[i])));
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ double group_sum(double v, int width) {
    for (int off = width / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// TPR threads per row (16, 64, 256 or 1024); each holds NCH chunks of 8
// values (16 bytes) in registers between the max reduction and the encode.
// Chunk c of a row is handled by thread c % TPR, so each load instruction
// of a wave reads 64 consecutive chunks (1 KiB) and each store writes 512
// consecutive code bytes.
//
// With a producer stage (PROD != PROD_NONE) the row to quantize is made
// first: x + residual (written back) and RMSNorm, or SiLU(gate) * up with
// the gate in columns [0, K) of x and up in [K, 2K). RMSNorm's sum of
// squares meets across the row's threads (shuffles, then LDS) before the
// normalization pass over the chunks still in registers.
template <int PROD, int QB, int TPR, int NCH>
__global__ __launch_bounds__(QB, (QB <= 256 && NCH <= 8) ? 4 : 1) void quant_rows_kernel(const uint16_t *__restrict__ x,
                                                            int64_t ldx, uint8_t *__restrict__ q,
                                                            int64_t ldq, float *__restrict__ scale,
                                                            int64_t M, int K, ProdParams pp) {
    constexpr int RPB = QB / TPR;
    const int tid = threadIdx.x;
    const int t = tid % TPR;
    const int64_t m = (int64_t)blockIdx.x * RPB + tid / TPR;
    const bool active = m < M;
    const int nch = K >> 3;
    const uint16_t *xr = x + (active ? m : 0) * ldx;

    uint4 v[NCH];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = t + i * TPR;
        if (active && c < nch) {
            if constexpr (PROD == PROD_NONE) {
                v[i] = ldg16(xr + 8 * c);
            } else if constexpr (PROD == PROD_RMS) {
                v[i] = ldg16(xr + 8 * c);
                sumsq8(v[i], ss);
            } else if constexpr (PROD == PROD_ADD_RMS) {
                const uint4 xv = ldg16(xr + 8 * c);
                const uint4 rv = ldg16(pp.res + m * pp.ldr + 8 * c);
                v[i] = add8(xv, rv, ss);
                *reinterpret_cast<uint4 *>(pp.res_out + m * pp.ldr + 8 * c) = v[i];
            } else {
                v[i] = silu_mul8(ldg16(xr + 8 * c), ldg16(xr + K + 8 * c));
            }
        } else {
            v[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    if constexpr (PROD == PROD_RMS || PROD == PROD_ADD_RMS) {
        if (TPR <= 64) {
            ss = group_sum(ss, TPR);
        } else {
            __shared__ double sred[QB / 64];
            ss = group_sum(ss, 64);
            if ((tid & 63) == 0) sred[tid >> 6] = ss;
            __syncthreads();
            const int w0 = (tid / TPR) * (TPR / 64);
            ss = sred[w0];
#pragma unroll
            for (int i = 1; i < TPR / 64; ++i) ss += sred[w0 + i];
        }
        const double inv = 1.0 / __builtin_sqrt(ss / (double)K + pp.eps);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = t + i * TPR;
            if (active && c < nch) v[i] = norm8(v[i], ldg16(pp.w + 8 * c), inv);
        }
    }
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) amax = max(amax, absmax8(v[i]));
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

template <int PROD, int QB, int TPR, int NCH>
void launch(const uint16_t *x, int64_t ldx, uint8_t *q, int64_t ldq, float *s, int64_t M, int K,
            const ProdParams &pp, hipStream_t st) {
    constexpr int RPB = QB / TPR;
    const dim3 grid((unsigned)((M + RPB - 1) / RPB));
    hipLaunchKernelGGL((quant_rows_kernel<PROD, QB, TPR, NCH>), grid, dim3(QB), 0, st, x, ldx, q,
                       ldq, s, M, K, pp);
}

// Register budget: 1024-thread blocks get 128 VGPRs per lane, enough for 4
// chunks; 256-thread blocks hold up to 16.
template <int PROD, int QB, int TPR>
bool launch_tpr(int nch_per_thread, const uint16_t *x, int64_t ldx, uint8_t *q, int64_t ldq,
                float *s, int64_t M, int K, const ProdParams &pp, hipStream_t st) {
    constexpr int CAP = QB > 256 ? 4 : 16;
    if (nch_per_thread <= 1) launch<PROD, QB, TPR, 1>(x, ldx, q, ldq, s, M, K, pp, st);
    else if (nch_per_thread <= 2) launch<PROD, QB, TPR, 2>(x, ldx, q, ldq, s, M, K, pp, st);
    else if (nch_per_thread <= 4) launch<PROD, QB, TPR, 4>(x, ldx, q, ldq, s, M, K, pp, st);
    else if (nch_per_thread <= 8 && CAP >= 8) launch<PROD, QB, TPR, (CAP >= 8 ? 8 : 1)>(x, ldx, q, ldq, s, M, K, pp, st);
    else if (nch_per_thread <= 16 && CAP >= 16) launch<PROD, QB, TPR, (CAP >= 16 ? 16 : 1)>(x, ldx, q, ldq, s, M, K, pp, st);
    else return false;
    return true;
}

}  // namespace

hipError_t launch_quant_rows(const uint16_t *x, int64_t ld_x, uint8_t *q, int64_t ld_q,
                             float *scale, int64_t M, int64_t K, hipStream_t stream) {
    const int k = (int)K;
    const int nch = k / 8;
    // Few rows: spread each row over a whole block (up to 1024 threads) to
    // cut the per-row latency, which is all a decode-sized call costs. Many
    // rows (a sweep on MI355X with inputs read from HBM): from 2048 rows, 256
    // threads a row with up to 4 chunks each past 4096 values, else 128
    // (4096 x 8192 in 26.3 us against 27.2 with 512 threads of 2 chunks,
    // 4096 x 5120 in 18.3 against 19.9); from 512 rows, one or two chunks
    // per thread, up to 512 threads a row (512 x 8192 in 6.2 us). A single
    // row takes 512 threads of two chunks: 1 x 7168 in 3.0-3.3 us against
    // 3.2-3.3 with 1024, and a quantize + GEMM step of 8.4 against 9.1 us;
    // from two rows on, 1024 (8 x 7168: 3.5-3.6 us against 3.5-3.8 with 512
    // and 4.2-4.3 with 256; 16 and 64 rows alike).
    int tpr = M == 1 ? 512 : M <= 64 ? 1024 : 256;
    if (M >= 2048) {
        tpr = nch > 512 ? 256 : 128;
    } else if (M >= 512) {
        tpr = 64;
        while (tpr < nch && tpr < 512) tpr <<= 1;
    }
    if (nch <= 16) tpr = 16;
    else if (nch <= 64) tpr = 64;
    else if (nch <= 256 && tpr > 256) tpr = 256;
    const int per = (nch + tpr - 1) / tpr;
    const ProdParams pp{};
    bool ok;
    if (tpr == 16) ok = launch_tpr<PROD_NONE, QBLOCK, 16>(per, x, ld_x, q, ld_q, scale, M, k, pp, stream);
    else if (tpr == 64) ok = launch_tpr<PROD_NONE, QBLOCK, 64>(per, x, ld_x, q, ld_q, scale, M, k, pp, stream);
    else if (tpr == 128) ok = launch_tpr<PROD_NONE, QBLOCK, 128>(per, x, ld_x, q, ld_q, scale, M, k, pp, stream);
    else if (tpr == 256) ok = launch_tpr<PROD_NONE, QBLOCK, 256>(per, x, ld_x, q, ld_q, scale, M, k, pp, stream);
    else if (tpr == 512) {
        ok = launch_tpr<PROD_NONE, 512, 512>(per, x, ld_x, q, ld_q, scale, M, k, pp, stream);
        if (!ok)   // long rows: 256 threads each hold more chunks
            ok = launch_tpr<PROD_NONE, QBLOCK, 256>((nch + 255) / 256, x, ld_x, q, ld_q, scale, M, k, pp, stream);
    } else {
        ok = launch_tpr<PROD_NONE, 1024, 1024>(per, x, ld_x, q, ld_q, scale, M, k, pp, stream);
        if (!ok)   // long rows: 256 threads each hold more chunks
            ok = launch_tpr<PROD_NONE, QBLOCK, 256>((nch + 255) / 256, x, ld_x, q, ld_q, scale, M, k, pp, stream);
    }
    if (!ok)
        hipLaunchKernelGGL(quant_rows_long_kernel, dim3((unsigned)M), dim3(QBLOCK), 0, stream, x,
                           ld_x, q, ld_q, scale, M, k);
    return hipGetLastError();
}

namespace {

// Static-scale quantization: one given scale for every row, so no reduction;
// each thread encodes 16-byte chunks of the flattened rows.
__global__ __launch_bounds__(256) void quant_static_kernel(const uint16_t *__restrict__ x,
                                                           int64_t ldx, uint8_t *__restrict__ q,
                                                           int64_t ldq,
                                                           const float *__restrict__ s_in,
                                                           float *__restrict__ s_out, int64_t M,
                                                           int K) {
    const float s = *s_in;
    bool r_ok;
    const float r = recip_of(s, r_ok);
    const int nch = K >> 3;
    const int64_t total = M * nch;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t m = idx / nch;
        const int c = (int)(idx - m * nch);
        *reinterpret_cast<uint2 *>(q + m * ldq + 8 * c) = encode8(ldg16(x + m * ldx + 8 * c), s, r, r_ok);
        if (s_out && c == 0) s_out[m] = s;
    }
}

// MXFP4 quantization (OCP MX): per 32-element block, the E8M0 byte of
// floor(log2 amax) - 2 (the exponent field of the bf16 amax minus 2, clamped
// at 0; a zero block gets 0), and each element's e2m1 code of x / 2^(byte -
// 127), nearest with ties to the even code, saturating at 6, sign kept.
//
// Each lane takes one 16-byte chunk (8 values), so a wave's load reads 1 KiB
// of consecutive bytes and its store writes 256; a block's 4 chunks sit in
// a quad of lanes, whose maxima meet through two DPP quad permutations. The
// codes come from gfx950's scaled bf16-pair to fp4 conversion with the
// scale 2^(byte - 127), one instruction per pair of values: on MI355X it
// divides by the scale, rounds to nearest even and saturates: it gave the
// same code as the rule above for every finite bf16 value at every scale
// byte this kernel can produce (0..252), subnormal scale (byte 0) and
// signed zeros included.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    // quad_perm [1,0,3,2] then [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
    return v;
}

__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t *__restrict__ x,
                                                          int64_t ldx, uint8_t *__restrict__ q,
                                                          int64_t ldq, uint8_t *__restrict__ sc,
                                                          int64_t M, int K) {
    const int CPR = K >> 3;                          // 16-byte chunks per row (a multiple of 4)
    const int64_t total = M * CPR;
    // the stride is a multiple of 4 and so is total: a quad is in or out as a whole
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t m = idx / CPR;
        const int c = (int)(idx - m * CPR);
        const uint4 v = ldg16(x + m * ldx + 8 * c);
        const uint32_t amax = quad_max(absmax8(v));
        const uint32_t e = amax >> 7;                // bf16 exponent field of amax
        const uint32_t byte = e >= 2 ? e - 2 : 0;
        const float scl = __uint_as_float(byte ? byte << 23 : 0x00400000u);   // 2^(byte - 127)
        uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
            v.x, __builtin_bit_cast(bf16x2_t, v.x), scl, 0);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, v.y), scl, 1);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, v.z), scl, 2);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2_t, v.w), scl, 3);
        *reinterpret_cast<uint32_t *>(q + m * ldq + 4 * c) = word;
        if ((c & 3) == 0) sc[m * (CPR >> 2) + (c >> 2)] = (uint8_t)byte;
    }
}

// Thread count per row for a producer: the quantizer's choice, widened
// until each thread holds at most 16 chunks (8 for 128 threads per row).
template <int PROD>
bool launch_producer(const uint16_t *x, int64_t ldx, uint8_t *q, int64_t ldq, float *s, int64_t M,
                     int K, const ProdParams &pp, hipStream_t st) {
    const int nch = K / 8;
    // Many rows: the fewest threads a row with at most 4 chunks each (a
    // sweep on MI355X at M = 4096: SiLU * up over 17408 in 96 us against 108
    // us with 256 threads of 9 chunks; RMSNorm over 5120 in 42 against 44 us
    // with 128 threads of 5, and slower again with 512 or 1024 threads, whose
    // sum of squares meets across more waves).
    int tpr = M >= 512 ? 64 : (M <= 64 ? 1024 : 256);
    if (M >= 512)
        while (nch > 4 * tpr && tpr < 1024) tpr <<= 1;
    if (nch <= 16) tpr = 16;
    else if (nch <= 64) tpr = 64;
    else if (nch <= 256 && tpr > 256) tpr = 256;
    if (tpr == 256 && nch > 256 * 16) tpr = 1024;
    const int per = (nch + tpr - 1) / tpr;
    switch (tpr) {
    case 16: return launch_tpr<PROD, QBLOCK, 16>(per, x, ldx, q, ldq, s, M, K, pp, st);
    case 64: return launch_tpr<PROD, QBLOCK, 64>(per, x, ldx, q, ldq, s, M, K, pp, st);
    case 128: return launch_tpr<PROD, QBLOCK, 128>(per, x, ldx, q, ldq, s, M, K, pp, st);
    case 256: return launch_tpr<PROD, QBLOCK, 256>(per, x, ldx, q, ldq, s, M, K, pp, st);
    case 512: return launch_tpr<PROD, 512, 512>(per, x, ldx, q, ldq, s, M, K, pp, st);
    default: return launch_tpr<PROD, 1024, 1024>(per, x, ldx, q, ldq, s, M, K, pp, st);
    }
}

}  // namespace

hipError_t launch_add_rms_quant(const uint16_t *x, int64_t ld_x, uint16_t *residual, int64_t ld_r,
                                const uint16_t *weight, double eps, uint8_t *q, int64_t ld_q,
                                float *scale, int64_t M, int64_t K, hipStream_t stream) {
    ProdParams pp{};
    pp.res = residual;
    pp.res_out = residual;
    pp.ldr = ld_r;
    pp.w = weight;
    pp.eps = eps;
    const bool ok = residual
        ? launch_producer<PROD_ADD_RMS>(x, ld_x, q, ld_q, scale, M, (int)K, pp, stream)
        : launch_producer<PROD_RMS>(x, ld_x, q, ld_q, scale, M, (int)K, pp, stream);
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

hipError_t launch_quant_mxfp4_rows(const uint16_t *x, int64_t ld_x, uint8_t *q, int64_t ld_q,
                                   uint8_t *scale, int64_t M, int64_t K, hipStream_t stream) {
    const int64_t chunks = M * (K / 8);
    const int64_t grid = (chunks + 255) / 256;
    hipLaunchKernelGGL(quant_mxfp4_kernel, dim3((unsigned)(grid < 8192 ? grid : 8192)), dim3(256),
                       0, stream, x, ld_x, q, ld_q, scale, M, (int)K);
    return hipGetLastError();
}

hipError_t launch_quant_rows_static(const uint16_t *x, int64_t ld_x, const float *scale_in,
                                    uint8_t *q, int64_t ld_q, float *scale_out, int64_t M,
                                    int64_t K, hipStream_t stream) {
    const int64_t chunks = M * (K / 8);
    const int64_t blocks = (chunks + 255) / 256;
    hipLaunchKernelGGL(quant_static_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                       dim3(256), 0, stream, x, ld_x, q, ld_q, scale_in, scale_out, M, (int)K);
    return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const uint16_t *gate_up, int64_t ld_gu, uint8_t *q, int64_t ld_q,
                                 float *scale, int64_t M, int64_t I, hipStream_t stream) {
    const ProdParams pp{};
    const bool ok = launch_producer<PROD_SILU_MUL>(gate_up, ld_gu, q, ld_q, scale, M, (int)I, pp, stream);
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

}  // namespace bsg
