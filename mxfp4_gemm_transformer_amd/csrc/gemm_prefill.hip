// Large-M ("prefill") block-scaled GEMM on V_MFMA_SCALE_F32_32X32X64_F8F6F4.
// The sly-radiance README gives large M to a separate LDS-tiled kernel (its
// W4A8 prefill row); here the E8M0 weight scales go straight into the MFMA's
// per-lane scale operand, one per 32-element K block, so a K step is MFMAs
// only, and the per-token fp32 activation scale is applied in the epilogue.
//
// Tiling: a BM x BN output tile per workgroup of 4 waves in a 2 x 2 grid,
// each wave owning (BM/2) x (BN/2) as 32x32 MFMA tiles. K advances 128 at a
// time through two LDS stages: while the MFMAs consume one stage, the next
// step's A and W tiles are fetched into registers and written to the other
// stage. LDS rows are 16-byte chunks XOR-swizzled by row so that the 32
// lanes reading one chunk column hit different banks.
#include "bs_device.hpp"
#include "bs_kernels.hpp"

namespace bsg {
namespace {

constexpr int PBLOCK = 256;
constexpr int BK = 128;

template <bool FP4, int BM, int BN>
struct PrefillCfg {
    static constexpr int WBYTES = FP4 ? BK / 2 : BK;   // weight bytes per row per K step
    static constexpr int ACH = BK / 16;                // 16-byte chunks per A row
    static constexpr int WCH = WBYTES / 16;            // chunks per W row
    static constexpr int A_STAGE = BM * BK;
    static constexpr int W_STAGE = BN * WBYTES;
    static constexpr int LDS = 2 * (A_STAGE + W_STAGE);
    static constexpr int A_PER_T = BM * ACH / PBLOCK;  // chunks each thread copies
    static constexpr int W_PER_T = BN * WCH / PBLOCK;
    static constexpr int TM = BM / 2 / 32, TN = BN / 2 / 32;
    static_assert(BM * ACH % PBLOCK == 0 && BN * WCH % PBLOCK == 0, "tile / block mismatch");
};

template <bool FP4, int BM, int BN>
__global__ __launch_bounds__(PBLOCK) void gemm_prefill_kernel(
    const uint8_t *__restrict__ A, int64_t lda, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ W, int64_t ldw, const uint8_t *__restrict__ WS,
    const uint16_t *__restrict__ bias, int epi, uint16_t *__restrict__ Y, int64_t ldy, int M, int N,
    int K) {
    using C = PrefillCfg<FP4, BM, BN>;
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t *sA = lds;                      // [2][BM][BK]
    uint8_t *sW = lds + 2 * C::A_STAGE;     // [2][BN][WBYTES]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, lg = lane >> 5;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int KB = K >> 5;
    const int nsteps = (K + BK - 1) / BK;

    // ---- global -> register copy of one K step
    uint4 ra[C::A_PER_T], rw[C::W_PER_T];
    auto fetch = [&](int s) {
        const int kbase = s * BK;
#pragma unroll
        for (int j = 0; j < C::A_PER_T; ++j) {
            const int c = tid + j * PBLOCK, row = c / C::ACH, ch = c % C::ACH;
            const int64_t m = m0 + row;
            const int k = kbase + ch * 16;
            ra[j] = (m < M && k < K) ? ldg16(A + m * lda + k) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < C::W_PER_T; ++j) {
            const int c = tid + j * PBLOCK, row = c / C::WCH, ch = c % C::WCH;
            const int64_t n = n0 + row;
            const int k = kbase + ch * (FP4 ? 32 : 16);    // first element of the chunk
            rw[j] = (n < N && k < K) ? ldg16(W + n * ldw + (FP4 ? k / 2 : k))
                                     : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int j = 0; j < C::A_PER_T; ++j) {
            const int c = tid + j * PBLOCK, row = c / C::ACH, ch = c % C::ACH;
            *reinterpret_cast<uint4 *>(sA + buf * C::A_STAGE + row * BK + ((ch ^ (row & 7)) << 4)) = ra[j];
        }
#pragma unroll
        for (int j = 0; j < C::W_PER_T; ++j) {
            const int c = tid + j * PBLOCK, row = c / C::WCH, ch = c % C::WCH;
            *reinterpret_cast<uint4 *>(sW + buf * C::W_STAGE + row * C::WBYTES +
                                       ((ch ^ (row & (C::WCH - 1))) << 4)) = rw[j];
        }
    };

    v16f acc[C::TM][C::TN];
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TN; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    // weight rows of this lane's B fragments, for the scale lookups
    const uint8_t *wsrow[C::TN];
#pragma unroll
    for (int b = 0; b < C::TN; ++b) {
        int64_t n = n0 + wn * (BN / 2) + b * 32 + li;
        if (n >= N) n = N - 1;
        wsrow[b] = FP4 ? WS + n * KB : WS + (n >> 5) * KB;
    }

    fetch(0);
    stash(0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        if (s + 1 < nsteps) fetch(s + 1);
        const uint8_t *tA = sA + buf * C::A_STAGE;
        const uint8_t *tW = sW + buf * C::W_STAGE;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // this lane's scale block: k = s*128 + kk*64 + 32*lg
            const int kb = s * 4 + kk * 2 + lg;
            v8i af[C::TM], bf[C::TN];
            int sc[C::TN];
#pragma unroll
            for (int a = 0; a < C::TM; ++a) {
                const int row = wm * (BM / 2) + a * 32 + li;
                const int c0 = kk * 4 + lg, c1 = kk * 4 + 2 + lg;
                const uint8_t *base = tA + row * BK;
                af[a] = pack8(*reinterpret_cast<const uint4 *>(base + ((c0 ^ (row & 7)) << 4)),
                              *reinterpret_cast<const uint4 *>(base + ((c1 ^ (row & 7)) << 4)));
            }
#pragma unroll
            for (int b = 0; b < C::TN; ++b) {
                const int row = wn * (BN / 2) + b * 32 + li;
                const uint8_t *base = tW + row * C::WBYTES;
                if (FP4) {
                    const int c0 = kk * 2 + lg;
                    bf[b] = pack8(*reinterpret_cast<const uint4 *>(base + ((c0 ^ (row & 3)) << 4)),
                                  make_uint4(0u, 0u, 0u, 0u));
                } else {
                    const int c0 = kk * 4 + lg, c1 = kk * 4 + 2 + lg;
                    bf[b] = pack8(*reinterpret_cast<const uint4 *>(base + ((c0 ^ (row & 7)) << 4)),
                                  *reinterpret_cast<const uint4 *>(base + ((c1 ^ (row & 7)) << 4)));
                }
                sc[b] = kb < KB ? wsrow[b][kb] : E8M0_ONE;
            }
#pragma unroll
            for (int a = 0; a < C::TM; ++a)
#pragma unroll
                for (int b = 0; b < C::TN; ++b)
                    acc[a][b] = mfma32<FP4>(af[a], bf[b], acc[a][b], E8M0_ONE, sc[b]);
        }
        if (s + 1 < nsteps) {
            __syncthreads();  // everyone is done reading the other stage
            stash(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: D lane l = i + 32 g, VGPR v -> row 8 (v/4) + 4 g + v%4, column i
#pragma unroll
    for (int a = 0; a < C::TM; ++a) {
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
            const int64_t n = n0 + wn * (BN / 2) + b * 32 + li;
            if (n >= N) continue;
            const float bv = epi != EPI_NONE ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * (BM / 2) + a * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
                if (m < M)
                    Y[m * ldy + n] = (uint16_t)f32_to_bf16(epilogue(acc[a][b][v], a_scale[m], bv, epi));
            }
        }
    }
}

template <bool FP4, int BM, int BN>
hipError_t launch_tile(const uint8_t *a, int64_t lda, const float *as, const uint8_t *w,
                       int64_t ldw, const uint8_t *ws, const uint16_t *bias, int epi, uint16_t *y,
                       int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    using C = PrefillCfg<FP4, BM, BN>;
    auto kern = gemm_prefill_kernel<FP4, BM, BN>;
    static bool attr_set = false;   // per template instance; idempotent
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    hipLaunchKernelGGL(kern, grid, dim3(PBLOCK), C::LDS, st, a, lda, as, w, ldw, ws, bias, epi, y,
                       ldy, (int)M, (int)N, (int)K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_prefill(bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                               const uint8_t *w, int64_t ldw, const uint8_t *ws,
                               const uint16_t *bias, int epi, uint16_t *y, int64_t ldy, int64_t M,
                               int64_t N, int64_t K, int num_cus, hipStream_t st) {
    (void)num_cus;
    if (fp4)
        return launch_tile<true, 128, 128>(a, lda, a_scale, w, ldw, ws, bias, epi, y, ldy, M, N, K, st);
    return launch_tile<false, 128, 128>(a, lda, a_scale, w, ldw, ws, bias, epi, y, ldy, M, N, K, st);
}

}  // namespace bsg
