// Small-M ("decode") block-scaled GEMM: the weight matrix is streamed from
// HBM exactly once. The sly-radiance README (its kernel row and decode-cell
// sweep row) routes small M to a separate decode kernel because the large-M
// kernel was more than twice as slow there; this is that role on gfx950.
//
// Work split: one workgroup per tile of 16 weight rows (8 with the folded
// layout below); its waves split K between them, each issuing every load of
// its share before the first MFMA so that the whole share is in flight at
// once. The waves' partial tiles meet in LDS, in a fixed order, and the
// bias / GELU epilogue writes bf16. No workspace, no inter-workgroup
// synchronisation.
//
// The MFMA is V_MFMA_SCALE_F32_16X16X128_F8F6F4: tokens on the A side
// (padded with zeros to 16), weight rows on the B side, the weights' E8M0
// block scales applied by the instruction per 32-element K block, and the
// activation scale (fp32, per token) applied in the epilogue.
//
// Folded layout for M <= 8: the 16 A rows hold 8 tokens twice and the 16 B
// columns hold 8 weight rows twice, each copy on a different 128-wide half
// of a 256-wide K window. The two diagonal 8x8 blocks of the 16x16 result
// are partial sums over the two halves and add up to the 8x8 output; the
// off-diagonal blocks are discarded. This halves the weight rows per
// workgroup, doubling the number of workgroups that stream W.
#include "bs_device.hpp"
#include "bs_kernels.hpp"

namespace bsg {
namespace {

template <bool FP4, bool FOLD, int MT, int NW, int SPW>
__global__ __launch_bounds__(NW * 64) void gemm_decode_kernel(
    const uint8_t *__restrict__ A, int64_t lda, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ W, int64_t ldw, const uint8_t *__restrict__ WS,
    const uint16_t *__restrict__ bias, int epi, uint16_t *__restrict__ Y, int64_t ldy, int M,
    int K) {
    constexpr int COLS = FOLD ? 8 : 16;
    constexpr int ROWS = FOLD ? 8 : 16 * MT;
    constexpr int KSTEP = FOLD ? 256 : 128;
    __shared__ float red[NW][ROWS][COLS + 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int col = FOLD ? (i & 7) : i;
    const int half = FOLD ? (i >> 3) : 0;
    const int64_t n = (int64_t)blockIdx.x * COLS + col;  // this lane's weight row
    const int KB = K >> 5;
    const int nsteps = (K + KSTEP - 1) / KSTEP;
    const uint8_t *wrow = W + n * ldw;
    const uint8_t *wsrow = FP4 ? WS + n * KB : WS + (n >> 5) * KB;

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int s0 = wave; s0 < nsteps; s0 += NW * SPW) {
        v8i wv[SPW];
        int wsc[SPW];
        v8i av[SPW][MT];
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            const int s = s0 + u * NW;
            const bool on = s < nsteps;
            const int k0 = s * KSTEP + half * 128;  // this lane's 128-wide window
            const int kblk = k0 + 32 * g;           // the block whose scale this lane supplies
            const int klo = k0 + 16 * g, khi = k0 + 64 + 16 * g;  // fp8 operand halves
            uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
            int sc = E8M0_ONE;
            if (FP4) {
                if (on && kblk < K) {
                    lo = ldg16(wrow + (kblk >> 1));
                    sc = wsrow[kblk >> 5];
                }
            } else {
                if (on && klo < K) lo = ldg16(wrow + klo);
                if (on && khi < K) hi = ldg16(wrow + khi);
                if (on && kblk < K) sc = wsrow[kblk >> 5];
            }
            wv[u] = pack8(lo, hi);
            wsc[u] = sc;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = FOLD ? (i & 7) : (mt * 16 + i);
                uint4 alo = make_uint4(0u, 0u, 0u, 0u), ahi = alo;
                if (on && m < M) {
                    const uint8_t *arow = A + (int64_t)m * lda;
                    if (klo < K) alo = ldg16(arow + klo);
                    if (khi < K) ahi = ldg16(arow + khi);
                }
                av[u][mt] = pack8(alo, ahi);
            }
        }
#pragma unroll
        for (int u = 0; u < SPW; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = mfma16<FP4>(av[u][mt], wv[u], acc[mt], E8M0_ONE, wsc[u]);
    }

    // D: lane l = i + 16 g, VGPR v -> token row 4 g + v, weight column i.
    if (FOLD) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[0][v] += __shfl_down(acc[0][v], 40, 64);
        if (g < 2 && i < 8) {
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][4 * g + v][i] = acc[0][v];
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][mt * 16 + 4 * g + v][i] = acc[mt][v];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < ROWS * COLS; idx += NW * 64) {
        const int r = idx / COLS, c = idx % COLS;
        if (r < M) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sum += red[w][r][c];
            const int64_t nn = (int64_t)blockIdx.x * COLS + c;
            const float b = epi != EPI_NONE ? bf16_to_f32(bias[nn]) : 0.f;
            Y[(int64_t)r * ldy + nn] = (uint16_t)f32_to_bf16(epilogue(sum, a_scale[r], b, epi));
        }
    }
}

template <bool FP4, bool FOLD, int MT, int NW, int SPW>
void launch_one(const uint8_t *a, int64_t lda, const float *as, const uint8_t *w, int64_t ldw,
                const uint8_t *ws, const uint16_t *bias, int epi, uint16_t *y, int64_t ldy,
                int64_t M, int64_t N, int64_t K, hipStream_t st) {
    constexpr int COLS = FOLD ? 8 : 16;
    hipLaunchKernelGGL((gemm_decode_kernel<FP4, FOLD, MT, NW, SPW>), dim3((unsigned)(N / COLS)),
                       dim3(NW * 64), 0, st, a, lda, as, w, ldw, ws, bias, epi, y, ldy, (int)M,
                       (int)K);
}

// Steps per wave held in registers at once: all of a wave's share when it
// fits (at most 8 weight fragments, and at most 8 fragments x M-tiles).
template <bool FP4, bool FOLD, int MT>
void launch_spw(int per_wave, const uint8_t *a, int64_t lda, const float *as, const uint8_t *w,
                int64_t ldw, const uint8_t *ws, const uint16_t *bias, int epi, uint16_t *y,
                int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    constexpr int NW = 8;
    constexpr int CAP = 8 / MT;
    if (per_wave <= 1 || CAP == 1)
        launch_one<FP4, FOLD, MT, NW, 1>(a, lda, as, w, ldw, ws, bias, epi, y, ldy, M, N, K, st);
    else if (per_wave <= 2 || CAP == 2)
        launch_one<FP4, FOLD, MT, NW, 2>(a, lda, as, w, ldw, ws, bias, epi, y, ldy, M, N, K, st);
    else if (per_wave <= 4 || CAP == 4)
        launch_one<FP4, FOLD, MT, NW, (CAP >= 4 ? 4 : 1)>(a, lda, as, w, ldw, ws, bias, epi, y,
                                                          ldy, M, N, K, st);
    else
        launch_one<FP4, FOLD, MT, NW, (CAP >= 8 ? 8 : 1)>(a, lda, as, w, ldw, ws, bias, epi, y,
                                                          ldy, M, N, K, st);
}

}  // namespace

hipError_t launch_gemm_decode(bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                              const uint8_t *w, int64_t ldw, const uint8_t *ws,
                              const uint16_t *bias, int epi, uint16_t *y, int64_t ldy, int64_t M,
                              int64_t N, int64_t K, int num_cus, hipStream_t st) {
    (void)num_cus;
    constexpr int NW = 8;
    if (M <= 8) {
        const int per = (int)(((K + 255) / 256 + NW - 1) / NW);
        if (fp4)
            launch_spw<true, true, 1>(per, a, lda, a_scale, w, ldw, ws, bias, epi, y, ldy, M, N, K, st);
        else
            launch_spw<false, true, 1>(per, a, lda, a_scale, w, ldw, ws, bias, epi, y, ldy, M, N, K, st);
        return hipGetLastError();
    }
    const int mt = (int)((M + 15) / 16);
    const int per = (int)(((K + 127) / 128 + NW - 1) / NW);
#define BSG_DECODE_MT(MT)                                                                          \
    if (fp4)                                                                                       \
        launch_spw<true, false, MT>(per, a, lda, a_scale, w, ldw, ws, bias, epi, y, ldy, M, N, K,  \
                                    st);                                                           \
    else                                                                                           \
        launch_spw<false, false, MT>(per, a, lda, a_scale, w, ldw, ws, bias, epi, y, ldy, M, N, K, \
                                     st);
    switch (mt) {
    case 1: BSG_DECODE_MT(1) break;
    case 2: BSG_DECODE_MT(2) break;
    case 3: BSG_DECODE_MT(3) break;
    default: BSG_DECODE_MT(4) break;
    }
#undef BSG_DECODE_MT
    return hipGetLastError();
}

}  // namespace bsg
