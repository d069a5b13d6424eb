// Small-M ("decode") block-scaled GEMM: the weight matrix is streamed from
// HBM exactly once. The sly-radiance README (its kernel row and decode-cell
// sweep row) routes small M to a separate decode kernel because the large-M
// kernel was more than twice as slow there; this is that role on gfx950.
//
// Work split: one workgroup per tile of 16 weight rows (8 with the folded
// layout below); its waves split K between them, each issuing every load of
// its share before the first MFMA so that the whole share is in flight at
// once. The waves' partial tiles meet in LDS, in a fixed order, and the
// bias / GELU epilogue writes bf16. Two more shapes of the same idea follow:
// for wide layers, one workgroup per CU with (row group, K step) units dealt
// evenly to its waves; for 16 < M <= 64 on narrow layers, K split across
// workgroups with fp32 partial sums in the caller's workspace, added in a
// fixed order by a second kernel. No inter-workgroup synchronisation.
//
// The MFMA is V_MFMA_SCALE_F32_16X16X128_F8F6F4: tokens on the A side
// (padded with zeros to 16), weight rows on the B side, the weights' E8M0
// block scales applied by the instruction per 32-element K block, and the
// activation scale (fp32, per token) applied in the epilogue.
//
// Folded layout for M <= 8 (and two such token groups for M <= 16 on
// narrow layers): the 16 A rows hold 8 tokens twice and the 16 B
// columns hold 8 weight rows twice, each copy on a different half of a
// 256-wide K window (the halves interleave at 64 bytes so that loads cover
// whole cache lines; see fold_k). The two diagonal 8x8 blocks of the 16x16 result
// are partial sums over the two halves and add up to the 8x8 output; the
// off-diagonal blocks are discarded. This halves the weight rows per
// workgroup, doubling the number of workgroups that stream W.
#include "bs_device.hpp"
#include "bs_kernels.hpp"

namespace bsg {
namespace {

constexpr uint32_t OOB_OFF = 0x80000000u;   // a per-lane offset past every buffer: reads zero

// A raw buffer descriptor over [base, base + bytes), bytes clipped to 2^31 - 16.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             (int)(bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes),
                                             0x00020000);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// A weight load, marked streaming (non-temporal) when NT: each weight byte is
// read once per call, and kept out of the way it leaves L2 to the
// activations every workgroup reads. Measured on MI355X: the balanced kernel
// on the MXFP4 gate_up (34816 x 5120) 21.5 -> 20.3 us at M=1 and 25.0 -> 23.9
// us at M=16; split-K at M=16 on a 2048 x 7168 layer 8.6 -> 8.3 us; but
// split-K over a 248320 x 5120 layer 256 -> 314 us, so large layers keep the
// default policy (and the folded kernel, where it made no difference).
// A streaming (non-temporal) 16-byte weight load through a pointer, for the
// grouped MoE kernel (123 -> 119 us over 32 experts of 4096 x 7168 MXFP4
// weights; see bloadw16 below for why).
__device__ __forceinline__ uint4 ldgw16_nt(const void *p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <bool NT>
__device__ __forceinline__ uint4 bloadw16(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, NT ? 2 : 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Where lane group g of K-half `half` finds its operand pieces in the folded
// layout's 256-wide window starting at kw. The instruction's 8-bit operand
// takes, per lane group g, a 16-byte "lo" piece (its K elements 16 g ...)
// and a "hi" piece (64 + 16 g ...); its K blocks of 32 are the lo pieces of
// groups 0-1 and 2-3, then the hi pieces of the same; an fp4 operand holds
// block g in group g. Any placement that gives each block one whole
// 32-element block of the window keeps the products and the E8M0 scales
// right. This one interleaves the halves at 64 bytes (lo at 64 half + 16 g,
// hi 128 bytes later), so each 16-byte-per-lane load covers whole 128-byte
// lines of 8 rows instead of one 64-byte half of each; block b of half h
// is block 2 h + (b & 1) + 4 (b >> 1) of the window.
struct FoldK {
    int kblk, klo, khi;   // scale / fp4 block start, fp8 lo and hi pieces (elements)
};
__device__ __forceinline__ FoldK fold_k(int kw, int half, int g) {
    const int klo = kw + 64 * half + 16 * g;
    return {kw + 32 * (2 * half + (g & 1) + 4 * (g >> 1)), klo, klo + 128};
}

template <bool FP4, bool FOLD, int MT, int NW, int SPW>
__global__ __launch_bounds__(NW * 64) void gemm_decode_kernel(
    const uint8_t *__restrict__ A, int64_t lda, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ W, int64_t ldw, const uint8_t *__restrict__ WS,
    const float *__restrict__ colscale, const uint16_t *__restrict__ bias, int epi,
    uint16_t *__restrict__ Y, int64_t ldy, int M, int K) {
    constexpr int COLS = FOLD ? 8 : 16;
    constexpr int ROWS = FOLD ? 8 * MT : 16 * MT;
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

    // the epilogue's per-token scales and bias, fetched first so that the
    // epilogue waits for no global load (entries idx = tid, tid + NW*64)
    constexpr int EPI_IT = (ROWS * COLS + NW * 64 - 1) / (NW * 64);
    float ep_as[EPI_IT], ep_b[EPI_IT], ep_cs[EPI_IT];
    {
        const __amdgpu_buffer_rsrc_t rsT = make_rsrc(a_scale, (int64_t)M * 4);
        const __amdgpu_buffer_rsrc_t rsB =
            epi != EPI_NONE ? make_rsrc(bias + (int64_t)blockIdx.x * COLS, COLS * 2)
                            : make_rsrc(bias, 0);
        const __amdgpu_buffer_rsrc_t rsC =
            colscale ? make_rsrc(colscale + (int64_t)blockIdx.x * COLS, COLS * 4)
                     : make_rsrc(colscale, 0);
#pragma unroll
        for (int it = 0; it < EPI_IT; ++it) {
            const int idx = threadIdx.x + it * NW * 64;
            const int r = idx / COLS, c = idx % COLS;
            const bool ok = idx < ROWS * COLS;
            ep_as[it] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rsT, (ok & (r < M)) ? (uint32_t)(4 * r) : OOB_OFF, 0, 0));
            ep_b[it] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(
                rsB, ok ? (uint32_t)(2 * c) : OOB_OFF, 0, 0));
            const float cs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rsC, ok ? (uint32_t)(4 * c) : OOB_OFF, 0, 0));
            ep_cs[it] = colscale ? cs : 1.0f;
        }
    }

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
            const int k0 = s * KSTEP + half * 128;  // this lane's 128-wide window (unfolded)
            const FoldK fk = fold_k(s * KSTEP, half, g);
            // the block whose scale this lane supplies, and the fp8 operand pieces
            const int kblk = FOLD ? fk.kblk : k0 + 32 * g;
            const int klo = FOLD ? fk.klo : k0 + 16 * g, khi = FOLD ? fk.khi : k0 + 64 + 16 * g;
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
                if (on && kblk < K && WS) sc = wsrow[kblk >> 5];   // no WS: per-channel scales
            }
            wv[u] = pack8(lo, hi);
            wsc[u] = sc;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = FOLD ? (mt * 8 + (i & 7)) : (mt * 16 + i);
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
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[mt][v] += __shfl_down(acc[mt][v], 40, 64);
            if (g < 2 && i < 8) {
#pragma unroll
                for (int v = 0; v < 4; ++v) red[wave][mt * 8 + 4 * g + v][i] = acc[mt][v];
            }
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][mt * 16 + 4 * g + v][i] = acc[mt][v];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < EPI_IT; ++it) {
        const int idx = threadIdx.x + it * NW * 64;
        const int r = idx / COLS, c = idx % COLS;
        if ((idx < ROWS * COLS) & (r < M)) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sum += red[w][r][c];
            const int64_t nn = (int64_t)blockIdx.x * COLS + c;
            Y[(int64_t)r * ldy + nn] =
                (uint16_t)f32_to_bf16(epilogue(sum, ep_as[it], ep_cs[it], ep_b[it], epi));
        }
    }
}

template <bool FP4, bool FOLD, int MT, int NW, int SPW>
void launch_one(const uint8_t *a, int64_t lda, const float *as, const uint8_t *w, int64_t ldw,
                const uint8_t *ws, const float *cs, const uint16_t *bias, int epi, uint16_t *y,
                int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    constexpr int COLS = FOLD ? 8 : 16;
    hipLaunchKernelGGL((gemm_decode_kernel<FP4, FOLD, MT, NW, SPW>), dim3((unsigned)(N / COLS)),
                       dim3(NW * 64), 0, st, a, lda, as, w, ldw, ws, cs, bias, epi, y, ldy, (int)M,
                       (int)K);
}

// Steps per wave held in registers at once: all of a wave's share when it
// fits (at most 8 weight fragments, and at most 8 fragments x M-tiles).
// Folded e4m3 weights take at most 2 (two passes of 2 measured 1.5 % faster
// than one of 4 at M=8, N=2048, K=7168 on MI355X).
template <bool FP4, bool FOLD, int MT, int NW>
void launch_spw(int per_wave, const uint8_t *a, int64_t lda, const float *as, const uint8_t *w,
                int64_t ldw, const uint8_t *ws, const float *cs, const uint16_t *bias, int epi,
                uint16_t *y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    constexpr int CAP = (FOLD && !FP4) ? 2 : 8 / MT;
    if (per_wave <= 1 || CAP == 1)
        launch_one<FP4, FOLD, MT, NW, 1>(a, lda, as, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
    else if (per_wave <= 2 || CAP == 2)
        launch_one<FP4, FOLD, MT, NW, 2>(a, lda, as, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
    else if (per_wave <= 4 || CAP == 4)
        launch_one<FP4, FOLD, MT, NW, (CAP >= 4 ? 4 : 1)>(a, lda, as, w, ldw, ws, cs, bias, epi, y,
                                                          ldy, M, N, K, st);
    else
        launch_one<FP4, FOLD, MT, NW, (CAP >= 8 ? 8 : 1)>(a, lda, as, w, ldw, ws, cs, bias, epi, y,
                                                          ldy, M, N, K, st);
}


// Balanced variant: one workgroup of 16 waves per CU, all of it resident at
// once. Workgroup b owns `gpw` consecutive groups of 8 weight rows; its work
// is the list of (group, 256-k step) units in group-major order, cut into 16
// equal contiguous ranges, one per wave, so every wave has the same number
// of weight loads in flight from the start whatever N / 8 / CUs is. The
// activations (a padded row per token) and the workgroup's E8M0 scales are
// read once per workgroup into LDS, ahead of the weights, so waiting for
// them does not wait for the weight stream. Tokens are folded as in the
// kernel above, MT groups of 8 sharing each weight fragment, but on two
// plain 128-wide halves of each window (the activations come from LDS,
// where the interleaved halves would put two lanes on one bank). Group sums go
// through LDS: a group a wave covers whole as that wave's sum, a group cut
// between waves (a wave's first and last group) as partial sums added in
// wave order; the epilogue runs after every weight has been consumed.
// Needs K % 128 == 0 (scale rows in whole 4-byte words).
constexpr int UNIT_WAVES = 16;

template <bool FP4, int MT, bool FP4A = false>
struct UnitsLds {
    static constexpr int TOK = 8 * MT;
    // a padded activation row per token (fp4 activations: K / 2 bytes, then
    // each token's K / 32 E8M0 bytes after the rows)
    __host__ __device__ static int a_row(int K) { return (FP4A ? K / 2 : K) + 16; }
    __host__ __device__ static size_t a_bytes(int K) {
        return (size_t)TOK * a_row(K) + (FP4A ? (size_t)TOK * (K / 32) : 0);
    }
    // scale rows of the workgroup: one per weight row (fp4) or per 32 rows
    __host__ __device__ static int scale_rows(int gpw) { return FP4 ? 8 * gpw : (8 * gpw + 31) / 32 + 1; }
    // then the sums: one slot per group (groups a wave covers whole) and
    // two per wave (its first and last group, when cut between waves)
    // and the per-token scales, the bias and the per-channel scales of the
    // workgroup's rows
    static size_t bytes(int K, int gpw) {
        return a_bytes(K) + (size_t)scale_rows(gpw) * (K / 32) +
               (size_t)(gpw + UNIT_WAVES * 2) * 64 * MT * sizeof(float) +
               (size_t)(TOK + 16 * gpw) * sizeof(float);
    }
};

// FP4A (W4A4): fp4 activations [M, K/2] with E8M0 scales AS [M, K/32] (rows
// of whole 4-byte words), staged in LDS after the activation rows; no
// per-token scale (a_scale is unused, 1).
template <bool FP4, int MT, int P, bool FP4A = false>
__global__ __launch_bounds__(1024) void gemm_decode_units_kernel(
    const uint8_t *__restrict__ A, int64_t lda, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ W, int64_t ldw, const uint8_t *__restrict__ WS,
    const float *__restrict__ colscale, const uint16_t *__restrict__ bias, int epi,
    uint16_t *__restrict__ Y, int64_t ldy, int M, int N, int K, int gpw,
    const uint8_t *__restrict__ AS = nullptr) {
    using L = UnitsLds<FP4, MT, FP4A>;
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int KSTEP = 256;
    constexpr int TOK = L::TOK;
    constexpr int PE = 64 * MT;                     // partial sums per group (tokens x rows)
    const int lds_row = L::a_row(K);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int col = i & 7, half = i >> 3;
    const int KB = K >> 5;
    const int S = (K + KSTEP - 1) / KSTEP;           // units per group
    const int G = N >> 3;
    const int gb = blockIdx.x * gpw;                 // first group of this workgroup
    const int ng = min(gpw, G - gb);
    const int U = ng * S;
    const int upw = (U + UNIT_WAVES - 1) / UNIT_WAVES;
    const int u0 = min(U, wave * upw), u1 = min(U, u0 + upw);
    const int row0 = gb * 8;                         // the workgroup's first weight row
    const int srow0 = FP4 ? row0 : (row0 >> 5);
    const int nsrows = FP4 ? ng * 8 : ((row0 + ng * 8 - 1) >> 5) - srow0 + 1;
    uint8_t *s_lds = lds + L::a_bytes(K);
    uint8_t *as_lds = lds + (size_t)TOK * lds_row;   // FP4A: [TOK][KB] activation scales
    float *gsum = reinterpret_cast<float *>(s_lds + (size_t)L::scale_rows(gpw) * KB);
    float *part = gsum + gpw * PE;
    float *tok_scale = part + UNIT_WAVES * 2 * PE;   // [TOK]
    float *row_bias = tok_scale + TOK;               // [8 gpw]
    float *row_cs = row_bias + 8 * gpw;              // [8 gpw] per-channel scales (1 if none)

    // ---- activations and scales into registers first, then the weights,
    // then the LDS writes (which wait only for the first two groups of
    // loads). Every load is a range-checked buffer load (reads past a
    // buffer's range return zeros), issued unconditionally, so the compiler
    // counts them exactly and waits for no more than it needs.
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc(A, (int64_t)M * lda);
    // no WS (per-channel scales): an empty range, every scale reads as 0
    const __amdgpu_buffer_rsrc_t rsS =
        WS ? make_rsrc(WS + (int64_t)srow0 * KB, (int64_t)nsrows * KB) : make_rsrc(WS, 0);
    const __amdgpu_buffer_rsrc_t rsW = make_rsrc(W + (int64_t)row0 * ldw, (int64_t)ng * 8 * ldw);
    constexpr int ACH = 8 * MT * (FP4A ? 4096 : 8192) / 16 / 1024;   // 16-byte chunks per thread for K <= 8192
    const int kc = (FP4A ? K >> 1 : K) >> 4, chunks = TOK * kc;
    uint4 av[ACH];
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
        const int c = threadIdx.x + j * 1024;
        const int t = c / kc, k = 16 * (c % kc);
        av[j] = bload16(rsA, ((c < chunks) & (t < M)) ? (uint32_t)(t * lda + k) : OOB_OFF);
    }
    // the epilogue's per-token scales and bias, fetched now so that the
    // epilogue waits for no global load (one value per thread at most)
    // (range-checked buffer loads: branch-free, so the compiler counts them)
    float ep_val, ep_cs;
    {
        const __amdgpu_buffer_rsrc_t rsT = make_rsrc(a_scale, FP4A ? 0 : (int64_t)M * 4);
        const __amdgpu_buffer_rsrc_t rsC =
            colscale ? make_rsrc(colscale + row0, (int64_t)(N - row0) * 4) : make_rsrc(colscale, 0);
        // bias of this workgroup's rows (no bias: an empty range, nothing read)
        const __amdgpu_buffer_rsrc_t rsB =
            epi != EPI_NONE ? make_rsrc(bias + row0, (int64_t)(N - row0) * 2) : make_rsrc(bias, 0);
        const int t = threadIdx.x;
        const uint32_t ts = __builtin_amdgcn_raw_buffer_load_b32(
            rsT, t < TOK ? (uint32_t)(4 * t) : OOB_OFF, 0, 0);
        const uint32_t bb = __builtin_amdgcn_raw_buffer_load_b16(
            rsB, ((t >= TOK) & (t < TOK + 8 * ng)) ? (uint32_t)(2 * (t - TOK)) : OOB_OFF, 0, 0);
        ep_val = t < TOK ? (FP4A ? 1.0f : __uint_as_float(ts)) : bf16_to_f32(bb);
        const uint32_t cw = __builtin_amdgcn_raw_buffer_load_b32(
            rsC, t < 8 * ng ? (uint32_t)(4 * t) : OOB_OFF, 0, 0);
        ep_cs = colscale ? __uint_as_float(cw) : 1.0f;
    }
    const int words = nsrows * (KB >> 2);
    constexpr int SCW = 8;                           // scale words per thread (the launcher checks the bound)
    // FP4A: the activation scale rows, one 4-byte word per thread at most
    // (TOK * K / 128 <= 1024 words for K <= 8192)
    uint32_t asv = 0;
    const int awords = TOK * (KB >> 2);
    if (FP4A) {
        const __amdgpu_buffer_rsrc_t rsAS = make_rsrc(AS, (int64_t)M * KB);
        const int c = threadIdx.x, t = c / (KB >> 2);
        asv = __builtin_amdgcn_raw_buffer_load_b32(
            rsAS, ((c < awords) & (t < M)) ? (uint32_t)(4 * c) : OOB_OFF, 0, 0);
    }
    uint32_t sv[SCW];
#pragma unroll
    for (int j = 0; j < SCW; ++j) {
        const int c = threadIdx.x + j * 1024;
        sv[j] = __builtin_amdgcn_raw_buffer_load_b32(rsS, c < words ? (uint32_t)(4 * c) : OOB_OFF,
                                                     0, 0);
    }

    // keep the weight loads behind the activation and scale loads, so that
    // waiting for those two does not wait for any weights
    __builtin_amdgcn_sched_barrier(0);

    // weights: a rolling window of WIN units in flight per wave (slot q % WIN);
    // (gl, st) of the next unit to load, advanced without division
    constexpr int WIN = FP4 ? 12 : 6;   // 12 KB (fp4) or 12 KB (e4m3) per wave
    uint4 wlo[WIN], whi[FP4 ? 1 : WIN];
    const int gl0 = u0 / S, st0 = u0 - gl0 * S;
    int lgl = gl0, lst = st0;
    auto load_unit = [&](int q) {
        const bool on = u0 + q < u1;
        const int k0 = lst * KSTEP + half * 128;
        const int kblk = k0 + 32 * g, klo = k0 + 16 * g, khi = k0 + 64 + 16 * g;
        const uint32_t rowoff = (uint32_t)((lgl * 8 + col) * ldw);
        if (FP4) {
            wlo[q % WIN] = bloadw16<true>(rsW, (on & (kblk < K)) ? rowoff + (kblk >> 1) : OOB_OFF);
        } else {
            wlo[q % WIN] = bloadw16<true>(rsW, (on & (klo < K)) ? rowoff + klo : OOB_OFF);
            whi[q % WIN] = bloadw16<true>(rsW, (on & (khi < K)) ? rowoff + khi : OOB_OFF);
        }
        if (++lst == S) { lst = 0; ++lgl; }
    };
#pragma unroll
    for (int q = 0; q < (P < WIN ? P : WIN); ++q) load_unit(q);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < ACH; ++j) {
        const int c = threadIdx.x + j * 1024;
        const int t = c / kc, k = 16 * (c % kc);
        if (c < chunks) *reinterpret_cast<uint4 *>(lds + t * lds_row + k) = av[j];
    }
#pragma unroll
    for (int j = 0; j < SCW; ++j) {
        const int c = threadIdx.x + j * 1024;
        if (c < words) *reinterpret_cast<uint32_t *>(s_lds + 4 * c) = sv[j];
    }
    if (FP4A && (int)threadIdx.x < awords) *reinterpret_cast<uint32_t *>(as_lds + 4 * threadIdx.x) = asv;
    if (threadIdx.x < TOK + 8 * ng) tok_scale[threadIdx.x] = ep_val;   // row_bias follows tok_scale
    if (threadIdx.x < 8 * ng) row_cs[threadIdx.x] = ep_cs;
    __syncthreads();

    // ---- this wave's units; a group's sum is flushed when the next group
    // starts and at the end
    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    auto flush = [&](int gl, int cover0, int cover1) {
        // fold: lanes g < 2, i < 8 hold tokens 8 mt + 4 g + v of row 8 gl + i
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[mt][v] += __shfl_down(acc[mt][v], 40, 64);
        // sums only go to LDS here: an epilogue's global loads (scales,
        // bias) would make the compiler wait for the whole weight window
        const bool whole = cover0 == gl * S && cover1 == (gl + 1) * S;
        if ((g < 2) & (i < 8)) {
            float *dst = whole ? gsum + gl * PE : part + (wave * 2 + (gl == gl0 ? 0 : 1)) * PE;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) dst[(mt * 8 + 4 * g + v) * 8 + i] = acc[mt][v];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    };
    int cgl = gl0, cst = st0, start = u0;   // (group, step) of the unit consumed next
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int u = u0 + q;
        if (u < u1) {
            if (cst == 0 && u != u0) {   // uniform: the previous group ended
                flush(cgl - 1, start, u);
                start = u;
            }
            const int k0 = cst * KSTEP + half * 128;
            const int kblk = k0 + 32 * g, klo = k0 + 16 * g, khi = k0 + 64 + 16 * g;
            const int srl = FP4 ? cgl * 8 + col : ((row0 + cgl * 8 + col) >> 5) - srow0;
            const int sc = (kblk < K) & (WS != nullptr) ? s_lds[srl * KB + (kblk >> 5)] : E8M0_ONE;
            const v8i wv = pack8(wlo[q % WIN], FP4 ? make_uint4(0u, 0u, 0u, 0u) : whi[FP4 ? 0 : q % WIN]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint8_t *arow = lds + (mt * 8 + col) * lds_row;
                uint4 alo = make_uint4(0u, 0u, 0u, 0u), ahi = alo;
                if (FP4A) {   // 32 fp4 values at kblk and their scale byte
                    int sa = E8M0_ONE;
                    if (kblk < K) {
                        alo = *reinterpret_cast<const uint4 *>(arow + (kblk >> 1));
                        sa = as_lds[(mt * 8 + col) * KB + (kblk >> 5)];
                    }
                    acc[mt] = mfma16x<FP4, true>(pack8(alo, ahi), wv, acc[mt], sa, sc);
                } else {
                    if (klo < K) alo = *reinterpret_cast<const uint4 *>(arow + klo);
                    if (khi < K) ahi = *reinterpret_cast<const uint4 *>(arow + khi);
                    acc[mt] = mfma16<FP4>(pack8(alo, ahi), wv, acc[mt], E8M0_ONE, sc);
                }
            }
            if (++cst == S) { cst = 0; ++cgl; }
        }
        if (q + WIN < P) load_unit(q + WIN);   // refill the slot just used
    }
    if (u0 < u1) flush(cst == 0 ? cgl - 1 : cgl, start, u1);
    __syncthreads();

    // ---- epilogue: a group's sum is its whole-owner's, or the partial sums
    // of the waves it was cut between, added in wave order
    // The waves holding group gl's units [gl S, gl S + S) are w0 .. w1 (the
    // ranges are contiguous, upw units each); if w0 == w1 it is whole. A cut
    // group is the first group of waves w0 + 1 .. w1 (slot 0), and of w0 too
    // if w0's range starts at the group's first unit, else w0's last (slot 1).
    for (int t = threadIdx.x; t < ng * PE; t += 1024) {
        const int gl = t / PE, e = t % PE;
        const int w0 = (gl * S) / upw, w1 = (gl * S + S - 1) / upw;
        float sum;
        if (w0 == w1) {
            sum = gsum[gl * PE + e];
        } else {
            sum = part[(w0 * 2 + (w0 * upw >= gl * S ? 0 : 1)) * PE + e];
            for (int w = w0 + 1; w <= w1; ++w) sum += part[(w * 2) * PE + e];
        }
        const int m = e / 8, r = e % 8;
        if (m >= M) continue;
        const int64_t nn = (int64_t)row0 + gl * 8 + r;
        Y[(int64_t)m * ldy + nn] = (uint16_t)f32_to_bf16(
            epilogue(sum, tok_scale[m], row_cs[gl * 8 + r], row_bias[gl * 8 + r], epi));
    }
}

template <bool FP4, int MT, int P, bool FP4A = false>
void launch_units(const uint8_t *a, int64_t lda, const float *as, const uint8_t *w, int64_t ldw,
                  const uint8_t *ws, const float *cs, const uint16_t *bias, int epi, uint16_t *y,
                  int64_t ldy, int64_t M, int64_t N, int64_t K, int gpw, hipStream_t st,
                  const uint8_t *a_e8m0 = nullptr) {
    const size_t lds = UnitsLds<FP4, MT, FP4A>::bytes((int)K, gpw);
    const int64_t groups = N / 8;
    hipLaunchKernelGGL((gemm_decode_units_kernel<FP4, MT, P, FP4A>),
                       dim3((unsigned)((groups + gpw - 1) / gpw)), dim3(1024), lds, st, a, lda, as,
                       w, ldw, ws, cs, bias, epi, y, ldy, (int)M, (int)N, (int)K, gpw, a_e8m0);
}


// The units kernel's instantiation for a wave's unit count: windows of 4, 8
// and 16 units for both weight formats, 24 and 32 for MXFP4 weights only
// (their e4m3 window would not fit the register budget; the caller keeps
// e4m3 at 16 units a wave, and any other count is refused here).
template <bool FP4, int MT>
hipError_t launch_units_upw(int64_t upw, const uint8_t *a, int64_t lda, const float *as,
                            const uint8_t *w, int64_t ldw, const uint8_t *ws, const float *cs,
                            const uint16_t *bias, int epi, uint16_t *y, int64_t ldy, int64_t M,
                            int64_t N, int64_t K, int gpw, hipStream_t st) {
    if (upw <= 4) launch_units<FP4, MT, 4>(a, lda, as, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, gpw, st);
    else if (upw <= 8) launch_units<FP4, MT, 8>(a, lda, as, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, gpw, st);
    else if (upw <= 16) launch_units<FP4, MT, 16>(a, lda, as, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, gpw, st);
    else {
        if constexpr (FP4) {
            if (upw <= 24) launch_units<FP4, MT, 24>(a, lda, as, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, gpw, st);
            else if (upw <= 32) launch_units<FP4, MT, 32>(a, lda, as, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, gpw, st);
            else return hipErrorInvalidValue;
        } else {
            return hipErrorInvalidValue;
        }
    }
    return hipSuccess;
}

// The units kernel stages its epilogue operands (TOK per-token scales, then
// the bias and the channel scales of its 8 gpw rows) one entry per thread of
// its 1024.
inline bool units_epilogue_fits(int mt, int gpw) { return 8 * mt + 8 * gpw <= 1024; }

// ---------------------------------------------------------------------------
// Split-K decode for 16 < M <= 64 on narrow layers. With every workgroup on
// all of K, each one would read all M x K activations (M/8 times the bytes
// of its 8-row weight slice at M = 64); here a workgroup takes 64 weight
// rows and a 1/S slice of K, with the activations' slice staged once in LDS,
// so activations and weights cost about the same. Partial sums go to the
// caller's workspace as fp32 [S][M][N]; a second kernel adds the S slices
// in order and applies the epilogue.
constexpr int SPLIT_MAX_STEPS = 8;   // 128-k steps per split at most

// Splits of K: enough workgroups to cover the CUs for a 256-CU part, and at
// most SPLIT_MAX_STEPS steps of 128 k each.
__host__ __device__ inline int64_t decode_splits(int64_t N, int64_t K) {
    const int64_t steps = (K + 127) / 128, blocks = (N + 63) / 64;
    int64_t s = blocks >= 256 ? 1 : 256 / blocks;
    const int64_t min_s = (steps + SPLIT_MAX_STEPS - 1) / SPLIT_MAX_STEPS;
    if (s < min_s) s = min_s;
    if (s > steps) s = steps;
    return s;
}

// 2 <= M <= 8 on a layer of at least 2^26 weights (when the wide-layer
// kernel does not take it): the folded kernel's workgroups would each read
// M x K activation bytes for 8 x K weight bytes; split-K reads M/8 of that
// per 64 rows and its second launch is small against a long first one.
__host__ __device__ inline bool large_splitk(int64_t M, int64_t N, int64_t K) {
    return M >= 2 && M <= 8 && N * K >= ((int64_t)1 << 26);
}

// FP4A (W4A4): the activations are fp4 [M, K/2] with E8M0 scales AS
// [M, K/32], staged in LDS as packed bytes plus a 32-byte scale row per token.
template <bool FP4, int MT, bool FP4A = false, bool NTW = false>
__global__ __launch_bounds__(256) void gemm_decode_splitk_kernel(
    const uint8_t *__restrict__ A, int64_t lda, const uint8_t *__restrict__ W, int64_t ldw,
    const uint8_t *__restrict__ WS, float *__restrict__ part, int M, int N, int K, int S,
    const uint8_t *__restrict__ AS = nullptr) {
    extern __shared__ __align__(16) uint8_t lds[];   // [16 MT][span + 16] activations (+ scales)
    constexpr int TOK = 16 * MT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int KB = K >> 5;
    const int steps = (K + 127) / 128;
    const int per = (steps + S - 1) / S;
    const int sp = blockIdx.y;
    const int st0 = min(steps, sp * per), st1 = min(steps, st0 + per);
    const int kbeg = st0 * 128;
    const int span = per * (FP4A ? 64 : 128);         // bytes of k per token staged
    const int lds_row = span + 16;
    constexpr int SROW = SPLIT_MAX_STEPS * 4;          // FP4A: scale bytes per token
    uint8_t *s_lds = lds + TOK * lds_row;
    const int row0 = blockIdx.x * 64;
    const int n = row0 + 16 * wave + i;               // this lane's weight row

    // ---- activations' K slice: registers first, weights next, then LDS
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc(A, (int64_t)M * lda);
    constexpr int ACH = TOK * SPLIT_MAX_STEPS * 128 / 16 / 256;   // 16-byte chunks per thread
    const int kc = span >> 4, chunks = TOK * kc;
    uint4 av[ACH];
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
        const int c = threadIdx.x + j * 256;
        const int t = c / kc;
        // element and byte offset of this chunk (fp4: 32 elements in 16 bytes)
        const int ke = kbeg + (FP4A ? 32 : 16) * (c % kc);
        const int kb = FP4A ? (kbeg >> 1) + 16 * (c % kc) : ke;
        av[j] = bload16(rsA, ((c < chunks) & (t < M) & (ke < K)) ? (uint32_t)(t * lda + kb) : OOB_OFF);
    }
    constexpr int SCH = FP4A ? TOK * SROW / 256 : 1;   // activation scale bytes per thread
    uint32_t asv[SCH];
    if (FP4A) {
        const __amdgpu_buffer_rsrc_t rsSA = make_rsrc(AS, (int64_t)M * KB);
#pragma unroll
        for (int j = 0; j < SCH; ++j) {
            const int c = threadIdx.x + j * 256;
            const int t = c / SROW, b = c % SROW, blk = (kbeg >> 5) + b;
            asv[j] = __builtin_amdgcn_raw_buffer_load_b8(
                rsSA, ((t < M) & (b < 4 * (st1 - st0)) & (blk < KB)) ? (uint32_t)(t * KB + blk) : OOB_OFF,
                0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- this wave's weights: SPLIT_MAX_STEPS steps (16x16x128 B operand)
    const __amdgpu_buffer_rsrc_t rsW = make_rsrc(W + (int64_t)row0 * ldw, (int64_t)(N - row0) * ldw);
    const __amdgpu_buffer_rsrc_t rsS =
        !WS ? make_rsrc(WS, 0)   // per-channel scales: no E8M0 bytes
        : FP4 ? make_rsrc(WS + (int64_t)row0 * KB, (int64_t)(N - row0) * KB)
              : make_rsrc(WS + (int64_t)(row0 >> 5) * KB, (int64_t)((N >> 5) - (row0 >> 5)) * KB);
    const uint32_t wrow = (uint32_t)((16 * wave + i) * ldw);
    const uint32_t srow = (uint32_t)((FP4 ? (16 * wave + i) : ((n >> 5) - (row0 >> 5))) * KB);
    uint4 wlo[SPLIT_MAX_STEPS], whi[FP4 ? 1 : SPLIT_MAX_STEPS];
    uint32_t wsc[SPLIT_MAX_STEPS];
#pragma unroll
    for (int u = 0; u < SPLIT_MAX_STEPS; ++u) {
        const int kk = (st0 + u) * 128;
        const bool on = (st0 + u < st1) & (n < N);
        const int kblk = kk + 32 * g, klo = kk + 16 * g, khi = kk + 64 + 16 * g;
        if (FP4) {
            wlo[u] = bloadw16<NTW>(rsW, (on & (kblk < K)) ? wrow + (kblk >> 1) : OOB_OFF);
        } else {
            wlo[u] = bloadw16<NTW>(rsW, (on & (klo < K)) ? wrow + klo : OOB_OFF);
            whi[u] = bloadw16<NTW>(rsW, (on & (khi < K)) ? wrow + khi : OOB_OFF);
        }
        wsc[u] = __builtin_amdgcn_raw_buffer_load_b8(rsS, (on & (kblk < K)) ? srow + (kblk >> 5) : OOB_OFF,
                                                     0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < ACH; ++j) {
        const int c = threadIdx.x + j * 256;
        const int t = c / kc, k = 16 * (c % kc);
        if (c < chunks) *reinterpret_cast<uint4 *>(lds + t * lds_row + k) = av[j];
    }
    if (FP4A) {
#pragma unroll
        for (int j = 0; j < SCH; ++j) s_lds[threadIdx.x + j * 256] = (uint8_t)asv[j];
    }
    __syncthreads();

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < SPLIT_MAX_STEPS; ++u) {
        if (st0 + u < st1) {   // uniform
            const int kl = u * (FP4A ? 64 : 128);        // offset in the staged slice
            const v8i wv = pack8(wlo[u], FP4 ? make_uint4(0u, 0u, 0u, 0u) : whi[FP4 ? 0 : u]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint8_t *arow = lds + (mt * 16 + i) * lds_row + kl;
                if (FP4A) {
                    const v8i a8 = pack8(*reinterpret_cast<const uint4 *>(arow + 16 * g),
                                         make_uint4(0u, 0u, 0u, 0u));
                    const int sa = s_lds[(mt * 16 + i) * SROW + 4 * u + g];
                    acc[mt] = mfma16x<FP4, true>(a8, wv, acc[mt], sa, (int)wsc[u]);
                } else {
                    const v8i a8 = pack8(*reinterpret_cast<const uint4 *>(arow + 16 * g),
                                         *reinterpret_cast<const uint4 *>(arow + 64 + 16 * g));
                    acc[mt] = mfma16<FP4>(a8, wv, acc[mt], E8M0_ONE, WS ? (int)wsc[u] : E8M0_ONE);
                }
            }
        }
    }
    // D: lane l = i + 16 g, VGPR v -> token 16 mt + 4 g + v, weight row n
    if (n < N) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = mt * 16 + 4 * g + v;
                if (t < M) part[((int64_t)sp * M + t) * N + n] = acc[mt][v];
            }
    }
}

// Y[m, n] = epilogue(sum over the S slices in order (fp32), a_scale[m], bias[n]);
// four columns per thread, eight slices' loads in flight before their adds.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part,
                                                            const float *__restrict__ a_scale,
                                                            const float *__restrict__ colscale,
                                                            const uint16_t *__restrict__ bias,
                                                            int epi, uint16_t *__restrict__ Y,
                                                            int64_t ldy, int M, int N, int S) {
    const int n4 = N >> 2;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)M * n4) return;
    const int t = (int)(idx / n4), c0 = 4 * (int)(idx % n4);
    const int64_t slice = (int64_t)M * N;
    const float *p = part + (int64_t)t * N + c0;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = 0;
    for (; s + 8 <= S; s += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4 *>(p + (s + u) * slice);
#pragma unroll
        for (int u = 0; u < 8; ++u) { sum.x += v[u].x; sum.y += v[u].y; sum.z += v[u].z; sum.w += v[u].w; }
    }
    for (; s < S; ++s) {
        const float4 v = *reinterpret_cast<const float4 *>(p + s * slice);
        sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
    }
    float4 bq = make_float4(0.f, 0.f, 0.f, 0.f);
    if (epi != EPI_NONE)   // bias is only 2-byte aligned
        bq = make_float4(bf16_to_f32(bias[c0]), bf16_to_f32(bias[c0 + 1]),
                         bf16_to_f32(bias[c0 + 2]), bf16_to_f32(bias[c0 + 3]));
    const float as = a_scale ? a_scale[t] : 1.0f;   // W4A4: the scales are in the blocks
    const float4 cq = colscale ? *reinterpret_cast<const float4 *>(colscale + c0)
                               : make_float4(1.f, 1.f, 1.f, 1.f);
    const uint32_t o01 = pack_bf16x2(epilogue(sum.x, as, cq.x, bq.x, epi),
                                     epilogue(sum.y, as, cq.y, bq.y, epi));
    const uint32_t o23 = pack_bf16x2(epilogue(sum.z, as, cq.z, bq.z, epi),
                                     epilogue(sum.w, as, cq.w, bq.w, epi));
    *reinterpret_cast<uint2 *>(Y + (int64_t)t * ldy + c0) = make_uint2(o01, o23);
}

template <bool FP4, int MT, bool FP4A = false>
hipError_t launch_splitk(const uint8_t *a, int64_t lda, const float *as, const uint8_t *w,
                         int64_t ldw, const uint8_t *ws, const float *cs, const uint16_t *bias,
                         int epi, uint16_t *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                         float *part, hipStream_t st, const uint8_t *a_e8m0 = nullptr) {
    const int64_t S = decode_splits(N, K);
    const int64_t steps = (K + 127) / 128, per = (steps + S - 1) / S;
    const size_t lds = (size_t)16 * MT * (per * (FP4A ? 64 : 128) + 16) +
                       (FP4A ? (size_t)16 * MT * SPLIT_MAX_STEPS * 4 : 0);
    // streaming weight loads below 2^26 weights only (see bloadw16)
    auto kern = N * K >= ((int64_t)1 << 26) ? gemm_decode_splitk_kernel<FP4, MT, FP4A, false>
                                            : gemm_decode_splitk_kernel<FP4, MT, FP4A, true>;
    hipLaunchKernelGGL(kern,
                       dim3((unsigned)((N + 63) / 64), (unsigned)S), dim3(256), lds, st, a, lda, w,
                       ldw, ws, part, (int)M, (int)N, (int)K, (int)S, a_e8m0);
    const int64_t quads = M * N / 4;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st,
                       part, as, cs, bias, epi, y, ldy, (int)M, (int)N, (int)S);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_decode(bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                              const uint8_t *w, int64_t ldw, const uint8_t *ws, const float *cs,
                              const uint16_t *bias, int epi, uint16_t *y, int64_t ldy, int64_t M,
                              int64_t N, int64_t K, void *workspace, int num_cus, hipStream_t st) {
    constexpr int NW = 8;
    // Balanced units kernel for wide layers (at least two 8-row groups per
    // CU; below that the split-K kernel, which reads its activations straight
    // into registers, is faster): one workgroup per CU, groups split evenly,
    // when the activations and scales fit in LDS and the scale rows are
    // whole, aligned 4-byte words.
    const int64_t groups = N / 8;
    const int gpw = (int)((groups + num_cus - 1) / num_cus);
    if (M <= 16 && gpw >= 2 && K % 128 == 0 && K <= 8192 &&
        (reinterpret_cast<uintptr_t>(ws) & 3u) == 0) {
        const int64_t S = (K + 255) / 256;
        const int64_t upw = (gpw * S + UNIT_WAVES - 1) / UNIT_WAVES;
        const int mt = M <= 8 ? 1 : 2;
        const size_t lds = mt == 1 ? UnitsLds<true, 1>::bytes((int)K, gpw)
                                   : UnitsLds<true, 2>::bytes((int)K, gpw);
        const size_t lds8 = mt == 1 ? UnitsLds<false, 1>::bytes((int)K, gpw)
                                    : UnitsLds<false, 2>::bytes((int)K, gpw);
        const int64_t scale_words = (fp4 ? 8 * gpw : (8 * gpw + 31) / 32 + 1) * (K / 128);
        if (upw <= (fp4 ? 32 : 16) && (fp4 ? lds : lds8) <= 160 * 1024 && scale_words <= 8 * 1024 &&
            units_epilogue_fits(mt, gpw)) {
            const hipError_t e =
                fp4 ? (mt == 1 ? launch_units_upw<true, 1>(upw, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, gpw, st)
                               : launch_units_upw<true, 2>(upw, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, gpw, st))
                    : (mt == 1 ? launch_units_upw<false, 1>(upw, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, gpw, st)
                               : launch_units_upw<false, 2>(upw, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, gpw, st));
            if (e != hipSuccess) return e;
            return hipGetLastError();
        }
    }
    if (M <= 8 && !large_splitk(M, N, K)) {
        // 16 waves a workgroup for one or two tokens on a layer of at most
        // two workgroups per CU, 8 otherwise (measured on the 2048 x 7168
        // layer: M = 1 5.25 against 5.47 us, M = 2 5.45 against 5.61; M = 4
        // 5.82 against 5.74, M = 8 6.41 against 6.23; on the 248320 x 5120
        // lm_head at M = 1, 324 against 219 us)
        if (M <= 2 && N / 8 <= 2 * (int64_t)num_cus) {
            constexpr int NW16 = 16;
            const int per = (int)(((K + 255) / 256 + NW16 - 1) / NW16);
            if (fp4)
                launch_spw<true, true, 1, NW16>(per, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
            else
                launch_spw<false, true, 1, NW16>(per, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
            return hipGetLastError();
        }
        const int per = (int)(((K + 255) / 256 + NW - 1) / NW);
        if (fp4)
            launch_spw<true, true, 1, NW>(per, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
        else
            launch_spw<false, true, 1, NW>(per, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
        return hipGetLastError();
    }
    if (M <= 16 && !large_splitk(8, N, K)) {
        // two folded 8-token groups on each weight fragment: every workgroup
        // reads M x K activation bytes (up to twice its weight slice, from
        // L2), against a second launch and fp32 partial sums for split-K
        // (measured on the 2048 x 7168 layer: M = 12 7.39 against 8.27 us,
        // M = 15 8.09-8.14 against 8.29-8.32, M = 16 8.33-8.38 either way;
        // the re-read grows with M). On a layer of at most two workgroups
        // per CU, 16 waves a workgroup, so that a wave's two steps are one
        // pass (M = 16: 8.04-8.11 against 8.35-8.36 us with 8 waves in two
        // passes; at M = 8 the single group keeps 8 waves, 6.27 against 6.35
        // with 16)
        if (N / 8 <= 2 * (int64_t)num_cus) {
            constexpr int NW16 = 16;
            const int per = (int)(((K + 255) / 256 + NW16 - 1) / NW16);
            if (fp4)
                launch_spw<true, true, 2, NW16>(per, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
            else
                launch_spw<false, true, 2, NW16>(per, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
            return hipGetLastError();
        }
        const int per = (int)(((K + 255) / 256 + NW - 1) / NW);
        if (fp4)
            launch_spw<true, true, 2, NW>(per, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
        else
            launch_spw<false, true, 2, NW>(per, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st);
        return hipGetLastError();
    }
    // 16 < M <= 64, or 2 <= M <= 16 on a large layer: split K over
    // workgroups, partial sums in the workspace
    float *part = static_cast<float *>(workspace);
    switch ((M + 15) / 16) {
    case 1: return fp4 ? launch_splitk<true, 1>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, part, st)
                       : launch_splitk<false, 1>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, part, st);
    case 2: return fp4 ? launch_splitk<true, 2>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, part, st)
                       : launch_splitk<false, 2>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, part, st);
    case 3: return fp4 ? launch_splitk<true, 3>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, part, st)
                       : launch_splitk<false, 3>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, part, st);
    default: return fp4 ? launch_splitk<true, 4>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, part, st)
                        : launch_splitk<false, 4>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, part, st);
    }
}

// ---------------------------------------------------------------------------
// Grouped (MoE) decode: one launch over (8-row weight group) x expert.
// Expert e's token rows are [off[e], off[e+1]) of A, sorted by expert; a
// workgroup of 8 waves (K split between them, folded layout as above)
// streams its 8 weight rows of expert e once and applies them to up to G
// folded 8-token groups per pass; more tokens take further passes (the rows
// come back from L2). Experts without rows exit at once. Offsets are read on
// the device and clamped to [0, T], so any offsets stay inside A and Y.
template <bool FP4, int G>
__global__ __launch_bounds__(512) void gemm_grouped_decode_kernel(
    const uint8_t *__restrict__ A, int64_t lda, const float *__restrict__ a_scale,
    const int32_t *__restrict__ off, const uint8_t *__restrict__ W, int64_t ldw,
    int64_t w_estride, const uint8_t *__restrict__ WS, const uint16_t *__restrict__ bias, int epi,
    uint16_t *__restrict__ Y, int64_t ldy, int T, int N, int K) {
    constexpr int NW = 8, COLS = 8, KSTEP = 256;
    __shared__ float red[NW][G][8][COLS + 1];
    const int e = blockIdx.y;
    const int r0 = min(max(off[e], 0), T);
    const int r1 = max(r0, min(off[e + 1], T));
    if (r0 == r1) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int col = i & 7, half = i >> 3;
    const int KB = K >> 5;
    const int nsteps = (K + KSTEP - 1) / KSTEP;
    const int64_t n = (int64_t)blockIdx.x * COLS + col;   // this lane's weight row
    const uint8_t *wrow = W + (int64_t)e * w_estride + n * ldw;
    const uint8_t *wsrow = FP4 ? WS + ((int64_t)e * N + n) * KB
                               : WS + ((int64_t)e * (N >> 5) + (n >> 5)) * KB;
    const uint16_t *bias_e = bias ? bias + (int64_t)e * N : nullptr;

    for (int p0 = r0; p0 < r1; p0 += 8 * G) {
        v4f acc[G];
#pragma unroll
        for (int q = 0; q < G; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int s = wave; s < nsteps; s += NW) {
            const FoldK fk = fold_k(s * KSTEP, half, g);
            const int kblk = fk.kblk, klo = fk.klo, khi = fk.khi;
            uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
            int sc = E8M0_ONE;
            if (FP4) {
                if (kblk < K) {
                    lo = ldgw16_nt(wrow + (kblk >> 1));
                    sc = wsrow[kblk >> 5];
                }
            } else {
                if (klo < K) lo = ldgw16_nt(wrow + klo);
                if (khi < K) hi = ldgw16_nt(wrow + khi);
                if (kblk < K) sc = wsrow[kblk >> 5];
            }
            const v8i wv = pack8(lo, hi);
#pragma unroll
            for (int q = 0; q < G; ++q) {
                const int m = p0 + 8 * q + (i & 7);
                uint4 alo = make_uint4(0u, 0u, 0u, 0u), ahi = alo;
                if (m < r1) {
                    const uint8_t *arow = A + (int64_t)m * lda;
                    if (klo < K) alo = ldg16(arow + klo);
                    if (khi < K) ahi = ldg16(arow + khi);
                }
                acc[q] = mfma16<FP4>(pack8(alo, ahi), wv, acc[q], E8M0_ONE, sc);
            }
        }
        // the two diagonal 8x8 blocks (K halves) meet in lanes g < 2, i < 8
#pragma unroll
        for (int q = 0; q < G; ++q) {
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[q][v] += __shfl_down(acc[q][v], 40, 64);
            if (g < 2 && i < 8) {
#pragma unroll
                for (int v = 0; v < 4; ++v) red[wave][q][4 * g + v][i] = acc[q][v];
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < G * 8 * COLS; idx += NW * 64) {
            const int q = idx / (8 * COLS), r = (idx / COLS) % 8, c = idx % COLS;
            const int m = p0 + 8 * q + r;
            if (m < r1) {
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) sum += red[w][q][r][c];
                const int64_t nn = (int64_t)blockIdx.x * COLS + c;
                const float b = (epi != EPI_NONE) ? bf16_to_f32(bias_e[nn]) : 0.f;
                Y[(int64_t)m * ldy + nn] = (uint16_t)f32_to_bf16(epilogue(sum, a_scale[m], b, epi));
            }
        }
        __syncthreads();   // red is reused by the next pass
    }
}

// W4A4 decode (fp4 activations staged with their scales; no per-token
// scale): on wide layers with M <= 16 the balanced units kernel, under the
// same conditions as for W4A8 (and 4-byte aligned activation scale rows);
// otherwise the split-K kernel, for every M <= DECODE_MAX_M.
hipError_t launch_gemm_decode_w4a4(const uint8_t *a, int64_t lda, const uint8_t *a_e8m0,
                                   const uint8_t *w, int64_t ldw, const uint8_t *ws,
                                   const uint16_t *bias, int epi, uint16_t *y, int64_t ldy,
                                   int64_t M, int64_t N, int64_t K, void *workspace,
                                   int num_cus, hipStream_t st) {
    const int64_t groups = N / 8;
    const int gpw = (int)((groups + num_cus - 1) / num_cus);
    if (M <= 16 && gpw >= 2 && K % 128 == 0 && K <= 8192 &&
        (reinterpret_cast<uintptr_t>(ws) & 3u) == 0 && (reinterpret_cast<uintptr_t>(a_e8m0) & 3u) == 0) {
        const int64_t S = (K + 255) / 256;
        const int64_t upw = (gpw * S + UNIT_WAVES - 1) / UNIT_WAVES;
        const int mt = M <= 8 ? 1 : 2;
        const size_t lds = mt == 1 ? UnitsLds<true, 1, true>::bytes((int)K, gpw)
                                   : UnitsLds<true, 2, true>::bytes((int)K, gpw);
        const int64_t scale_words = 8 * gpw * (K / 128);
        if (upw <= 32 && lds <= 160 * 1024 && scale_words <= 8 * 1024 && units_epilogue_fits(mt, gpw)) {
#define BSG_UNITS4(MT_)                                                                            \
    if (upw <= 8) launch_units<true, MT_, 8, true>(a, lda, nullptr, w, ldw, ws, nullptr, bias, epi, y, ldy, M, N, K, gpw, st, a_e8m0); \
    else if (upw <= 16) launch_units<true, MT_, 16, true>(a, lda, nullptr, w, ldw, ws, nullptr, bias, epi, y, ldy, M, N, K, gpw, st, a_e8m0); \
    else if (upw <= 24) launch_units<true, MT_, 24, true>(a, lda, nullptr, w, ldw, ws, nullptr, bias, epi, y, ldy, M, N, K, gpw, st, a_e8m0); \
    else launch_units<true, MT_, 32, true>(a, lda, nullptr, w, ldw, ws, nullptr, bias, epi, y, ldy, M, N, K, gpw, st, a_e8m0);
            if (mt == 1) { BSG_UNITS4(1) } else { BSG_UNITS4(2) }
#undef BSG_UNITS4
            return hipGetLastError();
        }
    }
    float *part = static_cast<float *>(workspace);
    switch ((M + 15) / 16) {
    case 1: return launch_splitk<true, 1, true>(a, lda, nullptr, w, ldw, ws, nullptr, bias, epi, y, ldy, M, N, K, part, st, a_e8m0);
    case 2: return launch_splitk<true, 2, true>(a, lda, nullptr, w, ldw, ws, nullptr, bias, epi, y, ldy, M, N, K, part, st, a_e8m0);
    case 3: return launch_splitk<true, 3, true>(a, lda, nullptr, w, ldw, ws, nullptr, bias, epi, y, ldy, M, N, K, part, st, a_e8m0);
    default: return launch_splitk<true, 4, true>(a, lda, nullptr, w, ldw, ws, nullptr, bias, epi, y, ldy, M, N, K, part, st, a_e8m0);
    }
}

hipError_t launch_gemm_grouped(bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                               const int32_t *offsets, int64_t E, int64_t max_rows,
                               const uint8_t *w, int64_t ldw, int64_t w_estride,
                               const uint8_t *ws, const uint16_t *bias, int epi, uint16_t *y,
                               int64_t ldy, int64_t T, int64_t N, int64_t K, hipStream_t st) {
    if (fp4 && max_rows > GROUPED_DECODE_MAX_ROWS && K % 64 == 0)
        return launch_gemm_grouped_prefill(a, lda, a_scale, offsets, E, max_rows, w, ldw, w_estride,
                                           ws, bias, epi, y, ldy, T, N, K, st);
    const dim3 grid((unsigned)(N / 8), (unsigned)E);
#define BSG_GROUPED(FP4_, G_)                                                                      \
    hipLaunchKernelGGL((gemm_grouped_decode_kernel<FP4_, G_>), grid, dim3(512), 0, st, a, lda,      \
                       a_scale, offsets, w, ldw, w_estride, ws, bias, epi, y, ldy, (int)T, (int)N,  \
                       (int)K)
    if (max_rows <= 8) { if (fp4) BSG_GROUPED(true, 1); else BSG_GROUPED(false, 1); }
    else if (max_rows <= 16) { if (fp4) BSG_GROUPED(true, 2); else BSG_GROUPED(false, 2); }
    else { if (fp4) BSG_GROUPED(true, 4); else BSG_GROUPED(false, 4); }
#undef BSG_GROUPED
    return hipGetLastError();
}

size_t decode_workspace_bytes_w4a4(int64_t M, int64_t N, int64_t K) {
    if (M > DECODE_MAX_M) return 0;
    return (size_t)decode_splits(N, K) * (size_t)M * (size_t)N * sizeof(float);
}

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if ((M <= 8 && !large_splitk(M, N, K)) || M > DECODE_MAX_M) return 0;
    return (size_t)decode_splits(N, K) * (size_t)M * (size_t)N * sizeof(float);
}

}  // namespace bsg
