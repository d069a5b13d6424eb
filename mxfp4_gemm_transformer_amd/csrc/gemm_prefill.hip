// Large-M ("prefill") block-scaled GEMM on V_MFMA_SCALE_F32_32X32X64_F8F6F4.
// The sly-radiance README gives large M to a separate LDS-tiled kernel (its
// W4A8 prefill row); here the E8M0 weight scales go straight into the MFMA's
// per-lane scale operand, one per 32-element K block, so a K step is MFMAs
// only, and the per-token fp32 activation scale is applied in the epilogue.
//
// Tiling: a BM x BN output tile per workgroup of four waves in a WGM x WGN
// grid; each wave owns (BM/WGM) x (BN/WGN) as 32x32 MFMA tiles, which keeps
// the LDS bytes read per MFMA low. K advances 64 at a time through a
// software pipeline: while the MFMAs of step s run, the wave reads step
// s+1's fragments from LDS into a second register set, writes step s+2's
// tiles (fetched into registers during step s-1) into the third LDS buffer,
// and fetches step s+3; those instructions are interleaved with the MFMAs so
// the matrix core stays fed, and one barrier per step publishes the writes.
// The fetches are buffer loads whose range check turns reads past the last
// row or past K into zeros, so ragged M, N and K need no special path.
//
// LDS rows hold 16-byte chunks XOR-swizzled by row, so that the 32 lanes of
// a fragment read (32 consecutive rows, one chunk column) spread over all
// banks. For 64-byte rows the chunk column is xor-ed with row bits 2-3:
// measured on gfx950 with this fragment pattern, that reads at the full
// ds_read_b128 rate, while xor-ing with row bits 1 and 3 (which also puts
// every 16 lanes on distinct 16-byte slots of a 256-byte window) reads
// 1.26x slower.
//
// Workgroups are numbered so that consecutive tiles in a grouped order land
// on the same XCD (workgroups are dispatched round-robin over the 8 XCDs),
// which keeps the A and W panels a group shares in that XCD's L2.
#include <type_traits>

#include "bs_device.hpp"
#include "bs_kernels.hpp"

namespace bsg {
namespace {

constexpr int BK = 64;
constexpr int NXCD = 8;

// E8M0 1.0 (127) bytes. When the weights carry no E8M0 grid (one fp32 scale
// per output channel instead), the scale loads read these, so the fragment
// reads hand the MFMA its scale byte straight from LDS in either case: a
// select on the loaded byte (or a branch around the read) would put a VALU
// instruction that waits on the next step's LDS reads inside the current
// step, and a branch also splits the step into blocks the scheduler cannot
// interleave across.
__device__ const uint8_t kE8M0Ones[16] = {127, 127, 127, 127, 127, 127, 127, 127,
                                          127, 127, 127, 127, 127, 127, 127, 127};

template <bool FP4, int BM, int BN, int WGM, int WGN>
struct Cfg {
    static constexpr int NW = WGM * WGN;
    static constexpr int NT = NW * 64;
    static constexpr int AROW = BK;                   // A bytes per row per step
    static constexpr int WROW = FP4 ? BK / 2 : BK;    // W bytes per row per step
    static constexpr int A_STAGE = BM * AROW;
    static constexpr int W_STAGE = BN * WROW;
    static constexpr int STAGE = A_STAGE + W_STAGE;
    static constexpr int A_LD = A_STAGE / 16 / NT;    // 16-byte chunks per thread per step
    static constexpr int W_LD = W_STAGE / 16 / NT;
    static constexpr int TM = BM / WGM / 32;
    static constexpr int TN = BN / WGN / 32;
    // E8M0 scales of the step's two K blocks travel with the step's tiles:
    // two bytes per 32x32 block row (e4m3 weights) or per weight row (MXFP4)
    static constexpr int SC_ROWS = FP4 ? BN : BN / 32;
    static constexpr int SC_STAGE = 2 * NT;   // one 2-byte slot per thread (branch-free)
    static constexpr int STAGE_ALL = STAGE + SC_STAGE;
    static constexpr int NBUF = 3;                    // LDS buffers in the ring
    static constexpr int LDS = NBUF * STAGE_ALL;
    static_assert(A_STAGE % (16 * NT) == 0 && W_STAGE % (16 * NT) == 0, "stage split");
    static_assert(SC_ROWS <= NT, "one scale row per thread");
    static_assert(TM >= 1 && TN >= 1, "wave tile");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// Swizzle of the 16-byte chunk column within a 128-byte row (8 chunks), a
// 64-byte row (4 chunks) and a 32-byte row (2 chunks). A ds_read_b128 serves
// 16 lanes at a time from 64 four-byte banks; a fragment read puts those 16
// lanes on 16 consecutive rows at one logical chunk, and each swizzle maps
// them to 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz2(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
template <int CHUNKS>
__device__ __forceinline__ int swz(int r) {
    return CHUNKS == 8 ? swz8(r) : CHUNKS == 4 ? swz4(r) : swz2(r);
}

__device__ __forceinline__ uint4 lds16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// An 8-byte output store marked non-temporal: nothing here reads Y back, and
// ordinary stores would fill L2 with output lines that evict the A and W
// panels other tiles are still reading (measured on MI355X: the MXFP4
// gate_up at M=4096 503 -> 466 us with fp4 activations, 600 -> 566 us with
// e4m3 ones; 4096x7168x8192 e4m3 220 -> 217 us).
__device__ __forceinline__ void store_y8(uint16_t *p, uint32_t lo, uint32_t hi) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = {lo, hi};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// A per-lane offset past every buffer: reads as zero. Scalar offsets stay
// below 2^31, so their sum with it cannot wrap back into range.
constexpr uint32_t OOB = 0x80000000u;

template <bool FP4, int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(256, 1) void gemm_prefill_kernel(
    const uint8_t *__restrict__ A, int64_t lda, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ W, int64_t ldw, const uint8_t *__restrict__ WS,
    const float *__restrict__ colscale, const uint16_t *__restrict__ bias, int epi,
    uint16_t *__restrict__ Y, int64_t ldy, int M, int N, int K, int group_m) {
    using C = Cfg<FP4, BM, BN, WGM, WGN>;
    static_assert(C::NT == 256, "launch bounds assume four waves");
    __shared__ __align__(16) uint8_t lds[C::NBUF * C::STAGE_ALL];

    // ---- tile of this workgroup (XCD-aware grouped order)
    const int Mt = (M + BM - 1) / BM, Nt = (N + BN - 1) / BN, T = Mt * Nt;
    int t = blockIdx.x;
    if (T % NXCD == 0) t = (t % NXCD) * (T / NXCD) + t / NXCD;
    const int per_group = group_m * Nt;
    const int first_m = (t / per_group) * group_m;
    const int gm = min(Mt - first_m, group_m);
    const int m0 = (first_m + (t % per_group) % gm) * BM;
    const int n0 = ((t % per_group) / gm) * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int li = lane & 31, lg = lane >> 5;
    const int KB = K >> 5;
    const int nsteps = (K + BK - 1) / BK;

    // buffer descriptors over the rows from this tile on; rows past M / N
    // are outside num_records and read as zero
    const int64_t a_bytes = (int64_t)(M - m0) * lda, w_bytes = (int64_t)(N - n0) * ldw;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + (int64_t)m0 * lda), (short)0, (int)(a_bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : a_bytes),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(W + (int64_t)n0 * ldw), (short)0, (int)(w_bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : w_bytes),
        0x00020000);

    // the scale rows of this tile: [N/32, KB] for e4m3 weights, [N, KB] for
    // MXFP4; rows past the end and K blocks past KB read as zero (a zero
    // E8M0 byte scales zero data there). No WS (per-channel fp32 scales
    // instead): every thread reads byte 0 of kE8M0Ones.
    const int srow0 = FP4 ? n0 : (n0 >> 5);
    const bool ws_on = WS != nullptr;
    const int64_t s_bytes = ws_on ? (int64_t)((FP4 ? N : (N >> 5)) - srow0) * KB
                                  : (int64_t)sizeof(kE8M0Ones);
    const __amdgpu_buffer_rsrc_t rsS = __builtin_amdgcn_make_buffer_rsrc(
        ws_on ? (void *)(WS + (int64_t)srow0 * KB) : (void *)kE8M0Ones, (short)0,
        (int)(s_bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : s_bytes), 0x00020000);
    const uint32_t s_off = (uint32_t)(tid * KB);   // this thread's scale row

    // This thread's 16-byte chunks of a step: physical chunk P = j*NT + tid of
    // the LDS stage holds logical chunk c of row P / (chunks per row). Rows
    // advance by NT / (chunks per row) with j, which leaves the swizzled
    // chunk column unchanged, so one per-thread offset serves every j and
    // the row step goes into the scalar offset of the load.
    constexpr int A_ROWS_PER_J = C::NT / 4;
    constexpr int W_ROWS_PER_J = FP4 ? C::NT / 2 : C::NT / 4;
    uint32_t a_off, w_off;
    int a_k, w_k;
    {
        const int row = tid >> 2, c = (tid & 3) ^ swz4(row);
        a_off = (uint32_t)(row * lda) + 16 * c;
        a_k = 16 * c;
    }
    if (FP4) {
        const int row = tid >> 1, c = (tid & 1) ^ swz2(row);
        w_off = (uint32_t)(row * ldw) + 16 * c;
        w_k = 32 * c;
    } else {
        const int row = tid >> 2, c = (tid & 3) ^ swz4(row);
        w_off = (uint32_t)(row * ldw) + 16 * c;
        w_k = 16 * c;
    }

    struct Regs {
        uint4 a[C::A_LD];
        uint4 w[C::W_LD];
        uint32_t sc0, sc1;   // the two scale bytes of this thread's row, if any; kept
                             // apart so nothing waits on them before the LDS write
    };
    // past the last step the offsets are out of range and read zeros, so the
    // fetch is unconditional and the compiler can count its loads exactly
    auto fetch = [&](Regs &r, int s) {
        // past the end: zeros; readfirstlane keeps the scalar offsets in SGPRs
        const int kbase = __builtin_amdgcn_readfirstlane(s < nsteps ? s * BK : K);
        const uint32_t va = kbase + a_k < K ? a_off : OOB;
        const uint32_t vw = kbase + w_k < K ? w_off : OOB;
#pragma unroll
        for (int j = 0; j < C::A_LD; ++j)
            r.a[j] = bload16(rsA, va, (uint32_t)(j * A_ROWS_PER_J * lda) + kbase);
#pragma unroll
        for (int j = 0; j < C::W_LD; ++j)
            r.w[j] = bload16(rsW, vw, (uint32_t)(j * W_ROWS_PER_J * ldw) + (FP4 ? kbase / 2 : kbase));
        {   // threads past the tile's scale rows read zeros into unused slots
            const int kb = kbase >> 5;
            // bitwise conditions: a short-circuit here becomes a branch that
            // splits the scheduling region and stalls the MFMA stream
            const bool row_ok = tid < C::SC_ROWS;
            const uint32_t o0 = !ws_on ? 0u : (row_ok & (kb < KB)) ? s_off + kb : OOB;
            const uint32_t o1 = !ws_on ? 0u : (row_ok & (kb + 1 < KB)) ? s_off + kb + 1 : OOB;
            r.sc0 = __builtin_amdgcn_raw_buffer_load_b8(rsS, o0, 0, 0);
            r.sc1 = __builtin_amdgcn_raw_buffer_load_b8(rsS, o1, 0, 0);
        }
    };
    auto stash = [&](const Regs &r, uint8_t *dst) {
#pragma unroll
        for (int j = 0; j < C::A_LD; ++j)
            *reinterpret_cast<uint4 *>(dst + 16 * (j * C::NT + tid)) = r.a[j];
#pragma unroll
        for (int j = 0; j < C::W_LD; ++j)
            *reinterpret_cast<uint4 *>(dst + C::A_STAGE + 16 * (j * C::NT + tid)) = r.w[j];
        dst[C::STAGE + 2 * tid] = (uint8_t)r.sc0;
        dst[C::STAGE + 2 * tid + 1] = (uint8_t)r.sc1;
    };
    v16f acc[C::TM][C::TN];
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TN; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    struct Frags {
        v8i a[C::TM];
        v8i b[C::TN];
        int sc[C::TN];
    };
    // fragments of step s from its LDS buffer (s % 3) and the scale chunk
    auto read_frags = [&](Frags &f, int s) {
        const uint8_t *sa = lds + (s % C::NBUF) * C::STAGE_ALL;
        const uint8_t *sw = sa + C::A_STAGE;
        const uint8_t *ss = sa + C::STAGE;
#pragma unroll
        for (int a = 0; a < C::TM; ++a) {
            const int row = wm * (BM / WGM) + a * 32 + li;
            const int fz = swz4(row);
            const uint8_t *base = sa + row * C::AROW;
            f.a[a] = pack8(lds16(base + 16 * (lg ^ fz)), lds16(base + 16 * ((2 + lg) ^ fz)));
        }
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
            const int row = wn * (BN / WGN) + b * 32 + li;
            if (FP4) {
                f.b[b] = pack8(lds16(sw + row * C::WROW + 16 * (lg ^ swz2(row))),
                               make_uint4(0u, 0u, 0u, 0u));
                f.sc[b] = ss[2 * row + lg];
            } else {
                const int fz = swz4(row);
                const uint8_t *base = sw + row * C::WROW;
                f.b[b] = pack8(lds16(base + 16 * (lg ^ fz)), lds16(base + 16 * ((2 + lg) ^ fz)));
                f.sc[b] = ss[2 * (row >> 5) + lg];
            }
        }
    };
    auto mfmas = [&](const Frags &f) {
#pragma unroll
        for (int a = 0; a < C::TM; ++a)
#pragma unroll
            for (int b = 0; b < C::TN; ++b)
                acc[a][b] = mfma32_wt<FP4>(f.b[b], f.a[a], acc[a][b], f.sc[b]);
    };
    // Interleave one MFMA with the memory instructions of the same step:
    // LDS reads of the next fragments, LDS writes of the staged tile, and
    // the global fetch that refills the staging registers.
    auto interleave = [&]() {
        constexpr int NM = C::TM * C::TN;
        constexpr int NR = 2 * (C::TM + C::TN) + C::TN;   // ds reads (incl. scale bytes)
        constexpr int NWR = C::A_LD + C::W_LD;             // ds writes == vmem reads
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, (NR + NM - 1) / NM, 0);  // DS read
            if (i < NWR) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
            if (i < NWR) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        }
    };
    // prologue: stages 0 and 1 into LDS, stage 2 in the staging registers,
    // step 0's fragments in registers
    Regs r;
    fetch(r, 0);
    stash(r, lds);
    fetch(r, 1);
    stash(r, lds + C::STAGE_ALL);
    fetch(r, 2);
    __syncthreads();
    Frags f0, f1;
    read_frags(f0, 0);

    // step s: MFMAs on step s's fragments; read step s+1's; write stage s+2
    // (already in r) into buffer (s+2) % 3; fetch stage s+3 into r
    auto step = [&](const Frags &cur, Frags &nxt, int s) {
        mfmas(cur);
        read_frags(nxt, s + 1);
        stash(r, lds + ((s + 2) % C::NBUF) * C::STAGE_ALL);
        fetch(r, s + 3);
        interleave();
        __syncthreads();
    };
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
        step(f0, f1, s);
        step(f1, f0, s + 1);
    }
    if (s < nsteps) mfmas(f0);  // odd step count: the last step's fragments are in f0

    // ---- epilogue. The MFMAs computed transposed tiles: lane l = i + 32 g,
    // VGPR v holds token m = tile row i and weight column n = 8 (v/4) + 4 g
    // + v%4, so VGPRs 4q..4q+3 are four consecutive columns of one output
    // row: one 8-byte store each.
#pragma unroll
    for (int a = 0; a < C::TM; ++a) {
        const int m = m0 + wm * (BM / WGM) + a * 32 + li;
        if (m >= M) continue;
        const float as = a_scale[m];
        uint16_t *yrow = Y + (int64_t)m * ldy;
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * (BN / WGN) + b * 32 + 8 * q + 4 * lg;
                if (n >= N) continue;
                float bv[4] = {0.f, 0.f, 0.f, 0.f}, cv[4] = {1.f, 1.f, 1.f, 1.f};
                if (epi != EPI_NONE) {  // bias is only 2-byte aligned
#pragma unroll
                    for (int j = 0; j < 4; ++j) bv[j] = bf16_to_f32(bias[n + j]);
                }
                if (colscale) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) cv[j] = colscale[n + j];
                }
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = epilogue(acc[a][b][4 * q + j], as, cv[j], bv[j], epi);
                store_y8(yrow + n, pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            }
        }
    }
}

template <bool FP4, int BM, int BN, int WGM, int WGN>
hipError_t launch_tile(const uint8_t *a, int64_t lda, const float *as, const uint8_t *w,
                       int64_t ldw, const uint8_t *ws, const float *cs, const uint16_t *bias,
                       int epi, uint16_t *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                       hipStream_t st) {
    using C = Cfg<FP4, BM, BN, WGM, WGN>;
    auto kern = gemm_prefill_kernel<FP4, BM, BN, WGM, WGN>;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(C::NT), 0, st, a, lda, as, w, ldw, ws,
                       cs, bias, epi, y, ldy, (int)M, (int)N, (int)K, 8);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// DMA-staged variant, for K a multiple of 64 (whole steps, and E8M0 byte pairs
// that start on even offsets). The tiles of a K step go from HBM/L2 straight
// into LDS with buffer loads in LDS mode, which write each lane's 16 bytes at
// M0 + 16 * lane, so the waves never hold tile data in registers and never
// write LDS themselves. A ring of NBUF stages keeps NBUF - 1 steps of loads
// in flight; one wait on the vector-memory counter and one barrier per step
// publish the stage the next step reads. The weight scales of a step travel
// as one 2-byte load per scale row into a 4-byte slot per thread, except in
// the MXFP4 tiles with scale slabs (two-step stages, see DCfg), which load
// their tile's E8M0 rows for all of K once, ahead of the first stage.
//
// The waits are written out because the compiler does not track LDS-mode
// loads issued from inline assembly: every thread issues the same loads in
// the same order (past the end they read zeros from outside the buffer's
// range), so a count of loads per stage states exactly which stages are done.

// The helpers below write M0, which the compiler reserves; nothing else in
// these kernels uses M0, so clobbering it is safe here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// One 16-byte LDS-mode buffer load: lane l's bytes land at m0 + 16 l.
// (One wait state between the M0 write and the load that reads it.)
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t rs, uint32_t m0, uint32_t voff,
                                         uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs), "s"(soff)
                 : "memory", "m0");
}

// One 4-byte LDS-mode buffer load: lane l's bytes land at m0 + 4 l.
__device__ __forceinline__ void dma_u32(__amdgpu_buffer_rsrc_t rs, uint32_t m0, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs)
                 : "memory", "m0");
}

// One 2-byte LDS-mode buffer load: lane l's two bytes land zero-extended in
// the 4-byte slot m0 + 4 l.
__device__ __forceinline__ void dma_u16(__amdgpu_buffer_rsrc_t rs, uint32_t m0, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_ushort %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs)
                 : "memory", "m0");
}

#pragma clang diagnostic pop

// Wait until at most N of this wave's vector-memory loads are in flight,
// then meet the other waves.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

// SPS: K steps (of BK) per LDS stage. SPS = 1: a ring of NBUF >= 4 stages,
// one barrier per step. SPS = 2: two stages of 128 K each, one barrier per
// two steps; each load then covers whole 128-byte lines of e4m3 rows (with
// 64-byte stages the two halves of a line are fetched a step apart, and the
// 32 KB L1 has evicted the line in between, so L2 serves it twice).
//
// SLAB_KB > 0 (MXFP4 weights, fp4 activations): the tile's E8M0 rows for
// all of K (K / 32 <= SLAB_KB bytes each, K % 128 == 0) are loaded into LDS
// once, ahead of the first stage, as contiguous 4-byte pieces. Per-row
// scales read a step at a time gather two bytes from each of the tile's 256
// rows, a separate cache line each, every step: more L2 requests than the
// tiles themselves.
template <bool FP4, int BM, int BN, int NBUF, int WGM, int WGN, bool FP4A = false, int SPS = 1,
          int SLAB_KB = 0, int WBUF = NBUF>
struct DCfg {
    static constexpr int NW = WGM * WGN;              // waves, WGM x WGN
    static constexpr int NT = NW * 64;
    static constexpr int KS = BK * SPS;               // K per stage
    static constexpr int WROW = FP4 ? KS / 2 : KS;    // W bytes per row per stage
    static constexpr int AROW = FP4A ? KS / 2 : KS;   // A bytes per row per stage
    static constexpr int A_CH = AROW / 16, W_CH = WROW / 16;   // 16-byte chunks per row
    static constexpr int A_STAGE = BM * AROW;
    static constexpr int W_STAGE = BN * WROW;
    static constexpr bool SLAB = SLAB_KB > 0;
    static constexpr int SC_OFF = A_STAGE + W_STAGE;  // per step: one 4-byte scale slot per thread
    static constexpr int SCA_OFF = SC_OFF + 4 * NT * SPS;   // fp4 activations: their scale slots
    static constexpr int STAGE = SLAB ? SC_OFF : SC_OFF + 4 * NT * SPS * (FP4A ? 2 : 1);
    static constexpr int A_LD = A_STAGE / 16 / NT;    // 16-byte loads per thread per stage
    static constexpr int W_LD = W_STAGE / 16 / NT;
    static constexpr int LPS = A_LD + W_LD + (SLAB ? 0 : SPS * (FP4A ? 2 : 1));   // loads per thread per stage
    static constexpr int TM = BM / WGM / 32;
    static constexpr int TN = BN / WGN / 32;
    static constexpr int SC_ROWS = FP4 ? BN : BN / 32;
    // epilogue staging: each wave's 32 x (32 TN) fp32 slab, rows padded by 16 bytes
    static constexpr int EP_ROW = TN * 32 * 4 + 16;
    static constexpr int EP_WAVE = 32 * EP_ROW;
    static constexpr int EP_ALL = NW * EP_WAVE;
    static_assert(64 % (TN * 8) == 0, "a lane reads the same 4 columns in every slab row it reads");
    // scale slabs after the stages: weight rows, then (fp4 activations) A
    // rows, each rounded up to whole rounds of 4-byte loads
    static constexpr int SLAB_ROUND = 4 * NT;
    static constexpr int WSLAB = SLAB ? (SC_ROWS * SLAB_KB + SLAB_ROUND - 1) / SLAB_ROUND * SLAB_ROUND : 0;
    static constexpr int ASLAB = SLAB && FP4A ? (BM * SLAB_KB + SLAB_ROUND - 1) / SLAB_ROUND * SLAB_ROUND : 0;
    // WBUF > NBUF (two-step stages with scale slabs only): the W tiles have
    // a ring of their own after the NBUF A tiles, one stage deeper, so each
    // W stage is fetched a stage earlier than its A stage
    static constexpr bool WRING = WBUF != NBUF;
    static constexpr int RING = WRING ? NBUF * A_STAGE + WBUF * W_STAGE : NBUF * STAGE;
    __host__ __device__ static constexpr int a_base(int b) { return WRING ? b * A_STAGE : b * STAGE; }
    __host__ __device__ static constexpr int w_base(int b) {
        return WRING ? NBUF * A_STAGE + b * W_STAGE : b * STAGE + A_STAGE;
    }
    static constexpr int WSLAB_OFF = RING, ASLAB_OFF = WSLAB_OFF + WSLAB;
    static constexpr int MAIN = RING + WSLAB + ASLAB;
    // the epilogue's operands, fetched by LDS-mode loads when the tile starts
    // into a region of their own past the ring and the epilogue's staging: a
    // 4-byte slot per row (per-token scale) and two per column (bias, whose
    // bf16 bits land in the slot's low half, and channel scale); each part
    // holds whole waves' worth of slots (64), every slot a wave writes
    static constexpr int EPO_AS = MAIN > EP_ALL ? MAIN : EP_ALL;
    static constexpr int EPO_B = EPO_AS + 4 * ((BM + 63) / 64 * 64);
    static constexpr int EPO_CS = EPO_B + 4 * ((BN + 63) / 64 * 64);
    static constexpr int LDS = EPO_CS + 4 * ((BN + 63) / 64 * 64);
    static_assert(A_STAGE % (16 * NT) == 0 && W_STAGE % (16 * NT) == 0, "stage split");
    static_assert(SC_ROWS <= NT, "one scale row per thread");
    static_assert(!FP4A || BM <= NT, "one activation scale row per thread");
    static_assert(SPS == 1 ? NBUF >= 4 : (SPS == 2 && NBUF == 2), "pipeline shape");
    static_assert(SPS != 1 || LPS * (NBUF - 3) <= 63, "vmcnt range");
    static_assert(!SLAB || FP4, "scale slabs hold per-row (MXFP4) scales");
    static_assert(!WRING || (SPS == 2 && NBUF == 2 && WBUF == 3 && SLAB), "W ring shape");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// FP4A: fp4 activations [M, K/2] with E8M0 scales AS [M, K/32] (W4A4); then
// a_scale is unused (1).
//
// GROUPED (MoE, prefill-sized expert batches): blockIdx.y is the expert e;
// its token rows are [gp.off[e], gp.off[e + 1]) of A, a_scale and Y (offsets
// read on the device, clamped to [0, gp.rows]), its weights start at
// W + e * gp.w_estride with scales WS + e * (N or N / 32) * K / 32 and bias
// + e * N. The grid's M (a bound on any expert's rows) sets the tiles per
// expert; a workgroup takes m-tiles m0, m0 + that, ... up to the expert's
// rows, so any distribution of rows is computed, whatever the bound.
struct GroupArgs {
    const int32_t *off;
    int64_t w_estride;
    int rows;
};

template <bool FP4, int BM, int BN, int NBUF, int WGM, int WGN, bool FP4A = false, int SPS = 1,
          int SLAB_KB = 0, bool GROUPED = false, int WBUF = NBUF>
__global__ __launch_bounds__(WGM * WGN * 64, 1) void gemm_prefill_dma_kernel(
    const uint8_t *__restrict__ A_in, int64_t lda, const float *__restrict__ a_scale_in,
    const uint8_t *__restrict__ W_in, int64_t ldw, const uint8_t *__restrict__ WS_in,
    const float *__restrict__ colscale, const uint16_t *__restrict__ bias_in, int epi,
    uint16_t *__restrict__ Y_in, int64_t ldy, int M_grid, int N, int K, int group_m,
    const uint8_t *__restrict__ AS, GroupArgs gp) {
    using C = DCfg<FP4, BM, BN, NBUF, WGM, WGN, FP4A, SPS, SLAB_KB, WBUF>;
    __shared__ __align__(16) uint8_t lds[C::LDS];

    // ---- tile of this workgroup (XCD-aware grouped order)
    const int Mt = (M_grid + BM - 1) / BM, Nt = (N + BN - 1) / BN, T = Mt * Nt;
    int t = blockIdx.x;
    if (T % NXCD == 0) t = (t % NXCD) * (T / NXCD) + t / NXCD;
    const int per_group = group_m * Nt;
    const int first_m = (t / per_group) * group_m;
    const int gm = min(Mt - first_m, group_m);
    const int m_first = (first_m + (t % per_group) % gm) * BM;
    const int n0 = ((t % per_group) / gm) * BN;

    const uint8_t *A = A_in;
    const float *a_scale = a_scale_in;
    const uint8_t *W = W_in;
    const uint8_t *WS = WS_in;
    const uint16_t *bias = bias_in;
    uint16_t *Y = Y_in;
    int M = M_grid;
    if constexpr (GROUPED) {
        const int e = blockIdx.y;
        const int r0 = min(max(gp.off[e], 0), gp.rows);
        const int r1 = max(r0, min(gp.off[e + 1], gp.rows));
        A += (int64_t)r0 * lda;
        a_scale += r0;
        Y += (int64_t)r0 * ldy;
        W += (int64_t)e * gp.w_estride;
        if (WS) WS += (int64_t)e * (FP4 ? N : N / 32) * (K >> 5);
        if (bias) bias += (int64_t)e * N;
        M = r1 - r0;
    }
    for (int m0 = m_first; m0 < M; m0 += Mt * BM) {

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int li = lane & 31, lg = lane >> 5;
    const int KB = K >> 5;
    const int nsteps = K / BK;
    const int nstages = (nsteps + SPS - 1) / SPS;   // a last half stage reads unused bytes

    const int64_t a_bytes = (int64_t)(M - m0) * lda, w_bytes = (int64_t)(N - n0) * ldw;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + (int64_t)m0 * lda), (short)0, (int)(a_bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : a_bytes),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(W + (int64_t)n0 * ldw), (short)0, (int)(w_bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : w_bytes),
        0x00020000);
    const int srow0 = FP4 ? n0 : (n0 >> 5);
    const bool ws_on = WS != nullptr;
    const int64_t s_bytes = ws_on ? (int64_t)((FP4 ? N : (N >> 5)) - srow0) * KB
                                  : (int64_t)sizeof(kE8M0Ones);
    const __amdgpu_buffer_rsrc_t rsS = __builtin_amdgcn_make_buffer_rsrc(
        ws_on ? (void *)(WS + (int64_t)srow0 * KB) : (void *)kE8M0Ones, (short)0,
        (int)(s_bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : s_bytes), 0x00020000);

    const int64_t sa_bytes = FP4A ? (int64_t)(M - m0) * KB : 0;
    const __amdgpu_buffer_rsrc_t rsSA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(FP4A ? AS + (int64_t)m0 * KB : AS), (short)0,
        (int)(sa_bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : sa_bytes), 0x00020000);

    // This thread's 16-byte chunk of each load: physical chunk j*NT + tid of
    // a stage (where the LDS-mode load of wave w, lane l, puts its bytes)
    // holds logical chunk c of its row, c = physical column ^ swizzle(row).
    constexpr int A_ROWS_PER_J = C::NT / C::A_CH;
    constexpr int W_ROWS_PER_J = C::NT / C::W_CH;
    uint32_t a_off, w_off;
    {
        const int row = tid / C::A_CH, c = (tid % C::A_CH) ^ swz<C::A_CH>(row);
        a_off = (uint32_t)(row * lda) + 16 * c;
    }
    {
        const int row = tid / C::W_CH, c = (tid % C::W_CH) ^ swz<C::W_CH>(row);
        w_off = (uint32_t)(row * ldw) + 16 * c;
    }
    // without a grid every thread reads the first two bytes of kE8M0Ones
    const uint32_t s_off = !ws_on ? 0u : tid < C::SC_ROWS ? (uint32_t)(tid * KB) : OOB;
    const uint32_t s_kshift = ws_on ? 5u : 31u;   // k / 32 (the step's block), or 0
    const uint32_t sa_off = tid < BM ? (uint32_t)(tid * KB) : OOB;
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t *)lds);

    // Load i (0 .. LPS-1) of stage p into buffer p % NBUF: the A chunks, the
    // W chunks, then each step's scale pairs (weights, then fp4 activations).
    // With a W ring of its own the W chunks are those of stage p + 1, into
    // W buffer (p + 1) % WBUF. Past the last stage every lane reads outside
    // the buffers' ranges, which writes zeros.
    auto issue_w = [&](int p, int j) {
        const bool live = p < nstages;
        const uint32_t kbase = (uint32_t)__builtin_amdgcn_readfirstlane(live ? p * C::KS : 0);
        const uint32_t base = lds0 + (uint32_t)C::w_base(p % WBUF) + (uint32_t)wave * 1024u;
        dma_b128(rsW, base + j * C::NT * 16, live ? w_off : OOB,
                 (uint32_t)(j * W_ROWS_PER_J * ldw) + (FP4 ? kbase / 2 : kbase));
    };
    auto issue_one = [&](int p, int i) {
        const bool live = p < nstages;
        const uint32_t kbase = (uint32_t)__builtin_amdgcn_readfirstlane(live ? p * C::KS : 0);
        const uint32_t sbase = lds0 + (uint32_t)((p % NBUF) * C::STAGE);
        const uint32_t base = lds0 + (uint32_t)C::a_base(p % NBUF) + (uint32_t)wave * 1024u;
        if (i < C::A_LD) {
            dma_b128(rsA, base + i * C::NT * 16, live ? a_off : OOB,
                     (uint32_t)(i * A_ROWS_PER_J * lda) + (FP4A ? kbase / 2 : kbase));
        } else if (i < C::A_LD + C::W_LD) {
            issue_w(C::WRING ? p + 1 : p, i - C::A_LD);
        } else if (C::SLAB) {
            // unreachable: with scale slabs a stage has only tile loads
        } else if (i < C::A_LD + C::W_LD + SPS) {
            const int q = i - C::A_LD - C::W_LD;   // the stage's step q
            dma_u16(rsS, sbase + (uint32_t)(C::SC_OFF + q * 4 * C::NT) + (uint32_t)wave * 256u,
                    live ? s_off + ((kbase + q * BK) >> s_kshift) : OOB);
        } else {   // FP4A: the activation rows' scale pairs
            const int q = i - C::A_LD - C::W_LD - SPS;
            dma_u16(rsSA, sbase + (uint32_t)(C::SCA_OFF + q * 4 * C::NT) + (uint32_t)wave * 256u,
                    live ? sa_off + ((kbase + q * BK) >> 5) : OOB);
        }
    };

    v16f acc[C::TM][C::TN];
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TN; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    struct Frags {
        v8i a[C::TM];
        v8i b[C::TN];
        int sc[C::TN];
        int sa[C::TM];
    };
    // fragments of step s (stage s / SPS in buffer (s / SPS) % NBUF, its
    // step q = s % SPS, given as the constant qk): A tile a, W tile b (+
    // their scales). A step takes 32 bytes of an e4m3 row (chunks 4q + lg and
    // 4q + 2 + lg) or 16 bytes of an fp4 row (chunk 2q + lg). With scale
    // slabs, step q = 0 reads the stage's 4 E8M0 bytes of the row as one
    // word, shifted so that byte 2q is this lane's block for step q (the
    // MFMA selects it); step q = 1 reuses that word (copied by the caller).
    auto read_a = [&](Frags &f, int s, int a, int qk) {
        const int q = SPS == 1 ? 0 : qk;
        const uint8_t *sa = lds + C::a_base((s / SPS) % NBUF);
        const int row = wm * (BM / WGM) + a * 32 + li;
        const int fz = swz<C::A_CH>(row);
        const uint8_t *p = sa + row * C::AROW;
        if (FP4A) {
            f.a[a] = pack8(lds16(p + 16 * ((2 * q + lg) ^ fz)), make_uint4(0u, 0u, 0u, 0u));
            if (C::SLAB) {
                if (q == 0)
                    f.sa[a] = (int)(*reinterpret_cast<const uint32_t *>(lds + C::ASLAB_OFF + row * KB + 2 * s) >>
                                    (8 * lg));
            } else {
                f.sa[a] = (sa + C::SCA_OFF + q * 4 * C::NT)[4 * row + lg];
            }
        } else {
            f.a[a] = pack8(lds16(p + 16 * ((4 * q + lg) ^ fz)), lds16(p + 16 * ((4 * q + 2 + lg) ^ fz)));
            f.sa[a] = E8M0_ONE;
        }
    };
    auto read_b = [&](Frags &f, int s, int b, int qk) {
        const int q = SPS == 1 ? 0 : qk;
        const uint8_t *sw = lds + C::w_base((s / SPS) % WBUF);
        const uint8_t *ss = lds + ((s / SPS) % NBUF) * C::STAGE + C::SC_OFF + q * 4 * C::NT;
        const int row = wn * (BN / WGN) + b * 32 + li;
        const int fz = swz<C::W_CH>(row);
        const uint8_t *p = sw + row * C::WROW;
        if (FP4) {
            f.b[b] = pack8(lds16(p + 16 * ((2 * q + lg) ^ fz)), make_uint4(0u, 0u, 0u, 0u));
            if (C::SLAB) {
                if (q == 0)
                    f.sc[b] = (int)(*reinterpret_cast<const uint32_t *>(lds + C::WSLAB_OFF + row * KB + 2 * s) >>
                                    (8 * lg));
            } else {
                f.sc[b] = ss[4 * row + lg];
            }
        } else {
            f.b[b] = pack8(lds16(p + 16 * ((4 * q + lg) ^ fz)), lds16(p + 16 * ((4 * q + 2 + lg) ^ fz)));
            f.sc[b] = ss[4 * (row >> 5) + lg];
        }
    };
    // The loads of a step go one before each fragment read, so that with the
    // MFMAs interleaved between the reads they spread over the whole step:
    // issued as one block they stall the wave's instruction stream, which
    // (one wave per SIMD) is the MFMA stream.
    // (nl loads of stage p_load, spread evenly before the TM + TN reads)
    auto reads_and_loads = [&](Frags &f, int s_read, int p_load, int nl, int qk) {
        constexpr int R = C::TM + C::TN;
        int k = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (; k < (r + 1) * nl / R; ++k) issue_one(p_load, k);
            if (r < C::TM) read_a(f, s_read, r, qk);
            else read_b(f, s_read, r - C::TM, qk);
        }
    };
    // MFMAs of a step with stage step qk (slab scales: byte 2 qk of each word)
    auto mfmas = [&](const Frags &f, auto qk) {
        constexpr int SEL = C::SLAB ? 2 * decltype(qk)::value : 0;
#pragma unroll
        for (int a = 0; a < C::TM; ++a)
#pragma unroll
            for (int b = 0; b < C::TN; ++b)
                acc[a][b] = mfma32_wt2<FP4, FP4A, SEL>(f.b[b], f.a[a], acc[a][b], f.sc[b], f.sa[a]);
    };
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    auto interleave = [&]() {
        constexpr int NM = C::TM * C::TN;
        constexpr int NR = 2 * (C::TM + C::TN) + C::TN;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, (NR + NM - 1) / NM, 0);  // DS read
        }
    };

    // prologue: SPS = 1, stages 0 .. NBUF-2 in flight, wait for stages 0 and
    // 1; SPS = 2, both stages in flight, wait for stage 0
    constexpr int PRO = SPS == 1 ? NBUF - 1 : 2;
    {
        // the epilogue's per-token scales, bias and channel scales first (the
        // oldest loads, so every wait below covers them): a lane's 4-byte slot
        // at M0 + 4 lane, waves past the tile's rows or columns issue none
        if (!FP4A && wave * 64 < BM) {
            const int64_t ab = (int64_t)(M - m0) * 4;
            const __amdgpu_buffer_rsrc_t rsT = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a_scale + m0), (short)0, (int)(ab > 0x7FFFFFF0 ? 0x7FFFFFF0 : ab), 0x00020000);
            dma_u32(rsT, lds0 + C::EPO_AS + (uint32_t)wave * 256u, tid < BM ? (uint32_t)(4 * tid) : OOB);
        }
        if (epi != EPI_NONE && wave * 64 < BN) {
            const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(bias + n0), (short)0, (int)((int64_t)(N - n0) * 2), 0x00020000);
            dma_u16(rsB, lds0 + C::EPO_B + (uint32_t)wave * 256u, tid < BN ? (uint32_t)(2 * tid) : OOB);
        }
        if (colscale && wave * 64 < BN) {
            const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(colscale + n0), (short)0, (int)((int64_t)(N - n0) * 4), 0x00020000);
            dma_u32(rsC, lds0 + C::EPO_CS + (uint32_t)wave * 256u, tid < BN ? (uint32_t)(4 * tid) : OOB);
        }
    }
    if constexpr (C::SLAB) {
        // the tile's scale rows, [rows, KB] bytes, in 4-byte pieces: piece d
        // of the flattened slab comes from row d / (KB / 4); pieces past the
        // last row of the tile or of the matrix read zeros
        const int kq = KB >> 2;
        const int w_pieces = C::SC_ROWS * kq;
        for (int j = 0; j * C::NT < w_pieces; ++j) {
            const int d = j * C::NT + tid, r = d / kq;
            const uint32_t off = d < w_pieces ? (uint32_t)(r * KB + 4 * (d - r * kq)) : OOB;
            dma_u32(rsS, (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + C::WSLAB_OFF + j * C::NT * 4 + wave * 256),
                    off);
        }
        if constexpr (FP4A) {
            const int a_pieces = BM * kq;
            for (int j = 0; j * C::NT < a_pieces; ++j) {
                const int d = j * C::NT + tid, r = d / kq;
                const uint32_t off = d < a_pieces ? (uint32_t)(r * KB + 4 * (d - r * kq)) : OOB;
                dma_u32(rsSA, (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + C::ASLAB_OFF + j * C::NT * 4 + wave * 256),
                        off);
            }
        }
    }
    if constexpr (C::WRING) {   // W stage 0 first: then A p and W p + 1 per stage
#pragma unroll
        for (int j = 0; j < C::W_LD; ++j) issue_w(0, j);
    }
#pragma unroll
    for (int p = 0; p < PRO; ++p)
#pragma unroll
        for (int i = 0; i < C::LPS; ++i) issue_one(p, i);
    wait_loads_and_barrier<SPS == 1 ? C::LPS * (NBUF - 3) : C::LPS + (C::WRING ? C::W_LD : 0)>();
    Frags f0, f1;
#pragma unroll
    for (int a = 0; a < C::TM; ++a) read_a(f0, 0, a, 0);
#pragma unroll
    for (int b = 0; b < C::TN; ++b) read_b(f0, 0, b, 0);

    // step s: MFMAs on step s's fragments, interleaved with the reads of
    // step s + 1's and the loads of step s + NBUF - 1; then wait until step
    // s + 2's stage has landed.
    // The scheduling barriers keep each step's MFMAs on their side of the
    // wait: the inline assembly orders memory operations only, so without
    // them the compiler moves MFMAs across it and the steps lose their
    // even MFMA / read / load mix.
    auto step = [&](const Frags &cur, Frags &nxt, int s) {
        mfmas(cur, Q0{});
        reads_and_loads(nxt, s + 1, s + NBUF - 1, C::LPS, 0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        wait_loads_and_barrier<C::LPS * (NBUF - 3)>();
        __builtin_amdgcn_sched_barrier(0);
    };
    // SPS = 2, steps 2p and 2p + 1 of stage p. Even step 2p: MFMAs, the
    // reads of step 2p + 1 (stage p), then wait until this wave's reads
    // are done and stage p + 1 has landed, and meet: stage p is then free
    // in every wave. Odd step 2p + 1: MFMAs, the reads of step 2p + 2
    // (stage p + 1) and the loads of stage p + 2 into stage p's buffer,
    // which have until the end of step 2p + 2 to land (with a W ring of its
    // own, W stage p + 3 into W buffer p % 3, with until the end of step
    // 2p + 4: W tiles that stream from HBM once wait a full memory latency,
    // while A tiles come from L2).
    auto step_even = [&](const Frags &cur, Frags &nxt, int s) {
        mfmas(cur, Q0{});
        reads_and_loads(nxt, s + 1, 0, 0, 1);
        if (C::SLAB) {   // step 2p + 1 uses step 2p's scale words
#pragma unroll
            for (int b = 0; b < C::TN; ++b) nxt.sc[b] = cur.sc[b];
#pragma unroll
            for (int a = 0; a < C::TM; ++a) nxt.sa[a] = cur.sa[a];
        }
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        wait_loads_and_barrier<C::WRING ? C::W_LD : 0>();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto step_odd = [&](const Frags &cur, Frags &nxt, int s) {
        mfmas(cur, Q1{});
        reads_and_loads(nxt, s + 1, (s + 3) / 2, C::LPS, 0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
    };
    int s = 0;
    if constexpr (SPS == 1) {
        for (; s + 1 < nsteps; s += 2) {
            step(f0, f1, s);
            step(f1, f0, s + 1);
        }
    } else {
        for (; s + 1 < nsteps; s += 2) {
            step_even(f0, f1, s);
            step_odd(f1, f0, s + 1);
        }
    }
    if (s < nsteps) mfmas(f0, Q0{});

    // ---- epilogue: every load has landed and every wave is done with the
    // ring. Each wave scales one 32-row slab of its tile by the per-token
    // scales (in the accumulator layout, where a lane holds one row), stages
    // it in LDS as fp32, and reads it back as 4-column chunks in row-major
    // order, adding the bias, applying GELU and rounding to bf16, so that
    // consecutive lanes write consecutive 8-byte pieces of an output row.
    // A wave's slab is its own, so the waves go through their slabs without
    // meeting: a wave's LDS writes complete before its reads (and its reads
    // before its next writes) by lgkmcnt(0). A lane reads the same 4
    // columns in every slab row it reads, so their bias and channel scales
    // are read once.
    wait_loads_and_barrier<0>();
    uint8_t *slab = lds + wave * C::EP_WAVE;
    constexpr int WCOLS = C::TN * 32;               // the wave's columns
    constexpr int CPR = WCOLS / 4;                  // 4-column chunks per slab row
    const int ncol0 = n0 + wn * (BN / WGN);         // the wave's first column
    const int cc = 4 * (lane % CPR);                // this lane's 4 columns (of the wave's)
    float4 bv = make_float4(0.f, 0.f, 0.f, 0.f), cv = make_float4(1.f, 1.f, 1.f, 1.f);
    {   // (zeros past N: those columns are not stored)
        const int cl = wn * (BN / WGN) + cc;
        if (epi != EPI_NONE) {
            const uint4 b4 = *reinterpret_cast<const uint4 *>(lds + C::EPO_B + 4 * cl);
            bv = make_float4(bf16_to_f32(b4.x & 0xFFFFu), bf16_to_f32(b4.y & 0xFFFFu),
                             bf16_to_f32(b4.z & 0xFFFFu), bf16_to_f32(b4.w & 0xFFFFu));
        }
        if (colscale) cv = *reinterpret_cast<const float4 *>(lds + C::EPO_CS + 4 * cl);
    }
    float asv[C::TM];
#pragma unroll
    for (int a = 0; a < C::TM; ++a)   // (zeros past M: those rows are not stored)
        asv[a] = FP4A ? 1.0f
                      : *reinterpret_cast<const float *>(lds + C::EPO_AS +
                                                         4 * (wm * (BM / WGM) + a * 32 + li));
#pragma unroll
    for (int a = 0; a < C::TM; ++a) {
#pragma unroll
        for (int b = 0; b < C::TN; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = b * 32 + 8 * q + 4 * lg;
                float4 v;
                v.x = asv[a] * acc[a][b][4 * q + 0];
                v.y = asv[a] * acc[a][b][4 * q + 1];
                v.z = asv[a] * acc[a][b][4 * q + 2];
                v.w = asv[a] * acc[a][b][4 * q + 3];
                *reinterpret_cast<float4 *>(slab + li * C::EP_ROW + 4 * col) = v;
            }
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        __builtin_amdgcn_wave_barrier();
        const int mrow = m0 + wm * (BM / WGM) + a * 32;
        // the read-back, with the bias / GELU / channel-scale work compiled
        // out when the call has none of it (a uniform choice per call; a
        // copy for every epilogue kind made the main loop of the
        // 4096x7168x8192 GEMM slower: 268-274 against 222 us)
        auto read_back = [&](auto plain_tag) {
            constexpr bool PLAIN = decltype(plain_tag)::value;
#pragma unroll
            for (int it = 0; it < 32 * CPR / 64; ++it) {
                const int rr = (it * 64 + lane) / CPR;
                const float4 v = *reinterpret_cast<const float4 *>(slab + rr * C::EP_ROW + 4 * cc);
                uint32_t h01, h23;
                if constexpr (PLAIN) {
                    h01 = pack_bf16x2(v.x, v.y);
                    h23 = pack_bf16x2(v.z, v.w);
                } else {
                    h01 = pack_bf16x2(epilogue_rest(v.x * cv.x, bv.x, epi),
                                      epilogue_rest(v.y * cv.y, bv.y, epi));
                    h23 = pack_bf16x2(epilogue_rest(v.z * cv.z, bv.z, epi),
                                      epilogue_rest(v.w * cv.w, bv.w, epi));
                }
                const int m = mrow + rr, n = ncol0 + cc;
                if (m < M && n < N)
                    store_y8(Y + (int64_t)m * ldy + n, h01, h23);
            }
        };
        if (epi == EPI_NONE && !colscale)
            read_back(std::true_type{});
        else
            read_back(std::false_type{});
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        __builtin_amdgcn_wave_barrier();
    }
    if constexpr (!GROUPED) break;   // one tile; the grid covers every m-tile
    __syncthreads();                 // the next m-tile's loads reuse every wave's LDS
    }
}

template <bool FP4, int BM, int BN, int NBUF, int WGM = 2, int WGN = 2, bool FP4A = false,
          int SPS = 1, int SLAB_KB = 0>
hipError_t launch_tile_dma(const uint8_t *a, int64_t lda, const float *as, const uint8_t *w,
                           int64_t ldw, const uint8_t *ws, const float *cs, const uint16_t *bias,
                           int epi, uint16_t *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                           hipStream_t st, const uint8_t *a_e8m0 = nullptr) {
    auto kern = gemm_prefill_dma_kernel<FP4, BM, BN, NBUF, WGM, WGN, FP4A, SPS, SLAB_KB>;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    // tile-rows per group of the tile order: 4 for 256-row tiles, 8 below
    // (one box, two alternating passes, 4 against 8: the MXFP4 gate_up at
    // M = 4096 552.6 against 575.1 us, W4A4 468.6 against 486.2, at M = 512
    // 95.4 against 96.9, 4096x7168x8192 212.5-213.7 against 214.9-216.2;
    // 2048x4096x1024 on 128x128 tiles 18.1 against 17.2 with bias, so
    // those keep 8; 2 and 16 slower on both)
    const int group_m = BM >= 256 ? 4 : 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(WGM * WGN * 64), 0, st, a, lda, as, w,
                       ldw, ws, cs, bias, epi, y, ldy, (int)M, (int)N, (int)K, group_m, a_e8m0,
                       GroupArgs{nullptr, 0, 0});
    return hipGetLastError();
}

// The grouped form over E experts: a grid of (m-tiles of max_rows) x
// (n-tiles) per expert, experts on the grid's y.
template <bool FP4, int BM, int BN, int NBUF, int WGM = 2, int WGN = 2, int SPS = 1, int SLAB_KB = 0,
          int WBUF = NBUF>
hipError_t launch_tile_dma_grouped(const uint8_t *a, int64_t lda, const float *as,
                                   const int32_t *off, int64_t E, int64_t max_rows, int64_t T,
                                   const uint8_t *w, int64_t ldw, int64_t w_estride,
                                   const uint8_t *ws, const uint16_t *bias, int epi, uint16_t *y,
                                   int64_t ldy, int64_t N, int64_t K, hipStream_t st) {
    auto kern = gemm_prefill_dma_kernel<FP4, BM, BN, NBUF, WGM, WGN, false, SPS, SLAB_KB, true, WBUF>;
    const int64_t rows = max_rows < T ? max_rows : T;
    const int64_t tiles = ((rows + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles, (unsigned)E), dim3(WGM * WGN * 64), 0, st, a, lda,
                       as, w, ldw, ws, nullptr, bias, epi, y, ldy, (int)rows, (int)N, (int)K, 8,
                       nullptr, GroupArgs{off, w_estride, (int)T});
    return hipGetLastError();
}


// ---- DMA-path planning. Workgroups run in rounds of one per CU; a round of
// tiles of one shape costs c * K + e (in units of one k of a 256x256 tile),
// c and e fitted to MI355X timings per tile shape: smaller tiles do less work
// per round at a lower MFMA efficiency. 128x128 tiles need at most 72 KB of
// LDS, so two share a CU and overlap one's prologue and epilogue with the
// other's MFMAs: a CU with two or more of them runs them in pairs, a pair
// costing PAIR x the work of two plus one e (fitted on 2048x4096x1024, where
// 512 such tiles run in 18.8 us against 20.0 us for 256 of 256x128).
struct TileShape {
    int bm, bn;
    double c, e;
    int per_cu;   // workgroups resident on a CU at once
};
constexpr TileShape SHAPES[] = {
    {256, 256, 1.0, 930.0, 1},
    {256, 128, 0.73, 465.0, 1},
    {128, 128, 0.415, 236.0, 2},
    // 64x64: a round of 256 at K = 5120 (the 512 x 2048 rest of the MXFP4
    // gate_up at M = 512) took 24.6 us next to 70.6 us for a round of
    // 256x256; no credit is given for their co-residence
    {64, 64, 0.388, 120.0, 1},
};
constexpr double LAUNCH_COST = 200.0;   // a second launch, same units
constexpr double PAIR = 1.06;

double shape_cost(const TileShape &t, int64_t M, int64_t N, int64_t K, int num_cus) {
    const int64_t tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    const int64_t per_cu = (tiles + num_cus - 1) / num_cus;
    if (t.per_cu == 2 && per_cu >= 2)
        return (double)((per_cu + 1) / 2) * (2.0 * PAIR * t.c * (double)K + t.e);
    return (double)per_cu * (t.c * (double)K + t.e);
}

// nshapes: how many of SHAPES the kernel variant in use offers (64x64 tiles
// need whole 16-byte loads per thread per stage: e4m3 weights, or MXFP4
// weights in two-step stages)
int best_shape(int64_t M, int64_t N, int64_t K, int num_cus, int nshapes, double *cost) {
    int best = -1;
    for (int i = 0; i < nshapes; ++i) {
        const double c = shape_cost(SHAPES[i], M, N, K, num_cus);
        if (best < 0 || c < *cost) { best = i; *cost = c; }
    }
    return best;
}

// MXFP4 tiles with their E8M0 rows in LDS (two-step stages): the largest
// K / 32 each variant holds.
constexpr int SLAB_KB_W4A8 = 224;   // K <= 7168 (256x256 tiles: 152 KB of LDS)
constexpr int SLAB_KB_W4A4 = 160;   // K <= 5120 (weight and activation slabs)

// num_cus: for the e4m3 128x128 tiles, which take two-step stages when at
// least two share every CU (2048x4096x1024: 18.6 -> 16.8 us) and one-step
// stages, whose ring runs a step further ahead, when a CU has one
// (4096x896 at K = 1024, 2048 and 4096: 11.9, 17.8 and 30.4 us against
// 12.4, 18.9 and 32.2 with two-step stages).
hipError_t launch_shape(int shape, bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                        const uint8_t *w, int64_t ldw, const uint8_t *ws, const float *cs,
                        const uint16_t *bias, int epi, uint16_t *y, int64_t ldy, int64_t M,
                        int64_t N, int64_t K, hipStream_t st, const uint8_t *a_e8m0, int num_cus) {
#define BSG_ARGS a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st
    if (a_e8m0) {   // W4A4: fp4 activations with their E8M0 scales, MXFP4 weights
        if (K % 128 == 0 && K / 32 <= SLAB_KB_W4A4) {
            switch (shape) {
            case 0: return launch_tile_dma<true, 256, 256, 2, 4, 2, true, 2, SLAB_KB_W4A4>(BSG_ARGS, a_e8m0);
            case 1: return launch_tile_dma<true, 256, 128, 2, 2, 2, true, 2, SLAB_KB_W4A4>(BSG_ARGS, a_e8m0);
            case 2: return launch_tile_dma<true, 128, 128, 2, 2, 2, true, 2, SLAB_KB_W4A4>(BSG_ARGS, a_e8m0);
            default: return launch_tile_dma<true, 64, 64, 2, 2, 2, true, 2, SLAB_KB_W4A4>(BSG_ARGS, a_e8m0);
            }
        }
        switch (shape) {
        case 0: return launch_tile_dma<true, 256, 256, 4, 4, 2, true>(BSG_ARGS, a_e8m0);
        case 1: return launch_tile_dma<true, 256, 128, 4, 2, 2, true>(BSG_ARGS, a_e8m0);
        default: return launch_tile_dma<true, 128, 128, 4, 2, 2, true>(BSG_ARGS, a_e8m0);
        }
    }
    if (fp4 && K % 128 == 0 && K / 32 <= SLAB_KB_W4A8) {
        switch (shape) {
        case 0: return launch_tile_dma<true, 256, 256, 2, 4, 2, false, 2, SLAB_KB_W4A8>(BSG_ARGS);
        case 1: return launch_tile_dma<true, 256, 128, 2, 2, 2, false, 2, SLAB_KB_W4A8>(BSG_ARGS);
        case 2: return launch_tile_dma<true, 128, 128, 2, 2, 2, false, 2, SLAB_KB_W4A8>(BSG_ARGS);
        default: return launch_tile_dma<true, 64, 64, 2, 2, 2, false, 2, SLAB_KB_W4A8>(BSG_ARGS);
        }
    }
    switch (shape) {
    case 0:
        // MXFP4 weights: eight waves (4 x 2, each 64 x 128) measured faster
        // than four for 256x256 tiles; e4m3 weights: four
        if (fp4) return launch_tile_dma<true, 256, 256, 4, 4, 2>(BSG_ARGS);
        return launch_tile_dma<false, 256, 256, 4>(BSG_ARGS);
    case 1:
        return fp4 ? launch_tile_dma<true, 256, 128, 4>(BSG_ARGS)
                   : launch_tile_dma<false, 256, 128, 4>(BSG_ARGS);
    case 2:
        if (fp4) return launch_tile_dma<true, 128, 128, 4>(BSG_ARGS);
        if (((M + 127) / 128) * ((N + 127) / 128) >= 2 * (int64_t)num_cus)
            return launch_tile_dma<false, 128, 128, 2, 2, 2, false, 2>(BSG_ARGS);
        return launch_tile_dma<false, 128, 128, 4>(BSG_ARGS);
    default:   // 64x64: e4m3 weights only here (the planner offers it to MXFP4 only with slabs)
        return fp4 ? launch_tile_dma<true, 128, 128, 4>(BSG_ARGS)
                   : launch_tile_dma<false, 64, 64, 4>(BSG_ARGS);
    }
#undef BSG_ARGS
}

// One launch of the cheapest tile shape, or two launches over column ranges
// [0, N1) and [N1, N): 256x256 tiles in whole rounds over the first, the
// cheapest shape over the rest (a last round that 256x256 tiles would leave
// part idle can be filled by smaller tiles). The two write disjoint columns.
hipError_t launch_prefill_dma(bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                              const uint8_t *w, int64_t ldw, const uint8_t *ws, const float *cs,
                              const uint16_t *bias, int epi, uint16_t *y, int64_t ldy, int64_t M,
                              int64_t N, int64_t K, int num_cus, hipStream_t st,
                              const uint8_t *a_e8m0 = nullptr) {
    const bool slab = fp4 && K % 128 == 0 && K / 32 <= (a_e8m0 ? SLAB_KB_W4A4 : SLAB_KB_W4A8);
    const int nshapes = (int)(sizeof(SHAPES) / sizeof(SHAPES[0])) - (fp4 && !slab ? 1 : 0);
    double one_cost = 0.0;
    const int one = best_shape(M, N, K, num_cus, nshapes, &one_cost);
    const int64_t mt = (M + 255) / 256, t256 = mt * ((N + 255) / 256);
    const int64_t rounds = t256 / num_cus;
    const int64_t nt1 = rounds > 0 ? rounds * num_cus / mt : 0;
    const int64_t n1 = nt1 * 256;
    if (n1 > 0 && n1 < N) {
        const double c1 = shape_cost(SHAPES[0], M, n1, K, num_cus);
        double c2 = 0.0;
        const int two = best_shape(M, N - n1, K, num_cus, nshapes, &c2);
        if (c1 + c2 + LAUNCH_COST < one_cost) {
            hipError_t e = launch_shape(0, fp4, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy,
                                        M, n1, K, st, a_e8m0, num_cus);
            if (e != hipSuccess) return e;
            const int64_t kb = K / 32;
            const uint8_t *w2 = w + n1 * ldw;
            const uint8_t *ws2 = ws ? ws + (fp4 ? n1 * kb : (n1 / 32) * kb) : nullptr;
            const float *cs2 = cs ? cs + n1 : nullptr;
            const uint16_t *bias2 = bias ? bias + n1 : nullptr;
            return launch_shape(two, fp4, a, lda, a_scale, w2, ldw, ws2, cs2, bias2, epi, y + n1,
                                ldy, M, N - n1, K, st, a_e8m0, num_cus);
        }
    }
    return launch_shape(one, fp4, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K, st,
                        a_e8m0, num_cus);
}

}  // namespace

// Grouped W4A8 for prefill-sized expert batches: MXFP4 weights, 64x64 tiles
// for at most 64 rows per expert, 128x128 up to 128, 160x256 (four waves
// side by side, each 160 x 64) up to 160, 192x256 (2 x 2 waves) up to 192,
// else 256x256 (every n-tile re-reads its expert's rows, so wider tiles halve
// that traffic). An expert's rows past its last tile row are zeros the
// MFMAs still process, so the tile height follows the row bound: with
// uniform top-8 routing of 512 tokens over 32 experts an expert gets about
// 128 +- 10 rows. With the tile's E8M0 rows in LDS when K % 128 == 0 and
// K / 32 <= 224 (K <= 7168), else one-step stages. Measured on 512 tokens
// top-8 over 32 experts of 4096 x 7168 (at most 142 rows): 245 us with
// 256x256 tiles and per-step scale loads, 210 us with the scale slab, 186 us
// with 192-row and 181 us with 160-row tiles, 166 us with the 160- and
// 192-row tiles' W stages in a ring of three (each expert's weights are read
// once, from HBM, so their loads get a stage more to land).
hipError_t launch_gemm_grouped_prefill(const uint8_t *a, int64_t lda, const float *a_scale,
                                       const int32_t *offsets, int64_t E, int64_t max_rows,
                                       const uint8_t *w, int64_t ldw, int64_t w_estride,
                                       const uint8_t *ws, const uint16_t *bias, int epi, uint16_t *y,
                                       int64_t ldy, int64_t T, int64_t N, int64_t K, hipStream_t st) {
#define BSG_GARGS a, lda, a_scale, offsets, E, max_rows, T, w, ldw, w_estride, ws, bias, epi, y, ldy, N, K, st
    if (K % 128 == 0 && K / 32 <= SLAB_KB_W4A8) {
        if (max_rows <= 64) return launch_tile_dma_grouped<true, 64, 64, 2, 2, 2, 2, SLAB_KB_W4A8>(BSG_GARGS);
        if (max_rows <= 128) return launch_tile_dma_grouped<true, 128, 128, 2, 2, 2, 2, SLAB_KB_W4A8>(BSG_GARGS);
        if (max_rows <= 160) return launch_tile_dma_grouped<true, 160, 256, 2, 1, 4, 2, SLAB_KB_W4A8, 3>(BSG_GARGS);
        if (max_rows <= 192) return launch_tile_dma_grouped<true, 192, 256, 2, 2, 2, 2, SLAB_KB_W4A8, 3>(BSG_GARGS);
        return launch_tile_dma_grouped<true, 256, 256, 2, 4, 2, 2, SLAB_KB_W4A8>(BSG_GARGS);
    }
    if (max_rows <= 128) return launch_tile_dma_grouped<true, 128, 128, 4>(BSG_GARGS);
    return launch_tile_dma_grouped<true, 256, 256, 4, 4, 2>(BSG_GARGS);
#undef BSG_GARGS
}

hipError_t launch_gemm_prefill_w4a4(const uint8_t *a, int64_t lda, const uint8_t *a_e8m0,
                                    const uint8_t *w, int64_t ldw, const uint8_t *ws,
                                    const uint16_t *bias, int epi, uint16_t *y, int64_t ldy,
                                    int64_t M, int64_t N, int64_t K, int num_cus, hipStream_t st) {
    return launch_prefill_dma(true, a, lda, nullptr, w, ldw, ws, nullptr, bias, epi, y, ldy, M, N,
                              K, num_cus, st, a_e8m0);
}

hipError_t launch_gemm_prefill(bool fp4, const uint8_t *a, int64_t lda, const float *a_scale,
                               const uint8_t *w, int64_t ldw, const uint8_t *ws, const float *cs,
                               const uint16_t *bias, int epi, uint16_t *y, int64_t ldy, int64_t M,
                               int64_t N, int64_t K, int num_cus, hipStream_t st) {
    if (K % 64 == 0)   // whole steps: LDS-mode staging
        return launch_prefill_dma(fp4, a, lda, a_scale, w, ldw, ws, cs, bias, epi, y, ldy, M, N, K,
                                  num_cus, st);
    // K % 64 == 32: the register-staged kernel on 128x128 tiles at every
    // size (its 256x256 form needs more registers than a lane has and
    // spills; shapes with K % 64 == 32 are a fallback, several times slower
    // than the LDS-mode path either way)
    (void)num_cus;
    return fp4 ? launch_tile<true, 128, 128, 2, 2>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y,
                                                   ldy, M, N, K, st)
               : launch_tile<false, 128, 128, 2, 2>(a, lda, a_scale, w, ldw, ws, cs, bias, epi, y,
                                                    ldy, M, N, K, st);
}

}  // namespace bsg
