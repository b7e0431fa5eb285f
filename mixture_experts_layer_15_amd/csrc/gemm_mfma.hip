// gemm_mfma.hip -- bf16 grouped expert GEMMs on gfx950 MFMA.
//
//   gate/up:  h = GELU_erf(X_e W_gate[e]) * (X_e W_up[e])   (GeGLU applied to
//             the accumulators in registers; only h is written -- the fusion of
//             GeGLU into the matmul that "AMD GPU深度学习优化与ZAYA1大模型实践"
//             section 3.2 describes for its expert MLP)
//   down:     O = h_e W_down[e]
//
// Workgroup: 8 waves as WM (M) x 8/WM (N), two per SIMD, so that one wave's LDS
// reads, barrier waits and MFMA issue gaps are covered by the other's MFMAs.
// A wave owns MI x NJ tiles of 16 x 16 (v_mfma_f32_16x16x32_bf16, fp32
// accumulators in registers), so the workgroup tile is (16 MI WM) rows x
// (16 NJ 8/WM) B-columns.  For gate/up the
// B-columns are half W_gate and half the same W_up columns, and a wave's gate
// tile j and up tile j + NJ/2 cover the same h columns: GeGLU is elementwise
// on matching registers.
//
// Data path per K-step of 64: global_load_lds (16 bytes per lane, straight
// into LDS, no VGPR round trip) fills one of two LDS stages while the other is
// consumed; each wave issues whole 1 KB rows-blocks, choosing per lane the
// global 16-byte chunk that belongs at LDS position base + 16 * lane, which
// applies an XOR swizzle that spreads the fragment reads over the LDS banks.
// A fragments: ds_read_b128 (row-major rows, K contiguous).  B fragments:
// ds_read_b64_tr_b16 on the weight tile kept in its [K][N] layout (each
// 16-lane group reads a 4 x 16 block; lane n receives column n).
// Rows past the expert's last row are clamped on load and their MFMAs are
// skipped per 16-row subtile.  The epilogue stores 8-byte pieces straight
// from the accumulators, except the 256-row down GEMM's, which goes through
// LDS and stores whole 128-byte row pieces.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "tiles.h"

#include <type_traits>

namespace moe {
namespace {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int GM = 4;   // M-tiles per group in the tile order (tiles.h)

// LDS swizzles.  An A row holds BK bf16 = BK/8 chunks of 16 bytes; chunk c of
// row r sits in slot c ^ fa(r), fa spreading the 16 rows a fragment read
// touches over distinct banks.  B rows hold 16-byte chunks too; chunk c of
// row r sits in slot c ^ 2 h(r) (below): the even mask keeps each aligned
// pair of chunks (the 32 bytes one transposing read takes from a row)
// together.  XOR is an involution, so the same map gives slot -> chunk when
// filling and chunk -> slot when reading.
template <int BKT>
__device__ __forceinline__ int fa(int r) {
    return BKT == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
// Pair swizzle h(r) of a B row holding CPR chunks (CPR/2 pairs of 32 bytes).
// One transposing read covers 16 rows, {0..3, 8..11, 16..19, 24..27} + base
// (four 16-lane groups), 32 bytes each; the LDS serves 256 bytes (eight
// 32-byte units) per pass, two groups at a time.  Rows of 256 or 512 bytes
// all start on the same bank, so the 8 rows of a pass need 8 distinct pair
// slots: h = (r & 3) | (r >> 3 & 1) << 2.  Rows of 128 bytes alternate
// between the two halves of the banks, so the 4 rows on each half need 4
// distinct slots: h = (r >> 1 & 1) | (r >> 3 & 1) << 1.  The fragment rows of
// one lane differ only in bits 2 and 5+ of r, so h is a lane constant.
template <int CPR>
__device__ __forceinline__ int hb(int r) {
    if (CPR == 8) return ((r >> 1) & 1) | (((r >> 3) & 1) << 1);
    return (r & 3) | (((r >> 3) & 1) << 2);
}

// x, hidden from the optimizer: values derived from it inside a loop are
// recomputed there instead of being hoisted out and kept live (or spilled)
// across the whole loop.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <bool GATEUP, int MI, int NJ, int BKT, int NA, int NB, int WM>
struct Shape {
    static constexpr int WAVES = 8;                 // WM (M) x WN (N)
    static constexpr int WN = WAVES / WM;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BM = 16 * MI * WM;         // rows per tile
    static constexpr int BN = 16 * NJ * WN;         // B-columns per tile
    static constexpr int KS = BKT / 32;             // 32-deep MFMA steps per stage
    static constexpr int A_ROWB = BKT * 2;          // bytes per A row
    static constexpr int ACH = BKT / 8;             // 16-byte chunks per A row
    static constexpr int A_RPK = 1024 / A_ROWB;     // A rows per 1 KB wave-load
    static constexpr int NSUB = GATEUP ? 2 : 1;     // B sub-tiles (W_gate, W_up)
    static constexpr int BNS = BN / NSUB;           // columns per sub-tile
    static constexpr int RB = BNS * 2;              // bytes per sub-tile row
    static constexpr int SUB = BKT * RB;            // bytes per sub-tile
    static constexpr int A_BYTES = BM * A_ROWB;     // one A stage
    static constexpr int B_BYTES = NSUB * SUB;      // one B stage
    // waves 0-3 fill the A stages, waves 4-7 the B stages (1 KB wave-loads)
    static constexpr int A_LOADS = A_BYTES / 4096;  // per A-loading wave per stage
    static constexpr int B_LOADS = B_BYTES / 4096;  // per B-loading wave per stage
    static constexpr int SUB_LOADS = SUB / 1024;    // wave-loads per sub-tile
    static constexpr int CPR = RB / 16;             // 16-byte chunks per sub-tile row
    static constexpr int RPK = 1024 / RB;           // sub-tile rows per 1 KB
    static constexpr int OUTC = GATEUP ? BN / 2 : BN;       // output columns per tile
    static constexpr int OUTW = OUTC / WN;                  // output columns per wave
    static constexpr int U = NA > NB ? NA : NB;              // K-loop unroll (static buffers)
    static_assert(U % NA == 0 && U % NB == 0, "the larger stage count is a multiple of the smaller");
    static_assert(BKT == 32 || BKT == 64, "K-step");
    static_assert(WM == 2 || WM == 4, "wave layout");
    static_assert(!GATEUP || NJ % 2 == 0, "gate and up halves");
    static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "whole wave-loads per loader");
    static_assert(SUB_LOADS % B_LOADS == 0 || B_LOADS % SUB_LOADS == 0, "uniform sources");
    static_assert(CPR <= 32 && CPR >= 8, "swizzle stays inside a row");
    static_assert(NA >= 2 && NA <= 4 && NB >= 2 && NB <= 8, "stage counts");
    static_assert(NA * A_BYTES + NB * B_BYTES + 4096 <= 160 * 1024, "LDS budget");
    static_assert(A_LOADS <= KS * MI && B_LOADS <= KS * MI, "a slot per wave-load");
};

// Per-lane constants of the fragment reads.
struct FragLane {
    int a_rd, a_sw, g4, b_rd;
};

// One stage: KS steps of 32 in K.  B fragments through transposing reads, A
// fragments prefetched one subtile ahead, MFMAs of the wave's valid 16-row
// subtiles (FULL: all MI, no branches).  iss(slot) is called once per
// (ks, subtile) slot, before that subtile's MFMAs, to issue this wave's share
// of a later stage's loads spread over the stage: issued in one burst, the
// loads back up the CU's vector memory queue and stall the issuing wave while
// its MFMAs wait.
template <int MI, int NJ, int KS, int A_ROWB, int RB, bool FULL, bool PRIO, typename Iss>
__device__ __forceinline__ void mfma_stage(const char* __restrict__ sa,
                                           const char* __restrict__ sbb,
                                           f32x4 (&acc)[MI][NJ], int nvm, const FragLane& fl,
                                           const int (&b_sub)[NJ], const int (&b_pair)[NJ],
                                           Iss&& iss) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        bf16x8 bfr[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const char* p = sbb + b_sub[j] + ks * 32 * RB + fl.b_rd + b_pair[j];
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * RB));
            bfr[j] = __builtin_bit_cast(
                bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        const int a_ch = ((ks * 4 + fl.g4) ^ fl.a_sw) << 4;
        bf16x8 a_cur = *(const bf16x8*)(sa + fl.a_rd + a_ch);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            iss(ks * MI + i);
            const int in = (i + 1 < MI) ? i + 1 : i;
            const bf16x8 a_nxt = *(const bf16x8*)(sa + fl.a_rd + in * 16 * A_ROWB + a_ch);
            if (FULL || i < nvm) {
                // raised wave priority while this wave issues its MFMAs, so the
                // other wave's loads and LDS reads on the SIMD wait for them
                // rather than the other way round (1-2% faster on the 2 x 4
                // wave layouts, 3% slower on the 4 x 2 one)
                if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], a_cur, acc[i][j],
                                                                        0, 0, 0);
                if (PRIO) __builtin_amdgcn_s_setprio(0);
            }
            a_cur = a_nxt;
        }
    }
}

// Wait until at most `later` of this wave's stages issued after the one to be
// read are still in flight (each stage is LOADS of this wave's wave-loads),
// and for this wave's LDS reads, then barrier: every wave's part of the stage
// has landed, and every wave is done reading the buffers about to be
// refilled.  A bare s_barrier: __syncthreads() adds a workgroup release
// fence, which waits for every outstanding vector memory operation --
// including the later stages' prefetches.
template <int LOADS>
__device__ __forceinline__ void stage_sync(int later) {
    switch (later) {
        case 0: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LOADS) : "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * LOADS) : "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(3 * LOADS) : "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(4 * LOADS) : "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(5 * LOADS) : "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(6 * LOADS) : "memory"); break;
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <bool GATEUP, int MI, int NJ, int BKT, int NA, int NB, int WM>
__global__ __launch_bounds__(512, 1) void gemm_mfma_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, uint16_t* __restrict__ C2,
    const int32_t* __restrict__ off, const int32_t* __restrict__ a_rows, int E, int K, int N,
    int dense_rows, const float* __restrict__ bias, int act, int rlo, int rhi,
    const float* __restrict__ gate, const int32_t* __restrict__ tor, uint16_t* __restrict__ Y,
    int ksplit, float* __restrict__ P, long long p_stride) {
    using S = Shape<GATEUP, MI, NJ, BKT, NA, NB, WM>;
    // one distinct __shared__ array per stage buffer, so that the compiler can
    // tell the reads of one stage from the fills of the others
    __shared__ __attribute__((aligned(1024))) char sa0[S::A_BYTES];
    __shared__ __attribute__((aligned(1024))) char sa1[S::A_BYTES];
    __shared__ __attribute__((aligned(1024))) char sa2[NA > 2 ? S::A_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sa3[NA > 3 ? S::A_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sb0[S::B_BYTES];
    __shared__ __attribute__((aligned(1024))) char sb1[S::B_BYTES];
    __shared__ __attribute__((aligned(1024))) char sb2[NB > 2 ? S::B_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sb3[NB > 3 ? S::B_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sb4[NB > 4 ? S::B_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sb5[NB > 5 ? S::B_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sb6[NB > 6 ? S::B_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sb7[NB > 7 ? S::B_BYTES : 16];
    __shared__ TileTable tt;
    __shared__ long long s_wave[S::WAVES];

    const int ntn = (N + S::OUTC - 1) / S::OUTC;
    build_tile_table<S::BM>(off, E, ntn, tt, s_wave, dense_rows, rlo, rhi);
    // ksplit > 1 (plain GEMMs only): each output tile is computed as ksplit
    // tiles over consecutive K slices, adjacent in the tile order, each
    // writing its fp32 partial product to P + slice * p_stride
    const long long total = tt.start[E] * ksplit;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w / S::WN, wn = w % S::WN;
    // Who loads what.  On 256-row tiles (the long-sequence layer) every wave
    // loads an eighth of each stage of both operands, its weight pieces
    // first (BAL): the weight slices miss in L2 more often than the
    // activation rows, and with waves 4-7 loading all of them the activation
    // loaders waited at each stage's barrier for a quarter of their time
    // (balanced: gate/up 9.61-9.69 -> 9.33-9.34 ms, down 4.81-4.85 -> 4.67-4.70
    // ms, alternated on one GPU, bit-identical; activation pieces first
    // 9.41 against 9.13 ms, loads spread over the whole stage 10.5 ms).
    // Otherwise waves 0-3 fill the A stages and 4-7 the B stages: on the
    // 640-row tiles, where the weights stream from HBM, the balanced loads
    // measured 8-10% slower, and the 320-row stages do not split into
    // eighths of whole 1 KB wave-loads.
    constexpr bool BAL = NA == NB && S::BM == 256 && S::A_BYTES % 8192 == 0 &&
                         S::B_BYTES % 8192 == 0;
    constexpr int AL = S::A_BYTES / 8192, BL = S::B_BYTES / 8192;   // wave-loads per wave (BAL)
    const bool a_loader = w < 4;
    const int lw = w & 3;                   // index among the loaders of its operand
    const int c16 = lane & 15, g4 = lane >> 4;
    const int G = gridDim.x;
    const int nk = K / BKT / ksplit;   // K-steps per tile

    // Per-lane LDS read offsets: the rows a lane reads differ only in
    // multiples of 16 (A) or 4 (B), so the swizzles are lane constants.
    FragLane fl;
    fl.a_rd = (wm * MI * 16 + c16) * S::A_ROWB;
    fl.a_sw = fa<BKT>(c16);
    fl.g4 = g4;
    const int hl = hb<S::CPR>(g4 * 8 + (c16 >> 2));   // = h of every B row this lane reads
    fl.b_rd = (g4 * 8 + (c16 >> 2)) * S::RB + ((c16 >> 1) & 1) * 16 + (c16 & 1) * 8;
    int b_sub[NJ], b_pair[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        int sub, colS;
        if (GATEUP) {
            sub = (j < NJ / 2) ? 0 : 1;
            colS = wn * (S::BNS / S::WN) + (j % (NJ / 2)) * 16;
        } else {
            sub = 0;
            colS = wn * (S::BN / S::WN) + j * 16;
        }
        b_sub[j] = sub * S::SUB;
        b_pair[j] = ((colS >> 4) ^ hl) * 32;
    }

    for (long long base = 0; base < total; base += G) {
        const long long t = sweep_tile(blockIdx.x, G, base, total);
        if (t < 0) continue;   // uniform across the workgroup
        const long long to = t / ksplit;                  // output tile
        const int slice = (int)(t - to * ksplit);         // its K slice
        const int kb = slice * nk;                        // first K-step of the slice
        int e, mtile, ntile;
        decode_tile<GM>(tt, E, ntn, to, e, mtile, ntile);
        const int row0 = (off ? off[e] : 0) + mtile * S::BM;
        const int rows = min(S::BM, (off ? off[e + 1] : dense_rows) - row0);
        const int n0 = ntile * S::OUTC;
        const int nvm = __builtin_amdgcn_readfirstlane(
            max(0, min(MI, (rows - wm * MI * 16 + 15) >> 4)));

        // uniform tile bases and this lane's 32-bit byte offsets for each of
        // its wave-loads (A loaders: A rows; B loaders: weight rows)
        const long long wofs = (long long)e * K * N + n0;
        // A rows: rows row0.. of A, or (a_rows != nullptr) the rows a_rows[row0..]
        // of A gathered (byte offsets then span all of A: the host checks they
        // fit 32 bits)
        const i32x4 rs_a = buffer_rsrc(a_rows ? A : A + (long long)row0 * K);
        const i32x4 rs_b0 = buffer_rsrc(B0 + wofs);
        const i32x4 rs_b1 = buffer_rsrc((GATEUP ? B1 : B0) + wofs);
        // this lane's offsets: (BAL) l_off[0 .. AL) for its A wave-loads and
        // l_off[AL .. AL + BL) for its B wave-loads, else those of its operand
        constexpr int NL = BAL ? AL + BL
                               : (S::A_LOADS > S::B_LOADS ? S::A_LOADS : S::B_LOADS);
        uint32_t l_off[NL];
        const int ln = opaque(lane);
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const bool is_a = BAL ? q < AL : a_loader;
            if (is_a) {
                const int wl = BAL ? w * AL + q : lw * S::A_LOADS + q;   // wave-load in the stage
                const int r = wl * S::A_RPK + ln / S::ACH;
                const int c = (ln % S::ACH) ^ fa<BKT>(r);
                const int rr = min(r, rows - 1);
                const int src = a_rows ? a_rows[row0 + rr] : rr;
                l_off[q] = (BAL || q < S::A_LOADS) ? ((uint32_t)src * (uint32_t)K + c * 8) * 2u
                                                   : 0u;
            } else {
                const int gl = BAL ? w * BL + (q - AL) : lw * S::B_LOADS + q;
                const int r = (gl % S::SUB_LOADS) * S::RPK + ln / S::CPR;
                const int c = (ln % S::CPR) ^ (hb<S::CPR>(r) << 1);
                const int col = min(n0 + c * 8, N - 8) - n0;
                l_off[q] = (BAL || q < S::B_LOADS) ? (r * N + col) * 2 : 0;
            }
        }

        // wave-load q of A stage kt / B stage kt into the stage buffer at LDS
        // address lb
        auto load_a = [&](int kt, uint32_t lb, int q) {
            load_to_lds(rs_a, l_off[q], (uint32_t)((kb + kt) * BKT * 2),
                        lb + ((BAL ? w * AL : lw * S::A_LOADS) + q) * 1024);
        };
        auto load_b = [&](int kt, uint32_t lb, int q) {
            const int gl = BAL ? w * BL + q : lw * S::B_LOADS + q;
            load_to_lds((GATEUP && gl >= S::SUB_LOADS) ? rs_b1 : rs_b0, l_off[BAL ? AL + q : q],
                        (uint32_t)(kb + kt) * (uint32_t)(BKT * 2) * (uint32_t)N,
                        lb + gl * 1024);
        };
        auto lds_base = [](char* p) { return __builtin_amdgcn_readfirstlane(lds_addr(p)); };

        f32x4 acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        char* abuf[4] = {sa0, sa1, sa2, sa3};
        char* bbuf[8] = {sb0, sb1, sb2, sb3, sb4, sb5, sb6, sb7};
        // prologue: A stages 0 .. NA-2, B stages 0 .. NB-2
        if constexpr (BAL) {
#pragma unroll
            for (int kt = 0; kt + 1 < NA; ++kt)
                if (kt < nk) {
                    const uint32_t lbb = lds_base(bbuf[kt]);
#pragma unroll
                    for (int q = 0; q < BL; ++q) load_b(kt, lbb, q);
                    const uint32_t lba = lds_base(abuf[kt]);
#pragma unroll
                    for (int q = 0; q < AL; ++q) load_a(kt, lba, q);
                }
        } else if (a_loader) {
#pragma unroll
            for (int kt = 0; kt + 1 < NA; ++kt)
                if (kt < nk) {
                    const uint32_t lb = lds_base(abuf[kt]);
#pragma unroll
                    for (int q = 0; q < S::A_LOADS; ++q) load_a(kt, lb, q);
                }
        } else {
#pragma unroll
            for (int kt = 0; kt + 1 < NB; ++kt)
                if (kt < nk) {
                    const uint32_t lb = lds_base(bbuf[kt]);
#pragma unroll
                    for (int q = 0; q < S::B_LOADS; ++q) load_b(kt, lb, q);
                }
        }

        // step k: wait for A and B stage k, run the MFMAs on stage k and,
        // spread among them, refill the buffers read at step k-1 with A stage
        // k+NA-1 (A loaders) or B stage k+NB-1 (B loaders), or both (BAL)
        auto k_loop = [&](auto full_tag, auto role_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            constexpr bool ROLE_A = decltype(role_tag)::value;
            constexpr int LOADS = BAL ? AL + BL : ROLE_A ? S::A_LOADS : S::B_LOADS;
            constexpr int NS = ROLE_A ? NA : NB;
            // slots per wave-load: spread over the whole stage with three or
            // more stages (two still in flight behind it), over its first
            // half with two, so that every load of the next stage has at
            // least half a stage of MFMAs to land before that stage's wait
            // (long-sequence layer, two 64-deep stages: gate/up 9.98 ->
            // 9.53 ms, down 5.28 -> 4.95 ms; the 320-row four-stage shapes
            // measured no gain)
            constexpr int STRIDE0 = S::KS * MI / LOADS / (NS == 2 ? 2 : 1);
            constexpr int STRIDE = STRIDE0 > 0 ? STRIDE0 : 1;
            for (int kt = 0; kt < nk; kt += S::U) {
#pragma unroll
                for (int s = 0; s < S::U; ++s) {
                    const int k = kt + s;
                    if (k >= nk) break;
                    stage_sync<LOADS>(min(nk - 1 - k, NS - 2));
                    const bool refill = k + NS - 1 < nk;
                    const uint32_t lb = lds_base(ROLE_A ? abuf[(s + NA - 1) % NA]
                                                        : bbuf[(s + NB - 1) % NB]);
                    const uint32_t lb2 = BAL ? lds_base(abuf[(s + NA - 1) % NA]) : 0u;
                    const uint32_t lb3 = BAL ? lds_base(bbuf[(s + NB - 1) % NB]) : 0u;
                    auto iss = [&](int slot) {
                        if (slot % STRIDE == 0 && slot / STRIDE < LOADS && refill) {
                            if constexpr (BAL) {
                                const int q = slot / STRIDE;   // B (weights) first
                                if (q < BL) load_b(k + NB - 1, lb3, q);
                                else load_a(k + NA - 1, lb2, q - BL);
                            } else if constexpr (ROLE_A) load_a(k + NA - 1, lb, slot / STRIDE);
                            else load_b(k + NB - 1, lb, slot / STRIDE);
                        }
                    };
                    mfma_stage<MI, NJ, S::KS, S::A_ROWB, S::RB, FULL, WM == 2>(
                        abuf[s % NA], bbuf[s % NB], acc, nvm, fl, b_sub, b_pair, iss);
                }
            }
        };
        if (BAL) {
            if (nvm == MI) k_loop(std::true_type{}, std::true_type{});
            else k_loop(std::false_type{}, std::true_type{});
        } else if (a_loader) {
            if (nvm == MI) k_loop(std::true_type{}, std::true_type{});
            else k_loop(std::false_type{}, std::true_type{});
        } else {
            if (nvm == MI) k_loop(std::true_type{}, std::false_type{});
            else k_loop(std::false_type{}, std::false_type{});
        }

        // epilogue straight from the accumulators: lane (g4, c16) of block
        // (i, j) holds output columns 4 g4 .. 4 g4 + 3 of row c16, one 8-byte
        // store per block.  Plain GEMMs may add a per-column fp32 bias and
        // apply GELU (act == 1).  gate/up with act == 2 stores the two
        // products themselves (x W_gate to C, x W_up to C2) instead of GeGLU.
        // The down GEMM with Y != nullptr (a top-1 layer that keeps every
        // token) writes the layer output itself: row r of expert order is
        // token t = tor[r], and y[t] = gate[t] * O[r], with O rounded to bf16
        // first and the product rounded like the combine rounds it, so the
        // result is bit-identical to writing O and combining.
        // Plain products of 64 columns per wave on 256-row tiles (the
        // long-sequence down GEMM writing O) go through LDS instead: each
        // 16-row block into this wave's 2 KB slice of the A stage buffer the
        // last K-step but one used (idle: nothing reads or fills it again in
        // this tile), then out in whole 128-byte row pieces, 8 rows per store,
        // against 16 rows x 8 bytes per store from the MFMA layout, which
        // moves about a quarter of the bytes per clock per CU (long-sequence
        // down 5.00 -> 4.80 ms).  Not taken elsewhere: on the 320-row tiles,
        // where the weights stream, it measured no faster, and for the GeGLU
        // output (32 columns per wave, staged per row half behind a barrier)
        // neither.  16-byte chunk c of row r sits in slot c ^ ((r >> 1) & 7).
        if constexpr (!GATEUP && S::BM == 256 && S::OUTW == 64 &&
                      S::WAVES * 2048 <= S::A_BYTES) {
            if (Y == nullptr && P == nullptr && bias == nullptr && act == 0 && (N & 7) == 0) {
                const int fb = (nk + NA - 2) % NA;
                char* const stg = (fb == 0 ? sa0 : fb == 1 ? sa1 : fb == 2 ? sa2 : sa3) + w * 2048;
                const int hl16 = opaque(lane);
                const int h16 = hl16 & 15, hg4 = hl16 >> 4;
                const int colw = n0 + wn * 64;
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    if (i >= nvm) continue;   // uniform: an empty block of this wave
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        bf16x4 v;
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = (__bf16)acc[i][jj][q];
                        // columns 16 jj + 4 g4 .. + 3: chunk 2 jj + g4 / 2, half g4 & 1
                        const int slot = (jj * 2 + (hg4 >> 1)) ^ ((h16 >> 1) & 7);
                        *(u32x2*)(stg + h16 * 128 + slot * 16 + (hg4 & 1) * 8) =
                            __builtin_bit_cast(u32x2, v);
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int rr = q * 8 + (hl16 >> 3), ch = hl16 & 7;
                        const u32x4 v =
                            *(const u32x4*)(stg + rr * 128 + ((ch ^ ((rr >> 1) & 7)) << 4));
                        const int r = wm * MI * 16 + i * 16 + rr;
                        if (r < rows && colw + ch * 8 < N)
                            *(u32x4*)(C + (long long)(row0 + r) * N + colw + ch * 8) = v;
                    }
                    // this block's reads are done before the next block's writes
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                continue;
            }
        }
        float bv[S::OUTW / 16][4];
#pragma unroll
        for (int jj = 0; jj < S::OUTW / 16; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gc = n0 + wn * S::OUTW + jj * 16 + g4 * 4 + q;
                bv[jj][q] = (!GATEUP && bias != nullptr && gc < N) ? bias[gc] : 0.f;
            }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int r = wm * MI * 16 + i * 16 + c16;
            if (i < nvm && r < rows) {
                if (!GATEUP && P != nullptr) {   // fp32 partial of this K slice
                    float* prow = P + slice * p_stride + (long long)(row0 + r) * N + n0;
#pragma unroll
                    for (int jj = 0; jj < S::OUTW / 16; ++jj) {
                        const int col = wn * S::OUTW + jj * 16 + g4 * 4;
                        if (n0 + col < N) *(f32x4*)(prow + col) = acc[i][jj];
                    }
                    continue;
                }
                uint16_t* crow = C + (long long)(row0 + r) * N + n0;
                float gr = 0.f;
                if (!GATEUP && Y != nullptr) {
                    const int t = tor[row0 + r];
                    crow = Y + (long long)t * N + n0;
                    gr = gate[t];
                }
#pragma unroll
                for (int jj = 0; jj < S::OUTW / 16; ++jj) {
                    const int col = wn * S::OUTW + jj * 16 + g4 * 4;
                    if (GATEUP && act == 2) {
                        bf16x4 vg, vu;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            vg[q] = (__bf16)acc[i][jj][q];
                            vu[q] = (__bf16)acc[i][jj + NJ / 2][q];
                        }
                        if (n0 + col < N) {
                            *(u32x2*)(crow + col) = __builtin_bit_cast(u32x2, vg);
                            *(u32x2*)(C2 + (long long)(row0 + r) * N + n0 + col) =
                                __builtin_bit_cast(u32x2, vu);
                        }
                        continue;
                    }
                    bf16x4 v;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float a = acc[i][jj][q];
                        float o;
                        if constexpr (GATEUP) {
                            o = gelu_erf_bf16(a) * acc[i][jj + NJ / 2][q];
                        } else {
                            o = a + bv[jj][q];
                            if (act == 1) o = gelu_erf_bf16(o);
                        }
                        v[q] = (__bf16)o;
                        if (!GATEUP && Y != nullptr)
                            v[q] = __builtin_bit_cast(
                                __bf16, (uint16_t)f32_to_bf16_bits(fmaf(gr, (float)v[q], 0.f)));
                    }
                    if (n0 + col < N) *(u32x2*)(crow + col) = __builtin_bit_cast(u32x2, v);
                }
            }
        }
        // LDS reads of this tile are done before the next tile's loads refill
        // the stage buffers (a bare barrier: the stores above need no wait)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
}

template <bool GATEUP, int MI, int NJ, int BKT, int NA, int NB, int WM = 2>
hipError_t launch_shape(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, uint16_t* C,
                        const int32_t* off, const int32_t* a_rows, int dense_rows,
                        const float* bias, int act, int E, int K, int N, long long max_rows, int cus,
                        hipStream_t s, uint16_t* C2 = nullptr, int rlo = 0,
                        int rhi = 0x7fffffff, const float* gate = nullptr,
                        const int32_t* tor = nullptr, uint16_t* Y = nullptr, int ksplit = 1,
                        float* P = nullptr, long long p_stride = 0) {
    using S = Shape<GATEUP, MI, NJ, BKT, NA, NB, WM>;
    const long long mt = (max_rows + S::BM - 1) / S::BM + E;   // >= sum_e ceil(rows_e / BM)
    const long long tiles = mt * ((N + S::OUTC - 1) / S::OUTC) * ksplit;
    long long g = std::min<long long>(cus, (tiles + 7) / 8 * 8);
    g = std::max<long long>(8, g / 8 * 8);
    hipLaunchKernelGGL((gemm_mfma_kernel<GATEUP, MI, NJ, BKT, NA, NB, WM>), dim3((unsigned)g),
                       dim3(S::THREADS), 0, s, A, B0, B1, C, C2, off, a_rows, E, K, N,
                       dense_rows, bias, act, rlo, rhi, gate, tor, Y, ksplit, P, p_stride);
    return hipGetLastError();
}

}  // namespace

// Tile shape policy.  Rows per expert are only known on the device; the host
// knows their mean (max_rows / E, exact when nothing is dropped).  Up to 512
// rows per expert on average the GEMMs take 320-row tiles: one M-tile covers a
// ZAYA1-like or wide-layer expert (about 256 rows: weight-streaming bound, so
// each weight tile is streamed once).  Above that, 256 x 256 tiles, whose
// waves load both operands (long-sequence layer, about 16k rows per expert:
// 16.5 against 17.4 ms per step on 320-row tiles before that; the skewed
// layer, 631 rows on average with its capacity-bound experts at 1280: 2.103
// -> 2.033 ms per step against 320-row tiles, which it took while the 256-row
// waves still split the operands; 1024 uniform rows: gate/up 2.41 -> 2.09 ms,
// down 1.15 -> 0.91 ms; 631 uniform rows: equal).
//   gate/up: 320 x 256, 32-deep K-steps in rings of four stages per operand
//     (three in flight while one is multiplied): 321 against 334 us with
//     64-deep steps in two stages on the ZAYA1-like layer, the same on the
//     wide layer.
//   down: 320 x 256 likewise when E * ceil(d / 256) tiles fill the CUs (each
//     CU then moves 36% fewer bytes per output than with 320 x 128: the wide
//     layer 2.95 -> 2.36 ms), else 320 x 128 with 64-deep K-steps (the
//     ZAYA1-like layer: 128 tiles of 320 x 256 would leave half the CUs idle,
//     261 against 214 us; 32-deep steps with 4 activation and 8 weight
//     stages measured 2% slower on this tile).  Its waves are arranged 4 (M) x 2 (N): 80 x 64 per wave
//     instead of 160 x 32 reads 27% fewer fragment bytes from LDS per stage
//     (measured 4% faster).
static bool tiles320(long long max_rows, int E) { return max_rows <= 512LL * E; }

// Between 320 and 640 rows per expert on average (the wide layer with 2-4
// experts per token: about 350 rows, up to 512 by its mean bound), 320-row
// tiles would take two M-tiles per expert, the second nearly empty, and so
// stream every weight tile twice.  There the GEMMs take 640 x 128 tiles (four
// waves in M, two in N, each still 160 x 64), 32-deep K-steps in rings of
// three stages per operand: one M-tile per expert, half the weight bytes per
// tile.  Measured with 351 rows per expert (E = 128, d = 4096, d_ff = 8192):
// gate/up 9.67 -> 7.64 ms, down 4.60 -> 3.61 ms; at 448 rows 9.76 -> 8.98
// and 4.53 -> 4.24 ms; at 512 rows 10.03 -> 9.75 and 4.83 -> 4.52 ms.  Rings
// of two activation and four or eight weight stages measured 15-25% slower.
static bool tiles640(long long max_rows, int E) {
    return max_rows > 320LL * E && max_rows <= 640LL * E;
}

// On 256-row tiles, experts with only a few rows (a skewed layer's tail) go
// to a second launch of 128 x 256 tiles with 32-deep K-steps and four stages
// per operand (more weight bytes in flight per CU for tiles that are all
// weight streaming); each launch skips the other's experts.  The per-row
// arithmetic is the same in every shape (K ascending in steps of 32), so the
// result is bit-identical to one launch.  Measured on the skewed layer (45 of
// 64 experts under 64 rows) when it ran on 256-row tiles: down 442 -> 399 us,
// gate/up 761 -> 740 us.  On the 320-row tiles it takes now, the same split
// measured slower (down 366 -> 420 us), so 320-row layers launch once.
constexpr int kFewRows = 64;
static bool split_few(long long max_rows, int E) { return !tiles320(max_rows, E); }

hipError_t launch_mfma_gate_up(const uint16_t* a, const int32_t* a_rows, const int32_t* off,
                               const uint16_t* w_gate,
                               const uint16_t* w_up, uint16_t* h, int E, int d, int d_ff,
                               long long max_rows, int cus, hipStream_t s) {
    if (tiles640(max_rows, E))
        return launch_shape<true, 10, 4, 32, 3, 3, 4>(a, w_gate, w_up, h, off, a_rows, 0, nullptr,
                                                      0, E, d, d_ff, max_rows, cus, s);
    const bool split = split_few(max_rows, E);
    const int lo = split ? kFewRows : 0;
    const hipError_t e =
        tiles320(max_rows, E)
            ? launch_shape<true, 10, 4, 32, 4, 4>(a, w_gate, w_up, h, off, a_rows, 0, nullptr, 0,
                                                  E, d, d_ff, max_rows, cus, s, nullptr, lo)
            : launch_shape<true, 8, 4, 64, 2, 2>(a, w_gate, w_up, h, off, a_rows, 0, nullptr, 0,
                                                 E, d, d_ff, max_rows, cus, s, nullptr, lo);
    if (e != hipSuccess || !split) return e;
    return launch_shape<true, 4, 4, 32, 4, 4>(a, w_gate, w_up, h, off, a_rows, 0, nullptr, 0, E,
                                              d, d_ff, max_rows, cus, s, nullptr, 0, kFewRows);
}

// Both products of the gate/up GEMM, unfused: g = X W_gate, u = X W_up (bf16),
// same tiles and schedule as the GeGLU-fused launch.
hipError_t launch_mfma_gate_up_pre(const uint16_t* a, const int32_t* a_rows, const int32_t* off,
                                   const uint16_t* w_gate, const uint16_t* w_up, uint16_t* g,
                                   uint16_t* u, int E, int d, int d_ff, long long max_rows,
                                   int cus, hipStream_t s) {
    if (tiles640(max_rows, E))
        return launch_shape<true, 10, 4, 32, 3, 3, 4>(a, w_gate, w_up, g, off, a_rows, 0, nullptr,
                                                      2, E, d, d_ff, max_rows, cus, s, u);
    const bool split = split_few(max_rows, E);
    const int lo = split ? kFewRows : 0;
    const hipError_t e =
        tiles320(max_rows, E)
            ? launch_shape<true, 10, 4, 32, 4, 4>(a, w_gate, w_up, g, off, a_rows, 0, nullptr, 2,
                                                  E, d, d_ff, max_rows, cus, s, u, lo)
            : launch_shape<true, 8, 4, 64, 2, 2>(a, w_gate, w_up, g, off, a_rows, 0, nullptr, 2,
                                                 E, d, d_ff, max_rows, cus, s, u, lo);
    if (e != hipSuccess || !split) return e;
    return launch_shape<true, 4, 4, 32, 4, 4>(a, w_gate, w_up, g, off, a_rows, 0, nullptr, 2, E,
                                              d, d_ff, max_rows, cus, s, u, 0, kFewRows);
}

hipError_t launch_mfma_grouped(const uint16_t* A, const int32_t* a_rows, const int32_t* off,
                               const uint16_t* B, uint16_t* C, int E, int K, int N,
                               long long max_rows, int cus, hipStream_t s, const float* gate,
                               const int32_t* tor, uint16_t* y) {
    const bool split = split_few(max_rows, E);
    const int lo = split ? kFewRows : 0;
    constexpr int HI = 0x7fffffff;
    if (tiles640(max_rows, E))
        return launch_shape<false, 10, 4, 32, 3, 3, 4>(A, B, nullptr, C, off, a_rows, 0, nullptr,
                                                       0, E, K, N, max_rows, cus, s, nullptr, 0,
                                                       HI, gate, tor, y);
    hipError_t e;
    if (!tiles320(max_rows, E))
        e = launch_shape<false, 8, 4, 64, 2, 2>(A, B, nullptr, C, off, a_rows, 0, nullptr, 0, E, K,
                                                N, max_rows, cus, s, nullptr, lo, HI, gate, tor, y);
    else if ((long long)E * ((N + 255) / 256) >= cus)
        e = launch_shape<false, 10, 4, 32, 4, 4>(A, B, nullptr, C, off, a_rows, 0, nullptr, 0, E,
                                                 K, N, max_rows, cus, s, nullptr, lo, HI, gate,
                                                 tor, y);
    else
        e = launch_shape<false, 5, 4, 64, 2, 4, 4>(A, B, nullptr, C, off, a_rows, 0, nullptr, 0,
                                                   E, K, N, max_rows, cus, s, nullptr, lo, HI,
                                                   gate, tor, y);
    if (e != hipSuccess || !split) return e;
    return launch_shape<false, 4, 4, 32, 4, 4>(A, B, nullptr, C, off, a_rows, 0, nullptr, 0, E, K,
                                               N, max_rows, cus, s, nullptr, 0, kFewRows, gate,
                                               tor, y);
}

// The down GEMM in two K slices on 320 x 256 tiles: fp32 partial products
// P[s][rows][d], s = 0, 1, to be summed by the consumer.  For layers whose
// 320 x 256 tiles alone would not fill the CUs (the ZAYA1-like layer: 128
// tiles), the two slices make 256 tiles, each CU moving 36% fewer bytes than
// with 320 x 128 tiles over the whole of K.
bool down_split_applies(long long max_rows, int E, int d, int d_ff, int cus) {
    return tiles320(max_rows, E) && (long long)E * ((d + 255) / 256) < cus &&
           d_ff % 128 == 0 && max_rows > 0;
}

hipError_t launch_mfma_down_split(const uint16_t* h, const int32_t* off, const uint16_t* w_down,
                                  float* P, long long p_stride, int E, int d, int d_ff,
                                  long long max_rows, int cus, hipStream_t s) {
    if (!down_split_applies(max_rows, E, d, d_ff, cus)) return hipErrorInvalidValue;
    return launch_shape<false, 10, 4, 64, 2, 2>(h, w_down, nullptr, nullptr, off, nullptr, 0,
                                                nullptr, 0, E, d_ff, d, max_rows, cus, s, nullptr,
                                                0, 0x7fffffff, nullptr, nullptr, nullptr, 2, P,
                                                p_stride);
}

hipError_t launch_mfma_down(const uint16_t* h, const int32_t* off, const uint16_t* w_down,
                            uint16_t* y_perm, int E, int d, int d_ff, long long max_rows,
                            int cus, hipStream_t s, const float* gate, const int32_t* tor,
                            uint16_t* y) {
    return launch_mfma_grouped(h, nullptr, off, w_down, y_perm, E, d_ff, d, max_rows, cus, s,
                               gate, tor, y);
}

// Dense bf16 GEMM C [M][N] = A [M][K] B [K][N] (+ bias[N]) (GELU when act ==
// 1), fp32 accumulation, one rounding to bf16: the same kernel with a single
// group of M rows.  Small products take 64 x 64 tiles so that they still
// spread over the CUs.
hipError_t launch_mfma_dense(const uint16_t* A, const uint16_t* B, const float* bias, int act,
                             uint16_t* C, int M, int K, int N, int cus, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const long long big_tiles = (long long)((M + 127) / 128) * ((N + 127) / 128);
    if (big_tiles >= cus)
        return launch_shape<false, 4, 2, 64, 2, 2>(A, B, nullptr, C, nullptr, nullptr, M, bias,
                                                    act, 1, K, N, M, cus, s);
    return launch_shape<false, 2, 1, 64, 2, 2>(A, B, nullptr, C, nullptr, nullptr, M, bias, act,
                                                1, K, N, M, cus, s);
}

}  // namespace moe
