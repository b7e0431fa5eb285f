// gemm_bw.hip -- the grouped GEMMs of the layer's backward pass on gfx950.
//
// The forward multiplies activations [rows][K] by weights [K][N].  Its
// backward needs the two other operand layouts:
//   NT  C[r][N] (+)= A[r][K] W[e]^T, W[e] stored [N][K]: dh = dy W_down^T and
//       dx = dg W_gate^T + du W_up^T over the rows r of each expert
//   TN  C[e][M][N] = sum over the rows r of expert e of A[r][M]^T B[r][N]: the
//       weight gradients, a different reduction length (its kept rows) per expert
// In NT both operands are stored with K contiguous, in TN both with K as the
// row index.  Both MFMA operands of v_mfma_f32_16x16x32_bf16 share one
// register layout (lane l: index l % 16, K values 8 (l / 16) .. + 7), so one
// fragment reader per storage order serves A and B: ds_read_b128 for K
// contiguous, the transposing ds_read_b64_tr_b16 for K rows (a 16-lane group
// reads a 4 x 16 block; lane n receives column n).
//
// Workgroup: WAVES waves as WMW (M) x WAVES/WMW (N), tile BM x BN, K-steps of
// 32, a ring of NS LDS stages per operand filled by buffer_load_dwordx4 ...
// lds (16 bytes per lane straight into LDS, no register round trip): NS - 1
// stages are in flight while one is multiplied.  A persistent grid walks the
// tiles in sweeps of one grid; inside a sweep each XCD takes a contiguous
// run, so tiles of one expert spread over the whole chip.  Every wave fills
// its share of the 1 KB blocks of each operand stage, each lane picking the
// global chunk that belongs at its LDS position (XOR swizzles that spread the fragment
// reads over the banks).  Rows past an expert's end: in NT they are clamped
// (their results are not stored); in TN, where they are reduction steps,
// the buffer descriptor's record count ends at the expert's last row, so they
// read as zeros.  fp32 results written from the accumulators, four
// consecutive columns per lane (weights in the MFMA's first operand slot).
// The NT launch for dh_raw = dy W_down^T instead ends in the GeGLU backward
// (EPI): it reads g, u of its elements and writes dg, du, gate h (bf16) and
// per-row partial sums of dgate, so dh_raw is never stored (2.1 GB of fp32
// on the long-sequence layer, written and read back by a separate kernel
// before).  Timed against that separate kernel on one GPU, alternating: the
// long-sequence backward 45.95 -> 45.74 ms, skewed 7.46 -> 7.38, ZAYA1-like
// 2.121 -> 2.134, wide 28.39 -> 28.57 ms: the epilogue's stores leave at the
// same per-CU rate the separate kernel's did.
#include "common.h"
#include "geglu_bwd.h"
#include "kernels.h"
#include "lds_dma.h"
#include "tiles.h"

namespace moe {
namespace {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// x, hidden from the optimizer: lane constants derived from it inside the
// epilogue are computed there instead of being hoisted out of the tile loop
// and kept live through the K-loop.
__device__ __forceinline__ int hidden(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <int BM, int BN, int WAVES, int WMW, int NS, int TK>
struct BwShape {
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WNW = WAVES / WMW;
    static constexpr int MI = BM / WMW / 16;            // 16-row blocks per wave
    static constexpr int NJ = BN / WNW / 16;            // 16-column blocks per wave
    static constexpr int A_STAGE = BM * TK * 2;         // bytes of one A stage
    static constexpr int B_STAGE = BN * TK * 2;
    static constexpr int A_WL = A_STAGE / 1024 / WAVES; // 1 KB wave-loads per wave and stage
    static constexpr int B_WL = B_STAGE / 1024 / WAVES;
    static constexpr int LOADS = A_WL + B_WL;
    static constexpr int KS = TK / 32;                  // MFMA steps per stage
    static constexpr int CR = TK / 8;                   // 16-byte chunks per K-contiguous row
    static_assert(TK == 32 || TK == 64, "K-step");
    static_assert(A_WL >= 1 && B_WL >= 1 && A_WL * WAVES * 1024 == A_STAGE &&
                  B_WL * WAVES * 1024 == B_STAGE, "whole wave-loads per wave");
    static_assert(MI >= 1 && NJ >= 1 && BM % (16 * WMW) == 0 && BN % (16 * WNW) == 0, "waves");
    static_assert(BM == 128 || BM == 256 || BM == 320, "K-row stage rows of 256 or 512 bytes");
    static_assert(BN == 128 || BN == 256, "K-row stage rows of 256 or 512 bytes");
    static_assert(NS >= 2 && NS <= 4, "stages");
    static_assert(NS * (A_STAGE + B_STAGE) + 4096 <= 160 * 1024, "LDS budget");
};

// K-contiguous stage [rows][TK]: row r at 2 TK r bytes, 16-byte slot s of the
// row holds K chunk s ^ kc_sw(r).  The 16 rows of a fragment read
// (r = base + 0..15) then spread over the banks: rows of 64 bytes (TK = 32)
// take four slots per bank group, rows of 128 bytes eight.
template <int TK>
__device__ __forceinline__ int kc_sw(int r) { return TK == 32 ? (r >> 2) & 3 : (r >> 1) & 7; }
// K-row stage [32 K rows][columns]: row k at k * (2 columns) bytes, 32-byte
// pair slot p holds column pair p ^ kr_sw(k) (the pair swizzle of the forward
// GEMM for rows of 256 or 512 bytes).
__device__ __forceinline__ int kr_sw(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

// Operands of one launch.  NT runs ksplit parts per source group: part p
// covers the K slice p % ksplit of K / ksplit, into its own fp32 buffer
// C + p * c_stride ([rows][N]); the parts are summed by their consumer, in
// part order.  With fuse == 0 each of the nsrc sources is its own group (part
// p multiplies source p / ksplit: A[s] [rows][K] by W = B[s] [E][N][K]); with
// fuse == 1 (nsrc == 2) one accumulator runs over the slice of source 0 and
// then the same slice of source 1, so the two products are summed in the
// tile and there are ksplit parts in all.  TN uses A[0], B[0] and C.
struct BwOperands {
    const uint16_t* A[2];
    const uint16_t* B[2];
    float* C;
    long long c_stride;
    int nsrc, ksplit, fuse;
    // GeGLU epilogue (NT, one source, one K slice): the product is dh_raw;
    // G, U (bf16 [rows][N], in place -> dG, dU), gH out, gate per row, and
    // the partial sums of h . dh_raw over each wave's 64 columns,
    // dot[row][N / 64]
    uint16_t* G;
    uint16_t* U;
    uint16_t* gH;
    const float* row_gate;
    float* dot;
};

// MODE 0 (NT): tiles from the expert row counts (ragged M) for every part;
//   A rows row0.. of A[s], B = W[e] of source s, one K slice.
// MODE 1 (TN): tiles (e, M-tile, N-tile); reduction over the rows off[e] ..
//   off[e+1]-1 of A [rows][M] and B [rows][N].
template <int MODE, int BM, int BN, int WAVES, int WMW, int NS, int TK, bool EPI = false>
__global__ __launch_bounds__(64 * WAVES, 2) void gemm_bw_kernel(
    const BwOperands ops, const int32_t* __restrict__ off, int E, int M, int N, int K) {
    using S = BwShape<BM, BN, WAVES, WMW, NS, TK>;
    constexpr bool KROW = MODE == 1;
    static_assert(!KROW || BM != 320, "320-row tiles only with K-contiguous (NT) operands");
    constexpr int MI = S::MI, NJ = S::NJ;
    // NT spreads each wave's loads of the next stage over the first half of
    // the current stage's MFMA slots (one (K-step, row block) pair per slot),
    // so that they do not back up the vector memory queue in one burst and
    // still have half a stage to land (long-sequence layer: dh 5.46 -> 5.24
    // ms, dx rows 10.26 -> 9.65 ms; the wide layer's dx rows 4.90 -> 4.64 ms).
    // TN keeps one burst: spread over its three-stage ring it measured 1-3%
    // slower.
    constexpr bool SPREAD = MODE == 0 && NS == 2;
    constexpr int STRIDE0 = S::KS * MI / S::LOADS / 2;
    constexpr int STRIDE = STRIDE0 > 0 ? STRIDE0 : 1;
    static_assert(!SPREAD || S::KS * MI >= STRIDE * S::LOADS, "a slot per wave-load");
    __shared__ __attribute__((aligned(1024))) char sa0[S::A_STAGE];
    __shared__ __attribute__((aligned(1024))) char sa1[S::A_STAGE];
    __shared__ __attribute__((aligned(1024))) char sa2[S::A_STAGE];
    __shared__ __attribute__((aligned(1024))) char sa3[NS > 3 ? S::A_STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char sb0[S::B_STAGE];
    __shared__ __attribute__((aligned(1024))) char sb1[S::B_STAGE];
    __shared__ __attribute__((aligned(1024))) char sb2[S::B_STAGE];
    __shared__ __attribute__((aligned(1024))) char sb3[NS > 3 ? S::B_STAGE : 16];
    __shared__ TileTable tt;
    __shared__ long long s_wave[WAVES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w / S::WNW, wn = w % S::WNW;
    const int c16 = lane & 15, g4 = lane >> 4;
    const int G = gridDim.x;   // a multiple of 8

    // persistent grid: sweeps of G tiles, workgroup b taking tile
    // sweep_tile(b, ...) of each sweep (each XCD a contiguous run of tiles)
    long long total;
    int mtn = 1;
    const int ntn = (N + BN - 1) / BN;
    long long per_part = 0;
    if (MODE == 0) {
        build_tile_table<BM>(off, E, ntn, tt, s_wave);
        per_part = tt.start[E];
        total = per_part * (ops.fuse ? 1 : ops.nsrc) * ops.ksplit;
    } else {
        mtn = (M + BM - 1) / BM;
        total = (long long)E * mtn * ntn;
    }
    char* abuf[4] = {sa0, sa1, sa2, sa3};
    char* bbuf[4] = {sb0, sb1, sb2, sb3};
    auto lds_base = [](char* p) { return __builtin_amdgcn_readfirstlane(lds_addr(p)); };

    for (long long sweep = 0; sweep < total; sweep += G) {
        const long long t = sweep_tile(blockIdx.x, G, sweep, total);
        if (t < 0) continue;   // uniform across the workgroup
        int e, row0, rows = BM, m0 = 0, n0, k_len, k_beg = 0, part = 0;
        const uint16_t* A = ops.A[0];
        const uint16_t* B = ops.B[0];
        if (MODE == 0) {
            part = (int)(t / per_part);
            const int src = ops.fuse ? 0 : part / ops.ksplit;
            A = src ? ops.A[1] : ops.A[0];
            B = src ? ops.B[1] : ops.B[0];
            k_len = K / ops.ksplit;
            k_beg = (part % ops.ksplit) * k_len;
            int mt, nt;
            decode_tile<4>(tt, E, ntn, t - (long long)part * per_part, e, mt, nt);
            row0 = off[e] + mt * BM;
            rows = min(BM, off[e + 1] - row0);
            n0 = nt * BN;
        } else {
            // an expert's tiles in groups of four M-tiles, M fastest inside a
            // group, so that the 32 tiles an XCD runs at once form a 4 x 8
            // block sharing 12 row slices per K-step instead of 2 x 16 sharing
            // 18 (alone on one GPU: the wide layer's dW_gate shape 4.63-4.71
            // -> 4.10-4.17 ms, its dW_down shape -2.7%, ZAYA1-like -3 to -6%,
            // the long-sequence dW_down shape -3%, the rest within 1%)
            constexpr int TGM = 4;
            e = (int)(t / (mtn * ntn));
            const int r = (int)(t % (mtn * ntn));
            const int g = r / (TGM * ntn);
            const int gs = min(TGM, mtn - g * TGM);
            const int rg = r - g * TGM * ntn;
            m0 = (g * TGM + rg % gs) * BM;
            n0 = (rg / gs) * BN;
            row0 = off[e];
            k_len = off[e + 1] - row0;
        }
        const int nks = (k_len + TK - 1) / TK;              // K-steps per source
        const bool two = MODE == 0 && ops.fuse;             // NT: both sources, one accumulator
        const int nk = two ? 2 * nks : nks;

        // this lane's byte offset for each of its wave-loads (q < A_WL: A, else B)
        uint32_t l_off[S::LOADS];
#pragma unroll
        for (int q = 0; q < S::LOADS; ++q) {
            const bool is_a = q < S::A_WL;
            const int blk = is_a ? w * S::A_WL + q : w * S::B_WL + (q - S::A_WL);
            if (!KROW) {   // [rows][TK]: 64 / CR rows per block, CR slots each
                const int r = blk * (64 / S::CR) + lane / S::CR;
                const int c = (lane % S::CR) ^ kc_sw<TK>(r);
                const int src = is_a ? min(r, rows - 1) : min(r, N - 1 - n0);
                l_off[q] = ((uint32_t)src * (uint32_t)K + c * 8) * 2u;
            } else {       // [32 K rows][columns]: (1024 / row bytes) rows per block
                const int cols = is_a ? BM : BN;
                const int spr = cols / 8;                     // 16-byte slots per row
                const int k = blk * (1024 / (cols * 2)) + lane / spr;
                const int sl = lane % spr;
                const int col = ((sl >> 1) ^ kr_sw(k)) * 16 + (sl & 1) * 8;
                const int ld = is_a ? M : N;
                const int c0 = is_a ? m0 : n0;
                l_off[q] = ((uint32_t)k * (uint32_t)ld + min(col, ld - c0 - 8)) * 2u;
            }
        }
        // NT: fixed descriptors from the tile's first row and the K slice, the
        // K step in the scalar offset (offsets stay tile-local)
        const uint16_t* a_base = MODE == 0 ? A + (long long)row0 * K + k_beg
                                           : A + (long long)row0 * M + m0;
        const uint16_t* b_base = MODE == 0 ? B + ((long long)e * N + n0) * K + k_beg
                                           : B + (long long)row0 * N + n0;
        const i32x4 rs_a0 = buffer_rsrc(a_base);
        const i32x4 rs_b0 = buffer_rsrc(b_base);
        // fused NT: the second source's descriptors (same rows, same K slice)
        const i32x4 rs_a1 =
            two ? buffer_rsrc(ops.A[1] + (long long)row0 * K + k_beg) : rs_a0;
        const i32x4 rs_b1 =
            two ? buffer_rsrc(ops.B[1] + ((long long)e * N + n0) * K + k_beg) : rs_b0;

        // the loads of K-step kt into stage buffers (la, lb): all of them, or
        // only wave-load number only_q (A loads first, then B)
        auto issue = [&](int kt, uint32_t la, uint32_t lb, int only_q = -1) {
            const bool second = two && kt >= nks;            // uniform
            const int k0 = (second ? kt - nks : kt) * TK;
            i32x4 ra = second ? rs_a1 : rs_a0, rb = second ? rs_b1 : rs_b0;
            uint32_t so = (uint32_t)k0 * 2u;
            if (MODE == 1) {
                // descriptors that start at row k0 and end at the expert's last
                // row: the rows past it read as zeros (no scalar offset, so the
                // range check sees the whole per-lane offset)
                const uint32_t left = (uint32_t)min(k_len - k0, TK);   // valid rows
                ra = buffer_rsrc(a_base + (long long)k0 * M,
                                 left * (uint32_t)M * 2u - (uint32_t)m0 * 2u);
                rb = buffer_rsrc(b_base + (long long)k0 * N,
                                 left * (uint32_t)N * 2u - (uint32_t)n0 * 2u);
                so = 0u;
            }
            // NT on 256-row tiles (long-sequence layer): the weight pieces
            // first, as they miss in L2 more often than the activation rows
            // (alone on one GPU: dh_raw-shaped product 5.22-5.27 -> 5.02-5.03
            // ms, dx_perm-shaped 9.48-9.51 -> 9.35-9.40 ms; on the wide
            // layer's 320-row tiles -1.6% and +1%, so there A first)
            constexpr bool WFIRST = MODE == 0 && BM == 256;
            constexpr int FIRST = WFIRST ? S::B_WL : S::A_WL;
#pragma unroll
            for (int q = 0; q < FIRST; ++q)
                if (only_q < 0 || only_q == q) {
                    if constexpr (WFIRST)
                        load_to_lds(rb, l_off[S::A_WL + q], so, lb + (w * S::B_WL + q) * 1024);
                    else
                        load_to_lds(ra, l_off[q], so, la + (w * S::A_WL + q) * 1024);
                }
#pragma unroll
            for (int q = 0; q < (WFIRST ? S::A_WL : S::B_WL); ++q)
                if (only_q < 0 || only_q == FIRST + q) {
                    if constexpr (WFIRST)
                        load_to_lds(ra, l_off[q], so, la + (w * S::A_WL + q) * 1024);
                    else
                        load_to_lds(rb, l_off[S::A_WL + q], so, lb + (w * S::B_WL + q) * 1024);
                }
        };

        // per-lane fragment read offsets (lane constants)
        const int kc_rd = c16 * (2 * TK);
        const int kc_s = kc_sw<TK>(c16);
        const int kr_row = g4 * 8 + (c16 >> 2);
        const int kr_h = kr_sw(kr_row);
        const int kr_in = ((c16 >> 1) & 1) * 16 + (c16 & 1) * 8;
        // 16 rows (K contiguous) or 16 columns (K rows of rb bytes) from index
        // b, K values 32 ks .. + 31 of the stage
        auto frag = [&](const char* st, int b, int rb, int ks) -> bf16x8 {
            if (!KROW) {
                return *(const bf16x8*)(st + b * (2 * TK) + kc_rd + (((ks * 4 + g4) ^ kc_s) << 4));
            } else {
                const char* p = st + (ks * 32 + kr_row) * rb + kr_in + (((b >> 4) ^ kr_h) << 5);
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
                const s16x4 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * rb));
                return __builtin_bit_cast(
                    bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };

        f32x4 acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int s = 0; s + 1 < NS; ++s)
            if (s < nk) issue(s, lds_base(abuf[s]), lds_base(bbuf[s]));

        for (int kt = 0; kt < nk; kt += NS) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int k = kt + s;
                if (k >= nk) break;
                // stage k has landed (up to NS-2 later stages may still be in
                // flight) and every wave is done with the buffer refilled below
                switch (min(nk - 1 - k, NS - 2)) {
                    case 0: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); break;
                    case 1:
                        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(S::LOADS) : "memory");
                        break;
                    default:
                        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * S::LOADS)
                                     : "memory");
                        break;
                }
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                const bool refill = k + NS - 1 < nk;
                const uint32_t rla = lds_base(abuf[(s + NS - 1) % NS]);
                const uint32_t rlb = lds_base(bbuf[(s + NS - 1) % NS]);
                if (!SPREAD && refill) issue(k + NS - 1, rla, rlb);
                const char* sa = abuf[s];
                const char* sb = bbuf[s];
#pragma unroll
                for (int ks = 0; ks < S::KS; ++ks) {
                    bf16x8 fb[NJ];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) fb[j] = frag(sb, (wn * NJ + j) * 16, BN * 2, ks);
#pragma unroll
                    for (int i = 0; i < MI; ++i) {
                        if (SPREAD && refill) {
                            const int slot = ks * MI + i;
                            if (slot % STRIDE == 0 && slot / STRIDE < S::LOADS)
                                issue(k + NS - 1, rla, rlb, slot / STRIDE);
                        }
                        const bf16x8 fa = frag(sa, (wm * MI + i) * 16, BM * 2, ks);
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa,
                                                                                acc[i][j], 0, 0, 0);
                    }
                }
            }
        }

        // lane (g4, c16) of block (i, j): row i*16 + c16, columns j*16 + 4 g4 .. + 3
        if constexpr (EPI) {
            // GeGLU backward of this tile's elements; each wave's 64 columns
            // (N % 64 == 0: all valid or all past N) give one partial of dgate.
            // g, u come in and dg, du, gate h go out in whole 128-byte row
            // pieces (8 rows per instruction) through this wave's 6 KB of an
            // idle stage buffer, switched to and from the MFMA layout there
            // (16 rows x 8 bytes per instruction straight from the MFMA layout
            // move about a quarter of the bytes per clock per CU).  Chunk c of
            // row r of a 16-row block sits in slot c ^ ((r >> 1) & 7).
            static_assert(MODE == 0 && NJ * 16 == 64, "epilogue: NT, 64 columns per wave");
            static_assert(WAVES / 2 * 6144 <= S::A_STAGE && WAVES / 2 * 6144 <= S::B_STAGE,
                          "staging room");
            const int cw = n0 + wn * 64;
            const int np = N / 64;
            const bool cols_ok = cw < N;
            const int fb = (nk + NS - 2) % NS;
            char* const fa = fb == 0 ? sa0 : fb == 1 ? sa1 : fb == 2 ? sa2 : sa3;
            char* const fbb = fb == 0 ? sb0 : fb == 1 ? sb1 : fb == 2 ? sb2 : sb3;
            char* const sG = w < WAVES / 2 ? fa + w * 6144 : fbb + (w - WAVES / 2) * 6144;
            char* const sU = sG + 2048;
            char* const sH = sG + 4096;
            const int ln = hidden(lane);
            const int h16 = ln & 15, hg4 = ln >> 4, l8 = ln >> 3, c8 = ln & 7;
            // row-contiguous piece q of a block: row 8 q + l8, chunk c8
            auto rc = [&](int q) {
                const int rr = q * 8 + l8;
                return rr * 128 + ((c8 ^ ((rr >> 1) & 7)) << 4);
            };
            // MFMA-layout piece jj: row c16, columns 16 jj + 4 g4 .. + 3
            auto ml = [&](int jj) {
                return h16 * 128 + (((jj * 2 + (hg4 >> 1)) ^ ((h16 >> 1) & 7)) << 4) +
                       (hg4 & 1) * 8;
            };
            // g, u of row block i + 1 are loaded before row block i is
            // computed and stored: one load latency per tile, not one per
            // row block (the loads are issued ahead of the stores in program
            // order, which the compiler keeps since the arrays are the same)
            // (the 320-row tile has no registers to spare for the second set:
            // there each row block loads its own)
            constexpr bool AHEAD = BM != 320;
            constexpr int NSET = AHEAD ? 2 : 1;
            u32x4 gq[NSET][2], uq[NSET][2];
            auto fetch = [&](int i, int b) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int r = (wm * MI + i) * 16 + q * 8 + l8;
                    if (r < rows && cols_ok) {
                        const long long o = (long long)(row0 + r) * N + cw + c8 * 8;
                        gq[b][q] = *(const u32x4*)(ops.G + o);
                        uq[b][q] = *(const u32x4*)(ops.U + o);
                    }
                }
            };
            if constexpr (AHEAD) fetch(0, 0);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int b = AHEAD ? i & 1 : 0;
                if constexpr (!AHEAD) fetch(i, 0);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    *(u32x4*)(sG + rc(q)) = gq[b][q];
                    *(u32x4*)(sU + rc(q)) = uq[b][q];
                }
                if constexpr (AHEAD)
                    if (i + 1 < MI) fetch(i + 1, (i + 1) & 1);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                const int r = (wm * MI + i) * 16 + h16;
                const bool row_ok = r < rows && cols_ok;
                const float gt = row_ok ? ops.row_gate[row0 + r] : 0.f;
                float dot = 0.f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const u32x2 gw = *(const u32x2*)(sG + ml(j));
                    const u32x2 uw = *(const u32x2*)(sU + ml(j));
                    float dg[4], du[4], gh[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t g2 = gw[q >> 1], u2 = uw[q >> 1];
                        const float g = bf16_bits_to_f32((q & 1) ? g2 >> 16 : g2 & 0xffffu);
                        const float u = bf16_bits_to_f32((q & 1) ? u2 >> 16 : u2 & 0xffffu);
                        float term;
                        geglu_bwd_elem(g, u, acc[i][j][q], gt, dg[q], du[q], gh[q], term);
                        dot += term;
                    }
                    *(u32x2*)(sG + ml(j)) = u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
                    *(u32x2*)(sU + ml(j)) = u32x2{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
                    *(u32x2*)(sH + ml(j)) = u32x2{pack_bf16x2(gh[0], gh[1]), pack_bf16x2(gh[2], gh[3])};
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int rq = (wm * MI + i) * 16 + q * 8 + l8;
                    if (rq < rows && cols_ok) {
                        const long long o = (long long)(row0 + rq) * N + cw + c8 * 8;
                        *(u32x4*)(ops.G + o) = *(const u32x4*)(sG + rc(q));
                        *(u32x4*)(ops.U + o) = *(const u32x4*)(sU + rc(q));
                        *(u32x4*)(ops.gH + o) = *(const u32x4*)(sH + rc(q));
                    }
                }
                // the four lanes of a row (g4 = 0..3), then lane g4 = 0 writes
                if (!row_ok) dot = 0.f;
                dot += __shfl_xor(dot, 16);
                dot += __shfl_xor(dot, 32);
                if (hg4 == 0 && row_ok) ops.dot[(row0 + r) * (long long)np + cw / 64] = dot;
                // this block's LDS reads are done before the next block's writes
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        } else {
            // Each 16-row block goes through this wave's 4 KB slice of an idle
            // stage buffer (the one the last K-step but one used: no wave
            // reads it any more and no load fills it again in this tile), so
            // that every store writes whole row pieces, 4 rows x 256 bytes,
            // instead of the MFMA layout's 16 rows x 64 bytes: per CU, stores
            // of 128 bytes or more per row move about three times the bytes
            // per clock.  Chunk c (16 bytes) of row r sits in slot c ^ r.
            static_assert(NJ == 4, "64 columns (16 chunks of 16 bytes) per wave row");
            const int fb = (nk + NS - 2) % NS;
            char* const fa = fb == 0 ? sa0 : fb == 1 ? sa1 : fb == 2 ? sa2 : sa3;
            char* const fbb = fb == 0 ? sb0 : fb == 1 ? sb1 : fb == 2 ? sb2 : sb3;
            char* stg;
            if constexpr (WAVES * 4096 <= S::A_STAGE) {
                stg = fa + w * 4096;
            } else {
                static_assert(WAVES / 2 * 4096 <= S::A_STAGE && WAVES / 2 * 4096 <= S::B_STAGE,
                              "staging room");
                stg = w < WAVES / 2 ? fa + w * 4096 : fbb + (w - WAVES / 2) * 4096;
            }
            const int colw = n0 + wn * 64;   // the wave's first column
            const int ln = hidden(lane);
            const int h16 = ln & 15, hg4 = ln >> 4;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                // lane (g4, c16) holds row c16, columns 16 j + 4 g4 .. + 3: chunk 4 j + g4
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    *(f32x4*)(stg + h16 * 256 + (((j * 4 + hg4) ^ h16) << 4)) = acc[i][j];
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rr = q * 4 + hg4, ch = h16;
                    const f32x4 v = *(const f32x4*)(stg + rr * 256 + ((ch ^ rr) << 4));
                    const int r = (wm * MI + i) * 16 + rr;
                    const int col = colw + ch * 4;
                    if ((MODE == 0 ? r < rows : m0 + r < M) && col < N) {
                        float* crow = MODE == 0
                                          ? ops.C + part * ops.c_stride + (long long)(row0 + r) * N
                                          : ops.C + ((long long)e * M + m0 + r) * N;
                        *(f32x4*)(crow + col) = v;
                    }
                }
                // this block's reads are done before the next block's writes
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        }
        // every wave is done reading this tile's stages before the next tile's
        // loads refill them
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
}

// Persistent grid of at most `cap` workgroups (a multiple of 8).
unsigned grid_of(long long tiles, int cap) {
    long long g = std::min<long long>(cap, (tiles + 7) / 8 * 8);
    return (unsigned)std::max<long long>(8, g / 8 * 8);
}

template <int BM, int BN, int WAVES, int WMW, int NS, int TK, bool EPI = false>
hipError_t launch_nt(const BwOperands& ops, const int32_t* off, int E, int N, int K,
                     long long max_rows, int cap, hipStream_t s) {
    const long long tiles = ((max_rows + BM - 1) / BM + E) * ((N + BN - 1) / BN) *
                            (ops.fuse ? 1 : ops.nsrc) * ops.ksplit;
    hipLaunchKernelGGL((gemm_bw_kernel<0, BM, BN, WAVES, WMW, NS, TK, EPI>),
                       dim3(grid_of(tiles, cap)), dim3(64 * WAVES), 0, s, ops, off, E, 0, N, K);
    return hipGetLastError();
}

template <int BM, int BN, int WAVES, int WMW, int NS, int TK>
hipError_t launch_tn(const BwOperands& ops, const int32_t* off, int E, int M, int N, int cap,
                     hipStream_t s) {
    const long long tiles = (long long)E * ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_bw_kernel<1, BM, BN, WAVES, WMW, NS, TK>), dim3(grid_of(tiles, cap)),
                       dim3(64 * WAVES), 0, s, ops, off, E, M, N, 0);
    return hipGetLastError();
}

// NT rows per tile: 320 when the experts hold up to 320 rows on average (one
// M-tile covers a ZAYA1-like expert, as in the forward GEMMs), else 256.
static int bw_nt_bm(long long max_rows, int E) { return max_rows <= 320LL * E ? 320 : 256; }
// K-step and ring depth: the NT products read their weight operand in 128-byte
// row pieces (64 K values) through a two-stage ring; the TN products, whose K
// runs over an expert's ragged rows, keep 32-deep steps and three stages
// (64-deep steps measured 2-3 % faster for NT, slower for TN)
constexpr int BW_NT_TK = 64, BW_NT_NS = 2;
constexpr int BW_TN_TK = 32, BW_TN_NS = 3;

}  // namespace

// One tile shape for both: 256 x 256 tiles, 8 waves as 2 (M) x 4 (N) (one
// workgroup per CU; cus counts two per CU); K-step and stages as above.  Measured on the
// four large layers against 128 x 128 tiles with 4 waves (two workgroups per
// CU) and 256 x 128: 256 x 256 is the fastest on every one (the backward of
// the ZAYA1-like layer 2.38 ms against 2.95 and 2.72); a 4 x 2 wave layout and
// a fourth stage measure within 1.5%.
int bw_nt_ksplit(long long max_rows, int E, int N, int K, int nsrc, int cus) {
    const int bm = bw_nt_bm(max_rows, E);
    const long long tiles = ((max_rows + bm - 1) / bm + E) * ((N + 255) / 256) * nsrc;
    const long long want = 3LL * (cus / 2);   // three sweeps of one workgroup per CU
    int ks = 1;
    while (ks < 4 && tiles * ks < want && (K / (2 * ks)) % BW_NT_TK == 0 && K % (2 * ks) == 0)
        ks *= 2;
    return ks;
}

hipError_t launch_bw_nt(const uint16_t* A0, const uint16_t* W0, const uint16_t* A1,
                        const uint16_t* W1, float* C, long long part_stride, int ksplit,
                        const int32_t* off, int E, int N, int K, long long max_rows, int cus,
                        hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    if (N % 8 != 0 || N < 8 || ksplit < 1 || K % ksplit != 0 || (K / ksplit) % BW_NT_TK != 0)
        return hipErrorInvalidValue;
    // two sources accumulate in one tile: ksplit parts in all
    BwOperands ops{{A0, A1}, {W0, W1}, C, part_stride, A1 ? 2 : 1, ksplit, A1 ? 1 : 0};
    if (bw_nt_bm(max_rows, E) == 320)
        return launch_nt<320, 256, 8, 2, BW_NT_NS, BW_NT_TK>(ops, off, E, N, K, max_rows, cus / 2,
                                                             s);
    return launch_nt<256, 256, 8, 2, BW_NT_NS, BW_NT_TK>(ops, off, E, N, K, max_rows, cus / 2, s);
}

hipError_t launch_bw_nt_geglu(const uint16_t* A, const uint16_t* W, uint16_t* G, uint16_t* U,
                              uint16_t* gH, const float* row_gate, float* dot,
                              const int32_t* off, int E, int N, int K, long long max_rows,
                              int cus, hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    if (N % 64 != 0 || N < 64 || K % BW_NT_TK != 0) return hipErrorInvalidValue;
    BwOperands ops{{A, nullptr}, {W, nullptr}, nullptr, 0, 1, 1, 0, G, U, gH, row_gate, dot};
    if (bw_nt_bm(max_rows, E) == 320)
        return launch_nt<320, 256, 8, 2, BW_NT_NS, BW_NT_TK, true>(ops, off, E, N, K, max_rows,
                                                                   cus / 2, s);
    return launch_nt<256, 256, 8, 2, BW_NT_NS, BW_NT_TK, true>(ops, off, E, N, K, max_rows,
                                                               cus / 2, s);
}

hipError_t launch_bw_tn(const uint16_t* A, const uint16_t* B, float* C, const int32_t* off,
                        int E, int M, int N, int cus, hipStream_t s) {
    if (E == 0) return hipSuccess;
    if (M % 8 != 0 || N % 8 != 0 || M < 8 || N < 8) return hipErrorInvalidValue;
    BwOperands ops{{A, nullptr}, {B, nullptr}, C, 0, 1, 1, 0};
    return launch_tn<256, 256, 8, 2, BW_TN_NS, BW_TN_TK>(ops, off, E, M, N, cus / 2, s);
}

}  // namespace moe
