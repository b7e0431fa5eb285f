// gemm_bw.hip -- the grouped GEMMs of the layer's backward pass on gfx950.
//
// The forward multiplies activations [rows][K] by weights [K][N].  Its
// backward needs the two other operand layouts:
//   NT  C[rows][N] (+)= A[rows][K] B^T, B stored [N][K]       dH = dO W_down^T,
//       dX = dG W_gate^T + dU W_up^T (rows of each expert, K and N fixed)
//   TN  C[e][M][N] = A^T B, A stored [rows][M], B [rows][N]   dW = X^T dG ...
//       (K = the rows of expert e: a different reduction length per expert)
// One kernel, two operand flavours chosen at compile time: an operand stored
// with K contiguous (A in NT, B in NT) is read into MFMA fragments with
// ds_read_b128; an operand stored with K as its row index (A in TN, B in TN)
// with the transposing read ds_read_b64_tr_b16 (a 16-lane group reads a 4 x 16
// block; lane n receives column n).  Both MFMA operands of
// v_mfma_f32_16x16x32_bf16 share one register layout (lane l: index l % 16,
// K values 8 (l / 16) .. + 7), so the same two read paths serve A and B.
//
// Workgroup: 4 waves (2 x 2), tile 128 x 128, K-steps of 32, two LDS buffers
// filled through registers (loads of step k+1 are in flight while step k
// multiplies).  Rows past the end (M, N or an expert's K range) load as zero,
// so the K tail of the ragged reductions adds nothing.  fp32 results; each
// lane holds four consecutive output columns of one row (weights in the
// MFMA's first operand slot) and writes them as one 16-byte store.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {
namespace {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int TB = 128;          // tile rows and columns
constexpr int TK = 32;           // K-step
constexpr int LD_KC = TK + 8;    // LDS row stride (elements) of a K-contiguous tile [128][32]
constexpr int LD_KR = TB + 8;    // LDS row stride of a K-row tile [32][128]
// elements of one LDS tile: [TK][LD_KR] (K-row) or [TB][LD_KC] (K-contiguous)
constexpr int tile_elems(bool krow) { return krow ? TK * LD_KR : TB * LD_KC; }

// 16 bytes per thread-chunk: tile chunk q (0..511) of an operand tile.
//  K-contiguous tile (rows x 32 K): row q / 4, K chunk q % 4
//  K-row tile (32 K x 128 cols):    K row q / 16, col chunk q % 16
template <bool KROW>
__device__ __forceinline__ void chunk_pos(int q, int& r, int& c8) {
    if (KROW) { r = q / 16; c8 = (q % 16) * 8; }
    else      { r = q / 4;  c8 = (q % 4) * 8; }
}

// Fragment of 16 (rows or columns) x 32 K at tile index base b (0, 16, ...).
template <bool KROW>
__device__ __forceinline__ bf16x8 frag(const uint16_t* tile, int b, int lane) {
    const int c = lane & 15, g = lane >> 4;
    if (!KROW) {
        return *(const bf16x8*)(tile + (b + c) * LD_KC + g * 8);
    } else {
        const uint16_t* p = tile + (g * 8 + (c >> 2)) * LD_KR + b + (c & 3) * 4;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * LD_KR));
        return __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}

// MODE 0 (NT): tile table over the rows of each expert (ragged M); K, N
//   fixed; A = act[rows][K] (row off[e] + m), B = W[e] stored [N][K].
// MODE 1 (TN): tiles (e, M-tile, N-tile), M and N fixed; K = rows of e;
//   A stored [rows][M] (row off[e] + k), B stored [rows][N].
// a_rows / b_rows (may be null) replace a row index r of A / B by
// a_rows[r] / b_rows[r]: the operand is then read from an unpermuted array
// (x or dy) through the dispatch map token_of_row.
template <int MODE>
__global__ __launch_bounds__(256) void gemm_bw_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows,
    const uint16_t* __restrict__ B, const int32_t* __restrict__ b_rows, float* __restrict__ C,
    const int32_t* __restrict__ off, int E, int M, int N, int K, long long b_stride,
    int accumulate) {
    constexpr bool A_KROW = MODE == 1;   // A tile stored with K as its row index
    constexpr bool B_KROW = MODE == 1;
    __shared__ __attribute__((aligned(16))) uint16_t sa[2][tile_elems(A_KROW)];
    __shared__ __attribute__((aligned(16))) uint16_t sb[2][tile_elems(B_KROW)];
    __shared__ TileTable tt;
    __shared__ long long s_wave[4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;   // 2 x 2 waves, 64 x 64 each

    int e, row0, rows, n0, m0 = 0, k_begin = 0, k_len = K;
    if (MODE == 0) {
        const int ntn = (N + TB - 1) / TB;
        build_tile_table<TB>(off, E, ntn, tt, s_wave);
        const long long t = blockIdx.x;
        if (t >= tt.start[E]) return;   // uniform
        int mt, nt;
        decode_tile<1>(tt, E, ntn, t, e, mt, nt);
        row0 = off[e] + mt * TB;
        rows = min(TB, off[e + 1] - row0);
        n0 = nt * TB;
    } else {
        const int mtn = (M + TB - 1) / TB, ntn = (N + TB - 1) / TB;
        const int t = blockIdx.x;
        e = t / (mtn * ntn);
        const int r = t % (mtn * ntn);
        m0 = (r / ntn) * TB;
        n0 = (r % ntn) * TB;
        row0 = 0;
        rows = TB;
        k_begin = off[e];
        k_len = off[e + 1] - off[e];
    }
    const uint16_t* Bw = B + (MODE == 0 ? (long long)e * b_stride : 0);

    // NT: the A rows of this thread's two chunks are the same for every K-step
    long long a_src[2] = {0, 0};
    if (MODE == 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            int r, c8;
            chunk_pos<A_KROW>(tid + 256 * s, r, c8);
            if (r < rows) a_src[s] = a_rows ? a_rows[row0 + r] : row0 + r;
        }
    }

    // global -> register loads of one K-step (two 16-byte chunks per thread and operand)
    auto load_a = [&](int k0, u32x4 (&v)[2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            int r, c8;
            chunk_pos<A_KROW>(tid + 256 * s, r, c8);
            bool ok;
            long long gi = 0;
            if (MODE == 0) {   // A[row0 + r][k0 + c8]
                ok = r < rows && k0 + c8 < K;
                if (ok) gi = a_src[s] * K + k0 + c8;
            } else {           // A[k_begin + k0 + r][m0 + c8]
                ok = k0 + r < k_len && m0 + c8 < M;
                if (ok) {
                    const int kr = k_begin + k0 + r;
                    gi = (long long)(a_rows ? a_rows[kr] : kr) * M + m0 + c8;
                }
            }
            v[s] = ok ? *(const u32x4*)(A + gi) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto load_b = [&](int k0, u32x4 (&v)[2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            int r, c8;
            chunk_pos<B_KROW>(tid + 256 * s, r, c8);
            bool ok;
            long long gi = 0;
            if (MODE == 0) {   // W[e][n0 + r][k0 + c8]
                ok = n0 + r < N && k0 + c8 < K;
                if (ok) gi = (long long)(n0 + r) * K + k0 + c8;
            } else {           // B[k_begin + k0 + r][n0 + c8]
                ok = k0 + r < k_len && n0 + c8 < N;
                if (ok) {
                    const int kr = k_begin + k0 + r;
                    gi = (long long)(b_rows ? b_rows[kr] : kr) * N + n0 + c8;
                }
            }
            v[s] = ok ? *(const u32x4*)(Bw + gi) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](uint16_t* tile, const u32x4 (&v)[2], bool krow) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            int r, c8;
            if (krow) chunk_pos<true>(tid + 256 * s, r, c8);
            else chunk_pos<false>(tid + 256 * s, r, c8);
            *(u32x4*)(tile + r * (krow ? LD_KR : LD_KC) + c8) = v[s];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (k_len + TK - 1) / TK;
    u32x4 va[2], vb[2];
    if (nk > 0) {
        load_a(0, va);
        load_b(0, vb);
        store(sa[0], va, A_KROW);
        store(sb[0], vb, B_KROW);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            load_a((kt + 1) * TK, va);
            load_b((kt + 1) * TK, vb);
        }
        bf16x8 fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = frag<A_KROW>(sa[cur], wm * 64 + i * 16, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = frag<B_KROW>(sb[cur], wn * 64 + j * 16, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        if (kt + 1 < nk) {
            store(sa[cur ^ 1], va, A_KROW);
            store(sb[cur ^ 1], vb, B_KROW);
        }
        __syncthreads();
    }

    // lane (g4, c16) of block (i, j): row i*16 + c16, columns j*16 + 4 g4 .. + 3
    const int c16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + c16;
        if (MODE == 0 ? r >= rows : m0 + r >= M) continue;
        float* crow = MODE == 0 ? C + (long long)(row0 + r) * N
                                : C + ((long long)e * M + m0 + r) * N;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + j * 16 + g4 * 4;
            if (col >= N) continue;
            f32x4 v = acc[i][j];
            if (accumulate) v += *(const f32x4*)(crow + col);
            *(f32x4*)(crow + col) = v;
        }
    }
}

}  // namespace

hipError_t launch_bw_nt(const uint16_t* act, const int32_t* act_rows, const uint16_t* W,
                        float* C, const int32_t* off, int E, int N, int K, long long max_rows,
                        bool accumulate, hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    if (N % 8 != 0 || K % TK != 0) return hipErrorInvalidValue;
    const long long tiles = ((max_rows + TB - 1) / TB + E) * ((N + TB - 1) / TB);
    hipLaunchKernelGGL(gemm_bw_kernel<0>, dim3((unsigned)tiles), dim3(256), 0, s, act, act_rows,
                       W, (const int32_t*)nullptr, C, off, E, 0, N, K, (long long)N * K,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_bw_tn(const uint16_t* A, const int32_t* a_rows, const uint16_t* B,
                        const int32_t* b_rows, float* C, const int32_t* off, int E, int M, int N,
                        hipStream_t s) {
    const long long tiles = (long long)E * ((M + TB - 1) / TB) * ((N + TB - 1) / TB);
    if (tiles == 0) return hipSuccess;
    if (M % 8 != 0 || N % 8 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_bw_kernel<1>, dim3((unsigned)tiles), dim3(256), 0, s, A, a_rows, B,
                       b_rows, C, off, E, M, N, 0, 0LL, 0);
    return hipGetLastError();
}

}  // namespace moe
