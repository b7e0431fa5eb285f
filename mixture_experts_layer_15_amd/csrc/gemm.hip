// gemm.hip -- grouped expert GEMMs of the MoE FFN on gfx950.
//
// Two kernels over the expert-grouped rows written by dispatch (rows of
// expert e are expert_offset[e] .. expert_offset[e+1]-1):
//   gate/up:  h = GELU_erf(X_e W_gate[e]) * (X_e W_up[e])   (GeGLU fused into
//             the GEMM epilogue, as the ZAYA1 page describes for its expert
//             MLP, "AMD GPU深度学习优化与ZAYA1大模型实践" section 3.2)
//   down:     O = h_e W_down[e]
//
// bf16 path: v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  A workgroup
// (4 waves, 2 x 2) owns a 128-row x 128-B-column tile; each wave a 64 x 64
// block = 4 x 4 MFMA tiles.  For gate/up the 128 B columns are 64 W_gate
// columns and the same 64 W_up columns, so the gate and up accumulators of
// one h element sit in the same lane and register, and the epilogue needs no
// data exchange.  Weights keep their [K][N] layout (N contiguous): the tile
// goes to LDS as-is and the B fragments are read with gfx950's transposing
// LDS read (ds_read_b64_tr_b16), which hands each lane four K-values of one
// column.  K-steps of 64 are double-buffered through LDS.
//
// Scheduling: a persistent grid walks a tile list ordered expert-major, then
// N-tile, then M-tile, built per workgroup from expert_offset (so the number
// of rows per expert never leaves the device).  Consecutive tiles are handed
// to the same XCD (workgroup b runs on XCD b % 8), so the M-tiles that share
// a weight tile, and the N-tiles that share an expert's rows, meet in one L2.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128;       // rows per tile
constexpr int BNB = 128;      // B columns per tile
constexpr int BK = 64;        // K per LDS stage
constexpr int A_LD = BK + 8;  // A row stride in LDS (elements): 144 B
constexpr int B_LD = BNB + 8; // B row stride in LDS (elements): 272 B

typedef short s16x8 __attribute__((ext_vector_type(8)));

// Exclusive prefix of per-expert tile counts, shared by the workgroup.
struct TileTable {
    long long start[257];   // tiles before expert e; start[E] = total
    int mtiles[256];        // M-tiles of expert e
};

// Block of 256 threads: builds the table.  ntn = N-tiles per expert.
template <int TBM>
__device__ void build_tile_table(const int32_t* __restrict__ off, int E, int ntn,
                                 TileTable& tt, long long* s_wave) {
    const int e = threadIdx.x;
    long long cnt = 0;
    int mt = 0;
    if (e < E) {
        int kept = off[e + 1] - off[e];
        mt = (kept + TBM - 1) / TBM;
        cnt = (long long)mt * ntn;
    }
    tt.mtiles[e] = mt;
    // inclusive scan over 256 threads: wave shuffles, then wave totals
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    long long v = cnt;
    for (int o = 1; o < 64; o <<= 1) {
        long long u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_wave[w] = v;
    __syncthreads();
    long long add = 0;
    for (int i = 0; i < w; ++i) add += s_wave[i];
    tt.start[e + 1] = v + add;
    if (e == 0) tt.start[0] = 0;
    __syncthreads();
}

// Tile id -> (expert, m-tile, n-tile).  Largest e with start[e] <= t.
__device__ __forceinline__ void decode_tile(const TileTable& tt, int E, long long t,
                                            int& e, int& m, int& n) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (tt.start[mid] <= t) lo = mid; else hi = mid - 1;
    }
    // skip experts with no tiles (start[e] == start[e+1])
    e = lo;
    long long local = t - tt.start[e];
    int mt = tt.mtiles[e];
    n = (int)(local / mt);
    m = (int)(local % mt);
}

// Workgroup b of G: its tile slot within one sweep, remapped so that each XCD
// (b % 8) receives a contiguous run of tile ids.
__device__ __forceinline__ long long xcd_slot(int b, int G) {
    const int per = G >> 3;
    return (long long)(b & 7) * per + (b >> 3);
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, uint16_t* __restrict__ C,
    const int32_t* __restrict__ off, int E, int K, int N) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * A_LD];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BK * B_LD];
    __shared__ TileTable tt;
    __shared__ long long s_wave[4];

    // N-tiles: gate/up covers 64 h columns per tile, down 128 output columns.
    const int ncols_tile = GATEUP ? BNB / 2 : BNB;
    const int ntn = (N + ncols_tile - 1) / ncols_tile;
    build_tile_table<BM>(off, E, ntn, tt, s_wave);
    const long long total = tt.start[E];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int G = gridDim.x;
    const int nk = K / BK;
    const long long KN = (long long)K * N;

    for (long long base = 0; base < total; base += G) {
        const long long t = base + xcd_slot(blockIdx.x, G);
        if (t >= total) continue;    // uniform across the workgroup
        int e, mtile, ntile;
        decode_tile(tt, E, t, e, mtile, ntile);
        const int row0 = off[e] + mtile * BM;       // first global row of the tile
        const int rows = min(BM, off[e + 1] - row0); // valid rows in the tile
        const int n0 = ntile * ncols_tile;

        // global source pointers for this thread's 4 A and 4 B vectors
        const uint16_t* a_src[4];
        const uint16_t* b_src[4];
        int a_dst[4], b_dst[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = tid + 256 * i;
            const int r = v >> 3, kc = v & 7;
            const int rr = min(r, rows - 1);
            a_src[i] = A + (long long)(row0 + rr) * K + kc * 8;
            a_dst[i] = r * A_LD + kc * 8;
            const int kr = v >> 4, nch = v & 15;
            const uint16_t* bsrc;
            if (GATEUP) {
                bsrc = (nch < 8 ? B0 : B1) + (long long)e * KN + (long long)kr * N + n0 + (nch & 7) * 8;
            } else {
                const int col = min(n0 + nch * 8, N - 8);
                bsrc = B0 + (long long)e * KN + (long long)kr * N + col;
            }
            b_src[i] = bsrc;
            b_dst[i] = kr * B_LD + nch * 8;
        }

        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        u32x4 ra[4], rb[4];
        // stage 0
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = *(const u32x4*)(a_src[i]);
            rb[i] = *(const u32x4*)(b_src[i]);
        }
        __syncthreads();   // previous tile's readers are done with both buffers
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(u32x4*)(&As[0][a_dst[i]]) = ra[i];
            *(u32x4*)(&Bs[0][b_dst[i]]) = rb[i];
        }
        __syncthreads();

        // B column base (within the 128-column tile) of this wave's n-tile j
        int bcol[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bcol[j] = GATEUP ? ((j < 2) ? wn * 32 + j * 16 : 64 + wn * 32 + (j - 2) * 16)
                             : wn * 64 + j * 16;
        const int c16 = lane & 15, g4 = lane >> 4;

        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) {
                const long long ka = (long long)(kt + 1) * BK;
                const long long kb = ka * N;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ra[i] = *(const u32x4*)(a_src[i] + ka);
                    rb[i] = *(const u32x4*)(b_src[i] + kb);
                }
            }
            const uint16_t* as = As[cur];
            const uint16_t* bs = Bs[cur];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 af[4], bfr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[i] = *(const bf16x8*)(&as[(wm * 64 + i * 16 + c16) * A_LD + ks * 32 + g4 * 8]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = ks * 32 + g4 * 8 + (c16 >> 2);
                    const int col = bcol[j] + (c16 & 3) * 4;
                    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(&bs[row * B_LD + col]));
                    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(&bs[(row + 4) * B_LD + col]));
                    s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    bfr[j] = __builtin_bit_cast(bf16x8, both);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < nk) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    *(u32x4*)(&As[cur ^ 1][a_dst[i]]) = ra[i];
                    *(u32x4*)(&Bs[cur ^ 1][b_dst[i]]) = rb[i];
                }
            }
            __syncthreads();
        }

        // epilogue: lane holds rows 4*(lane/16)+r, column lane%16 of each 16x16 tile
        if (GATEUP) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = n0 + wn * 32 + j * 16 + c16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rt = wm * 64 + i * 16 + g4 * 4 + r;
                        if (rt < rows) {
                            const float hv = gelu_erf(acc[i][j][r]) * acc[i][j + 2][r];
                            C[(long long)(row0 + rt) * N + col] = (uint16_t)f32_to_bf16_bits(hv);
                        }
                    }
                }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = n0 + wn * 64 + j * 16 + c16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rt = wm * 64 + i * 16 + g4 * 4 + r;
                        if (rt < rows && col < N)
                            C[(long long)(row0 + rt) * N + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
                    }
                }
        }
    }
}

// ---------------------------------------------------------------- fp32 path
// Plain fp32 FMA tiles (64 x 64, K-steps of 16, 4 x 4 outputs per thread) for
// fp32 layers; same tile list and scheduling as the bf16 path.
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <bool GATEUP>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B0, const float* __restrict__ B1,
    float* __restrict__ C, const int32_t* __restrict__ off, int E, int K, int N) {
    __shared__ float As[FBK][FBM + 4];
    __shared__ float Bg[FBK][FBN + 4];
    __shared__ float Bu[FBK][FBN + 4];
    __shared__ TileTable tt;
    __shared__ long long s_wave[4];
    const int ntn = (N + FBN - 1) / FBN;
    build_tile_table<FBM>(off, E, ntn, tt, s_wave);
    const long long total = tt.start[E];
    const int tid = threadIdx.x;
    const int tr = tid >> 4, tc = tid & 15;   // 16 x 16 threads, 4 x 4 outputs each
    const long long KN = (long long)K * N;
    for (long long t = blockIdx.x; t < total; t += gridDim.x) {
        int e, mtile, ntile;
        decode_tile(tt, E, t, e, mtile, ntile);
        const int row0 = off[e] + mtile * FBM;
        const int rows = min(FBM, off[e + 1] - row0);
        const int n0 = ntile * FBN;
        float g[4][4] = {}, u[4][4] = {};
        for (int k0 = 0; k0 < K; k0 += FBK) {
            __syncthreads();
            for (int v = tid; v < FBM * FBK; v += 256) {
                const int r = v / FBK, kk = v % FBK;
                As[kk][r] = A[(long long)(row0 + min(r, rows - 1)) * K + k0 + kk];
            }
            for (int v = tid; v < FBK * FBN; v += 256) {
                const int kk = v / FBN, c = v % FBN;
                const int col = min(n0 + c, N - 1);
                const long long src = (long long)e * KN + (long long)(k0 + kk) * N + col;
                Bg[kk][c] = B0[src];
                if (GATEUP) Bu[kk][c] = B1[src];
            }
            __syncthreads();
            for (int kk = 0; kk < FBK; ++kk) {
                float a[4], bg[4], bu[4];
                for (int i = 0; i < 4; ++i) a[i] = As[kk][tr * 4 + i];
                for (int j = 0; j < 4; ++j) {
                    bg[j] = Bg[kk][tc * 4 + j];
                    if (GATEUP) bu[j] = Bu[kk][tc * 4 + j];
                }
                for (int i = 0; i < 4; ++i)
                    for (int j = 0; j < 4; ++j) {
                        g[i][j] = fmaf(a[i], bg[j], g[i][j]);
                        if (GATEUP) u[i][j] = fmaf(a[i], bu[j], u[i][j]);
                    }
            }
        }
        for (int i = 0; i < 4; ++i) {
            const int rt = tr * 4 + i;
            if (rt >= rows) continue;
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + tc * 4 + j;
                if (col >= N) continue;
                C[(long long)(row0 + rt) * N + col] = GATEUP ? gelu_erf(g[i][j]) * u[i][j] : g[i][j];
            }
        }
    }
}

}  // namespace

namespace {
int grid_for(long long tiles, int grid_cap) {
    const long long g = std::min<long long>(grid_cap, (tiles + 7) / 8 * 8);
    return (int)std::max<long long>(g, 8);
}
}  // namespace

hipError_t launch_gate_up(int dtype, const void* x_perm, const int32_t* off, const void* w_gate,
                          const void* w_up, void* h, int E, int d, int d_ff, long long max_rows,
                          int grid_cap, hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    if (dtype == 1) {
        // bound on sum over e of ceil(rows_e / BM): ceil(max_rows / BM) + E
        const long long mt = (max_rows + BM - 1) / BM + E;
        hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, dim3(grid_for(mt * (d_ff / (BNB / 2)), grid_cap)),
                           dim3(256), 0, s, (const uint16_t*)x_perm, (const uint16_t*)w_gate,
                           (const uint16_t*)w_up, (uint16_t*)h, off, E, d, d_ff);
    } else {
        const long long mt = (max_rows + FBM - 1) / FBM + E;
        hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3(grid_for(mt * ((d_ff + FBN - 1) / FBN), grid_cap)),
                           dim3(256), 0, s, (const float*)x_perm, (const float*)w_gate,
                           (const float*)w_up, (float*)h, off, E, d, d_ff);
    }
    return hipGetLastError();
}

hipError_t launch_down(int dtype, const void* h, const int32_t* off, const void* w_down,
                       void* y_perm, int E, int d, int d_ff, long long max_rows, int grid_cap,
                       hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    if (dtype == 1) {
        const long long mt = (max_rows + BM - 1) / BM + E;
        hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, dim3(grid_for(mt * ((d + BNB - 1) / BNB), grid_cap)),
                           dim3(256), 0, s, (const uint16_t*)h, (const uint16_t*)w_down,
                           (const uint16_t*)nullptr, (uint16_t*)y_perm, off, E, d_ff, d);
    } else {
        const long long mt = (max_rows + FBM - 1) / FBM + E;
        hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3(grid_for(mt * ((d + FBN - 1) / FBN), grid_cap)),
                           dim3(256), 0, s, (const float*)h, (const float*)w_down,
                           (const float*)nullptr, (float*)y_perm, off, E, d_ff, d);
    }
    return hipGetLastError();
}

hipError_t launch_expert_ffn(int dtype, const void* x_perm, const int32_t* off,
                             const void* w_gate, const void* w_up, const void* w_down,
                             void* h, void* y_perm, int E, int d, int d_ff,
                             long long max_rows, int grid_cap, hipStream_t s) {
    hipError_t err = launch_gate_up(dtype, x_perm, off, w_gate, w_up, h, E, d, d_ff, max_rows,
                                    grid_cap, s);
    if (err != hipSuccess) return err;
    return launch_down(dtype, h, off, w_down, y_perm, E, d, d_ff, max_rows, grid_cap, s);
}

}  // namespace moe
