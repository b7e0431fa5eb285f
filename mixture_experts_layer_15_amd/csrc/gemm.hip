// gemm.hip -- launchers of the grouped expert GEMMs, and the fp32 path.
//
// bf16 layers run the MFMA kernels of gemm_mfma.hip.  fp32 layers run plain
// fp32 FMA tiles here: 64 x 64 outputs per workgroup, K-steps of 16, 4 x 4
// outputs per thread, walking the same device-built tile list (tiles.h).
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int FBM = 64, FBN = 64, FBK = 16;

// GATEUP with C2 != nullptr: the two products unfused, g into C and u into C2
// (the backward's recompute).
template <bool GATEUP>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B0, const float* __restrict__ B1,
    float* __restrict__ C, const int32_t* __restrict__ off, int E, int K, int N,
    float* __restrict__ C2) {
    __shared__ float As[FBK][FBM + 4];
    __shared__ float Bg[FBK][FBN + 4];
    __shared__ float Bu[FBK][FBN + 4];
    __shared__ TileTable tt;
    __shared__ long long s_wave[8];
    const int ntn = (N + FBN - 1) / FBN;
    build_tile_table<FBM>(off, E, ntn, tt, s_wave);
    const long long total = tt.start[E];
    const int tid = threadIdx.x;
    const int tr = tid >> 4, tc = tid & 15;   // 16 x 16 threads, 4 x 4 outputs each
    const long long KN = (long long)K * N;
    for (long long t = blockIdx.x; t < total; t += gridDim.x) {
        int e, mtile, ntile;
        decode_tile<1>(tt, E, ntn, t, e, mtile, ntile);
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
                const long long o = (long long)(row0 + rt) * N + col;
                if (GATEUP && C2 != nullptr) {
                    C[o] = g[i][j];
                    C2[o] = u[i][j];
                } else {
                    C[o] = GATEUP ? gelu_erf(g[i][j]) * u[i][j] : g[i][j];
                }
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
                          int grid_cap, hipStream_t s, const int32_t* gather_rows) {
    if (max_rows == 0) return hipSuccess;
    if (gather_rows != nullptr && dtype != 1) return hipErrorInvalidValue;   // bf16 only
    if (dtype == 1)
        return launch_mfma_gate_up((const uint16_t*)x_perm, gather_rows, off, (const uint16_t*)w_gate,
                                   (const uint16_t*)w_up, (uint16_t*)h, E, d, d_ff, max_rows,
                                   grid_cap / 2, s);
    {
        const long long mt = (max_rows + FBM - 1) / FBM + E;
        hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3(grid_for(mt * ((d_ff + FBN - 1) / FBN), grid_cap)),
                           dim3(256), 0, s, (const float*)x_perm, (const float*)w_gate,
                           (const float*)w_up, (float*)h, off, E, d, d_ff, (float*)nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_gate_up_pre_f32(const float* x_perm, const int32_t* off, const float* w_gate,
                                  const float* w_up, float* g, float* u, int E, int d, int d_ff,
                                  long long max_rows, int grid_cap, hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    const long long mt = (max_rows + FBM - 1) / FBM + E;
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>,
                       dim3(grid_for(mt * ((d_ff + FBN - 1) / FBN), grid_cap)), dim3(256), 0, s,
                       x_perm, w_gate, w_up, g, off, E, d, d_ff, u);
    return hipGetLastError();
}

hipError_t launch_down(int dtype, const void* h, const int32_t* off, const void* w_down,
                       void* y_perm, int E, int d, int d_ff, long long max_rows, int grid_cap,
                       hipStream_t s, const float* gate, const int32_t* token_of_row, void* y) {
    if (max_rows == 0) return hipSuccess;
    if (y != nullptr && dtype != 1) return hipErrorInvalidValue;   // bf16 only
    if (dtype == 1)
        return launch_mfma_down((const uint16_t*)h, off, (const uint16_t*)w_down,
                                (uint16_t*)y_perm, E, d, d_ff, max_rows, grid_cap / 2, s, gate,
                                token_of_row, (uint16_t*)y);
    {
        const long long mt = (max_rows + FBM - 1) / FBM + E;
        hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3(grid_for(mt * ((d + FBN - 1) / FBN), grid_cap)),
                           dim3(256), 0, s, (const float*)h, (const float*)w_down,
                           (const float*)nullptr, (float*)y_perm, off, E, d_ff, d, (float*)nullptr);
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
