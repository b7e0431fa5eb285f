// backward_f32.hip -- the products of the backward pass for fp32 layers.
//
// Plain fp32 FMA tiles, as gemm.hip's fp32 forward path: 64 x 64 outputs per
// workgroup of 256 threads, 4 x 4 outputs per thread, K-steps of 16 through
// LDS, every sum over K in ascending order.  The bf16 layers' MFMA kernels
// (gemm_bw.hip, backward.hip) compute the same quantities; here nothing is
// rounded below fp32.
//   NT  C[r][n] = sum_k A[r][k] W[e][n][k] (+ A2[r][k] W2[e][n][k]) over the
//       rows r of each expert e: dh_raw = dy W_down^T (with the GeGLU backward
//       in the epilogue) and dx_perm = dg W_gate^T + du W_up^T
//   TN  C[e][m][n] = sum over the rows r of expert e of A[r][m] B[r][n]: the
//       expert weight gradients
//   dx  dx[t][i] = sum_e dl[t][e] Wr[i][e] + sum_j dx_perm[row_of[t][j]][i]
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int TB = 64, TK16 = 16;

// GeGLU backward of one fp32 element (GELU in its erf form, the device
// library's erff and expf): dg, du, gate h and the term h dh_raw of dgate.
__device__ __forceinline__ void geglu_bwd_f32(float g, float u, float dh_raw, float gt, float& dg,
                                              float& du, float& gh, float& term) {
    const float Phi = 0.5f * (1.0f + erff(g * 0.70710678118654752440f));
    const float phi = expf(-0.5f * g * g) * 0.39894228040143267794f;
    const float a = g * Phi;
    const float h = a * u;
    term = h * dh_raw;
    const float dh = gt * dh_raw;
    du = dh * a;
    dg = dh * u * fmaf(g, phi, Phi);
    gh = gt * h;
}

// NT over the expert-grouped rows.  TWO: a second source summed in the same
// accumulator (its K loop after the first's).  EPI: the result is dh_raw and
// the epilogue applies the GeGLU backward: G, U in place -> dg, du, gH = gate
// h, and dot[row][n0 / 64] = this tile's 64 columns of h . dh_raw.
template <bool TWO, bool EPI>
__global__ __launch_bounds__(256) void nt_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ W, const float* __restrict__ A2,
    const float* __restrict__ W2, float* __restrict__ C, const int32_t* __restrict__ off, int E,
    int K, int N, float* __restrict__ G, float* __restrict__ U, float* __restrict__ gH,
    const float* __restrict__ row_gate, float* __restrict__ dot) {
    __shared__ float As[TK16][TB + 4];
    __shared__ float Ws[TK16][TB + 4];
    __shared__ TileTable tt;
    __shared__ long long s_wave[8];
    const int ntn = (N + TB - 1) / TB;
    build_tile_table<TB>(off, E, ntn, tt, s_wave);
    const long long total = tt.start[E];
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    for (long long t = blockIdx.x; t < total; t += gridDim.x) {
        int e, mtile, ntile;
        decode_tile<1>(tt, E, ntn, t, e, mtile, ntile);
        const int row0 = off[e] + mtile * TB;
        const int rows = min(TB, off[e + 1] - row0);
        const int n0 = ntile * TB;
        float acc[4][4] = {};
        for (int src = 0; src < (TWO ? 2 : 1); ++src) {
            const float* a = src ? A2 : A;
            const float* w = src ? W2 : W;
            for (int k0 = 0; k0 < K; k0 += TK16) {
                __syncthreads();
                for (int v = tid; v < TB * TK16; v += 256) {
                    const int r = v / TK16, kk = v % TK16;
                    As[kk][r] = a[(long long)(row0 + min(r, rows - 1)) * K + k0 + kk];
                    Ws[kk][r] = w[((long long)e * N + min(n0 + r, N - 1)) * K + k0 + kk];
                }
                __syncthreads();
                for (int kk = 0; kk < TK16; ++kk) {
                    float av[4], wv[4];
                    for (int i = 0; i < 4; ++i) av[i] = As[kk][tr * 4 + i];
                    for (int j = 0; j < 4; ++j) wv[j] = Ws[kk][tc * 4 + j];
                    for (int i = 0; i < 4; ++i)
                        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
                }
            }
        }
        for (int i = 0; i < 4; ++i) {
            const int r = tr * 4 + i;
            float part = 0.f;
            const bool row_ok = r < rows;
            if (row_ok) {
                const long long rowg = row0 + r;
                const float gt = EPI ? row_gate[rowg] : 0.f;
                for (int j = 0; j < 4; ++j) {
                    const int col = n0 + tc * 4 + j;
                    if (col >= N) continue;
                    const long long o = rowg * N + col;
                    if (EPI) {
                        float dg, du, gh, term;
                        geglu_bwd_f32(G[o], U[o], acc[i][j], gt, dg, du, gh, term);
                        G[o] = dg;
                        U[o] = du;
                        gH[o] = gh;
                        part += term;
                    } else {
                        C[o] = acc[i][j];
                    }
                }
            }
            if (EPI) {
                // the 16 threads of this row (tc = 0..15, consecutive lanes of one wave)
                for (int m = 1; m < 16; m <<= 1) part += __shfl_xor(part, m);
                if (tc == 0 && row_ok) dot[(long long)(row0 + r) * (N / TB) + n0 / TB] = part;
            }
        }
    }
}

// TN: tiles (e, m-tile, n-tile); the K loop walks the rows of expert e.
__global__ __launch_bounds__(256) void tn_f32_kernel(const float* __restrict__ A,
                                                     const float* __restrict__ B,
                                                     float* __restrict__ C,
                                                     const int32_t* __restrict__ off, int E, int M,
                                                     int N) {
    __shared__ float As[TK16][TB + 4];
    __shared__ float Bs[TK16][TB + 4];
    const int mtn = (M + TB - 1) / TB, ntn = (N + TB - 1) / TB;
    const long long total = (long long)E * mtn * ntn;
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    for (long long t = blockIdx.x; t < total; t += gridDim.x) {
        const int e = (int)(t / ((long long)mtn * ntn));
        const int rem = (int)(t % ((long long)mtn * ntn));
        const int m0 = (rem / ntn) * TB, n0 = (rem % ntn) * TB;
        const int r_beg = off[e], r_end = off[e + 1];
        float acc[4][4] = {};
        for (int k0 = r_beg; k0 < r_end; k0 += TK16) {
            __syncthreads();
            for (int v = tid; v < TB * TK16; v += 256) {
                const int kk = v / TB, c = v % TB;
                const int r = k0 + kk;
                As[kk][c] = (r < r_end && m0 + c < M) ? A[(long long)r * M + m0 + c] : 0.f;
                Bs[kk][c] = (r < r_end && n0 + c < N) ? B[(long long)r * N + n0 + c] : 0.f;
            }
            __syncthreads();
            for (int kk = 0; kk < TK16; ++kk) {
                float av[4], bv[4];
                for (int i = 0; i < 4; ++i) av[i] = As[kk][tr * 4 + i];
                for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tc * 4 + j];
                for (int i = 0; i < 4; ++i)
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
            }
        }
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + tr * 4 + i;
            if (m >= M) continue;
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + tc * 4 + j;
                if (n < N) C[((long long)e * M + m) * N + n] = acc[i][j];
            }
        }
    }
}

// One thread per (token, column): the router part (experts ascending), then
// the expert parts in choice order.
__global__ __launch_bounds__(256) void dx_f32_kernel(const float* __restrict__ dl,
                                                     const float* __restrict__ wr,
                                                     const float* __restrict__ dXp,
                                                     const int32_t* __restrict__ row_of,
                                                     float* __restrict__ dx, long long T, int d,
                                                     int E, int k) {
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
    if (q >= T * d) return;
    const long long t = q / d;
    const int i = (int)(q % d);
    float v = 0.f;
    for (int e = 0; e < E; ++e) v = fmaf(dl[t * E + e], wr[(long long)i * E + e], v);
    for (int j = 0; j < k; ++j) {
        const int r = row_of[t * k + j];
        if (r >= 0) v += dXp[(long long)r * d + i];
    }
    dx[q] = v;
}

int grid_f32(long long tiles, int cap) {
    const long long g = std::min<long long>(cap, (tiles + 7) / 8 * 8);
    return (int)std::max<long long>(g, 8);
}

}  // namespace

hipError_t launch_bw_nt_f32(const float* A, const float* W, const float* A2, const float* W2,
                            float* C, const int32_t* off, int E, int N, int K, long long max_rows,
                            int cus, hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    if (K % TK16 != 0) return hipErrorInvalidValue;
    const long long tiles = ((max_rows + TB - 1) / TB + E) * ((N + TB - 1) / TB);
    if (A2 != nullptr)
        hipLaunchKernelGGL((nt_f32_kernel<true, false>), dim3(grid_f32(tiles, cus)), dim3(256), 0, s,
                           A, W, A2, W2, C, off, E, K, N, nullptr, nullptr, nullptr, nullptr,
                           nullptr);
    else
        hipLaunchKernelGGL((nt_f32_kernel<false, false>), dim3(grid_f32(tiles, cus)), dim3(256), 0,
                           s, A, W, nullptr, nullptr, C, off, E, K, N, nullptr, nullptr, nullptr,
                           nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_bw_nt_geglu_f32(const float* A, const float* W, float* G, float* U, float* gH,
                                  const float* row_gate, float* dot, const int32_t* off, int E,
                                  int N, int K, long long max_rows, int cus, hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    if (K % TK16 != 0 || N % TB != 0) return hipErrorInvalidValue;
    const long long tiles = ((max_rows + TB - 1) / TB + E) * ((N + TB - 1) / TB);
    hipLaunchKernelGGL((nt_f32_kernel<false, true>), dim3(grid_f32(tiles, cus)), dim3(256), 0, s,
                       A, W, nullptr, nullptr, nullptr, off, E, K, N, G, U, gH, row_gate, dot);
    return hipGetLastError();
}

hipError_t launch_bw_tn_f32(const float* A, const float* B, float* C, const int32_t* off, int E,
                            int M, int N, int cus, hipStream_t s) {
    if (E == 0) return hipSuccess;
    const long long tiles = (long long)E * ((M + TB - 1) / TB) * ((N + TB - 1) / TB);
    hipLaunchKernelGGL(tn_f32_kernel, dim3(grid_f32(tiles, cus)), dim3(256), 0, s, A, B, C, off, E,
                       M, N);
    return hipGetLastError();
}

hipError_t launch_dx_f32(const float* dl, const float* wr, const float* dXp,
                         const int32_t* row_of, float* dx, long long T, int d, int E, int k,
                         hipStream_t s) {
    if (T == 0) return hipSuccess;
    const long long n = T * d;
    hipLaunchKernelGGL(dx_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dl, wr,
                       dXp, row_of, dx, T, d, E, k);
    return hipGetLastError();
}

}  // namespace moe
