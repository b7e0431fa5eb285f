// combine.hip -- gate-weighted un-permute and combine on gfx950.
//
// y[t] = sum over j = 0..k-1 (ascending) with row_of[t][j] >= 0 of
//        gate[t][j] * y_perm[row_of[t][j]], accumulated in fp32 and rounded
//        once to the output type; y[t] = 0 when nothing was kept.
// A gather (each output row is written exactly once, no atomics), so the
// result is deterministic.  One wave per token, 16-byte vector loads and
// stores; bound by HBM bandwidth.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// KMAX >= k choices per token; U vectors per lane in flight at once (the
// loads of all U are issued before any is used: one memory round trip per U
// vectors of each row).  NT: non-temporal loads and stores, for layers whose
// data are several times the 256 MB last-level cache.
template <typename T, int KMAX, int U, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y_perm,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gate,
                                                      u32x4* __restrict__ y, long long ntok,
                                                      int nvec, int k) {
    constexpr int PV = Elem<T>::kPerVec;
    const int lane = threadIdx.x & 63;
    const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= ntok) return;
    // row and gate of each choice, loaded together (the gate of a dropped
    // choice is read but never used)
    int rows[KMAX];
    float g[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        rows[j] = (j < k) ? row_of[t * k + j] : -1;
        g[j] = (j < k) ? gate[t * k + j] : 0.f;
    }
    u32x4* dst = y + t * nvec;
    for (int v0 = lane; v0 < nvec; v0 += U * 64) {
        float acc[U][PV];
        u32x4 in[U][KMAX];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int i = 0; i < PV; ++i) acc[u][i] = 0.f;
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (rows[j] >= 0 && v0 + u * 64 < nvec)
                    in[u][j] = NT ? __builtin_nontemporal_load(y_perm + (long long)rows[j] * nvec +
                                                               v0 + u * 64)
                                  : y_perm[(long long)rows[j] * nvec + v0 + u * 64];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (v0 + u * 64 >= nvec) continue;
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (rows[j] < 0) continue;
#pragma unroll
                for (int i = 0; i < PV; ++i)
                    acc[u][i] = fmaf(g[j], Elem<T>::to_f32(in[u][j], i), acc[u][i]);
            }
            u32x4 out;
            if constexpr (PV == 8) {
#pragma unroll
                for (int p = 0; p < 4; ++p) out[p] = pack_bf16x2(acc[u][2 * p], acc[u][2 * p + 1]);
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p) out[p] = __float_as_uint(acc[u][p]);
            }
            if (NT) __builtin_nontemporal_store(out, dst + v0 + u * 64);
            else dst[v0 + u * 64] = out;
        }
    }
}

// Top-1 layer that keeps every token, down GEMM in two K slices: one wave
// per token, 8 columns per lane and step; o = bf16(P0 + P1) as the GEMM's
// epilogue rounds its accumulators, then y = bf16(g * o) as the combine does.
__global__ __launch_bounds__(256) void combine_split_kernel(const float* __restrict__ P,
                                                            long long p_stride,
                                                            const int32_t* __restrict__ row_of,
                                                            const float* __restrict__ gate,
                                                            u32x4* __restrict__ y, long long ntok,
                                                            int d) {
    const int lane = threadIdx.x & 63;
    const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= ntok) return;
    const int r = row_of[t];
    const float g = gate[t];
    const f32x4* p0 = (const f32x4*)(P + (long long)r * d);
    const f32x4* p1 = (const f32x4*)(P + p_stride + (long long)r * d);
    u32x4* dst = y + t * (d / 8);
    for (int v = lane; v < d / 8; v += 64) {
        const f32x4 a0 = p0[2 * v], a1 = p0[2 * v + 1];
        const f32x4 b0 = p1[2 * v], b1 = p1[2 * v + 1];
        float o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[q] = (float)(__bf16)(a0[q] + b0[q]);
            o[q + 4] = (float)(__bf16)(a1[q] + b1[q]);
        }
        u32x4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            out[q] = pack_bf16x2(fmaf(g, o[2 * q], 0.f), fmaf(g, o[2 * q + 1], 0.f));
        dst[v] = out;
    }
}

}  // namespace

hipError_t launch_combine_split(const float* P, long long p_stride, const int32_t* row_of,
                                const float* gate, void* y, long long T, int d, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (d % 8 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_split_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, P,
                       p_stride, row_of, gate, (u32x4*)y, T, d);
    return hipGetLastError();
}

hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* row_of,
                          const float* gate, void* y, long long T, int d, int k,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    const dim3 grid((unsigned)((T + 3) / 4));
    // Stream past the caches only when the output alone is at least twice
    // the 256 MB last-level cache: smaller layers still find the down GEMM's
    // y_perm there, and non-temporal loads then measured 3-12% slower (wide
    // and skewed layers) against 7% faster on the long-sequence layer.
    const bool nt = (double)T * d * (dtype == 1 ? 2 : 4) >= 512.0 * (1 << 20);
    if (dtype == 1) {
        if (k <= 2) {
            if (nt)
                hipLaunchKernelGGL((combine_kernel<uint16_t, 2, 4, true>), grid, dim3(256), 0, s,
                                   (const u32x4*)y_perm, row_of, gate, (u32x4*)y, T, d / 8, k);
            else
                hipLaunchKernelGGL((combine_kernel<uint16_t, 2, 4, false>), grid, dim3(256), 0, s,
                                   (const u32x4*)y_perm, row_of, gate, (u32x4*)y, T, d / 8, k);
        } else {
            hipLaunchKernelGGL((combine_kernel<uint16_t, 8, 2, false>), grid, dim3(256), 0, s,
                               (const u32x4*)y_perm, row_of, gate, (u32x4*)y, T, d / 8, k);
        }
    } else {
        hipLaunchKernelGGL((combine_kernel<float, 8, 2, false>), grid, dim3(256), 0, s,
                           (const u32x4*)y_perm, row_of, gate, (u32x4*)y, T, d / 4, k);
    }
    return hipGetLastError();
}

}  // namespace moe
