// backward.hip -- the non-GEMM kernels of the layer's backward pass (bf16
// layers): the gate of each kept row and the sum of the gate gradient's
// partials (the GeGLU backward itself runs in the epilogue of the NT GEMM
// that computes dHr, gemm_bw.hip), softmax/top-k backward into the router
// logits, the router's weight, bias and input gradients, and the token-side
// gather-sum of the expert input gradients.
//
// Notation (per kept assignment (t, j) of expert e, row r of the expert-
// grouped layout): g = x Wg[e], u = x Wu[e], a = GELU(g), h = a u,
// o = h Wd[e], y_t = sum_j gate_tj o_tj.  With dHr = dy_t Wd[e]^T (the
// gradient of h before the gate):  dgate_tj = dy_t . o = h . dHr, dh = gate
// dHr, du = dh a, dg = dh u GELU'(g).  The softmax with temperature tau and
// optional renormalisation over the chosen experts is differentiated in the
// router kernel; top-k selection and capacity drops are piecewise constant.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Sum over the 64 lanes of a wave, the same butterfly order every time.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// row_gate[r] = the gate of the assignment (t, j) that row r < offset[E]
// holds, 0 for an empty row of the padded layout.
__global__ __launch_bounds__(256) void row_gate_kernel(const int32_t* __restrict__ offset,
                                                       const int32_t* __restrict__ token_of_row,
                                                       const int32_t* __restrict__ row_of,
                                                       const float* __restrict__ gate, int E,
                                                       int k, float* __restrict__ row_gate) {
    const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
    if (r >= offset[E]) return;
    const long long t = token_of_row[r];   // -1: an empty row of the padded layout
    float gt = 0.f;
    for (int j = 0; j < k && t >= 0; ++j)
        if (row_of[t * k + j] == r) gt = gate[t * k + j];
    row_gate[r] = gt;
}

// dgate_row[r] = h . dh_raw of row r < n_kept: its np partial sums (one per
// 64 columns of d_ff, from the NT epilogue) added in column order.
__global__ __launch_bounds__(256) void dgate_sum_kernel(const float* __restrict__ dot, int np,
                                                        const int32_t* __restrict__ offset, int E,
                                                        float* __restrict__ dgate_row) {
    const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
    if (r >= offset[E]) return;
    const float* p = dot + r * np;
    float v = 0.f;
    for (int c = 0; c < np; ++c) v += p[c];
    dgate_row[r] = v;
}

// One wave per token: p = softmax(l / tau) from the fp32 logits, dp from the
// gate gradients of the chosen experts (renormalised: gate_j = p_j / S, S the
// sum over the chosen ones, dp_j = (dgate_j - sum_j' dgate_j' gate_j') / S),
// dl = p (dp - p . dp) / tau.
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const int32_t* __restrict__ row_of,
    const float* __restrict__ dgate_row, long long T, int E, int k, float tau, int renorm,
    float* __restrict__ dl, float* __restrict__ dgate) {
    __shared__ float sp[4][256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const long long t = (long long)blockIdx.x * 4 + w;
    if (t >= T) return;   // whole wave
    const float* l = logits + t * E;
    float lv[4], p[4];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        lv[q] = e < E ? l[e] : -INFINITY;
        m = fmaxf(m, lv[q]);
    }
    m = wave_max(m);
    const float sc = 1.44269504088896341f / tau;
    float z = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        p[q] = e < E ? __builtin_amdgcn_exp2f((lv[q] - m) * sc) : 0.f;
        z += p[q];
    }
    z = wave_sum(z);
    const float rz = 1.0f / z;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        p[q] *= rz;
        const int e = lane + 64 * q;
        if (e < E) sp[w][e] = p[q];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // every lane walks the k choices (k <= 8); a slot holding -1 (a token
    // that took fewer than k experts) has no expert, gate 0 and no gradient
    float S = 0.f, sg = 0.f;
    float dga[8];
    int ej[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        dga[j] = 0.f;
        ej[j] = -1;
        if (j < k) {
            const long long a = t * k + j;
            const int rr = row_of[a];
            dga[j] = rr >= 0 ? dgate_row[rr] : 0.f;
            ej[j] = idx[a];
            if (ej[j] >= 0) S += sp[w][ej[j]];
            sg = fmaf(dga[j], gate[a], sg);
        }
    }
    const float rS = 1.0f / S;
    float dp[4], pd = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        dp[q] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k && ej[j] == e) dp[q] = renorm ? (dga[j] - sg) * rS : dga[j];
        pd = fmaf(p[q], dp[q], pd);
    }
    pd = wave_sum(pd);
    const float rt = 1.0f / tau;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        if (e < E) dl[t * E + e] = p[q] * (dp[q] - pd) * rt;
    }
    if (dgate != nullptr && lane < k) {
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j == lane) v = dga[j];
        dgate[t * k + lane] = v;
    }
}

// dx[t][i] = sum_j sum_p dXp_p[row_of[t, j]][i] + sum_e dl[t][e] Wr[i][e]
// (bf16 out; the parts p of the expert input gradient in part order).
// dl W_r^T on v_mfma_f32_16x16x32_bf16 with dl split into two bf16 terms
// (hi = bf16(dl), lo = bf16(dl - hi): about 16 bits of dl, W_r exact), both
// operands read from global memory straight into the fragment layout (lane
// (c16, g4): index c16, K values 8 g4 .. + 7).  Workgroup: 64 tokens x 256
// columns, each wave 64 x 64 (4 x 4 blocks of 16 x 16).  The expert parts are
// then added to the accumulators where they lie (each lane four consecutive
// columns of one token), with no trip through LDS, at three waves per SIMD
// (long-sequence layer 1.49 -> 0.94 ms against a version that staged the
// router part through LDS and added one token row per wave).  VEC: E % 8 ==
// 0, so eight K values are one aligned vector.
template <bool VEC>
__global__ __launch_bounds__(256, 3) void dx_kernel(
    const float* __restrict__ dl, const uint16_t* __restrict__ wr,
    const float* __restrict__ dXp, int nparts, long long part_stride,
    const int32_t* __restrict__ row_of, uint16_t* __restrict__ dx, long long T, int d, int E,
    int k) {
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15, g4 = lane >> 4;
    const long long t0 = (long long)blockIdx.x * 64;
    const int i0 = blockIdx.y * 256 + w * 64;
    // the expert rows of this lane's four tokens t0 + 16 ib + c16 (k <= 8),
    // loaded before the router product so that their latency is hidden; -1
    // past the last token and for dropped assignments
    int rj[4][8];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
        const long long t = t0 + ib * 16 + c16;
#pragma unroll
        for (int j = 0; j < 8; ++j) rj[ib][j] = j < k && t < T ? row_of[t * k + j] : -1;
    }
    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int e0 = 0; e0 < E; e0 += 32) {
        const int ek = e0 + 8 * g4;   // this lane's first K value
        bf16x8 fb[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const int i = i0 + jb * 16 + c16;
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (i < d) {
                const uint16_t* src = wr + (long long)i * E + ek;
                if (VEC) {
                    if (ek < E) raw = *(const u32x4*)src;
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) h[u] = ek + u < E ? src[u] : 0u;
                    raw = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                h[6] | (h[7] << 16)};
                }
            }
            fb[jb] = __builtin_bit_cast(bf16x8, raw);
        }
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            const long long t = t0 + ib * 16 + c16;
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (t < T) {
                const float* src = dl + t * E + ek;
                if (VEC) {
                    if (ek < E) {
                        const f32x4 v0 = *(const f32x4*)src, v1 = *(const f32x4*)(src + 4);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            v[u] = v0[u];
                            v[4 + u] = v1[u];
                        }
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < 8; ++u) v[u] = ek + u < E ? src[u] : 0.f;
                }
            }
            bf16x8 hi, lo;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                hi[u] = (__bf16)v[u];
                lo[u] = (__bf16)(v[u] - (float)hi[u]);
            }
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                acc[ib][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[jb], hi, acc[ib][jb], 0, 0, 0);
                acc[ib][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[jb], lo, acc[ib][jb], 0, 0, 0);
            }
        }
    }
    // the expert parts added in the MFMA layout itself (lane (g4, c16) of
    // block (ib, jb): token t0 + 16 ib + c16, columns i0 + 16 jb + 4 g4 .. + 3),
    // in choice order, then part order, one 16-token block at a time
    if (i0 >= d) return;   // d is a multiple of 64: the wave's 64 columns are all in or all out
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= k) break;   // uniform
            const int rr = rj[ib][j];
            for (int p = 0; p < nparts; ++p) {
                const float* base = dXp + p * part_stride + i0 + 4 * g4 + (long long)rr * d;
                f32x4 g[4];
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
                    if (rr >= 0) g[jb] = *(const f32x4*)(base + jb * 16);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
                    if (rr >= 0) acc[ib][jb] += g[jb];
            }
        }
        const long long t = t0 + ib * 16 + c16;
        if (t < T) {
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                *(u32x2*)(dx + t * d + i0 + jb * 16 + 4 * g4) =
                    u32x2{pack_bf16x2(acc[ib][jb][0], acc[ib][jb][1]),
                          pack_bf16x2(acc[ib][jb][2], acc[ib][jb][3])};
        }
    }
}

// Eight consecutive elements of x (bf16 or fp32; 16-byte aligned) as fp32.
template <typename XT>
__device__ __forceinline__ void load8(const XT* p, float v[8]) {
    if constexpr (sizeof(XT) == 2) {
        const u32x4 raw = *(const u32x4*)p;
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = Elem<uint16_t>::to_f32(raw, u);
    } else {
        const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[u] = a[u];
            v[4 + u] = b[u];
        }
    }
}

// Partial router weight gradients over one split of the tokens:
// part[s][i][e] = sum_{t in split s} x[t][i] dl[t][e]; the first column tile
// also writes bpart[s][e] = sum_t dl[t][e].  Tile 256 (i) x 64 (e), 8 x 8 per
// thread, t in chunks of 16 through LDS.
template <typename XT>
__global__ __launch_bounds__(256, 2) void dwr_part_kernel(
    const XT* __restrict__ x, const float* __restrict__ dl, float* __restrict__ part,
    float* __restrict__ bpart, long long T, int d, int E, long long split) {
    __shared__ __attribute__((aligned(16))) float s_x[16][256];
    __shared__ __attribute__((aligned(16))) float s_l[16][64];
    const int tid = threadIdx.x, ti = tid >> 3, te = tid & 7;
    const int i0 = blockIdx.x * 256, e0 = blockIdx.y * 64, s = blockIdx.z;
    const long long ta = (long long)s * split, tb = min(T, ta + split);
    float acc[8][8] = {};
    float bacc[8] = {};
    const bool do_b = blockIdx.x == 0 && ti == 0;
    for (long long tc = ta; tc < tb; tc += 16) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {   // x: 16 tokens x 256 columns, 8 per thread
            const int q = tid + 256 * r, kk = q >> 5, c8 = (q & 31) * 8;
            const long long t = tc + kk;
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (t < tb && i0 + c8 < d) load8(x + t * d + i0 + c8, v);
            *(f32x4*)&s_x[kk][c8] = f32x4{v[0], v[1], v[2], v[3]};
            *(f32x4*)&s_x[kk][c8 + 4] = f32x4{v[4], v[5], v[6], v[7]};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {   // dl: 16 tokens x 64 e
            const int q = tid + 256 * r, kk = q >> 6, c = q & 63;
            const long long t = tc + kk;
            s_l[kk][c] = (t < tb && e0 + c < E) ? dl[t * E + e0 + c] : 0.f;
        }
        __syncthreads();
#pragma unroll 2
        for (int kk = 0; kk < 16; ++kk) {
            const f32x4 a0 = *(const f32x4*)&s_x[kk][ti * 8];
            const f32x4 a1 = *(const f32x4*)&s_x[kk][ti * 8 + 4];
            const f32x4 b0 = *(const f32x4*)&s_l[kk][te * 8];
            const f32x4 b1 = *(const f32x4*)&s_l[kk][te * 8 + 4];
            const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int xx = 0; xx < 8; ++xx)
#pragma unroll
                for (int y = 0; y < 8; ++y) acc[xx][y] = fmaf(a[xx], b[y], acc[xx][y]);
            if (do_b)
#pragma unroll
                for (int y = 0; y < 8; ++y) bacc[y] += b[y];
        }
        __syncthreads();
    }
#pragma unroll
    for (int xx = 0; xx < 8; ++xx) {
        const int i = i0 + ti * 8 + xx;
        if (i >= d) continue;
#pragma unroll
        for (int y = 0; y < 8; ++y) {
            const int e = e0 + te * 8 + y;
            if (e < E) part[((long long)s * d + i) * E + e] = acc[xx][y];
        }
    }
    if (do_b)
#pragma unroll
        for (int y = 0; y < 8; ++y) {
            const int e = e0 + te * 8 + y;
            if (e < E) bpart[(long long)s * E + e] = bacc[y];
        }
}

// The same partial sums for layers with few experts (E <= TE, TE = 8 or 16):
// a thread owns 8 consecutive columns i and all TE experts, so every x
// element is read once, straight from global memory (16 bytes per thread and
// token, a workgroup covering 2048 columns), and the dl row of each token is
// uniform across the workgroup.  Tokens of the split ascending, four at a
// time so that four x loads are in flight.  The 64-expert tile of
// dwr_part_kernel would spend 64 / E of its multiply-adds on padding here.
template <int TE, typename XT>
__global__ __launch_bounds__(256) void dwr_narrow_kernel(
    const XT* __restrict__ x, const float* __restrict__ dl, float* __restrict__ part,
    float* __restrict__ bpart, long long T, int d, int E, long long split) {
    const int tid = threadIdx.x;
    const int i0 = blockIdx.x * 2048 + tid * 8;
    const int s = blockIdx.z;
    const long long ta = (long long)s * split, tb = min(T, ta + split);
    const bool active = i0 < d;   // d % 64 == 0: whole 8-column groups
    float acc[8][TE] = {};
    float bacc[TE] = {};
    for (long long t0 = ta; t0 < tb; t0 += 4) {
        float xv[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const long long t = t0 + q;
            if (active && t < tb) {
                load8(x + t * d + i0, xv[q]);
            } else {
#pragma unroll
                for (int u = 0; u < 8; ++u) xv[q][u] = 0.f;
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const long long t = t0 + q;
            if (t >= tb) break;   // uniform
            float b[TE];
#pragma unroll
            for (int e = 0; e < TE; ++e) b[e] = e < E ? dl[t * E + e] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float a = xv[q][u];
#pragma unroll
                for (int e = 0; e < TE; ++e) acc[u][e] = fmaf(a, b[e], acc[u][e]);
            }
#pragma unroll
            for (int e = 0; e < TE; ++e) bacc[e] += b[e];
        }
    }
    if (active) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < TE; ++e)
                if (e < E) part[((long long)s * d + i0 + u) * E + e] = acc[u][e];
    }
    if (blockIdx.x == 0 && tid == 0)
#pragma unroll
        for (int e = 0; e < TE; ++e)
            if (e < E) bpart[(long long)s * E + e] = bacc[e];
}

// Sum of the splits in split order: dwr [d][E], dbias [E] (may be null).
__global__ __launch_bounds__(256) void dwr_reduce_kernel(const float* __restrict__ part,
                                                         const float* __restrict__ bpart,
                                                         float* __restrict__ dwr,
                                                         float* __restrict__ dbias, int d, int E,
                                                         int nsplit) {
    const long long n = (long long)d * E;
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
    if (q < n) {
        float v = 0.f;
        for (int s = 0; s < nsplit; ++s) v += part[(long long)s * n + q];
        dwr[q] = v;
    } else if (dbias != nullptr && q < n + E) {
        const int e = (int)(q - n);
        float v = 0.f;
        for (int s = 0; s < nsplit; ++s) v += bpart[(long long)s * E + e];
        dbias[e] = v;
    }
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, long long n) {
    for (long long q = (long long)blockIdx.x * 256 + threadIdx.x; q < n;
         q += (long long)gridDim.x * 256)
        p[q] = 0.f;
}

}  // namespace

hipError_t launch_row_gate(const int32_t* offset, const int32_t* token_of_row,
                           const int32_t* row_of, const float* gate, int E, int k,
                           long long max_rows, float* row_gate, hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(row_gate_kernel, dim3((unsigned)((max_rows + 255) / 256)), dim3(256), 0, s,
                       offset, token_of_row, row_of, gate, E, k, row_gate);
    return hipGetLastError();
}

hipError_t launch_dgate_sum(const float* dot, int np, const int32_t* offset, int E,
                            long long max_rows, float* dgate_row, hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(dgate_sum_kernel, dim3((unsigned)((max_rows + 255) / 256)), dim3(256), 0, s,
                       dot, np, offset, E, dgate_row);
    return hipGetLastError();
}

hipError_t launch_router_bwd(const float* logits, const int32_t* idx, const float* gate,
                             const int32_t* row_of, const float* dgate_row, long long T, int E,
                             int k, float tau, int renorm, float* dl, float* dgate,
                             hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (E > 256 || k > 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits,
                       idx, gate, row_of, dgate_row, T, E, k, tau, renorm, dl, dgate);
    return hipGetLastError();
}

hipError_t launch_dx(const float* dl, const uint16_t* wr, const float* dXp, int nparts,
                     long long part_stride, const int32_t* row_of, uint16_t* dx, long long T,
                     int d, int E, int k, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (d % 64 != 0 || k < 1 || k > 8) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((T + 63) / 64), (d + 255) / 256);
    if (E % 8 == 0)
        hipLaunchKernelGGL(dx_kernel<true>, grid, dim3(256), 0, s, dl, wr, dXp, nparts,
                           part_stride, row_of, dx, T, d, E, k);
    else
        hipLaunchKernelGGL(dx_kernel<false>, grid, dim3(256), 0, s, dl, wr, dXp, nparts,
                           part_stride, row_of, dx, T, d, E, k);
    return hipGetLastError();
}

// Column tiles and token splits: about two workgroups per CU, splits of at
// least 64 tokens.
static long long dwr_splits_for(long long T, long long tiles) {
    long long ns = (512 + tiles - 1) / tiles;
    ns = std::min<long long>(ns, std::max<long long>(1, (T + 63) / 64));
    return std::max<long long>(1, std::min<long long>(ns, 4096));
}

// Few experts and enough tokens to fill the chip with 2048-column
// workgroups: dwr_narrow_kernel (long-sequence layer 1046 -> 262 us), else
// dwr_part_kernel, 256 columns x 64 experts (the ZAYA1-like layer, whose
// 4,096 tokens would make only 64 narrow workgroups: 50 us against 86).
static bool dwr_narrow(long long T, int d, int E) {
    const long long tiles = (d + 2047) / 2048;
    return E <= 16 && tiles * dwr_splits_for(T, tiles) >= 256;
}

int dwr_splits(long long T, int d, int E) {
    const long long tiles = dwr_narrow(T, d, E) ? (long long)((d + 2047) / 2048)
                                                : (long long)((d + 255) / 256) * ((E + 63) / 64);
    return (int)dwr_splits_for(T, tiles);
}

size_t dwr_workspace_bytes(long long T, int d, int E) {
    const int ns = dwr_splits(T, d, E);
    return (size_t)ns * ((size_t)d * E + E) * sizeof(float);
}

namespace {
template <typename XT>
hipError_t dwr_parts(const XT* x, const float* dl, float* part, float* bpart, long long T, int d,
                     int E, int ns, long long split, hipStream_t s) {
    const bool narrow = dwr_narrow(T, d, E);
    if (narrow && E <= 8)
        hipLaunchKernelGGL((dwr_narrow_kernel<8, XT>), dim3((d + 2047) / 2048, 1, ns), dim3(256), 0,
                           s, x, dl, part, bpart, T, d, E, split);
    else if (narrow)
        hipLaunchKernelGGL((dwr_narrow_kernel<16, XT>), dim3((d + 2047) / 2048, 1, ns), dim3(256),
                           0, s, x, dl, part, bpart, T, d, E, split);
    else
        hipLaunchKernelGGL(dwr_part_kernel<XT>, dim3((d + 255) / 256, (E + 63) / 64, ns),
                           dim3(256), 0, s, x, dl, part, bpart, T, d, E, split);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_dwr(int dtype, const void* x, const float* dl, float* dwr, float* dbias,
                      long long T, int d, int E, void* ws, hipStream_t s) {
    if (d % 64 != 0) return hipErrorInvalidValue;
    const int ns = dwr_splits(T, d, E);
    const long long split = T == 0 ? 1 : ((T + ns - 1) / ns + 15) / 16 * 16;
    float* part = (float*)ws;
    float* bpart = part + (size_t)ns * d * E;
    hipError_t e = dtype == 1
        ? dwr_parts((const uint16_t*)x, dl, part, bpart, T, d, E, ns, split, s)
        : dwr_parts((const float*)x, dl, part, bpart, T, d, E, ns, split, s);
    if (e != hipSuccess) return e;
    const long long n = (long long)d * E + E;
    hipLaunchKernelGGL(dwr_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                       bpart, dwr, dbias, d, E, ns);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, long long n, hipStream_t s) {
    if (n == 0 || p == nullptr) return hipSuccess;
    const long long blocks = std::min<long long>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace moe
