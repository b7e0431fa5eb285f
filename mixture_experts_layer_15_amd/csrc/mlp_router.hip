// mlp_router.hip -- the ZAYA1 MLP router, forward, on gfx950.
//
// A variant of the linear router ("AMD MI300X平台上的MoE模型训练实践", section
// 3.2): per token
//   u  = x Wd + bd                          down-projection to r
//   z  = RMSnorm(u + gamma * prev)          depth averaging with the previous
//                                           layer's router state, RMS norm with
//                                           no learned scale
//   h1 = GELU(z W1 + b1), h2 = GELU(h1 W2 + b2)
//   l  = h2 W3 + b3 + pid                   pid: the load-balance controller's
//                                           per-expert bias
// then the same temperature softmax and top-k as the linear router.  The
// three wide products run on the grouped MFMA GEMM in its dense mode (bias and
// GELU in the epilogue, bf16 out); the output layer is the linear router's
// kernel with W3 as its weight and b3 + pid as its bias, so the ranking and
// gates are the linear router's code.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// One wave per token: v = u + gamma * prev in fp32, z = v / sqrt(mean v^2 +
// eps), rounded once to bf16.  Workgroup 0 also sums the output biases.
__global__ __launch_bounds__(256) void eda_rmsnorm_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ prev, float gamma, float eps,
    uint16_t* __restrict__ z, long long T, int r, const float* __restrict__ b3,
    const float* __restrict__ pid, float* __restrict__ bias_sum, int E) {
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e < E; e += 256)
            bias_sum[e] = (b3 ? b3[e] : 0.f) + (pid ? pid[e] : 0.f);
    const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    // r <= 1024 (checked on the host): at most 16 values per lane
    float v[16];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const int j = lane + 64 * c;
        v[c] = 0.f;
        if (j < r) {
            float a = bf16_bits_to_f32(u[t * r + j]);
            if (prev) a = fmaf(gamma, bf16_bits_to_f32(prev[t * r + j]), a);
            v[c] = a;
            ss = fmaf(a, a, ss);
        }
    }
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.0f / sqrtf(ss / (float)r + eps);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const int j = lane + 64 * c;
        if (j < r) z[t * r + j] = (uint16_t)f32_to_bf16_bits(v[c] * inv);
    }
}

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t mlp_router_workspace_bytes(long long T, int r, int m, int E) {
    return 2 * al256((size_t)T * r * 2) + 2 * al256((size_t)T * m * 2) + al256((size_t)E * 4);
}

hipError_t launch_route_mlp(const uint16_t* x, const uint16_t* prev, float gamma, float eps,
                            const uint16_t* wd, const float* bd, const uint16_t* w1,
                            const float* b1, const uint16_t* w2, const float* b2,
                            const uint16_t* w3, const float* b3, const float* pid,
                            float* logits, int32_t* idx, float* gate, long long T, int d, int r,
                            int m, int E, TopkParams tp, void* ws, int cus,
                            hipStream_t s) {
    if (T == 0) return hipSuccess;
    char* w = (char*)ws;
    uint16_t* u = (uint16_t*)w;
    w += al256((size_t)T * r * 2);
    uint16_t* z = (uint16_t*)w;
    w += al256((size_t)T * r * 2);
    uint16_t* h1 = (uint16_t*)w;
    w += al256((size_t)T * m * 2);
    uint16_t* h2 = (uint16_t*)w;
    w += al256((size_t)T * m * 2);
    float* bias_sum = (float*)w;
    hipError_t e = launch_mfma_dense(x, wd, bd, 0, u, (int)T, d, r, cus, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(eda_rmsnorm_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, u, prev,
                       gamma, eps, z, T, r, b3, pid, bias_sum, E);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_mfma_dense(z, w1, b1, 1, h1, (int)T, r, m, cus, s);
    if (e != hipSuccess) return e;
    e = launch_mfma_dense(h1, w2, b2, 1, h2, (int)T, m, m, cus, s);
    if (e != hipSuccess) return e;
    return launch_route(1, h2, w3, bias_sum, logits, idx, gate, T, m, E, tp, s);
}

}  // namespace moe
