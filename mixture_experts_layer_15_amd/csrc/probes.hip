// probes.hip -- measurement probes (include/moe_probe.h): a streaming copy,
// a streaming read and a dense bf16 MFMA stream with clock stamps.  They
// measure the chip; the layer's path never calls them.
#include <hip/hip_runtime.h>

#include "../../include/moe_probe.h"
#include "common.h"

namespace {

using moe::f32x4;
using moe::u32x4;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, long long n) {
    const long long stride = (long long)gridDim.x * 256 * 4;
    long long i = (long long)blockIdx.x * 256 * 4 + threadIdx.x;
    for (; i + 3 * 256 < n; i += stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * 256);
    }
    for (int u = 0; u < 4; ++u)   // the ragged end of the last stride
        if (i + u * 256 < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i + u * 256),
                                                         dst + i + u * 256);
}

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src,
                                                         long long n, float* __restrict__ sink) {
    const long long stride = (long long)gridDim.x * 256 * 4;
    long long i = (long long)blockIdx.x * 256 * 4 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * 256 < n; i += stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (int u = 0; u < 4; ++u)
        if (i + u * 256 < n) {
            const u32x4 v = __builtin_nontemporal_load(src + i + u * 256);
            acc += v[0] ^ v[1] ^ v[2] ^ v[3];
        }
    sink[(long long)blockIdx.x * 256 + threadIdx.x] = (float)acc;
}

__global__ __launch_bounds__(512) void probe_mfma_kernel(int iters, float* __restrict__ sink,
                                                         uint64_t* __restrict__ stamps) {
    const int tid = threadIdx.x;
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    bf16x8_t a, b;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        a[q] = (__bf16)(0.001f * (float)((tid + q) & 15));
        b[q] = (__bf16)(0.001f * (float)((tid * 3 + q) & 15));
    }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[(long long)blockIdx.x * 512 + tid] = s;
    if (tid == 0) {
        uint64_t* st = stamps + (long long)blockIdx.x * 4;
        st[0] = c0;
        st[1] = c1;
        st[2] = r0;
        st[3] = r1;
    }
}

int default_blocks() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    return 8 * cus;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

moe_status moe_probe_copy(const void* src, void* dst, size_t bytes, int32_t blocks,
                          void* stream) {
    if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst) || bytes % 16 != 0 ||
        blocks < 0 || blocks > 65536)
        return MOE_ERR_INVALID_ARG;
    const char* s = (const char*)src;
    const char* d = (const char*)dst;
    if (s < d + bytes && d < s + bytes && bytes > 0) return MOE_ERR_INVALID_ARG;   // overlap
    if (bytes == 0) return MOE_OK;
    const int g = blocks ? blocks : default_blocks();
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)g), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)src, (u32x4*)dst, (long long)(bytes / 16));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_probe_read(const void* src, size_t bytes, float* sink, int32_t blocks,
                          void* stream) {
    if (src == nullptr || sink == nullptr || !aligned16(src) || !aligned16(sink) ||
        bytes % 16 != 0 || blocks < 0 || blocks > 65536)
        return MOE_ERR_INVALID_ARG;
    const int g = blocks ? blocks : default_blocks();
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)g), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)src, (long long)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_probe_mfma(int32_t blocks, int32_t iters, float* sink, uint64_t* stamps,
                          void* stream) {
    if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 24) || sink == nullptr ||
        stamps == nullptr || !aligned16(sink) || !aligned16(stamps))
        return MOE_ERR_INVALID_ARG;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(512), 0,
                       (hipStream_t)stream, iters, sink, stamps);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
