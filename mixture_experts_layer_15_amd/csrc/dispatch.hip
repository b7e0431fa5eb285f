// dispatch.hip -- capacity, token-order drops and the expert-grouped
// permutation on gfx950.
//
// Definition: the assignment (t, j) of token t to expert e = idx[t][j] is
// kept iff fewer than C earlier tokens (t' < t, at any rank j') chose e
// (overflow dropped in token order; capacity factor 1.25 of the TorchTitan
// 1K-GPU article, section 2.1).  Kept rows are grouped by expert, ascending
// token inside an expert.  Everything here is integer work, so the result is
// unique and bit-exact; no atomic decides a position.
//
// Four launches (two for small batches, see dispatch_small_kernel):
//   hist    tokens are cut into nblk <= 256 blocks; LDS histogram per block
//           -> blockcount[b][e]  (LDS atomics only count, order-free)
//   scan    one workgroup: per-expert exclusive scan over blocks ->
//           blockbase[b][e], count[e], kept[e] = min(count, C), offset[]
//   place   per block, 256 tokens at a time: rank of each assignment among
//           the earlier tokens of its wave (wave ballots over the expert id
//           bits), plus the counts of earlier waves and chunks -> row_of,
//           token_of_row
//   scatter one wave per token: the x row is read once and written to each
//           of its kept rows with 16-byte vector stores (HBM-bound)
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kInvalid = 256;   // expert code of an empty / out-of-range slot

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ blockcount,
                                                   long long T, int E, int k, int blk_tokens) {
    __shared__ int h[256];
    for (int e = threadIdx.x; e < 256; e += 256) h[e] = 0;
    __syncthreads();
    const long long tb = (long long)blockIdx.x * blk_tokens;
    const long long te = min(T, tb + blk_tokens);
    for (long long t = tb + threadIdx.x; t < te; t += 256)
        for (int j = 0; j < k; ++j) {
            const int e = idx[t * k + j];
            if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
        }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) blockcount[(long long)blockIdx.x * E + e] = h[e];
}

__global__ __launch_bounds__(256) void scan_kernel(const int32_t* __restrict__ blockcount,
                                                   int32_t* __restrict__ blockbase, int nblk,
                                                   int E, long long C,
                                                   int32_t* __restrict__ count,
                                                   int32_t* __restrict__ offset) {
    __shared__ int s_wave[4];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
#pragma unroll 8
        for (int b = 0; b < nblk; ++b) {
            const int v = blockcount[b * E + e];
            blockbase[b * E + e] = run;
            run += v;
        }
        count[e] = run;
    }
    const int kept = (e < E) ? (int)min((long long)run, C) : 0;
    // exclusive scan of kept over the 256 threads
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int v = kept;
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_wave[w] = v;
    __syncthreads();
    int add = 0;
    for (int i = 0; i < w; ++i) add += s_wave[i];
    const int incl = v + add;
    if (e < E) offset[e] = incl - kept;
    if (e == E - 1) offset[E] = incl;
}

// Places the assignments of the 256 tokens [tb, tb + 256): run[e] holds, on
// entry, the number of assignments to e by tokens before tb (in LDS); on exit
// it also counts this chunk's.  offset[] may live in LDS or global memory.
// All 256 threads call this together.
__device__ __forceinline__ void place_chunk(const int32_t* __restrict__ idx, int* run,
                                            int (*wcnt)[256], const int32_t* offset, int n_kept,
                                            long long C, long long T, int E, int k, long long tb,
                                            int32_t* __restrict__ row_of,
                                            int32_t* __restrict__ token_of_row) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i = tid; i < 4 * 256; i += 256) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const long long t = tb + tid;
    const bool valid = t < T;
    int code[8], rank[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        code[j] = kInvalid;
        rank[j] = 0;
        if (j < k && valid) {
            const int e = idx[t * k + j];
            if ((unsigned)e < (unsigned)E) code[j] = e;
        }
    }
    // rank among earlier lanes of this wave: lanes whose choices include my expert
#pragma unroll
    for (int jp = 0; jp < 8; ++jp) {
        if (jp < k) {
            unsigned long long bal[9];
#pragma unroll
            for (int b = 0; b < 9; ++b) bal[b] = __ballot((code[jp] >> b) & 1);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < k) {
                    unsigned long long m = ~0ull;
#pragma unroll
                    for (int b = 0; b < 9; ++b) m &= ((code[j] >> b) & 1) ? bal[b] : ~bal[b];
                    rank[j] += __popcll(m & lt);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < k && code[j] != kInvalid) atomicAdd(&wcnt[w][code[j]], 1);
    __syncthreads();
    if (valid) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= k) continue;
            const long long a = t * k + j;
            int row = -1;
            if (code[j] != kInvalid) {
                const int e = code[j];
                int pos = run[e] + rank[j];
                for (int i = 0; i < w; ++i) pos += wcnt[i][e];
                if (pos < C) {
                    row = offset[e] + pos;
                    token_of_row[row] = (int32_t)t;
                }
            }
            row_of[a] = row;
            // every slot index a >= rows kept is past the kept rows: mark it empty
            if (a >= n_kept) token_of_row[a] = -1;
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) run[e] += wcnt[0][e] + wcnt[1][e] + wcnt[2][e] + wcnt[3][e];
    __syncthreads();
}

__global__ __launch_bounds__(256) void place_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ blockbase,
    const int32_t* __restrict__ offset, long long C, long long T, int E, int k,
    int blk_tokens, int32_t* __restrict__ row_of, int32_t* __restrict__ token_of_row) {
    __shared__ int run[256];
    __shared__ int wcnt[4][256];
    for (int e = threadIdx.x; e < 256; e += 256)
        run[e] = (e < E) ? blockbase[(long long)blockIdx.x * E + e] : 0;
    const int n_kept = offset[E];
    const long long tb = (long long)blockIdx.x * blk_tokens;
    for (int c = 0; c < blk_tokens; c += 256)
        place_chunk(idx, run, wcnt, offset, n_kept, C, T, E, k, tb + c, row_of, token_of_row);
}

// Small batches (T*k <= kSmallAssign): histogram, capacity, offsets and
// placement in one launch, one 256-token chunk per workgroup.  Every
// workgroup counts all T*k assignments itself (a few KB, from L2) -- the
// totals and the counts before its chunk -- so no workgroup waits for
// another; workgroup 0 publishes count[] and offset[].
constexpr long long kSmallAssign = 16384;

__global__ __launch_bounds__(256) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, long long C, long long T, int E, int k,
    int32_t* __restrict__ count, int32_t* __restrict__ offset_out,
    int32_t* __restrict__ row_of, int32_t* __restrict__ token_of_row) {
    __shared__ int h_all[256], run[256];
    __shared__ int32_t s_off[257];
    __shared__ int wcnt[4][256];
    __shared__ int s_wave[4];
    const int tid = threadIdx.x;
    h_all[tid] = 0;
    run[tid] = 0;
    __syncthreads();
    const long long tb = (long long)blockIdx.x * 256;
    const long long n_assign = T * k, pre = tb * k;
    for (long long a = tid; a < n_assign; a += 256) {
        const int e = idx[a];
        if ((unsigned)e < (unsigned)E) {
            atomicAdd(&h_all[e], 1);
            if (a < pre) atomicAdd(&run[e], 1);
        }
    }
    __syncthreads();
    // kept = min(count, C); exclusive scan over the experts
    const int e = tid;
    const int kept = (e < E) ? (int)min((long long)h_all[e], C) : 0;
    const int lane = tid & 63, w = tid >> 6;
    int v = kept;
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_wave[w] = v;
    __syncthreads();
    int add = 0;
    for (int i = 0; i < w; ++i) add += s_wave[i];
    const int incl = v + add;
    if (e < E) s_off[e] = incl - kept;
    if (e == E - 1) s_off[E] = incl;
    if (blockIdx.x == 0 && e < E) {
        count[e] = h_all[e];
        offset_out[e] = incl - kept;
        if (e == E - 1) offset_out[E] = incl;
    }
    __syncthreads();
    place_chunk(idx, run, wcnt, s_off, s_off[E], C, T, E, k, tb, row_of, token_of_row);
}

// One wave per token: copy x[t] to each kept row (16-byte vectors).
__global__ __launch_bounds__(256) void scatter_kernel(const u32x4* __restrict__ x,
                                                      const int32_t* __restrict__ row_of,
                                                      u32x4* __restrict__ x_perm, long long T,
                                                      int nvec, int k) {
    const int lane = threadIdx.x & 63;
    const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int rows[8];
    bool any = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        rows[j] = (j < k) ? row_of[t * k + j] : -1;
        any |= rows[j] >= 0;
    }
    if (!any) return;
    const u32x4* src = x + t * nvec;
    for (int v0 = lane; v0 < nvec; v0 += 4 * 64) {
        u32x4 val[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (v0 + u * 64 < nvec) val[u] = src[v0 + u * 64];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (rows[j] < 0) continue;
            u32x4* dst = x_perm + (long long)rows[j] * nvec;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (v0 + u * 64 < nvec) dst[v0 + u * 64] = val[u];
        }
    }
}

}  // namespace

DispatchPlan plan_dispatch(long long T, int E, int k, long long C) {
    DispatchPlan p;
    p.T = T;
    p.E = E;
    p.k = k;
    p.C = C;
    const long long chunks = (T + 255) / 256;            // 256-token chunks
    const long long per_blk = (chunks + 255) / 256;      // chunks per block, so nblk <= 256
    p.blk_tokens = (int)(std::max<long long>(per_blk, 1) * 256);
    p.nblk = (int)((T + p.blk_tokens - 1) / p.blk_tokens);
    return p;
}

size_t dispatch_workspace_bytes(const DispatchPlan& p) {
    return (size_t)2 * (size_t)std::max(p.nblk, 1) * (size_t)p.E * sizeof(int32_t);
}

hipError_t launch_dispatch(const DispatchPlan& p, int dtype, const int32_t* idx, const void* x,
                           void* x_perm, int32_t* count, int32_t* offset, int32_t* row_of,
                           int32_t* token_of_row, void* workspace, int d, hipStream_t s,
                           bool scatter) {
    const int nvec = d * (dtype == 1 ? 2 : 4) / 16;
    if (p.T > 0 && p.T * p.k <= kSmallAssign) {
        hipLaunchKernelGGL(dispatch_small_kernel, dim3((unsigned)((p.T + 255) / 256)), dim3(256), 0,
                           s, idx, p.C, p.T, p.E, p.k, count, offset, row_of, token_of_row);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess || !scatter) return err;
        hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((p.T + 3) / 4)), dim3(256), 0, s,
                           (const u32x4*)x, row_of, (u32x4*)x_perm, p.T, nvec, p.k);
        return hipGetLastError();
    }
    int32_t* blockcount = (int32_t*)workspace;
    int32_t* blockbase = blockcount + (size_t)std::max(p.nblk, 1) * p.E;
    if (p.nblk > 0) {
        hipLaunchKernelGGL(hist_kernel, dim3(p.nblk), dim3(256), 0, s, idx, blockcount, p.T,
                           p.E, p.k, p.blk_tokens);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, blockcount, blockbase, p.nblk,
                       p.E, p.C, count, offset);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || p.nblk == 0) return err;
    hipLaunchKernelGGL(place_kernel, dim3(p.nblk), dim3(256), 0, s, idx, blockbase, offset, p.C,
                       p.T, p.E, p.k, p.blk_tokens, row_of, token_of_row);
    err = hipGetLastError();
    if (err != hipSuccess || !scatter) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((p.T + 3) / 4)), dim3(256), 0, s,
                       (const u32x4*)x, row_of, (u32x4*)x_perm, p.T, nvec, p.k);
    return hipGetLastError();
}

}  // namespace moe
