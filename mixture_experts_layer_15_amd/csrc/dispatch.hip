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
//           of its kept rows with 16-byte vector stores (HBM-bound; both
//           sides non-temporal: every byte is touched once, and streaming
//           past the caches measured 2-9% faster on the four bf16 layers)
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kInvalid = 256;   // expert code of an empty / out-of-range slot

// Sum of one value per thread over a 256-thread workgroup (every thread must
// call it; s4 holds 4 entries of LDS).
__device__ __forceinline__ long long block_sum256(long long v, long long* s4) {
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if ((threadIdx.x & 63) == 0) s4[threadIdx.x >> 6] = v;
    __syncthreads();
    const long long t = ((s4[0] + s4[1]) + s4[2]) + s4[3];
    __syncthreads();
    return t;
}

// Capacity of a dynamically routed batch (tokens taking varying numbers of
// experts): the factor cap_num / cap_den scales the realised mean load,
// C = ceil(cap_num A / (cap_den E)) for A assignments, at most T (a limit of T
// or more never drops anything); no limit (cap_den == 0) gives T.
__device__ __forceinline__ long long realised_capacity(long long A, int cap_num, int cap_den,
                                                       int E, long long T) {
    if (cap_den == 0) return T;
    const long long num = (long long)cap_num * A, den = (long long)cap_den * E;
    const long long c = (num + den - 1) / den;
    return c < T ? c : T;
}

// Slot (index into topk_idx / row_of) of choice j of walked token v, and the
// real token it belongs to.  Token order walks the real tokens (slot v*k + j);
// choice order walks the Tr*kr single choices v = j'*Tr + t (k = 1), whose
// slot is t*kr + j'.
template <bool CM>
__device__ __forceinline__ int slot_of(int v, int j, int k, int Tr, int kr) {
    return CM ? (v % Tr) * kr + v / Tr : v * k + j;
}
template <bool CM>
__device__ __forceinline__ int token_of(int v, int Tr) {
    return CM ? v % Tr : v;
}

template <bool CM>
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ blockcount,
                                                   long long T, int E, int k, int blk_tokens,
                                                   int Tr, int kr) {
    __shared__ int h[256];
    for (int e = threadIdx.x; e < 256; e += 256) h[e] = 0;
    __syncthreads();
    const long long tb = (long long)blockIdx.x * blk_tokens;
    const long long te = min(T, tb + blk_tokens);
    for (long long t = tb + threadIdx.x; t < te; t += 256)
        for (int j = 0; j < k; ++j) {
            const int e = idx[slot_of<CM>((int)t, j, k, Tr, kr)];
            if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
        }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) blockcount[(long long)blockIdx.x * E + e] = h[e];
}

__global__ __launch_bounds__(256) void scan_kernel(const int32_t* __restrict__ blockcount,
                                                   int32_t* __restrict__ blockbase, int nblk,
                                                   int E, long long C, int padded,
                                                   int32_t* __restrict__ count,
                                                   int32_t* __restrict__ offset, int dyn,
                                                   int cap_num, int cap_den, long long Tr) {
    __shared__ int s_wave[4];
    __shared__ long long s_red[4];
    __shared__ int s_part[256];
    // per-block prefix: with Ep = E rounded up to a power of two, thread
    // (part, ex) = (tid / Ep, tid % Ep) scans a contiguous range of the nblk
    // blocks of expert ex, so the 256 threads share the loads (a chain of nblk
    // dependent loads per expert was the cost of this kernel)
    int Ep = 1;
    while (Ep < E) Ep <<= 1;
    const int P = 256 / Ep, part = threadIdx.x / Ep, ex = threadIdx.x % Ep;
    const int b0 = (int)((long long)nblk * part / P), b1 = (int)((long long)nblk * (part + 1) / P);
    int psum = 0;
    if (ex < E) {
#pragma unroll 8
        for (int b = b0; b < b1; ++b) psum += blockcount[b * E + ex];
    }
    s_part[threadIdx.x] = psum;
    __syncthreads();
    if (ex < E) {
        int base = 0;
        for (int q = 0; q < part; ++q) base += s_part[q * Ep + ex];
#pragma unroll 8
        for (int b = b0; b < b1; ++b) {
            const int v = blockcount[b * E + ex];
            blockbase[b * E + ex] = base;
            base += v;
        }
    }
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int q = 0; q < P; ++q) run += s_part[q * Ep + e];
        count[e] = run;
    }
    if (dyn) C = realised_capacity(block_sum256(run, s_red), cap_num, cap_den, E, Tr);
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
    // padded layout: every expert owns C rows
    if (e < E) offset[e] = padded ? (int)(e * C) : incl - kept;
    if (e == E - 1) offset[E] = padded ? (int)(E * C) : incl;
}

// Places the assignments of the 256 tokens [tb, tb + 256): run[e] holds, on
// entry, the number of assignments to e by tokens before tb (in LDS); on exit
// it also counts this chunk's.  offset[] may live in LDS or global memory.
// All 256 threads call this together.
template <bool CM>
__device__ __forceinline__ void place_chunk(const int32_t* __restrict__ idx, int* run,
                                            int (*wcnt)[256], const int32_t* offset, int n_kept,
                                            long long C, long long T, int E, int k, long long tb,
                                            int Tr, int kr, int32_t* __restrict__ row_of,
                                            int32_t* __restrict__ token_of_row,
                                            int (*rows_out)[8] = nullptr) {
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
            const int e = idx[slot_of<CM>((int)t, j, k, Tr, kr)];
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
                    token_of_row[row] = token_of<CM>((int)t, Tr);
                }
            }
            row_of[slot_of<CM>((int)t, j, k, Tr, kr)] = row;
            if (rows_out != nullptr) rows_out[tid][j] = row;
            // every slot index a >= rows kept is past the kept rows: mark it empty
            if (a >= n_kept) token_of_row[a] = -1;
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) run[e] += wcnt[0][e] + wcnt[1][e] + wcnt[2][e] + wcnt[3][e];
    __syncthreads();
}

template <bool CM>
__global__ __launch_bounds__(256) void place_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ blockbase,
    const int32_t* __restrict__ offset, long long C, long long T, int E, int k,
    int blk_tokens, int Tr, int kr, int32_t* __restrict__ row_of,
    int32_t* __restrict__ token_of_row, const int32_t* __restrict__ count, int dyn,
    int cap_num, int cap_den) {
    __shared__ int run[256];
    __shared__ int wcnt[4][256];
    __shared__ long long s_red[4];
    if (dyn) {
        const long long c = threadIdx.x < E ? count[threadIdx.x] : 0;
        C = realised_capacity(block_sum256(c, s_red), cap_num, cap_den, E, Tr);
    }
    for (int e = threadIdx.x; e < 256; e += 256)
        run[e] = (e < E) ? blockbase[(long long)blockIdx.x * E + e] : 0;
    const int n_kept = offset[E];
    const long long tb = (long long)blockIdx.x * blk_tokens;
    for (int c = 0; c < blk_tokens; c += 256)
        place_chunk<CM>(idx, run, wcnt, offset, n_kept, C, T, E, k, tb + c, Tr, kr, row_of,
                        token_of_row);
}

// Small batches (T*k <= kSmallAssign): histogram, capacity, offsets and
// placement in one launch, one 256-token chunk per workgroup.  Every
// workgroup counts all T*k assignments itself (a few KB, from L2) -- the
// totals and the counts before its chunk -- so no workgroup waits for
// another; workgroup 0 publishes count[] and offset[].
constexpr long long kSmallAssign = 16384;

template <bool CM>
__global__ __launch_bounds__(256) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, long long C, long long T, int E, int k, int Tr, int kr,
    int padded, int32_t* __restrict__ count, int32_t* __restrict__ offset_out,
    int32_t* __restrict__ row_of, int32_t* __restrict__ token_of_row, int dyn, int cap_num,
    int cap_den) {
    __shared__ int h_all[256], run[256];
    __shared__ int32_t s_off[257];
    __shared__ int wcnt[4][256];
    __shared__ int s_wave[4];
    __shared__ long long s_red[4];
    const int tid = threadIdx.x;
    h_all[tid] = 0;
    run[tid] = 0;
    __syncthreads();
    const long long tb = (long long)blockIdx.x * 256;
    const long long n_assign = T * k, pre = tb * k;
    // eight independent loads in flight per thread before their counts: one
    // L2 round trip per 2048 assignments instead of one per 256
    constexpr int U = 8;
    for (long long a0 = tid; a0 < n_assign; a0 += 256 * U) {
        int ev[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long a = a0 + 256LL * u;
            ev[u] = a < n_assign ? idx[CM ? slot_of<CM>((int)a, 0, 1, Tr, kr) : a] : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = ev[u];
            if ((unsigned)e < (unsigned)E) {
                atomicAdd(&h_all[e], 1);
                if (a0 + 256LL * u < pre) atomicAdd(&run[e], 1);
            }
        }
    }
    __syncthreads();
    if (dyn) C = realised_capacity(block_sum256(tid < E ? h_all[tid] : 0, s_red), cap_num, cap_den,
                                   E, Tr);
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
    const int off_e = padded ? (int)(e * C) : incl - kept;
    const int off_end = padded ? (int)(E * C) : incl;
    if (e < E) s_off[e] = off_e;
    if (e == E - 1) s_off[E] = off_end;
    if (blockIdx.x == 0 && e < E) {
        count[e] = h_all[e];
        offset_out[e] = off_e;
        if (e == E - 1) offset_out[E] = off_end;
    }
    __syncthreads();
    place_chunk<CM>(idx, run, wcnt, s_off, s_off[E], C, T, E, k, tb, Tr, kr, row_of,
                    token_of_row);
}

// Small batches with the scatter (compact layout): the one-launch index work
// of dispatch_small_kernel and the copy of x rows into x_perm in one launch.
// Each workgroup takes tpb (<= 256) consecutive walked tokens -- few enough
// that the grid spreads the copy over the CUs -- counts all assignments
// itself, places its tokens, keeps their rows in LDS and copies their x rows
// (one wave per walked token, 16-byte non-temporal loads and stores).
template <bool CM>
__global__ __launch_bounds__(256) void dispatch_small_scatter_kernel(
    const int32_t* __restrict__ idx, long long C, long long T, int E, int k, int Tr, int kr,
    int32_t* __restrict__ count, int32_t* __restrict__ offset_out,
    int32_t* __restrict__ row_of, int32_t* __restrict__ token_of_row, int dyn, int cap_num,
    int cap_den, const u32x4* __restrict__ x, u32x4* __restrict__ x_perm, int nvec, int tpb) {
    __shared__ int h_all[256], run[256];
    __shared__ int32_t s_off[257];
    __shared__ int wcnt[4][256];
    __shared__ int s_wave[4];
    __shared__ long long s_red[4];
    __shared__ int s_rows[256][8];
    const int tid = threadIdx.x;
    h_all[tid] = 0;
    run[tid] = 0;
    __syncthreads();
    const long long tb = (long long)blockIdx.x * tpb;
    const long long n_assign = T * k, pre = tb * k;
    constexpr int U = 8;
    for (long long a0 = tid; a0 < n_assign; a0 += 256 * U) {
        int ev[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long a = a0 + 256LL * u;
            ev[u] = a < n_assign ? idx[CM ? slot_of<CM>((int)a, 0, 1, Tr, kr) : a] : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = ev[u];
            if ((unsigned)e < (unsigned)E) {
                atomicAdd(&h_all[e], 1);
                if (a0 + 256LL * u < pre) atomicAdd(&run[e], 1);
            }
        }
    }
    __syncthreads();
    if (dyn) C = realised_capacity(block_sum256(tid < E ? h_all[tid] : 0, s_red), cap_num, cap_den,
                                   E, Tr);
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
    const long long te = min(T, tb + tpb);   // walked tokens of this block: [tb, te)
    place_chunk<CM>(idx, run, wcnt, s_off, s_off[E], C, te, E, k, tb, Tr, kr, row_of,
                    token_of_row, s_rows);
    // place_chunk ends with a barrier: s_rows holds every token's rows
    for (long long t = tb + w; t < te; t += 4) {
        const int tl = (int)(t - tb);
        const u32x4* src = x + (long long)token_of<CM>((int)t, Tr) * nvec;
        for (int v0 = lane; v0 < nvec; v0 += 4 * 64) {
            u32x4 val[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (v0 + u * 64 < nvec) val[u] = __builtin_nontemporal_load(src + v0 + u * 64);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j >= k) break;
                const int r = s_rows[tl][j];
                if (r < 0) continue;
                u32x4* dst = x_perm + (long long)r * nvec;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (v0 + u * 64 < nvec) __builtin_nontemporal_store(val[u], dst + v0 + u * 64);
            }
        }
    }
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
            if (v0 + u * 64 < nvec) val[u] = __builtin_nontemporal_load(src + v0 + u * 64);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (rows[j] < 0) continue;
            u32x4* dst = x_perm + (long long)rows[j] * nvec;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (v0 + u * 64 < nvec) __builtin_nontemporal_store(val[u], dst + v0 + u * 64);
        }
    }
}

// Padded layout: the rows of expert e past its kept ones (pos >= min(count_e,
// C) in its C-row segment) are empty: token_of_row -1 and, when x_perm is
// given, a zero row.  One wave per row.
__global__ __launch_bounds__(256) void pad_rows_kernel(const int32_t* __restrict__ count,
                                                       long long C, int E,
                                                       int32_t* __restrict__ token_of_row,
                                                       u32x4* __restrict__ x_perm, int nvec) {
    const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= (long long)E * C) return;
    const int e = (int)(r / C);
    const long long pos = r - (long long)e * C;
    if (pos < min((long long)count[e], C)) return;
    const int lane = threadIdx.x & 63;
    if (lane == 0) token_of_row[r] = -1;
    if (x_perm != nullptr)
        for (int v = lane; v < nvec; v += 64) x_perm[r * nvec + v] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

DispatchPlan plan_dispatch(long long T, int E, int k, long long C, int policy, int layout,
                           bool dyn, int cap_num, int cap_den) {
    DispatchPlan p;
    p.dyn = dyn;
    p.cap_num = cap_num;
    p.cap_den = cap_den;
    p.padded = layout == 1;
    p.Tr = T;
    p.kr = k;
    p.choice_order = policy == 1 && k > 1;   // with one choice the orders coincide
    p.T = p.choice_order ? T * k : T;
    p.k = p.choice_order ? 1 : k;
    T = p.T;
    p.E = E;
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

namespace {

template <bool CM>
hipError_t dispatch_kernels(const DispatchPlan& p, const int32_t* idx, int32_t* count,
                            int32_t* offset, int32_t* row_of, int32_t* token_of_row,
                            void* workspace, hipStream_t s) {
    const int Tr = (int)p.Tr, kr = p.kr;
    if (p.T > 0 && p.T * p.k <= kSmallAssign) {
        hipLaunchKernelGGL(dispatch_small_kernel<CM>, dim3((unsigned)((p.T + 255) / 256)),
                           dim3(256), 0, s, idx, p.C, p.T, p.E, p.k, Tr, kr, p.padded ? 1 : 0,
                           count, offset, row_of, token_of_row, p.dyn ? 1 : 0, p.cap_num,
                           p.cap_den);
        return hipGetLastError();
    }
    int32_t* blockcount = (int32_t*)workspace;
    int32_t* blockbase = blockcount + (size_t)std::max(p.nblk, 1) * p.E;
    if (p.nblk > 0) {
        hipLaunchKernelGGL(hist_kernel<CM>, dim3(p.nblk), dim3(256), 0, s, idx, blockcount, p.T,
                           p.E, p.k, p.blk_tokens, Tr, kr);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, blockcount, blockbase, p.nblk,
                       p.E, p.C, p.padded ? 1 : 0, count, offset, p.dyn ? 1 : 0, p.cap_num,
                       p.cap_den, p.Tr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || p.nblk == 0) return err;
    hipLaunchKernelGGL(place_kernel<CM>, dim3(p.nblk), dim3(256), 0, s, idx, blockbase, offset,
                       p.C, p.T, p.E, p.k, p.blk_tokens, Tr, kr, row_of, token_of_row, count,
                       p.dyn ? 1 : 0, p.cap_num, p.cap_den);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const DispatchPlan& p, int dtype, const int32_t* idx, const void* x,
                           void* x_perm, int32_t* count, int32_t* offset, int32_t* row_of,
                           int32_t* token_of_row, void* workspace, int d, hipStream_t s,
                           bool scatter) {
    const int nvec = d * (dtype == 1 ? 2 : 4) / 16;
    if (scatter && !p.padded && p.T > 0 && p.T * p.k <= kSmallAssign) {
        // tokens per workgroup: the grid covers about 256 CUs (4 .. 256 tokens each)
        int tpb = 4;
        while (tpb < 256 && (p.T + tpb - 1) / tpb > 256) tpb *= 2;
        const unsigned grid = (unsigned)((p.T + tpb - 1) / tpb);
        if (p.choice_order)
            hipLaunchKernelGGL(dispatch_small_scatter_kernel<true>, dim3(grid), dim3(256), 0, s, idx,
                               p.C, p.T, p.E, p.k, (int)p.Tr, p.kr, count, offset, row_of,
                               token_of_row, p.dyn ? 1 : 0, p.cap_num, p.cap_den, (const u32x4*)x,
                               (u32x4*)x_perm, nvec, tpb);
        else
            hipLaunchKernelGGL(dispatch_small_scatter_kernel<false>, dim3(grid), dim3(256), 0, s,
                               idx, p.C, p.T, p.E, p.k, (int)p.Tr, p.kr, count, offset, row_of,
                               token_of_row, p.dyn ? 1 : 0, p.cap_num, p.cap_den, (const u32x4*)x,
                               (u32x4*)x_perm, nvec, tpb);
        return hipGetLastError();
    }
    hipError_t err = p.choice_order
        ? dispatch_kernels<true>(p, idx, count, offset, row_of, token_of_row, workspace, s)
        : dispatch_kernels<false>(p, idx, count, offset, row_of, token_of_row, workspace, s);
    if (err != hipSuccess) return err;
    const long long padded_rows = p.padded ? p.C * p.E : 0;
    if (padded_rows > 0) {
        hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)((padded_rows + 3) / 4)), dim3(256), 0,
                           s, count, p.C, p.E, token_of_row,
                           scatter ? (u32x4*)x_perm : (u32x4*)nullptr, nvec);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (!scatter || p.Tr == 0) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((p.Tr + 3) / 4)), dim3(256), 0, s,
                       (const u32x4*)x, row_of, (u32x4*)x_perm, p.Tr, nvec, p.kr);
    return hipGetLastError();
}

hipError_t launch_zero_empty_rows(const int32_t* count, long long C, int E, int32_t* token_of_row,
                                  void* buf, int row_bytes, hipStream_t s) {
    const long long padded_rows = (long long)E * C;
    if (padded_rows == 0) return hipSuccess;
    if (row_bytes % 16 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)((padded_rows + 3) / 4)), dim3(256), 0, s,
                       count, C, E, token_of_row, (u32x4*)buf, row_bytes / 16);
    return hipGetLastError();
}

hipError_t launch_scatter_rows(const void* x, const int32_t* row_of, void* x_perm, long long T,
                               int row_bytes, int k, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (row_bytes % 16 != 0 || k > 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s,
                       (const u32x4*)x, row_of, (u32x4*)x_perm, T, row_bytes / 16, k);
    return hipGetLastError();
}

// Expert-load telemetry: one workgroup, fp64.  stats as documented in moe.h.
__global__ __launch_bounds__(256) void load_stats_kernel(const int32_t* __restrict__ count,
                                                         int E, long long C,
                                                         double* __restrict__ stats, int dyn,
                                                         int cap_num, int cap_den, long long T) {
    __shared__ long long s_red[4];
    if (dyn)   // capacity from the realised assignments (uniform branch)
        C = realised_capacity(block_sum256(threadIdx.x < E ? count[threadIdx.x] : 0, s_red),
                              cap_num, cap_den, E, T);
    __shared__ double s_sum[4], s_max[4], s_min[4], s_drop[4], s_empty[4], s_dev[4], s_ss[4];
    const int e = threadIdx.x, lane = e & 63, w = e >> 6;
    const bool ok = e < E;
    const double c = ok ? (double)count[e] : 0.0;
    auto wave_sum = [](double v) {
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
        return v;
    };
    auto wave_max = [](double v) {
        for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
        return v;
    };
    const double sum = wave_sum(c);
    const double mx = wave_max(ok ? c : -1.0);
    const double mn = -wave_max(ok ? -c : -1e300);
    const double drop = wave_sum(ok && c > (double)C ? c - (double)C : 0.0);
    const double empty = wave_sum(ok && c == 0.0 ? 1.0 : 0.0);
    if (lane == 0) { s_sum[w] = sum; s_max[w] = mx; s_min[w] = mn; s_drop[w] = drop; s_empty[w] = empty; }
    __syncthreads();
    // fixed order over the four waves: the same sums on every run
    const double tot = ((s_sum[0] + s_sum[1]) + s_sum[2]) + s_sum[3];
    const double m = tot / (double)E;
    const double diff = ok ? c - m : 0.0;
    const double dev = wave_max(diff < 0 ? -diff : diff);
    const double ss = wave_sum(diff * diff);
    if (lane == 0) { s_dev[w] = dev; s_ss[w] = ss; }
    __syncthreads();
    if (e == 0) {
        double gmax = s_max[0], gmin = s_min[0], gdev = s_dev[0];
        for (int i = 1; i < 4; ++i) {
            gmax = fmax(gmax, s_max[i]);
            gmin = fmin(gmin, s_min[i]);
            gdev = fmax(gdev, s_dev[i]);
        }
        const double gss = ((s_ss[0] + s_ss[1]) + s_ss[2]) + s_ss[3];
        stats[0] = m;
        stats[1] = gmax;
        stats[2] = gmin;
        stats[3] = m > 0 ? gmax / m : 0.0;
        stats[4] = m > 0 ? gdev / m : 0.0;
        stats[5] = m > 0 ? sqrt(gss / (double)E) / m : 0.0;
        stats[6] = ((s_drop[0] + s_drop[1]) + s_drop[2]) + s_drop[3];
        stats[7] = ((s_empty[0] + s_empty[1]) + s_empty[2]) + s_empty[3];
    }
}

// Load-balance PID controller, one workgroup, one thread per expert, fp64
// (update rule as documented at moe_pid_update).  No contraction into fused
// multiply-adds: every operation rounds once, in the documented order.
__global__ __launch_bounds__(256) void pid_update_kernel(const int32_t* __restrict__ count, int E,
                                                         double kp, double ki, double kd,
                                                         double scale, double* __restrict__ state,
                                                         float* __restrict__ bias) {
#pragma clang fp contract(off)
    __shared__ long long s_red[4];
    const int e = threadIdx.x;
    const long long tot = block_sum256(e < E ? count[e] : 0, s_red);   // exact
    if (e >= E) return;
    const double mean = (double)tot / (double)E;
    const double err = mean > 0 ? (mean - (double)count[e]) / mean : 0.0;
    const double integral = state[e] + err;
    const double deriv = err - state[E + e];
    const double p_term = kp * err, i_term = ki * integral, d_term = kd * deriv;
    bias[e] = (float)(scale * ((p_term + i_term) + d_term));
    state[e] = integral;
    state[E + e] = err;
}

hipError_t launch_pid_update(const int32_t* count, int E, double kp, double ki, double kd,
                             double scale, double* state, float* bias, hipStream_t s) {
    hipLaunchKernelGGL(pid_update_kernel, dim3(1), dim3(256), 0, s, count, E, kp, ki, kd, scale,
                       state, bias);
    return hipGetLastError();
}

hipError_t launch_load_stats(const int32_t* count, int E, long long C, double* stats,
                             hipStream_t s, bool dyn, int cap_num, int cap_den, long long T) {
    hipLaunchKernelGGL(load_stats_kernel, dim3(1), dim3(256), 0, s, count, E, C, stats,
                       dyn ? 1 : 0, cap_num, cap_den, T);
    return hipGetLastError();
}

}  // namespace moe
