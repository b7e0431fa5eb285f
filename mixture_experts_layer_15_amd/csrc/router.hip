// router.hip -- linear router, temperature softmax and top-k on gfx950.
//
// logits l = x W_r + b (fp32 accumulation); p = softmax(l / tau) over all E
// experts; the k largest logits are chosen (lower expert index first on equal
// logits) and their gates are p, or p renormalised over the chosen k.
// Sources: linear router -- "AMD MI300X平台上的MoE模型训练实践" section 3.2;
// router temperature -- "AMD GPU深度学习优化与ZAYA1大模型实践" section 7 and the
// TorchTitan 1K-GPU article section 2.1; top-1 / top-2 -- ZAYA1 page section 2,
// TorchTitan article section 2.1.
//
// bf16 path: one fused kernel.  A workgroup of 4 waves takes 64*MT tokens;
// each wave multiplies 16*MT token rows by the whole (16*NT-padded) router
// matrix with v_mfma_f32_16x16x32_bf16.  Token rows stream straight from HBM
// into A fragments (each row is read once); the router matrix is staged
// through LDS in its natural [d][E] layout in K-steps of 64 and read with the
// transposing LDS read.  The MFMA result layout already puts the E logits of
// one token in one 16-lane group (lane q holds experts q, q+16, ...), so the
// softmax and top-k run on the accumulators with 16-lane shuffles: no logits
// round trip through memory.
//
// The ranking uses the fp32 logits themselves (tau > 0 keeps the order;
// ranking rounded l/tau or p could merge distinct logits).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kNone = 0x7fffffff;

// One token per 16-lane group; lane q owns experts q + 16 m.  All 16 lanes
// must call this together (shuffles); only `write` lanes store.
template <int NT>
__device__ __forceinline__ void topk_group16(const float (&v)[NT], int q, int E,
                                             const TopkParams& tp, bool write,
                                             int32_t* __restrict__ idx_row,
                                             float* __restrict__ gate_row) {
    const int k = tp.k;
    const float tau = tp.tau;
    const int renorm = tp.renorm;
    unsigned taken = 0;
    float cv[8];
    int ce[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        cv[j] = 0.f;
        ce[j] = 0;
        if (j < k) {
            float bv = 0.f;
            int be = kNone;
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                const int e = m * 16 + q;
                const bool ok = e < E && !((taken >> m) & 1u);
                // experts visited in ascending order: strict '>' keeps the lower index on ties
                if (ok && (be == kNone || v[m] > bv)) { bv = v[m]; be = e; }
            }
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 16);
                const int oe = __shfl_xor(be, o, 16);
                const bool better = oe != kNone &&
                    (be == kNone || ov > bv || (ov == bv && oe < be));
                if (better) { bv = ov; be = oe; }
            }
            cv[j] = bv;
            ce[j] = be;
            if ((be & 15) == q) taken |= 1u << (be >> 4);
        }
    }
    // softmax denominator over all E experts (max = the top-1 logit)
    const float mx = cv[0];
    float z = 0.f;
#pragma unroll
    for (int m = 0; m < NT; ++m)
        if (m * 16 + q < E) z += expf((v[m] - mx) / tau);
    // butterfly sum: every lane ends with the same value (pairs add x+y / y+x)
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) z += __shfl_xor(z, o, 16);
    // dynamic count (theta > 0): the fewest of the k ranked experts, at least
    // k_min, whose softmax mass reaches theta.  This integer decision is taken
    // in fp64 from the fp32 logits (exp and sums in double), so that it agrees
    // with an fp64 evaluation of the same definition except when the mass
    // lies within a few fp64 rounding steps of theta.
    int kt = k;
    if (tp.theta > 0.f) {
        const double dmx = (double)mx, dtau = (double)tau;
        double zd = 0.0;
#pragma unroll
        for (int m = 0; m < NT; ++m)
            if (m * 16 + q < E) zd += exp(((double)v[m] - dmx) / dtau);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) zd += __shfl_xor(zd, o, 16);
        double mass = 0.0;
        bool done = false;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < k && !done) {
                mass += exp(((double)cv[j] - dmx) / dtau) / zd;
                if (j + 1 >= tp.k_min && mass >= (double)tp.theta) { kt = j + 1; done = true; }
            }
        }
    }
    float ev[8];
    float sk = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ev[j] = 0.f;
        if (j < kt) { ev[j] = expf((cv[j] - mx) / tau); sk += ev[j]; }
    }
    if (write && q == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) {
                // slots past the token's count hold no assignment
                idx_row[j] = j < kt ? ce[j] : -1;
                gate_row[j] = j < kt ? (renorm ? ev[j] / sk : ev[j] / z) : 0.f;
            }
    }
}

constexpr int RBK = 64;   // router K-step

template <int NT, int MT>
__global__ __launch_bounds__(256) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ gate, long long T, int d, int E, TopkParams tp) {
    constexpr int EP = 16 * NT;
    constexpr int W_LD = EP + 8;   // LDS row stride (elements)
    __shared__ __attribute__((aligned(16))) uint16_t ws[RBK * W_LD];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c16 = lane & 15, g4 = lane >> 4;
    const long long t0 = (long long)blockIdx.x * (64 * MT) + wave * 16 * MT;

    const uint16_t* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        long long t = t0 + mt * 16 + c16;
        if (t > T - 1) t = T - 1;
        xrow[mt] = x + t * d + g4 * 8;
    }
    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const bool vec_ok = (E % 8) == 0;
    for (int k0 = 0; k0 < d; k0 += RBK) {
        bf16x8 a[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                a[mt][ks] = *(const bf16x8*)(xrow[mt] + k0 + ks * 32);
        __syncthreads();
        // stage W_r[k0 .. k0+64)[0 .. EP) (zero past E)
        for (int v = threadIdx.x; v < RBK * (EP / 8); v += 256) {
            const int kr = v / (EP / 8), c8 = (v % (EP / 8)) * 8;
            const uint16_t* src = wr + (long long)(k0 + kr) * E + c8;
            u32x4 val;
            if (vec_ok) {
                val = (c8 < E) ? *(const u32x4*)src : u32x4{0u, 0u, 0u, 0u};
            } else {
                uint32_t w[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t lo = (c8 + 2 * p < E) ? src[2 * p] : 0u;
                    const uint32_t hi = (c8 + 2 * p + 1 < E) ? src[2 * p + 1] : 0u;
                    w[p] = lo | (hi << 16);
                }
                val = u32x4{w[0], w[1], w[2], w[3]};
            }
            *(u32x4*)(&ws[kr * W_LD + c8]) = val;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int row = ks * 32 + g4 * 8 + (c16 >> 2);
                const int col = nt * 16 + (c16 & 3) * 4;
                s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(&ws[row * W_LD + col]));
                s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(&ws[(row + 4) * W_LD + col]));
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][ks], b, acc[mt][nt], 0, 0, 0);
            }
        }
    }

    // lane holds token rows 4*g4 + r (r = 0..3) of each 16-row tile, expert nt*16 + c16
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const long long t = t0 + mt * 16 + g4 * 4 + r;
            float v[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int e = nt * 16 + c16;
                float l = acc[mt][nt][r];
                if (bias != nullptr && e < E) l += bias[e];
                v[nt] = l;
                if (t < T && e < E) logits[t * E + e] = l;
            }
            const bool ok = t < T;
            const long long tt = ok ? t : 0;
            topk_group16<NT>(v, c16, E, tp, ok, idx + tt * tp.k, gate + tt * tp.k);
        }
    }
}

// K-split variant for E <= 128 (E % 8 == 0): a workgroup of 4 waves takes 16*MT
// tokens and wave w accumulates the K-steps w, w+4, w+8, ... of all of them,
// so a small batch still spreads over every CU and each wave keeps D K-steps
// of token rows in flight.  Each wave stages its own K-step of W_r in LDS.
// The four partial logits are summed in LDS in wave order (deterministic);
// wave w then owns row r = w of every 4-row accumulator group for the top-k.
template <int NT, int MT, int D>
__global__ __launch_bounds__(256) void router_ks_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ gate, long long T, int d, int E, TopkParams tp) {
    constexpr int EP = 16 * NT;
    constexpr int W_LD = EP + 8;               // LDS row stride (elements)
    constexpr int WCH = RBK * EP / 8 / 64;     // 16-byte W_r chunks per lane per K-step
    __shared__ __attribute__((aligned(16))) uint16_t ws[4][RBK * W_LD];
    __shared__ float part[4][MT][NT][4][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15, g4 = lane >> 4;
    const long long t0 = (long long)blockIdx.x * (16 * MT);
    const int nk = d / RBK;
    const int nw = nk > wave ? (nk - wave + 3) / 4 : 0;   // K-steps of this wave

    const uint16_t* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        long long t = t0 + mt * 16 + c16;
        if (t > T - 1) t = T - 1;
        xrow[mt] = x + t * d + g4 * 8;
    }
    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // register ring of D K-steps: token-row fragments and this lane's W_r chunks
    bf16x8 ra[D][MT][2];
    u32x4 rw[D][WCH];
    auto issue = [&](int i, bf16x8 (&a)[MT][2], u32x4 (&wv)[WCH]) {
        const int k0 = (wave + 4 * i) * RBK;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) a[mt][ks] = *(const bf16x8*)(xrow[mt] + k0 + ks * 32);
#pragma unroll
        for (int c = 0; c < WCH; ++c) {
            const int v = lane + 64 * c;
            const int kr = v / (EP / 8), c8 = (v % (EP / 8)) * 8;
            wv[c] = (c8 < E) ? *(const u32x4*)(wr + (long long)(k0 + kr) * E + c8)
                             : u32x4{0u, 0u, 0u, 0u};
        }
    };
    uint16_t* wsw = ws[wave];
    auto step = [&](const bf16x8 (&a)[MT][2], const u32x4 (&wv)[WCH]) {
#pragma unroll
        for (int c = 0; c < WCH; ++c) {
            const int v = lane + 64 * c;
            const int kr = v / (EP / 8), c8 = (v % (EP / 8)) * 8;
            *(u32x4*)(&wsw[kr * W_LD + c8]) = wv[c];
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int row = ks * 32 + g4 * 8 + (c16 >> 2);
                const int col = nt * 16 + (c16 & 3) * 4;
                s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(&wsw[row * W_LD + col]));
                s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(&wsw[(row + 4) * W_LD + col]));
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][ks], b, acc[mt][nt], 0, 0, 0);
            }
        }
    };
#pragma unroll
    for (int j = 0; j + 1 < D; ++j)
        if (j < nw) issue(j, ra[j], rw[j]);
    for (int i0 = 0; i0 < nw; i0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int i = i0 + j;
            if (i >= nw) break;
            if (i + D - 1 < nw) issue(i + D - 1, ra[(j + D - 1) % D], rw[(j + D - 1) % D]);
            step(ra[j], rw[j]);
        }
    }

    // sum the four partials in wave order; wave w finishes accumulator row w
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[wave][mt][nt][r][lane] = acc[mt][nt][r];
    __syncthreads();
    const int r = wave;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const long long t = t0 + mt * 16 + g4 * 4 + r;
        float v[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int e = nt * 16 + c16;
            float l = part[0][mt][nt][r][lane];
            l += part[1][mt][nt][r][lane];
            l += part[2][mt][nt][r][lane];
            l += part[3][mt][nt][r][lane];
            if (bias != nullptr && e < E) l += bias[e];
            v[nt] = l;
            if (t < T && e < E) logits[t * E + e] = l;
        }
        const bool ok = t < T;
        const long long tt = ok ? t : 0;
        topk_group16<NT>(v, c16, E, tp, ok, idx + tt * tp.k, gate + tt * tp.k);
    }
}

// fp32 path: plain fp32 FMA dot products (64 tokens per workgroup) into an
// LDS logits tile, then the same 16-lane top-k.
template <int NT>
__global__ __launch_bounds__(256) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ gate,
    long long T, int d, int E, TopkParams tp) {
    constexpr int EP = 16 * NT;
    __shared__ float lg[64][EP + 1];
    const long long t0 = (long long)blockIdx.x * 64;
    for (int p = threadIdx.x; p < 64 * EP; p += 256) {
        const int tl = p / EP, e = p % EP;
        const long long t = t0 + tl;
        float acc = 0.f;
        if (t < T && e < E) {
            const float* xr = x + t * d;
            for (int i = 0; i < d; ++i) acc = fmaf(xr[i], wr[(long long)i * E + e], acc);
            if (bias != nullptr) acc += bias[e];
            logits[t * E + e] = acc;
        }
        lg[tl][e] = acc;
    }
    __syncthreads();
    const int q = threadIdx.x & 15, grp = threadIdx.x >> 4;   // 16 groups
    for (int tl = grp; tl < 64; tl += 16) {
        const long long t = t0 + tl;
        float v[NT];
#pragma unroll
        for (int m = 0; m < NT; ++m) v[m] = lg[tl][m * 16 + q];
        const bool ok = t < T;
        const long long tt = ok ? t : 0;
        topk_group16<NT>(v, q, E, tp, ok, idx + tt * tp.k, gate + tt * tp.k);
    }
}

// Top-k and gates from fp32 logits in memory; 16 tokens per workgroup.
template <int NT>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ gate, long long T,
                                                   int E, TopkParams tp) {
    const int q = threadIdx.x & 15, grp = threadIdx.x >> 4;
    const long long t = (long long)blockIdx.x * 16 + grp;
    const bool ok = t < T;
    const long long tt = ok ? t : 0;
    float v[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
        const int e = m * 16 + q;
        v[m] = (e < E) ? logits[tt * E + e] : 0.f;
    }
    topk_group16<NT>(v, q, E, tp, ok, idx + tt * tp.k, gate + tt * tp.k);
}

// K-split router launch: 16*MT tokens per workgroup, MT grown only while at
// least 512 workgroups remain; D K-steps in flight per wave.
template <int NT>
hipError_t route_ks(const uint16_t* x, const uint16_t* w, const float* bias, float* logits,
                    int32_t* idx, float* gate, long long T, int d, int E, TopkParams tp,
                    hipStream_t s) {
    // E > 64: W_r chunks take 64 registers per K-step in flight, so two steps
    // in flight.  At most two token tiles per wave: four (fewer re-reads of
    // W_r per token) need more than 256 registers, which leaves one wave per
    // SIMD, and measured slower on the skewed (E = 64: 69.5 against 55.7 us)
    // and long-sequence (E = 8: 165 against 151 us) layers.
    constexpr int D2 = NT <= 4 ? 3 : 2, D1 = NT <= 4 ? 4 : 2;
    if (T >= 16LL * 2 * 512)
        hipLaunchKernelGGL((router_ks_kernel<NT, 2, D2>), dim3((unsigned)((T + 31) / 32)), dim3(256),
                           0, s, x, w, bias, logits, idx, gate, T, d, E, tp);
    else
        hipLaunchKernelGGL((router_ks_kernel<NT, 1, D1>), dim3((unsigned)((T + 15) / 16)), dim3(256),
                           0, s, x, w, bias, logits, idx, gate, T, d, E, tp);
    return hipGetLastError();
}

template <int NT>
hipError_t route_nt(int dtype, const void* x, const void* w, const float* bias, float* logits,
                    int32_t* idx, float* gate, long long T, int d, int E, TopkParams tp,
                    hipStream_t s) {
    if (dtype == 1) {
        if constexpr (NT <= 8) {
            if (E % 8 == 0)
                return route_ks<NT>((const uint16_t*)x, (const uint16_t*)w, bias, logits, idx,
                                    gate, T, d, E, tp, s);
        }
        if (T >= 64LL * 1024 && NT <= 8) {
            // two 16-row tiles per wave once there are enough tokens to fill the GPU
            const long long grid = (T + 127) / 128;
            hipLaunchKernelGGL((router_bf16_kernel<NT, 2>), dim3((unsigned)grid), dim3(256), 0, s,
                               (const uint16_t*)x, (const uint16_t*)w, bias, logits, idx, gate,
                               T, d, E, tp);
        } else {
            const long long grid = (T + 63) / 64;
            hipLaunchKernelGGL((router_bf16_kernel<NT, 1>), dim3((unsigned)grid), dim3(256), 0, s,
                               (const uint16_t*)x, (const uint16_t*)w, bias, logits, idx, gate,
                               T, d, E, tp);
        }
    } else {
        const long long grid = (T + 63) / 64;
        hipLaunchKernelGGL(router_f32_kernel<NT>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const float*)x, (const float*)w, bias, logits, idx, gate, T, d, E,
                           tp);
    }
    return hipGetLastError();
}

int nt_for(int E) {
    const int nt = (E + 15) / 16;
    return nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : nt <= 8 ? 8 : 16;
}

}  // namespace

hipError_t launch_route(int dtype, const void* x, const void* w_router, const float* bias,
                        float* logits, int32_t* idx, float* gate, long long T, int d, int E,
                        TopkParams tp, hipStream_t s) {
    if (T == 0) return hipSuccess;
    switch (nt_for(E)) {
        case 1: return route_nt<1>(dtype, x, w_router, bias, logits, idx, gate, T, d, E, tp, s);
        case 2: return route_nt<2>(dtype, x, w_router, bias, logits, idx, gate, T, d, E, tp, s);
        case 4: return route_nt<4>(dtype, x, w_router, bias, logits, idx, gate, T, d, E, tp, s);
        case 8: return route_nt<8>(dtype, x, w_router, bias, logits, idx, gate, T, d, E, tp, s);
        default: return route_nt<16>(dtype, x, w_router, bias, logits, idx, gate, T, d, E, tp, s);
    }
}

hipError_t launch_route_from_logits(const float* logits, int32_t* idx, float* gate,
                                    long long T, int E, TopkParams tp, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const dim3 grid((unsigned)((T + 15) / 16));
    switch (nt_for(E)) {
        case 1: hipLaunchKernelGGL(topk_kernel<1>, grid, dim3(256), 0, s, logits, idx, gate, T, E, tp); break;
        case 2: hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(256), 0, s, logits, idx, gate, T, E, tp); break;
        case 4: hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, s, logits, idx, gate, T, E, tp); break;
        case 8: hipLaunchKernelGGL(topk_kernel<8>, grid, dim3(256), 0, s, logits, idx, gate, T, E, tp); break;
        default: hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, s, logits, idx, gate, T, E, tp); break;
    }
    return hipGetLastError();
}

}  // namespace moe
