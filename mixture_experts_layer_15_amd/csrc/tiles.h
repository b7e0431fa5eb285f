// tiles.h -- the grouped GEMMs' tile list, built on the device from
// expert_offset (the number of kept rows per expert never leaves the GPU).
//
// Tiles are numbered expert-major, then N-tile, then M-tile (M fastest), so
// the M-tiles that share one weight tile are adjacent, and consecutive
// N-tiles of one expert reuse that expert's rows.  A persistent grid walks
// the list in sweeps of gridDim.x tiles; within a sweep workgroup b takes
// tile sweep_tile(b, ...), which hands each XCD (workgroups b, b+8, ... run
// on XCD b % 8) a contiguous run of tile ids, so tiles that share data meet
// in the same L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct TileTable {
    long long start[257];   // tiles before expert e; start[E] = total
    int mtiles[256];        // M-tiles of expert e
};

// Every thread of the block (a multiple of 64, at least 256) calls this; the
// first 256 own one expert each.  ntn = N-tiles per expert.  s_wave holds one
// entry per wave.  Without an offset table (off == nullptr, E == 1) the single
// group has dense_rows rows.  Experts whose row count lies outside
// [rlo, rhi) get no tiles (they are left to another launch).
template <int TBM>
__device__ __forceinline__ void build_tile_table(const int32_t* __restrict__ off, int E, int ntn,
                                                 TileTable& tt, long long* s_wave,
                                                 int dense_rows = 0, int rlo = 0,
                                                 int rhi = 0x7fffffff) {
    const int e = threadIdx.x;
    long long cnt = 0;
    int mt = 0;
    if (e < E) {
        // off == nullptr: one group (E == 1) of dense_rows rows
        int kept = off ? off[e + 1] - off[e] : dense_rows;
        if (kept < rlo || kept >= rhi) kept = 0;
        mt = (kept + TBM - 1) / TBM;
        cnt = (long long)mt * ntn;
    }
    if (e < 256) tt.mtiles[e] = mt;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    long long v = cnt;
    for (int o = 1; o < 64; o <<= 1) {
        const long long u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_wave[w] = v;
    __syncthreads();
    long long add = 0;
    for (int i = 0; i < w; ++i) add += s_wave[i];
    if (e < 256) tt.start[e + 1] = v + add;
    if (e == 0) tt.start[0] = 0;
    __syncthreads();
}

// Tile id -> (expert, m-tile, n-tile): the largest e with start[e] <= t (an
// expert with no tiles has start[e] == start[e+1] and is never chosen).
// Inside an expert the M-tiles go in groups of GM: for each group, every
// N-tile, M fastest.  Experts with at most GM M-tiles get the plain order
// (N-tile, then M); larger ones get GM x N blocks, so a run of consecutive
// tiles on one XCD shares both its activation rows and its weight columns.
template <int GM>
__device__ __forceinline__ void decode_tile(const TileTable& tt, int E, int ntn, long long t,
                                            int& e, int& m, int& n) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tt.start[mid] <= t) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const long long local = t - tt.start[e];
    const int mt = tt.mtiles[e];
    const int g = (int)(local / ((long long)GM * ntn));
    const int gs = min(GM, mt - g * GM);
    const int r = (int)(local - (long long)g * GM * ntn);
    n = r / gs;
    m = g * GM + r % gs;
}

// Tile of workgroup b in the sweep that starts at tile `base`, or -1.  The
// sweep holds n = min(G, total - base) tiles (G a multiple of 8, the grid),
// cut into 8 contiguous runs of ceil(n / 8); run x goes to XCD x, tile i of
// the run to the XCD's i-th workgroup (b = 8 i + x).  Sizing the runs by n
// rather than by G matters when a sweep is not full: the grid is sized on the
// host from an upper bound on the tiles, and runs of G / 8 would put the
// whole of a short sweep on the first few XCDs, leaving the others idle.
__device__ __forceinline__ long long sweep_tile(int b, int G, long long base, long long total) {
    const long long n = min((long long)G, total - base);
    const long long per = (n + 7) >> 3;
    const long long i = b >> 3;
    const long long t = base + (long long)(b & 7) * per + i;
    return (i < per && t < base + n) ? t : -1;
}

}  // namespace moe
