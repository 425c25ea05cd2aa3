// Device-side construction of a grouped GEMM's tile table (shared by the
// permutation kernel, which builds the layer's tables right after the group
// offsets are known, and by the stand-alone tile-map kernel).
#pragma once
#include "device_common.h"

namespace w8a8 {

constexpr int TILES_MAX_G = 4096;   // groups a tile table supports (LDS prefix)

// Tiles are numbered group-major, then column block, then row tile
// (v = prefix[g] + nb * mt_g + mt), where mt_g = ceil(rows_g / BM) and there
// are nbn column blocks per group.  A launched block v runs tile tiles[v'],
// where the blocks of XCD x (bid % 8 == x, the hardware's round-robin
// placement) take one contiguous range of v, so tiles that share a weight
// block or an activation block run side by side on one XCD's L2.

// Exclusive prefix of the tile counts over the groups into pre[0..G] (LDS);
// returns the total.  Called by all 256 threads of a block; sc is LDS scratch
// of at least 4 ints.  offsets may be in LDS or global memory.
__device__ inline int tile_table_prefix(const int32_t *offsets, int G, int BM, int nbn, int32_t *pre, int32_t *sc)
{
    const int tid = threadIdx.x;
    int carry = 0;
    for (int g0 = 0; g0 < G; g0 += 256) {
        const int g = g0 + tid;
        const int32_t cnt = g < G ? (offsets[g + 1] - offsets[g] + BM - 1) / BM * nbn : 0;
        int tot;
        const int ex = block_excl_scan256(cnt, sc, &tot);
        if (g < G) pre[g] = carry + ex;
        carry += tot;
    }
    if (tid == 0) pre[G] = carry;
    __syncthreads();
    return carry;
}

// Writes the descriptors {group, first grouped row, rows, column block} of
// the tiles, each at its dispatch slot (see above).  Thread `first` of
// `stride` threads writes one contiguous run of tile numbers: it finds the
// group of the run's first tile by bisection over pre and then walks the
// groups forward.
__device__ inline void tile_fill(const int32_t *offsets, int G, int BM, int nbn, const int32_t *pre, int total,
                                 int4 *__restrict__ tiles, int first, int stride)
{
    const int q = total >> 3, r = total & 7;
    const int chunk = (total + stride - 1) / stride;
    int v = first * chunk;
    const int vend = min(total, v + chunk);
    if (v >= vend) return;
    int lo = 0, hi = G;   // largest g with pre[g] <= v
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= v) lo = mid;
        else hi = mid;
    }
    int g = lo, gend = pre[g + 1];
    int32_t row_begin = offsets[g], rows_g = offsets[g + 1] - row_begin;
    int mt_g = (rows_g + BM - 1) / BM;
    for (; v < vend; ++v) {
        while (v >= gend) {   // next non-empty group
            ++g;
            gend = pre[g + 1];
            row_begin = offsets[g];
            rows_g = offsets[g + 1] - row_begin;
            mt_g = (rows_g + BM - 1) / BM;
        }
        const int local = v - pre[g];
        const int nb = local / mt_g, mt = local - nb * mt_g;
        int x = 7;   // XCD x owns v in [x*q + min(x, r), (x+1)*q + min(x+1, r))
        while (x > 0 && v < x * q + (x < r ? x : r)) --x;
        const int slot = v - (x * q + (x < r ? x : r));
        tiles[slot * 8 + x] = make_int4(g, row_begin + mt * BM, min(BM, rows_g - mt * BM), nb);
    }
}

}  // namespace w8a8
