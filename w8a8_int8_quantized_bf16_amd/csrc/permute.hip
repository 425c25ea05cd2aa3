// Grouping of the routed (token, slot) pairs by expert, for the grouped GEMM
// ("Qwen3-Next-80B-A3B-Instruct in AMCT" case, section 6: the MoE runs as one
// packed grouped matmul over the experts).
//
// A deterministic, stable counting sort of the P = T*k pair ids by expert:
//   1. count:   one block per chunk of 512 pairs -> per-chunk histograms
//   2. scan + scatter: one block per chunk.  Each block walks the histograms
//               of all chunks (per expert: the pairs before its own chunk and
//               the total), forms offsets[E+1] with one scan over experts, and
//               places its chunk's pairs in pair order, 256 at a time: equal
//               experts inside a wavefront are matched with eight ballots (one
//               per bit of the id), waves are ordered through LDS.  The same
//               blocks first write the grouped GEMMs' tile tables.
//   (up to 4096 pairs one block does all of it in a single launch)
// The result depends only on the ids: no atomics decide any position.
#include "device_common.h"
#include "launch.h"
#include "tiles.h"

namespace w8a8 {

namespace {
constexpr int PM_THREADS = 256;
constexpr int PM_PER_THREAD = 2;
constexpr int PM_CHUNK = PM_THREADS * PM_PER_THREAD;   // pairs per chunk
constexpr int PM_MAX_E = 256;
constexpr int64_t PM_SMALL_P = 4096;   // up to this many pairs: one block does everything

inline int64_t pm_chunks(int64_t P) { return (P + PM_CHUNK - 1) / PM_CHUNK; }
}  // namespace

__global__ __launch_bounds__(PM_THREADS) void permute_count_kernel(const int32_t *__restrict__ ids, int64_t P,
                                                                   int E, int32_t *__restrict__ chunk_counts)
{
    __shared__ int32_t hist[PM_MAX_E];
    const int tid = threadIdx.x;
    hist[tid] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * PM_CHUNK;
    for (int i = 0; i < PM_PER_THREAD; ++i) {
        const int64_t p = base + i * PM_THREADS + tid;
        if (p < P) atomicAdd(&hist[ids[p]], 1);
    }
    __syncthreads();
    if (tid < E) chunk_counts[(int64_t)blockIdx.x * E + tid] = hist[tid];
}

// chunk_counts[c][e] -> exclusive prefix over c (in place); offsets = exclusive
// prefix over e of the totals.
__global__ __launch_bounds__(PM_THREADS) void permute_scan_kernel(int32_t *__restrict__ chunk_counts,
                                                                  int64_t nchunks, int E, int64_t P,
                                                                  int32_t *__restrict__ offsets)
{
    __shared__ int32_t tot[PM_MAX_E];
    const int tid = threadIdx.x;
    int32_t run = 0;
    if (tid < E) {
        int64_t c = 0;
        // 32 independent loads in flight (a thread's walk over the chunks is a
        // chain of memory round trips: 128 chunks take four, not sixteen)
        for (; c + 32 <= nchunks; c += 32) {
            int32_t v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = chunk_counts[(c + u) * E + tid];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                chunk_counts[(c + u) * E + tid] = run;
                run += v[u];
            }
        }
        for (; c < nchunks; ++c) {
            const int32_t v = chunk_counts[c * E + tid];
            chunk_counts[c * E + tid] = run;
            run += v;
        }
    }
    int all;
    const int32_t ex = block_excl_scan256(tid < E ? run : 0, tot, &all);
    if (tid < E) offsets[tid] = ex;
    if (tid == 0) offsets[E] = (int32_t)P;
}

// Stable placement of the pairs p = first + 256 r + tid (r < rounds, p < P):
// pairs are ranked in pair order, 256 at a time; equal experts inside a
// wavefront are matched with eight ballots (one per bit of the id), waves are
// ordered through LDS.  base[e] (LDS) holds expert e's next free row and is
// advanced; wcnt is LDS scratch.
__device__ inline void scatter_rounds(const int32_t *__restrict__ ids, int64_t P, int64_t first, int rounds, int E,
                                      int32_t *base, int32_t (*wcnt)[PM_MAX_E], int32_t *__restrict__ sorted_pair,
                                      int32_t *__restrict__ pair_pos)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int round = 0; round < rounds; ++round) {
#pragma unroll
        for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
        __syncthreads();
        const int64_t p = first + (int64_t)round * PM_THREADS + tid;
        const bool valid = p < P;
        const int e = valid ? ids[p] : 0;
        // lanes of this wave holding the same expert id
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint64_t ones = __ballot(valid && ((e >> b) & 1));
            same &= ((e >> b) & 1) ? ones : ~ones;
        }
        const int rank_in_wave = __popcll(same & lt_mask);
        if (valid && rank_in_wave == 0) wcnt[wave][e] = __popcll(same);
        __syncthreads();
        if (valid) {
            int32_t before = 0;
            for (int w = 0; w < wave; ++w) before += wcnt[w][e];
            const int32_t row = base[e] + before + rank_in_wave;
            sorted_pair[row] = (int32_t)p;
            pair_pos[p] = row;
        }
        __syncthreads();
        if (tid < E) base[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
        __syncthreads();
    }
}

// The tile tables of up to four grouped GEMMs (TileTableReq): every block
// forms the tile prefixes from the offsets, block 0 stores them, and the
// blocks of the scatter grid share the descriptor writes.  extra > 0 appends
// one group of `extra` rows after the E expert groups (rows P .. P + extra of
// the grouped order, sorted_pair[P + t] = t * k: each token once, in order).
struct ScanTables {
    TileTableReq r[4];
    int n;
    int32_t extra;
    int k;
};

// Tile table j from the expert offsets in LDS (off_l[0..E], and off_l[E + 1]
// when tt.extra > 0); dn: LDS scratch of 2 ints.  All threads of the block
// call it; `first` / `stride` split the descriptor writes.
__device__ inline void build_table(const ScanTables &tt, int j, const int32_t *off_l, int E, int32_t *pre,
                                   int32_t *sc, int32_t *dn, bool store_prefix, int first, int stride)
{
    const TileTableReq &r = tt.r[j];
    const int32_t *offs = off_l;
    int G = tt.extra > 0 ? E + 1 : E;
    if (r.dense_rows > 0) {
        if (threadIdx.x == 0) {
            dn[0] = 0;
            dn[1] = r.dense_rows;
        }
        __syncthreads();
        offs = dn;
        G = 1;
    }
    const int total = tile_table_prefix(offs, G, r.BM, r.nblocks_n, pre, sc);
    if (store_prefix)
        for (int g = threadIdx.x; g <= G; g += PM_THREADS) r.prefix[g] = pre[g];
    tile_fill(offs, G, r.BM, r.nblocks_n, pre, total, r.tiles, first, stride);
    __syncthreads();
}

// Steps 2 and 3 in one launch (P > PM_SMALL_P): block b's thread e walks
// expert e's counts over all chunks, 32 loads in flight (the pairs of e before
// chunk b, and its total); one block scan over the totals gives the offsets
// (block 0 stores them), and the block scatters chunk b from offsets[e] plus
// the pairs of e before it.
__global__ __launch_bounds__(PM_THREADS) void permute_scan_scatter_kernel(const int32_t *__restrict__ ids, int64_t P,
                                                                          int E,
                                                                          const int32_t *__restrict__ chunk_counts,
                                                                          int64_t nchunks,
                                                                          int32_t *__restrict__ offsets,
                                                                          int32_t *__restrict__ sorted_pair,
                                                                          int32_t *__restrict__ pair_pos, ScanTables tt)
{
    __shared__ int32_t base[PM_MAX_E];     // next free row of each expert inside this chunk
    __shared__ int32_t wcnt[4][PM_MAX_E];  // per-wave counts of the current round
    __shared__ int32_t off_l[PM_MAX_E + 2];
    __shared__ int32_t pre[PM_MAX_E + 2];
    __shared__ int32_t dn[2];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;

    // ---- this block's offsets and chunk base
    int32_t before = 0, total = 0;
    if (tid < E) {
        int64_t c = 0;
        for (; c + 32 <= nchunks; c += 32) {
            int32_t v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = chunk_counts[(c + u) * E + tid];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                total += v[u];
                before += c + u < b ? v[u] : 0;
            }
        }
        for (; c < nchunks; ++c) {
            const int32_t v = chunk_counts[c * E + tid];
            total += v;
            before += c < b ? v : 0;
        }
    }
    int all;
    const int32_t ex = block_excl_scan256(tid < E ? total : 0, &wcnt[0][0], &all);
    if (tid < E) {
        off_l[tid] = ex;
        base[tid] = ex + before;
        if (b == 0) offsets[tid] = ex;
    }
    if (tid == 0) {
        off_l[E] = (int32_t)P;
        off_l[E + 1] = (int32_t)P + tt.extra;
        if (b == 0) offsets[E] = (int32_t)P;
    }
    // ---- tile tables (and the extra group's rows)
    for (int64_t t = b * PM_THREADS + tid; t < tt.extra; t += (int64_t)gridDim.x * PM_THREADS)
        sorted_pair[P + t] = (int32_t)(t * tt.k);
    __syncthreads();
    for (int j = 0; j < tt.n; ++j)
        build_table(tt, j, off_l, E, pre, &wcnt[0][0], dn, b == 0, (int)b * PM_THREADS + tid,
                    gridDim.x * PM_THREADS);

    // ---- scatter
    scatter_rounds(ids, P, b * PM_CHUNK, PM_PER_THREAD, E, base, wcnt, sorted_pair, pair_pos);
}

// P <= PM_SMALL_P: the whole permutation in one launch of 1 + tt.n blocks.
// Every block forms the histogram and offsets of the (at most 4096) ids
// itself; block 0 then stores the offsets and scatters the pairs, block
// 1 + j builds tile table j, side by side.
__global__ __launch_bounds__(PM_THREADS) void permute_small_kernel(const int32_t *__restrict__ ids, int64_t P, int E,
                                                                   int32_t *__restrict__ offsets,
                                                                   int32_t *__restrict__ sorted_pair,
                                                                   int32_t *__restrict__ pair_pos, ScanTables tt)
{
    __shared__ int32_t base[PM_MAX_E];
    __shared__ int32_t wcnt[4][PM_MAX_E];
    __shared__ int32_t off_l[PM_MAX_E + 2];
    __shared__ int32_t pre[PM_MAX_E + 2];
    __shared__ int32_t dn[2];
    __shared__ int32_t ids_l[PM_SMALL_P];
    const int tid = threadIdx.x;
    int32_t *hist = &wcnt[0][0];
    hist[tid] = 0;
    // the ids into LDS, up to 16 loads per thread in flight
    constexpr int PER = (int)(PM_SMALL_P / PM_THREADS);
    int32_t v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int p = u * PM_THREADS + tid;
        v[u] = p < P ? ids[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u)
        if (u * PM_THREADS + tid < P) ids_l[u * PM_THREADS + tid] = v[u];
    __syncthreads();
    for (int p = tid; p < P; p += PM_THREADS) atomicAdd(&hist[ids_l[p]], 1);   // counts only
    __syncthreads();
    int all;
    const int32_t ex = block_excl_scan256(tid < E ? hist[tid] : 0, &wcnt[1][0], &all);
    if (tid < E) {
        off_l[tid] = ex;
        if (blockIdx.x == 0) offsets[tid] = ex;
    }
    if (tid == 0) {
        off_l[E] = (int32_t)P;
        if (blockIdx.x == 0) offsets[E] = (int32_t)P;
        off_l[E + 1] = (int32_t)P + tt.extra;
    }
    __syncthreads();
    if (blockIdx.x > 0) {   // one tile table
        build_table(tt, blockIdx.x - 1, off_l, E, pre, &wcnt[2][0], dn, true, tid, PM_THREADS);
        return;
    }
    for (int t = tid; t < tt.extra; t += PM_THREADS) sorted_pair[P + t] = t * tt.k;
    if (tid < E) base[tid] = off_l[tid];
    scatter_rounds(ids_l, P, 0, (int)((P + PM_THREADS - 1) / PM_THREADS), E, base, wcnt, sorted_pair, pair_pos);
}

size_t permute_ws_bytes(int64_t T, int k, int E) { return (size_t)pm_chunks(T * k) * (size_t)E * sizeof(int32_t); }

hipError_t launch_permute(const int32_t *ids, int64_t T, int k, int E, int32_t *offsets, int32_t *sorted_pair,
                          int32_t *pair_pos, void *ws, hipStream_t st, const TileTableReq *req, int nreq,
                          int32_t extra_rows)
{
    ScanTables tt;
    tt.n = nreq < 4 ? nreq : 4;
    for (int j = 0; j < tt.n; ++j) tt.r[j] = req[j];
    tt.extra = extra_rows;
    tt.k = k;
    const int64_t P = T * k;
    if (P > 0 && P <= PM_SMALL_P) {
        hipLaunchKernelGGL(permute_small_kernel, dim3(1 + tt.n), dim3(PM_THREADS), 0, st, ids, P, E, offsets,
                           sorted_pair, pair_pos, tt);
        return hipGetLastError();
    }
    const int64_t nch = pm_chunks(P);
    int32_t *cc = (int32_t *)ws;
    if (nch == 0) {
        // P == 0: only the scan runs, it writes all-zero offsets (and no tile
        // table is needed: a GEMM over zero rows launches nothing)
        hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(PM_THREADS), 0, st, cc, nch, E, P, offsets);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(permute_count_kernel, dim3((unsigned)nch), dim3(PM_THREADS), 0, st, ids, P, E, cc);
    hipLaunchKernelGGL(permute_scan_scatter_kernel, dim3((unsigned)nch), dim3(PM_THREADS), 0, st, ids, P, E, cc,
                       nch, offsets, sorted_pair, pair_pos, tt);
    return hipGetLastError();
}

}  // namespace w8a8
