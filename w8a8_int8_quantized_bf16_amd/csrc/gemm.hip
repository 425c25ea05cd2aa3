// Grouped W8A8 GEMM on CDNA4 int8 matrix cores.
//
// int8 x int8 -> int32 products against static per-output-channel int8
// weights, dequantised per token x per channel ("Qwen3.6-35B-A3B-w8a8
// config.json and recipe.yaml" walkthrough, group_0 "weights" and
// "input_activations"; "Qwen3-30B-A3B-Instruct-2507-quantized.w8a8" explainer,
// FAQ Q1: W8A8 runs the matmul on integers), with the SwiGLU of the packed
// gate_up_proj fused into the epilogue ("Qwen3-Next-80B-A3B-Instruct in AMCT"
// case, section 2.2: gate and up rows concatenated along the output dim).
//
// Work decomposition
//   * A tile is (group g, BM grouped rows, one column block).  A column block
//     is 4 wavefronts x 64 columns; with SwiGLU each wave owns 32 output
//     columns, i.e. 32 gate rows and the 32 matching up rows of B.
//   * B (the weights, the dominant HBM stream) goes straight from global
//     memory into registers in MFMA operand order: each lane loads 64
//     contiguous bytes of one weight row per 128-byte K step, so a wave reads
//     whole 128-byte lines.  Each weight byte is loaded by exactly one wave of
//     the tile; a ring of DEPTH K steps keeps loads in flight.
//   * A (the activation codes, gathered rows) is shared by the 4 waves through
//     LDS, double buffered, with a 16-byte-chunk XOR swizzle (chunk ^ row%8)
//     so that both the staging stores and the fragment reads are conflict free.
//   * The K order inside one MFMA step is permuted identically for A and B
//     (lane half h, sub-step s takes bytes 64h+16s..+16 of the 128-byte step);
//     integer sums are exact, so any common K permutation gives the same acc.
//   * v_mfma_i32_32x32x32_i8: A lane l supplies row l%32, B lane l column l%32,
//     16 bytes each; accumulator value i of lane l is row 8(i/4)+4(l/32)+i%4,
//     column l%32.
//   * Tiles are enumerated group-major, then column block, then row tile, and
//     handed out so that each of the 8 XCDs gets one contiguous range: the row
//     tiles that share a weight block, and the column blocks that share an A
//     block, run at the same time on the same L2.
//   * The tile map (tiles per group) is built on the device from the group
//     offsets, so the host never waits for the routing result.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {
constexpr int G_THREADS = 256;
constexpr int G_BK = 128;          // K bytes per step
constexpr int G_COLS_PER_WAVE = 64;
constexpr int G_BLOCK_COLS = 4 * G_COLS_PER_WAVE;

struct GemmArgs {
    const int8_t *A;
    const float *a_scales;
    const int32_t *gather;
    int gather_div;
    const int8_t *B;
    const float *b_scales;
    const int32_t *offsets;
    int G;
    int64_t M_total, N, K;
    void *out;
    const int32_t *tile_prefix;   // [G+1]: first tile of each group; [G] = total tiles
    int nblocks_n;                // column blocks per group
};

template <typename T>
__device__ __forceinline__ void store_out(T *p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float v) { *p = (uint16_t)float_to_bf16_bits(v); }
}  // namespace

// tile_prefix[g] = sum over g' < g of ceil(rows(g') / BM) * nblocks_n
__global__ __launch_bounds__(256) void gemm_tilemap_kernel(const int32_t *__restrict__ offsets, int G, int BM,
                                                           int nblocks_n, int32_t *__restrict__ tile_prefix)
{
    __shared__ int32_t sc[256];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int g0 = 0; g0 < G; g0 += 256) {
        const int g = g0 + tid;
        int32_t cnt = 0;
        if (g < G) {
            const int32_t rows = offsets[g + 1] - offsets[g];
            cnt = (rows + BM - 1) / BM * nblocks_n;
        }
        sc[tid] = cnt;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int32_t v = tid >= d ? sc[tid - d] : 0;
            __syncthreads();
            sc[tid] += v;
            __syncthreads();
        }
        if (g < G) tile_prefix[g] = carry + sc[tid] - cnt;
        __syncthreads();
        if (tid == 255) carry += sc[255];
        __syncthreads();
    }
    if (tid == 0) tile_prefix[G] = carry;
}

template <int BM, int EPI, typename OutT, int DEPTH>
__global__ __launch_bounds__(G_THREADS) void grouped_gemm_kernel(GemmArgs a)
{
    constexpr int MI = BM / 32;      // 32-row MFMA tiles per wave
    constexpr int APASS = BM / 32;   // A chunks staged per thread per K step
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * G_BK];
    __shared__ int32_t arow[BM];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // ---- which tile
    const int total = a.tile_prefix[a.G];
    const int bid = blockIdx.x;
    if (bid >= total) return;
    const int xq = total >> 3, xr = total & 7, xcd = bid & 7;
    const int v = xcd * xq + (xcd < xr ? xcd : xr) + (bid >> 3);
    int lo = 0, hi = a.G;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.tile_prefix[mid] <= v) lo = mid;
        else hi = mid;
    }
    const int g = lo;
    const int32_t row_begin = a.offsets[g];
    const int32_t rows_g = a.offsets[g + 1] - row_begin;
    const int mt_g = (rows_g + BM - 1) / BM;
    const int local = v - a.tile_prefix[g];
    const int nb = local / mt_g, mt = local - nb * mt_g;
    const int64_t row0 = (int64_t)row_begin + (int64_t)mt * BM;
    const int rows = min(BM, rows_g - mt * BM);
    const int64_t N = a.N, K = a.K;

    if (tid < BM) {
        int32_t src = -1;
        if (tid < rows) src = a.gather ? a.gather[row0 + tid] / a.gather_div : (int32_t)(row0 + tid);
        arow[tid] = src;
    }

    // ---- B rows of this lane
    const int8_t *brow[2];
    bool bvalid[2];
    int64_t col[2];
    if constexpr (EPI == 2) {
        const int64_t Nh = N >> 1;
        const int64_t hc = (int64_t)nb * (G_BLOCK_COLS / 2) + wave * 32 + (lane & 31);
        col[0] = hc;
        col[1] = Nh + hc;
        bvalid[0] = bvalid[1] = hc < Nh;
    } else {
        const int64_t c0 = (int64_t)nb * G_BLOCK_COLS + wave * G_COLS_PER_WAVE + (lane & 31);
        col[0] = c0;
        col[1] = c0 + 32;
        bvalid[0] = c0 < N;
        bvalid[1] = c0 + 32 < N;
    }
    const int8_t *Bg = a.B + (int64_t)g * N * K;
#pragma unroll
    for (int f = 0; f < 2; ++f) brow[f] = Bg + (bvalid[f] ? col[f] : 0) * K + 64 * (lane >> 5);

    __syncthreads();

    // ---- A staging assignment: chunk c of rows (tid/8) + 32j
    const int ac = tid & 7;
    const int8_t *asrc[APASS];
    int arr[APASS];
#pragma unroll
    for (int j = 0; j < APASS; ++j) {
        arr[j] = (tid >> 3) + 32 * j;
        const int32_t s = arow[arr[j]];
        asrc[j] = s >= 0 ? a.A + (int64_t)s * K + 16 * ac : nullptr;
    }

    const int nk = (int)((K + G_BK - 1) / G_BK);
    const v4i zero4 = {0, 0, 0, 0};

    v4i breg[DEPTH][2][4];
    v4i areg[APASS];
    v16i acc[MI][2];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][f][i] = 0;

    auto load_b = [&](int slot, int it) {
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int64_t koff = (int64_t)it * G_BK + 64 * (lane >> 5) + 16 * s;
                breg[slot][f][s] = (it < nk && bvalid[f] && koff < K)
                                       ? *reinterpret_cast<const v4i *>(brow[f] + (int64_t)it * G_BK + 16 * s)
                                       : zero4;
            }
    };
    auto load_a = [&](int it) {
        const int64_t koff = (int64_t)it * G_BK + 16 * ac;
#pragma unroll
        for (int j = 0; j < APASS; ++j)
            areg[j] = (asrc[j] && koff < K) ? *reinterpret_cast<const v4i *>(asrc[j] + (int64_t)it * G_BK) : zero4;
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < APASS; ++j)
            *reinterpret_cast<v4i *>(&As[buf][arr[j] * G_BK + ((ac ^ (arr[j] & 7)) << 4)]) = areg[j];
    };

#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_b(d, d);
    load_a(0);
    store_a(0);
    __syncthreads();

    for (int it0 = 0; it0 < nk; it0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int it = it0 + d;
            if (it < nk) {
                const bool more = it + 1 < nk;
                if (more) load_a(it + 1);
                const int8_t *Ab = As[it & 1];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi) {
                        const int r = mi * 32 + (lane & 31);
                        const int ch = 4 * (lane >> 5) + s;
                        const v4i av = *reinterpret_cast<const v4i *>(Ab + r * G_BK + ((ch ^ (r & 7)) << 4));
#pragma unroll
                        for (int f = 0; f < 2; ++f)
                            acc[mi][f] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, breg[d][f][s], acc[mi][f], 0, 0, 0);
                    }
                }
                load_b(d, it + DEPTH);
                if (more) store_a((it + 1) & 1);
                __syncthreads();
            }
        }
    }

    // ---- epilogue
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (r >= rows) continue;
            const int64_t grow = row0 + r;
            if constexpr (EPI == 0) {
#pragma unroll
                for (int f = 0; f < 2; ++f)
                    if (bvalid[f]) reinterpret_cast<int32_t *>(a.out)[grow * N + col[f]] = acc[mi][f][i];
            } else if constexpr (EPI == 1) {
                const float sa = a.a_scales[arow[r]];
#pragma unroll
                for (int f = 0; f < 2; ++f)
                    if (bvalid[f]) {
                        const float sb = a.b_scales[(int64_t)g * N + col[f]];
                        store_out<OutT>(reinterpret_cast<OutT *>(a.out) + grow * N + col[f],
                                        ((float)acc[mi][f][i] * sa) * sb);
                    }
            } else {
                if (bvalid[0]) {
                    const float sa = a.a_scales[arow[r]];
                    const float gate = ((float)acc[mi][0][i] * sa) * a.b_scales[(int64_t)g * N + col[0]];
                    const float up = ((float)acc[mi][1][i] * sa) * a.b_scales[(int64_t)g * N + col[1]];
                    const float h = gate / (1.0f + expf(-gate)) * up;
                    store_out<OutT>(reinterpret_cast<OutT *>(a.out) + grow * (N >> 1) + col[0], h);
                }
            }
        }
    }
}

size_t gemm_ws_bytes(int64_t M_total, int64_t N, int G)
{
    (void)M_total;
    (void)N;
    return ((size_t)(G + 1) * sizeof(int32_t) + 255) & ~(size_t)255;
}

namespace {
int gemm_bm(int64_t M_total, int G)
{
    const double avg_rows = (double)M_total / (double)G;
    return avg_rows <= 32.0 ? 32 : (avg_rows <= 64.0 ? 64 : 128);
}

int gemm_nblocks(int64_t N, int epilogue)
{
    const int64_t cols = epilogue == 2 ? N / 2 : N;
    const int64_t per_block = epilogue == 2 ? G_BLOCK_COLS / 2 : G_BLOCK_COLS;
    return (int)((cols + per_block - 1) / per_block);
}

template <int BM, int DEPTH>
hipError_t launch_main_bm(const GemmArgs &ga, int epilogue, int out_dtype, hipStream_t st)
{
    const int64_t max_tiles = ((ga.M_total + BM - 1) / BM + ga.G) * ga.nblocks_n;
    dim3 grid((unsigned)max_tiles), block(G_THREADS);
    if (epilogue == 0)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, 0, int32_t, DEPTH>), grid, block, 0, st, ga);
    else if (epilogue == 1 && out_dtype == 0)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, 1, uint16_t, DEPTH>), grid, block, 0, st, ga);
    else if (epilogue == 1)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, 1, float, DEPTH>), grid, block, 0, st, ga);
    else if (out_dtype == 0)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, 2, uint16_t, DEPTH>), grid, block, 0, st, ga);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, 2, float, DEPTH>), grid, block, 0, st, ga);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_tilemap(const int32_t *offsets, int G, int64_t M_total, int64_t N, int epilogue, void *ws,
                               hipStream_t st)
{
    if (M_total == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_tilemap_kernel, dim3(1), dim3(256), 0, st, offsets, G, gemm_bm(M_total, G),
                       gemm_nblocks(N, epilogue), (int32_t *)ws);
    return hipGetLastError();
}

hipError_t launch_gemm_main(const int8_t *A, const float *a_scales, const int32_t *gather, int gather_div,
                            const int8_t *B, const float *b_scales, const int32_t *offsets, int G, int64_t M_total,
                            int64_t N, int64_t K, int epilogue, int out_dtype, void *out, const void *ws,
                            hipStream_t st)
{
    if (M_total == 0) return hipSuccess;
    GemmArgs ga;
    ga.A = A;
    ga.a_scales = a_scales;
    ga.gather = gather;
    ga.gather_div = gather_div > 0 ? gather_div : 1;
    ga.B = B;
    ga.b_scales = b_scales;
    ga.offsets = offsets;
    ga.G = G;
    ga.M_total = M_total;
    ga.N = N;
    ga.K = K;
    ga.out = out;
    ga.tile_prefix = (const int32_t *)ws;
    ga.nblocks_n = gemm_nblocks(N, epilogue);
    switch (gemm_bm(M_total, G)) {
    case 32: return launch_main_bm<32, 4>(ga, epilogue, out_dtype, st);
    case 64: return launch_main_bm<64, 3>(ga, epilogue, out_dtype, st);
    default: return launch_main_bm<128, 2>(ga, epilogue, out_dtype, st);
    }
}

hipError_t launch_grouped_gemm(const int8_t *A, const float *a_scales, const int32_t *gather, int gather_div,
                               const int8_t *B, const float *b_scales, const int32_t *offsets, int G,
                               int64_t M_total, int64_t N, int64_t K, int epilogue, int out_dtype, void *out,
                               void *ws, hipStream_t st)
{
    hipError_t e = launch_gemm_tilemap(offsets, G, M_total, N, epilogue, ws, st);
    if (e != hipSuccess) return e;
    return launch_gemm_main(A, a_scales, gather, gather_div, B, b_scales, offsets, G, M_total, N, K, epilogue,
                            out_dtype, out, ws, st);
}

}  // namespace w8a8
