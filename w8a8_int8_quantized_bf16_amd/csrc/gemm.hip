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

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "quant_common.h"
#include "tiles.h"

namespace w8a8 {

namespace {
constexpr int G_THREADS = 256;
constexpr int G_BK = 128;          // K bytes per step

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
    int64_t A_bytes;              // bytes of A addressable (rows * K)
    void *out;
    int8_t *out_exp;              // EPI_FIXED16 only: [M][ceil(N/64)] power-of-two exponents
    const int32_t *tile_prefix;   // [G+1]: first tile of each group; [G] = total tiles
    const int4 *tiles;            // per launched block: {group, first grouped row, rows, column block}
    int nblocks_n;                // column blocks per group
    int packed_b;                 // B in the MFMA-fragment packed layout (see w8a8_pack_weights)
    const float *b_gscales;       // W4: per (group, 128-step, column) scales [G][KS][N]
    const int8_t *b_goffs;        //     and offsets [G][KS][N] (step-major: one coalesced read per step)
    int G_routed;                 // groups g >= G_routed take their weights from
    const int8_t *B_extra;        //   B_extra / b_extra_scales (one group's worth,
    const float *b_extra_scales;  //   same layout) instead of B and b_scales
    int32_t dense_rows;           // > 0: one group of this many rows, tiles from
                                  //   the block index (no tile table)
    int ksplit, ksteps;           // dense: K in ksplit slices of ksteps 128-byte
                                  //   steps, each writing int32 sums to out + slice * M * N
    const uint16_t *A_h;          // quantise on load: A as bf16 rows (no gather, A_bytes
    int8_t *a_codes_out;          //   still rows * K); the tiles of column block 0 also
    float *a_scales_out;          //   store the rows' int8 codes [rows][K] and scales
};

// The tile of block `bid` of a one-group GEMM without a table: the same
// numbering and XCD split as tile_fill (column block, then row tile; XCD x =
// bid % 8 runs one contiguous range of tile numbers).  False past the last tile.
// With K split into ksplit slices the tiles are numbered slice-major (the
// slice goes to the descriptor's group field).
__device__ __forceinline__ bool dense_tile(int bid, int32_t M, int BM, int nbn, int ksplit, int4 *t)
{
    const int mt_n = (M + BM - 1) / BM;
    const int per = mt_n * nbn, total = per * ksplit;
    if (bid >= total) return false;
    const int q = total >> 3, r = total & 7;
    const int x = bid & 7, slot = bid >> 3;
    int v = x * q + min(x, r) + slot;
    const int ks = v / per;
    v -= ks * per;
    const int nb = v / mt_n, mt = v - nb * mt_n;
    *t = make_int4(ks, mt * BM, min(BM, M - mt * BM), nb);
    return true;
}

template <typename T>
__device__ __forceinline__ T to_out(float v);
template <>
__device__ __forceinline__ float to_out<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t to_out<uint16_t>(float v) { return (uint16_t)float_to_bf16_bits(v); }
}  // namespace

// Stand-alone tile map of one grouped GEMM (see tiles.h): every block forms
// the tile prefix from the offsets, block 0 stores it, and the blocks share
// the descriptor writes.  offsets == nullptr: one group of dense_rows rows.
__global__ __launch_bounds__(256) void gemm_tilemap_kernel(const int32_t *__restrict__ offsets, int G, int BM,
                                                           int nblocks_n, int32_t *__restrict__ tile_prefix,
                                                           int4 *__restrict__ tiles, int32_t dense_rows)
{
    __shared__ int32_t pre[TILES_MAX_G + 1];
    __shared__ int32_t sc[256];
    __shared__ int32_t dense_off[2];
    if (!offsets) {
        if (threadIdx.x == 0) {
            dense_off[0] = 0;
            dense_off[1] = dense_rows;
        }
        __syncthreads();
        offsets = dense_off;
    }
    const int total = tile_table_prefix(offsets, G, BM, nblocks_n, pre, sc);
    if (blockIdx.x == 0)
        for (int g = threadIdx.x; g <= G; g += 256) tile_prefix[g] = pre[g];
    tile_fill(offsets, G, BM, nblocks_n, pre, total, tiles, blockIdx.x * 256 + threadIdx.x, gridDim.x * 256);
}

// Packed weight layout: B [G][N][K] int8 re-laid so that one wavefront's
// MFMA operand fetch is 1 KiB of contiguous memory.  For group g, 32-row block
// nb and 128-byte K step ks, a 4 KiB chunk at ((g * NB + nb) * KS + ks) * 4096
// holds, at s * 1024 + l * 16 (sub-step s, lane l), bytes
// [64 * (l / 32) + 16 * s, +16) of step ks of row 32 * nb + l % 32.  Rows
// beyond N and bytes beyond K are zero.  NB = ceil(N / 32), KS = ceil(K / 128).
__global__ __launch_bounds__(256) void pack_weights_kernel(const int8_t *__restrict__ B, int64_t G, int64_t N,
                                                           int64_t K, int8_t *__restrict__ P)
{
    const int64_t NB = (N + 31) / 32, KS = (K + 127) / 128;
    const int64_t n16 = G * NB * KS * 256;   // 16-byte pieces
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
        const int64_t chunk = i >> 8;
        const int within = (int)(i & 255);
        const int s = within >> 6, l = within & 63;
        const int64_t ks = chunk % KS, nbk = (chunk / KS) % NB, g = chunk / (KS * NB);
        const int64_t row = nbk * 32 + (l & 31);
        const int64_t k0 = ks * 128 + 64 * (l >> 5) + 16 * s;
        v4i v = {0, 0, 0, 0};
        if (row < N && k0 < K) v = *reinterpret_cast<const v4i *>(B + (g * N + row) * K + k0);
        *reinterpret_cast<v4i *>(P + i * 16) = v;
    }
}

// Packed W4 layout: codes B [G][N][K] (one per byte, in [-8, 7]) re-laid so
// that a lane's MFMA operands of one 128-column step are 32 contiguous bytes.
// For group g, 32-row block nb and step ks, a 2 KiB chunk at
// ((g * NB + nb) * KS + ks) * 2048 holds at l * 32 + 16 p + 4 j + i (lane l,
// piece p, dword j, byte i) the code of sub-step 2p in the low nibble and of
// sub-step 2p + 1 in the high nibble, both at index 4 j + i of lane l's 16
// operand bytes (row 32 nb + l % 32, column 128 ks + 64 (l / 32) + 16 s + 4 j
// + i).  A nibble moved to the top of its byte is 16 times the code as an
// int8, so a shift and a mask unpack four operands at once.  Zero padded.
__global__ __launch_bounds__(256) void pack_w4_kernel(const int8_t *__restrict__ B, int64_t G, int64_t N,
                                                      int64_t K, uint32_t *__restrict__ P)
{
    const int64_t NB = (N + 31) / 32, KS = (K + 127) / 128;
    const int64_t nd = G * NB * KS * 512;   // dwords
    for (int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x; d < nd; d += (int64_t)gridDim.x * 256) {
        const int64_t chunk = d >> 9;
        const int within = (int)(d & 511);
        const int l = within >> 3, pj = within & 7, p = pj >> 2, j = pj & 3;
        const int64_t ks = chunk % KS, nbk = (chunk / KS) % NB, g = chunk / (KS * NB);
        const int64_t row = nbk * 32 + (l & 31);
        const int64_t k0 = ks * 128 + 64 * (l >> 5) + 4 * j;
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t klo = k0 + 16 * (2 * p) + i, khi = k0 + 16 * (2 * p + 1) + i;
            const int lo = (row < N && klo < K) ? B[(g * N + row) * K + klo] : 0;
            const int hi = (row < N && khi < K) ? B[(g * N + row) * K + khi] : 0;
            word |= (uint32_t)((lo & 0xf) | ((hi & 0xf) << 4)) << (8 * i);
        }
        P[d] = word;
    }
}

// Buffer-resource loads: an offset at or beyond num_records returns zero
// without touching memory, which masks ragged rows, column tails and the K
// tail without branches (so the compiler's wait counters stay exact and the
// prefetch ring below keeps its loads in flight).
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr uint32_t OOB_BASE = 0xC0000000u;   // above any resource size (< 2^31)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes)
{
    const int n = bytes > 0x7ffffff0LL ? 0x7ffffff0 : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, n, 0x00020000);
}

__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return __builtin_bit_cast(v4i, v);
}

// Direct memory-to-LDS transfer: lane l's 16 bytes at offset off of r land in
// LDS at lds + 16 l (lds wave-uniform, through M0).  Written in asm so that
// the compiler, which would otherwise make every later LDS read wait for all
// outstanding loads, leaves the waits to lds_barrier; the asm names M0, the
// only register it changes besides the memory.  Offsets out of range return
// zeros, as for buf_load16.
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier after this wave's LDS operations have completed and at
// most N of its memory loads (transfers included, oldest first) are still in
// flight.  A compiler memory barrier too: no load or LDS access moves across.
template <int N>
__device__ __forceinline__ void lds_barrier()
{
    static_assert(N >= 0 && N <= 63, "vmcnt counts up to 63");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Epilogue of one tile.  Each wave stages its results through its own LDS
// region (stage_base + wave * 32 * ROWB, see gemm_stage_bytes), one 32-row
// block and at most two 32-column fragments at a time, and writes them back
// as 16-byte row segments (the MFMA layout gives a lane one column of many
// rows; a store wants many columns of one row).  ascale: the tile's
// activation scales (LDS); bsc: this lane's column scales.  FACC: acc holds
// fp32 bit patterns already scaled per column (W4A8), bsc all ones.
template <int EPI, typename OutT>
struct EpiTypes {
    // staged element: the int32 accumulator, the output value, or (16-bit
    // fixed point) the fp32 value before its segment scale is known
    using ET = std::conditional_t<EPI == 0, int32_t, std::conditional_t<EPI == EPI_FIXED16, float, OutT>>;
};
template <int WN, int EPI, typename OutT>
constexpr int gemm_stage_bytes()
{
    using ET = typename EpiTypes<EPI, OutT>::ET;
    constexpr int NOF = EPI == 2 ? WN / 2 : WN;
    constexpr int FP = NOF < 2 ? NOF : 2;
    return 4 * 32 * (32 * FP * (int)sizeof(ET) + 16);
}

template <int BM, int WN, int EPI, typename OutT, bool FACC = false>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &a, v16i (&acc)[BM / 32][WN], const float *ascale,
                                              const float (&bsc)[WN], unsigned char *stage_base, int rows,
                                              int64_t row0, int nb, int N)
{
    constexpr int MI = BM / 32;
    constexpr int WCOLS = 32 * WN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    auto accv = [](int32_t v) -> float { return FACC ? __int_as_float(v) : (float)v; };
    using ET = typename EpiTypes<EPI, OutT>::ET;
    constexpr int NOF = EPI == 2 ? WN / 2 : WN;          // output fragments of 32 columns
    constexpr int FP = NOF < 2 ? NOF : 2;                 // fragments per pass
    constexpr int ROWB = 32 * FP * (int)sizeof(ET) + 16;  // padded staging row, bytes
    constexpr int CPR = 32 * FP * (int)sizeof(ET) / 16;   // 16-byte chunks per staged row
    unsigned char *stage = stage_base + wave * 32 * ROWB;
    const int ldo = EPI == 2 ? (N >> 1) : N;
    // first output column of this wave's fragment f is ocol0 + 32 f
    const int ocol0 = EPI == 2 ? nb * (4 * WCOLS / 2) + wave * (WCOLS / 2) : nb * (4 * WCOLS) + wave * WCOLS;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int f0 = 0; f0 < NOF; f0 += FP) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int rl = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                const float sa = ascale[mi * 32 + rl];
#pragma unroll
                for (int ff = 0; ff < FP; ++ff) {
                    const int f = f0 + ff;
                    ET val;
                    if constexpr (EPI == 0) {
                        val = acc[mi][f][i];
                    } else if constexpr (EPI == 1) {
                        val = to_out<OutT>((accv(acc[mi][f][i]) * sa) * bsc[f]);
                    } else if constexpr (EPI == EPI_FIXED16) {
                        val = (accv(acc[mi][f][i]) * sa) * bsc[f];
                    } else {
                        const float gate = (accv(acc[mi][f][i]) * sa) * bsc[f];
                        const float up = (accv(acc[mi][NOF + f][i]) * sa) * bsc[NOF + f];
                        // silu(g) = g / (1 + e^-g); the result is rounded to bf16 (or
                        // compared within a tolerance), so the hardware exp and
                        // reciprocal are accurate enough
                        val = to_out<OutT>(gate * up * __builtin_amdgcn_rcpf(1.0f + __expf(-gate)));
                    }
                    *reinterpret_cast<ET *>(stage + rl * ROWB + (32 * ff + (lane & 31)) * (int)sizeof(ET)) = val;
                }
            }
            wave_lds_sync();   // the staging region is this wave's own
            if constexpr (EPI == EPI_FIXED16) {
                // 8 lanes hold one row's 64 columns (8 each): the row's largest
                // magnitude over them fixes a power-of-two scale 2^e that maps it
                // into [2^13, 2^14); codes = rint(v * 2^-e) fit int16 with room,
                // and each lane stores its 8 codes as one 16-byte piece.
                static_assert(CPR == 16, "one 64-column segment per pass");
                constexpr int CPR8 = CPR / 2;   // 8-value pieces per staged row
#pragma unroll
                for (int idx = lane; idx < 32 * CPR8; idx += 64) {
                    const int rl = idx / CPR8, ch = idx % CPR8;
                    const int r = mi * 32 + rl;
                    const int ocol = ocol0 + 32 * f0 + ch * 8;
                    const float4 v0 = *reinterpret_cast<const float4 *>(stage + rl * ROWB + ch * 32);
                    const float4 v1 = *reinterpret_cast<const float4 *>(stage + rl * ROWB + ch * 32 + 16);
                    const float vs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                    float m = 0.0f;
#pragma unroll
                    for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf(vs[u]));
                    // max over the 8-lane row: lane swaps 1 and 2 within quads,
                    // then the mirror within 8 lanes
                    m = fmaxf(m, dpp_move<0xB1>(m));
                    m = fmaxf(m, dpp_move<0x4E>(m));
                    m = fmaxf(m, dpp_move<0x141>(m));
                    int e = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 255u) - 127 - 13 : 0;
                    e = e < -126 ? -126 : e;
                    const float sc = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, exact
                    // rint(v * 2^-e) as an integer: adding 1.5 * 2^23 rounds the
                    // (exact) product half-to-even into the mantissa
                    uint32_t q[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        q[u] = (uint32_t)(__float_as_int(fmaf(vs[u], sc, 12582912.0f)) - 0x4B400000) & 0xffffu;
                    if (r < rows && ocol < ldo) {
                        *reinterpret_cast<uint4 *>(reinterpret_cast<int16_t *>(a.out) + (row0 + r) * ldo + ocol) =
                            make_uint4(q[0] | (q[1] << 16), q[2] | (q[3] << 16), q[4] | (q[5] << 16),
                                       q[6] | (q[7] << 16));
                        if (ch == 0) a.out_exp[(row0 + r) * ((ldo + 63) / 64) + (ocol0 + 32 * f0) / 64] = (int8_t)e;
                    }
                }
            } else {
#pragma unroll
                for (int idx = lane; idx < 32 * CPR; idx += 64) {
                    const int rl = idx / CPR, ch = idx % CPR;
                    const int r = mi * 32 + rl;
                    const int ocol = ocol0 + 32 * f0 + ch * (16 / (int)sizeof(ET));
                    if (r < rows && ocol < ldo)
                        *reinterpret_cast<uint4 *>(reinterpret_cast<ET *>(a.out) + (row0 + r) * ldo + ocol) =
                            *reinterpret_cast<const uint4 *>(stage + rl * ROWB + ch * 16);
                }
            }
            wave_lds_sync();   // the staging region is this wave's own
        }
    }
}

// 16-bit fixed point of y, one 64-column segment of a row at a time: the
// segment's largest magnitude m fixes a power-of-two scale 2^e (e = the
// exponent of m less 13, at least -126) that maps it into [2^13, 2^14); the
// codes rint(v * 2^-e) then fit int16 with room.
__device__ __forceinline__ int fixed16_exponent(float m)
{
    const int e = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 255u) - 127 - 13 : 0;
    return e < -126 ? -126 : e;
}
__device__ __forceinline__ float fixed16_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }   // 2^-e, exact
// rint(v * sc) as a 16-bit two's complement code: adding 1.5 * 2^23 rounds the
// (exact) product half-to-even into the mantissa
__device__ __forceinline__ uint32_t fixed16_code(float v, float sc)
{
    return (uint32_t)(__float_as_int(fmaf(v, sc, 12582912.0f)) - 0x4B400000) & 0xffffu;
}

// Epilogue of one tile straight from registers.  With the weights as the
// MFMA's first operand, lane l holds token row l % 32 of each 32-row block
// and, of each 32-column fragment, columns 8 g + 4 (l / 32) + j in
// acc[..][4 g + j]: four consecutive columns per group g, written as one 8- or
// 16-byte piece.  ascale: the tile's row scales (LDS); csc: this wave's column
// scales (LDS, 32 per fragment).  The 16-bit fixed-point segment of a row
// (two fragments) lies in lanes l and l ^ 32, so its largest magnitude takes
// one lane exchange.  The arithmetic per value is that of gemm_epilogue.
template <int BM, int WN, int EPI, typename OutT>
__device__ __forceinline__ void gemm_epilogue_rows(const GemmArgs &a, v16i (&acc)[BM / 32][WN], const float *ascale,
                                                   const float *csc, int rows, int64_t row0, int nb, int N)
{
    constexpr int MI = BM / 32;
    constexpr int WCOLS = 32 * WN;
    constexpr int NOF = EPI == 2 ? WN / 2 : WN;   // output fragments of 32 columns
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ldo = EPI == 2 ? (N >> 1) : N;
    // first output column of this wave's fragment f is ocol0 + 32 f
    const int ocol0 = EPI == 2 ? nb * (4 * WCOLS / 2) + wave * (WCOLS / 2) : nb * (4 * WCOLS) + wave * WCOLS;
    const int half = 4 * (lane >> 5);
    auto scales4 = [&](int f, int g) { return *reinterpret_cast<const float4 *>(csc + 32 * f + 8 * g + half); };
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int r = mi * 32 + (lane & 31);
        const bool live = r < rows;
        const float sa = EPI != 0 ? ascale[r] : 0.0f;
        const int64_t obase = (row0 + r) * (int64_t)ldo;
        if constexpr (EPI == EPI_FIXED16) {
#pragma unroll
            for (int p = 0; p < NOF; p += 2) {
                float v[2][16];
                float m = 0.0f;
#pragma unroll
                for (int ff = 0; ff < 2; ++ff)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 cs = scales4(p + ff, g);
                        const float c4[4] = {cs.x, cs.y, cs.z, cs.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            v[ff][4 * g + j] = ((float)acc[mi][p + ff][4 * g + j] * sa) * c4[j];
                            m = fmaxf(m, fabsf(v[ff][4 * g + j]));
                        }
                    }
                m = fmaxf(m, __shfl_xor(m, 32));
                const int e = fixed16_exponent(m);
                const float sc = fixed16_scale(e);
#pragma unroll
                for (int ff = 0; ff < 2; ++ff)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int c = ocol0 + 32 * (p + ff) + 8 * g + half;
                        if (live && c < ldo) {
                            const float *vv = &v[ff][4 * g];
                            *reinterpret_cast<uint2 *>(reinterpret_cast<int16_t *>(a.out) + obase + c) =
                                make_uint2(fixed16_code(vv[0], sc) | (fixed16_code(vv[1], sc) << 16),
                                           fixed16_code(vv[2], sc) | (fixed16_code(vv[3], sc) << 16));
                        }
                    }
                if (live && lane < 32 && ocol0 + 32 * p < ldo)
                    a.out_exp[(row0 + r) * ((ldo + 63) / 64) + (ocol0 + 32 * p) / 64] = (int8_t)e;
            }
        } else {
#pragma unroll
            for (int f = 0; f < NOF; ++f)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = ocol0 + 32 * f + 8 * g + half;
                    if (!(live && c < ldo)) continue;
                    int q[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) q[j] = acc[mi][f][4 * g + j];
                    if constexpr (EPI == 0) {
                        *reinterpret_cast<int4 *>(reinterpret_cast<int32_t *>(a.out) + obase + c) =
                            make_int4(q[0], q[1], q[2], q[3]);
                    } else {
                        float o[4];
                        const float4 cs = scales4(f, g);
                        const float c4[4] = {cs.x, cs.y, cs.z, cs.w};
                        if constexpr (EPI == 1) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) o[j] = ((float)q[j] * sa) * c4[j];
                        } else {
                            int u[4];
#pragma unroll
                            for (int j = 0; j < 4; ++j) u[j] = acc[mi][NOF + f][4 * g + j];
                            const float4 cu = scales4(NOF + f, g);
                            const float u4[4] = {cu.x, cu.y, cu.z, cu.w};
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const float gate = ((float)q[j] * sa) * c4[j];
                                const float up = ((float)u[j] * sa) * u4[j];
                                // silu(g) = g / (1 + e^-g), as in gemm_epilogue
                                o[j] = gate * up * __builtin_amdgcn_rcpf(1.0f + __expf(-gate));
                            }
                        }
                        if constexpr (sizeof(OutT) == 4)
                            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + obase + c) =
                                make_float4(o[0], o[1], o[2], o[3]);
                        else
                            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + obase + c) =
                                make_uint2(bf16x2_bits(o[0], o[1]), bf16x2_bits(o[2], o[3]));
                    }
                }
        }
    }
}

// BM rows x (4 waves x WN fragments of 32 columns); DEPTH K steps of B in flight.
// Tiles of up to 128 x 256 run two blocks per CU (two waves per SIMD, at most
// 256 registers per lane, accumulators in VGPRs); 128 x 512 tiles run one.
// Waves per SIMD the kernel is compiled for: three for 64 x 256 tiles (their
// registers fit 168 VGPRs: three blocks per CU overlap one block's start-up
// and epilogue with the others' loops), except the variants that would spill
// there; two for tiles up to 128 x 256; one above.
constexpr int gemm_min_waves(int BM, int WN, int EPI, int out_bytes, bool packed)
{
    if (BM <= 64 && WN == 2 && packed && !(EPI == 2 && out_bytes == 4)) return 3;
    return BM * WN <= 256 ? 2 : 1;
}

// QA: A arrives as bf16 rows (a.A_h, in grouped order) and the tile forms
// their int8 codes itself, with the per-row quantisation of the quantiser
// kernels: the prologue finds each row's largest magnitude over all of K
// (the tile's rows are whole rows of A), and every staged A chunk is coded
// from its bf16 values on the way into LDS.  The tiles of column block 0 also
// store the codes and scales (a.a_codes_out, a.a_scales_out).  Built for the
// down GEMM of few rows per expert, where the weight stream bounds the tile
// and the coding costs no time of its own.
template <int BM, int WN, int DEPTH, int EPI, typename OutT, bool PACKED, bool QA = false>
__global__ __launch_bounds__(G_THREADS) __attribute__((amdgpu_waves_per_eu(gemm_min_waves(BM, WN, EPI, (int)sizeof(OutT), PACKED), 8)))
void grouped_gemm_kernel(GemmArgs a)
{
    static_assert(!QA || (PACKED && BM == 32), "quantise-on-load: packed weights, 32-row tiles");
    static_assert(DEPTH % 2 == 0, "the K loop is unrolled by DEPTH and alternates two LDS buffers");
    static_assert(EPI != 2 || WN % 2 == 0, "SwiGLU pairs gate and up fragments");
    constexpr int MI = BM / 32;      // 32-row MFMA tiles per wave
    constexpr int APASS = BM / 32;   // 16-byte A chunks staged per thread per K step
    constexpr int WCOLS = 32 * WN;   // B rows (output columns) per wave
    // LDS: the two A buffers during the K loop, the epilogue staging after it
    constexpr int SMEM = (2 * BM * G_BK > 4 * 32 * (64 * 4 + 16)) ? 2 * BM * G_BK : 4 * 32 * (64 * 4 + 16);
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    int8_t(*As)[BM * G_BK] = reinterpret_cast<int8_t(*)[BM * G_BK]>(smem);
    __shared__ int32_t arow[BM];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    __shared__ float ascale[BM];

    // ---- which tile (one table load, or from the block index)
    const int bid = blockIdx.x;
    int4 tinfo;
    int kbeg = 0;   // first K step of this tile's slice (dense, split K)
    if (a.dense_rows > 0) {
        if (!dense_tile(bid, a.dense_rows, BM, a.nblocks_n, a.ksplit, &tinfo)) return;
        kbeg = tinfo.x * a.ksteps;
        tinfo.x = 0;
    } else {
        if (bid >= a.tile_prefix[a.G]) return;
        tinfo = a.tiles[bid];
    }
    const int g = tinfo.x, rows = tinfo.z, nb = tinfo.w;
    const int64_t row0 = tinfo.y;
    const int N = (int)a.N, K = (int)a.K;
    const int nk_all = (K + G_BK - 1) / G_BK;
    // steps of this tile: all of K, or its slice (packed B only, so no K
    // masking of A: bytes beyond K meet zero weights)
    const int nk = a.ksplit > 1 ? min(nk_all - kbeg, a.ksteps) : nk_all;

    // ---- B rows (output columns) of this lane, one per fragment
    int col[WN];
    bool cvalid[WN];
    if constexpr (EPI == 2) {
        const int Nh = N >> 1;
        const int hc0 = nb * (4 * WCOLS / 2) + wave * (WCOLS / 2) + (lane & 31);
#pragma unroll
        for (int f = 0; f < WN / 2; ++f) {
            col[f] = hc0 + 32 * f;
            col[WN / 2 + f] = Nh + hc0 + 32 * f;
            cvalid[f] = cvalid[WN / 2 + f] = hc0 + 32 * f < Nh;
        }
    } else {
        const int c0 = nb * (4 * WCOLS) + wave * WCOLS + (lane & 31);
#pragma unroll
        for (int f = 0; f < WN; ++f) {
            col[f] = c0 + 32 * f;
            cvalid[f] = col[f] < N;
        }
    }
    // B is [N][K] row-major, or packed: per 32-row block and 128-byte K step a
    // 4 KiB chunk holding, for sub-step s and lane l, the 16 bytes that lane l
    // feeds to the MFMA (row l%32, bytes 64*(l/32) + 16*s of the step), zero
    // padded in N and K.  Offsets are unsigned: an invalid lane starts at
    // OOB_BASE, above every resource size, and stays out of range as steps are
    // added, so its loads return zeros.
    const int64_t b_bytes = PACKED ? (int64_t)((N + 31) / 32) * nk_all * 4096 : (int64_t)N * K;
    const bool xg = g >= a.G_routed;   // the extra group: weights of its own
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(xg ? a.B_extra : a.B + (int64_t)g * b_bytes, b_bytes);
    const float *bsg = xg ? a.b_extra_scales : a.b_scales + (int64_t)g * N;
    const __amdgpu_buffer_rsrc_t rA =
        QA ? make_rsrc(a.A_h, 2 * a.A_bytes) : make_rsrc(a.A, a.A_bytes);   // QA: bf16 rows
    const int khalf = 64 * (lane >> 5);
    uint32_t boff[WN];
#pragma unroll
    for (int f = 0; f < WN; ++f)
        boff[f] = !cvalid[f] ? OOB_BASE
                             : (PACKED ? (uint32_t)(((col[f] >> 5) * nk_all + kbeg) * 4096 + lane * 16)
                                       : (uint32_t)(col[f] * K + khalf));
    constexpr uint32_t BSTEP = PACKED ? 4096 : G_BK, BSUB = PACKED ? 1024 : 16;

    // per-column weight scales, kept in registers for the epilogue
    float bsc[WN];
#pragma unroll
    for (int f = 0; f < WN; ++f) bsc[f] = (EPI != 0 && cvalid[f]) ? bsg[col[f]] : 0.0f;

    // ---- activation rows of the tile: the gathered row index is loaded
    // first (used after the weight loads below are issued)
    const bool has_row = tid < BM && tid < rows;
    int32_t graw = 0;
    if (has_row && a.gather) graw = a.gather[row0 + tid];

    // ---- A staging assignment: 16-byte chunk ac of rows (tid/8) + 32j
    const int ac = tid & 7;
    uint32_t aoff[APASS];
    int arr[APASS];

    // Software pipeline over K steps of 128 bytes.  A ring of DEPTH register
    // slots holds the B fragments of the next DEPTH steps and the A chunks of
    // the steps after the current one; A(j) sits in slot j % DEPTH from its
    // load (DEPTH steps ahead) until it is copied into LDS at the end of step
    // j - 1.  LDS holds two A buffers (current step, next step).
    v4i breg[DEPTH][WN][4];
    constexpr int AH = QA ? 2 : 1;   // 16-byte loads per A chunk (bf16 rows: two)
    v4i areg[DEPTH][APASS][AH];
    v16i acc[MI][WN];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int f = 0; f < WN; ++f)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][f][i] = 0;
    // QA: this thread's row scale s, its reciprocal and the fast-quotient flag
    // (the quantiser's arithmetic, quant_common.h), and whether this tile
    // stores the codes
    float qs = 0.0f, qy = 0.0f;
    bool qfast = true;
    int32_t qrow = -1;   // the grouped row this thread stages (QA: one per thread)
    const bool qstore = QA && nb == 0;

    // Steps at or beyond nk (the padding of the trip count) load nothing: the
    // step index is wave-uniform, so that choice is a scalar select.  With
    // packed (zero-padded) weights the K tail needs no masking of A: whatever
    // A bytes lie beyond K meet zero weights.
    auto load_b_sub = [&](int slot, int it, int s) {
        const bool live = it < nk;
        const bool kin = PACKED || it * G_BK + khalf + 16 * s < K;
#pragma unroll
        for (int f = 0; f < WN; ++f)
            breg[slot][f][s] = buf_load16(rB, (live && kin) ? boff[f] + it * BSTEP + s * BSUB : OOB_BASE);
    };
    auto load_b = [&](int slot, int it) {
#pragma unroll
        for (int s = 0; s < 4; ++s) load_b_sub(slot, it, s);
    };
    auto load_a = [&](int slot, int it) {
        const bool live = it < nk;
        const bool kin = PACKED || it * G_BK + 16 * ac < K;
#pragma unroll
        for (int j = 0; j < APASS; ++j)
#pragma unroll
            for (int h = 0; h < AH; ++h)   // QA: element offsets, two bytes each
                areg[slot][j][h] = buf_load16(
                    rA, (live && kin && aoff[j] != OOB_BASE) ? (aoff[j] + it * G_BK) * AH + 16 * h : OOB_BASE);
    };
    // A(it) from register slot `slot` into LDS buffer `buf`; with QA its 16
    // bf16 values per chunk are coded first (bytes past K meet zero weights,
    // so whatever they code to does not matter, and they are not stored)
    auto store_a = [&](int slot, int buf, int it) {
#pragma unroll
        for (int j = 0; j < APASS; ++j) {
            v4i v = areg[slot][j][0];
            if constexpr (QA) {
                uint2 c[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float f[8];
                    const v4i u = areg[slot][j][h];
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        f[2 * w] = __uint_as_float((uint32_t)u[w] << 16);
                        f[2 * w + 1] = __uint_as_float((uint32_t)u[w] & 0xffff0000u);
                    }
                    c[h] = qs != 0.0f ? pack8(f, qs, qy, qfast) : make_uint2(0u, 0u);
                }
                v = v4i{(int)c[0].x, (int)c[0].y, (int)c[1].x, (int)c[1].y};
                const int kc = it * G_BK + 16 * ac;
                if (qstore && qrow >= 0 && it < nk && kc < K)
                    *reinterpret_cast<v4i *>(a.a_codes_out + (int64_t)qrow * K + kc) = v;
            }
            *reinterpret_cast<v4i *>(&As[buf][arr[j] * G_BK + ((ac ^ (arr[j] & 7)) << 4)]) = v;
        }
    };

    // Prologue.  Three memory round trips lie on its path: the tile's
    // descriptor, the gathered row indices, then the first A steps.  The
    // first DEPTH weight steps (which need only the descriptor) fly beside
    // the row-index gather, the row scales beside the A loads; the row scales
    // reach LDS after the first A step, and the loop's barriers publish them
    // before the epilogue reads them.  QA (rows not gathered): the rows follow
    // from the descriptor, so the weights, the first A steps and the rows'
    // largest magnitudes are all loaded at once (two round trips).
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_b(d, d);
    float as_reg = 0.0f;
    if constexpr (QA) {
        arr[0] = tid >> 3;   // one 32-row block: one A chunk per thread
        qrow = arr[0] < rows ? (int32_t)(row0 + arr[0]) : -1;
        aoff[0] = qrow >= 0 ? (uint32_t)(qrow * K + 16 * ac) : OOB_BASE;
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load_a(d, d);
        // the largest magnitude of row qrow (the row this thread stages): its
        // 8 threads read 8 elements each per 64-element pass, QB loads in
        // flight per thread (rows of up to 768 in one round trip), then a max
        // over the 8 lanes
        constexpr int QB = 12;
        float m = 0.0f;
        for (int c0 = 8 * ac; c0 < K; c0 += 64 * QB) {
            v4i u[QB];
#pragma unroll
            for (int q = 0; q < QB; ++q) {
                const int c = c0 + 64 * q;
                u[q] = buf_load16(rA, (qrow >= 0 && c < K) ? (uint32_t)(qrow * K + c) * 2u : OOB_BASE);
            }
#pragma unroll
            for (int q = 0; q < QB; ++q)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    m = fmaxf(m, fmaxf(fabsf(__uint_as_float((uint32_t)u[q][w] << 16)),
                                       fabsf(__uint_as_float((uint32_t)u[q][w] & 0xffff0000u))));
        }
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        qs = m / 127.0f;
        qy = qs > 0.0f ? 1.0f / qs : 0.0f;
        qfast = qs >= QUANT_FAST_MIN_SCALE;
        if (ac == 0) {
            ascale[arr[0]] = qs;
            if (qstore && qrow >= 0) a.a_scales_out[qrow] = qs;
        }
    } else {
        const int32_t src = !has_row ? -1 : (a.gather ? graw / a.gather_div : (int32_t)(row0 + tid));
        if (tid < BM) arow[tid] = src;
        __syncthreads();
        as_reg = (EPI != 0 && tid < BM && src >= 0) ? a.a_scales[src] : 0.0f;
#pragma unroll
        for (int j = 0; j < APASS; ++j) {
            arr[j] = (tid >> 3) + 32 * j;
            const int32_t sr = arow[arr[j]];
            aoff[j] = sr >= 0 ? (uint32_t)(sr * K + kbeg * G_BK + 16 * ac) : OOB_BASE;
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load_a(d, d);
    }
    store_a(0, 0, 0);
    if (!QA && tid < BM) ascale[tid] = as_reg;
    load_a(0, DEPTH);
    __syncthreads();

    // The trip count is padded to a multiple of DEPTH; the padding steps issue
    // only out-of-range (zero, no traffic) loads.  Loads are never inside a
    // branch, so the compiler counts outstanding loads exactly and each wait
    // covers only the data it needs.  The last row tile of a group is usually
    // ragged: with RAGGED the MFMAs of the 32-row blocks that hold no row are
    // skipped (ma is uniform over the block, so each test is a scalar branch).
    // The tests split the step into blocks that scheduling groups cannot span,
    // which costs more than it saves with four fragments per wave (16 MFMAs
    // per sub-step); those tiles keep the fixed issue order.  A second copy of
    // the loop in one kernel makes the register allocator spill, so the choice
    // is per instantiation.
    constexpr bool RAGGED = MI > 1 && WN == 2;
    const int ma = (rows + 31) >> 5;
    const int nk_pad = (nk + DEPTH - 1) / DEPTH * DEPTH;
    {
        for (int it0 = 0; it0 < nk_pad; it0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int it = it0 + d;
                // Padding steps (it >= nk) multiply zeros: their A rows and B
                // fragments were loaded out of range.  Each sub-step's B
                // registers are refilled with step it + DEPTH as soon as its
                // MFMAs are issued, so the weight loads are spread through the
                // step.
                const int8_t *Ab = As[d & 1];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi) {
                        const int r = mi * 32 + (lane & 31);
                        const int ch = 4 * (lane >> 5) + s;
                        const v4i av = *reinterpret_cast<const v4i *>(Ab + r * G_BK + ((ch ^ (r & 7)) << 4));
                        if (!RAGGED || mi == 0 || mi < ma) {
#pragma unroll
                            for (int f = 0; f < WN; ++f)
                                acc[mi][f] =
                                    __builtin_amdgcn_mfma_i32_32x32x32_i8(av, breg[d][f][s], acc[mi][f], 0, 0, 0);
                        }
                    }
                    load_b_sub(d, it + DEPTH, s);
                }
                const int dn = (d + 1) % DEPTH;
                store_a(dn, (d + 1) & 1, it + 1);   // A(it+1), loaded DEPTH steps ago
                load_a(dn, it + 1 + DEPTH);
                if constexpr (!RAGGED) {
                    // issue order of the step: per sub-step the A fragment
                    // reads, its MFMAs, then the refill of its B registers;
                    // then the A staging
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        __builtin_amdgcn_sched_group_barrier(0x100, MI, 0);        // LDS reads
                        __builtin_amdgcn_sched_group_barrier(0x008, MI * WN, 0);   // MFMAs
                        __builtin_amdgcn_sched_group_barrier(0x020, WN, 0);        // B loads
                    }
                    __builtin_amdgcn_sched_group_barrier(0x200, APASS, 0);         // LDS stores
                    __builtin_amdgcn_sched_group_barrier(0x020, APASS, 0);         // A loads
                }
                __syncthreads();
            }
        }
    }

    __syncthreads();   // every wave is done with the A buffers
    static_assert(gemm_stage_bytes<WN, EPI, OutT>() <= (int)sizeof(smem), "epilogue staging exceeds the LDS buffer");
    if constexpr (EPI == 0) {
        if (a.ksplit > 1) {   // this slice's int32 sums
            GemmArgs as = a;
            as.out = reinterpret_cast<int32_t *>(a.out) + (int64_t)(kbeg / a.ksteps) * a.M_total * N;
            gemm_epilogue<BM, WN, EPI, OutT>(as, acc, ascale, bsc, smem, rows, row0, nb, N);
            return;
        }
    }
    gemm_epilogue<BM, WN, EPI, OutT>(a, acc, ascale, bsc, smem, rows, row0, nb, N);
}

// The same tiles and results as grouped_gemm_kernel, for the 128 x 512 tiles
// (one block per CU, every register taken by the accumulators and the B ring).
// There the A staging registers are better spent on A fragments: the A steps
// go from memory straight into a ring of three LDS buffers, each sub-step's A
// fragments are read one sub-step ahead so that no MFMA waits on LDS, and a
// step has one barrier.  The weights are the MFMAs' first operand, so a lane
// ends with four consecutive output columns per group and the epilogue writes
// from registers (gemm_epilogue_rows), with no staging and no barrier.  On the
// narrower tiles, which run two or three blocks per CU, the extra registers of
// this loop cost more than it saves, and the 16-bit fixed-point output is
// written faster in rows staged through LDS.
template <int BM, int WN, int DEPTH, int EPI, typename OutT, bool PACKED>
__global__ __launch_bounds__(G_THREADS) __attribute__((amdgpu_waves_per_eu(1, 8)))
void grouped_gemm_ring_kernel(GemmArgs a)
{
    static_assert(WN == 4 && EPI != EPI_FIXED16, "built for the 128 x 512 tiles");
    static_assert(DEPTH % 2 == 0, "the K loop is unrolled by DEPTH");
    constexpr int MI = BM / 32;      // 32-row MFMA tiles per wave
    constexpr int WCOLS = 32 * WN;   // B rows (output columns) per wave
    // LDS: the ring of A_BUFS A buffers of the K loop
    constexpr int A_BUFS = 3;
    constexpr int ABUF = BM * G_BK;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[A_BUFS * ABUF];
    __shared__ int32_t arow[BM];
    // each wave's column scales, fragment-major (32 per fragment)
    __shared__ __attribute__((aligned(16))) float csc[4 * WCOLS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    __shared__ float ascale[BM];

    // ---- which tile (one table load, or from the block index)
    const int bid = blockIdx.x;
    int4 tinfo;
    int kbeg = 0;   // first K step of this tile's slice (dense, split K)
    if (a.dense_rows > 0) {
        if (!dense_tile(bid, a.dense_rows, BM, a.nblocks_n, a.ksplit, &tinfo)) return;
        kbeg = tinfo.x * a.ksteps;
        tinfo.x = 0;
    } else {
        if (bid >= a.tile_prefix[a.G]) return;
        tinfo = a.tiles[bid];
    }
    const int g = tinfo.x, rows = tinfo.z, nb = tinfo.w;
    const int64_t row0 = tinfo.y;
    const int N = (int)a.N, K = (int)a.K;
    const int nk_all = (K + G_BK - 1) / G_BK;
    // steps of this tile: all of K, or its slice (packed B only, so no K
    // masking of A: bytes beyond K meet zero weights)
    const int nk = a.ksplit > 1 ? min(nk_all - kbeg, a.ksteps) : nk_all;

    // ---- B rows (output columns) of this lane, one per fragment
    int col[WN];
    bool cvalid[WN];
    if constexpr (EPI == 2) {
        const int Nh = N >> 1;
        const int hc0 = nb * (4 * WCOLS / 2) + wave * (WCOLS / 2) + (lane & 31);
#pragma unroll
        for (int f = 0; f < WN / 2; ++f) {
            col[f] = hc0 + 32 * f;
            col[WN / 2 + f] = Nh + hc0 + 32 * f;
            cvalid[f] = cvalid[WN / 2 + f] = hc0 + 32 * f < Nh;
        }
    } else {
        const int c0 = nb * (4 * WCOLS) + wave * WCOLS + (lane & 31);
#pragma unroll
        for (int f = 0; f < WN; ++f) {
            col[f] = c0 + 32 * f;
            cvalid[f] = col[f] < N;
        }
    }
    // B is [N][K] row-major, or packed: per 32-row block and 128-byte K step a
    // 4 KiB chunk holding, for sub-step s and lane l, the 16 bytes that lane l
    // feeds to the MFMA (row l%32, bytes 64*(l/32) + 16*s of the step), zero
    // padded in N and K.  Offsets are unsigned: an invalid lane starts at
    // OOB_BASE, above every resource size, and stays out of range as steps are
    // added, so its loads return zeros.
    const int64_t b_bytes = PACKED ? (int64_t)((N + 31) / 32) * nk_all * 4096 : (int64_t)N * K;
    const bool xg = g >= a.G_routed;   // the extra group: weights of its own
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(xg ? a.B_extra : a.B + (int64_t)g * b_bytes, b_bytes);
    const float *bsg = xg ? a.b_extra_scales : a.b_scales + (int64_t)g * N;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.A, a.A_bytes);
    const int khalf = 64 * (lane >> 5);
    uint32_t boff[WN];
#pragma unroll
    for (int f = 0; f < WN; ++f)
        boff[f] = !cvalid[f] ? OOB_BASE
                             : (PACKED ? (uint32_t)(((col[f] >> 5) * nk_all + kbeg) * 4096 + lane * 16)
                                       : (uint32_t)(col[f] * K + khalf));
    constexpr uint32_t BSTEP = PACKED ? 4096 : G_BK, BSUB = PACKED ? 1024 : 16;

    // ---- A staging: the A tile of a K step (BM rows x 128 bytes) goes from
    // memory straight into an LDS buffer, AD 1 KiB transfers per wave (8 rows
    // each, lane l writes bytes 16l..16l+15 of its transfer).  The buffer keeps
    // a row's 16-byte chunk ch at slot ch ^ (row & 7), so lane l fetches chunk
    // (l & 7) ^ ((l >> 3) & 7) of row 8 * transfer + (l >> 3): the swizzle is in
    // the source addresses, and the fragment reads below hit distinct banks.
    constexpr int AD = BM / 32;
    const int ach = (lane & 7) ^ ((lane >> 3) & 7);
    uint32_t aoff[AD];
    const uint32_t lds_a = (uint32_t)(uintptr_t)(lds_u8_t *)&smem[0];

    // Software pipeline over K steps of 128 bytes.  B fragments go to a ring
    // of DEPTH register slots (step j in slot j % DEPTH, loaded DEPTH steps
    // ahead, one sub-step's fragments refilled right after that sub-step's
    // MFMAs); A steps go to a ring of three LDS buffers (step j in buffer
    // j % 3, loaded three steps ahead).  The A fragments of a sub-step are read
    // from LDS one sub-step ahead, into the other of two register sets, so the
    // matrix cores never wait on an LDS read.  Each step has one barrier,
    // between its sub-steps 2 and 3: before it every wave waits for its own
    // transfer of the next step's A and for its fragment reads of this step;
    // after it the next step's A is complete in LDS and this step's buffer is
    // free, so the transfer of step + 3 into it is issued there.
    v4i breg[DEPTH][WN][4];
    v16i acc[MI][WN];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int f = 0; f < WN; ++f)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][f][i] = 0;

    // Steps at or beyond nk (the padding of the trip count) load nothing: the
    // step index is wave-uniform, so that choice is a scalar select.  With
    // packed (zero-padded) weights the K tail needs no masking of A: whatever
    // A bytes lie beyond K meet zero weights.
    auto load_b_sub = [&](int slot, int it, int s) {
        const bool live = it < nk;
        const bool kin = PACKED || it * G_BK + khalf + 16 * s < K;
#pragma unroll
        for (int f = 0; f < WN; ++f)
            breg[slot][f][s] = buf_load16(rB, (live && kin) ? boff[f] + it * BSTEP + s * BSUB : OOB_BASE);
    };
    auto load_a = [&](int it) {
        const bool live = it < nk;
        const bool kin = PACKED || it * G_BK + 16 * ach < K;
        const uint32_t dst = lds_a + (uint32_t)((it % A_BUFS) * ABUF + wave * AD * 1024);
#pragma unroll
        for (int j = 0; j < AD; ++j)
            lds_load16(rA, (live && kin) ? aoff[j] + it * G_BK : OOB_BASE,
                       __builtin_amdgcn_readfirstlane(dst + j * 1024));
    };
    v4i av[2][MI];
    auto read_a = [&](int set, int it, int s) {
        const int8_t *Ab = reinterpret_cast<const int8_t *>(smem) + (it % A_BUFS) * ABUF;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int r = mi * 32 + (lane & 31);
            const int ch = 4 * (lane >> 5) + s;
            av[set][mi] = *reinterpret_cast<const v4i *>(Ab + r * G_BK + ((ch ^ (r & 7)) << 4));
        }
    };
    // Every 32-row block of the tile is multiplied, ragged tiles included:
    // skipping the empty blocks (a branch per block, or a loop copy per count
    // of occupied blocks) measured slower on these tiles.
    auto mfma_sub = [&](int set, int d, int s) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int f = 0; f < WN; ++f)
                acc[mi][f] = __builtin_amdgcn_mfma_i32_32x32x32_i8(breg[d][f][s], av[set][mi], acc[mi][f], 0, 0, 0);
    };

    // Prologue.  Three memory round trips lie on its path: the tile's
    // descriptor, its gathered row indices, then the first A steps.  The row
    // indices are loaded first; the column scales and the weight steps 0 and
    // 1 (which need only the descriptor) fly beside them, and the row scales
    // beside the A transfers.  Then A0, A1, A2 and B1's last sub-step: a wait
    // for A0 and A1 leaves A2 with as many loads behind it as the loop leaves
    // behind each A transfer (8 WN + AD) when its barrier waits for it.
    const bool has_row = tid < BM && tid < rows;
    int32_t graw = 0;
    if (has_row && a.gather) graw = a.gather[row0 + tid];   // used after the weight loads are issued
    // per-column weight scales, for the epilogue: lane l < 32 holds the
    // scale of column l of each fragment, which the epilogue needs in the
    // lanes that hold that column's outputs
    float cs_reg[WN];
#pragma unroll
    for (int f = 0; f < WN; ++f) cs_reg[f] = (EPI != 0 && lane < 32 && cvalid[f]) ? bsg[col[f]] : 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) load_b_sub(0, 0, s);
#pragma unroll
    for (int s = 0; s < 3; ++s) load_b_sub(1 % DEPTH, 1, s);
    const int32_t src = !has_row ? -1 : (a.gather ? graw / a.gather_div : (int32_t)(row0 + tid));
    if (tid < BM) arow[tid] = src;
    __syncthreads();
    const float as_reg = (EPI != 0 && tid < BM && src >= 0) ? a.a_scales[src] : 0.0f;
#pragma unroll
    for (int j = 0; j < AD; ++j) {
        const int32_t sr = arow[(wave * AD + j) * 8 + (lane >> 3)];
        aoff[j] = sr >= 0 ? (uint32_t)(sr * K + kbeg * G_BK + 16 * ach) : OOB_BASE;
    }
    load_a(0);
    load_a(1);
    load_a(2);
    load_b_sub(1 % DEPTH, 1, 3);
    static_assert(DEPTH == 2, "the prologue's issue order assumes a two-step B ring");
    constexpr int VM_AFTER = 8 * WN + AD;   // loads issued behind an A transfer until its barrier
    static_assert(VM_AFTER + AD <= 63, "vmcnt holds at most 63 outstanding loads");
    lds_barrier<AD + WN>();   // A0 and A1 complete (A2 and B1's last sub-step may fly)
    // the scales into LDS for the epilogue (the loop's barriers publish them)
    float *cscw = csc + wave * WCOLS;
    if (tid < BM) ascale[tid] = as_reg;
    if (lane < 32) {
#pragma unroll
        for (int f = 0; f < WN; ++f) cscw[32 * f + lane] = cs_reg[f];
    }
    read_a(0, 0, 0);

    // The trip count is padded to a multiple of DEPTH; the padding steps issue
    // only out-of-range (zero, no traffic) loads.  B loads are never inside a
    // branch, so the compiler counts outstanding loads exactly and each wait
    // covers only the data it needs (the A transfers it does not see only make
    // its waits a little later than needed).
    const int nk_pad = (nk + DEPTH - 1) / DEPTH * DEPTH;
    for (int it0 = 0; it0 < nk_pad; it0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int it = it0 + d;
            // sub-steps 0-2: fragments of the next sub-step, this one's MFMAs,
            // then the refill of its B registers with step it + DEPTH
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                read_a((s + 1) & 1, it, s + 1);
                mfma_sub(s & 1, d, s);
                load_b_sub(d, it + DEPTH, s);
                __builtin_amdgcn_sched_group_barrier(0x100, MI, 0);        // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, MI * WN, 0);   // MFMAs
                __builtin_amdgcn_sched_group_barrier(0x020, WN, 0);        // B loads
            }
            lds_barrier<VM_AFTER>();   // step it + 1's A is in LDS; buffer it % 3 is free
            load_a(it + A_BUFS);
            read_a(0, it + 1, 0);
            mfma_sub(1, d, 3);
            load_b_sub(d, it + DEPTH, 3);
            __builtin_amdgcn_sched_group_barrier(0x100, MI, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, MI * WN, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, WN, 0);
        }
    }

    // the transfers issued for steps past the end still write LDS: drain them
    // (and every wave's last fragment reads) before the epilogue reuses it
    lds_barrier<0>();
    if constexpr (EPI == 0) {
        if (a.ksplit > 1) {   // this slice's int32 sums
            GemmArgs as = a;
            as.out = reinterpret_cast<int32_t *>(a.out) + (int64_t)(kbeg / a.ksteps) * a.M_total * N;
            gemm_epilogue_rows<BM, WN, EPI, OutT>(as, acc, ascale, cscw, rows, row0, nb, N);
            return;
        }
    }
    gemm_epilogue_rows<BM, WN, EPI, OutT>(a, acc, ascale, cscw, rows, row0, nb, N);
}

// Grouped W4A8 GEMM ("Qwen3-1.7B-W4A8 on Ascend", 4bit weights items 1-2):
// the same tiles and A path as grouped_gemm_kernel, B in the packed W4 layout
// (pack_w4_kernel).  A lane loads 32 bytes of codes per fragment and step and
// unpacks them with a shift and a mask into operands worth 16 times the
// codes.  One 128-column step is exactly one group of the weights, and the
// row r, column c result is
//   sum_g s_g * (sum16_g / 16) - sum_g (s_g * o_g) * xsum_g[r],
// sum16_g the int32 MFMA sum of the step, s_g and o_g the group's scale and
// offset of column c, xsum_g the sum of row r's A codes over the step.  The
// first term is folded into fp32 accumulators after every step (a convert and
// one fma per value); the second is a contraction over the groups, which
// v_mfma_f32_32x32x2_f32 adds into the same accumulators two groups at a
// time (row sums as the A operand, -s*o of the lane's column as B), so it
// costs matrix-core cycles instead of vector ones.  The row sums are formed by
// the threads that stage the A tile.  Columns are scaled per group here; the
// epilogue applies the per-token scale (and SwiGLU).
template <int BM, int WN, int DEPTH, int EPI, typename OutT>
__global__ __launch_bounds__(G_THREADS) __attribute__((amdgpu_waves_per_eu(2, 8)))
void grouped_gemm_w4_kernel(GemmArgs a)
{
    static_assert(DEPTH % 2 == 0, "the K loop is unrolled by DEPTH and alternates two LDS buffers");
    static_assert(EPI == 1 || EPI == 2, "dequantising epilogues only");
    static_assert(EPI != 2 || WN % 2 == 0, "SwiGLU pairs gate and up fragments");
    constexpr int MI = BM / 32;
    constexpr int APASS = BM / 32;
    constexpr int WCOLS = 32 * WN;
    constexpr int SMEM = 2 * BM * G_BK > gemm_stage_bytes<WN, EPI, OutT>() ? 2 * BM * G_BK
                                                                            : gemm_stage_bytes<WN, EPI, OutT>();
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    int8_t(*As)[BM * G_BK] = reinterpret_cast<int8_t(*)[BM * G_BK]>(smem);
    __shared__ int32_t arow[BM];
    __shared__ float ascale[BM];
    __shared__ float xs[4][BM];   // row sums of the staged A codes, a ring of four steps

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int bid = blockIdx.x;
    if (bid >= a.tile_prefix[a.G]) return;
    const int4 tinfo = a.tiles[bid];
    const int g = tinfo.x, rows = tinfo.z, nb = tinfo.w;
    const int64_t row0 = tinfo.y;
    const int N = (int)a.N, K = (int)a.K;
    const int nk = (K + G_BK - 1) / G_BK;

    int col[WN];
    bool cvalid[WN];
    if constexpr (EPI == 2) {
        const int Nh = N >> 1;
        const int hc0 = nb * (4 * WCOLS / 2) + wave * (WCOLS / 2) + (lane & 31);
#pragma unroll
        for (int f = 0; f < WN / 2; ++f) {
            col[f] = hc0 + 32 * f;
            col[WN / 2 + f] = Nh + hc0 + 32 * f;
            cvalid[f] = cvalid[WN / 2 + f] = hc0 + 32 * f < Nh;
        }
    } else {
        const int c0 = nb * (4 * WCOLS) + wave * WCOLS + (lane & 31);
#pragma unroll
        for (int f = 0; f < WN; ++f) {
            col[f] = c0 + 32 * f;
            cvalid[f] = col[f] < N;
        }
    }
    const int64_t b_bytes = (int64_t)((N + 31) / 32) * nk * 2048;
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.B + (int64_t)g * b_bytes, b_bytes);
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.b_gscales + (int64_t)g * N * nk, (int64_t)N * nk * 4);
    const __amdgpu_buffer_rsrc_t rO = make_rsrc(a.b_goffs + (int64_t)g * N * nk, (int64_t)N * nk);
    const uint32_t sstep = (uint32_t)N * 4, ostep = (uint32_t)N;   // bytes per step
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.A, a.A_bytes);
    // byte offsets of the column's codes, step-0 scale and step-0 offset
    uint32_t boff[WN], soff[WN], ooff[WN];
#pragma unroll
    for (int f = 0; f < WN; ++f) {
        boff[f] = cvalid[f] ? (uint32_t)((col[f] >> 5) * nk * 2048 + lane * 32) : OOB_BASE;
        soff[f] = cvalid[f] ? (uint32_t)(col[f] * 4) : OOB_BASE;
        ooff[f] = cvalid[f] ? (uint32_t)col[f] : OOB_BASE;
    }
    float ones[WN];
#pragma unroll
    for (int f = 0; f < WN; ++f) ones[f] = 1.0f;

    if (tid < BM) {
        int32_t src = -1;
        if (tid < rows) src = a.gather ? a.gather[row0 + tid] / a.gather_div : (int32_t)(row0 + tid);
        arow[tid] = src;
        ascale[tid] = src >= 0 ? a.a_scales[src] : 0.0f;
    }
    __syncthreads();
    const int ac = tid & 7;
    uint32_t aoff[APASS];
    int arr[APASS];
#pragma unroll
    for (int j = 0; j < APASS; ++j) {
        arr[j] = (tid >> 3) + 32 * j;
        const int32_t sr = arow[arr[j]];
        aoff[j] = sr >= 0 ? (uint32_t)(sr * K + 16 * ac) : OOB_BASE;
    }

    v4i breg[DEPTH][WN][2];
    float gsc[DEPTH][WN], gof[DEPTH][WN];
    v4i areg[DEPTH][APASS];
    v16f accf[MI][WN];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int f = 0; f < WN; ++f)
#pragma unroll
            for (int i = 0; i < 16; ++i) accf[mi][f][i] = 0.0f;

    auto load_b = [&](int slot, int it) {
        const bool live = it < nk;
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int f = 0; f < WN; ++f)
                breg[slot][f][p] = buf_load16(rB, live ? boff[f] + it * 2048 + p * 16 : OOB_BASE);
#pragma unroll
        for (int f = 0; f < WN; ++f) {
            gsc[slot][f] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rS, live ? soff[f] + it * sstep : OOB_BASE, 0, 0));
            gof[slot][f] =
                (float)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(rO, live ? ooff[f] + it * ostep : OOB_BASE, 0, 0);
        }
    };
    auto load_a = [&](int slot, int it) {
        const bool live = it < nk;
        const bool kin = it * G_BK + 16 * ac < K;
#pragma unroll
        for (int j = 0; j < APASS; ++j)
            areg[slot][j] = buf_load16(rA, (live && kin) ? aoff[j] + it * G_BK : OOB_BASE);
    };
    // the A chunks into LDS, and each row's code sum over step `it` (its 8
    // chunks are staged by 8 neighbouring lanes)
    auto store_a = [&](int slot, int buf, int it) {
#pragma unroll
        for (int j = 0; j < APASS; ++j) {
            const v4i v = areg[slot][j];
            *reinterpret_cast<v4i *>(&As[buf][arr[j] * G_BK + ((ac ^ (arr[j] & 7)) << 4)]) = v;
            int sum = __builtin_amdgcn_sdot4(v[0], 0x01010101, 0, false);
            sum = __builtin_amdgcn_sdot4(v[1], 0x01010101, sum, false);
            sum = __builtin_amdgcn_sdot4(v[2], 0x01010101, sum, false);
            sum = __builtin_amdgcn_sdot4(v[3], 0x01010101, sum, false);
            sum += __shfl_xor(sum, 1, 64);
            sum += __shfl_xor(sum, 2, 64);
            sum += __shfl_xor(sum, 4, 64);
            if (ac == 0) xs[it & 3][arr[j]] = (float)sum;
        }
    };

#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_a(d, d);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_b(d, d);
    store_a(0, 0, 0);
    load_a(0, DEPTH);
    __syncthreads();

    const int nk_pad = (nk + DEPTH - 1) / DEPTH * DEPTH;
    // 32-row blocks that hold rows of this tile: the fold of an empty block
    // (the last row tile of a group is usually ragged), the vector work that
    // bounds this kernel, is skipped (ma is uniform over the block: a scalar
    // branch); its MFMAs and offset term still run on zero rows (guarding
    // them too made the 64-row tiles spill)
    const int ma = (rows + 31) >> 5;
    float so_even[WN];   // -s*o of the even step of the current pair
    for (int it0 = 0; it0 < nk_pad; it0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int it = it0 + d;
            const int8_t *Ab = As[d & 1];
            v16i acs[MI][WN];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                v4i bop[WN];
#pragma unroll
                for (int f = 0; f < WN; ++f) {
                    const v4i P = breg[d][f][s >> 1];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        bop[f][q] = (s & 1) ? (int)((uint32_t)P[q] & 0xf0f0f0f0u)
                                            : (int)(((uint32_t)P[q] << 4) & 0xf0f0f0f0u);
                }
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const int r = mi * 32 + (lane & 31);
                    const int ch = 4 * (lane >> 5) + s;
                    const v4i av = *reinterpret_cast<const v4i *>(Ab + r * G_BK + ((ch ^ (r & 7)) << 4));
#pragma unroll
                    for (int f = 0; f < WN; ++f) {
                        const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                        acs[mi][f] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bop[f], s == 0 ? zero : acs[mi][f],
                                                                           0, 0, 0);
                    }
                }
            }
            // fold the step's sums (one weight group) into the fp32 accumulators
#pragma unroll
            for (int f = 0; f < WN; ++f) {
                const float sc = gsc[d][f] * 0.0625f;
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    if (mi == 0 || mi < ma) {
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            accf[mi][f][i] = fmaf((float)acs[mi][f][i], sc, accf[mi][f][i]);
                    }
            }
            if ((d & 1) == 0) {
#pragma unroll
                for (int f = 0; f < WN; ++f) so_even[f] = -gsc[d][f] * gof[d][f];
            } else {
                // offsets of the pair of groups (it - 1, it): lanes 0-31 carry
                // the even group's row sums and -s*o, lanes 32-63 the odd one's
                const int gl = it - 1 + (lane >> 5);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const float xa = xs[gl & 3][mi * 32 + (lane & 31)];
#pragma unroll
                    for (int f = 0; f < WN; ++f) {
                        const float ob = lane < 32 ? so_even[f] : -gsc[d][f] * gof[d][f];
                        accf[mi][f] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa, ob, accf[mi][f], 0, 0, 0);
                    }
                }
            }
            load_b(d, it + DEPTH);
            const int dn = (d + 1) % DEPTH;
            store_a(dn, (d + 1) & 1, it + 1);
            load_a(dn, it + 1 + DEPTH);
            __syncthreads();
        }
    }
    v16i accb[MI][WN];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int f = 0; f < WN; ++f) accb[mi][f] = __builtin_bit_cast(v16i, accf[mi][f]);
    __syncthreads();   // every wave is done with the A buffers
    gemm_epilogue<BM, WN, EPI, OutT, true>(a, accb, ascale, ones, smem, rows, row0, nb, N);
}

namespace {
// Tile shapes by the average rows per group: decode-like groups (<= 32 rows)
// use 32 x 256 tiles, then 64 x 256 (<= 192), 128 x 256 (<= 384) and 128 x 512
// tiles that reuse each weight byte over more rows and each activation row
// over more columns; the 16-bit fixed-point epilogue stays at 64 x 256 up to
// 384 rows and 128 x 256 above.
struct TileCfg {
    int BM, WN;
};

int gemm_nblocks(int64_t N, int epilogue, int WN);

TileCfg gemm_cfg_groups(int64_t M_total, int G, int epilogue)
{
    const double avg_rows = (double)M_total / (double)G;
    if (avg_rows <= 32.0) return {32, 2};
    if (avg_rows <= 192.0) return {64, 2};
    // the 16-bit fixed-point epilogue does more work per tile: smaller tiles
    // keep it short next to the other block's MFMAs
    if (epilogue == EPI_FIXED16) return avg_rows <= 384.0 ? TileCfg{64, 2} : TileCfg{128, 2};
    if (avg_rows <= 384.0) return {128, 2};
    return {128, 4};
}

// One group (a dense linear): step the tile down while the launch would have
// fewer tiles than two per compute unit (tiles up to 128 x 256 run two blocks
// per CU), keeping at least 64 rows per tile unless the GEMM has at most 256
// rows (decode-sized, where the weight stream, not reuse, sets the time).
TileCfg gemm_cfg(int64_t M_total, int64_t N, int G, int epilogue)
{
    TileCfg c = gemm_cfg_groups(M_total, G, epilogue);
    if (G != 1) return c;
    const TileCfg order[] = {{128, 4}, {128, 2}, {64, 2}, {32, 2}};
    const int last = M_total <= 256 ? 3 : 2;
    int i = 0;
    while (order[i].BM != c.BM || order[i].WN != c.WN) ++i;
    for (; i < last; ++i) {
        const int64_t tiles = (M_total + order[i].BM - 1) / order[i].BM * gemm_nblocks(N, epilogue, order[i].WN);
        if (tiles >= 512) break;
    }
    return order[i];
}

// column blocks per group: 4 waves x WN fragments of 32 B rows; with SwiGLU
// half of them are gate rows and half the matching up rows
int gemm_nblocks(int64_t N, int epilogue, int WN)
{
    const int64_t cols = epilogue == 2 ? N / 2 : N;
    const int64_t per_block = epilogue == 2 ? 4 * 32 * WN / 2 : 4 * 32 * WN;
    return (int)((cols + per_block - 1) / per_block);
}

// upper bound of the tile count over every tile shape and epilogue
int64_t gemm_max_tiles(int64_t M_total, int64_t N, int G)
{
    int64_t most = 0;
    for (const TileCfg c : {TileCfg{32, 2}, TileCfg{64, 2}, TileCfg{128, 2}, TileCfg{128, 4}}) {
        const int nb = std::max(gemm_nblocks(N, 1, c.WN), gemm_nblocks(N, 2, c.WN));
        most = std::max<int64_t>(most, ((M_total + c.BM - 1) / c.BM + G) * nb);
    }
    return most;
}

size_t prefix_bytes(int G) { return ((size_t)(G + 1) * sizeof(int32_t) + 255) & ~(size_t)255; }

template <int BM, int WN, int DEPTH, int EPI, typename OutT, bool PACKED>
void launch_main_kernel(const GemmArgs &ga, dim3 grid, hipStream_t st)
{
    // 128 x 512 tiles: the LDS-ring kernel (the 16-bit fixed-point epilogue,
    // which no tile table pairs with them, keeps the staged kernel)
    if constexpr (WN == 4 && EPI != EPI_FIXED16)
        hipLaunchKernelGGL((grouped_gemm_ring_kernel<BM, WN, DEPTH, EPI, OutT, PACKED>), grid, dim3(G_THREADS), 0, st,
                           ga);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, WN, DEPTH, EPI, OutT, PACKED>), grid, dim3(G_THREADS), 0, st, ga);
}

template <int BM, int WN, int DEPTH, bool PACKED>
hipError_t launch_main_layout(const GemmArgs &ga, int epilogue, int out_dtype, hipStream_t st)
{
    const int64_t max_tiles = ga.dense_rows > 0 ? (ga.M_total + BM - 1) / BM * ga.nblocks_n * ga.ksplit
                                                : ((ga.M_total + BM - 1) / BM + ga.G) * ga.nblocks_n;
    const dim3 grid((unsigned)max_tiles);
    if (epilogue == 0)
        launch_main_kernel<BM, WN, DEPTH, 0, int32_t, PACKED>(ga, grid, st);
    else if (epilogue == 1 && out_dtype == 0)
        launch_main_kernel<BM, WN, DEPTH, 1, uint16_t, PACKED>(ga, grid, st);
    else if (epilogue == 1)
        launch_main_kernel<BM, WN, DEPTH, 1, float, PACKED>(ga, grid, st);
    else if (epilogue == EPI_FIXED16)
        launch_main_kernel<BM, WN, DEPTH, EPI_FIXED16, int16_t, PACKED>(ga, grid, st);
    else if (out_dtype == 0)
        launch_main_kernel<BM, WN, DEPTH, 2, uint16_t, PACKED>(ga, grid, st);
    else
        launch_main_kernel<BM, WN, DEPTH, 2, float, PACKED>(ga, grid, st);
    return hipGetLastError();
}

template <int BM, int WN, int DEPTH>
hipError_t launch_main_cfg(const GemmArgs &ga, int epilogue, int out_dtype, hipStream_t st)
{
    return ga.packed_b ? launch_main_layout<BM, WN, DEPTH, true>(ga, epilogue, out_dtype, st)
                       : launch_main_layout<BM, WN, DEPTH, false>(ga, epilogue, out_dtype, st);
}
}  // namespace

// workspace: tile prefix [G+1] int32 (256-byte aligned), then the tile table
size_t gemm_ws_bytes(int64_t M_total, int64_t N, int G)
{
    return prefix_bytes(G) + (size_t)gemm_max_tiles(M_total, N, G) * sizeof(int4);
}

void gemm_tile_params(int64_t M_total, int64_t N, int G, int epilogue, int *BM, int *nblocks_n)
{
    const TileCfg c = gemm_cfg(M_total, N, G, epilogue);
    *BM = c.BM;
    *nblocks_n = gemm_nblocks(N, epilogue, c.WN);
}

void *gemm_tiles_ptr(void *ws, int G) { return (char *)ws + prefix_bytes(G); }

static hipError_t launch_tilemap_cfg(const int32_t *offsets, int G, int64_t M_total, int64_t N, TileCfg c,
                                     int epilogue, void *ws, hipStream_t st)
{
    const int64_t blocks = std::min<int64_t>((gemm_max_tiles(M_total, N, G) + 255) / 256, 64);
    hipLaunchKernelGGL(gemm_tilemap_kernel, dim3((unsigned)blocks), dim3(256), 0, st, offsets, G, c.BM,
                       gemm_nblocks(N, epilogue, c.WN), (int32_t *)ws, (int4 *)((char *)ws + prefix_bytes(G)),
                       (int32_t)M_total);
    return hipGetLastError();
}

hipError_t launch_gemm_tilemap(const int32_t *offsets, int G, int64_t M_total, int64_t N, int epilogue, void *ws,
                               hipStream_t st)
{
    if (M_total == 0) return hipSuccess;
    return launch_tilemap_cfg(offsets, G, M_total, N, gemm_cfg(M_total, N, G, epilogue), epilogue, ws, st);
}

// ---- W4A8
// Tile shapes: 32 x 256 up to 32 rows per group on average, 64 x 256 above
// (the fp32 accumulators and the step's int32 sums both stay in registers,
// which 128-row tiles would not fit).
static TileCfg gemm_cfg_w4(int64_t M_total, int G)
{
    return (double)M_total / (double)G <= 32.0 ? TileCfg{32, 2} : TileCfg{64, 2};
}

void gemm_tile_params_w4(int64_t M_total, int64_t N, int G, int epilogue, int *BM, int *nblocks_n)
{
    const TileCfg c = gemm_cfg_w4(M_total, G);
    *BM = c.BM;
    *nblocks_n = gemm_nblocks(N, epilogue, c.WN);
}

// Packed W4 buffer: the codes (pack_w4_kernel), then the group scales
// [G][KS][N] fp32 and offsets [G][KS][N] int8, each part 256-byte aligned.
static size_t w4_codes_bytes(int64_t G, int64_t N, int64_t K)
{
    return (size_t)(G * ((N + 31) / 32) * ((K + 127) / 128) * 2048);
}
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
size_t w4_scales_offset(int64_t G, int64_t N, int64_t K) { return align256(w4_codes_bytes(G, N, K)); }
size_t w4_offsets_offset(int64_t G, int64_t N, int64_t K)
{
    return w4_scales_offset(G, N, K) + align256((size_t)(G * ((K + 127) / 128) * N) * 4);
}
size_t packed_w4_bytes(int64_t G, int64_t N, int64_t K)
{
    return w4_offsets_offset(G, N, K) + align256((size_t)(G * ((K + 127) / 128) * N));
}

// scales / offsets [G][N][KS] (as quantised, one row per output channel) to
// step-major [G][KS][N]
__global__ __launch_bounds__(256) void w4_scales_t_kernel(const float *__restrict__ s, const int8_t *__restrict__ o,
                                                          int64_t G, int64_t N, int64_t KS, float *__restrict__ st,
                                                          int8_t *__restrict__ ot)
{
    const int64_t n_all = G * KS * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_all; i += (int64_t)gridDim.x * 256) {
        const int64_t n = i % N, ks = (i / N) % KS, g = i / (N * KS);
        st[i] = s[(g * N + n) * KS + ks];
        ot[i] = o[(g * N + n) * KS + ks];
    }
}

hipError_t launch_pack_w4(const int8_t *B, const float *scales, const int8_t *offs, int64_t G, int64_t N, int64_t K,
                          uint8_t *P, hipStream_t st)
{
    const int64_t nd = (int64_t)w4_codes_bytes(G, N, K) / 4;
    if (nd == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((nd + 255) / 256, 65536);
    hipLaunchKernelGGL(pack_w4_kernel, dim3((unsigned)blocks), dim3(256), 0, st, B, G, N, K, (uint32_t *)P);
    const int64_t KS = (K + 127) / 128;
    const int64_t ns = G * KS * N;
    hipLaunchKernelGGL(w4_scales_t_kernel, dim3((unsigned)std::min<int64_t>((ns + 255) / 256, 16384)), dim3(256), 0,
                       st, scales, offs, G, N, KS, (float *)(P + w4_scales_offset(G, N, K)),
                       (int8_t *)(P + w4_offsets_offset(G, N, K)));
    return hipGetLastError();
}

template <int BM>
static hipError_t launch_w4_bm(const GemmArgs &ga, int epilogue, int out_dtype, hipStream_t st)
{
    const int64_t grid = ((ga.M_total + BM - 1) / BM + ga.G) * ga.nblocks_n;
    const dim3 g((unsigned)grid), b(G_THREADS);
    if (epilogue == 1 && out_dtype == 0)
        hipLaunchKernelGGL((grouped_gemm_w4_kernel<BM, 2, 2, 1, uint16_t>), g, b, 0, st, ga);
    else if (epilogue == 1)
        hipLaunchKernelGGL((grouped_gemm_w4_kernel<BM, 2, 2, 1, float>), g, b, 0, st, ga);
    else if (out_dtype == 0)
        hipLaunchKernelGGL((grouped_gemm_w4_kernel<BM, 2, 2, 2, uint16_t>), g, b, 0, st, ga);
    else
        hipLaunchKernelGGL((grouped_gemm_w4_kernel<BM, 2, 2, 2, float>), g, b, 0, st, ga);
    return hipGetLastError();
}

hipError_t launch_gemm_w4_main(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *gather,
                               int gather_div, const uint8_t *Bp, const int32_t *offsets, int G, int64_t M_total,
                               int64_t N, int64_t K, int epilogue, int out_dtype, void *out, const void *ws,
                               hipStream_t st)
{
    const float *gscales = (const float *)(Bp + w4_scales_offset(G, N, K));
    const int8_t *goffs = (const int8_t *)(Bp + w4_offsets_offset(G, N, K));
    if (M_total == 0) return hipSuccess;
    GemmArgs ga{};
    ga.G_routed = G;
    ga.A = A;
    ga.a_scales = a_scales;
    ga.gather = gather;
    ga.gather_div = gather_div > 0 ? gather_div : 1;
    ga.B = (const int8_t *)Bp;
    ga.b_scales = nullptr;
    ga.b_gscales = gscales;
    ga.b_goffs = goffs;
    ga.offsets = offsets;
    ga.G = G;
    ga.M_total = M_total;
    ga.N = N;
    ga.K = K;
    ga.out = out;
    ga.out_exp = nullptr;
    ga.tile_prefix = (const int32_t *)ws;
    ga.tiles = (const int4 *)((const char *)ws + prefix_bytes(G));
    ga.A_bytes = A_rows * K;
    ga.packed_b = 1;
    const TileCfg c = gemm_cfg_w4(M_total, G);
    ga.nblocks_n = gemm_nblocks(N, epilogue, c.WN);
    return c.BM == 32 ? launch_w4_bm<32>(ga, epilogue, out_dtype, st) : launch_w4_bm<64>(ga, epilogue, out_dtype, st);
}

hipError_t launch_grouped_gemm_w4(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *gather,
                                  int gather_div, const uint8_t *Bp, const int32_t *offsets, int G, int64_t M_total,
                                  int64_t N, int64_t K, int epilogue, int out_dtype, void *out, void *ws,
                                  hipStream_t st)
{
    if (M_total == 0) return hipSuccess;
    hipError_t e = launch_tilemap_cfg(offsets, G, M_total, N, gemm_cfg_w4(M_total, G), epilogue, ws, st);
    if (e != hipSuccess) return e;
    return launch_gemm_w4_main(A, A_rows, a_scales, gather, gather_div, Bp, offsets, G, M_total, N, K, epilogue,
                               out_dtype, out, ws, st);
}

static GemmArgs main_args(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *gather,
                          int gather_div, const int8_t *B, int b_packed, const float *b_scales,
                          const int32_t *offsets, int G, int64_t M_total, int64_t N, int64_t K, void *out,
                          const void *ws, int8_t *out_exp, const int8_t *B_extra, const float *b_extra_scales)
{
    GemmArgs ga{};
    ga.ksplit = 1;
    ga.G_routed = B_extra ? G - 1 : G;
    ga.B_extra = B_extra;
    ga.b_extra_scales = b_extra_scales;
    ga.out_exp = out_exp;
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
    ga.tiles = (const int4 *)((const char *)ws + prefix_bytes(G));
    ga.A_bytes = A_rows * K;
    ga.packed_b = b_packed;
    return ga;
}

hipError_t launch_gemm_main(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *gather,
                            int gather_div, const int8_t *B, int b_packed, const float *b_scales,
                            const int32_t *offsets, int G, int64_t M_total, int64_t N, int64_t K, int epilogue,
                            int out_dtype, void *out, const void *ws, hipStream_t st, int8_t *out_exp,
                            const int8_t *B_extra, const float *b_extra_scales)
{
    if (M_total == 0) return hipSuccess;
    GemmArgs ga = main_args(A, A_rows, a_scales, gather, gather_div, B, b_packed, b_scales, offsets, G, M_total, N, K,
                            out, ws, out_exp, B_extra, b_extra_scales);
    const TileCfg c = gemm_cfg(M_total, N, G, epilogue);
    ga.nblocks_n = gemm_nblocks(N, epilogue, c.WN);
    if (c.BM == 32) return launch_main_cfg<32, 2, 2>(ga, epilogue, out_dtype, st);
    if (c.BM == 64) return launch_main_cfg<64, 2, 2>(ga, epilogue, out_dtype, st);
    if (c.WN == 2) return launch_main_cfg<128, 2, 2>(ga, epilogue, out_dtype, st);
    return launch_main_cfg<128, 4, 2>(ga, epilogue, out_dtype, st);
}

bool gemm_down_fuses_quant(int64_t M_total, int64_t N, int64_t K, int G)
{
    return M_total > 0 && gemm_cfg(M_total, N, G, EPI_FIXED16).BM == 32 && 2 * M_total * K <= INT32_MAX - 256;
}

hipError_t launch_gemm_down_qa(const uint16_t *A_h, int64_t M_total, int8_t *a_codes_out, float *a_scales_out,
                               const int8_t *B, const float *b_scales, const int32_t *offsets, int G, int64_t N,
                               int64_t K, void *out, int8_t *out_exp, const void *ws, hipStream_t st,
                               const int8_t *B_extra, const float *b_extra_scales)
{
    if (M_total == 0) return hipSuccess;
    if (!gemm_down_fuses_quant(M_total, N, K, G)) return hipErrorInvalidValue;
    GemmArgs ga = main_args(nullptr, M_total, nullptr, nullptr, 1, B, 1, b_scales, offsets, G, M_total, N, K, out,
                            ws, out_exp, B_extra, b_extra_scales);
    ga.A_h = A_h;
    ga.a_codes_out = a_codes_out;
    ga.a_scales_out = a_scales_out;
    ga.nblocks_n = gemm_nblocks(N, EPI_FIXED16, 2);
    const dim3 grid((unsigned)(((M_total + 31) / 32 + G) * ga.nblocks_n));
    hipLaunchKernelGGL((grouped_gemm_kernel<32, 2, 2, EPI_FIXED16, int16_t, true, true>), grid, dim3(G_THREADS), 0,
                       st, ga);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *gather,
                               int gather_div, const int8_t *B, int b_packed, const float *b_scales,
                               const int32_t *offsets, int G, int64_t M_total, int64_t N, int64_t K, int epilogue,
                               int out_dtype, void *out, void *ws, hipStream_t st)
{
    hipError_t e = launch_gemm_tilemap(offsets, G, M_total, N, epilogue, ws, st);
    if (e != hipSuccess) return e;
    return launch_gemm_main(A, A_rows, a_scales, gather, gather_div, B, b_packed, b_scales, offsets, G, M_total, N,
                            K, epilogue, out_dtype, out, ws, st);
}

// Split K for dense linears with fewer tiles than half the compute units: as
// many slices of at least four steps as bring the tile count to about 128.  A
// slice saves the weight stream of the steps it drops from a tile (about a
// quarter of a microsecond per 32 KB step) and costs the sum kernel (a few
// microseconds), so K is split only from 24 steps (3072 inputs) up.
static int linear_ksplit(int64_t M, int64_t N, int64_t K, int *ksteps)
{
    const TileCfg c = gemm_cfg(M, N, 1, 1);
    const int64_t tiles = (M + c.BM - 1) / c.BM * gemm_nblocks(N, 1, c.WN);
    const int nk = (int)((K + G_BK - 1) / G_BK);
    int S = 1;
    if (tiles < 128 && nk >= 24) S = (int)std::min<int64_t>(nk / 4, (128 + tiles - 1) / tiles);
    const int steps = (nk + S - 1) / S;
    *ksteps = steps;
    return (nk + steps - 1) / steps;
}

size_t linear_partials_bytes(int64_t M, int64_t N, int64_t K)
{
    int steps;
    const int S = linear_ksplit(M, N, K, &steps);
    return S > 1 ? (size_t)S * (size_t)(M * N) * sizeof(int32_t) : 0;
}

// out[m][n] = ((float)sum_s part[s][m][n] * sx[m]) * s_w[n]: the int32 sums of
// the slices add exactly, so the result equals the unsplit GEMM's bit for bit.
template <typename OT>
__global__ __launch_bounds__(256) void linear_reduce_kernel(const int32_t *__restrict__ part, int S, int64_t M,
                                                            int64_t N, const float *__restrict__ sx,
                                                            const float *__restrict__ sw, OT *__restrict__ out)
{
    const int64_t n4 = M * N / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        int4 acc = reinterpret_cast<const int4 *>(part)[i];
        for (int s = 1; s < S; ++s) {
            const int4 v = reinterpret_cast<const int4 *>(part + (int64_t)s * M * N)[i];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        const int64_t m = (4 * i) / N, n = 4 * i - m * N;
        const float sa = sx[m];
        const float r[4] = {((float)acc.x * sa) * sw[n], ((float)acc.y * sa) * sw[n + 1],
                            ((float)acc.z * sa) * sw[n + 2], ((float)acc.w * sa) * sw[n + 3]};
#pragma unroll
        for (int u = 0; u < 4; ++u) out[4 * i + u] = to_out<OT>(r[u]);
    }
}

hipError_t launch_linear(const int8_t *xq, const float *sx, int64_t M, int64_t K, const int8_t *Bp,
                         const float *b_scales, int64_t N, int out_dtype, void *out, hipStream_t st,
                         int32_t *partials)
{
    if (M == 0) return hipSuccess;
    GemmArgs ga{};
    ga.A = xq;
    ga.a_scales = sx;
    ga.gather_div = 1;
    ga.B = Bp;
    ga.b_scales = b_scales;
    ga.G = 1;
    ga.G_routed = 1;
    ga.M_total = M;
    ga.N = N;
    ga.K = K;
    ga.out = out;
    ga.A_bytes = M * K;
    ga.packed_b = 1;
    ga.dense_rows = (int32_t)M;
    ga.ksplit = partials ? linear_ksplit(M, N, K, &ga.ksteps) : 1;
    const int epi = ga.ksplit > 1 ? 0 : 1;
    if (ga.ksplit > 1) ga.out = partials;
    const TileCfg c = gemm_cfg(M, N, 1, 1);
    ga.nblocks_n = gemm_nblocks(N, 1, c.WN);
    hipError_t e;
    if (c.BM == 32) e = launch_main_cfg<32, 2, 2>(ga, epi, out_dtype, st);
    else if (c.BM == 64) e = launch_main_cfg<64, 2, 2>(ga, epi, out_dtype, st);
    else if (c.WN == 2) e = launch_main_cfg<128, 2, 2>(ga, epi, out_dtype, st);
    else e = launch_main_cfg<128, 4, 2>(ga, epi, out_dtype, st);
    if (e != hipSuccess || ga.ksplit == 1) return e;
    const int64_t blocks = std::min<int64_t>((M * N / 4 + 255) / 256, 2048);
    if (out_dtype == 0)
        hipLaunchKernelGGL(linear_reduce_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st, partials,
                           ga.ksplit, M, N, sx, b_scales, (uint16_t *)out);
    else
        hipLaunchKernelGGL(linear_reduce_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, partials,
                           ga.ksplit, M, N, sx, b_scales, (float *)out);
    return hipGetLastError();
}

size_t packed_weights_bytes(int64_t G, int64_t N, int64_t K) { return (size_t)(G * ((N + 31) / 32) * ((K + 127) / 128) * 4096); }

hipError_t launch_pack_weights(const int8_t *B, int64_t G, int64_t N, int64_t K, int8_t *P, hipStream_t st)
{
    const int64_t n16 = (int64_t)packed_weights_bytes(G, N, K) / 16;
    if (n16 == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 65536);
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, st, B, G, N, K, P);
    return hipGetLastError();
}

}  // namespace w8a8
