// MoE router: unquantised bf16 gate -> fp32 scores -> top-k -> softmax weights
// ("Qwen3-30B-A3B-Instruct-2507-quantized.w8a8" explainer, sections 3.1-3.3:
// the gate maps the hidden state to one score per expert, softmax, top-8; it
// stays in bf16 because a swapped ranking is a discrete error).
//
// Scores: fp32 fused multiply-add chain over the hidden index, ascending, from
// +0.  The chain order is fixed so that every implementation that follows it
// produces bit-identical scores, and therefore identical expert ids.
//
// Two kernels compute the same chains: route_mfma_kernel for bf16 x (matrix
// cores, below) and route_topk_kernel for fp32 x (vector FMA: a bf16 x fp32
// product is not exact in fp32, so only a true fused multiply-add reproduces
// the chain).  In the vector kernel a block holds 16 tokens x all E (<= 256)
// experts; thread (wave w, lane l) owns tokens 4w..4w+3 and experts l, l+64,
// l+128, l+192, with x and W_g staged through LDS in 32-wide slices of the
// hidden dimension.  Top-k is a wave argmax repeated k times (ties -> lower
// expert index).
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {
constexpr int RT_TOK = 16;   // tokens per block
constexpr int RT_KC = 32;    // hidden slice staged per step
}

template <typename T>
__device__ __forceinline__ float load_elem(const T *p);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p) { return bf16_bits_to_float(*p); }
template <>
__device__ __forceinline__ float load_elem<float>(const float *p) { return *p; }

// Top-k of one token whose E (<= 256) scores sit in one wavefront, lane l
// holding experts l + 64 j in l4[j]: k rounds of a wave argmax (ties -> lower
// expert index), then softmax weights of the selected experts.
__device__ __forceinline__ void select_topk(const float l4[4], int64_t t, int E, int k, int renorm,
                                            int32_t *__restrict__ ids, float *__restrict__ wout,
                                            float *__restrict__ logits_out)
{
    const int lane = threadIdx.x & 63;
    bool taken[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        taken[j] = !(lane + 64 * j < E);
        if (logits_out && !taken[j]) logits_out[t * E + lane + 64 * j] = l4[j];
    }
    float m = 0.0f;
    float mysel[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // score of slot lane + 64q
    for (int s = 0; s < k; ++s) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            if (!taken[j] && (l4[j] > bv || (l4[j] == bv && e < bi))) {
                bv = l4[j];
                bi = e;
            }
        }
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) {
            const float ov = __shfl_xor(bv, msk, 64);
            const int oi = __shfl_xor(bi, msk, 64);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (lane + 64 * j == bi) taken[j] = true;
        if (lane == 0) ids[t * k + s] = bi;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane == (s & 63) && q == (s >> 6)) mysel[q] = bv;
        if (s == 0) m = bv;
    }
    // softmax over all E scores; weights of the selected, optionally renormalised
    float zsum = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (lane + 64 * j < E) zsum += expf(l4[j] - m);
    zsum = wave_sum(zsum);
    float z[4], ssum = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        z[q] = (lane + 64 * q < k) ? expf(mysel[q] - m) : 0.0f;
        ssum += z[q];
    }
    ssum = wave_sum(ssum);
    const float denom = renorm ? ssum : zsum;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (lane + 64 * q < k) wout[t * k + lane + 64 * q] = z[q] / denom;
}

template <typename T>
__global__ __launch_bounds__(256) void route_topk_kernel(const T *__restrict__ x, const uint16_t *__restrict__ wg,
                                                         int64_t T_, int64_t H, int E, int k, int renorm,
                                                         int32_t *__restrict__ ids, float *__restrict__ wout,
                                                         float *__restrict__ logits_out)
{
    __shared__ float xs[RT_TOK][RT_KC];
    __shared__ float wsl[256][RT_KC + 1];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t t0 = (int64_t)blockIdx.x * RT_TOK;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    for (int64_t k0 = 0; k0 < H; k0 += RT_KC) {
        const int kend = (int)((H - k0) < RT_KC ? (H - k0) : RT_KC);
        for (int idx = tid; idx < RT_TOK * RT_KC; idx += 256) {
            const int i = idx / RT_KC, kk = idx % RT_KC;
            const int64_t t = t0 + i;
            xs[i][kk] = (t < T_ && kk < kend) ? load_elem<T>(x + t * H + k0 + kk) : 0.0f;
        }
        for (int idx = tid; idx < E * RT_KC; idx += 256) {
            const int e = idx / RT_KC, kk = idx % RT_KC;
            wsl[e][kk] = kk < kend ? bf16_bits_to_float(wg[(int64_t)e * H + k0 + kk]) : 0.0f;
        }
        __syncthreads();
        for (int kk = 0; kk < kend; ++kk) {
            float xv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = xs[wave * 4 + i][kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (lane + 64 * j < E) {
                    const float wv = wsl[lane + 64 * j][kk];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i][j] = fmaf(xv[i], wv, acc[i][j]);
                }
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + wave * 4 + i;
        if (t >= T_) break;
        select_topk(acc[i], t, E, k, renorm, ids, wout, logits_out);
    }
}

// bf16 activations: the score chains run on the matrix cores.  With bf16
// operands every product is exact in fp32, so one v_mfma_f32_4x4x1_16b step
// (c += a * b, one rounding) is exactly one fused multiply-add of the chain;
// the instruction keeps 16 independent 4x4 outer products.  A wavefront owns
// 4 tokens x 64 experts: lane l feeds token l % 4 and expert 64 s + l, and
// after the H steps holds the scores of tokens 0..3 for expert 64 s + l.
// A block of S x TG wavefronts (S slices of 64 experts, TG groups of 4
// tokens) stages 64-wide hidden slices of W_g and x through LDS (rows padded
// to 144 bytes: the 16-byte reads of 8 consecutive rows hit distinct banks),
// three slices in flight.  Zero padding beyond H or E adds +0 * 0 terms,
// which leave every chain unchanged.
namespace {
constexpr int RM_KC = 64;                  // hidden indices per staged slice
constexpr int RM_ROW = RM_KC * 2 + 16;     // padded LDS row, bytes
constexpr int RM_STAGES = 3;               // slices in flight (registers)
}

template <int S>   // 64-expert slices (E <= 64 S)
__global__ __launch_bounds__(512) void route_mfma_kernel(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ wg, int64_t T_, int64_t H,
                                                         int E, int k, int renorm, int32_t *__restrict__ ids,
                                                         float *__restrict__ wout, float *__restrict__ logits_out)
{
    constexpr int TG = S == 1 ? 8 : (S == 2 ? 4 : 2);   // token groups of 4 per block
    constexpr int NT = 64 * S * TG;                       // threads
    constexpr int WROWS = 64 * S, XROWS = 4 * TG;
    constexpr int WPIECES = WROWS * 8, XPIECES = XROWS * 8;        // 16-byte pieces per slice
    constexpr int WPT = (WPIECES + NT - 1) / NT, XPT = (XPIECES + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) unsigned char wl[2][WROWS * RM_ROW];
    __shared__ __attribute__((aligned(16))) unsigned char xl[2][XROWS * RM_ROW];
    __shared__ float lg[XROWS][WROWS + 1];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tg = wave / S, sl = wave % S;
    const int64_t tb = (int64_t)blockIdx.x * XROWS;
    const int nsl = (int)((H + RM_KC - 1) / RM_KC);

    // buffer resources: an out-of-range offset reads zero without a branch
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x), 0, 0x7ffffff0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(wg), 0, 0x7ffffff0, 0x00020000);
    // staging assignment: piece p = row * 8 + c (16 bytes, hidden 8c..8c+7 of the slice)
    int woff[WPT], xoff[XPT];
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int p = tid + j * NT, row = p >> 3, c = p & 7;
        woff[j] = (p < WPIECES && row < E) ? (int)((int64_t)row * H * 2) + 16 * c : 0x7fffffff;
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
        const int p = tid + j * NT, row = p >> 3, c = p & 7;
        xoff[j] = (p < XPIECES && tb + row < T_) ? (int)((tb + row) * H * 2) + 16 * c : 0x7fffffff;
    }
    uint4 wr[RM_STAGES][WPT], xr[RM_STAGES][XPT];
    auto load = [&](int st, int slc) {
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            const int p = tid + j * NT, c = p & 7;
            const bool ok = woff[j] != 0x7fffffff && slc * RM_KC + 8 * c < H;
            wr[st][j] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? woff[j] + slc * RM_KC * 2 : 0x7fffffff, 0, 0));
        }
#pragma unroll
        for (int j = 0; j < XPT; ++j) {
            const int p = tid + j * NT, c = p & 7;
            const bool ok = xoff[j] != 0x7fffffff && slc * RM_KC + 8 * c < H;
            xr[st][j] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? xoff[j] + slc * RM_KC * 2 : 0x7fffffff, 0, 0));
        }
    };
    auto store = [&](int st, int buf) {
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            const int p = tid + j * NT;
            if (p < WPIECES) *reinterpret_cast<uint4 *>(&wl[buf][(p >> 3) * RM_ROW + 16 * (p & 7)]) = wr[st][j];
        }
#pragma unroll
        for (int j = 0; j < XPT; ++j) {
            const int p = tid + j * NT;
            if (p < XPIECES) *reinterpret_cast<uint4 *>(&xl[buf][(p >> 3) * RM_ROW + 16 * (p & 7)]) = xr[st][j];
        }
    };

#pragma unroll
    for (int st = 0; st < RM_STAGES; ++st) load(st, st);
    store(0, 0);
    load(0, RM_STAGES);
    __syncthreads();

    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const unsigned char *wrow0 = &wl[0][(sl * 64 + lane) * RM_ROW];
    const unsigned char *xrow0 = &xl[0][(tg * 4 + (lane & 3)) * RM_ROW];
    const int nsl_pad = (nsl + RM_STAGES - 1) / RM_STAGES * RM_STAGES;
    for (int s0 = 0; s0 < nsl_pad; s0 += RM_STAGES) {
#pragma unroll
        for (int d = 0; d < RM_STAGES; ++d) {
            const int slc = s0 + d;
            const int buf = slc & 1;
            if (slc < nsl) {
                const unsigned char *wrow = wrow0 + buf * (WROWS * RM_ROW);
                const unsigned char *xrow = xrow0 + buf * (XROWS * RM_ROW);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + 16 * c);
                    const uint4 xv = *reinterpret_cast<const uint4 *>(xrow + 16 * c);
                    const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
                    const uint32_t x4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc = __builtin_amdgcn_mfma_f32_4x4x1f32(__uint_as_float(x4[j] << 16),
                                                                __uint_as_float(w4[j] << 16), acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_4x4x1f32(__uint_as_float(x4[j] & 0xffff0000u),
                                                                __uint_as_float(w4[j] & 0xffff0000u), acc, 0, 0, 0);
                    }
                }
            }
            const int dn = (d + 1) % RM_STAGES;
            store(dn, (slc + 1) & 1);            // slice slc+1, loaded RM_STAGES slices ago
            load(dn, slc + 1 + RM_STAGES);
            __syncthreads();
        }
    }
    // lane l, value i: score of token tb + 4 tg + i for expert 64 sl + l
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[tg * 4 + i][sl * 64 + lane] = acc[i];
    __syncthreads();
    constexpr int NW = S * TG;
    for (int tt = wave; tt < XROWS; tt += NW) {
        const int64_t t = tb + tt;
        if (t >= T_) break;
        float l4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) l4[j] = (j < S) ? lg[tt][lane + 64 * j] : 0.0f;
        select_topk(l4, t, E, k, renorm, ids, wout, logits_out);
    }
}

hipError_t launch_route_topk(const void *x, int dtype, const uint16_t *wg, int64_t T, int64_t H, int E, int k,
                             int renormalize, int32_t *ids, float *w, float *logits, hipStream_t st)
{
    if (T == 0) return hipSuccess;
    if (dtype == 0) {
        const int S = (E + 63) / 64;
        const int TG = S == 1 ? 8 : (S == 2 ? 4 : 2);
        dim3 g((unsigned)((T + 4 * TG - 1) / (4 * TG))), b(64 * S * TG);
        const uint16_t *xb = (const uint16_t *)x;
        switch (S) {
        case 1: hipLaunchKernelGGL(route_mfma_kernel<1>, g, b, 0, st, xb, wg, T, H, E, k, renormalize, ids, w, logits); break;
        case 2: hipLaunchKernelGGL(route_mfma_kernel<2>, g, b, 0, st, xb, wg, T, H, E, k, renormalize, ids, w, logits); break;
        case 3: hipLaunchKernelGGL(route_mfma_kernel<3>, g, b, 0, st, xb, wg, T, H, E, k, renormalize, ids, w, logits); break;
        default: hipLaunchKernelGGL(route_mfma_kernel<4>, g, b, 0, st, xb, wg, T, H, E, k, renormalize, ids, w, logits); break;
        }
        return hipGetLastError();
    }
    dim3 grid((unsigned)((T + RT_TOK - 1) / RT_TOK)), block(256);
    if (dtype == 0)
        hipLaunchKernelGGL(route_topk_kernel<uint16_t>, grid, block, 0, st, (const uint16_t *)x, wg, T, H, E, k,
                           renormalize, ids, w, logits);
    else
        hipLaunchKernelGGL(route_topk_kernel<float>, grid, block, 0, st, (const float *)x, wg, T, H, E, k,
                           renormalize, ids, w, logits);
    return hipGetLastError();
}

}  // namespace w8a8
