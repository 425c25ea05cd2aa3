// MoE router: unquantised bf16 gate -> fp32 scores -> top-k -> softmax weights
// ("Qwen3-30B-A3B-Instruct-2507-quantized.w8a8" explainer, sections 3.1-3.3:
// the gate maps the hidden state to one score per expert, softmax, top-8; it
// stays in bf16 because a swapped ranking is a discrete error).
//
// Scores: fp32 fused multiply-add chain over the hidden index, ascending, from
// +0.  The chain order is fixed so that every implementation that follows it
// produces bit-identical scores, and therefore identical expert ids.
//
// Block = 16 tokens x all E (<= 256) experts, 256 threads.  Thread (wave w,
// lane l) owns tokens 4w..4w+3 and experts l, l+64, l+128, l+192: up to 16
// independent chains.  x and W_g are staged through LDS as fp32 in 32-wide
// slices of the hidden dimension.  A token's scores all live in one wavefront,
// so top-k is a wave argmax repeated k times (ties -> lower expert index).
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
        bool taken[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            taken[j] = !(lane + 64 * j < E);
            if (logits_out && !taken[j]) logits_out[t * E + lane + 64 * j] = acc[i][j];
        }
        float m = 0.0f;
        float mysel[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // score of slot lane + 64q
        for (int s = 0; s < k; ++s) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + 64 * j;
                if (!taken[j] && (acc[i][j] > bv || (acc[i][j] == bv && e < bi))) {
                    bv = acc[i][j];
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
            if (lane + 64 * j < E) zsum += expf(acc[i][j] - m);
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
}

hipError_t launch_route_topk(const void *x, int dtype, const uint16_t *wg, int64_t T, int64_t H, int E, int k,
                             int renormalize, int32_t *ids, float *w, float *logits, hipStream_t st)
{
    if (T == 0) return hipSuccess;
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
