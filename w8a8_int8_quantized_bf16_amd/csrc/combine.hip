// Weighted combine of the expert outputs: each token's output is the sum, over
// its k routed slots, of the routing weight times that slot's expert output
// (the top-k experts of the router take part in the token's forward pass:
// "Qwen3-30B-A3B-Instruct-2507-quantized.w8a8" explainer, section 3.1).
//
// One block per token; each thread owns 8 consecutive columns (16-byte bf16
// loads), accumulates the k slots in fp32 in slot order and rounds once.  For
// k <= 8 the k rows' columns are all loaded before the sum starts, so the k
// reads are in flight together rather than one after another.
#include "device_common.h"
#include "launch.h"

namespace w8a8 {

template <typename YT, typename OT, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const YT *__restrict__ y, const float *__restrict__ w,
                                                      const int32_t *__restrict__ pair_pos, int k, int64_t H,
                                                      OT *__restrict__ out)
{
    const int64_t t = blockIdx.x;
    for (int64_t c = (int64_t)threadIdx.x * 8; c < H; c += 256 * 8) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        if constexpr (KMAX > 0) {
            float v[KMAX][8];
            float wj[KMAX];
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (j < k) {
                    wj[j] = w[t * k + j];
                    load8_f32(y + (int64_t)pair_pos[t * k + j] * H + c, v[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (j < k)
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[j], v[j][i], acc[i]);
        } else {
            for (int j = 0; j < k; ++j) {
                const float wj = w[t * k + j];
                const int64_t row = pair_pos[t * k + j];
                float v[8];
                load8_f32(y + row * H + c, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
            }
        }
        store8(out + t * H + c, acc);
    }
}

template <typename YT, typename OT>
static void launch_typed(const YT *y, const float *w, const int32_t *pair_pos, int64_t T, int k, int64_t H, OT *out,
                         hipStream_t st)
{
    dim3 grid((unsigned)T), block(256);
    if (k <= 8) hipLaunchKernelGGL((combine_kernel<YT, OT, 8>), grid, block, 0, st, y, w, pair_pos, k, H, out);
    else hipLaunchKernelGGL((combine_kernel<YT, OT, 0>), grid, block, 0, st, y, w, pair_pos, k, H, out);
}

// y as 16-bit fixed point with a power-of-two exponent per row and 64-column
// segment (the layer's down GEMM epilogue): a thread's 8 columns lie in one
// segment, so each slot contributes w * 2^e * code.
//
// SHARED: the layer's shared expert ("Qwen3-Next-80B-A3B-Instruct in AMCT"
// section 2.2; its gate stays bf16 in the "Qwen3.6-35B-A3B-w8a8" recipe).
// The block first forms the token's gate logit x . w_sg (fp32 fmas over its
// columns, then a wave and a block sum), takes its sigmoid, and after the k
// routed slots adds sigmoid * y of row shared_row0 + t.
// y is read exactly once, after the down GEMM has pushed most of it out of the
// caches: a non-temporal load keeps the stream from evicting what the other
// blocks still use (235B-shaped layer: combine 122 -> 104 us)
__device__ __forceinline__ uint4 load_stream16(const int16_t *p)
{
    typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
    const v4u_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename OT, typename XT, bool SHARED>
__global__ __launch_bounds__(256) void combine_fixed16_kernel(const int16_t *__restrict__ y16,
                                                              const int8_t *__restrict__ y_exp,
                                                              const float *__restrict__ w,
                                                              const int32_t *__restrict__ pair_pos, int k, int64_t H,
                                                              OT *__restrict__ out, const XT *__restrict__ x,
                                                              const uint16_t *__restrict__ w_sg, int64_t shared_row0,
                                                              float *__restrict__ gate_out)
{
    const int64_t t = blockIdx.x;
    const int64_t nseg = (H + 63) / 64;
    float sig = 0.0f;
    if constexpr (SHARED) {
        __shared__ float part_l[4];
        float part = 0.0f;
        for (int64_t c = (int64_t)threadIdx.x * 8; c < H; c += 256 * 8) {
            float xv[8], gv[8];
            load8_f32(x + t * H + c, xv);
            load8_f32(w_sg + c, gv);
#pragma unroll
            for (int i = 0; i < 8; ++i) part = fmaf(xv[i], gv[i], part);
        }
        part = wave_sum(part);
        if ((threadIdx.x & 63) == 0) part_l[threadIdx.x >> 6] = part;
        __syncthreads();
        const float logit = (part_l[0] + part_l[1]) + (part_l[2] + part_l[3]);
        sig = 1.0f / (1.0f + expf(-logit));
        if (threadIdx.x == 0) gate_out[t] = sig;
    }
    for (int64_t c = (int64_t)threadIdx.x * 8; c < H; c += 256 * 8) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        constexpr int KMAX = 8;
        uint4 v[KMAX];
        float sc[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < k) {
                const int64_t row = pair_pos[t * k + j];
                v[j] = load_stream16(y16 + row * H + c);
                sc[j] = ldexpf(w[t * k + j], (int)y_exp[row * nseg + c / 64]);
            }
        }
        uint4 vs;
        float ss = 0.0f;
        if constexpr (SHARED) {
            const int64_t row = shared_row0 + t;
            vs = *reinterpret_cast<const uint4 *>(y16 + row * H + c);
            ss = ldexpf(sig, (int)y_exp[row * nseg + c / 64]);
        }
        for (int j0 = 0; j0 < k; j0 += KMAX) {
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (j0 + j >= k) break;
                if (j0 > 0) {
                    const int64_t row = pair_pos[t * k + j0 + j];
                    v[j] = load_stream16(y16 + row * H + c);
                    sc[j] = ldexpf(w[t * k + j0 + j], (int)y_exp[row * nseg + c / 64]);
                }
                const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = fmaf(sc[j], (float)(int16_t)(u[i] & 0xffffu), acc[2 * i]);
                    acc[2 * i + 1] = fmaf(sc[j], (float)(int16_t)(u[i] >> 16), acc[2 * i + 1]);
                }
            }
        }
        if constexpr (SHARED) {
            const uint32_t u[4] = {vs.x, vs.y, vs.z, vs.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(ss, (float)(int16_t)(u[i] & 0xffffu), acc[2 * i]);
                acc[2 * i + 1] = fmaf(ss, (float)(int16_t)(u[i] >> 16), acc[2 * i + 1]);
            }
        }
        store8(out + t * H + c, acc);
    }
}

template <typename OT, typename XT, bool SHARED>
static void launch_fixed16(const int16_t *y16, const int8_t *y_exp, const float *w, const int32_t *pair_pos,
                           int64_t T, int k, int64_t H, OT *out, const XT *x, const uint16_t *w_sg,
                           int64_t shared_row0, float *gate_out, hipStream_t st)
{
    hipLaunchKernelGGL((combine_fixed16_kernel<OT, XT, SHARED>), dim3((unsigned)T), dim3(256), 0, st, y16, y_exp, w,
                       pair_pos, k, H, out, x, w_sg, shared_row0, gate_out);
}

hipError_t launch_combine_fixed16(const int16_t *y16, const int8_t *y_exp, const float *w, const int32_t *pair_pos,
                                  int64_t T, int k, int64_t H, void *out, int out_dtype, hipStream_t st,
                                  const void *x, const uint16_t *w_sg, float *gate_out)
{
    if (T == 0) return hipSuccess;
    const int64_t r0 = T * k;   // the shared expert's rows follow the routed ones
    if (!w_sg) {
        if (out_dtype == 0)
            launch_fixed16<uint16_t, uint16_t, false>(y16, y_exp, w, pair_pos, T, k, H, (uint16_t *)out, nullptr,
                                                      nullptr, 0, nullptr, st);
        else
            launch_fixed16<float, float, false>(y16, y_exp, w, pair_pos, T, k, H, (float *)out, nullptr, nullptr, 0,
                                                nullptr, st);
    } else if (out_dtype == 0) {
        launch_fixed16<uint16_t, uint16_t, true>(y16, y_exp, w, pair_pos, T, k, H, (uint16_t *)out,
                                                 (const uint16_t *)x, w_sg, r0, gate_out, st);
    } else {
        launch_fixed16<float, float, true>(y16, y_exp, w, pair_pos, T, k, H, (float *)out, (const float *)x, w_sg,
                                           r0, gate_out, st);
    }
    return hipGetLastError();
}

hipError_t launch_combine(const void *y, int y_dtype, const float *w, const int32_t *pair_pos, int64_t T, int k,
                          int64_t H, void *out, int out_dtype, hipStream_t st)
{
    if (T == 0) return hipSuccess;
    if (y_dtype == 0 && out_dtype == 0)
        launch_typed((const uint16_t *)y, w, pair_pos, T, k, H, (uint16_t *)out, st);
    else if (y_dtype == 0)
        launch_typed((const uint16_t *)y, w, pair_pos, T, k, H, (float *)out, st);
    else if (out_dtype == 0)
        launch_typed((const float *)y, w, pair_pos, T, k, H, (uint16_t *)out, st);
    else
        launch_typed((const float *)y, w, pair_pos, T, k, H, (float *)out, st);
    return hipGetLastError();
}

}  // namespace w8a8
