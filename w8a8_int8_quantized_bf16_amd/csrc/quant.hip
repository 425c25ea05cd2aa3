// Per-row symmetric int8 quantisation (dynamic per-token activations, and the
// static per-output-channel weights, which are the same computation on the
// rows of a weight matrix): "Qwen3.6-35B-A3B-w8a8 config.json and recipe.yaml"
// walkthrough, quantization_config group_0 "input_activations" / "weights".
//
// scale = amax / 127 (IEEE fp32 divide), code = rint(x / scale) (IEEE fp32
// divide, round half to even), clamped to [-127, 127]; an all-zero row has
// scale 0 and codes 0.
//
// One 64-lane wavefront per row.  Each lane owns 8 consecutive elements of
// every 512-element stripe (16-byte loads of bf16, 32 bytes of fp32), so a
// wave reads 1 KiB of bf16 per instruction, fully coalesced.  Rows of up to
// 512 * MAXC elements are read once and held in registers (all loads issued
// before the max reduction); longer rows are read twice (max pass, then code
// pass; the second read hits L2).
#include "device_common.h"
#include "launch.h"

namespace w8a8 {

__device__ __forceinline__ uint32_t quant_code(float v, float s)
{
    float c = rintf(v / s);
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    return (uint32_t)((int32_t)c) & 0xffu;
}

template <typename T>
__global__ __launch_bounds__(256) void quant_rows_kernel(const T *__restrict__ x, int64_t rows, int64_t cols,
                                                         int64_t ld, int8_t *__restrict__ q,
                                                         float *__restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const T *xr = x + r * ld;
    float amax = 0.0f;
    for (int64_t c = (int64_t)lane * 8; c < cols; c += 512) {
        float v[8];
        load8_f32(xr + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = wave_max(amax);
    const float s = amax / 127.0f;
    if (lane == 0) scales[r] = s;
    int8_t *qr = q + r * cols;
    for (int64_t c = (int64_t)lane * 8; c < cols; c += 512) {
        uint2 packed = make_uint2(0u, 0u);
        if (s != 0.0f) {
            float v[8];
            load8_f32(xr + c, v);
            packed.x = quant_code(v[0], s) | (quant_code(v[1], s) << 8) | (quant_code(v[2], s) << 16) |
                       (quant_code(v[3], s) << 24);
            packed.y = quant_code(v[4], s) | (quant_code(v[5], s) << 8) | (quant_code(v[6], s) << 16) |
                       (quant_code(v[7], s) << 24);
        }
        *reinterpret_cast<uint2 *>(qr + c) = packed;
    }
}

template <typename T, int MAXC>
__global__ __launch_bounds__(256) void quant_rows_reg_kernel(const T *__restrict__ x, int64_t rows, int64_t cols,
                                                             int64_t ld, int8_t *__restrict__ q,
                                                             float *__restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const T *xr = x + r * ld;
    float v[MAXC][8];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int64_t col = (int64_t)lane * 8 + 512 * c;
        if (col < cols) load8_f32(xr + col, v[c]);
        else
#pragma unroll
            for (int i = 0; i < 8; ++i) v[c][i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    amax = wave_max(amax);
    const float s = amax / 127.0f;
    if (lane == 0) scales[r] = s;
    int8_t *qr = q + r * cols;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int64_t col = (int64_t)lane * 8 + 512 * c;
        if (col >= cols) break;
        uint2 packed = make_uint2(0u, 0u);
        if (s != 0.0f) {
            packed.x = quant_code(v[c][0], s) | (quant_code(v[c][1], s) << 8) | (quant_code(v[c][2], s) << 16) |
                       (quant_code(v[c][3], s) << 24);
            packed.y = quant_code(v[c][4], s) | (quant_code(v[c][5], s) << 8) | (quant_code(v[c][6], s) << 16) |
                       (quant_code(v[c][7], s) << 24);
        }
        *reinterpret_cast<uint2 *>(qr + col) = packed;
    }
}

template <typename T>
static void launch_typed(const T *x, int64_t rows, int64_t cols, int64_t ld, int8_t *q, float *scales,
                         hipStream_t st)
{
    dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const int64_t nc = (cols + 511) / 512;
    if (nc <= 1) hipLaunchKernelGGL((quant_rows_reg_kernel<T, 1>), grid, block, 0, st, x, rows, cols, ld, q, scales);
    else if (nc <= 2) hipLaunchKernelGGL((quant_rows_reg_kernel<T, 2>), grid, block, 0, st, x, rows, cols, ld, q, scales);
    else if (nc <= 4) hipLaunchKernelGGL((quant_rows_reg_kernel<T, 4>), grid, block, 0, st, x, rows, cols, ld, q, scales);
    else if (nc <= 8) hipLaunchKernelGGL((quant_rows_reg_kernel<T, 8>), grid, block, 0, st, x, rows, cols, ld, q, scales);
    else hipLaunchKernelGGL(quant_rows_kernel<T>, grid, block, 0, st, x, rows, cols, ld, q, scales);
}

hipError_t launch_quant_rows(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld, int8_t *q,
                             float *scales, hipStream_t st)
{
    if (rows == 0) return hipSuccess;
    if (dtype == 0) launch_typed((const uint16_t *)x, rows, cols, ld, q, scales, st);
    else launch_typed((const float *)x, rows, cols, ld, q, scales, st);
    return hipGetLastError();
}

}  // namespace w8a8
