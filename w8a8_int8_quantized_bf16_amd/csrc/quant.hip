// Per-row symmetric int8 quantisation (dynamic per-token activations, and the
// static per-output-channel weights, which are the same computation on the
// rows of a weight matrix): "Qwen3.6-35B-A3B-w8a8 config.json and recipe.yaml"
// walkthrough, quantization_config group_0 "input_activations" / "weights".
//
// scale = amax / 127 (IEEE fp32 divide), code = rint(x / scale) (IEEE fp32
// divide, round half to even), clamped to [-127, 127]; an all-zero row has
// scale 0 and codes 0.
//
// One 64-lane wavefront handles R rows at once (all their loads are issued
// before any reduction, so short rows still keep enough bytes in flight).
// Each lane owns 8 consecutive elements of every 512-element stripe (16-byte
// loads of bf16, 32 bytes of fp32), a wave reading 1 KiB of bf16 per
// instruction, fully coalesced.  Rows of up to 512 * MAXC elements are held in
// registers; longer rows are read twice (max pass, then code pass; the second
// read hits L2).  The row maximum is a DPP reduction inside 16-lane rows plus
// four lane reads.  The per-element code (and the division behind it) is in
// quant_common.h.
#include "device_common.h"
#include "launch.h"
#include "quant_common.h"

namespace w8a8 {

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
    amax = wave_max_nonneg(amax);
    const float s = amax / 127.0f;
    const float y = s > 0.0f ? 1.0f / s : 0.0f;
    const bool fast = s >= QUANT_FAST_MIN_SCALE;
    if (lane == 0) scales[r] = s;
    int8_t *qr = q + r * cols;
    for (int64_t c = (int64_t)lane * 8; c < cols; c += 512) {
        uint2 packed = make_uint2(0u, 0u);
        if (s != 0.0f) {
            float v[8];
            load8_f32(xr + c, v);
            packed = pack8(v, s, y, fast);
        }
        *reinterpret_cast<uint2 *>(qr + c) = packed;
    }
}

template <typename T, int MAXC, int R>
__global__ __launch_bounds__(256) void quant_rows_reg_kernel(const T *__restrict__ x, int64_t rows, int64_t cols,
                                                             int64_t ld, int8_t *__restrict__ q,
                                                             float *__restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (r0 >= rows) return;
    float v[R][MAXC][8];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int64_t col = (int64_t)lane * 8 + 512 * c;
            if (r0 + j < rows && col < cols) load8_f32(x + (r0 + j) * ld + col, v[j][c]);
            else
#pragma unroll
                for (int i = 0; i < 8; ++i) v[j][c][i] = 0.0f;
        }
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t r = r0 + j;
        if (r >= rows) break;
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < MAXC; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[j][c][i]));
        amax = wave_max_nonneg(amax);
        const float s = amax / 127.0f;
        const float y = s > 0.0f ? 1.0f / s : 0.0f;
        const bool fast = s >= QUANT_FAST_MIN_SCALE;
        if (lane == 0) scales[r] = s;
        int8_t *qr = q + r * cols;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int64_t col = (int64_t)lane * 8 + 512 * c;
            if (col >= cols) break;
            const uint2 packed = s != 0.0f ? pack8(v[j][c], s, y, fast) : make_uint2(0u, 0u);
            *reinterpret_cast<uint2 *>(qr + col) = packed;
        }
    }
}

// Rows of 256 * G4 columns with G4 not a power of two (768, 1536: the
// models' expert widths), where 512-wide stripes would leave lanes idle: lane
// l holds the 4-value groups l + 64 g (g < G4), contiguous across the wave.
// Same arithmetic per element as the stripe kernel.
template <typename T>
__device__ __forceinline__ void load4_f32(const T *p, float v[4]);
template <>
__device__ __forceinline__ void load4_f32<uint16_t>(const uint16_t *p, float v[4])
{
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load4_f32<float>(const float *p, float v[4])
{
    const float4 f = *reinterpret_cast<const float4 *>(p);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
}

template <typename T, int G4>
__global__ __launch_bounds__(256) void quant_rows_g4_kernel(const T *__restrict__ x, int64_t rows, int64_t ld,
                                                            int8_t *__restrict__ q, float *__restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    constexpr int64_t cols = 256 * G4;
    float v[G4][4];
#pragma unroll
    for (int g = 0; g < G4; ++g) load4_f32<T>(x + r * ld + 4 * (lane + 64 * g), v[g]);
    float amax = 0.0f;
#pragma unroll
    for (int g = 0; g < G4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(v[g][i]));
    amax = wave_max_nonneg(amax);
    const float s = amax / 127.0f;
    const float y = s > 0.0f ? 1.0f / s : 0.0f;
    const bool fast = s >= QUANT_FAST_MIN_SCALE;
    if (lane == 0) scales[r] = s;
#pragma unroll
    for (int g = 0; g < G4; ++g) {
        uint32_t c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = fast ? quant_code_fma(v[g][i], s, y) : quant_code(v[g][i], s);
        *reinterpret_cast<uint32_t *>(q + r * cols + 4 * (lane + 64 * g)) =
            s != 0.0f ? pack_low_bytes(c[0], c[1], c[2], c[3]) : 0u;
    }
}

template <typename T>
static void launch_typed(const T *x, int64_t rows, int64_t cols, int64_t ld, int8_t *q, float *scales,
                         hipStream_t st)
{
    dim3 block(256);
    const int64_t nc = (cols + 511) / 512;
    auto grid = [&](int R) { return dim3((unsigned)((rows + 4 * R - 1) / (4 * R))); };
    if (cols == 768 && ld % 4 == 0) {
        hipLaunchKernelGGL((quant_rows_g4_kernel<T, 3>), grid(1), block, 0, st, x, rows, ld, q, scales);
        return;
    }
    if (cols == 1536 && ld % 4 == 0) {
        hipLaunchKernelGGL((quant_rows_g4_kernel<T, 6>), grid(1), block, 0, st, x, rows, ld, q, scales);
        return;
    }
    if (nc <= 1) hipLaunchKernelGGL((quant_rows_reg_kernel<T, 1, 4>), grid(4), block, 0, st, x, rows, cols, ld, q, scales);
    else if (nc <= 2) hipLaunchKernelGGL((quant_rows_reg_kernel<T, 2, 1>), grid(1), block, 0, st, x, rows, cols, ld, q, scales);
    else if (nc <= 4) hipLaunchKernelGGL((quant_rows_reg_kernel<T, 4, 1>), grid(1), block, 0, st, x, rows, cols, ld, q, scales);
    else if (nc <= 8) hipLaunchKernelGGL((quant_rows_reg_kernel<T, 8, 1>), grid(1), block, 0, st, x, rows, cols, ld, q, scales);
    else hipLaunchKernelGGL(quant_rows_kernel<T>, grid(1), block, 0, st, x, rows, cols, ld, q, scales);
}

// W4 codes of fp32 weights ("Qwen3-1.7B-W4A8 on Ascend", 4bit weights items
// 1-2: groups of 128 inputs with a scale and an offset, 4-bit two's
// complement).  Per group of one row, over the range [min(w, 0), max(w, 0)]
// (zero stays representable): s = (max - min) / 15, z = rint(-min / s),
// u = clamp(rint(w / s) + z, 0, 15); code u - 8 and offset z - 8, both in
// [-8, 7] (a group of zeros: s = 0, codes and offset 0).  Every division is
// the IEEE fp32 quotient.  One wavefront per (row, group), two columns per
// lane; a short last group reads zeros past the row, which leave the range
// (it always holds 0) unchanged.
__global__ __launch_bounds__(256) void quant_w4_kernel(const float *__restrict__ w, int64_t rows, int64_t cols,
                                                       int8_t *__restrict__ q, float *__restrict__ scales,
                                                       int8_t *__restrict__ offs)
{
    const int lane = threadIdx.x & 63;
    const int64_t ng = (cols + 127) / 128;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= rows * ng) return;
    const int64_t r = unit / ng, g = unit % ng;
    const int64_t c = g * 128 + 2 * lane;   // cols is even: c < cols covers both columns
    float2 v = make_float2(0.0f, 0.0f);
    if (c < cols) v = *reinterpret_cast<const float2 *>(w + r * cols + c);
    const float mx = wave_max_nonneg(fmaxf(fmaxf(v.x, v.y), 0.0f));
    const float nmn = wave_max_nonneg(fmaxf(fmaxf(-v.x, -v.y), 0.0f));   // -min(w, 0)
    const float s = (mx + nmn) / 15.0f;
    int q0 = 0, q1 = 0, o = 0;
    if (s != 0.0f) {
        const float z = rintf(nmn / s);
        const float u0 = fminf(fmaxf(rintf(v.x / s) + z, 0.0f), 15.0f);
        const float u1 = fminf(fmaxf(rintf(v.y / s) + z, 0.0f), 15.0f);
        q0 = (int)u0 - 8;
        q1 = (int)u1 - 8;
        o = (int)z - 8;
    }
    if (c < cols)
        *reinterpret_cast<uint16_t *>(q + r * cols + c) = (uint16_t)((q0 & 0xff) | ((q1 & 0xff) << 8));
    if (lane == 0) {
        scales[r * ng + g] = s;
        offs[r * ng + g] = (int8_t)o;
    }
}

hipError_t launch_quant_w4(const float *w, int64_t rows, int64_t cols, int8_t *q, float *scales, int8_t *offs,
                           hipStream_t st)
{
    const int64_t units = rows * ((cols + 127) / 128);
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_w4_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, st, w, rows, cols, q,
                       scales, offs);
    return hipGetLastError();
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
