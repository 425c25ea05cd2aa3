// Device-side helpers shared by the HIP kernels of the W8A8 MoE library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// bf16 is the upper half of a binary32: widening is exact.
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// Round a finite fp32 to bf16, nearest with ties to even: the bits of
// (u + 0x7fff + bit 16 of u) >> 16.  gfx950 converts in one instruction
// (v_cvt_pk_bf16_f32, two values at a time), which rounds the same way: on the
// GPU it matched that integer formula on 2^25 finite inputs (random bit
// patterns, exact ties with even and odd last bits, subnormals, the largest
// finite values).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// lo in the low half, hi in the high half
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// A lane's 32-bit value moved by a DPP lane pattern (quad permutes, row mirrors).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Maximum of a non-negative value over the wavefront, in every lane: DPP
// swaps within each 16-lane row (xor 1, xor 2, mirror of 8, mirror of 16),
// then the four row maxima read as scalars (non-negative floats order like
// their bit patterns).
__device__ __forceinline__ float wave_max_nonneg(float m)
{
    m = fmaxf(m, dpp_move<0xB1>(m));
    m = fmaxf(m, dpp_move<0x4E>(m));
    m = fmaxf(m, dpp_move<0x141>(m));
    m = fmaxf(m, dpp_move<0x140>(m));
    const uint32_t b = __float_as_uint(m);
    const uint32_t r0 = __builtin_amdgcn_readlane(b, 0), r1 = __builtin_amdgcn_readlane(b, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(b, 32), r3 = __builtin_amdgcn_readlane(b, 48);
    return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// Order this wavefront's LDS accesses: the LDS performs one wave's operations
// in issue order, so a compiler barrier is all it takes for lanes to read
// what other lanes of the same wave wrote before it (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// Exclusive prefix sum over the 256 threads of a block (all must call it);
// *total gets the sum of all 256 values.  sc: 4 ints of LDS scratch, free
// again when the call returns.
__device__ __forceinline__ int block_excl_scan256(int v, int *sc, int *total)
{
    const int wave = threadIdx.x >> 6;
    const int inc = wave_incl_scan(v);
    if ((threadIdx.x & 63) == 63) sc[wave] = inc;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) before += w < wave ? sc[w] : 0;
    *total = sc[0] + sc[1] + sc[2] + sc[3];
    __syncthreads();
    return before + inc - v;
}

// Load 8 consecutive elements (16-byte aligned) widened to fp32.
__device__ __forceinline__ void load8_f32(const uint16_t *p, float v[8])
{
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
    v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xffff0000u);
    v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xffff0000u);
}

__device__ __forceinline__ void load8_f32(const float *p, float v[8])
{
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void store8(uint16_t *p, const float v[8])
{
    uint4 u;
    u.x = bf16x2_bits(v[0], v[1]);
    u.y = bf16x2_bits(v[2], v[3]);
    u.z = bf16x2_bits(v[4], v[5]);
    u.w = bf16x2_bits(v[6], v[7]);
    *reinterpret_cast<uint4 *>(p) = u;
}

__device__ __forceinline__ void store8(float *p, const float v[8])
{
    reinterpret_cast<float4 *>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
