// Shared device helpers for the Prox gfx950 kernels (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prox {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (inputs are finite; NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

template <typename T> struct elem;
template <> struct elem<float> {
    static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t *p, int64_t i) { return __uint_as_float((uint32_t)p[i] << 16); }
    static __device__ __forceinline__ void store(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// 16-byte vector of T unpacked to floats: 8 for bf16, 4 for fp32
template <typename T> struct vec16;
template <> struct vec16<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void unpack(const u32x4 &v, float *f)
    {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
};
template <> struct vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void unpack(const u32x4 &v, float *f)
    {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
};

// streaming 16-byte load of data read exactly once (weights, proxy codes)
__device__ __forceinline__ u32x4 ld_stream(const void *p)
{
    return __builtin_nontemporal_load((const u32x4 *)p);
}

// ---------------------------------------------------------------- silu
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ uint32_t wave_and(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v &= (uint32_t)__shfl_xor((int)v, o, kWave);
    return v;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o, kWave);
    return v;
}

// inclusive prefix sum within a wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t t = (uint32_t)__shfl_up((int)v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix sum over the block in thread order; returns the block
// total through *total.  scratch: >= NW uint32 in LDS.  All threads call.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *scratch, uint32_t *total)
{
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    uint32_t incl = wave_incl_scan(v);
    if (lane == kWave - 1) scratch[wid] = incl;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        uint32_t s = scratch[w];
        base += (w < wid) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_and_or(uint32_t a, uint32_t o, uint32_t *scratch, uint32_t *or_out)
{
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    a = wave_and(a);
    o = wave_or(o);
    if (lane == 0) {
        scratch[wid] = a;
        scratch[NW + wid] = o;
    }
    __syncthreads();
    uint32_t ra = 0xFFFFFFFFu, ro = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        ra &= scratch[w];
        ro |= scratch[NW + w];
    }
    __syncthreads();
    *or_out = ro;
    return ra;
}

}  // namespace prox
