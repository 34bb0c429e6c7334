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

// OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinities, largest finite 448).  Encoding: the nearest E4M3 value, ties to
// the even code, magnitudes >= 448 saturating to 448, the sign bit copied
// (so -0 -> 0x80).  Finite inputs only.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v)
{
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < 0.015625f)  // below 2^-6: subnormal steps of 2^-9 (8 -> the least normal, 0x08)
        return sign | (uint32_t)rintf(a * 512.0f);
    // normal: keep 3 mantissa bits of the binary32 value, rounding half to even
    // at bit 20; a carry moves into the exponent field, as it should
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    const uint32_t code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);  // exponent bias 127 -> 7
    return sign | min(code, 0x7Eu);
}

// Four E4M3 codes (byte 0 first) to binary32, by the hardware conversion
// (gfx950 decodes the OCP format).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float *f)
{
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo[0];
    f[1] = lo[1];
    f[2] = hi[0];
    f[3] = hi[1];
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// streaming 16-byte load of data read exactly once (weights, proxy codes)
__device__ __forceinline__ u32x4 ld_stream(const void *p)
{
    return __builtin_nontemporal_load((const u32x4 *)p);
}

// the same for 8 bytes
__device__ __forceinline__ u32x2 ld_stream8(const void *p)
{
    return __builtin_nontemporal_load((const u32x2 *)p);
}

// ------------------------------------------------- cross-workgroup data
// Partial results handed from one workgroup to another within a kernel are
// stored and loaded as relaxed agent-scope atomics: each access is coherent
// across the XCDs' L2 caches on its own, so no release/acquire fence (which
// would write back and invalidate the whole L2) is needed.  The writer waits
// for its stores to complete before taking its ticket (publish_and_ticket).
__device__ __forceinline__ void store_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two consecutive floats (8-byte aligned) as one 64-bit coherent access:
// half the instructions of two 32-bit ones, and the reads cost a fraction.
__device__ __forceinline__ void store_agent2(float *p, float a, float b)
{
    const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void load_agent2(const float *p, float &a, float &b)
{
    const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    a = __uint_as_float((uint32_t)v);
    b = __uint_as_float((uint32_t)(v >> 32));
}

// Batches of coherent loads whose count is only known at run time.  A load
// under a branch is followed by a wait for it (the loads of a batch would
// run one at a time), so the batch goes through a buffer resource instead:
// every load is issued, and one whose offset is at or beyond the resource's
// size reads as zero without a memory access.  The loads carry the same
// device-scope coherence bit as the relaxed agent-scope atomic loads above.
struct CoherentBuf {
    static constexpr int kWord3 = 0x00020000;  // 32-bit data format, untyped access
    static constexpr int kSc1 = 16;            // cache policy: device-scope coherent
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ __forceinline__ CoherentBuf(const void *base, uint32_t bytes)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kWord3))
    {
    }
    // two floats at byte offset `off` (8-byte aligned)
    __device__ __forceinline__ void load2(uint32_t off, float &a, float &b) const
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, (int)off, 0, kSc1);
        a = __uint_as_float(v[0]);
        b = __uint_as_float(v[1]);
    }
    __device__ __forceinline__ float load(uint32_t off) const
    {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)off, 0, kSc1));
    }
};

// Plain 32-bit stores through a buffer resource of `bytes` bytes: a store at
// an offset >= bytes is dropped by the hardware's range check, so a lane that
// must not store passes `bytes` as its offset instead of branching.
struct OutBuf {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t end;
    __device__ __forceinline__ OutBuf(void *base, uint32_t bytes)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, CoherentBuf::kWord3)), end(bytes)
    {
    }
    __device__ __forceinline__ void store(uint32_t off, uint32_t v) const
    {
        __builtin_amdgcn_raw_buffer_store_b32(v, rsrc, (int)off, 0, 0);
    }
};

// All threads call after their store_agent()s.  Returns true in exactly one
// workgroup of the `n` that share `counter`: the last to arrive, which then
// resets the counter for the next use.
__device__ __forceinline__ bool publish_and_ticket(uint32_t *counter, uint32_t n, int *s_flag)
{
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t t = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = (t == n - 1);
        if (t == n - 1) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return *s_flag != 0;
}

// wave-uniform value in a scalar register
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ---------------------------------------------------------------- silu
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// The gate activation h = act(g): 0 = silu (SwiGLU FFNs), 1 = gelu in its
// tanh form (GeGLU FFNs, e.g. the Gemma family).
__device__ __forceinline__ float gate_act(int act, float z)
{
    if (act == 1) return 0.5f * z * (1.0f + tanhf(0.7978845608028654f * (z + 0.044715f * z * z * z)));
    return silu(z);
}

// A channel's salience term for the selection signal: 0 = |h u| (the
// intermediate state), 1 = |h| (gate branch only), 2 = |u| (up branch only).
__device__ __forceinline__ float salience(int signal, int act, float g, float u)
{
    const float h = gate_act(act, g);
    return signal == 1 ? fabsf(h) : (signal == 2 ? fabsf(u) : fabsf(h * u));
}

// ---------------------------------------------------------- reductions
// Cross-lane steps use DPP (row shifts within 16-lane rows, then row
// broadcasts), which run at VALU speed; lane 63 ends with the full result.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dppf(float old, float v)
{
    return __uint_as_float(dpp<CTRL, ROWMASK>(__float_as_uint(old), __float_as_uint(v)));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// inclusive prefix sum within a wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v)
{
    v += dpp<kRowShr1>(0u, v);
    v += dpp<kRowShr2>(0u, v);
    v += dpp<kRowShr4>(0u, v);
    v += dpp<kRowShr8>(0u, v);
    v += dpp<kRowBcast15, 0xA>(0u, v);
    v += dpp<kRowBcast31, 0xC>(0u, v);
    return v;
}

// wave-wide reductions; the result is uniform (scalar)
__device__ __forceinline__ float wave_sum(float v)
{
    v += dppf<kRowShr1>(0.0f, v);
    v += dppf<kRowShr2>(0.0f, v);
    v += dppf<kRowShr4>(0.0f, v);
    v += dppf<kRowShr8>(0.0f, v);
    v += dppf<kRowBcast15, 0xA>(0.0f, v);
    v += dppf<kRowBcast31, 0xC>(0.0f, v);
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

__device__ __forceinline__ uint32_t wave_and(uint32_t v)
{
    v &= dpp<kRowShr1>(~0u, v);
    v &= dpp<kRowShr2>(~0u, v);
    v &= dpp<kRowShr4>(~0u, v);
    v &= dpp<kRowShr8>(~0u, v);
    v &= dpp<kRowBcast15, 0xA>(~0u, v);
    v &= dpp<kRowBcast31, 0xC>(~0u, v);
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v)
{
    v |= dpp<kRowShr1>(0u, v);
    v |= dpp<kRowShr2>(0u, v);
    v |= dpp<kRowShr4>(0u, v);
    v |= dpp<kRowShr8>(0u, v);
    v |= dpp<kRowBcast15, 0xA>(0u, v);
    v |= dpp<kRowBcast31, 0xC>(0u, v);
    return __builtin_amdgcn_readlane(v, 63);
}

// The NW per-wave words at `p` (LDS, 16-byte aligned, NW a multiple of 4)
// read with 16-byte reads, all issued before any is used: a loop of single
// reads would wait for each in turn.
template <int NW>
__device__ __forceinline__ void lds_words(const uint32_t *p, uint32_t (&v)[NW])
{
    static_assert(NW % 4 == 0, "whole 16-byte reads");
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
        const u32x4 q = reinterpret_cast<const u32x4 *>(p)[i];
        v[4 * i] = q.x;
        v[4 * i + 1] = q.y;
        v[4 * i + 2] = q.z;
        v[4 * i + 3] = q.w;
    }
}

// Exclusive prefix sum over the block in thread order; returns the block
// total through *total.  scratch: >= NW uint32 in LDS, 16-byte aligned.  All
// threads call.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *scratch, uint32_t *total)
{
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan(v);
    if (lane == kWave - 1) scratch[wid] = incl;
    __syncthreads();
    uint32_t sw[NW];
    lds_words<NW>(scratch, sw);
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        base += (w < wid) ? sw[w] : 0u;
        tot += sw[w];
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// block_excl_scan, and in the same barrier round the block sum of one
// wave-uniform value per wave (through *wave_sum_out).  scratch: >= 2 NW.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_and_sum(uint32_t v, uint32_t wave_val, uint32_t *scratch,
                                                            uint32_t *total, uint32_t *wave_sum_out)
{
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan(v);
    if (lane == kWave - 1) scratch[wid] = incl;
    if (lane == 0) scratch[NW + wid] = wave_val;
    __syncthreads();
    uint32_t sw[NW], sv[NW];
    lds_words<NW>(scratch, sw);
    lds_words<NW>(scratch + NW, sv);
    uint32_t base = 0, tot = 0, vs = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        base += (w < wid) ? sw[w] : 0u;
        tot += sw[w];
        vs += sv[w];
    }
    __syncthreads();
    *total = tot;
    *wave_sum_out = vs;
    return base + incl - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_and_or(uint32_t a, uint32_t o, uint32_t *scratch, uint32_t *or_out)
{
    constexpr int NW = NT / kWave;
    const int wid = threadIdx.x / kWave;
    a = wave_and(a);
    o = wave_or(o);
    if ((threadIdx.x & (kWave - 1)) == 0) {
        scratch[wid] = a;
        scratch[NW + wid] = o;
    }
    __syncthreads();
    uint32_t wa[NW], wo[NW];
    lds_words<NW>(scratch, wa);
    lds_words<NW>(scratch + NW, wo);
    uint32_t ra = 0xFFFFFFFFu, ro = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        ra &= wa[w];
        ro |= wo[w];
    }
    __syncthreads();
    *or_out = ro;
    return ra;
}

}  // namespace prox
