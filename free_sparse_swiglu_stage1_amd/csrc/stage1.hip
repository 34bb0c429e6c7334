// Stage 1 of Prox ("Lightweight Proxy Construction"): input sparsification,
// proxy gate/up projections with quantized weights, channel salience
// |silu(g~) * u~| and the top-k channel mask.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"
#include "select.h"

namespace prox {

// ------------------------------------------------------------------------
// K1a: per-token input sparsification.  One workgroup per token keeps the
// k_in largest |x_i| (ties: lower i) and writes the sparse copy xh[b][d]
// (fp32, zeros elsewhere).  Block 0 also clears the workspace counters the
// later kernels of the same call use.
// ------------------------------------------------------------------------
template <typename T, int KPT>
__global__ __launch_bounds__(1024) void xselect_kernel(const T *__restrict__ x, int d, int k_in,
                                                       float *__restrict__ xh, uint32_t *__restrict__ counters,
                                                       int n_counters)
{
    __shared__ SelectSmem sm;
    const int b = blockIdx.x;
    const int base = threadIdx.x * KPT;
    if (b == 0)
        for (int c = threadIdx.x; c < n_counters; c += 1024) counters[c] = 0u;
    const T *xb = x + (int64_t)b * d;
    float v[KPT];
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        v[r] = (base + r < d) ? elem<T>::load(xb, base + r) : 0.0f;
        key[r] = __float_as_uint(v[r]) & 0x7FFFFFFFu;
    }
    SelectResult sr = block_select_kth<1024, KPT, 11>(key, d, k_in, sm);
    uint32_t before, total;
    uint64_t fl = block_select_flags<1024, KPT>(key, d, sr, sm, &before, &total);
    float *ob = xh + (int64_t)b * d;
#pragma unroll
    for (int r = 0; r < KPT; ++r)
        if (base + r < d) ob[base + r] = ((fl >> r) & 1ull) ? v[r] : 0.0f;
}

// ------------------------------------------------------------------------
// K1: proxy GEMV over the input-major code layout.
//
// Grid (F/CB channel blocks, S input splits).  A workgroup owns CB channels
// (gate and up) and the inputs [s*R, s*R+R).  Its prologue compacts the
// inputs some token kept into an LDS list; the main loop streams only those
// inputs' code runs (skipped inputs are never read), each wave taking every
// 4th listed input and each lane CPL consecutive channels.  The four waves'
// sums are added in LDS in a fixed order and stored as this split's partial
// g~ / u~; the last split to finish a channel block (atomic ticket) adds the
// partials in split order, applies the per-channel scale (int8), and writes
// score_j = sum_b |silu(g~_bj) u~_bj|.  Bitwise deterministic.
//
// int4-g128: codes are biased nibbles (q + 8); per 128-input group each lane
// accumulates sum x*(q+8) and sum x, and at the group end adds
// scale_g * (acc - 8 * sum x) to its running total.
// ------------------------------------------------------------------------
template <int QBITS, int CPL>
struct CodeLoad;
// int8, 16 channels per lane: 16 bytes
template <> struct CodeLoad<8, 16> {
    static __device__ __forceinline__ void get(const uint8_t *p, float *q)
    {
        u32x4 v = ld_stream(p);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int n = 0; n < 4; ++n) q[a * 4 + n] = (float)(int8_t)(w[a] >> (8 * n));
    }
};
// int8, 4 channels per lane: 4 bytes
template <> struct CodeLoad<8, 4> {
    static __device__ __forceinline__ void get(const uint8_t *p, float *q)
    {
        uint32_t w = __builtin_nontemporal_load((const uint32_t *)p);
#pragma unroll
        for (int n = 0; n < 4; ++n) q[n] = (float)(int8_t)(w >> (8 * n));
    }
};
// int4 (biased nibbles), 16 channels per lane: 8 bytes.  Byte p holds
// channel 2p (low nibble) and 2p+1 (high nibble).
template <> struct CodeLoad<4, 16> {
    static __device__ __forceinline__ void get(const uint8_t *p, float *q)
    {
        u32x2 v = __builtin_nontemporal_load((const u32x2 *)p);
        uint32_t w[2] = {v.x, v.y};
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            uint32_t lo = w[a] & 0x0F0F0F0Fu, hi = (w[a] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                q[a * 8 + 2 * n] = (float)((lo >> (8 * n)) & 0xFFu);
                q[a * 8 + 2 * n + 1] = (float)((hi >> (8 * n)) & 0xFFu);
            }
        }
    }
};
// int4, 8 channels per lane: 4 bytes
template <> struct CodeLoad<4, 8> {
    static __device__ __forceinline__ void get(const uint8_t *p, float *q)
    {
        uint32_t w = __builtin_nontemporal_load((const uint32_t *)p);
        uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            q[2 * n] = (float)((lo >> (8 * n)) & 0xFFu);
            q[2 * n + 1] = (float)((hi >> (8 * n)) & 0xFFu);
        }
    }
};

template <int QBITS, int CPL, int NB>
__global__ __launch_bounds__(256) void proxy_kernel(const float *__restrict__ xh, int B, int d, int F,
                                                    const uint8_t *__restrict__ codes,
                                                    const float *__restrict__ scales, int R, int S,
                                                    float *__restrict__ part, float *__restrict__ score,
                                                    uint32_t *__restrict__ counters)
{
    constexpr int NT = 256;
    constexpr int CB = 64 * CPL;            // channels per workgroup
    __shared__ int li[kMaxSplitRange];
    __shared__ float lx[kMaxSplitRange * NB];
    __shared__ int gstart[kMaxSplitRange / 128 + 1];
    __shared__ uint32_t scr[64];
    __shared__ float red[4][2][CB];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int cb = blockIdx.x, s = blockIdx.y;
    const int i0 = s * R;
    const int i1 = min(d, i0 + R);
    const int64_t half_bytes = (int64_t)F * QBITS / 8;  // bytes of one half (gate or up) of a code row

    // ---- prologue: list of inputs some token kept, with their x values
    int nk = 0;
    for (int c0 = i0; c0 < i1; c0 += NT) {
        const int i = c0 + tid;
        float xv[NB];
        bool any = false;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            xv[b] = (i < i1 && b < B) ? xh[(int64_t)b * d + i] : 0.0f;
            any |= xv[b] != 0.0f;
        }
        uint32_t tot;
        uint32_t pos = block_excl_scan<NT>(any ? 1u : 0u, scr, &tot);
        if (QBITS == 4 && i < i1 && ((i - i0) & 127) == 0) gstart[(i - i0) >> 7] = nk + (int)pos;
        if (any) {
            li[nk + pos] = i;
#pragma unroll
            for (int b = 0; b < NB; ++b) lx[(nk + pos) * NB + b] = xv[b];
        }
        nk += (int)tot;
    }
    const int ngroups = (i1 - i0 + 127) / 128;
    if (QBITS == 4 && tid == 0) gstart[ngroups] = nk;
    __syncthreads();

    // ---- main loop
    const int c = cb * CB + lane * CPL;  // first channel of this lane
    const bool active = c < F;
    const int cc = active ? c : 0;
    float acc[NB][2][CPL];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int n = 0; n < CPL; ++n) acc[b][0][n] = acc[b][1][n] = 0.0f;

    const uint8_t *colg = codes + (int64_t)cc * QBITS / 8;
    if (QBITS == 8) {
        constexpr int U = (CPL >= 16) ? 4 : 8;  // rows in flight per wave
        int t = wv;
        for (; t + 4 * (U - 1) < nk; t += 4 * U) {
            float qg[U][CPL], qu[U][CPL];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint8_t *row = colg + (int64_t)li[t + 4 * u] * 2 * half_bytes;
                CodeLoad<QBITS, CPL>::get(row, qg[u]);
                CodeLoad<QBITS, CPL>::get(row + half_bytes, qu[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float xv = lx[(t + 4 * u) * NB + b];
#pragma unroll
                    for (int n = 0; n < CPL; ++n) {
                        acc[b][0][n] = fmaf(xv, qg[u][n], acc[b][0][n]);
                        acc[b][1][n] = fmaf(xv, qu[u][n], acc[b][1][n]);
                    }
                }
        }
        for (; t < nk; t += 4) {
            float qg[CPL], qu[CPL];
            const uint8_t *row = colg + (int64_t)li[t] * 2 * half_bytes;
            CodeLoad<QBITS, CPL>::get(row, qg);
            CodeLoad<QBITS, CPL>::get(row + half_bytes, qu);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float xv = lx[t * NB + b];
#pragma unroll
                for (int n = 0; n < CPL; ++n) {
                    acc[b][0][n] = fmaf(xv, qg[n], acc[b][0][n]);
                    acc[b][1][n] = fmaf(xv, qu[n], acc[b][1][n]);
                }
            }
        }
    } else {
        const int g0 = i0 / 128;
        for (int g = 0; g < ngroups; ++g) {
            float ga[NB][2][CPL], sx[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                sx[b] = 0.0f;
#pragma unroll
                for (int n = 0; n < CPL; ++n) ga[b][0][n] = ga[b][1][n] = 0.0f;
            }
            const int te = gstart[g + 1];
            for (int t = gstart[g] + wv; t < te; t += 4) {
                float qg[CPL], qu[CPL];
                const uint8_t *row = colg + (int64_t)li[t] * 2 * half_bytes;
                CodeLoad<QBITS, CPL>::get(row, qg);
                CodeLoad<QBITS, CPL>::get(row + half_bytes, qu);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float xv = lx[t * NB + b];
                    sx[b] += xv;
#pragma unroll
                    for (int n = 0; n < CPL; ++n) {
                        ga[b][0][n] = fmaf(xv, qg[n], ga[b][0][n]);
                        ga[b][1][n] = fmaf(xv, qu[n], ga[b][1][n]);
                    }
                }
            }
            if (gstart[g] < te) {
                const float *scg = scales + ((int64_t)(g0 + g) * 2) * F + cc;
                float sg[CPL], su[CPL];
#pragma unroll
                for (int n = 0; n < CPL; n += 4) {
                    float4 a = *(const float4 *)(scg + n);
                    float4 e = *(const float4 *)(scg + F + n);
                    sg[n] = a.x; sg[n + 1] = a.y; sg[n + 2] = a.z; sg[n + 3] = a.w;
                    su[n] = e.x; su[n + 1] = e.y; su[n + 2] = e.z; su[n + 3] = e.w;
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float bias = 8.0f * sx[b];
#pragma unroll
                    for (int n = 0; n < CPL; ++n) {
                        acc[b][0][n] = fmaf(sg[n], ga[b][0][n] - bias, acc[b][0][n]);
                        acc[b][1][n] = fmaf(su[n], ga[b][1][n] - bias, acc[b][1][n]);
                    }
                }
            }
        }
    }

    // ---- combine the four waves (fixed order), one token at a time
    for (int b = 0; b < B && b < NB; ++b) {
#pragma unroll
        for (int n = 0; n < CPL; ++n) {
            red[wv][0][lane * CPL + n] = acc[b][0][n];
            red[wv][1][lane * CPL + n] = acc[b][1][n];
        }
        __syncthreads();
        for (int e = tid; e < 2 * CB; e += NT) {
            const int h = e / CB, jj = e % CB, j = cb * CB + jj;
            if (j < F) {
                float v = ((red[0][h][jj] + red[1][h][jj]) + red[2][h][jj]) + red[3][h][jj];
                part[(((int64_t)s * B + b) * 2 + h) * F + j] = v;
            }
        }
        __syncthreads();
    }

    // ---- last split of this channel block reduces the partials
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&counters[cb], 1u) == (uint32_t)(S - 1));
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int jj = tid; jj < CB; jj += NT) {
        const int j = cb * CB + jj;
        if (j >= F) continue;
        float sc = 0.0f;
        for (int b = 0; b < B; ++b) {
            float g = 0.0f, u = 0.0f;
            for (int q = 0; q < S; ++q) {
                g += __builtin_nontemporal_load(&part[(((int64_t)q * B + b) * 2 + 0) * F + j]);
                u += __builtin_nontemporal_load(&part[(((int64_t)q * B + b) * 2 + 1) * F + j]);
            }
            if (QBITS == 8) {
                g *= scales[j];
                u *= scales[F + j];
            }
            sc += fabsf(silu(g) * u);
        }
        score[j] = sc;
    }
    if (tid == 0) counters[cb] = 0u;
}

// ------------------------------------------------------------------------
// K2: top-k channel mask.  One workgroup of 1024 threads: radix select of the
// k-th largest |score| bit pattern, then an ordered compaction that writes the
// selected channel indices in ascending order.
// ------------------------------------------------------------------------
template <int KPT>
__global__ __launch_bounds__(1024) void topk_kernel(const float *__restrict__ score, int n, int k,
                                                    int32_t *__restrict__ sel)
{
    __shared__ SelectSmem sm;
    const int base = threadIdx.x * KPT;
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) key[r] = (base + r < n) ? (__float_as_uint(score[base + r]) & 0x7FFFFFFFu) : 0u;
    SelectResult sr = block_select_kth<1024, KPT, 11>(key, n, k, sm);
    uint32_t before, total;
    uint64_t fl = block_select_flags<1024, KPT>(key, n, sr, sm, &before, &total);
#pragma unroll
    for (int r = 0; r < KPT; ++r)
        if ((fl >> r) & 1ull) {
            if (before < (uint32_t)k) sel[before] = base + r;
            ++before;
        }
}

// ------------------------------------------------------------------------
// host-side launchers
// ------------------------------------------------------------------------
template <typename T>
static hipError_t launch_xselect_t(const void *x, int B, int d, int k_in, float *xh, uint32_t *counters,
                                   int n_counters, hipStream_t st)
{
    const int kpt = (d + 1023) / 1024;
    const T *xp = (const T *)x;
#define XS(K) \
    if (kpt <= K) { xselect_kernel<T, K><<<B, 1024, 0, st>>>(xp, d, k_in, xh, counters, n_counters); return hipGetLastError(); }
    XS(1) XS(2) XS(4) XS(8) XS(16)
#undef XS
    return hipErrorInvalidValue;
}

hipError_t launch_xselect(int dtype, const void *x, int B, int d, int k_in, float *xh, uint32_t *counters,
                          int n_counters, hipStream_t st)
{
    return dtype == 0 ? launch_xselect_t<float>(x, B, d, k_in, xh, counters, n_counters, st)
                      : launch_xselect_t<uint16_t>(x, B, d, k_in, xh, counters, n_counters, st);
}

hipError_t launch_proxy(const ProxyPlan &pl, const float *xh, int B, int d, int F, const uint8_t *codes,
                        const float *scales, float *part, float *score, uint32_t *counters, hipStream_t st)
{
    dim3 grid(pl.n_cblocks, pl.S);
#define PX(Q, C, N) proxy_kernel<Q, C, N><<<grid, 256, 0, st>>>(xh, B, d, F, codes, scales, pl.R, pl.S, part, score, counters)
    if (pl.qbits == 8) {
        if (pl.cpl == 4 && pl.nb == 1) PX(8, 4, 1);
        else if (pl.cpl == 16 && pl.nb == 1) PX(8, 16, 1);
        else if (pl.cpl == 4 && pl.nb == 4) PX(8, 4, 4);
        else if (pl.cpl == 4 && pl.nb == 16) PX(8, 4, 16);
        else return hipErrorInvalidValue;
    } else {
        if (pl.cpl == 8 && pl.nb == 1) PX(4, 8, 1);
        else if (pl.cpl == 16 && pl.nb == 1) PX(4, 16, 1);
        else if (pl.cpl == 8 && pl.nb == 4) PX(4, 8, 4);
        else return hipErrorInvalidValue;
    }
#undef PX
    return hipGetLastError();
}

hipError_t launch_topk(const float *score, int n, int k, int32_t *sel, hipStream_t st)
{
    const int kpt = (n + 1023) / 1024;
#define TK(K) \
    if (kpt <= K) { topk_kernel<K><<<1, 1024, 0, st>>>(score, n, k, sel); return hipGetLastError(); }
    TK(4) TK(8) TK(16) TK(32) TK(64)
#undef TK
    return hipErrorInvalidValue;
}

}  // namespace prox
