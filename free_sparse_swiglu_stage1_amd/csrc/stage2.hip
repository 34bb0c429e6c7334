// Stage 2 of Prox ("Exact Sparse Computation"): exact gate/up projections
// and SiLU-multiply on the selected channels only, then the down projection
// restricted to the same channels.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace prox {

// ------------------------------------------------------------------------
// K3: gathered gate/up GEMV.  w_gu is channel-major [F][2][d], so channel j's
// gate and up rows are one contiguous 2*d run.  Each wave takes a selected
// channel, streams both rows with 16-byte loads (whole row in flight), dots
// them with x (staged once per workgroup in LDS as fp32) and writes
// s[b][r] = silu(g) * u in fp32.
// ------------------------------------------------------------------------
template <typename T, int NB>
__global__ __launch_bounds__(256) void gateup_kernel(const T *__restrict__ x, int B, int d,
                                                     const T *__restrict__ w_gu, const int32_t *__restrict__ sel,
                                                     int k, float *__restrict__ s_sp, int32_t *__restrict__ iota_out)
{
    constexpr int V = vec16<T>::N;  // elements per 16-byte load
    constexpr int UNR = 8;          // 16-byte chunks in flight per row
    extern __shared__ float xs[];   // [NB][d]
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int e = tid; e < NB * d; e += 256) {
        const int b = e / d;
        xs[e] = (b < B) ? elem<T>::load(x, (int64_t)b * d + (e - b * d)) : 0.0f;
    }
    __syncthreads();
    const int nwaves = gridDim.x * 4;
    for (int r = blockIdx.x * 4 + wv; r < k; r += nwaves) {
        const int j = sel ? sel[r] : r;
        if (iota_out && lane == 0) iota_out[r] = r;
        const T *grow = w_gu + (int64_t)j * 2 * d;
        const T *urow = grow + d;
        float ag[NB], au[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) ag[b] = au[b] = 0.0f;
        for (int e0 = lane * V; e0 < d; e0 += 64 * V * UNR) {
            u32x4 vg[UNR], vu[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int e = e0 + u * 64 * V;
                if (e < d) {
                    vg[u] = ld_stream(grow + e);
                    vu[u] = ld_stream(urow + e);
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int e = e0 + u * 64 * V;
                if (e < d) {
                    float fg[V], fu[V];
                    vec16<T>::unpack(vg[u], fg);
                    vec16<T>::unpack(vu[u], fu);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const float *xb = xs + b * d + e;
#pragma unroll
                        for (int q = 0; q < V; ++q) {
                            ag[b] = fmaf(fg[q], xb[q], ag[b]);
                            au[b] = fmaf(fu[q], xb[q], au[b]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float g = wave_sum(ag[b]);
            const float u = wave_sum(au[b]);
            if (lane == 0 && b < B) s_sp[(int64_t)b * k + r] = silu(g) * u;
        }
    }
}

// ------------------------------------------------------------------------
// K4: down projection over the selected rows of W_down^T [F][d].
// Grid (column slices of 64*VEC outputs, S rank splits).  Each wave takes
// every 4th selected channel of its split and adds s[b][r] * W_down^T[j][cols]
// into VEC columns per lane; the four waves are combined in LDS in a fixed
// order into this split's partial; the last split of a slice (atomic ticket)
// adds the partials in split order, adds the residual if any, and stores.
// ------------------------------------------------------------------------
template <typename T, int NB>
__global__ __launch_bounds__(256) void down_kernel(const float *__restrict__ s_sp, int B, int k,
                                                   const T *__restrict__ wdt, const int32_t *__restrict__ sel,
                                                   int d, int S, float *__restrict__ part,
                                                   const T *residual, T *out, uint32_t *__restrict__ counters)
{
    constexpr int V = vec16<T>::N;
    constexpr int COLS = 64 * V;
    constexpr int UNR = 8;
    __shared__ float red[4][NB][COLS];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int sl = blockIdx.x, s = blockIdx.y;
    const int c = sl * COLS + lane * V;
    const bool active = c < d;
    const int r0 = (int)(((int64_t)k * s) / S), r1 = (int)(((int64_t)k * (s + 1)) / S);
    float acc[NB][V];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < V; ++q) acc[b][q] = 0.0f;

    int r = r0 + wv;
    for (; r + 4 * (UNR - 1) < r1; r += 4 * UNR) {
        u32x4 w[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int rr = r + 4 * u;
            const int j = sel ? sel[rr] : rr;
            w[u] = active ? ld_stream(wdt + (int64_t)j * d + c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            float f[V];
            vec16<T>::unpack(w[u], f);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float sv = (b < B) ? s_sp[(int64_t)b * k + r + 4 * u] : 0.0f;
#pragma unroll
                for (int q = 0; q < V; ++q) acc[b][q] = fmaf(sv, f[q], acc[b][q]);
            }
        }
    }
    for (; r < r1; r += 4) {
        const int j = sel ? sel[r] : r;
        u32x4 w = u32x4{0u, 0u, 0u, 0u};
        if (active) w = ld_stream(wdt + (int64_t)j * d + c);
        float f[V];
        vec16<T>::unpack(w, f);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float sv = (b < B) ? s_sp[(int64_t)b * k + r] : 0.0f;
#pragma unroll
            for (int q = 0; q < V; ++q) acc[b][q] = fmaf(sv, f[q], acc[b][q]);
        }
    }

#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < V; ++q) red[wv][b][lane * V + q] = acc[b][q];
    __syncthreads();
    for (int e = tid; e < NB * COLS; e += 256) {
        const int b = e / COLS, cc = e % COLS, col = sl * COLS + cc;
        if (b < B && col < d) {
            const float v = ((red[0][b][cc] + red[1][b][cc]) + red[2][b][cc]) + red[3][b][cc];
            part[((int64_t)s * B + b) * d + col] = v;
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&counters[sl], 1u) == (uint32_t)(S - 1));
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int e = tid; e < B * COLS; e += 256) {
        const int b = e / COLS, col = sl * COLS + e % COLS;
        if (col >= d) continue;
        float y = 0.0f;
        for (int q = 0; q < S; ++q) y += __builtin_nontemporal_load(&part[((int64_t)q * B + b) * d + col]);
        if (residual) y += elem<T>::load(residual, (int64_t)b * d + col);
        elem<T>::store(out, (int64_t)b * d + col, y);
    }
    if (tid == 0) counters[sl] = 0u;
}

// out = residual (or 0): the k == 0 case
template <typename T>
__global__ void fill_out_kernel(int n, const T *residual, T *out)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) elem<T>::store(out, i, residual ? elem<T>::load(residual, i) : 0.0f);
}

__global__ void zero_u32_kernel(uint32_t *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// RMSNorm with unit gain, fp32 math: out = h / sqrt(mean(h^2) + eps)
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T *h, int d, float eps, T *out)
{
    __shared__ float red[4];
    const int b = blockIdx.x, tid = threadIdx.x;
    const T *hb = h + (int64_t)b * d;
    float ss = 0.0f;
    for (int i = tid; i < d; i += 256) {
        const float v = elem<T>::load(hb, i);
        ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    const float rms = sqrtf(tot / (float)d + eps);
    T *ob = out + (int64_t)b * d;
    for (int i = tid; i < d; i += 256) elem<T>::store(ob, i, elem<T>::load(hb, i) / rms);
}

// ------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------
template <typename T>
static hipError_t gateup_t(const void *x, int B, int d, const void *w_gu, const int32_t *sel, int k, float *s_sp,
                           int32_t *iota_out, hipStream_t st)
{
    if (k <= 0) return hipSuccess;
    int blocks = (k + 7) / 8;  // two channels per wave
    if (blocks < 1) blocks = 1;
    // x of up to 4 tokens staged in LDS as fp32, within 64 KB
    const int tb = (4 * d * (int)sizeof(float) <= 65536) ? 4 : 1;
    for (int b0 = 0; b0 < B; b0 += tb) {
        const int nb = (B - b0 >= tb) ? tb : B - b0;
        const T *xp = (const T *)x + (int64_t)b0 * d;
        float *sp = s_sp + (int64_t)b0 * k;
        int32_t *io = (b0 == 0) ? iota_out : nullptr;
        if (nb == 1)
            gateup_kernel<T, 1><<<blocks, 256, d * sizeof(float), st>>>(xp, 1, d, (const T *)w_gu, sel, k, sp, io);
        else
            gateup_kernel<T, 4><<<blocks, 256, 4 * d * sizeof(float), st>>>(xp, nb, d, (const T *)w_gu, sel, k, sp, io);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gateup(int dtype, const void *x, int B, int d, const void *w_gu, const int32_t *sel, int k,
                         float *s_sp, int32_t *iota_out, hipStream_t st)
{
    return dtype == 0 ? gateup_t<float>(x, B, d, w_gu, sel, k, s_sp, iota_out, st)
                      : gateup_t<uint16_t>(x, B, d, w_gu, sel, k, s_sp, iota_out, st);
}

template <typename T>
static hipError_t down_t(const DownPlan &pl, const float *s_sp, int B, int k, const void *wdt, const int32_t *sel,
                         int d, float *part, const void *residual, void *out, uint32_t *counters, hipStream_t st)
{
    dim3 grid(pl.n_slices, pl.S);
    // tokens in passes of at most 4 (a pass re-reads the selected rows)
    for (int b0 = 0; b0 < B; b0 += 4) {
        const int nb = (B - b0 >= 4) ? 4 : B - b0;
        const float *sp = s_sp + (int64_t)b0 * k;
        const T *res = residual ? (const T *)residual + (int64_t)b0 * d : nullptr;
        T *o = (T *)out + (int64_t)b0 * d;
        if (nb == 1)
            down_kernel<T, 1><<<grid, 256, 0, st>>>(sp, 1, k, (const T *)wdt, sel, d, pl.S, part, res, o, counters);
        else
            down_kernel<T, 4><<<grid, 256, 0, st>>>(sp, nb, k, (const T *)wdt, sel, d, pl.S, part, res, o, counters);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_down(int dtype, const DownPlan &pl, const float *s_sp, int B, int k, const void *w_down_t,
                       const int32_t *sel, int d, float *part, const void *residual, void *out,
                       uint32_t *counters, hipStream_t st)
{
    return dtype == 0 ? down_t<float>(pl, s_sp, B, k, w_down_t, sel, d, part, residual, out, counters, st)
                      : down_t<uint16_t>(pl, s_sp, B, k, w_down_t, sel, d, part, residual, out, counters, st);
}

hipError_t launch_fill_out(int dtype, int B, int d, const void *residual, void *out, hipStream_t st)
{
    const int n = B * d;
    if (dtype == 0)
        fill_out_kernel<float><<<(n + 255) / 256, 256, 0, st>>>(n, (const float *)residual, (float *)out);
    else
        fill_out_kernel<uint16_t><<<(n + 255) / 256, 256, 0, st>>>(n, (const uint16_t *)residual, (uint16_t *)out);
    return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t *p, int n, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    zero_u32_kernel<<<(n + 255) / 256, 256, 0, st>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const void *h, int B, int d, float eps, void *out, hipStream_t st)
{
    if (dtype == 0)
        rmsnorm_kernel<float><<<B, 256, 0, st>>>((const float *)h, d, eps, (float *)out);
    else
        rmsnorm_kernel<uint16_t><<<B, 256, 0, st>>>((const uint16_t *)h, d, eps, (uint16_t *)out);
    return hipGetLastError();
}

}  // namespace prox
