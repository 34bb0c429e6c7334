// Offline preparation: weight repacking into the channel-major layout and
// proxy quantization of W_gate / W_up (Stage 1 "Input Sparsity &
// Quantization": quantized proxy copies of the up and gate projections).
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace prox {

// w_gu[j][0][:] = w_gate[j][:], w_gu[j][1][:] = w_up[j][:]
template <typename T>
__global__ void pack_gu_kernel(const T *__restrict__ wg, const T *__restrict__ wu, int d, int64_t n,
                               T *__restrict__ w_gu)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n) return;
    const int64_t j = e / d, i = e - j * d;
    w_gu[(j * 2) * d + i] = wg[e];
    w_gu[(j * 2 + 1) * d + i] = wu[e];
}

// w_down_t[j][m] = w_down[m][j]: 64x64 tiles through LDS
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T *__restrict__ src, int rows, int cols,
                                                        T *__restrict__ dst)
{
    __shared__ T tile[64][65];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4)
        if (r0 + r < rows && c0 + tx < cols) tile[r][tx] = src[(int64_t)(r0 + r) * cols + c0 + tx];
    __syncthreads();
    for (int c = ty; c < 64; c += 4)
        if (c0 + c < cols && r0 + tx < rows) dst[(int64_t)(c0 + c) * rows + r0 + tx] = tile[tx][c];
}

// Symmetric absmax quantization, binary32 round-to-nearest-even throughout:
// scale = fl(a / qmax), q = clamp(rint(fl(w / scale)), -qmax, qmax); a == 0 -> 0.
__device__ __forceinline__ int quant_one(float w, float scale, int qmax)
{
    if (scale == 0.0f) return 0;
    float t = rintf(__fdiv_rn(w, scale));
    t = fminf(fmaxf(t, (float)-qmax), (float)qmax);
    return (int)t;
}

// int8 per row.  Workgroup: 64 channels of one half (blockIdx.y = 0 gate,
// 1 up).  codes [d][2][F] int8, scales [2][F].
template <typename T>
__global__ __launch_bounds__(256) void quant_int8_kernel(const T *__restrict__ w_gu, int d, int F,
                                                         int8_t *__restrict__ codes, float *__restrict__ scales)
{
    __shared__ float pmax[4][64];
    __shared__ float sc[64];
    const int h = blockIdx.y;
    const int cl = threadIdx.x & 63, part = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + cl;
    const bool ok = j < F;
    const T *row = w_gu + ((int64_t)(ok ? j : 0) * 2 + h) * d;
    float m = 0.0f;
    if (ok)
        for (int i = part; i < d; i += 4) m = fmaxf(m, fabsf(elem<T>::load(row, i)));
    pmax[part][cl] = m;
    __syncthreads();
    if (part == 0) {
        const float a = fmaxf(fmaxf(pmax[0][cl], pmax[1][cl]), fmaxf(pmax[2][cl], pmax[3][cl]));
        const float s = __fdiv_rn(a, 127.0f);
        sc[cl] = s;
        if (ok) scales[(int64_t)h * F + j] = s;
    }
    __syncthreads();
    if (!ok) return;
    const float s = sc[cl];
    for (int i = part; i < d; i += 4)
        codes[(int64_t)i * 2 * F + (int64_t)h * F + j] = (int8_t)quant_one(elem<T>::load(row, i), s, 127);
}

// int4 per (channel, 128-input group).  Workgroup: 64 channels of one half,
// one group (blockIdx.z).  codes [d][2][F/2] biased nibbles, scales [d/128][2][F].
template <typename T>
__global__ __launch_bounds__(256) void quant_int4_kernel(const T *__restrict__ w_gu, int d, int F,
                                                         uint8_t *__restrict__ codes, float *__restrict__ scales)
{
    __shared__ float pmax[4][64];
    __shared__ float sc[64];
    __shared__ uint8_t qv[128][64];
    const int h = blockIdx.y, g = blockIdx.z;
    const int cl = threadIdx.x & 63, part = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + cl;
    const bool ok = j < F;
    const T *row = w_gu + ((int64_t)(ok ? j : 0) * 2 + h) * d + g * 128;
    float m = 0.0f;
    if (ok)
        for (int i = part; i < 128; i += 4) m = fmaxf(m, fabsf(elem<T>::load(row, i)));
    pmax[part][cl] = m;
    __syncthreads();
    if (part == 0) {
        const float a = fmaxf(fmaxf(pmax[0][cl], pmax[1][cl]), fmaxf(pmax[2][cl], pmax[3][cl]));
        const float s = __fdiv_rn(a, 7.0f);
        sc[cl] = s;
        if (ok) scales[((int64_t)g * 2 + h) * F + j] = s;
    }
    __syncthreads();
    const float s = sc[cl];
    for (int i = part; i < 128; i += 4) qv[i][cl] = ok ? (uint8_t)(quant_one(elem<T>::load(row, i), s, 7) + 8) : 8;
    __syncthreads();
    // 128 inputs x 32 bytes (64 channels) per workgroup
    const int64_t half_bytes = F / 2;
    for (int e = threadIdx.x; e < 128 * 32; e += 256) {
        const int i = e >> 5, p = e & 31;
        const int jc = blockIdx.x * 64 + 2 * p;
        if (jc < F) {
            const uint8_t b = (uint8_t)(qv[i][2 * p] | (qv[i][2 * p + 1] << 4));
            codes[((int64_t)(g * 128 + i) * 2 + h) * half_bytes + jc / 2] = b;
        }
    }
}

template <typename T>
static hipError_t pack_t(const void *wg, const void *wu, const void *wd, int d, int F, void *w_gu, void *w_down_t,
                         hipStream_t st)
{
    const int64_t n = (int64_t)F * d;
    pack_gu_kernel<T><<<(unsigned)((n + 255) / 256), 256, 0, st>>>((const T *)wg, (const T *)wu, d, n, (T *)w_gu);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((F + 63) / 64, (d + 63) / 64);
    transpose_kernel<T><<<grid, 256, 0, st>>>((const T *)wd, d, F, (T *)w_down_t);
    return hipGetLastError();
}

hipError_t launch_pack(int dtype, const void *w_gate, const void *w_up, const void *w_down, int d, int F,
                       void *w_gu, void *w_down_t, hipStream_t st)
{
    return dtype == 0 ? pack_t<float>(w_gate, w_up, w_down, d, F, w_gu, w_down_t, st)
                      : pack_t<uint16_t>(w_gate, w_up, w_down, d, F, w_gu, w_down_t, st);
}

template <typename T>
static hipError_t quant_t(int qbits, const void *w_gu, int d, int F, uint8_t *codes, float *scales, hipStream_t st)
{
    if (qbits == 8) {
        dim3 grid((F + 63) / 64, 2);
        quant_int8_kernel<T><<<grid, 256, 0, st>>>((const T *)w_gu, d, F, (int8_t *)codes, scales);
    } else {
        dim3 grid((F + 63) / 64, 2, d / 128);
        quant_int4_kernel<T><<<grid, 256, 0, st>>>((const T *)w_gu, d, F, codes, scales);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(int dtype, int qbits, const void *w_gu, int d, int F, uint8_t *codes, float *scales,
                           hipStream_t st)
{
    return dtype == 0 ? quant_t<float>(qbits, w_gu, d, F, codes, scales, st)
                      : quant_t<uint16_t>(qbits, w_gu, d, F, codes, scales, st);
}

}  // namespace prox
