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

// Rows of w_gu as the proxy quantizers read them: row r = 2 j + h (h = 0
// gate, 1 up), element i, as binary32.
template <typename T>
struct GuRows {
    const T *w;
    int d;
    __device__ __forceinline__ float operator()(int64_t r, int i) const { return elem<T>::load(w, r * d + i); }
};
// FP8 weights: the binary32 value the row stands for, fl32(scale * decode).
struct GuRowsFp8 {
    const uint8_t *w;
    const float *sc;
    int d;
    __device__ __forceinline__ float operator()(int64_t r, int i) const
    {
        return __fmul_rn(sc[r], e4m3_to_f32(w[r * d + i]));
    }
};

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
template <typename RD>
__global__ __launch_bounds__(256) void quant_int8_kernel(RD rd, int d, int F, int8_t *__restrict__ codes,
                                                         float *__restrict__ scales)
{
    __shared__ float pmax[4][64];
    __shared__ float sc[64];
    const int h = blockIdx.y;
    const int cl = threadIdx.x & 63, part = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + cl;
    const bool ok = j < F;
    const int64_t row = (int64_t)(ok ? j : 0) * 2 + h;
    float m = 0.0f;
    if (ok)
        for (int i = part; i < d; i += 4) m = fmaxf(m, fabsf(rd(row, i)));
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
        codes[(int64_t)i * 2 * F + (int64_t)h * F + j] = (int8_t)quant_one(rd(row, i), s, 127);
}

// int4 per (channel, 128-input group).  Workgroup: 64 channels of one half,
// one group (blockIdx.z).  codes [d][2][F/2] biased nibbles, scales [d/128][2][F].
template <typename RD>
__global__ __launch_bounds__(256) void quant_int4_kernel(RD rd, int d, int F, uint8_t *__restrict__ codes,
                                                         float *__restrict__ scales)
{
    __shared__ float pmax[4][64];
    __shared__ float sc[64];
    __shared__ uint8_t qv[128][64];
    const int h = blockIdx.y, g = blockIdx.z;
    const int cl = threadIdx.x & 63, part = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + cl;
    const bool ok = j < F;
    const int64_t row = (int64_t)(ok ? j : 0) * 2 + h;
    const int i0 = g * 128;
    float m = 0.0f;
    if (ok)
        for (int i = part; i < 128; i += 4) m = fmaxf(m, fabsf(rd(row, i0 + i)));
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
    for (int i = part; i < 128; i += 4) qv[i][cl] = ok ? (uint8_t)(quant_one(rd(row, i0 + i), s, 7) + 8) : 8;
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

template <typename RD>
static hipError_t quant_t(int qbits, RD rd, int d, int F, uint8_t *codes, float *scales, hipStream_t st)
{
    if (qbits == 8) {
        dim3 grid((F + 63) / 64, 2);
        quant_int8_kernel<RD><<<grid, 256, 0, st>>>(rd, d, F, (int8_t *)codes, scales);
    } else {
        dim3 grid((F + 63) / 64, 2, d / 128);
        quant_int4_kernel<RD><<<grid, 256, 0, st>>>(rd, d, F, codes, scales);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(int dtype, int wfmt, const void *w_gu, const float *gu_scales, int qbits, int d, int F,
                           uint8_t *codes, float *scales, hipStream_t st)
{
    if (wfmt == 1) return quant_t(qbits, GuRowsFp8{(const uint8_t *)w_gu, gu_scales, d}, d, F, codes, scales, st);
    return dtype == 0 ? quant_t(qbits, GuRows<float>{(const float *)w_gu, d}, d, F, codes, scales, st)
                      : quant_t(qbits, GuRows<uint16_t>{(const uint16_t *)w_gu, d}, d, F, codes, scales, st);
}

// ------------------------------------------------------------------------
// FP8 (OCP E4M3) exact weights, one binary32 scale per output row:
// scale = fl32(amax / 448), code = E4M3 of fl32(w / scale) (nearest, ties to
// the even code, saturating); an all-zero row gets scale 0 and codes 0.
// ------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float row_absmax(const T *__restrict__ row, int n, float *red)
{
    float m = 0.0f;
    for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, fabsf(elem<T>::load(row, i)));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ uint8_t fp8_code(float w, float s)
{
    return s == 0.0f ? (uint8_t)0 : (uint8_t)f32_to_e4m3(__fdiv_rn(w, s));
}

// gate/up: one workgroup per row r = 2 j + h of w_gu8 [F][2][d]; scales [F][2]
template <typename T>
__global__ __launch_bounds__(256) void pack_fp8_gu_kernel(const T *__restrict__ wg, const T *__restrict__ wu, int d,
                                                          uint8_t *__restrict__ w_gu8, float *__restrict__ gu_scales)
{
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const T *src = ((r & 1) ? wu : wg) + (r >> 1) * d;
    const float s = __fdiv_rn(row_absmax(src, d, red), 448.0f);
    if (threadIdx.x == 0) gu_scales[r] = s;
    uint8_t *dst = w_gu8 + r * d;
    for (int i = threadIdx.x; i < d; i += 256) dst[i] = fp8_code(elem<T>::load(src, i), s);
}

// down: scale of each row m of W_down [d][F]
template <typename T>
__global__ __launch_bounds__(256) void fp8_row_scale_kernel(const T *__restrict__ w, int cols,
                                                            float *__restrict__ scales)
{
    __shared__ float red[4];
    const float s = __fdiv_rn(row_absmax(w + (int64_t)blockIdx.x * cols, cols, red), 448.0f);
    if (threadIdx.x == 0) scales[blockIdx.x] = s;
}

// w_down_t8[j][m] = code of W_down[m][j] with row m's scale: 64x64 tiles
template <typename T>
__global__ __launch_bounds__(256) void fp8_transpose_kernel(const T *__restrict__ src, const float *__restrict__ scales,
                                                            int rows, int cols, uint8_t *__restrict__ dst)
{
    __shared__ uint8_t tile[64][65];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4)
        if (r0 + r < rows && c0 + tx < cols)
            tile[r][tx] = fp8_code(elem<T>::load(src, (int64_t)(r0 + r) * cols + c0 + tx), scales[r0 + r]);
    __syncthreads();
    for (int c = ty; c < 64; c += 4)
        if (c0 + c < cols && r0 + tx < rows) dst[(int64_t)(c0 + c) * rows + r0 + tx] = tile[tx][c];
}

template <typename T>
static hipError_t pack_fp8_t(const void *wg, const void *wu, const void *wd, int d, int F, uint8_t *w_gu8,
                             float *gu_scales, uint8_t *w_down_t8, float *down_scales, hipStream_t st)
{
    pack_fp8_gu_kernel<T><<<2 * F, 256, 0, st>>>((const T *)wg, (const T *)wu, d, w_gu8, gu_scales);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    fp8_row_scale_kernel<T><<<d, 256, 0, st>>>((const T *)wd, F, down_scales);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((F + 63) / 64, (d + 63) / 64);
    fp8_transpose_kernel<T><<<grid, 256, 0, st>>>((const T *)wd, down_scales, d, F, w_down_t8);
    return hipGetLastError();
}

hipError_t launch_pack_fp8(int dtype, const void *w_gate, const void *w_up, const void *w_down, int d, int F,
                           uint8_t *w_gu8, float *gu_scales, uint8_t *w_down_t8, float *down_scales, hipStream_t st)
{
    return dtype == 0 ? pack_fp8_t<float>(w_gate, w_up, w_down, d, F, w_gu8, gu_scales, w_down_t8, down_scales, st)
                      : pack_fp8_t<uint16_t>(w_gate, w_up, w_down, d, F, w_gu8, gu_scales, w_down_t8, down_scales,
                                             st);
}

}  // namespace prox
