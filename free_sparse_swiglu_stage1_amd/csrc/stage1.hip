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
// (fp32, zeros elsewhere); with no tie at the threshold T the kept set is
// simply |x_i| >= T.  Block 0 also clears the workspace counters the
// later kernels of the same call use.
// ------------------------------------------------------------------------
template <typename T, int KPT>
__global__ __launch_bounds__(1024) void xselect_kernel(const T *__restrict__ x, int d, int k_in,
                                                       float *__restrict__ xh, uint32_t *__restrict__ counters,
                                                       int n_counters, float norm_eps, T *__restrict__ xn_out)
{
    __shared__ SelectSmem<16384> sm;
    const int b = blockIdx.x;
    if (b == 0)
        for (int c = threadIdx.x; c < n_counters; c += 1024) counters[c] = 0u;
    const T *xb = x + (int64_t)b * d;
    float v[KPT];
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {  // all loads issued before any use
        const int i = slot_index<KPT>(r);
        v[r] = elem<T>::load(xb, i < d ? i : d - 1);
    }
    if (norm_eps >= 0.0f) {  // x is h: select on RMSNorm(h) and write it to xn_out
        // the squares summed as rmsnorm_kernel sums them: threads 0..255,
        // each over its 16-byte vectors t + 256 q in order (vectors past d
        // add exact zeros there), then each wave, then the four waves
        constexpr int VV = vec16<T>::N;
        constexpr int NQ = 16384 / VV / 256;
        const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
        float ssq = 0.0f;
        if (tid < 256) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<T *>(xb), (short)0, (int)(sizeof(T) * d), CoherentBuf::kWord3);
            u32x4 hv[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                hv[q] = __builtin_bit_cast(u32x4,
                                           __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (tid + 256 * q), 0, 0));
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                float f[VV];
                vec16<T>::unpack(hv[q], f);
#pragma unroll
                for (int i = 0; i < VV; ++i) ssq = fmaf(f[i], f[i], ssq);
            }
        }
        ssq = wave_sum(ssq);
        if (lane == 0 && wv < 4) sm.scratch[wv] = __float_as_uint(ssq);  // the bits (a word array)
        __syncthreads();
        const float s0 = __uint_as_float(sm.scratch[0]), s1 = __uint_as_float(sm.scratch[1]);
        const float s2 = __uint_as_float(sm.scratch[2]), s3 = __uint_as_float(sm.scratch[3]);
        const float rms = sqrtf((((s0 + s1) + s2) + s3) / (float)d + norm_eps);
        __syncthreads();
        T *xo = xn_out + (int64_t)b * d;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {  // rounded to x's dtype, as rmsnorm_kernel stores it
            const float y = v[r] / rms;
            v[r] = sizeof(T) == 2 ? __uint_as_float((uint32_t)f32_to_bf16(y) << 16) : y;
            if (slot_index<KPT>(r) < d) elem<T>::store(xo, slot_index<KPT>(r), v[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        if (slot_index<KPT>(r) >= d) v[r] = 0.0f;
        key[r] = __float_as_uint(v[r]) & 0x7FFFFFFFu;
    }
    // magnitudes are sign-free, and a bf16 value's low 16 bits are zero
    const SelectResult sr = block_select_window<1024, KPT>(key, d, k_in, 30, sizeof(T) == 2 ? 16 : 0, sm);
    float *ob = xh + (int64_t)b * d;
    if (uniform_u32(sr.need_eq) == uniform_u32(sr.count_eq)) {  // no tie to break: keep key >= T
        const uint32_t thr = uniform_u32(sr.T);
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int i = slot_index<KPT>(r);
            if (i < d) ob[i] = key[r] >= thr ? v[r] : 0.0f;
        }
        return;
    }
    selection_bitmap<1024, KPT>(key, d, sr, sm);
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const int i = slot_index<KPT>(r);
        if (i < d) ob[i] = bitmap_test(sm.bits, i) ? v[r] : 0.0f;
    }
}

// ------------------------------------------------------------------------
// K1: proxy GEMV over the input-major code layout.
//
// Grid (F/CB channel blocks, S input splits).  A workgroup owns CB channels
// (gate and up) and the inputs [s*R, s*R+R).  Its prologue compacts the
// inputs some token kept into an LDS list; the main loop streams only those
// inputs' code runs (skipped inputs are never read).  Each wave takes every
// 4th listed input, 16 inputs in flight, and each lane one 32-bit word of
// codes per half (4 int8 channels or 8 int4 channels).  The four waves' sums
// are added in LDS in a fixed order into this split's partial g~ / u~; the
// last split to finish a channel block (atomic ticket) adds the partials in
// split order, applies the per-channel scale (int8), and writes
// score_j = sum_b of the signal's salience term (|act(g~) u~| for Prox).
// Bitwise deterministic.
//
// int4-g128: codes are biased nibbles (q + 8); per 128-input group each lane
// accumulates sum x*(q+8) and sum x, and when the group changes adds
// scale_g * (acc - 8 * sum x) to its running total; the group scales of the
// workgroup's channels are staged in LDS by the prologue.
// ------------------------------------------------------------------------
template <int QBITS>
struct Codes;
template <> struct Codes<8> {  // 4 signed bytes -> channels c..c+3
    static constexpr int CPL = 4;
    static __device__ __forceinline__ void decode(uint32_t w, float *q)
    {
#pragma unroll
        for (int n = 0; n < 4; ++n) q[n] = (float)(int8_t)(w >> (8 * n));
    }
};
template <> struct Codes<4> {  // 8 biased nibbles; byte p holds channels 2p (low), 2p+1 (high)
    static constexpr int CPL = 8;
    static __device__ __forceinline__ void decode(uint32_t w, float *q)
    {
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            q[2 * n] = (float)((lo >> (8 * n)) & 0xFFu);
            q[2 * n + 1] = (float)((hi >> (8 * n)) & 0xFFu);
        }
    }
};

template <int QBITS, int NB>
__global__ __launch_bounds__(256) void proxy_kernel(const float *__restrict__ xh, int B, int d, int F,
                                                    const uint8_t *__restrict__ codes,
                                                    const float *__restrict__ scales, int R, int S,
                                                    float *__restrict__ part, float *__restrict__ score,
                                                    uint32_t *__restrict__ counters, int act, int signal)
{
    constexpr int NT = 256;
    constexpr int CPL = Codes<QBITS>::CPL;
    constexpr int CB = 64 * CPL;                 // channels per workgroup
    constexpr int U = 16;                        // listed inputs in flight per wave
    constexpr int NG = kMaxSplitRange / 128;     // int4 groups per split
    __shared__ int li[kMaxSplitRange];
    __shared__ float lx[kMaxSplitRange * NB];
    __shared__ float gsc[QBITS == 4 ? NG : 1][2][QBITS == 4 ? CB : 1];
    __shared__ __align__(16) uint32_t scr[64];
    __shared__ float red[4][2][CB];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int cb = blockIdx.x, s = blockIdx.y;
    const int i0 = s * R;
    const int i1 = min(d, i0 + R);
    const int64_t half_bytes = (int64_t)F * QBITS / 8;  // one half (gate or up) of a code row
    const int c = cb * CB + lane * CPL;                  // first channel of this lane
    const bool active = c < F;
    const int cc = active ? c : 0;

    // ---- prologue: int4 group scales of this block, and the kept-input list
    if (QBITS == 4) {
        const int ng = (i1 - i0 + 127) / 128;
        for (int e = tid; e < ng * 2 * CB; e += NT) {
            const int g = e / (2 * CB), h = (e / CB) & 1, jj = e % CB, j = cb * CB + jj;
            const float v = scales[((int64_t)(i0 / 128 + g) * 2 + h) * F + (j < F ? j : F - 1)];
            gsc[g][h][jj] = (j < F) ? v : 0.0f;
        }
    }
    int nk = 0;
    for (int c0 = i0; c0 < i1; c0 += NT) {
        const int i = c0 + tid;
        float xv[NB];
        bool any = false;
#pragma unroll
        for (int b = 0; b < NB; ++b) xv[b] = xh[(int64_t)(b < B ? b : 0) * d + (i < i1 ? i : i1 - 1)];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (!(i < i1 && b < B)) xv[b] = 0.0f;
            any |= xv[b] != 0.0f;
        }
        uint32_t tot;
        const uint32_t pos = block_excl_scan<NT>(any ? 1u : 0u, scr, &tot);
        if (any) {
            li[nk + pos] = i;
#pragma unroll
            for (int b = 0; b < NB; ++b) lx[(nk + pos) * NB + b] = xv[b];
        }
        nk += (int)tot;
    }
    __syncthreads();

    // ---- main loop
    float acc[NB][2][CPL];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int n = 0; n < CPL; ++n) acc[b][0][n] = acc[b][1][n] = 0.0f;
    float ga[NB][2][CPL], sx[NB];  // int4: current group's sums
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        sx[b] = 0.0f;
#pragma unroll
        for (int n = 0; n < CPL; ++n) ga[b][0][n] = ga[b][1][n] = 0.0f;
    }
    int cur_g = 0;
    auto flush_group = [&](int g) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float bias = 8.0f * sx[b];
#pragma unroll
            for (int n = 0; n < CPL; ++n) {
                acc[b][0][n] = fmaf(gsc[g][0][lane * CPL + n], ga[b][0][n] - bias, acc[b][0][n]);
                acc[b][1][n] = fmaf(gsc[g][1][lane * CPL + n], ga[b][1][n] - bias, acc[b][1][n]);
                ga[b][0][n] = ga[b][1][n] = 0.0f;
            }
            sx[b] = 0.0f;
        }
    };

    // codes through a buffer resource on 32-bit offsets (the codes are below
    // 2 GiB at every supported shape: d <= 16384 rows of at most 131040
    // bytes); a load past the list reads zeros without touching memory, so
    // no load sits under a branch.  At 8192 x 28672 (int8) Stage 1 took 0.55
    // us less than with global loads on 64-bit addresses under a branch.
    const uint32_t row_bytes = (uint32_t)(2 * half_bytes), col_off = (uint32_t)((int64_t)cc * QBITS / 8);
    const uint32_t code_bytes = row_bytes * (uint32_t)d;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(codes), (short)0,
                                                                         (int)code_bytes, CoherentBuf::kWord3);
    for (int t0 = wv; t0 < nk; t0 += 4 * U) {
        uint32_t wg[U], wu[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 4 * u;
            const uint32_t o = t < nk ? (uint32_t)li[min(t, nk - 1)] * row_bytes + col_off : code_bytes;
            wg[u] = __builtin_amdgcn_raw_buffer_load_b32(crs, (int)o, 0, 2);  // streaming
            wu[u] = __builtin_amdgcn_raw_buffer_load_b32(crs, (int)(o + (uint32_t)half_bytes), 0, 2);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 4 * u;
            if (t < nk) {
                float qg[CPL], qu[CPL];
                Codes<QBITS>::decode(wg[u], qg);
                Codes<QBITS>::decode(wu[u], qu);
                if (QBITS == 4) {
                    const int g = (li[t] - i0) >> 7;
                    if (g != cur_g) {
                        flush_group(cur_g);
                        cur_g = g;
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float xv = lx[t * NB + b];
                    if (QBITS == 4) sx[b] += xv;
                    float(&dst)[2][CPL] = (QBITS == 4) ? ga[b] : acc[b];
#pragma unroll
                    for (int n = 0; n < CPL; ++n) {
                        dst[0][n] = fmaf(xv, qg[n], dst[0][n]);
                        dst[1][n] = fmaf(xv, qu[n], dst[1][n]);
                    }
                }
            }
        }
    }
    if (QBITS == 4) flush_group(cur_g);

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
                const float v = ((red[0][h][jj] + red[1][h][jj]) + red[2][h][jj]) + red[3][h][jj];
                store_agent(&part[(((int64_t)s * B + b) * 2 + h) * F + j], v);
            }
        }
        __syncthreads();
    }

    // ---- the last split of this channel block reduces the partials
    if (!publish_and_ticket(&counters[cb], (uint32_t)S, &s_last)) return;
    constexpr int QC = (NB >= 16) ? 2 : (NB >= 4 ? 8 : 32);  // splits per batch of loads
    for (int jj = tid; jj < CB; jj += NT) {
        const int j = cb * CB + jj;
        if (j >= F) continue;
        float g[NB], u[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) g[b] = u[b] = 0.0f;
        for (int q0 = 0; q0 < S; q0 += QC) {
            float vg[QC][NB], vu[QC][NB];
#pragma unroll
            for (int qq = 0; qq < QC; ++qq)
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int q = q0 + qq;
                    const bool ok = q < S && b < B;
                    const int64_t o = (((int64_t)(ok ? q : 0) * B + (ok ? b : 0)) * 2) * F + j;
                    vg[qq][b] = load_agent(&part[o]);
                    vu[qq][b] = load_agent(&part[o + F]);
                    if (!ok) vg[qq][b] = vu[qq][b] = 0.0f;
                }
#pragma unroll
            for (int qq = 0; qq < QC; ++qq)
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    g[b] += vg[qq][b];
                    u[b] += vu[qq][b];
                }
        }
        const float sg = (QBITS == 8) ? scales[j] : 1.0f;
        const float su = (QBITS == 8) ? scales[F + j] : 1.0f;
        float sc = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b < B) sc += salience(signal, act, g[b] * sg, u[b] * su);
        score[j] = sc;
    }
}

// ------------------------------------------------------------------------
// K2: top-k channel mask.  One workgroup of 1024 threads: radix select of the
// k-th largest |score| bit pattern, then the selected channel indices in
// ascending order (one ballot per row when no tie is broken at the
// threshold, else an ordered compaction of the selection bitmap).
// ------------------------------------------------------------------------
template <int KPT>
__global__ __launch_bounds__(1024) void topk_kernel(const float *__restrict__ score, int n, int k,
                                                    int32_t *__restrict__ sel)
{
    __shared__ SelectSmem<65536> sm;
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {  // all loads issued before any use
        const int i = slot_index<KPT>(r);
        key[r] = __float_as_uint(score[i < n ? i : n - 1]);
    }
    // slots past n get the key 0xFFFFFFFF, which no selection step takes
#pragma unroll
    for (int r = 0; r < KPT; ++r) key[r] = (slot_index<KPT>(r) < n) ? (key[r] & 0x7FFFFFFFu) : 0xFFFFFFFFu;
    // scores are sign-free: the window is bits 30..0
    const SelectResult sr = block_select_window<1024, KPT>(key, n, k, 30, 0, sm);
    if (uniform_u32(sr.need_eq) == uniform_u32(sr.count_eq)) {  // no tie to break: key >= T
        emit_at_least<1024, KPT>(key, uniform_u32(sr.T), sel, (uint32_t)k, sm);
        return;
    }
    selection_bitmap<1024, KPT>(key, n, sr, sm);
    emit_bitmap<1024>(n, sm, [&](int i, uint32_t pos) {
        if (pos < (uint32_t)k) sel[pos] = i;
    });
}

// The same top-k for the scores of stage1_fused_kernel beyond the channels
// whose top-k it runs itself: its channel blocks' counts of their scores by
// exponent byte (256 16-bit fields per block, 128 words) are summed first,
// which is the first radix pass (bits 30..23) without a histogram of the
// keys; the passes over bits 22..0 then count only the keys of the crossing
// bin.  Thread t sums bins 4m..4m+3 (m = t mod 64) of the blocks t/64 + 16 i.
template <int KPT>
__global__ __launch_bounds__(1024) void topk_counts_kernel(const float *__restrict__ score, int n, int k,
                                                           int32_t *__restrict__ sel,
                                                           const uint32_t *__restrict__ blk_cnt, int n_blocks)
{
    constexpr int HB = 8;  // blocks a thread sums: at most 128
    __shared__ SelectSmem<65536> sm;
    const int tid = threadIdx.x;
    const CoherentBuf hbuf(blk_cnt, (uint32_t)(4 * 128 * n_blocks));  // blocks past n_blocks read 0
    float hc[HB][2];
#pragma unroll
    for (int i = 0; i < HB; ++i)
        hbuf.load2(8u * (uint32_t)((16 * i + (tid >> 6)) * 64 + (tid & 63)), hc[i][0], hc[i][1]);
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const int i = slot_index<KPT>(r);
        key[r] = __float_as_uint(score[i < n ? i : n - 1]);
    }
    uint32_t w0 = 0, w1 = 0;  // 16-bit fields add without carry: at most HB x 512 each
#pragma unroll
    for (int i = 0; i < HB; ++i) {
        w0 += __float_as_uint(hc[i][0]);
        w1 += __float_as_uint(hc[i][1]);
    }
    *reinterpret_cast<u32x4 *>(&sm.hist[(tid >> 6) * 256 + 4 * (tid & 63)]) =
        u32x4{w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
    __syncthreads();
    uint32_t h1[1] = {0u};
    if (tid < 256) {
#pragma unroll
        for (int g = 0; g < 16; ++g) h1[0] += sm.hist[g * 256 + tid];
    }
    find_crossing<1024, 1>(h1, (uint32_t)k, sm.scratch, sm.found);
    const uint32_t prefix = uniform_u32(sm.found[0]) << 23;
    const uint32_t rem = (uint32_t)k - uniform_u32(sm.found[1]), in_bin = uniform_u32(sm.found[2]);
    // slots past n get the key 0xFFFFFFFF, which no selection step takes
#pragma unroll
    for (int r = 0; r < KPT; ++r) key[r] = (slot_index<KPT>(r) < n) ? (key[r] & 0x7FFFFFFFu) : 0xFFFFFFFFu;
    SelectResult sr;
    if (rem == in_bin) {  // the whole bin is selected
        sr.T = prefix;
        sr.need_eq = sr.count_eq = rem;
    } else {
        sr = radix_select_from<1024, KPT>(key, n, prefix, 0xFF800000u, rem, 22, 0, sm);
    }
    if (uniform_u32(sr.need_eq) == uniform_u32(sr.count_eq)) {  // no tie to break: key >= T
        emit_at_least<1024, KPT>(key, uniform_u32(sr.T), sel, (uint32_t)k, sm);
        return;
    }
    selection_bitmap<1024, KPT>(key, n, sr, sm);
    emit_bitmap<1024>(n, sm, [&](int i, uint32_t pos) {
        if (pos < (uint32_t)k) sel[pos] = i;
    });
}

// ------------------------------------------------------------------------
// host-side launchers
// ------------------------------------------------------------------------
template <typename T>
static hipError_t launch_xselect_t(const void *x, int B, int d, int k_in, float *xh, uint32_t *counters,
                                   int n_counters, hipStream_t st, float norm_eps, void *xn_out)
{
    const int kpt = (d + 1023) / 1024;
    const T *xp = (const T *)x;
#define XS(K) \
    if (kpt <= K) {                                                                                             \
        xselect_kernel<T, K><<<B, 1024, 0, st>>>(xp, d, k_in, xh, counters, n_counters, norm_eps, (T *)xn_out); \
        return hipGetLastError();                                                                               \
    }
    XS(1) XS(2) XS(4) XS(8) XS(16)
#undef XS
    return hipErrorInvalidValue;
}

hipError_t launch_xselect(int dtype, const void *x, int B, int d, int k_in, float *xh, uint32_t *counters,
                          int n_counters, hipStream_t st, float norm_eps, void *xn_out)
{
    return dtype == 0 ? launch_xselect_t<float>(x, B, d, k_in, xh, counters, n_counters, st, norm_eps, xn_out)
                      : launch_xselect_t<uint16_t>(x, B, d, k_in, xh, counters, n_counters, st, norm_eps, xn_out);
}

hipError_t launch_proxy(const ProxyPlan &pl, const float *xh, int B, int d, int F, const uint8_t *codes,
                        const float *scales, float *part, float *score, uint32_t *counters, int act, int signal,
                        hipStream_t st)
{
    dim3 grid(pl.n_cblocks, pl.S);
#define PX(Q, N) \
    proxy_kernel<Q, N><<<grid, 256, 0, st>>>(xh, B, d, F, codes, scales, pl.R, pl.S, part, score, counters, act, signal)
    if (pl.qbits == 8) {
        if (pl.nb == 1) PX(8, 1);
        else if (pl.nb == 4) PX(8, 4);
        else if (pl.nb == 16) PX(8, 16);
        else return hipErrorInvalidValue;
    } else {
        if (pl.nb == 1) PX(4, 1);
        else if (pl.nb == 4) PX(4, 4);
        else return hipErrorInvalidValue;
    }
#undef PX
    return hipGetLastError();
}

hipError_t launch_topk_counts(const float *score, int n, int k, int32_t *sel, const uint32_t *blk_cnt,
                              int n_blocks, hipStream_t st)
{
    if (n_blocks < 1 || n_blocks > 128 || k < 1 || k > n) return hipErrorInvalidValue;
    const int kpt = (n + 1023) / 1024;
#define TK(K) \
    if (kpt <= K) { topk_counts_kernel<K><<<1, 1024, 0, st>>>(score, n, k, sel, blk_cnt, n_blocks); return hipGetLastError(); }
    TK(32) TK(64)
#undef TK
    return hipErrorInvalidValue;
}

hipError_t launch_topk(const float *score, int n, int k, int32_t *sel, hipStream_t st)
{
    const int kpt = (n + 1023) / 1024;
#define TK(K) \
    if (kpt <= K) { topk_kernel<K><<<1, 1024, 0, st>>>(score, n, k, sel); return hipGetLastError(); }
    TK(1) TK(2) TK(4) TK(8) TK(16) TK(32) TK(64)
#undef TK
    return hipErrorInvalidValue;
}

}  // namespace prox
