// Stage 1 of Prox for batches of 2..16 tokens with bf16 activations: the
// proxy gate/up projections on the matrix cores ("Lightweight Proxy
// Construction": g~ = sum over kept inputs of x_i q_ij, scaled per channel).
//
// At B tokens each code byte feeds 2 B multiply-adds (gate and up); at
// B = 16 the vector ALUs cannot keep up with HBM, so the contraction runs on
// v_mfma_f32_16x16x32_bf16 with the tokens (padded to 16) as one operand.
// int8 codes and bf16 inputs are exact in bf16, so every product is exact in
// fp32; the sums accumulate in fp32.
//
// proxy_batch_kernel: grid (ceil(F/128) channel blocks, S input splits of R
// inputs); 4 waves, all on the block's 128 channels (gate and up).  The
// prologue lists the split's inputs that some token kept (the codes of the
// others are never read) and lays their x values out in LDS as MFMA
// operands.  A K-step is 32 listed inputs; wave w takes K-steps w, w + 4, ...,
// two in flight.  Lane l loads 8 channels (8 bytes) of 8 code rows -- the
// K-step's inputs 8 g .. 8 g + 7, g = l / 16 -- so one load instruction reads
// 128 contiguous bytes of each of 4 rows; for each of its 8 channels it then
// builds the 8 rows' codes as bf16 (sign-extending byte extracts) for an MFMA
// whose output rows are the channels 8 i + c of the block.  The waves' sums
// are added in LDS in a fixed order; with S > 1 the split's partial g~, u~ go
// to `part` and the last split of a channel block (ticket) adds them in split
// order.  That workgroup writes score_j = sum_b of the salience term.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace prox {

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPxWaves = 4;
constexpr int kPxCh = 128;     // channels per workgroup
constexpr int kPxMaxR = 1024;  // inputs per split, at most

__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// 16-byte loads through a buffer resource: an offset at or beyond `bytes`
// reads zeros without touching memory.
struct ZeroBuf {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t end;
    __device__ __forceinline__ ZeroBuf(const void *base, uint32_t bytes)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                                 CoherentBuf::kWord3)),
          end(bytes)
    {
    }
    __device__ __forceinline__ u32x4 load16(uint32_t off) const
    {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 0));
    }
};

// the upper halves of two binary32 values, a's in the low half
__device__ __forceinline__ uint32_t pack_hi(float a, float b)
{
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// byte C of the 8 bytes `w` as a signed integer, in binary32
template <int C>
__device__ __forceinline__ float code(const u32x2 &w)
{
    return (float)(int8_t)(w[C >> 2] >> (8 * (C & 3)));
}

// the MFMA operand of channel C: the 8 rows' codes as bf16
template <int C>
__device__ __forceinline__ u32x4 rows_operand(const u32x2 (&w)[8])
{
    return u32x4{pack_hi(code<C>(w[0]), code<C>(w[1])), pack_hi(code<C>(w[2]), code<C>(w[3])),
                 pack_hi(code<C>(w[4]), code<C>(w[5])), pack_hi(code<C>(w[6]), code<C>(w[7]))};
}

}  // namespace

__global__ __launch_bounds__(256) void proxy_batch_kernel(const float *__restrict__ xh, int B, int d, int F,
                                                          const uint8_t *__restrict__ codes,
                                                          const float *__restrict__ scales, int R, int S,
                                                          float *__restrict__ part, float *__restrict__ score,
                                                          uint32_t *__restrict__ counters, int act, int signal)
{
    __shared__ __align__(16) uint16_t xt[kPxMaxR / 32][4][16][8];  // [K-step][g][token][8 inputs], 32 KB
    __shared__ int lst[kPxMaxR];                                    // the listed inputs
    __shared__ __align__(16) uint32_t scr[64];
    __shared__ int s_last;
    float *red = reinterpret_cast<float *>(&xt[0][0][0][0]);  // after the MFMAs: [2][16 tokens][2][128]

    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int cb = blockIdx.x, s = blockIdx.y;
    const int i0 = s * R, i1 = min(d, i0 + R);
    const int c0 = cb * kPxCh;

    // ---- prologue: the inputs of [i0, i1) some token kept, and their x.
    // Thread t reads inputs i0 + 4t .. + 3 of every token, all 16-byte loads
    // issued at once (past i1 or past the tokens: zeros), and keeps them for
    // the layout below.
    const ZeroBuf xb(xh, (uint32_t)(4u * B * d));
    const int ix = i0 + 4 * tid;
    u32x4 xv[16];
#pragma unroll
    for (int b = 0; b < 16; ++b)
        xv[b] = xb.load16(b < B && ix < i1 ? (uint32_t)(4 * (b * d + ix)) : xb.end);
    uint32_t keep = 0;  // bit q: input ix + q is kept by some token (+0 and -0 are not)
#pragma unroll
    for (int b = 0; b < 16; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) keep |= ((xv[b][q] << 1) != 0u ? 1u : 0u) << q;
    uint32_t tot;
    int p = (int)block_excl_scan<256>((uint32_t)__popc(keep), scr, &tot);
    const int nk = (int)tot;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (keep & (1u << q)) {
            lst[p] = ix + q;
#pragma unroll
            for (int b = 0; b < 16; ++b) xt[p >> 5][(p >> 3) & 3][b][p & 7] = (uint16_t)(xv[b][q] >> 16);
            ++p;
        }
    const int nk32 = (nk + 31) & ~31;  // the last K-step padded with input i0 and x = 0
    for (int p = nk + tid; p < nk32; p += 256) {
        lst[p] = i0;
#pragma unroll
        for (int b = 0; b < 16; ++b) xt[p >> 5][(p >> 3) & 3][b][p & 7] = 0;
    }
    __syncthreads();

    // ---- MFMAs: lane l owns channels c0 + 8 li .. + 7 (clamped into [0, F))
    const int ch = min(c0 + 8 * li, F - 8);
    const int64_t rowlen = 2 * (int64_t)F;
    f32x4 ag[8], au[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) ag[c] = au[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    struct Buf {
        u32x2 wg[8], wu[8];
    };
    const int nks = nk32 / 32;
    const int nmine = uniform(wv < nks ? (nks - wv + kPxWaves - 1) / kPxWaves : 0);
    // codes through a buffer resource: a K-step past this wave's last loads
    // through an empty resource (zeros, no memory access), so the loop below
    // has no branch around its loads
    const uint32_t code_bytes = (uint32_t)((int64_t)d * rowlen);
    const auto rs_codes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(codes), (short)0,
                                                            (int)code_bytes, CoherentBuf::kWord3);
    const auto rs_none = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(codes), (short)0, 0,
                                                           CoherentBuf::kWord3);
    constexpr int kNt = 2;  // cache policy: streaming
    auto issue = [&](int n, Buf &b) {
        const int t = n < nmine ? wv + n * kPxWaves : wv;
        const auto rs = n < nmine ? rs_codes : rs_none;
        const int p0 = t * 32 + 8 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t off = (uint32_t)((int64_t)lst[p0 + e] * rowlen + ch);
            b.wg[e] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, kNt));
            b.wu[e] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(off + F), 0, kNt));
        }
    };
    auto compute = [&](int n, const Buf &b) {  // a K-step past the last: codes 0 times a finite x, adds 0
        const int t = n < nmine ? wv + n * kPxWaves : wv;
        const u32x4 xb = *reinterpret_cast<const u32x4 *>(&xt[t][g][li][0]);
        ag[0] = mfma16(rows_operand<0>(b.wg), xb, ag[0]);
        au[0] = mfma16(rows_operand<0>(b.wu), xb, au[0]);
        __builtin_amdgcn_sched_barrier(0);  // one channel's operands live at a time
        ag[1] = mfma16(rows_operand<1>(b.wg), xb, ag[1]);
        au[1] = mfma16(rows_operand<1>(b.wu), xb, au[1]);
        __builtin_amdgcn_sched_barrier(0);  // one channel's operands live at a time
        ag[2] = mfma16(rows_operand<2>(b.wg), xb, ag[2]);
        au[2] = mfma16(rows_operand<2>(b.wu), xb, au[2]);
        __builtin_amdgcn_sched_barrier(0);  // one channel's operands live at a time
        ag[3] = mfma16(rows_operand<3>(b.wg), xb, ag[3]);
        au[3] = mfma16(rows_operand<3>(b.wu), xb, au[3]);
        __builtin_amdgcn_sched_barrier(0);  // one channel's operands live at a time
        ag[4] = mfma16(rows_operand<4>(b.wg), xb, ag[4]);
        au[4] = mfma16(rows_operand<4>(b.wu), xb, au[4]);
        __builtin_amdgcn_sched_barrier(0);  // one channel's operands live at a time
        ag[5] = mfma16(rows_operand<5>(b.wg), xb, ag[5]);
        au[5] = mfma16(rows_operand<5>(b.wu), xb, au[5]);
        __builtin_amdgcn_sched_barrier(0);  // one channel's operands live at a time
        ag[6] = mfma16(rows_operand<6>(b.wg), xb, ag[6]);
        au[6] = mfma16(rows_operand<6>(b.wu), xb, au[6]);
        __builtin_amdgcn_sched_barrier(0);  // one channel's operands live at a time
        ag[7] = mfma16(rows_operand<7>(b.wg), xb, ag[7]);
        au[7] = mfma16(rows_operand<7>(b.wu), xb, au[7]);
        __builtin_amdgcn_sched_barrier(0);  // one channel's operands live at a time
    };
    Buf b0, b1;
    issue(0, b0);
    __builtin_amdgcn_sched_barrier(0);
    for (int n = 0; n < nmine; n += 2) {  // two K-steps in flight
        issue(n + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        compute(n, b0);
        issue(n + 2, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute(n + 1, b1);
    }

    // ---- the four waves' sums: (w0 + w2) + (w1 + w3), through LDS.
    // a[c][r]: channel 8 (4 g + r) + c of the block, token li
    __syncthreads();  // x no longer read
    // (register r of MFMA c: channels 8 (4 g + r) + c, c = 0..7 contiguous)
    auto put = [&](int slot) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float *dg = &red[((slot * 16 + li) * 2 + 0) * kPxCh + 8 * (4 * g + r)];
            float *du = dg + kPxCh;
            *reinterpret_cast<f32x4 *>(dg) = f32x4{ag[0][r], ag[1][r], ag[2][r], ag[3][r]};
            *reinterpret_cast<f32x4 *>(dg + 4) = f32x4{ag[4][r], ag[5][r], ag[6][r], ag[7][r]};
            *reinterpret_cast<f32x4 *>(du) = f32x4{au[0][r], au[1][r], au[2][r], au[3][r]};
            *reinterpret_cast<f32x4 *>(du + 4) = f32x4{au[4][r], au[5][r], au[6][r], au[7][r]};
        }
    };
    auto add = [&](int slot) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float *dg = &red[((slot * 16 + li) * 2 + 0) * kPxCh + 8 * (4 * g + r)];
            const float *du = dg + kPxCh;
            const f32x4 g0 = *reinterpret_cast<const f32x4 *>(dg), g1 = *reinterpret_cast<const f32x4 *>(dg + 4);
            const f32x4 u0 = *reinterpret_cast<const f32x4 *>(du), u1 = *reinterpret_cast<const f32x4 *>(du + 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                ag[c][r] += g0[c];
                ag[c + 4][r] += g1[c];
                au[c][r] += u0[c];
                au[c + 4][r] += u1[c];
            }
        }
    };
    if (wv >= 2) put(wv - 2);
    __syncthreads();
    if (wv < 2) add(wv);
    __syncthreads();
    if (wv == 1) put(0);
    __syncthreads();
    if (wv == 0) {
        add(0);
        put(0);
    }
    __syncthreads();
    // red[0][b][h][ci]: the workgroup's g~ (h = 0) and u~ (h = 1), unscaled

    if (S > 1) {
        // element pairs e, e + 1 = (b, h, ci) of the block, e = 2 (t + 256 m):
        // 64-bit coherent stores, and for the last split 64-bit coherent
        // loads, every split's in one batch, added in split order
        constexpr int MP = 16 * 2 * kPxCh / 2 / 256;  // pairs per thread at 16 tokens
        for (int m = 0; m < MP; ++m) {
            const int e = 2 * (tid + 256 * m);
            const int b = e / (2 * kPxCh), h = (e / kPxCh) & 1, j = c0 + e % kPxCh;
            if (b < B && j < F) store_agent2(&part[(((int64_t)s * B + b) * 2 + h) * F + j], red[e], red[e + 1]);
        }
        if (!publish_and_ticket(&counters[cb], (uint32_t)S, &s_last)) return;
        const ZeroBuf pb(part, (uint32_t)(4u * S * B * 2 * F));
        float acc[MP][2];
#pragma unroll
        for (int m = 0; m < MP; ++m) acc[m][0] = acc[m][1] = 0.0f;
        for (int q0 = 0; q0 < S; q0 += 4) {
            u32x2 v[4][MP];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int m = 0; m < MP; ++m) {
                    const int e = 2 * (tid + 256 * m);
                    const int b = e / (2 * kPxCh), h = (e / kPxCh) & 1, j = c0 + e % kPxCh;
                    const bool ok = q0 + q < S && b < B && j < F;
                    const uint32_t off = ok ? (uint32_t)(4 * ((((q0 + q) * B + b) * 2 + h) * F + j)) : pb.end;
                    v[q][m] = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_raw_buffer_load_b64(pb.rsrc, (int)off, 0, CoherentBuf::kSc1));
                }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int m = 0; m < MP; ++m)
                    if (q0 + q < S) {
                        acc[m][0] += __uint_as_float(v[q][m][0]);
                        acc[m][1] += __uint_as_float(v[q][m][1]);
                    }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MP; ++m) {
            const int e = 2 * (tid + 256 * m);
            red[e] = acc[m][0];
            red[e + 1] = acc[m][1];
        }
        __syncthreads();
    }
    // ---- scores of the block's channels (thread t < 128: channel c0 + t)
    const int j = c0 + tid;
    if (tid >= kPxCh || j >= F) return;
    const float sg = scales[j], su = scales[F + j];
    float sc = 0.0f;
    for (int b = 0; b < B; ++b)
        sc += salience(signal, act, red[(b * 2 + 0) * kPxCh + tid] * sg, red[(b * 2 + 1) * kPxCh + tid] * su);
    score[j] = sc;
}

int proxy_batch_splits(int d) { return (d + kPxMaxR - 1) / kPxMaxR; }

hipError_t launch_proxy_batch(const float *xh, int B, int d, int F, const uint8_t *codes, const float *scales,
                              float *part, float *score, uint32_t *counters, int act, int signal, hipStream_t st)
{
    if (B < 2 || B > 16 || F % 16 != 0) return hipErrorInvalidValue;
    // splits of a multiple of 32 inputs: the prologue reads 4 at a time
    const int R = ((d + proxy_batch_splits(d) - 1) / proxy_batch_splits(d) + 31) / 32 * 32;
    const int S = (d + R - 1) / R;
    const int n_cb = (F + kPxCh - 1) / kPxCh;
    if (R > kPxMaxR || n_cb > kFusedScoreSlot) return hipErrorInvalidValue;
    proxy_batch_kernel<<<dim3(n_cb, S), 256, 0, st>>>(xh, B, d, F, codes, scales, R, S, part, score, counters, act,
                                                       signal);
    return hipGetLastError();
}

}  // namespace prox
