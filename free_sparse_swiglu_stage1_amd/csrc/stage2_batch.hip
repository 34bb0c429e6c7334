// Stage 2 of Prox (technical summary, "Stage 2: Exact Sparse Computation":
// exact gate/up, SiLU-multiply and the down projection on the selected
// channels) for batches of 2..16 tokens with bf16 activations, on the matrix
// cores.
//
// At B tokens each weight byte feeds B multiply-adds; at B = 16 that is above
// what the vector ALUs sustain at HBM speed, so both projections run on
// v_mfma_f32_16x16x32_bf16 with the tokens (padded to 16) as one operand.
// Every product is exact in fp32 (bf16 x bf16); the sums accumulate in fp32.
//
//  gu_batch_kernel   exact gate/up of 16 selected channels x 16 tokens over
//                    all inputs (or a chunk of them when there are few
//                    channels: then the last chunk to finish (ticket) adds
//                    the chunks' sums in chunk order) and writes s = act(g) u
//                    as three bf16 pieces (below).
//  dn_batch_kernel   y[b][m] = sum_r s[b][r] W_down^T[sel[r]][m] over 128
//                    columns per workgroup and a range of ranks; the
//                    last rank split of a column tile (ticket) adds the
//                    splits' partials in split order, scales (FP8), adds the
//                    residual and rounds.
//
// s in three pieces: s = p0 + p1 + p2 exactly, each a bf16 (p0 keeps the top
// 8 significand bits of s, p1 the next 8 of the remainder, p2 the rest), so
// the down projection multiplies the binary32 value of s, not a rounding of
// it.  The pieces live in sp[3][16 tokens][KP ranks] (KP = k rounded up to
// 32; ranks >= k and tokens >= B hold zeros).
//
// The down projection's contraction runs over ranks, which are rows of
// W_down^T: a lane loads 8 consecutive columns of 8 rows and regroups them
// with byte permutes into 8 operands of 8 rows x 1 column each.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace prox {

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBT = 16;                      // token slots of a tile (B padded)
constexpr int kGuWaves = 4;                  // waves per gate/up workgroup
constexpr int kGuWaveK = 256;                // inputs per wave
constexpr int kGuK = kGuWaves * kGuWaveK;    // inputs per gate/up workgroup
constexpr int kDnWaves = 8;                  // waves per down workgroup
constexpr int kGuSplitK = 512;               // inputs per chunk of a split gate/up tile
constexpr int kDnTargetWgs = 256;           // down workgroups aimed at (column tiles x rank splits)
constexpr int kDnMaxKps = 64;                // K-steps (32 ranks) per down workgroup, at most

// D[i][j] += sum_k A[i][k] B[k][j], 16 x 16 x 32.  Lane l holds A row l % 16
// and B column l % 16, elements k = 8 (l / 16) .. + 7 of each; D row
// 4 (l / 16) + r, column l % 16 in register r.
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
    __device__ __forceinline__ uint32_t load4(uint32_t off) const
    {
        return __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)off, 0, 0);
    }
    // device-coherent (partials written by other workgroups of this launch)
    __device__ __forceinline__ u32x4 load16_coherent(uint32_t off) const
    {
        return __builtin_bit_cast(u32x4,
                                  __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, CoherentBuf::kSc1));
    }
};

// Two binary32 values' upper halves (their bf16 truncations), a's in the low half.
__device__ __forceinline__ uint32_t pack_hi(float a, float b)
{
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// Eight E4M3 codes (two words, byte 0 first) as eight bf16 values (exact:
// an E4M3 value has at most 4 significand bits).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1)
{
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
    const auto e = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
    return u32x4{pack_hi(a[0], a[1]), pack_hi(b[0], b[1]), pack_hi(c[0], c[1]), pack_hi(e[0], e[1])};
}

// s = p0 + p1 + p2 exactly, each piece a bf16 (bit pattern returned).
__device__ __forceinline__ void split3(float s, uint16_t &p0, uint16_t &p1, uint16_t &p2)
{
    const uint32_t b0 = __float_as_uint(s) & 0xFFFF0000u;
    const float r1 = s - __uint_as_float(b0);  // exact: the low 16 significand bits
    const uint32_t b1 = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(b1);  // exact, at most 8 significant bits
    p0 = (uint16_t)(b0 >> 16);
    p1 = (uint16_t)(b1 >> 16);
    p2 = (uint16_t)(__float_as_uint(r2) >> 16);
}

// Runs issue(i, buf) for i = 0 .. n-1 and compute(buf) on each in order,
// with two buffers in flight.  Every issue sits unconditionally in its
// block: a load under a branch would make the compiler wait, where the
// branches meet, for the loads of whichever path issued fewer.  A
// scheduling barrier after each issue keeps the instruction scheduler from
// hoisting the previous buffer's MFMAs (and their waits) above the loads.
template <class Buf, class Issue, class Compute>
__device__ __forceinline__ void pipeline2(int n, Buf &A, Buf &B, Issue issue, Compute compute)
{
    if (n <= 0) return;
    issue(0, A);
    __builtin_amdgcn_sched_barrier(0);
    int i = 1;
    while (n - i >= 2) {
        issue(i, B);
        __builtin_amdgcn_sched_barrier(0);
        compute(A);
        issue(i + 1, A);
        __builtin_amdgcn_sched_barrier(0);
        compute(B);
        i += 2;
    }
    if (n - i == 1) {
        issue(i, B);
        __builtin_amdgcn_sched_barrier(0);
        compute(A);
        compute(B);
    } else {
        compute(A);
    }
}

}  // namespace

// ------------------------------------------------------------------------
// Gate/up.  1-D grid: tiles [0, n_full) whole, one workgroup each, then the
// tiles [n_full, ceil(k/16)) in SK input chunks of KW each; 4 waves.  n_full
// is a multiple of the CU count, so the whole tiles take one workgroup slot
// on every CU and the chunks of the rest fill second slots evenly (269
// whole tiles on 256 CUs left 13 CUs with two, which ended at 16 us against
// a median of 9.3; per-workgroup timestamps show each CU's share of the
// bandwidth, not a workgroup's, setting its pace).  Wave w takes the 256-input sub-chunks w, w + 4, ... of
// its range, two in flight.
//
// The MFMA wants channel l % 16 of the tile in lane l (A) and token l % 16
// (B).  Loading A that way makes each load instruction touch 16 rows, which
// streams at about half the rate of 4 rows per instruction, so the rows are
// loaded 4 at a time -- lanes 16 q' .. 16 q' + 15 read 256 contiguous bytes
// of row 4 q + q' -- and regrouped through a per-wave LDS tile (gate, then
// up).  Above 8 tokens x is read from L2 the same way, 4 tokens per
// instruction, and regrouped through a second tile: read as MFMA operands,
// 16 tokens per instruction, it cost 4.7 us of 22 at B = 16; at 4 tokens the
// extra LDS round trip costs more than it saves, and x is read as operands
// (token slots >= B read zeros either way).
// MFMA step t of a sub-chunk takes inputs 32 t + 8 g .. + 7 in lane group
// g = l / 16.
// ------------------------------------------------------------------------
template <typename TW>
struct GuRowsB;
template <> struct GuRowsB<uint16_t> {  // bf16: a sub-chunk row is 512 B, two 16-byte loads per lane
    static constexpr int LPR = 2;         // loads per row (per half) per lane
    static constexpr int PITCH = 528;     // LDS bytes per row (16-byte pad: conflict-free reads)
    static __device__ __forceinline__ u32x4 operand(const uint8_t *rowp, int t, int g)
    {
        return *reinterpret_cast<const u32x4 *>(rowp + 2 * (32 * t + 8 * g));
    }
};
template <> struct GuRowsB<uint8_t> {  // FP8: a sub-chunk row is 256 B, one 16-byte load per lane
    static constexpr int LPR = 1;
    static constexpr int PITCH = 272;
    static __device__ __forceinline__ u32x4 operand(const uint8_t *rowp, int t, int g)
    {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(rowp + 32 * t + 8 * g);
        return e4m3x8_to_bf16(v[0], v[1]);
    }
};

template <typename TW, bool XTILE>
__global__ __launch_bounds__(256) void gu_batch_kernel(const uint16_t *__restrict__ x, int B, int d, int F,
                                                       const TW *__restrict__ w_gu, const float *__restrict__ gsc,
                                                       const int32_t *__restrict__ sel, int k, int n_full, int SK,
                                                       int KW,
                                                       float *__restrict__ part, uint32_t *__restrict__ counters,
                                                       uint16_t *__restrict__ sp, int KP, int act,
                                                       int32_t *__restrict__ iota_out)
{
    constexpr int EPL = 16 / sizeof(TW);  // weights per 16-byte load
    constexpr int LPR = GuRowsB<TW>::LPR;
    constexpr int PITCH = GuRowsB<TW>::PITCH;
    constexpr int NLW = 4 * LPR;          // weight loads per half per sub-chunk
    constexpr int XPITCH = 528;  // LDS bytes per token row of a sub-chunk (256 bf16 + 16-byte pad)
    __shared__ __align__(16) uint8_t tiles[kGuWaves][16 * PITCH];
    __shared__ __align__(16) uint8_t xtiles[XTILE ? kGuWaves : 1][XTILE ? 16 * XPITCH : 16];
    __shared__ __align__(16) float red[kGuWaves * 2 * 64 * 4];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int L = blockIdx.x, split = L >= n_full;
    const int tile = split ? n_full + (L - n_full) / SK : L;
    const int kc = split ? (L - n_full) % SK : 0;
    const int c0 = kc * KW, c1 = split ? min(d, c0 + KW) : d;
    uint8_t *my = tiles[wv];
    uint8_t *myx = xtiles[wv];

    // lane l loads rows 4 q + g (q = 0..3) of the tile (ranks past k repeat
    // rank k - 1; not stored)
    const TW *grow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int rc = min(tile * 16 + 4 * q + g, k - 1);
        const int j = (int)min((uint32_t)(sel ? sel[rc] : rc), (uint32_t)(F - 1));
        grow[q] = w_gu + (int64_t)j * 2 * d;
    }
    const int rr = tile * 16 + li;
    if (iota_out && kc == 0 && wv == 0 && g == 0 && rr < k) iota_out[rr] = rr;
    const ZeroBuf xb(x, (uint32_t)(2u * B * d));
    constexpr bool xtile = XTILE;  // x through the LDS tile (else read as operands)

    struct Buf {
        u32x4 wg[NLW], wu[NLW], xv[8];
    };
    const int ibw = c0 + wv * kGuWaveK;
    auto issue = [&](int n, Buf &b) {  // this wave's n-th sub-chunk: inputs [ib, ib + 256)
        const int ib = ibw + n * kGuWaves * kGuWaveK;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int p = 0; p < LPR; ++p) {
                const int i = ib + (p * 16 + li) * EPL;
                const int ic = i < c1 ? i : 0;  // past the chunk: any row data, x reads 0 there
                b.wg[q * LPR + p] = ld_stream(grow[q] + ic);
                b.wu[q * LPR + p] = ld_stream(grow[q] + d + ic);
            }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                // tile: tokens 4 q + g, 256 contiguous bytes each; operands:
                // token li, inputs 32 t + 8 g (t = 2 q + p)
                const int tok = xtile ? 4 * q + g : li;
                const int i = ib + (xtile ? p * 128 + 8 * li : 32 * (2 * q + p) + 8 * g);
                b.xv[q * 2 + p] = xb.load16(tok < B && i < c1 ? (uint32_t)(2 * (tok * d + i)) : xb.end);
            }
    };
    f32x4 ag = {0.0f, 0.0f, 0.0f, 0.0f}, au = {0.0f, 0.0f, 0.0f, 0.0f};
    auto half = [&](const u32x4 (&w)[NLW], const u32x4 (&xv)[8], f32x4 &acc) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int p = 0; p < LPR; ++p)
                *reinterpret_cast<u32x4 *>(my + (4 * q + g) * PITCH + (p * 16 + li) * 16) = w[q * LPR + p];
        const uint8_t *rowp = my + li * PITCH;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc = mfma16(GuRowsB<TW>::operand(rowp, t, g), xv[t], acc);
    };
    auto compute = [&](const Buf &b) {
        if constexpr (xtile) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    *reinterpret_cast<u32x4 *>(myx + (4 * q + g) * XPITCH + (p * 128 + 8 * li) * 2) =
                        b.xv[q * 2 + p];
            u32x4 xo[8];  // the MFMA B operands: token li, inputs 32 t + 8 g .. + 7
#pragma unroll
            for (int t = 0; t < 8; ++t)
                xo[t] = *reinterpret_cast<const u32x4 *>(myx + li * XPITCH + (32 * t + 8 * g) * 2);
            half(b.wg, xo, ag);
            half(b.wu, xo, au);
        } else {
            half(b.wg, b.xv, ag);
            half(b.wu, b.xv, au);
        }
    };
    Buf b0, b1;
    const int nsub = uniform(ibw < c1 ? (c1 - ibw + kGuWaves * kGuWaveK - 1) / (kGuWaves * kGuWaveK) : 0);
    pipeline2(nsub, b0, b1, issue, compute);

    *reinterpret_cast<f32x4 *>(&red[((wv * 2 + 0) * 64 + lane) * 4]) = ag;
    *reinterpret_cast<f32x4 *>(&red[((wv * 2 + 1) * 64 + lane) * 4]) = au;
    __syncthreads();
    // thread t: gate (v0) and up (v1) of lane t / 4's register t % 4
    float v0 = ((red[tid] + red[512 + tid]) + red[1024 + tid]) + red[1536 + tid];
    float v1 = ((red[256 + tid] + red[768 + tid]) + red[1280 + tid]) + red[1792 + tid];
    if (split && SK > 1) {
        float *pp = part + ((int64_t)(tile - n_full) * SK + kc) * 512;
        store_agent2(&pp[2 * tid], v0, v1);
        if (!publish_and_ticket(&counters[tile], (uint32_t)SK, &s_last)) return;
        const ZeroBuf pb(part + (int64_t)(tile - n_full) * SK * 512, (uint32_t)(4 * SK * 512));
        v0 = v1 = 0.0f;
        for (int q0 = 0; q0 < SK; q0 += 8) {
            float a[8], b[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {  // past the last chunk: reads 0
                const uint32_t off = q0 + q < SK ? (uint32_t)(4 * ((q0 + q) * 512 + 2 * tid)) : pb.end;
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(pb.rsrc, (int)off, 0, CoherentBuf::kSc1);
                a[q] = __uint_as_float(v[0]);
                b[q] = __uint_as_float(v[1]);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q0 + q < SK) {
                    v0 += a[q];
                    v1 += b[q];
                }
        }
    }
    // s for channel 4 (lp / 16) + r of the tile, token lp % 16
    const int lp = tid >> 2, r = tid & 3;
    const int rank = tile * 16 + 4 * (lp >> 4) + r, tok = lp & 15;
    float s = 0.0f;
    if (rank < k) {
        if (gsc) {
            const int jj = (int)min((uint32_t)(sel ? sel[rank] : rank), (uint32_t)(F - 1));
            v0 *= gsc[2 * jj];
            v1 *= gsc[2 * jj + 1];
        }
        s = gate_act(act, v0) * v1;
    }
    uint16_t p0, p1, p2;
    split3(s, p0, p1, p2);
    sp[(0 * kBT + tok) * (int64_t)KP + rank] = p0;
    sp[(1 * kBT + tok) * (int64_t)KP + rank] = p1;
    sp[(2 * kBT + tok) * (int64_t)KP + rank] = p2;
    // the last tile also clears the ranks up to KP
    const int rz = (tile + 1) * 16 + (tid >> 4);
    if (tile == (k + 15) / 16 - 1 && rz < KP) {
#pragma unroll
        for (int p = 0; p < 3; ++p) sp[(p * kBT + (tid & 15)) * (int64_t)KP + rz] = 0;
    }
}

// ------------------------------------------------------------------------
// Down projection.  Grid (S rank splits, column tiles); 8 waves.  A column
// tile is 128 columns, NC = 8 per lane: 256 bytes of each bf16 row (against
// 128 with 64 columns, 0.5-0.8 us faster at 4 and 16 tokens) or 128 of each
// FP8 row.  Split s owns K-steps [s kps, (s+1) kps) of 32 ranks; wave w takes
// every 8th of them, two in flight.  In a K-step lane l's group g = l / 16
// owns ranks 8g .. 8g+7 and lane l % 16 owns columns NC (l % 16) .. + NC - 1:
// it loads those columns of its 8 rows (16 or 8 bytes a row) and builds, for each
// column c, the operand of the 8 rows' values in column c (MFMA c: output
// columns NC j + c, j = 0..15).  The A operand is token l % 16's pieces of s
// for the same 8 ranks.
// ------------------------------------------------------------------------
template <typename TW>
struct DnRows;
template <> struct DnRows<uint16_t> {  // bf16: 8 columns a row, one 16-byte load
    static constexpr int NC = 8;
    using row_t = u32x4;
    static __device__ __forceinline__ row_t load(const uint16_t *p) { return ld_stream(p); }
    // operands of columns C0 and C0 + 1 (C0 even) of 8 rows
    template <int C0>
    static __device__ __forceinline__ void operands(const row_t (&w)[8], u32x4 &o0, u32x4 &o1)
    {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t lo = w[2 * p][C0 >> 1], hi = w[2 * p + 1][C0 >> 1];
            o0[p] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            o1[p] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
        }
    }
};
template <> struct DnRows<uint8_t> {  // FP8: 8 columns a row, one 8-byte load
    static constexpr int NC = 8;
    using row_t = u32x2;
    static __device__ __forceinline__ row_t load(const uint8_t *p) { return ld_stream8(p); }
    template <int C0>
    static __device__ __forceinline__ void operands(const row_t (&w)[8], u32x4 &o0, u32x4 &o1)
    {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[2 * p][C0 >> 2], (C0 & 2) != 0);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[2 * p + 1][C0 >> 2], (C0 & 2) != 0);
            o0[p] = pack_hi(lo[0], hi[0]);
            o1[p] = pack_hi(lo[1], hi[1]);
        }
    }
};

template <typename TW>
__global__ __launch_bounds__(512) void dn_batch_kernel(const uint16_t *__restrict__ sp, int KP, int k, int B, int d,
                                                       int F, const TW *__restrict__ wdt,
                                                       const float *__restrict__ dsc, const int32_t *__restrict__ sel,
                                                       int kps, int S, float *__restrict__ part,
                                                       const uint16_t *residual,  // may alias out
                                                       uint16_t *out, uint32_t *__restrict__ counters)
{
    constexpr int NC = DnRows<TW>::NC;
    constexpr int COLS = 16 * NC;
    constexpr int CPT = COLS / 32;  // output columns per thread at the end
    __shared__ int ssel[kDnMaxKps * 32];
    __shared__ __align__(16) float red[4][kBT][COLS];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int s = blockIdx.x, ct = blockIdx.y;
    const int KS = KP / 32;
    const int ks0 = s * kps, ks1 = min(KS, ks0 + kps);
    const int m0 = ct * COLS;
    const int col = m0 + NC * li < d ? m0 + NC * li : 0;  // past d: any column, not stored

    // the split's channel indices (ranks past k: channel 0, whose s is 0)
    {
        const ZeroBuf sb(sel, sel ? (uint32_t)(4 * k) : 0u);
        for (int e = tid; e < (ks1 - ks0) * 32; e += 512) {
            const int rank = ks0 * 32 + e;
            const uint32_t jj = sel ? sb.load4((uint32_t)(4 * rank)) : (uint32_t)(rank < k ? rank : 0);
            ssel[e] = (int)min(jj, (uint32_t)(F - 1));
        }
    }
    __syncthreads();

    f32x4 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    struct Buf {
        typename DnRows<TW>::row_t w[8];
        u32x4 a[3];
    };
    auto issue = [&](int n, Buf &b) {  // this wave's n-th K-step
        const int rb = (ks0 + wv + n * kDnWaves) * 32 + 8 * g;
        const int *sl = &ssel[rb - ks0 * 32];
#pragma unroll
        for (int e = 0; e < 8; ++e) b.w[e] = DnRows<TW>::load(wdt + (int64_t)sl[e] * d + col);
#pragma unroll
        for (int p = 0; p < 3; ++p)
            b.a[p] = *reinterpret_cast<const u32x4 *>(sp + (int64_t)(p * kBT + li) * KP + rb);
    };
    auto pair = [&](const u32x4 &o0, const u32x4 &o1, const u32x4 (&a)[3], f32x4 &c0, f32x4 &c1) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            c0 = mfma16(a[p], o0, c0);
            c1 = mfma16(a[p], o1, c1);
        }
    };
    auto compute = [&](const Buf &b) {
        u32x4 o0, o1;
        DnRows<TW>::template operands<0>(b.w, o0, o1);
        pair(o0, o1, b.a, acc[0], acc[1]);
        DnRows<TW>::template operands<2>(b.w, o0, o1);
        pair(o0, o1, b.a, acc[2], acc[3]);
        if constexpr (NC == 8) {
            DnRows<TW>::template operands<4>(b.w, o0, o1);
            pair(o0, o1, b.a, acc[4], acc[5]);
            DnRows<TW>::template operands<6>(b.w, o0, o1);
            pair(o0, o1, b.a, acc[6], acc[7]);
        }
    };
    Buf b0, b1;
    const int nks = uniform(ks0 + wv < ks1 ? (ks1 - ks0 - wv + kDnWaves - 1) / kDnWaves : 0);
    pipeline2(nks, b0, b1, issue, compute);

    // waves w and w + 4 pair up, then the four pairs are added in order;
    // acc[c][r]: token 4 g + r, column NC li + c
    if (wv >= 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c) red[wv - 4][4 * g + r][NC * li + c] = acc[c][r];
    }
    __syncthreads();
    if (wv < 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[c][r] += red[wv][4 * g + r][NC * li + c];
    }
    __syncthreads();
    if (wv < 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c) red[wv][4 * g + r][NC * li + c] = acc[c][r];
    }
    __syncthreads();
    // thread t: token t / 32, columns CPT (t % 32) .. + CPT - 1 of the tile
    const int tok = tid >> 5, cq = (tid & 31) * CPT, m = m0 + cq;
    const bool mine = tok < B && m < d;
    float y[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q)
        y[q] = ((red[0][tok][cq + q] + red[1][tok][cq + q]) + red[2][tok][cq + q]) + red[3][tok][cq + q];
    if (S > 1) {
        if (mine) {
            float *pp = part + ((int64_t)s * B + tok) * d + m;
#pragma unroll
            for (int q = 0; q < CPT; q += 2) store_agent2(pp + q, y[q], y[q + 1]);
        }
        if (!publish_and_ticket(&counters[ct], (uint32_t)S, &s_last)) return;
        const ZeroBuf pb(part, (uint32_t)(4u * S * B * d));
        const uint32_t base = mine ? (uint32_t)(4 * (tok * d + m)) : pb.end;
        const uint32_t stride = (uint32_t)(4 * B * d);
#pragma unroll
        for (int q = 0; q < CPT; ++q) y[q] = 0.0f;
        for (int q0 = 0; q0 < S; q0 += 8) {
            float v[8][CPT];
#pragma unroll
            for (int q = 0; q < 8; ++q) {  // past the last split, or not this thread's: reads 0
                const uint32_t off = q0 + q < S && mine ? base + (uint32_t)(q0 + q) * stride : pb.end;
                if constexpr (CPT == 4) {
                    const u32x4 w4 = pb.load16_coherent(off);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[q][e] = __uint_as_float(w4[e]);
                } else {
                    const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(pb.rsrc, (int)off, 0, CoherentBuf::kSc1);
                    v[q][0] = __uint_as_float(w2[0]);
                    v[q][1] = __uint_as_float(w2[1]);
                }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q0 + q < S) {
#pragma unroll
                    for (int e = 0; e < CPT; ++e) y[e] += v[q][e];
                }
        }
    }
    if (!mine) return;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
        float v = y[q];
        if (dsc) v *= dsc[m + q];
        if (residual) v += elem<uint16_t>::load(residual, (int64_t)tok * d + m + q);
        elem<uint16_t>::store(out, (int64_t)tok * d + m + q, v);
    }
}

// ------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------
BatchPlan batch_plan(int d, int k, int B, int fp8)
{
    BatchPlan p;
    p.n_tiles = (k + 15) / 16;
    // whole tiles in multiples of the CU count; the rest in input chunks.
    // The CUs share the bandwidth about evenly, so the chunks are small:
    // 512 inputs (16 KB of a bf16 tile) on top of a CU's whole tile.
    // Measured at 4301 channels: 1024-input chunks (64 KB on 52 CUs) ended
    // Stage 2 about 1 us later, 256-input ones (16 partials a tile) 0.2 us.
    // Without whole tiles, chunks of 1024 (one per wave of 4 x 256).
    constexpr int kCUs = 256;
    const int unit = kGuWaves * kGuWaveK;
    p.n_full = p.n_tiles / kCUs * kCUs;
    p.KW = p.n_full > 0 ? kGuSplitK : unit;
    p.SK = (d + p.KW - 1) / p.KW;
    p.KP = (k + 31) / 32 * 32;
    const int KS = p.KP / 32;
    const int cols = 128;
    p.n_ct = (d + cols - 1) / cols;
    // rank splits: about 2048 waves, partials (S B d floats, written and
    // read back) under about 1/8 of the down rows' bytes (k d b_w), at least
    // 8 K-steps per split, at most kDnMaxKps
    int S = (kDnTargetWgs + p.n_ct - 1) / p.n_ct;
    const int cap = fp8 ? k / (64 * B) : k / (32 * B);
    if (S > cap) S = cap;
    if (S > (KS + 7) / 8) S = (KS + 7) / 8;
    const int smin = (KS + kDnMaxKps - 1) / kDnMaxKps;
    if (S < smin) S = smin;
    if (S < 1) S = 1;
    p.kps = (KS + S - 1) / S;
    p.S = (KS + p.kps - 1) / p.kps;
    return p;
}

size_t batch_gu_part_floats(int d, int F)
{
    // (n_tiles - n_full) SK 512 at most: fewer than 256 split tiles, of
    // at most ceil(d / 256) chunks
    const int tiles = (F + 15) / 16;
    return (size_t)(tiles < 255 ? tiles : 255) * (size_t)((d + kGuWaveK - 1) / kGuWaveK) * 512;
}

int batch_max_splits(int d, int F)
{
    const int n_ct = (d + 127) / 128;
    const int a = (kDnTargetWgs + n_ct - 1) / n_ct;
    const int b = ((F + 31) / 32 + kDnMaxKps - 1) / kDnMaxKps;
    return a > b ? a : b;
}

hipError_t launch_stage2_batch(const S2Weights &w, const void *x, int B, int d, int F, const int32_t *sel, int k,
                               const BatchPlan &pl, float *gu_part, uint16_t *s_pieces, float *dn_part,
                               const void *residual, void *out, uint32_t *gu_counters, uint32_t *dn_counters,
                               int32_t *iota_out, hipStream_t st)
{
    if (k <= 0 || B < 2 || B > kBT) return hipErrorInvalidValue;
    if (pl.kps > kDnMaxKps || pl.n_ct > kDownSliceEnd - kDownSliceBase) return hipErrorInvalidValue;
    const dim3 ggrid(pl.n_full + (pl.n_tiles - pl.n_full) * pl.SK), dgrid(pl.S, pl.n_ct);
    const uint16_t *xp = (const uint16_t *)x;
    // x through the LDS tile above 8 tokens (see gu_batch_kernel)
#define GU(TW, XT, SC)                                                                                          \
    gu_batch_kernel<TW, XT><<<ggrid, 256, 0, st>>>(xp, B, d, F, (const TW *)w.w_gu, SC, sel, k, pl.n_full, pl.SK, \
                                                   pl.KW,                                                        \
                                                   gu_part, gu_counters, s_pieces, pl.KP, w.act, iota_out)
    if (w.fmt == 1) {
        if (B > 8) GU(uint8_t, true, w.gu_scales);
        else GU(uint8_t, false, w.gu_scales);
    } else {
        if (B > 8) GU(uint16_t, true, nullptr);
        else GU(uint16_t, false, nullptr);
    }
#undef GU
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (w.fmt == 1) {
        dn_batch_kernel<uint8_t><<<dgrid, 512, 0, st>>>(s_pieces, pl.KP, k, B, d, F, (const uint8_t *)w.w_down_t,
                                                        w.down_scales, sel, pl.kps, pl.S, dn_part,
                                                        (const uint16_t *)residual, (uint16_t *)out, dn_counters);
    } else {
        dn_batch_kernel<uint16_t><<<dgrid, 512, 0, st>>>(s_pieces, pl.KP, k, B, d, F, (const uint16_t *)w.w_down_t,
                                                         nullptr, sel, pl.kps, pl.S, dn_part,
                                                         (const uint16_t *)residual, (uint16_t *)out, dn_counters);
    }
    return hipGetLastError();
}

}  // namespace prox
