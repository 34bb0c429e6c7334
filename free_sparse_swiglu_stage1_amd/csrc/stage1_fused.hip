// Stage 1 of Prox for one token in a single kernel: input sparsification,
// proxy gate/up GEMV, channel salience and the top-k channel mask
// ("Lightweight Proxy Construction").  Fusing the four steps removes three
// dependent launches, each worth a few microseconds on this device, from a
// step that streams ~60 MB of codes in ~10 us.
//
// Grid (channel blocks, input splits) sized to one wave of workgroups, two
// per CU; 512 threads.  Every workgroup
//  1. selects the kept inputs itself (every workgroup takes the same exact
//     decision on the same keys) and lists those of its input split in LDS,
//     in ascending order;
//  2. streams the code rows of those inputs for its CB channels, 32 rows in
//     flight per wave, one 32-bit code word per lane per half (gate, up);
//  3. adds its eight waves' sums in LDS in a fixed order and publishes the
//     split's partial g~ / u~ with coherent 64-bit stores.
// The last split of a channel block to finish (ticket) adds the partials in
// split order and publishes score_j = |silu(g~_j) u~_j| for its channels,
// with a count of them by exponent byte (256 bins); the last channel block to
// finish (ticket) loads all F scores and those counts, whose sum is the first
// radix pass of the top-k, and writes the k selected channel indices in
// ascending order.  Bitwise deterministic.
//
// Above kFusedMaxF channels the kernel stops at the scores and their counts
// (topk_here = 0) and launch_stage1_fused adds a top-k launch that starts
// from the counts.
//
// Counters: counters[cb] and counters[kFusedScoreSlot] must be zero on
// entry; the last arriver of each ticket resets it, so a completed launch
// leaves them zero again.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"
#include "select.h"

namespace prox {

constexpr int kFT = 512;          // threads per workgroup
constexpr int kFW = kFT / 64;     // waves per workgroup
constexpr int kFRows = 32;        // kept inputs in flight per wave
constexpr int kFusedSlots = 512;  // workgroups resident at once (two per CU)
constexpr int kCoarseBins = 256;  // score counts per channel block: bits 30..23 of the key

template <int QBITS>
struct Fused;
template <> struct Fused<8> {  // 4 signed bytes -> channels c..c+3
    static constexpr int CPL = 4, RMAX = 2048, GRAN = 32, NG = 1;
    static __device__ __forceinline__ void decode(uint32_t w, float *q)
    {
#pragma unroll
        for (int n = 0; n < 4; ++n) q[n] = (float)(int8_t)(w >> (8 * n));
    }
};
template <> struct Fused<4> {  // 8 biased nibbles; byte p holds channels 2p (low), 2p+1 (high)
    static constexpr int CPL = 8, RMAX = 1024, GRAN = 128, NG = 1024 / 128;
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

template <int QBITS>
struct FusedSmem {
    static constexpr int CB = 64 * Fused<QBITS>::CPL;
    int li[Fused<QBITS>::RMAX];    // this split's kept inputs, ascending
    float lx[Fused<QBITS>::RMAX];  // their values
    union {
        SelectSmem<kFusedMaxF> sel;
        struct {
            float red[kFW][2][CB];
            float gsc[Fused<QBITS>::NG][2][QBITS == 4 ? CB : 1];
        } p;
    };
    int flag;
};

template <typename T, int QBITS, int KX, int KF>
__global__ __launch_bounds__(kFT, 4) void stage1_fused_kernel(const T *__restrict__ x, int d, int F, int k_in, int k,
                                                           const uint8_t *__restrict__ codes,
                                                           const float *__restrict__ scales, int R, int S,
                                                           int n_cblocks, float *__restrict__ part,
                                                           float *__restrict__ score, int32_t *__restrict__ sel,
                                                           uint32_t *__restrict__ counters, int act, int signal,
                                                           float norm_eps, T *__restrict__ xn_out, int topk_here)
{
    using Q = Fused<QBITS>;
    constexpr int CPL = Q::CPL;
    constexpr int CB = 64 * CPL;  // channels per workgroup
    constexpr int U = kFRows;
    __shared__ FusedSmem<QBITS> sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int cb = blockIdx.x, s = blockIdx.y;
    const int i0 = s * R, i1 = min(d, i0 + R);
    const int64_t half_bytes = (int64_t)F * QBITS / 8;
    // the channel blocks' score counts follow the split partials
    uint32_t *const blk_hist = reinterpret_cast<uint32_t *>(part + (int64_t)S * 2 * F);
    const int c = cb * CB + lane * CPL;
    const int cc = c < F ? c : 0;

    // ---- 1. input selection; x (and the int4 group scales) loaded first
    constexpr int XR = Q::RMAX / kFT;  // list rows of this split
    float xv[KX], xr[XR];
#pragma unroll
    for (int r = 0; r < KX; ++r) xv[r] = elem<T>::load(x, min(slot_index<KX>(r), d - 1));
#pragma unroll
    for (int q = 0; q < XR; ++q) xr[q] = elem<T>::load(x, min(i0 + q * kFT + tid, d - 1));
    constexpr int GS = QBITS == 4 ? Q::NG * 2 * CB / kFT : 1;  // group scales per thread
    float gs_reg[GS];
    if (QBITS == 4) {
        const int ng = (i1 - i0 + 127) / 128;
#pragma unroll
        for (int q = 0; q < GS; ++q) {
            const int e = tid + q * kFT;
            const int g = e / (2 * CB), h = (e / CB) & 1, j = min(cb * CB + e % CB, F - 1);
            gs_reg[q] = scales[((int64_t)(i0 / 128 + min(g, ng - 1)) * 2 + h) * F + j];
        }
    }
    if (norm_eps >= 0.0f) {  // x is h: use RMSNorm(h) (uniform branch)
        // the squares summed as rmsnorm_kernel sums them: threads 0..255,
        // each over its 16-byte vectors t + 256 q in order (vectors past d
        // add exact zeros there), then each wave, then the four waves
        constexpr int VV = vec16<T>::N;
        constexpr int NQ = (kFusedMaxD / VV + 255) / 256;
        float ssq = 0.0f;
        if (tid < 256) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<T *>(x), (short)0, (int)(sizeof(T) * d), CoherentBuf::kWord3);
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
        if (lane == 0 && wv < 4) sm.sel.scratch[wv] = __float_as_uint(ssq);  // the bits (a word array)
        __syncthreads();
        const float s0 = __uint_as_float(sm.sel.scratch[0]), s1 = __uint_as_float(sm.sel.scratch[1]);
        const float s2 = __uint_as_float(sm.sel.scratch[2]), s3 = __uint_as_float(sm.sel.scratch[3]);
        const float rms = sqrtf((((s0 + s1) + s2) + s3) / (float)d + norm_eps);
        __syncthreads();
        auto norm = [&](float v) {  // rounded to x's dtype, as rmsnorm_kernel stores it
            const float y = v / rms;
            return sizeof(T) == 2 ? __uint_as_float((uint32_t)f32_to_bf16(y) << 16) : y;
        };
#pragma unroll
        for (int r = 0; r < KX; ++r) xv[r] = norm(xv[r]);
#pragma unroll
        for (int q = 0; q < XR; ++q) xr[q] = norm(xr[q]);
        if (xn_out && blockIdx.x == 0 && blockIdx.y == 0) {
#pragma unroll
            for (int r = 0; r < KX; ++r)
                if (slot_index<KX>(r) < d) elem<T>::store(xn_out, slot_index<KX>(r), xv[r]);
        }
    }
    uint32_t key[KX];
#pragma unroll
    for (int r = 0; r < KX; ++r) {
        if (slot_index<KX>(r) >= d) xv[r] = 0.0f;
        key[r] = __float_as_uint(xv[r]) & 0x7FFFFFFFu;
    }
    // keys of bf16 values have 16 zero low bits
    const SelectResult sr = block_select_window<kFT, KX>(key, d, k_in, 30, sizeof(T) == 2 ? 16 : 0, sm.sel);
    const uint32_t T_x = uniform_u32(sr.T), need_eq = uniform_u32(sr.need_eq);
    const bool all_eq = need_eq == uniform_u32(sr.count_eq);
    // keys equal to T_x: the need_eq of lowest index are kept; avail of them
    // are left for this split once those before it (c_eq, this wave's count)
    // are added up, in the same barrier round as the list's first scan
    uint32_t c_eq = 0;
    if (!all_eq) {
#pragma unroll
        for (int r = 0; r < KX; ++r)
            c_eq += (uint32_t)__popcll(__ballot((slot_index<KX>(r) < i0) & (key[r] == T_x)));
    }
    uint32_t avail = need_eq;
    // the split's kept inputs, listed in ascending order: one scan of packed
    // (greater, equal) counts gives every position
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int q = 0; q < XR; ++q) {
        if (q * kFT >= R) break;  // uniform
        const int i = i0 + q * kFT + tid;
        const uint32_t kk = __float_as_uint(xr[q]) & 0x7FFFFFFFu;
        const bool in = i < i1;
        const bool gt = in && (all_eq ? kk >= T_x : kk > T_x);
        const bool eq = in && !all_eq && kk == T_x;
        const uint32_t v = (gt ? 1u : 0u) | (eq ? 0x10000u : 0u);
        uint32_t tot, before;
        if (q == 0) {
            uint32_t eq_before_split;
            before = block_excl_scan_and_sum<kFT>(v, c_eq, sm.sel.scratch, &tot, &eq_before_split);
            eq_before_split = uniform_u32(eq_before_split);
            avail = need_eq > eq_before_split ? need_eq - eq_before_split : 0u;
        } else {
            before = block_excl_scan<kFT>(v, sm.sel.scratch, &tot);
        }
        const uint32_t gt_before = n_gt + (before & 0xFFFFu), eq_before = n_eq + (before >> 16);
        if (gt || (eq && eq_before < avail)) {
            const uint32_t pos = gt_before + min(eq_before, avail);
            sm.li[pos] = i;
            sm.lx[pos] = xr[q];
        }
        n_gt += uniform_u32(tot) & 0xFFFFu;
        n_eq += uniform_u32(tot) >> 16;
    }
    const int nk = (int)(n_gt + min(n_eq, avail));
    if (QBITS == 4) {
#pragma unroll
        for (int q = 0; q < GS; ++q) {
            const int e = tid + q * kFT;
            sm.p.gsc[e / (2 * CB)][(e / CB) & 1][e % CB] = gs_reg[q];
        }
    }
    __syncthreads();

    // ---- 2. proxy GEMV over this split's kept inputs
    float acc[2][CPL], ga[2][CPL], sx = 0.0f;  // int4: ga, sx = current group's sums
#pragma unroll
    for (int n = 0; n < CPL; ++n) acc[0][n] = acc[1][n] = ga[0][n] = ga[1][n] = 0.0f;
    int cur_g = 0;
    const uint32_t col_off = (uint32_t)cc * QBITS / 8;  // codes are < 1 GiB here: 32-bit offsets
    const uint32_t row_bytes = 2u * (uint32_t)half_bytes;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(codes), (short)0, (int)(row_bytes * (uint32_t)d), CoherentBuf::kWord3);
    for (int t0 = wv; t0 < nk; t0 += kFW * U) {
        uint32_t wg[U], wu[U];
        // every load issued (clamped), no branches: buffer loads on a 32-bit
        // offset (global loads on 64-bit addresses: Stage 1 1.2 us slower at
        // 4096 x 14336), streaming.  The cache policies of the two stages'
        // streams were chosen together, over back-to-back layers: with the
        // rows Stage 2's down rows read plainly, streaming codes here give
        // 47.1-47.3 us a layer at 4096 x 14336 against 47.6-47.8 for the
        // default policy here and streaming down rows.
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = min(t0 + kFW * u, nk - 1);
            const uint32_t o = (uint32_t)sm.li[t] * row_bytes + col_off;
            wg[u] = __builtin_amdgcn_raw_buffer_load_b32(crs, (int)o, 0, 2);
            wu[u] = __builtin_amdgcn_raw_buffer_load_b32(crs, (int)(o + (uint32_t)half_bytes), 0, 2);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + kFW * u;
            if (t < nk) {
                float qg[CPL], qu[CPL];
                Q::decode(wg[u], qg);
                Q::decode(wu[u], qu);
                const float xk = sm.lx[t];
                if (QBITS == 4) {
                    const int g = (sm.li[t] - i0) >> 7;
                    if (g != cur_g) {  // group change: fold the finished group in
                        const float bias = 8.0f * sx;
#pragma unroll
                        for (int n = 0; n < CPL; ++n) {
                            acc[0][n] = fmaf(sm.p.gsc[cur_g][0][lane * CPL + n], ga[0][n] - bias, acc[0][n]);
                            acc[1][n] = fmaf(sm.p.gsc[cur_g][1][lane * CPL + n], ga[1][n] - bias, acc[1][n]);
                            ga[0][n] = ga[1][n] = 0.0f;
                        }
                        sx = 0.0f;
                        cur_g = g;
                    }
                    sx += xk;
                }
                float(&dst)[2][CPL] = (QBITS == 4) ? ga : acc;
#pragma unroll
                for (int n = 0; n < CPL; ++n) {
                    dst[0][n] = fmaf(xk, qg[n], dst[0][n]);
                    dst[1][n] = fmaf(xk, qu[n], dst[1][n]);
                }
            }
        }
    }
    if (QBITS == 4) {
        const float bias = 8.0f * sx;
#pragma unroll
        for (int n = 0; n < CPL; ++n) {
            acc[0][n] = fmaf(sm.p.gsc[cur_g][0][lane * CPL + n], ga[0][n] - bias, acc[0][n]);
            acc[1][n] = fmaf(sm.p.gsc[cur_g][1][lane * CPL + n], ga[1][n] - bias, acc[1][n]);
        }
    }

    // ---- 3. the split's partial: waves added in a fixed order, 64-bit stores
#pragma unroll
    for (int n = 0; n < CPL; ++n) {
        sm.p.red[wv][0][lane * CPL + n] = acc[0][n];
        sm.p.red[wv][1][lane * CPL + n] = acc[1][n];
    }
    __syncthreads();
    // the list is read no more: its first words become the score counts
    uint32_t *const chist = reinterpret_cast<uint32_t *>(sm.li);
    if (k > 0 && tid < kCoarseBins) chist[tid] = 0u;
    for (int e = tid; e < CB; e += kFT) {  // e = (half, channel pair)
        const int h = e / (CB / 2), jj = 2 * (e % (CB / 2)), j = cb * CB + jj;
        if (j < F) {
            float v0 = sm.p.red[0][h][jj], v1 = sm.p.red[0][h][jj + 1];
#pragma unroll
            for (int w = 1; w < kFW; ++w) {
                v0 += sm.p.red[w][h][jj];
                v1 += sm.p.red[w][h][jj + 1];
            }
            store_agent2(&part[((int64_t)s * 2 + h) * F + j], v0, v1);
        }
    }
    if (!publish_and_ticket(&counters[cb], (uint32_t)S, &sm.flag)) return;

    // ---- the last split of this channel block: scores of its channels
    const CoherentBuf pbuf(part, (uint32_t)(sizeof(float) * S * 2 * F));
    for (int e = tid; e < CB; e += kFT) {
        const int h = e / (CB / 2), jj = 2 * (e % (CB / 2)), j = cb * CB + jj;
        float v0 = 0.0f, v1 = 0.0f;
        if (j < F) {
            for (int q0 = 0; q0 < S; q0 += 16) {
                float a0[16], a1[16];
#pragma unroll
                for (int i = 0; i < 16; ++i)  // splits >= S: beyond the buffer, read 0
                    pbuf.load2((uint32_t)(sizeof(float) * ((min(q0 + i, S) * 2 + h) * F + j)), a0[i], a1[i]);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (q0 + i < S) {
                        v0 += a0[i];
                        v1 += a1[i];
                    }
            }
        }
        sm.p.red[0][h][jj] = v0;
        sm.p.red[0][h][jj + 1] = v1;
    }
    __syncthreads();
    for (int e = tid; e < CB / 2; e += kFT) {
        const int jj = 2 * e, j = cb * CB + jj;
        if (j < F) {
            float sc[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float g = sm.p.red[0][0][jj + q], u = sm.p.red[0][1][jj + q];
                if (QBITS == 8) {  // per-row scales
                    g *= scales[j + q];
                    u *= scales[F + j + q];
                }
                sc[q] = salience(signal, act, g, u);
            }
            store_agent2(&score[j], sc[0], sc[1]);
            if (k > 0) {  // F is even: both channels exist
                atomicAdd(&chist[(__float_as_uint(sc[0]) & 0x7FFFFFFFu) >> 23], 1u);
                atomicAdd(&chist[(__float_as_uint(sc[1]) & 0x7FFFFFFFu) >> 23], 1u);
            }
        }
    }
    if (k > 0) {  // the counts as 16-bit fields (a block has < 2^16 channels), four bins a store
        __syncthreads();
        if (tid < kCoarseBins / 4) {
            const u32x4 c4 = *reinterpret_cast<const u32x4 *>(&chist[4 * tid]);
            store_agent2(reinterpret_cast<float *>(&blk_hist[(cb * kCoarseBins + 4 * tid) / 2]),
                         __uint_as_float(c4[0] | (c4[1] << 16)), __uint_as_float(c4[2] | (c4[3] << 16)));
        }
    }
    if (!publish_and_ticket(&counters[kFusedScoreSlot], (uint32_t)n_cblocks, &sm.flag)) return;

    // ---- 4. the last channel block: top-k over all F scores, every
    // coherent load issued before any is used: the counts first
    if (k <= 0 || !topk_here) return;
    // the blocks' counts: thread t loads bins 4m..4m+3 (m = t mod 64) of the
    // blocks t / 64 + 8i, as two words of two 16-bit fields (blocks past
    // n_cblocks read 0)
    constexpr int HB = kFusedMaxF / CB / 8;
    static_assert(kFT == 8 * (kCoarseBins / 4), "eight threads per four bins");
    const CoherentBuf hbuf(blk_hist, (uint32_t)(sizeof(uint16_t) * kCoarseBins * n_cblocks));
    float hc[HB][2];
#pragma unroll
    for (int i = 0; i < HB; ++i)
        hbuf.load2(8u * (uint32_t)((8 * i + (tid >> 6)) * (kCoarseBins / 4) + (tid & 63)), hc[i][0], hc[i][1]);
    // then the scores: the counts' crossing is found while they arrive (loads retire in order)
    uint32_t fk[KF];
#pragma unroll
    for (int r = 0; r < KF; ++r) fk[r] = __float_as_uint(load_agent(&score[min(slot_index<KF>(r), F - 1)]));
    uint32_t w0 = 0, w1 = 0;  // fields add without carry: at most HB x CB = 2048 per field
#pragma unroll
    for (int i = 0; i < HB; ++i) {
        w0 += __float_as_uint(hc[i][0]);
        w1 += __float_as_uint(hc[i][1]);
    }
    *reinterpret_cast<u32x4 *>(&sm.sel.hist[(tid >> 6) * kCoarseBins + 4 * (tid & 63)]) =
        u32x4{w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
    __syncthreads();
    // first radix pass (bits 30..23, scores being sign-free) from the counts,
    // then the passes over bits 22..0 below the crossing bin
    uint32_t h1[1] = {0u};
    if (tid < kCoarseBins) {
#pragma unroll
        for (int g = 0; g < 8; ++g) h1[0] += sm.sel.hist[g * kCoarseBins + tid];
    }
    find_crossing<kFT, 1>(h1, (uint32_t)k, sm.sel.scratch, sm.sel.found);
    const uint32_t prefix = uniform_u32(sm.sel.found[0]) << 23;
    const uint32_t rem = (uint32_t)k - uniform_u32(sm.sel.found[1]), in_bin = uniform_u32(sm.sel.found[2]);
    // slots past F get the key 0xFFFFFFFF, which no selection step takes
#pragma unroll
    for (int r = 0; r < KF; ++r) fk[r] = (slot_index<KF>(r) < F) ? (fk[r] & 0x7FFFFFFFu) : 0xFFFFFFFFu;
    SelectResult st;
    if (rem == in_bin) {  // the whole bin is selected
        st.T = prefix;
        st.need_eq = st.count_eq = rem;
    } else {
        st = radix_select_from<kFT, KF>(fk, F, prefix, 0xFF800000u, rem, 22, 0, sm.sel);
    }
    auto put = [&](int i, uint32_t pos) {
        if (pos < (uint32_t)k) sel[pos] = i;
    };
    if (uniform_u32(st.need_eq) == uniform_u32(st.count_eq)) {  // no tie to break: key >= T
        emit_at_least<kFT, KF>(fk, uniform_u32(st.T), sel, (uint32_t)k, sm.sel);
    } else {
        selection_bitmap<kFT, KF>(fk, F, st, sm.sel);
        emit_bitmap<kFT>(F, sm.sel, put);
    }
}

// ------------------------------------------------------------------------
FusedPlan fused_plan(int qbits, int64_t d, int64_t F)
{
    FusedPlan p;
    const int cpl = qbits == 8 ? Fused<8>::CPL : Fused<4>::CPL;
    const int rmax = qbits == 8 ? Fused<8>::RMAX : Fused<4>::RMAX;
    const int gran = qbits == 8 ? Fused<8>::GRAN : Fused<4>::GRAN;
    p.n_cblocks = (int)((F + 64 * cpl - 1) / (64 * cpl));
    int s = kFusedSlots / p.n_cblocks;
    if (s < 1) s = 1;
    int R = (int)((d + s - 1) / s);
    R = (R + gran - 1) / gran * gran;
    if (R > rmax) R = rmax;
    p.R = R;
    p.S = (int)((d + R - 1) / R);
    return p;
}

int64_t fused_part_floats(int qbits, int64_t d, int64_t F)
{
    const FusedPlan p = fused_plan(qbits, d, F);
    return (int64_t)p.S * 2 * F + (int64_t)kCoarseBins / 2 * p.n_cblocks;
}

// Beyond kFusedMaxF channels only the int4 proxy takes this kernel (the scores,
// then a top-k launch): measured at 8192 x 28672, keep 0.4, Stage 1 takes
// 51.1 us this way against 57.0 us for the input-selection, vector-ALU proxy
// and top-k launches; with the int8 proxy (188 MB) it took 59.5 against 57.0.
bool fused_supported(int64_t B, int64_t d, int64_t F, int qbits)
{
    if (B != 1 || d > kFusedMaxD) return false;
    return F <= kFusedMaxF || (qbits == 4 && F <= kFusedGemvMaxF);
}

hipError_t launch_stage1_fused(int dtype, int qbits, const void *x, int d, int F, int k_in, int k,
                               const uint8_t *codes, const float *scales, float *part, float *score, int32_t *sel,
                               uint32_t *counters, int act, int signal, hipStream_t st, float norm_eps, void *xn_out)
{
    if (!fused_supported(1, d, F, qbits)) return hipErrorInvalidValue;
    const FusedPlan pl = fused_plan(qbits, d, F);
    const int kx = (d + kFT - 1) / kFT;
    const bool topk_inside = F <= kFusedMaxF;  // else the kernel only scores, and the top-k is a second launch
    const int kf = topk_inside ? (F + kFT - 1) / kFT : 32;
    const int k_kernel = k;
    const dim3 grid(pl.n_cblocks, pl.S);
#define L1(T, Q, KXV, KFV)                                                                               \
    stage1_fused_kernel<T, Q, KXV, KFV><<<grid, kFT, 0, st>>>((const T *)x, d, F, k_in, k_kernel, codes, scales, \
                                                             pl.R, pl.S, pl.n_cblocks, part, score, sel,  \
                                                             counters, act, signal, norm_eps, (T *)xn_out, \
                                                             topk_inside ? 1 : 0)
#define L3(T, Q, KXV)                               \
    do {                                            \
        if (kf <= 16) L1(T, Q, KXV, 16);            \
        else if (kf <= 28) L1(T, Q, KXV, 28);       \
        else L1(T, Q, KXV, 32);                     \
    } while (0)
#define L2(T, Q)                 \
    do {                         \
        if (kx <= 2) L3(T, Q, 2);      \
        else if (kx <= 8) L3(T, Q, 8); \
        else L3(T, Q, 16);             \
    } while (0)
    if (dtype == 0) {
        if (qbits == 8) L2(float, 8);
        else L2(float, 4);
    } else {
        if (qbits == 8) L2(uint16_t, 8);
        else L2(uint16_t, 4);
    }
#undef L2
#undef L3
#undef L1
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || topk_inside || k <= 0) return e;
    return launch_topk_counts(score, F, k, sel, reinterpret_cast<const uint32_t *>(part + (int64_t)pl.S * 2 * F),
                              pl.n_cblocks, st);
}

}  // namespace prox
