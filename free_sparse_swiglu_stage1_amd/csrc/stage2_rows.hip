// Stage 2 of Prox for one bf16 token ("Stage 2: Exact Sparse Computation"):
// on the selected channels only, g = W_gate x, u = W_up x, s = act(g) u and
// y = sum_j s_j W_down[:, j], for d_model 4096 or 8192, with bf16 weights or
// FP8 E4M3 weights with per-row scales (the gate and up scales multiply the
// finished dot products, the down scale each output).
//
// One 1024-thread workgroup per CU.  Workgroup w takes the selected channels
// of rank [wk/G, (w+1)k/G) and streams all three rows of each: the gate and
// up rows give s_j, which scales the down row into a partial y of d columns
// held in registers.  No workgroup waits for another before its partial is
// stored, so the gate/up -> down dependency never crosses workgroups.
//  - A row is covered by a group of threads, each holding the columns of one
//    16-byte load per row (8 bf16 weights or 16 FP8 codes): with bf16 weights
//    the two halves of the workgroup are two groups at d_model 4096 and the
//    whole workgroup one group at 8192; with FP8 weights four and two.  The
//    groups take channels in turn.  Each group takes 3 channels a round (2
//    with FP8, whose 16 columns per thread need more registers);
//    a round's rows are requested together and the next round's before the
//    current one is reduced; g and u are added over lanes and the group's
//    waves in a fixed order.  The groups' partials are added (first +
//    second) and stored with device-coherent 16-byte stores.
//  - The end: each workgroup takes an arrival ticket.  The last R arrivals
//    (R = min(G, d / 32)) each add up 32-column slices of y over the G
//    partials in a fixed order (32 groups of every 32nd partial, then the
//    groups in order), add the residual and round.  The very last arrival
//    releases the other R - 1 by writing the launch's number into each one's
//    release word (128-byte lines 4 KB apart, so the polls spread over the
//    memory channels).
// Every sum runs in a fixed order: the result is bitwise deterministic and
// independent of which workgroup adds which slice.
//
// Waits are bounded.  The arrival count is a 64-bit count that only grows
// (launch e's arrivals are the tickets e G .. e G + G - 1) and the release
// words hold launch numbers, so nothing is reset and a wait that gives up
// leaves no state behind for the next launch.  A workgroup whose wait gives
// up computes every workgroup's partial itself -- bitwise the value that
// workgroup stores -- stores it, and goes on: the result is the same, only
// later, and the give-up is counted in the fallback slot.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace prox {

constexpr int kRT = 1024;         // threads per workgroup
constexpr int kRW = kRT / 64;     // waves
constexpr int kRSumGroups = 32;   // partial groups of a slice sum
constexpr int kRSliceCols = 32;   // columns of a slice
constexpr int kStream = 2;        // buffer-load cache policy: streaming (non-temporal)

struct RowsArgs {
    const uint16_t *x;         // [d] bf16
    const void *w_gu;          // [F][2][d] bf16, or FP8 E4M3 codes
    const void *w_dt;          // [F][d] bf16, or FP8 E4M3 codes
    const float *gsc;          // FP8: [F][2] gate and up row scales (else null)
    const float *dsc;          // FP8: [d] down row scales, one per output (else null)
    const int32_t *sel;        // [k] ascending, or null: channel r at rank r
    const uint16_t *residual;  // [d] or null (may alias out)
    uint16_t *out;             // [d]
    int32_t *iota_out;         // [k] or null: the ranks' channels are written (sel null only)
    float *ypart;              // [G][d]
    uint32_t *counters;
    uint64_t spin_ticks;
    int d, F, k, G, act;
};

// A thread's piece of a row: 16 bytes, 8 consecutive bf16 columns or 16 FP8
// E4M3 codes.
template <typename TW> struct RowPiece;
template <> struct RowPiece<uint16_t> {
    using V = u32x4;
    static constexpr int N = 8;  // columns
    template <int AUX>  // cache policy
    static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
    }
    static __device__ __forceinline__ void unpack(const V &v, float *f) { vec16<uint16_t>::unpack(v, f); }
};
template <> struct RowPiece<uint8_t> {
    using V = u32x4;
    static constexpr int N = 16;
    template <int AUX>  // cache policy
    static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
    }
    static __device__ __forceinline__ void unpack(const V &v, float *f)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) e4m3x4_to_f32(v[i], f + 4 * i);
    }
};

// H: channel groups of the workgroup, kRT / H threads each covering a row
// (bf16: 2 at d_model 4096, 1 at 8192; FP8: 4 and 2)
template <int H, typename TW>
struct alignas(16) RowsSmem {
    static constexpr int CPT = RowPiece<TW>::N;  // columns per thread
    static constexpr int RC = sizeof(TW) == 1 ? 2 : 3;  // channels per group and round
    union {
        struct {
            float r2[kRW][2 * RC];
            float sv[H][RC];
        } e;
        float yg[H - 1 > 0 ? H - 1 : 1][kRT / H][CPT + 1];  // groups 1.. sums (padded: no bank conflicts)
        float sums[kRSumGroups][kRSliceCols];
    } u;
    int chan[kRowsMaxChan];
    float gs[kRowsMaxChan][2];  // FP8: the channels' gate and up scales
    int flag;
    uint32_t epoch;
    int pos;
};

// Workgroup v's partial y over its ranks, stored to ypart[v]: all threads
// call; the value depends on v and the inputs only.
template <int H, typename TW>
__device__ void rows_partial(const RowsArgs &a, int v, RowsSmem<H, TW> &sm, const float (&xs)[RowPiece<TW>::N])
{
    using RP = RowPiece<TW>;
    using V = typename RP::V;
    constexpr int CPT = RowsSmem<H, TW>::CPT;
    constexpr int RC = RowsSmem<H, TW>::RC;
    constexpr bool FP8 = sizeof(TW) == 1;
    constexpr int GT = kRT / H, GW = kRW / H;  // threads and waves of a group
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int grp = uniform(tid / GT), ht = tid % GT;
    const int d = a.d, F = a.F;
    const int r0 = (int)((int64_t)v * a.k / a.G), r1 = (int)((int64_t)(v + 1) * a.k / a.G);
    const int nc = r1 - r0;
    __syncthreads();  // the previous user of the channel list and the LDS is done
    if (tid < nc) {
        const int j = a.sel ? min(max(a.sel[r0 + tid], 0), F - 1) : r0 + tid;  // clamped into [0, F)
        sm.chan[tid] = j;
        if (FP8) {
            sm.gs[tid][0] = a.gsc[2 * j];
            sm.gs[tid][1] = a.gsc[2 * j + 1];
        }
    }
    __syncthreads();

    float yacc[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q) yacc[q] = 0.0f;
    const uint32_t rowb = (uint32_t)(sizeof(TW) * d);  // bytes of a row
    const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(a.w_gu), (short)0, (int)(2u * rowb * (uint32_t)F), CoherentBuf::kWord3);
    const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(a.w_dt), (short)0, (int)(rowb * (uint32_t)F), CoherentBuf::kWord3);
    const uint32_t goob = 2u * rowb * (uint32_t)F, doob = rowb * (uint32_t)F;
    const uint32_t coff = (uint32_t)(ht * CPT * sizeof(TW));
    V ag[RC], au[RC], ad[RC], bg[RC], bu[RC], bd[RC];
    // a round's rows: list entries (rd RC + c) H + grp; past the list the
    // offsets are out of range and read zero without touching memory
    auto issue = [&](V(&vg)[RC], V(&vu)[RC], V(&vd)[RC], int rd) {
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            const int i = (rd * RC + c) * H + grp;
            const bool live = i < nc;
            const uint32_t j = (uint32_t)sm.chan[live ? i : 0];
            // gate and up rows streaming, down rows with the default policy:
            // over back-to-back layers (with the proxy codes of the fused
            // Stage 1 streaming) 47.1-47.3 us a layer at 4096 x 14336 against
            // 47.6-47.8 with every stream's other choice; this stage alone
            // 23.6 against 24.6-24.9 us
            vg[c] = RP::template load<kStream>(grs, live ? j * 2u * rowb + coff : goob);
            vu[c] = RP::template load<kStream>(grs, live ? j * 2u * rowb + rowb + coff : goob);
            vd[c] = RP::template load<0>(drs, live ? j * rowb + coff : doob);
        }
    };
    auto process = [&](const V(&vg)[RC], const V(&vu)[RC], const V(&vd)[RC], int rd) {
        float pg[RC], pu[RC];
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            float g = 0.0f, u = 0.0f;
            float fg[CPT], fu[CPT];
            RP::unpack(vg[c], fg);
            RP::unpack(vu[c], fu);
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                g = fmaf(fg[e], xs[e], g);
                u = fmaf(fu[e], xs[e], u);
            }
            pg[c] = wave_sum(g);
            pu[c] = wave_sum(u);
        }
        if (lane == 0) {
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                sm.u.e.r2[wv][c] = pg[c];
                sm.u.e.r2[wv][RC + c] = pu[c];
            }
        }
        __syncthreads();
        if (tid < H * RC) {  // channel c of group h: that group's waves in order
            const int h = tid / RC, c = tid % RC;
            float tg[GW], tu[GW];
#pragma unroll
            for (int ww = 0; ww < GW; ++ww) {
                tg[ww] = sm.u.e.r2[GW * h + ww][c];
                tu[ww] = sm.u.e.r2[GW * h + ww][RC + c];
            }
            float g = tg[0], u = tu[0];
#pragma unroll
            for (int ww = 1; ww < GW; ++ww) {
                g += tg[ww];
                u += tu[ww];
            }
            const int i = (rd * RC + c) * H + h;
            if (FP8 && i < nc) {  // the row scales multiply the finished dot products
                g *= sm.gs[i][0];
                u *= sm.gs[i][1];
            }
            sm.u.e.sv[h][c] = i < nc ? gate_act(a.act, g) * u : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            const float sv = sm.u.e.sv[grp][c];
            float fd[CPT];
            RP::unpack(vd[c], fd);
#pragma unroll
            for (int e = 0; e < CPT; ++e) yacc[e] = fmaf(sv, fd[e], yacc[e]);
        }
    };
    const int nr = (nc + H * RC - 1) / (H * RC);
    if (nr > 0) issue(ag, au, ad, 0);
    for (int rd = 0; rd < nr; rd += 2) {
        issue(bg, bu, bd, rd + 1);
        process(ag, au, ad, rd);
        if (rd + 1 < nr) {
            issue(ag, au, ad, rd + 2);
            process(bg, bu, bd, rd + 1);
        }
    }
    // the groups' sums added in group order and stored by group 0
    __syncthreads();
    if (grp > 0) {
#pragma unroll
        for (int q = 0; q < CPT; ++q) sm.u.yg[grp - 1][ht][q] = yacc[q];
    }
    __syncthreads();
    if (grp == 0) {  // 16-byte device-coherent stores
        const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
            a.ypart + (int64_t)v * d, (short)0, (int)(sizeof(float) * d), CoherentBuf::kWord3);
#pragma unroll
        for (int h = 1; h < H; ++h)
#pragma unroll
            for (int q = 0; q < CPT; ++q) yacc[q] += sm.u.yg[h - 1][ht][q];
#pragma unroll
        for (int q = 0; q < CPT; q += 4) {
            u32x4 val;
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] = __float_as_uint(yacc[q + e]);
            __builtin_amdgcn_raw_buffer_store_b128(val, yrs, (int)(sizeof(float) * (ht * CPT + q)), 0,
                                                   CoherentBuf::kSc1);
        }
    }
}

template <int H, typename TW>
__global__ __launch_bounds__(kRT, 1) void stage2_rows_kernel(RowsArgs a)
{
    __shared__ RowsSmem<H, TW> sm;
    const int tid = threadIdx.x, w = blockIdx.x, G = a.G, d = a.d;
    constexpr int CPT = RowPiece<TW>::N;
    const int ht = tid % (kRT / H);
    float xs[CPT];
#pragma unroll
    for (int q = 0; q < CPT; q += 8)
        vec16<uint16_t>::unpack(*reinterpret_cast<const u32x4 *>(a.x + CPT * ht + q), xs + q);
    rows_partial<H, TW>(a, w, sm, xs);
    if (a.iota_out && !a.sel) {
        const int r0 = (int)((int64_t)w * a.k / G), r1 = (int)((int64_t)(w + 1) * a.k / G);
        if (tid < r1 - r0) a.iota_out[r0 + tid] = r0 + tid;
    }

    // ---- arrival: the last R arrivals add up the slices
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0) {
        uint64_t *arrive = reinterpret_cast<uint64_t *>(&a.counters[kRowsArriveSlot]);
        const uint64_t t = __hip_atomic_fetch_add(arrive, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.pos = (int)(t % (uint64_t)G);
        sm.epoch = (uint32_t)(t / (uint64_t)G) + 1u;
    }
    __syncthreads();
    const int pos = sm.pos;
    const uint32_t epoch = sm.epoch;
    const int n_chunks = d / kRSliceCols;
    const int R = G < n_chunks ? G : n_chunks;
    if (pos < G - R) return;
    const int s = pos - (G - R);
    if (pos == G - 1) {  // every partial is stored: release the other slice workgroups
        for (int i = tid; i < R - 1; i += kRT)
            __hip_atomic_store(&a.counters[s2_sync_line(kRowsReleaseBase + i)], epoch, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else {
        if (tid == 0) {
            const uint32_t *rel = &a.counters[s2_sync_line(kRowsReleaseBase + s)];
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            bool ok = true;
            while ((int32_t)(__hip_atomic_load(const_cast<uint32_t *>(rel), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) - epoch) < 0) {
                __builtin_amdgcn_s_sleep(1);
                if (__builtin_amdgcn_s_memrealtime() - t0 > a.spin_ticks) {
                    ok = false;
                    break;
                }
            }
            if (!ok) __hip_atomic_fetch_add(&a.counters[kFallbackSlot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sm.flag = ok;
        }
        __syncthreads();
        if (!sm.flag) {  // gave up: every partial computed here, bitwise as its workgroup stores it
            for (int v = 0; v < G; ++v) rows_partial<H, TW>(a, v, sm, xs);
            __builtin_amdgcn_s_waitcnt(0);
        }
    }
    __syncthreads();

    // ---- slices s, s + R, ...: 32 columns each over the G partials
    const CoherentBuf ybuf(a.ypart, (uint32_t)(sizeof(float) * G * d));
    const uint32_t yend = (uint32_t)(sizeof(float) * G * d);
    const int col = tid & (kRSliceCols - 1), grp = tid >> 5;  // grp: partials grp, grp + 32, ...
    for (int ch = s; ch < n_chunks; ch += R) {
        const int cA = ch * kRSliceCols;
        float v = 0.0f;
        for (int p0 = grp; p0 < G; p0 += kRSumGroups * 8) {
            float t8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int p = p0 + kRSumGroups * i;
                t8[i] = ybuf.load(p < G ? (uint32_t)(sizeof(float) * ((int64_t)p * d + cA + col)) : yend);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (p0 + kRSumGroups * i < G) v += t8[i];
        }
        sm.u.sums[grp][col] = v;
        __syncthreads();
        if (tid < kRSliceCols) {
            float t[kRSumGroups];
#pragma unroll
            for (int g = 0; g < kRSumGroups; ++g) t[g] = sm.u.sums[g][tid];
            float y = t[0];
#pragma unroll
            for (int g = 1; g < kRSumGroups; ++g) y += t[g];
            if (a.dsc) y *= a.dsc[cA + tid];
            if (a.residual) y += __uint_as_float((uint32_t)a.residual[cA + tid] << 16);
            a.out[cA + tid] = f32_to_bf16(y);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------
bool rows_supported(int64_t d, int64_t F, int64_t k, int G)
{
    if ((d != 4096 && d != 8192) || F < 16 || k <= 0 || k > F) return false;
    if (G < kRSumGroups || G > kRowsMaxGroups) return false;
    return (k + G - 1) / G <= kRowsMaxChan;
}

hipError_t launch_stage2_rows(const void *x, int d, int F, const int32_t *sel, int k, const S2Weights &w,
                              const void *residual, void *out, int32_t *iota_out, float *ypart, uint32_t *counters,
                              uint64_t spin_ticks, int G, hipStream_t st)
{
    if (!rows_supported(d, F, k, G)) return hipErrorInvalidValue;
    if (w.fmt == 1 && (!w.gu_scales || !w.down_scales)) return hipErrorInvalidValue;
    RowsArgs a;
    a.x = (const uint16_t *)x;
    a.w_gu = w.w_gu;
    a.w_dt = w.w_down_t;
    a.gsc = w.fmt == 1 ? w.gu_scales : nullptr;
    a.dsc = w.fmt == 1 ? w.down_scales : nullptr;
    a.sel = sel;
    a.residual = (const uint16_t *)residual;
    a.out = (uint16_t *)out;
    a.iota_out = iota_out;
    a.ypart = ypart;
    a.counters = counters;
    a.spin_ticks = spin_ticks ? spin_ticks : kDefaultSpinTicks;
    a.d = d;
    a.F = F;
    a.k = k;
    a.G = G;
    a.act = w.act;
    if (w.fmt == 1) {
        if (d == 4096) stage2_rows_kernel<4, uint8_t><<<G, kRT, 0, st>>>(a);
        else stage2_rows_kernel<2, uint8_t><<<G, kRT, 0, st>>>(a);
    } else {
        if (d == 4096) stage2_rows_kernel<2, uint16_t><<<G, kRT, 0, st>>>(a);
        else stage2_rows_kernel<1, uint16_t><<<G, kRT, 0, st>>>(a);
    }
    return hipGetLastError();
}

int rows_groups()
{
    constexpr int kMaxDevices = 64;
    static int cache[kMaxDevices];  // groups + 1 per device; 0: not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    const int c = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (c) return c - 1;
    int cus = 0, g = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) {
        const void *fns[] = {(const void *)stage2_rows_kernel<2, uint16_t>, (const void *)stage2_rows_kernel<1, uint16_t>,
                             (const void *)stage2_rows_kernel<4, uint8_t>, (const void *)stage2_rows_kernel<2, uint8_t>};
        int occ = 1 << 30;
        for (const void *f : fns) {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kRT, 0) != hipSuccess) n = 0;
            occ = n < occ ? n : occ;
        }
        if (occ >= 1) g = cus < kRowsMaxGroups ? cus : kRowsMaxGroups;
    }
    (void)hipGetLastError();  // a failed query leaves no error for the next call to report
    __atomic_store_n(&cache[dev], g + 1, __ATOMIC_RELAXED);
    return g;
}

}  // namespace prox
