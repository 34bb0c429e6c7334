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
// x of a workgroup in registers: up to kStageRegs 16-byte vectors per thread.
constexpr int kStageRegs = 2;

template <typename T, int NB>
__device__ __forceinline__ void load_rows_regs(const T *__restrict__ x, int B, int d, u32x4 (&xr)[kStageRegs])
{
    constexpr int V = vec16<T>::N;
    const int nvec = NB * d / V;
#pragma unroll
    for (int q = 0; q < kStageRegs; ++q) {
        int e = threadIdx.x + q * 256;
        e = min(e, nvec - 1);
        const int b = (e * V) / d;
        xr[q] = *(const u32x4 *)(x + (int64_t)(b < B ? b : 0) * d + (e * V - b * d));
    }
}

// x in LDS, optionally padded: with CH > 0, 4 floats of padding follow every
// CH elements, so that lanes reading consecutive CH-element chunks with
// 16-byte reads hit distinct banks (a chunk of 16 floats read per lane is a
// 64-byte stride: 4-way conflicts without the padding, none with it).
template <int CH>
__host__ __device__ constexpr int xpad_index(int i)
{
    return CH > 0 ? i + (i / CH) * 4 : i;
}
template <int CH>
__host__ __device__ constexpr int xpad_row(int d)
{
    return xpad_index<CH>(d);
}

template <typename T, int NB, int CH>
__device__ __forceinline__ void store_rows_lds(const u32x4 (&xr)[kStageRegs], int B, int d, float *xs)
{
    constexpr int V = vec16<T>::N;
    static_assert(CH == 0 || CH % V == 0, "an x vector must not straddle padding");
    const int nvec = NB * d / V;
#pragma unroll
    for (int q = 0; q < kStageRegs; ++q) {
        const int e = threadIdx.x + q * 256;
        if (e < nvec) {
            float f[V];
            vec16<T>::unpack(xr[q], f);
            const int b = (e * V) / d;
            const bool live = b < B;
            float *dst = xs + b * xpad_row<CH>(d) + xpad_index<CH>(e * V - b * d);
#pragma unroll
            for (int i = 0; i < V; ++i) dst[i] = live ? f[i] : 0.0f;
        }
    }
    __syncthreads();
}

// Stage rows [0, min(B, NB)) of a [B][d] tensor into LDS as fp32 (rows up to
// NB zero-filled), 16-byte loads, all of a thread's loads issued before use.
template <typename T, int NB, int CH>
__device__ __forceinline__ void stage_rows_f32(const T *__restrict__ x, int B, int d, float *xs)
{
    constexpr int V = vec16<T>::N;
    static_assert(CH == 0 || CH % V == 0, "an x vector must not straddle padding");
    constexpr int PER = 2;  // 16-byte loads per thread per batch
    const int nvec = NB * d / V;
    for (int e0 = threadIdx.x; e0 < nvec; e0 += 256 * PER) {
        u32x4 v[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            int e = e0 + q * 256;
            e = e < nvec ? e : nvec - 1;
            const int b = (e * V) / d;
            v[q] = *(const u32x4 *)(x + (int64_t)(b < B ? b : 0) * d + (e * V - b * d));
        }
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = e0 + q * 256;
            if (e < nvec) {
                float f[V];
                vec16<T>::unpack(v[q], f);
                const int b = (e * V) / d;
                const bool live = b < B;
                float *dst = xs + b * xpad_row<CH>(d) + xpad_index<CH>(e * V - b * d);
#pragma unroll
                for (int i = 0; i < V; ++i) dst[i] = live ? f[i] : 0.0f;
            }
        }
    }
    __syncthreads();
}

// How Stage 2 streams weight rows of element type TW (float, bf16 bits, or
// FP8 E4M3 codes as uint8_t): gate/up rows in 16-byte vectors of GV
// elements, UNR per lane per row and pass; down rows in DV elements per
// lane (16 bytes, or 8 for FP8 so that a slice stays 512 columns wide).
template <typename TW> struct WRows;
template <> struct WRows<float> {
    static constexpr int GV = 4, UNR = 8, DV = 4;
    using dvec = u32x4;
    static __device__ __forceinline__ void gunpack(const u32x4 &v, float *f) { vec16<float>::unpack(v, f); }
    static __device__ __forceinline__ dvec dload(const float *p) { return ld_stream(p); }
    static __device__ __forceinline__ void dunpack(const dvec &v, float *f) { vec16<float>::unpack(v, f); }
};
template <> struct WRows<uint16_t> {
    static constexpr int GV = 8, UNR = 8, DV = 8;
    using dvec = u32x4;
    static __device__ __forceinline__ void gunpack(const u32x4 &v, float *f) { vec16<uint16_t>::unpack(v, f); }
    static __device__ __forceinline__ dvec dload(const uint16_t *p) { return ld_stream(p); }
    static __device__ __forceinline__ void dunpack(const dvec &v, float *f) { vec16<uint16_t>::unpack(v, f); }
};
template <> struct WRows<uint8_t> {
    static constexpr int GV = 16, UNR = 4, DV = 8;
    using dvec = u32x2;
    static __device__ __forceinline__ void gunpack(const u32x4 &v, float *f)
    {
        e4m3x4_to_f32(v.x, f);
        e4m3x4_to_f32(v.y, f + 4);
        e4m3x4_to_f32(v.z, f + 8);
        e4m3x4_to_f32(v.w, f + 12);
    }
    static __device__ __forceinline__ dvec dload(const uint8_t *p) { return ld_stream8(p); }
    static __device__ __forceinline__ void dunpack(const dvec &v, float *f)
    {
        e4m3x4_to_f32(v.x, f);
        e4m3x4_to_f32(v.y, f + 4);
    }
};

// x padding chunk of gateup_block: a lane reads GV consecutive x values per
// weight vector; pad when that stride would conflict (GV >= 8), for one
// token only (4 tokens of padded x would not fit the 64 KB the batched
// launch allows).
template <typename TW, int NB>
__host__ __device__ constexpr int gu_xpad()
{
    return (NB == 1 && WRows<TW>::GV >= 8) ? WRows<TW>::GV : 0;
}

// One gate/up workgroup (4 waves, one selected channel each: ranks
// 4 blk .. 4 blk + 3).  xs: LDS for x as fp32, [NB][d].  COHERENT: s is stored with
// device-coherent stores, for other workgroups of the same launch.  gsc: the
// FP8 scales [F][2], applied to the finished dot products (else null).
template <typename T, typename TW, int NB, bool COHERENT>
__device__ __forceinline__ void gateup_block(const T *__restrict__ x, int B, int d, int F,
                                             const TW *__restrict__ w_gu, const float *__restrict__ gsc,
                                             const int32_t *__restrict__ sel, int k, float *__restrict__ s_sp,
                                             int32_t *__restrict__ iota_out, float *xs, int blk, int act)
{
    constexpr int V = WRows<TW>::GV;     // elements per 16-byte load
    constexpr int UNR = WRows<TW>::UNR;  // 16-byte vectors per lane per pass (two rows: 2*UNR loads)
    constexpr int CH = gu_xpad<TW, NB>();  // x padding chunk in LDS (0: none)
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    (void)tid;
    const int r = blk * 4 + wv;  // one selected channel per wave
    const bool live = r < k;
    const int j = (int)min((uint32_t)(live ? (sel ? sel[r] : r) : (sel ? sel[0] : 0)), (uint32_t)(F - 1));
    if (iota_out && live && lane == 0) iota_out[r] = r;
    const TW *grow = w_gu + (int64_t)j * 2 * d;
    const TW *urow = grow + d;
    const int nv = d / V;  // 16-byte vectors per row
    float gs = 1.0f, us = 1.0f;
    if (gsc) {
        gs = gsc[2 * j];
        us = gsc[2 * j + 1];
    }

    // x first (vmcnt retires in order: waiting for x must not wait for the rows)
    const bool x_in_regs = NB * (d / vec16<T>::N) <= 256 * kStageRegs;  // x's own 16-byte vectors
    u32x4 xr[kStageRegs];
    if (x_in_regs) load_rows_regs<T, NB>(x, B, d, xr);
    // first pass of both rows, every load issued (clamped index), no branches
    u32x4 vg[UNR], vu[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        const int vi = min(lane + u * 64, nv - 1);
        vg[u] = ld_stream(grow + vi * V);
        vu[u] = ld_stream(urow + vi * V);
    }
    if (x_in_regs)
        store_rows_lds<T, NB, CH>(xr, B, d, xs);
    else
        stage_rows_f32<T, NB, CH>(x, B, d, xs);

    float ag[NB], au[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) ag[b] = au[b] = 0.0f;
    for (int base = 0; base < nv; base += 64 * UNR) {
        if (base > 0) {
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int vi = min(base + lane + u * 64, nv - 1);
                vg[u] = ld_stream(grow + vi * V);
                vu[u] = ld_stream(urow + vi * V);
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int vi = base + lane + u * 64;
            if (vi < nv) {
                float fg[V], fu[V];
                WRows<TW>::gunpack(vg[u], fg);
                WRows<TW>::gunpack(vu[u], fu);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float *xb = xs + b * xpad_row<CH>(d) + xpad_index<CH>(vi * V);
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
        const float g = gs * wave_sum(ag[b]);
        const float u = us * wave_sum(au[b]);
        if (live && lane == 0 && b < B) {
            if (COHERENT)
                store_agent(&s_sp[(int64_t)b * k + r], gate_act(act, g) * u);
            else
                s_sp[(int64_t)b * k + r] = gate_act(act, g) * u;
        }
    }
}

template <typename T, typename TW, int NB>
__global__ __launch_bounds__(256) void gateup_kernel(const T *__restrict__ x, int B, int d, int F,
                                                     const TW *__restrict__ w_gu, const float *__restrict__ gsc,
                                                     const int32_t *__restrict__ sel, int k, float *__restrict__ s_sp,
                                                     int32_t *__restrict__ iota_out, int act)
{
    extern __shared__ float xs[];  // [NB][d]
    gateup_block<T, TW, NB, false>(x, B, d, F, w_gu, gsc, sel, k, s_sp, iota_out, xs, blockIdx.x, act);
}

// ------------------------------------------------------------------------
// K4: down projection over the selected rows of W_down^T [F][d].
// Grid (column slices of 64*VEC outputs, S rank splits); a workgroup of
// NW waves owns the ranks [s*U*NW, (s+1)*U*NW) of its slice, each wave U
// consecutive ranks, all U rows in flight at once: one vector load brings
// the wave's U channel indices and s values, then the U row segments are
// loaded (16-byte loads, VEC columns per lane) and accumulated.  The waves
// are combined in LDS in a fixed order into this split's partial; the last
// split of a slice (atomic ticket) adds the partials -- interleaved groups
// of splits in parallel, each group in split order, then the groups in
// order -- adds the residual if any, rounds and stores.
// ------------------------------------------------------------------------

// Waits (one thread) until (*ctr & mask) >= target; false once `ticks` of
// the 100 MHz real-time counter have passed without it.
__device__ __forceinline__ bool spin_wait_geq(uint32_t *ctr, uint32_t target, uint64_t ticks,
                                              uint32_t mask = 0xFFFFFFFFu)
{
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while ((__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & mask) < target) {
        __builtin_amdgcn_s_sleep(8);
        if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) return false;
    }
    return true;
}

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The end of a down-projection workgroup: its waves' accumulators are added
// in LDS in wave order into this split's partial (coherent 64-bit stores),
// then it takes a ticket on its slice.  The last TG arrivals (TG when the
// slice has at least TG splits, else 1) share the slice's tail, one of TG
// column groups each: a group adds its columns' partials -- interleaved
// groups of splits in parallel, each group in split order, then the groups
// in order -- multiplies by the output row's FP8 scale if any (dsc), adds the
// residual if any, rounds and stores.  The last arrival knows every partial
// is written and finishes group TG-1 at once; an earlier one first waits
// (bounded by spin_ticks) until every split has arrived, then claims its
// group with one bit of *claim.  After its own group the last arrival claims
// every group still unclaimed and finishes it too, so a wait that gives up
// (counted in *fallback) costs time, never a missing or wrong output.  The
// last of the tail workgroups to finish resets the slice's words
// (slice_counter: arrivals; pass_counter: finished tails; claim).
// s_flags: two ints of LDS.
template <typename T, int V, int NB, int NW, int TG>
__device__ __forceinline__ void down_finish(const float (&acc)[NB][V], float (&red)[NW][NB][64 * V], int *s_flags,
                                            int sl, int s, int B, int d, int S, float *__restrict__ part,
                                            const float *__restrict__ dsc, const T *residual, T *out,
                                            uint32_t *slice_counter, uint32_t *pass_counter, uint32_t *claim,
                                            uint32_t *fallback, uint64_t spin_ticks)
{
    constexpr int NT = 64 * NW;
    constexpr int COLS = 64 * V;
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < V; ++q) red[wv][b][lane * V + q] = acc[b][q];
    __syncthreads();
    for (int e = tid; e < NB * COLS / 2; e += NT) {  // column pairs
        const int b = e / (COLS / 2), ci = 2 * (e % (COLS / 2)), col = sl * COLS + ci;
        if (b < B && col < d) {
            float v0 = red[0][b][ci], v1 = red[0][b][ci + 1];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                v0 += red[w][b][ci];
                v1 += red[w][b][ci + 1];
            }
            store_agent2(&part[((int64_t)s * B + b) * d + col], v0, v1);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
    __syncthreads();
    if (tid == 0) s_flags[0] = (int)atomic_add_agent(slice_counter, 1u);
    __syncthreads();
    const int t = uniform(s_flags[0]);
    const int ng = (TG > 1 && S >= TG) ? TG : 1;  // column groups of the tail
    if (t < S - ng) return;

    // one column group of the tail: thread t takes column pair t % PAIRS of
    // the group, of the splits grp, grp + GROUPS, grp + 2*GROUPS, ... (grp =
    // t / PAIRS); every load is one this thread needs, issued before any is
    // added (wave-uniform predicate)
    const int CG = COLS / ng, PAIRS = CG / 2, GROUPS = NT / PAIRS;
    constexpr int QMAX = 36;  // splits per thread the loads cover in one batch
    const int pair = tid % PAIRS, grp = tid / PAIRS;
    const int nq = (S - grp + GROUPS - 1) / GROUPS;  // this thread's splits
    float *gsum = &red[0][0][0];                     // [GROUPS][NB][CG]
    const CoherentBuf pbuf(part, (uint32_t)(sizeof(float) * S * B * d));
    auto tail_group = [&](int g) {
        const int c0 = sl * COLS + g * CG;  // the group's first column
        const int col0 = c0 + pair * 2;
        __syncthreads();  // gsum free (red read, or a previous group's sums used)
        for (int b = 0; b < NB; ++b) {
            float y0 = 0.0f, y1 = 0.0f;
            if (b < B && col0 < d) {
                for (int q0 = 0; q0 < nq; q0 += QMAX) {
                    float v0[QMAX], v1[QMAX];
#pragma unroll
                    for (int i = 0; i < QMAX; ++i) {  // past this thread's splits: beyond the buffer, reads 0
                        const uint32_t q = (uint32_t)min(grp + (q0 + i) * GROUPS, S);
                        pbuf.load2((uint32_t)(sizeof(float) * ((q * B + b) * d + col0)), v0[i], v1[i]);
                    }
#pragma unroll
                    for (int i = 0; i < QMAX; ++i)
                        if (q0 + i < nq) {
                            y0 += v0[i];
                            y1 += v1[i];
                        }
                }
            }
            gsum[(grp * NB + b) * CG + pair * 2] = y0;
            gsum[(grp * NB + b) * CG + pair * 2 + 1] = y1;
        }
        __syncthreads();
        for (int e = tid; e < B * CG; e += NT) {
            const int b = e / CG, ci = e % CG, col = c0 + ci;
            if (col >= d || b >= NB) continue;
            float y = gsum[b * CG + ci];
            for (int gg = 1; gg < GROUPS; ++gg) y += gsum[(gg * NB + b) * CG + ci];
            if (dsc) y *= dsc[col];
            if (residual) y += elem<T>::load(residual, (int64_t)b * d + col);
            elem<T>::store(out, (int64_t)b * d + col, y);
        }
    };
    // claims group g for this workgroup (one thread asks, all get the answer)
    auto claim_group = [&](int g) {
        if (tid == 0)
            s_flags[1] = (__hip_atomic_fetch_or(claim, 1u << g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                          (1u << g)) == 0u;
        __syncthreads();
        const bool mine = uniform(s_flags[1]) != 0;
        __syncthreads();  // s_flags[1] read by every thread before its next write
        return mine;
    };

    if (t == S - 1) {  // the last arrival: every partial is in place
        tail_group(ng - 1);
        for (int g = 0; g < ng - 1; ++g)
            if (claim_group(g)) tail_group(g);
    } else {  // an earlier tail workgroup: wait for the last, then claim its group
        const int g = t - (S - ng);
        if (tid == 0) {
            const bool ok = spin_wait_geq(slice_counter, (uint32_t)S, spin_ticks);
            if (!ok) atomic_add_agent(fallback, 1u);
            s_flags[1] = ok ? 1 : 0;
        }
        __syncthreads();
        const bool arrived = uniform(s_flags[1]) != 0;
        __syncthreads();
        if (arrived && claim_group(g)) tail_group(g);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {  // the slice's words back to zero once no tail workgroup touches them
        if (ng == 1 || atomic_add_agent(pass_counter, 1u) == (uint32_t)ng - 1) {
            __hip_atomic_store(slice_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (ng > 1) {
                __hip_atomic_store(pass_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <typename T, typename TW, int NB, int NW>
__global__ __launch_bounds__(64 * NW) void down_kernel(const float *__restrict__ s_sp, int B, int k,
                                                       const TW *__restrict__ wdt, const float *__restrict__ dsc,
                                                       const int32_t *__restrict__ sel, int d, int F, int S,
                                                       float *__restrict__ part, const T *residual, T *out,
                                                       uint32_t *__restrict__ counters)
{
    constexpr int V = WRows<TW>::DV;
    constexpr int COLS = 64 * V;
    constexpr int U = kDownRowsPerWave;
    __shared__ float red[NW][NB][COLS];
    __shared__ int s_flags[2];
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int sl = blockIdx.x, s = blockIdx.y;
    const int c = sl * COLS + lane * V;
    const bool active = c < d;
    const int cc = active ? c : 0;
    const int rw0 = (s * NW + wv) * U;                    // this wave's first rank
    const int nr = max(0, min(U, k - rw0));               // ranks it holds (wave-uniform)
    // lanes 0..U-1 fetch the channel index and s values of rank rw0 + lane
    const int rl = rw0 + (lane & (U - 1));
    const int rlc = rl < k ? rl : k - 1;
    const int jl = (int)min((uint32_t)(sel ? sel[rlc] : rlc), (uint32_t)(F - 1));
    float sl_v[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) sl_v[b] = s_sp[(int64_t)(b < B ? b : 0) * k + rlc];
    float acc[NB][V];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < V; ++q) acc[b][q] = 0.0f;
    if (nr > 0) {
        typename WRows<TW>::dvec w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = __builtin_amdgcn_readlane(jl, u);
            if (u < nr) w[u] = WRows<TW>::dload(wdt + (int64_t)j * d + cc);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u < nr) {
                float f[V];
                WRows<TW>::dunpack(w[u], f);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float sv = (b < B) ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sl_v[b]), u)) : 0.0f;
#pragma unroll
                    for (int q = 0; q < V; ++q) acc[b][q] = fmaf(sv, f[q], acc[b][q]);
                }
            }
        }
    }

    down_finish<T, V, NB, NW, 1>(acc, red, s_flags, sl, s, B, d, S, part, dsc, residual, out, &counters[sl], nullptr,
                                 nullptr, nullptr, 0);
}

// ------------------------------------------------------------------------
// K3 + K4 for one token in one launch, so that the down projection's start
// overlaps the gate/up tail instead of following a kernel boundary.
//
// Workgroups [0, n_gu) are gate/up workgroups (gateup_block, s stored
// device-coherently) that count themselves done in their split's arrival
// word (its own 128-byte line, s2_sync_line); a split is 64 ranks, i.e. 16
// gate/up workgroups.  Workgroups [n_gu, n_gu + n_down) are down workgroups
// (slice, split): each waits until the gate/up workgroups of its split are
// done, then streams its 64 rows (4 waves x 16 rows, all in flight) and ends
// as down_kernel does.  Waiting before loading keeps the down rows out of the
// memory queue while the gate/up rows drain.
//
// Workgroups are dispatched in index order on every XCD, so every gate/up
// workgroup has been dispatched before any down workgroup waits, and gate/up
// workgroups wait for nothing.  No result rests on that: every wait is
// bounded (spin_ticks), and a down workgroup whose wait gives up computes
// its split's s values itself, bitwise as the gate/up workgroups do (the
// same code on the same data), before going on; the slice tail covers a
// tail workgroup that gave up (down_finish).  Each such wait adds one to
// counters[kFallbackSlot].  The arrival word counts gate/up workgroups in
// its low half and down workgroups (one 1 << 16 each, after their wait) in
// its high half; whichever arrival is the last of them all resets it, so a
// late arrival can never leave it nonzero for the next launch.
// ------------------------------------------------------------------------
constexpr int kS2Waves = 4;
constexpr int kS2Rows = 16;                           // down rows per wave, all in flight
constexpr int kS2Ranks = kS2Waves * kS2Rows;          // ranks per split
constexpr int kS2GuPerSplit = kS2Ranks / 4;           // gate/up workgroups (4 ranks each) per split

template <typename T, typename TW>
__global__ __launch_bounds__(64 * kS2Waves) void stage2_fused_kernel(
    const T *__restrict__ x, int d, int F, const TW *__restrict__ w_gu, const float *__restrict__ gsc,
    const TW *__restrict__ wdt, const float *__restrict__ dsc, const int32_t *__restrict__ sel, int k, int n_gu,
    int n_slices, int S, float *__restrict__ s_sp, float *__restrict__ part, const T *residual, T *out,
    uint32_t *__restrict__ counters, int32_t *__restrict__ iota_out, int act, uint64_t spin_ticks)
{
    constexpr int V = WRows<TW>::DV;
    constexpr int COLS = 64 * V;
    extern __shared__ float dyn[];  // gate/up: x [d]; down: red [kS2Waves][1][COLS]
    __shared__ int s_flags[2];
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);

    if ((int)blockIdx.x < n_gu) {
        gateup_block<T, TW, 1, true>(x, 1, d, F, w_gu, gsc, sel, k, s_sp, iota_out, dyn, blockIdx.x, act);
        __builtin_amdgcn_s_waitcnt(0);  // this thread's s stores have completed
        __syncthreads();
        if (tid == 0) {
            const int sp = blockIdx.x / kS2GuPerSplit;
            const uint32_t total = (uint32_t)min(kS2GuPerSplit, n_gu - sp * kS2GuPerSplit) + ((uint32_t)n_slices << 16);
            uint32_t *line = &counters[s2_sync_line(sp)];
            if (atomic_add_agent(line, 1u) + 1u == total)
                __hip_atomic_store(line, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }

    // ---- down: (slice sl, split s) over ranks [64 s, 64 s + 64)
    const int dw = (int)blockIdx.x - n_gu;
    const int sl = dw % n_slices, s = dw / n_slices;
    const int gu0 = s * kS2GuPerSplit, gu1 = min(n_gu, gu0 + kS2GuPerSplit);  // the split's gate/up workgroups
    if (tid == 0) {
        uint32_t *line = &counters[s2_sync_line(s)];
        const uint32_t total = (uint32_t)(gu1 - gu0) + ((uint32_t)n_slices << 16);
        const bool ok = spin_wait_geq(line, (uint32_t)(gu1 - gu0), spin_ticks, 0xFFFFu);
        if (!ok) atomic_add_agent(&counters[kFallbackSlot], 1u);
        s_flags[0] = ok ? 0 : 1;
        if (atomic_add_agent(line, 1u << 16) + (1u << 16) == total)
            __hip_atomic_store(line, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (uniform(s_flags[0])) {  // the wait gave up: the split's s values computed here
        for (int b = gu0; b < gu1; ++b) {
            __syncthreads();  // x in LDS no longer read by the previous block
            gateup_block<T, TW, 1, true>(x, 1, d, F, w_gu, gsc, sel, k, s_sp, iota_out, dyn, b, act);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    const int c = sl * COLS + lane * V;
    const int cc = c < d ? c : 0;
    const int rw0 = (s * kS2Waves + wv) * kS2Rows;  // this wave's first rank
    const int nr = max(0, min(kS2Rows, k - rw0));    // ranks it holds (wave-uniform)
    const int rl = rw0 + (lane & (kS2Rows - 1));
    const int rlc = rl < k ? rl : k - 1;
    const int jl = (int)min((uint32_t)(sel ? sel[rlc] : rlc), (uint32_t)(F - 1));
    const float sv_l = load_agent(&s_sp[rlc]);
    float acc[1][V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[0][q] = 0.0f;
    if (nr > 0) {
        typename WRows<TW>::dvec w[kS2Rows];
#pragma unroll
        for (int u = 0; u < kS2Rows; ++u) {
            const int j = __builtin_amdgcn_readlane(jl, u);
            if (u < nr) w[u] = WRows<TW>::dload(wdt + (int64_t)j * d + cc);
        }
#pragma unroll
        for (int u = 0; u < kS2Rows; ++u) {
            if (u < nr) {
                float f[V];
                WRows<TW>::dunpack(w[u], f);
                const float sv = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sv_l), u));
#pragma unroll
                for (int q = 0; q < V; ++q) acc[0][q] = fmaf(sv, f[q], acc[0][q]);
            }
        }
    }
    __syncthreads();  // dyn (x of a fallback) free before it holds the wave sums
    down_finish<T, V, 1, kS2Waves, 2>(acc, *reinterpret_cast<float(*)[kS2Waves][1][COLS]>(dyn), s_flags, sl, s, 1, d,
                                      S, part, dsc, residual, out, &counters[kDownSliceBase + sl],
                                      &counters[kDownPassBase + sl], &counters[kDownClaimBase + sl],
                                      &counters[kFallbackSlot], spin_ticks);
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

// RMSNorm with unit gain, fp32 math: out = h / sqrt(mean(h^2) + eps).  One
// workgroup per token.  Every 16-byte load of the row is issued at once
// through a buffer resource (vectors past d read as zeros, no branch), the
// row stays in registers for the scaling pass, and each thread's squares are
// summed in its vector order, then over the wave and the four waves.  (A
// loop of dependent 2-byte loads took 9.3 us per token row.)
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T *h, int d, float eps, T *out)
{
    constexpr int V = vec16<T>::N;          // elements per 16-byte vector
    constexpr int NV = 16384 / V / 256;     // vectors per thread at the largest d
    __shared__ float red[4];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int nvec = d / V;  // d % 8 == 0
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(h + (int64_t)b * d), (short)0, (int)(sizeof(T) * d), CoherentBuf::kWord3);
    u32x4 v[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q)
        v[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (tid + 256 * q), 0, 0));
    float ss = 0.0f;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        float f[V];
        vec16<T>::unpack(v[q], f);
#pragma unroll
        for (int i = 0; i < V; ++i) ss = fmaf(f[i], f[i], ss);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    const float rms = sqrtf(tot / (float)d + eps);
    u32x4 *ob = reinterpret_cast<u32x4 *>(out + (int64_t)b * d);
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int e = tid + 256 * q;
        if (e >= nvec) continue;
        float f[V];
        vec16<T>::unpack(v[q], f);
        u32x4 o;
        if constexpr (V == 8) {  // bf16, rounded to nearest even
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = (uint32_t)f32_to_bf16(f[2 * i] / rms) | ((uint32_t)f32_to_bf16(f[2 * i + 1] / rms) << 16);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(f[i] / rms);
        }
        ob[e] = o;
    }
}

// ------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------
template <typename T, typename TW>
static hipError_t gateup_t(const void *x, int B, int d, int F, const S2Weights &w, const int32_t *sel, int k,
                           float *s_sp, int32_t *iota_out, hipStream_t st)
{
    if (k <= 0) return hipSuccess;
    const int blocks = (k + 3) / 4;  // one channel per wave
    // x of up to 4 tokens staged in LDS as fp32, within 64 KB
    const int tb = (4 * d * (int)sizeof(float) <= 65536) ? 4 : 1;
    const TW *wgu = (const TW *)w.w_gu;
    for (int b0 = 0; b0 < B; b0 += tb) {
        const int nb = (B - b0 >= tb) ? tb : B - b0;
        const T *xp = (const T *)x + (int64_t)b0 * d;
        float *sp = s_sp + (int64_t)b0 * k;
        int32_t *io = (b0 == 0) ? iota_out : nullptr;
        if (nb == 1)
            gateup_kernel<T, TW, 1><<<blocks, 256, xpad_row<gu_xpad<TW, 1>()>(d) * sizeof(float), st>>>(
                xp, 1, d, F, wgu, w.gu_scales, sel, k, sp, io, w.act);
        else
            gateup_kernel<T, TW, 4><<<blocks, 256, 4 * d * sizeof(float), st>>>(xp, nb, d, F, wgu, w.gu_scales,
                                                                                sel, k, sp, io, w.act);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gateup(int dtype, const S2Weights &w, const void *x, int B, int d, int F, const int32_t *sel,
                         int k, float *s_sp, int32_t *iota_out, hipStream_t st)
{
    if (w.fmt == 1)
        return dtype == 0 ? gateup_t<float, uint8_t>(x, B, d, F, w, sel, k, s_sp, iota_out, st)
                          : gateup_t<uint16_t, uint8_t>(x, B, d, F, w, sel, k, s_sp, iota_out, st);
    return dtype == 0 ? gateup_t<float, float>(x, B, d, F, w, sel, k, s_sp, iota_out, st)
                      : gateup_t<uint16_t, uint16_t>(x, B, d, F, w, sel, k, s_sp, iota_out, st);
}

template <typename T, typename TW>
static hipError_t down_t(const DownPlan &pl, const float *s_sp, int B, int k, const S2Weights &w,
                         const int32_t *sel, int d, int F, float *part, const void *residual, void *out,
                         uint32_t *counters, hipStream_t st)
{
    dim3 grid(pl.n_slices, pl.S);
    dim3 grid4(pl.n_slices, 2 * pl.S);  // half-size workgroups for 4-token passes
    const TW *wdt = (const TW *)w.w_down_t;
    // tokens in passes of at most 4 (a pass re-reads the selected rows)
    for (int b0 = 0; b0 < B; b0 += 4) {
        const int nb = (B - b0 >= 4) ? 4 : B - b0;
        const float *sp = s_sp + (int64_t)b0 * k;
        const T *res = residual ? (const T *)residual + (int64_t)b0 * d : nullptr;
        T *o = (T *)out + (int64_t)b0 * d;
        if (nb == 1)
            down_kernel<T, TW, 1, kDownWaves><<<grid, 64 * kDownWaves, 0, st>>>(
                sp, 1, k, wdt, w.down_scales, sel, d, F, pl.S, part, res, o, counters);
        else
            down_kernel<T, TW, 4, kDownWaves / 2><<<grid4, 32 * kDownWaves, 0, st>>>(
                sp, nb, k, wdt, w.down_scales, sel, d, F, 2 * pl.S, part, res, o, counters);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_down(int dtype, const S2Weights &w, const DownPlan &pl, const float *s_sp, int B, int k,
                       const int32_t *sel, int d, int F, float *part, const void *residual, void *out,
                       uint32_t *counters, hipStream_t st)
{
    if (w.fmt == 1)
        return dtype == 0 ? down_t<float, uint8_t>(pl, s_sp, B, k, w, sel, d, F, part, residual, out, counters, st)
                          : down_t<uint16_t, uint8_t>(pl, s_sp, B, k, w, sel, d, F, part, residual, out, counters,
                                                      st);
    return dtype == 0 ? down_t<float, float>(pl, s_sp, B, k, w, sel, d, F, part, residual, out, counters, st)
                      : down_t<uint16_t, uint16_t>(pl, s_sp, B, k, w, sel, d, F, part, residual, out, counters, st);
}

template <typename T, typename TW>
static hipError_t stage2_fused_t(const void *x, int d, int F, const S2Weights &w, const int32_t *sel, int k,
                                 float *s_sp, float *part, const void *residual, void *out, uint32_t *counters,
                                 int32_t *iota_out, hipStream_t st, uint64_t spin_ticks)
{
    constexpr int V = WRows<TW>::DV;
    const int n_gu = (k + 3) / 4;
    const int n_slices = (d + 64 * V - 1) / (64 * V);
    const int S = (k + kS2Ranks - 1) / kS2Ranks;
    // slice words within [kDownSliceBase, kDownSliceEnd) and 32 claim bits;
    // at most 1 << 15 down workgroups per split line
    if (S > kS2MaxSplits || n_slices > kDownSliceEnd - kDownSliceBase) return hipErrorInvalidValue;
    const dim3 grid(n_gu + n_slices * S);
    const size_t lds = sizeof(float) * (size_t)max(xpad_row<gu_xpad<TW, 1>()>(d), kS2Waves * 64 * V);
    stage2_fused_kernel<T, TW><<<grid, 64 * kS2Waves, lds, st>>>(
        (const T *)x, d, F, (const TW *)w.w_gu, w.gu_scales, (const TW *)w.w_down_t, w.down_scales, sel, k, n_gu,
        n_slices, S, s_sp, part, (const T *)residual, (T *)out, counters, iota_out, w.act,
        spin_ticks ? spin_ticks : kDefaultSpinTicks);
    return hipGetLastError();
}

hipError_t launch_stage2_fused(int dtype, const S2Weights &w, const void *x, int d, int F, const int32_t *sel, int k,
                               float *s_sp, float *part, const void *residual, void *out, uint32_t *counters,
                               int32_t *iota_out, hipStream_t st, uint64_t spin_ticks)
{
    if (k <= 0) return hipErrorInvalidValue;
#define S2F(T, TW) stage2_fused_t<T, TW>(x, d, F, w, sel, k, s_sp, part, residual, out, counters, iota_out, st, spin_ticks)
    if (w.fmt == 1) return dtype == 0 ? S2F(float, uint8_t) : S2F(uint16_t, uint8_t);
    return dtype == 0 ? S2F(float, float) : S2F(uint16_t, uint16_t);
#undef S2F
}

// ------------------------------------------------------------------------
// The exact-state signal (no proxy): score_j = sum_b |s_bj| from the dense
// exact gate/up of every channel, and the gather of the selected channels'
// s values in rank order for the down projection.
// ------------------------------------------------------------------------
__global__ void score_from_s_kernel(const float *__restrict__ s, int B, int F, float *__restrict__ score)
{
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= F) return;
    float sc = 0.0f;
    for (int b = 0; b < B; ++b) sc += fabsf(s[(int64_t)b * F + j]);
    score[j] = sc;
}

__global__ void gather_s_kernel(const float *__restrict__ s, int B, int F, const int32_t *__restrict__ sel, int k,
                                float *__restrict__ s_sel)
{
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= k) return;
    const int j = (int)min((uint32_t)sel[r], (uint32_t)(F - 1));
    for (int b = 0; b < B; ++b) s_sel[(int64_t)b * k + r] = s[(int64_t)b * F + j];
}

hipError_t launch_score_from_s(const float *s, int B, int F, float *score, hipStream_t st)
{
    score_from_s_kernel<<<(F + 255) / 256, 256, 0, st>>>(s, B, F, score);
    return hipGetLastError();
}

hipError_t launch_gather_s(const float *s, int B, int F, const int32_t *sel, int k, float *s_sel, hipStream_t st)
{
    if (k <= 0) return hipSuccess;
    gather_s_kernel<<<(k + 255) / 256, 256, 0, st>>>(s, B, F, sel, k, s_sel);
    return hipGetLastError();
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
