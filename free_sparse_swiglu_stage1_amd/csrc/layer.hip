// The whole Prox forward for one token in a single launch: both stages of
// the technical summary ("Stage 1: Lightweight Proxy Construction", "Stage 2:
// Exact Sparse Computation"), one 1024-thread workgroup per CU, every
// workgroup resident at once.
//
// Opt-in (the two-launch path is faster on MI355X: the phase joins below
// cost more than a launch boundary).
//
// Phases, each workgroup w of G:
//  A. x is loaded; the k_in largest |x_i| are selected (every workgroup
//     takes the same exact decision) and this workgroup's share of them is
//     listed in LDS in ascending index order, index and value in one word.
//  B. Proxy GEMV: the channels fall into blocks of 1024 (16 per lane, one
//     16-byte load per lane and row); the workgroups of block c split its
//     kept inputs into equal rank ranges.  The 16 waves' sums are added in
//     a fixed tree in LDS and the block partial is stored (coherent).
//  C. Block barrier: once a block's workgroups have all stored, each of them
//     adds the block's partials over its own slice of the block's channels
//     in workgroup order, applies the row scales and stores
//     score_j = |act(g~_j) u~_j| (or the chosen signal).  The last workgroup
//     to score (a ticket) selects the top k of all F scores and publishes
//     the selection as a bitmap of 32-channel words with each word's count
//     of selected channels before it.
//  D. Grid barrier; each workgroup reads the bitmap and the counts and takes
//     the selected channels of rank [wk/G, (w+1)k/G) in ascending channel
//     order -- a balanced share of Stage 2 -- and writes those entries of
//     the mask if asked.
//  E. Stage 2 on its channels, in rounds.  The two halves of the workgroup
//     take alternate channels; thread t of a half holds columns [t*CPT,
//     (t+1)*CPT) of the gate, up and down rows of its channels (16-byte
//     loads).  A round's rows are requested together and the next round's
//     before the current one is reduced; g and u are added over lanes and the
//     half's waves in a fixed order, s = act(g) u, and the down rows scaled by
//     s are accumulated per thread.  The halves' sums are added and the
//     workgroup's partial y is stored.
//  F. Grid barrier; workgroup w adds the G partials of its columns [wd/G,
//     (w+1)d/G) in a fixed order, adds the residual, rounds and stores.
// Every sum runs in a fixed order: the result is bitwise deterministic.
//
// Grid barriers: a workgroup adds one to an arrival count; the last arrival
// writes the barrier's number into every workgroup's release word (each in
// its own 128-byte line, the lines 4 KB apart so that the polls spread over
// the memory channels), and each workgroup polls its own word.  The arrival
// count is reset by the last arrival of the last barrier, each release word
// by its workgroup once past that barrier, the tickets by their last
// arrivals: a completed launch leaves every counter at zero.  The launch is
// an ordinary one of at most one workgroup per CU, the most the kernel's
// registers allow, so on an otherwise idle device every workgroup is resident
// at once; a poll is bounded in time all the same, and one that gives up
// records an error (never reset by the kernel) and makes every output column
// of the workgroups that saw it NaN.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"
#include "select.h"

namespace prox {

// Phase timestamps for measurement builds (-DPROX_LAYER_MARKS): thread 0 of
// each workgroup stores the real-time counter at each phase boundary.
#ifdef PROX_LAYER_MARKS
__device__ uint64_t g_layer_marks[256][16];
#define LAYER_MARK(i)                                                                                    \
    do {                                                                                                 \
        if (threadIdx.x == 0 && blockIdx.x < 256) g_layer_marks[blockIdx.x][i] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define LAYER_MARK(i) \
    do {              \
    } while (0)
#endif

constexpr int kLT = 1024;             // threads per workgroup
constexpr int kLW = kLT / 64;         // waves
constexpr int kLCB = 1024;            // proxy channels per block: 16 per lane, 16-byte loads
constexpr int kLUnits = 8;            // GEMV units in flight per wave
constexpr int kLMaxChan = 64;         // Stage-2 channels per workgroup
constexpr int kLSumGroups = 32;       // partial groups of the final reduction
constexpr int kLSelWords = 512;       // selection bitmap words (d_ff <= 16384)

struct LayerArgs {
    const uint16_t *x;         // [d] bf16
    const uint8_t *codes;      // int8 proxy [d][2][F]
    const float *qscales;      // [2][F]
    const uint16_t *w_gu;      // [F][2][d]
    const uint16_t *w_dt;      // [F][d]
    const uint16_t *residual;  // [d] or null (may alias out)
    uint16_t *out;             // [d]
    int32_t *sel_out;          // [k] or null
    float *part;               // [G][2][kLCB]: each GEMV workgroup's gate and up sums of its block
    float *score;              // [F]
    uint32_t *selw;            // [2][kLSelWords]: selection bitmap words, selected channels before each word
    float *ypart;              // [G][d]
    uint32_t *counters;
    uint64_t spin_ticks;
    int d, F, k_in, k, G, n_cb, act, signal;
};

template <int KX, int KF>
struct alignas(16) LayerSmem {
    static constexpr int CPT = 2 * KX;   // Stage-2 columns per thread (one half covers a row)
    static constexpr int RC = 24 / CPT;  // Stage-2 channels per half and round
    union {
        struct {
            SelectSmem<1024 * KX> sel;
            uint32_t wpre[32 * KX];         // kept inputs before each bitmap word
            uint32_t list[2048];            // this workgroup's kept inputs: index | bf16 value << 16
        } a;
        float tree[kLW / 2][64][20];        // GEMV wave sums in the adding tree (16 per lane, padded to 20)
        struct {
            SelectSmem<1024 * KF> sel;
        } topk;
        struct {
            float r2[kLW][2 * RC];
            float sv[2][RC];
            int chan[kLMaxChan];
        } e;
        float yhalf[kLT / 2][CPT + 1];      // the second half's sums of y (padded: no bank conflicts)
        float sums[kLSumGroups][32];
    } u;
    int flag;
    int err;
};

__device__ __forceinline__ uint32_t atomic_add_u32(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_agent_u32(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_agent_u32(const uint32_t *p)
{
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier number `epoch` (1, 2, ...; `last_epoch` the launch's final
// one).  All threads call.  Returns false if the wait gave up.
__device__ bool grid_barrier(uint32_t *counters, int G, uint32_t epoch, uint32_t last_epoch, uint64_t ticks,
                             int *s_flag)
{
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t *ctr = &counters[kLayerBarrierSlot];
        const uint32_t t = atomic_add_u32(ctr, 1u);
        const bool last = t == epoch * (uint32_t)G - 1u;
        if (last && epoch == last_epoch) store_agent_u32(ctr, 0u);
        *s_flag = last;
    }
    __syncthreads();
    if (*s_flag) {  // the last arrival releases every workgroup
        for (int i = threadIdx.x; i < G; i += kLT) store_agent_u32(&counters[s2_sync_line(i)], epoch);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t *rel = &counters[s2_sync_line(blockIdx.x)];
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        bool ok = true;
        while (load_agent_u32(rel) < epoch) {
            __builtin_amdgcn_s_sleep(1);
            if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) {
                ok = false;
                break;
            }
        }
        if (epoch == last_epoch) store_agent_u32(rel, 0u);
        if (!ok) atomic_add_u32(&counters[kLayerErrorSlot], 1u);
        *s_flag = ok;
    }
    __syncthreads();
    return *s_flag != 0;
}

__device__ __forceinline__ u32x4 ld_buf16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));  // nontemporal
}

template <int KX, int KF>
__global__ __launch_bounds__(kLT, 1) void layer_kernel(LayerArgs a)
{
    constexpr int CPT = LayerSmem<KX, KF>::CPT;  // Stage-2 columns per thread
    constexpr int NV = CPT / 8;                  // 16-byte vectors per row and thread
    constexpr int RC = LayerSmem<KX, KF>::RC;
    __shared__ LayerSmem<KX, KF> sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int w = blockIdx.x, G = a.G, d = a.d, F = a.F, k_in = a.k_in, k = a.k;
    const int half = uniform(tid >> 9), ht = tid & 511;  // Stage-2 half, thread within it
    LAYER_MARK(0);
    if (tid == 0) sm.err = 0;

    // ---- A. the input: selection slots (wave-contiguous) and Stage-2 columns
    float xv[KX], xs[CPT];
#pragma unroll
    for (int r = 0; r < KX; ++r) xv[r] = __uint_as_float((uint32_t)a.x[slot_index<KX>(r)] << 16);
#pragma unroll
    for (int v = 0; v < NV; ++v)
        vec16<uint16_t>::unpack(*reinterpret_cast<const u32x4 *>(a.x + ht * CPT + 8 * v), xs + 8 * v);
    // the GEMV's share: block c = w / gpb, kept-input ranks [ra, rb); the
    // last G - n_cb * gpb workgroups have none
    const int n_cb = a.n_cb, gpb = G / n_cb;
    const bool gemv = w < n_cb * gpb;
    const int c = gemv ? w / gpb : 0, jw = w % gpb;
    const int ra = gemv ? (int)((int64_t)jw * k_in / gpb) : 0, rb = gemv ? (int)((int64_t)(jw + 1) * k_in / gpb) : 0;
    uint32_t key[KX];
#pragma unroll
    for (int r = 0; r < KX; ++r) key[r] = __float_as_uint(xv[r]) & 0x7FFFFFFFu;
    {
        // the k_in largest |x| (keys of bf16 values have 16 zero low bits)
        const SelectResult sr = block_select_window<kLT, KX>(key, d, k_in, 30, 16, sm.u.a.sel);
        LAYER_MARK(1);
        selection_bitmap<kLT, KX>(key, d, sr, sm.u.a.sel);
        // this workgroup's kept inputs, ranks [ra, rb) in ascending index
        // order: each slot's rank from its word's count of kept inputs before it
        const int nw = d >> 5;
        uint32_t tot;
        const uint32_t wm = tid < nw ? sm.u.a.sel.bits[tid] : 0u;
        const uint32_t pre = block_excl_scan<kLT>((uint32_t)__popc(wm), sm.u.a.sel.scratch, &tot);
        if (tid < nw) sm.u.a.wpre[tid] = pre;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < KX; ++r) {
            const int i = slot_index<KX>(r);
            const uint32_t m = sm.u.a.sel.bits[i >> 5];
            if ((m >> (i & 31)) & 1u) {
                const uint32_t rank = sm.u.a.wpre[i >> 5] + (uint32_t)__popc(m & ((1u << (i & 31)) - 1u));
                if (rank >= (uint32_t)ra && rank < (uint32_t)rb)
                    sm.u.a.list[rank - ra] = (uint32_t)i | (__float_as_uint(xv[r]) & 0xFFFF0000u);
            }
        }
    }
    __syncthreads();
    LAYER_MARK(2);

    // ---- B. proxy GEMV: kept inputs [ra, rb) of block c; a lane holds 16
    // channels of gate and of up (16-byte loads: 1 KB of a half-row per wave)
    float acc[2][16];
#pragma unroll
    for (int n = 0; n < 16; ++n) acc[0][n] = acc[1][n] = 0.0f;
    {
        const uint32_t half_bytes = (uint32_t)F, row_bytes = 2u * (uint32_t)F;
        const __amdgpu_buffer_rsrc_t crs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.codes), (short)0, (int)(row_bytes * (uint32_t)d),
                                              CoherentBuf::kWord3);
        const uint32_t oob = row_bytes * (uint32_t)d;  // reads 0, touches no memory
        const int col = c * kLCB + lane * 16;
        for (int rbase = ra + wv; rbase < rb; rbase += kLW * kLUnits) {
            u32x4 qg[kLUnits], qu[kLUnits];
#pragma unroll
            for (int m = 0; m < kLUnits; ++m) {
                const int r = rbase + kLW * m;
                const uint32_t row = sm.u.a.list[min(r, rb - 1) - ra] & 0xFFFFu;
                const uint32_t o = (r < rb && col < F) ? row * row_bytes + (uint32_t)col : oob;
                qg[m] = ld_buf16(crs, o);
                qu[m] = ld_buf16(crs, o + half_bytes);
            }
#pragma unroll
            for (int m = 0; m < kLUnits; ++m) {
                const int r = rbase + kLW * m;
                if (r < rb) {  // wave-uniform
                    const float xk = __uint_as_float(sm.u.a.list[r - ra] & 0xFFFF0000u);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int n = 0; n < 4; ++n) {
                            acc[0][4 * q + n] = fmaf(xk, (float)(int8_t)(qg[m][q] >> (8 * n)), acc[0][4 * q + n]);
                            acc[1][4 * q + n] = fmaf(xk, (float)(int8_t)(qu[m][q] >> (8 * n)), acc[1][4 * q + n]);
                        }
                }
            }
        }
    }
    __syncthreads();  // the list is read: red may take its place
    LAYER_MARK(3);
    // the block's partial: the waves' sums added in a fixed tree (wave w + s
    // into wave w, s = 8, 4, 2, 1), gate then up, every lane of the writing
    // waves active (an LDS instruction costs its whole wave's slots even with
    // lanes masked off); wave 0 stores the sums, 16-byte coherent stores
    if (gemv) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int st = kLW / 2; st >= 1; st >>= 1) {
                if (wv >= st && wv < 2 * st) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<float4 *>(&sm.u.tree[wv - st][lane][4 * q]) =
                            make_float4(acc[h][4 * q], acc[h][4 * q + 1], acc[h][4 * q + 2], acc[h][4 * q + 3]);
                }
                __syncthreads();
                if (wv < st) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 o = *reinterpret_cast<const float4 *>(&sm.u.tree[wv][lane][4 * q]);
                        acc[h][4 * q] += o.x;
                        acc[h][4 * q + 1] += o.y;
                        acc[h][4 * q + 2] += o.z;
                        acc[h][4 * q + 3] += o.w;
                    }
                }
                __syncthreads();
            }
        }
        if (wv == 0) {
            const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
                a.part + (int64_t)w * 2 * kLCB, (short)0, (int)(sizeof(float) * 2 * kLCB), CoherentBuf::kWord3);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(acc[h][4 * q + e]);
                    __builtin_amdgcn_raw_buffer_store_b128(
                        v, prs, (int)(sizeof(float) * (h * kLCB + lane * 16 + 4 * q)), 0, CoherentBuf::kSc1);
                }
        }
    }
    LAYER_MARK(4);
    // block barrier: every workgroup of block c has stored its partial.  Each
    // then scores its slice of the block's channels, adding the workgroups'
    // partials in workgroup order (a single scorer per block would read all
    // of them through one CU); the last workgroup to store its scores selects
    // the top k
    bool topk_here = false;
    if (gemv) {
        __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
        __syncthreads();
        if (tid == 0) {
            uint32_t *arrived = &a.counters[kLayerBlockSyncBase + kLayerBlockSyncStride * c], *passed = arrived + 1;
            atomic_add_u32(arrived, 1u);
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (load_agent_u32(arrived) < (uint32_t)gpb) {
                __builtin_amdgcn_s_sleep(1);
                if (__builtin_amdgcn_s_memrealtime() - t0 > a.spin_ticks) {
                    atomic_add_u32(&a.counters[kLayerErrorSlot], 1u);
                    sm.err = 1;
                    break;
                }
            }
            if (atomic_add_u32(passed, 1u) == (uint32_t)gpb - 1u) {  // every workgroup of the block is past the wait
                store_agent_u32(arrived, 0u);
                store_agent_u32(passed, 0u);
            }
        }
        __syncthreads();
        LAYER_MARK(5);
        const int ch0 = jw * kLCB / gpb, nch = (jw + 1) * kLCB / gpb - ch0;  // this workgroup's channels of the block
        if (tid < nch) {
            const int ch = ch0 + tid, j = c * kLCB + ch;
            float g = 0.0f, u = 0.0f;
            const CoherentBuf pbuf(a.part, (uint32_t)(sizeof(float) * G * 2 * kLCB));
            const uint32_t end = (uint32_t)(sizeof(float) * G * 2 * kLCB);
            for (int q0 = 0; q0 < gpb; q0 += 24) {
                float tg[24], tu[24];
#pragma unroll
                for (int i = 0; i < 24; ++i) {
                    const int ww = c * gpb + q0 + i;
                    const bool in = q0 + i < gpb;
                    tg[i] = pbuf.load(in ? (uint32_t)(sizeof(float) * ((ww * 2) * kLCB + ch)) : end);
                    tu[i] = pbuf.load(in ? (uint32_t)(sizeof(float) * ((ww * 2 + 1) * kLCB + ch)) : end);
                }
#pragma unroll
                for (int i = 0; i < 24; ++i)
                    if (q0 + i < gpb) {
                        g += tg[i];
                        u += tu[i];
                    }
            }
            if (j < F) store_agent(&a.score[j], salience(a.signal, a.act, g * a.qscales[j], u * a.qscales[F + j]));
        }
        LAYER_MARK(6);
        __builtin_amdgcn_s_waitcnt(0);  // the scores have completed
        __syncthreads();
        if (tid == 0) {
            const uint32_t n_gemv = (uint32_t)(n_cb * gpb);
            const uint32_t t = atomic_add_u32(&a.counters[kFusedScoreSlot], 1u);
            if (t == n_gemv - 1u) store_agent_u32(&a.counters[kFusedScoreSlot], 0u);
            sm.flag = t == n_gemv - 1u;
        }
        __syncthreads();
        topk_here = sm.flag != 0;
        LAYER_MARK(7);
    }
    if (topk_here) {  // every score is in place: the top k, published as bitmap words and counts
        uint32_t fk[KF];
#pragma unroll
        for (int r = 0; r < KF; ++r) fk[r] = __float_as_uint(load_agent(&a.score[min(slot_index<KF>(r), F - 1)]));
        // slots past F get the key 0xFFFFFFFF, which no selection step takes
#pragma unroll
        for (int r = 0; r < KF; ++r) fk[r] = (slot_index<KF>(r) < F) ? (fk[r] & 0x7FFFFFFFu) : 0xFFFFFFFFu;
        LAYER_MARK(8);
        // scores are sign-free: the window is bits 30..0
        const SelectResult st = block_select_window<kLT, KF>(fk, F, k, 30, 0, sm.u.topk.sel);
        LAYER_MARK(9);
        selection_bitmap<kLT, KF>(fk, F, st, sm.u.topk.sel);
        const int nw = (F + 31) >> 5;  // <= kLSelWords
        const uint32_t m = tid < nw ? sm.u.topk.sel.bits[tid] : 0u;
        uint32_t tot;
        const uint32_t pre = block_excl_scan<kLT>((uint32_t)__popc(m), sm.u.topk.sel.scratch, &tot);
        if (tid < nw) {
            store_agent_u32(&a.selw[tid], m);
            store_agent_u32(&a.selw[kLSelWords + tid], pre);
        }
        LAYER_MARK(10);
    }

    // ---- C. the selection in place
    if (!grid_barrier(a.counters, G, 1u, 2u, a.spin_ticks, &sm.flag) && tid == 0) sm.err = 1;
    LAYER_MARK(11);

    // ---- D. this workgroup's ranks [r0, r1) of the selected channels
    const int r0 = (int)((int64_t)w * k / G), r1 = (int)((int64_t)(w + 1) * k / G);
    const int nc = r1 - r0;
    {
        const int nw = (F + 31) >> 5;
        const uint32_t m = tid < nw ? load_agent_u32(&a.selw[tid]) : 0u;
        uint32_t p = tid < nw ? load_agent_u32(&a.selw[kLSelWords + tid]) : 0u;
        const uint32_t cnt = (uint32_t)__popc(m);
        if (cnt && p < (uint32_t)r1 && p + cnt > (uint32_t)r0) {
            uint32_t b = m;
            while (b) {
                const int bit = __ffs(b) - 1;
                if (p >= (uint32_t)r0 && p < (uint32_t)r1) sm.u.e.chan[p - r0] = 32 * tid + bit;
                ++p;
                b &= b - 1u;
            }
        }
    }
    __syncthreads();
    if (a.sel_out && tid < nc) a.sel_out[r0 + tid] = sm.u.e.chan[tid];
    LAYER_MARK(12);

    // ---- E. Stage 2 on channels r0 .. r1 - 1: half h takes list entries
    // 2i + h; round rd covers entries [2 RC rd, 2 RC (rd + 1))
    float yacc[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q) yacc[q] = 0.0f;
    {
        const uint32_t rowb = 2u * (uint32_t)d;  // bytes of a row
        const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.w_gu), (short)0, (int)(2u * rowb * (uint32_t)F), CoherentBuf::kWord3);
        const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.w_dt), (short)0, (int)(rowb * (uint32_t)F), CoherentBuf::kWord3);
        const uint32_t goob = 2u * rowb * (uint32_t)F, doob = rowb * (uint32_t)F;
        const uint32_t coff = (uint32_t)(ht * CPT * 2);
        u32x4 ag[RC][NV], au[RC][NV], ad[RC][NV], bg[RC][NV], bu[RC][NV], bd[RC][NV];
        auto issue = [&](u32x4(&vg)[RC][NV], u32x4(&vu)[RC][NV], u32x4(&vd)[RC][NV], int rd) {
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                const int i = (rd * RC + c) * 2 + half;
                const bool live = i < nc;
                const uint32_t j = (uint32_t)sm.u.e.chan[live ? i : 0];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    vg[c][v] = ld_buf16(grs, live ? j * 2u * rowb + coff + 16u * v : goob);
                    vu[c][v] = ld_buf16(grs, live ? j * 2u * rowb + rowb + coff + 16u * v : goob);
                    vd[c][v] = ld_buf16(drs, live ? j * rowb + coff + 16u * v : doob);
                }
            }
        };
        auto process = [&](const u32x4(&vg)[RC][NV], const u32x4(&vu)[RC][NV], const u32x4(&vd)[RC][NV],
                           int rd) {
            float pg[RC], pu[RC];
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                float g = 0.0f, u = 0.0f;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float fg[8], fu[8];
                    vec16<uint16_t>::unpack(vg[c][v], fg);
                    vec16<uint16_t>::unpack(vu[c][v], fu);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        g = fmaf(fg[q], xs[8 * v + q], g);
                        u = fmaf(fu[q], xs[8 * v + q], u);
                    }
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
            if (tid < 2 * RC) {  // channel c of half h: that half's eight waves in order
                const int h = tid / RC, c = tid % RC;
                float tg[kLW / 2], tu[kLW / 2];
#pragma unroll
                for (int ww = 0; ww < kLW / 2; ++ww) {
                    tg[ww] = sm.u.e.r2[8 * h + ww][c];
                    tu[ww] = sm.u.e.r2[8 * h + ww][RC + c];
                }
                float g = tg[0], u = tu[0];
#pragma unroll
                for (int ww = 1; ww < kLW / 2; ++ww) {
                    g += tg[ww];
                    u += tu[ww];
                }
                sm.u.e.sv[h][c] = ((rd * RC + c) * 2 + h < nc) ? gate_act(a.act, g) * u : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                const float sv = sm.u.e.sv[half][c];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float fd[8];
                    vec16<uint16_t>::unpack(vd[c][v], fd);
#pragma unroll
                    for (int q = 0; q < 8; ++q) yacc[8 * v + q] = fmaf(sv, fd[q], yacc[8 * v + q]);
                }
            }
        };
        const int nr = (nc + 2 * RC - 1) / (2 * RC);
        if (nr > 0) issue(ag, au, ad, 0);
        for (int rd = 0; rd < nr; rd += 2) {
            issue(bg, bu, bd, rd + 1);  // past the last round: no memory is touched
            process(ag, au, ad, rd);
            if (rd + 1 < nr) {
                issue(ag, au, ad, rd + 2);
                process(bg, bu, bd, rd + 1);
            }
        }
    }
    LAYER_MARK(13);
    // the halves' sums added (first half + second half), the partial stored
    __syncthreads();  // the Stage-2 LDS is read
    if (half == 1) {
#pragma unroll
        for (int q = 0; q < CPT; ++q) sm.u.yhalf[ht][q] = yacc[q];
    }
    __syncthreads();
    if (half == 0) {  // 16-byte stores, device-coherent like the atomic stores
        const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
            a.ypart + (int64_t)w * d, (short)0, (int)(sizeof(float) * d), CoherentBuf::kWord3);
#pragma unroll
        for (int q = 0; q < CPT; q += 4) {
            u32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(yacc[q + i] + sm.u.yhalf[ht][q + i]);
            __builtin_amdgcn_raw_buffer_store_b128(v, yrs, (int)(sizeof(float) * (ht * CPT + q)), 0, CoherentBuf::kSc1);
        }
    }

    // ---- F. every partial in place; this workgroup's columns
    if (!grid_barrier(a.counters, G, 2u, 2u, a.spin_ticks, &sm.flag) && tid == 0) sm.err = 1;
    LAYER_MARK(14);
    const int cA = (int)((int64_t)w * d / G), cB = (int)((int64_t)(w + 1) * d / G);
    const int ncol = cB - cA;  // <= 32
    {
        const int col = tid & 31, grp = tid >> 5;  // grp: partials grp, grp + 32, ...
        float v = 0.0f;
        if (col < ncol) {
            const CoherentBuf ybuf(a.ypart, (uint32_t)(sizeof(float) * G * d));
            constexpr int QB = 8;
            for (int p0 = grp; p0 < G; p0 += kLSumGroups * QB) {
                float t8[QB];
#pragma unroll
                for (int i = 0; i < QB; ++i) {
                    const int p = p0 + kLSumGroups * i;
                    t8[i] = ybuf.load(p < G ? (uint32_t)(sizeof(float) * ((int64_t)p * d + cA + col))
                                            : (uint32_t)(sizeof(float) * G * d));
                }
#pragma unroll
                for (int i = 0; i < QB; ++i)
                    if (p0 + kLSumGroups * i < G) v += t8[i];
            }
        }
        sm.u.sums[grp][col] = v;
    }
    __syncthreads();
    if (tid < ncol) {
        float t[kLSumGroups];
#pragma unroll
        for (int g = 0; g < kLSumGroups; ++g) t[g] = sm.u.sums[g][tid];
        float y = t[0];
#pragma unroll
        for (int g = 1; g < kLSumGroups; ++g) y += t[g];
        const bool bad = sm.err != 0 || load_agent_u32(&a.counters[kLayerErrorSlot]) != 0u;
        if (a.residual) y += __uint_as_float((uint32_t)a.residual[cA + tid] << 16);
        a.out[cA + tid] = bad ? (uint16_t)0x7FC0u : f32_to_bf16(y);
    }
    LAYER_MARK(15);
}

// ------------------------------------------------------------------------
bool layer_supported(int64_t B, int64_t d, int64_t F, int64_t k_in, int64_t k, int G)
{
    if (B != 1 || (d != 4096 && d != 8192) || F > kFusedMaxF || F < 16) return false;
    if (G < 64 || G > kLayerMaxGroups) return false;
    if (k <= 0 || k >= F || k_in < 1 || k_in > d) return false;
    // G >= 64 >= 4 blocks per workgroup: each GEMV share is at most d / 4 <= 2048 kept inputs
    return (k + G - 1) / G <= kLMaxChan && (d + G - 1) / G <= 32;
}

hipError_t launch_layer(const void *x, int d, int F, int k_in, int k, const uint8_t *codes, const float *qscales,
                        const void *w_gu, const void *w_dt, const void *residual, void *out, int32_t *sel_out,
                        float *part, float *score, uint32_t *selw, float *ypart, uint32_t *counters, int act,
                        int signal, uint64_t spin_ticks, int G, hipStream_t st)
{
    if (!layer_supported(1, d, F, k_in, k, G)) return hipErrorInvalidValue;
    LayerArgs a;
    a.x = (const uint16_t *)x;
    a.codes = codes;
    a.qscales = qscales;
    a.w_gu = (const uint16_t *)w_gu;
    a.w_dt = (const uint16_t *)w_dt;
    a.residual = (const uint16_t *)residual;
    a.out = (uint16_t *)out;
    a.sel_out = sel_out;
    a.part = part;
    a.score = score;
    a.selw = selw;
    a.ypart = ypart;
    a.counters = counters;
    a.spin_ticks = spin_ticks ? spin_ticks : kDefaultSpinTicks;
    a.d = d;
    a.F = F;
    a.k_in = k_in;
    a.k = k;
    a.G = G;
    a.n_cb = (F + kLCB - 1) / kLCB;
    a.act = act;
    a.signal = signal;
    const int kf = (F + kLT - 1) / kLT;
    if (d == 4096) {
        if (kf <= 8) layer_kernel<4, 8><<<G, kLT, 0, st>>>(a);
        else layer_kernel<4, 16><<<G, kLT, 0, st>>>(a);
    } else {
        if (kf <= 8) layer_kernel<8, 8><<<G, kLT, 0, st>>>(a);
        else layer_kernel<8, 16><<<G, kLT, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace prox

namespace prox {

int layer_groups()
{
    constexpr int kMaxDevices = 64;
    static int cache[kMaxDevices];  // groups + 1 per device; 0: not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    const int c = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (c) return c - 1;
    int cus = 0, g = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) {
        const void *fns[] = {(const void *)layer_kernel<4, 8>, (const void *)layer_kernel<4, 16>,
                             (const void *)layer_kernel<8, 8>, (const void *)layer_kernel<8, 16>};
        int occ = 1 << 30;
        for (const void *f : fns) {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kLT, 0) != hipSuccess) n = 0;
            occ = n < occ ? n : occ;
        }
        if (occ >= 1) g = cus < kLayerMaxGroups ? cus : kLayerMaxGroups;
    }
    (void)hipGetLastError();  // a failed query leaves no error for the next call to report
    __atomic_store_n(&cache[dev], g + 1, __ATOMIC_RELAXED);
    return g;
}

}  // namespace prox
