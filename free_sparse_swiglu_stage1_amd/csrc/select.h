// Block-wide exact top-k selection over uint32 keys (larger key first, ties
// to the lower index), used for Stage 1's input sparsification and for the
// channel mask.  Keys are magnitudes' IEEE bit patterns (sign bit clear),
// whose unsigned order is the order of the magnitudes.
//
// Ownership is wave-contiguous: wave w holds the indices
// [w*64*KPT, (w+1)*64*KPT), lane l's slot r being index w*64*KPT + r*64 + l,
// so every register load is a coalesced 256-byte wave access and the ordered
// compaction needs only ballots within a wave plus one scan over waves.
//
// The k-th largest key T is found by MSB-first radix select over the bit
// window where the keys differ (bits all keys share are skipped).  The first
// pass takes the top 15 bits of the window at once, into 32768 bins of packed
// 16-bit counters (64 KB of LDS): with that many bins, keys of nearby value
// rarely hit the same counter, so the LDS atomics do not serialize, and for
// bf16-derived keys this one pass decides T.  The at most 16 bits left are
// resolved over the few remaining candidates with 8-bit passes whose
// histogram has 16 copies, one per (lane mod 16), to spread equal bins.
#pragma once

#include "common.h"

namespace prox {

struct SelectResult {
    uint32_t T;         // k-th largest key
    uint32_t need_eq;   // how many keys equal to T are selected (lowest indices)
    uint32_t count_eq;  // how many keys equal T
};

constexpr int kWideBits = 15;
constexpr int kNarrowBits = 8;
constexpr int kCopies = 16;

struct SelectSmem {
    union {
        uint32_t wide[1 << (kWideBits - 1)];          // 2^15 16-bit counters, two per word
        uint32_t narrow[kCopies][1 << kNarrowBits];   // 16 copies of 256 bins
    };
    uint32_t scratch[64];
    uint32_t found[3];
};

template <int KPT>
__device__ __forceinline__ int slot_index(int r)
{
    return (threadIdx.x >> 6) * 64 * KPT + r * 64 + (threadIdx.x & 63);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive scan of one value per wave (in wave order) and the block total.
template <int NT>
__device__ __forceinline__ uint32_t waves_excl_scan(uint32_t wave_val, uint32_t *scratch, uint32_t *total)
{
    constexpr int NW = NT / kWave;
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) scratch[wid] = wave_val;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t s = scratch[w];
        before += (w < wid) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return before;
}

// The wide pass: 2^15 bins of the 15 bits at `shift`, packed 16-bit
// counters.  Thread t owns the 2^15/NT bins just below 2^15 - t*2^15/NT (the
// highest bins go to thread 0), reads its counter words once with 16-byte
// LDS loads and finds the crossing bin in registers.
template <int NT, int KPT>
__device__ __forceinline__ uint32_t wide_pass(const uint32_t (&key)[KPT], int n, int shift, uint32_t &prefix,
                                              uint32_t &known, uint32_t &remaining, SelectSmem &sm)
{
    constexpr int NWORDS = 1 << (kWideBits - 1);
    constexpr int WPT = NWORDS / NT;  // counter words per thread
    static_assert(WPT % 4 == 0, "16-byte LDS accesses");
    const int tid = threadIdx.x;
    const int w0 = NWORDS - (tid + 1) * WPT;  // this thread's first word
    u32x4 *mine = reinterpret_cast<u32x4 *>(&sm.wide[w0]);
#pragma unroll
    for (int i = 0; i < WPT / 4; ++i) mine[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    const uint32_t dmask = (1u << kWideBits) - 1u;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        if (slot_index<KPT>(r) < n && (key[r] & known) == prefix) {
            const uint32_t dg = (key[r] >> shift) & dmask;
            atomicAdd(&sm.wide[dg >> 1], 1u << ((dg & 1u) * 16u));
        }
    }
    __syncthreads();
    uint32_t w[WPT];
#pragma unroll
    for (int i = 0; i < WPT / 4; ++i) {
        const u32x4 v = mine[i];
        w[4 * i] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < WPT; ++i) local += (w[i] & 0xFFFFu) + (w[i] >> 16);
    uint32_t tot;
    uint32_t above = block_excl_scan<NT>(local, sm.scratch, &tot);
    if (above < remaining && remaining <= above + local) {
        bool done = false;
#pragma unroll
        for (int i = WPT - 1; i >= 0; --i) {
#pragma unroll
            for (int half = 1; half >= 0; --half) {
                const uint32_t h = (w[i] >> (16 * half)) & 0xFFFFu;
                if (!done && above < remaining && remaining <= above + h) {
                    sm.found[0] = (uint32_t)(2 * (w0 + i) + half);
                    sm.found[1] = above;
                    sm.found[2] = h;
                    done = true;
                }
                above += h;
            }
        }
    }
    __syncthreads();
    const uint32_t digit = sm.found[0];
    remaining -= sm.found[1];
    const uint32_t in_bin = sm.found[2];
    prefix |= digit << shift;
    known |= dmask << shift;
    __syncthreads();
    return in_bin;
}

// A narrow pass: bins of `width` (<= 8) bits at `shift` among the keys whose
// `known` bits equal `prefix`, 16 counter copies.
template <int NT, int KPT>
__device__ __forceinline__ uint32_t narrow_pass(const uint32_t (&key)[KPT], int n, int width, int shift,
                                                uint32_t &prefix, uint32_t &known, uint32_t &remaining,
                                                SelectSmem &sm)
{
    static_assert(NT >= (1 << kNarrowBits), "one thread per bin");
    const int tid = threadIdx.x;
    const uint32_t dmask = (1u << width) - 1u;
    const int nb = 1 << width;
    for (int e = tid; e < kCopies * (1 << kNarrowBits); e += NT) (&sm.narrow[0][0])[e] = 0u;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < KPT; ++r)
        if (slot_index<KPT>(r) < n && (key[r] & known) == prefix)
            atomicAdd(&sm.narrow[tid & (kCopies - 1)][(key[r] >> shift) & dmask], 1u);
    __syncthreads();
    const int bin = nb - 1 - tid;  // thread t owns bin nb-1-t
    uint32_t h = 0;
    if (bin >= 0)
#pragma unroll
        for (int q = 0; q < kCopies; ++q) h += sm.narrow[q][bin];
    uint32_t tot;
    const uint32_t above = block_excl_scan<NT>(h, sm.scratch, &tot);
    if (bin >= 0 && above < remaining && remaining <= above + h) {
        sm.found[0] = (uint32_t)bin;
        sm.found[1] = above;
        sm.found[2] = h;
    }
    __syncthreads();
    const uint32_t digit = sm.found[0];
    remaining -= sm.found[1];
    const uint32_t in_bin = sm.found[2];
    prefix |= digit << shift;
    known |= dmask << shift;
    __syncthreads();
    return in_bin;
}

// n valid keys in total; slots with index >= n are ignored.  1 <= k <= n.
template <int NT, int KPT>
__device__ SelectResult block_select_kth(const uint32_t (&key)[KPT], int n, int k, SelectSmem &sm)
{
    uint32_t a = 0xFFFFFFFFu, o = 0u;
#pragma unroll
    for (int r = 0; r < KPT; ++r)
        if (slot_index<KPT>(r) < n) {
            a &= key[r];
            o |= key[r];
        }
    uint32_t all_or;
    const uint32_t all_and = block_and_or<NT>(a, o, sm.scratch, &all_or);
    const uint32_t diff = all_and ^ all_or;
    SelectResult res;
    if (diff == 0u) {  // every key equal
        res.T = all_and;
        res.need_eq = (uint32_t)k;
        res.count_eq = (uint32_t)n;
        return res;
    }
    int cursor = 31 - __clz(diff);       // highest bit where keys differ
    const int lowest = __ffs(diff) - 1;  // lowest bit where keys differ
    uint32_t known = (cursor == 31) ? 0u : ~((2u << cursor) - 1u);
    known |= (1u << lowest) - 1u;        // common bits below the window
    uint32_t prefix = all_and & known;
    uint32_t remaining = (uint32_t)k;
    // wide pass: the 15 bits from the top of the window (extending below the
    // window when it is narrower; those bits are common to every key)
    int shift = max(cursor + 1 - kWideBits, 0);
    uint32_t in_bin;
    if (cursor + 1 >= kWideBits) {
        known &= ~(((1u << kWideBits) - 1u) << shift);
        prefix &= known;
        in_bin = wide_pass<NT, KPT>(key, n, shift, prefix, known, remaining, sm);
        cursor = shift - 1;
    } else {
        in_bin = (uint32_t)n;
    }
    while (cursor >= lowest) {
        const int span = cursor - lowest + 1;
        const int width = span < kNarrowBits ? span : kNarrowBits;
        shift = cursor + 1 - width;
        in_bin = narrow_pass<NT, KPT>(key, n, width, shift, prefix, known, remaining, sm);
        cursor = shift - 1;
    }
    res.T = prefix;
    res.need_eq = remaining;
    res.count_eq = in_bin;  // the last pass's bin holds exactly the keys equal to T
    return res;
}

// Selection of this thread's slots given the threshold: returns a bit mask
// (bit r = slot r selected) and, per selected slot, its rank among the
// selected indices in ascending index order (pos[r]).  When every key equal
// to T is selected (the usual case), no ranking among equal keys is needed.
template <int NT, int KPT>
__device__ uint64_t block_select_flags(const uint32_t (&key)[KPT], int n, SelectResult sr, SelectSmem &sm,
                                       uint32_t (&pos)[KPT])
{
    uint64_t selm[KPT];
    if (sr.need_eq == sr.count_eq) {
#pragma unroll
        for (int r = 0; r < KPT; ++r) selm[r] = __ballot(slot_index<KPT>(r) < n && key[r] >= sr.T);
    } else {
        uint64_t eqm[KPT];
        uint32_t eqc[KPT];
        uint32_t eq_wave = 0;
#pragma unroll
        for (int r = 0; r < KPT; ++r) eqm[r] = __ballot(slot_index<KPT>(r) < n && key[r] == sr.T);
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            eqc[r] = eq_wave;
            eq_wave += (uint32_t)__popcll(eqm[r]);
        }
        uint32_t eq_tot;
        const uint32_t eq_before = waves_excl_scan<NT>(eq_wave, sm.scratch, &eq_tot);
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const bool valid = slot_index<KPT>(r) < n;
            bool s = valid && key[r] > sr.T;
            if (valid && key[r] == sr.T) s = (eq_before + eqc[r] + lanes_below(eqm[r])) < sr.need_eq;
            selm[r] = __ballot(s);
        }
    }
    uint32_t selc[KPT];
    uint32_t sel_wave = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        selc[r] = sel_wave;
        sel_wave += (uint32_t)__popcll(selm[r]);
    }
    uint32_t sel_tot;
    const uint32_t sel_before = waves_excl_scan<NT>(sel_wave, sm.scratch, &sel_tot);
    uint64_t flags = 0;
    const uint64_t me = 1ull << (threadIdx.x & 63);
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        if (selm[r] & me) {
            flags |= 1ull << r;
            pos[r] = sel_before + selc[r] + lanes_below(selm[r]);
        }
    }
    return flags;
}

}  // namespace prox
