// Block-wide exact top-k selection over uint32 keys (larger key first, ties
// to the lower index), used for Stage 1's input sparsification and for the
// channel mask.  Keys are magnitudes' IEEE bit patterns, whose unsigned order
// is the order of the magnitudes.
//
// Ownership is wave-contiguous: wave w holds the indices
// [w*64*KPT, (w+1)*64*KPT), lane l's slot r being index w*64*KPT + r*64 + l,
// so every register load is a coalesced 256-byte wave access and the ordered
// compaction needs only ballots within a wave plus one scan over waves.
//
// The k-th largest key T is found by MSB-first radix select over the bit
// window where the keys differ (bits all keys share, above and below, are
// skipped), 9 bits per pass.  The LDS histogram has 16 copies, one per
// (lane mod 16), so lanes of a wave that land in the same bin are spread over
// copies: same-address LDS atomics serialize, and score distributions are
// peaked enough that a single copy would make them the bottleneck.
#pragma once

#include "common.h"

namespace prox {

struct SelectResult {
    uint32_t T;        // k-th largest key
    uint32_t need_eq;  // how many keys equal to T are selected (lowest indices)
};

constexpr int kDigit = 9;
constexpr int kBins = 1 << kDigit;
constexpr int kCopies = 16;

struct SelectSmem {
    uint32_t hist[kCopies][kBins];
    uint32_t scratch[64];
    uint32_t found[2];
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

// n valid keys in total; slots with index >= n are ignored.  1 <= k <= n.
template <int NT, int KPT>
__device__ SelectResult block_select_kth(const uint32_t (&key)[KPT], int n, int k, SelectSmem &sm)
{
    static_assert(NT >= kBins, "one thread per bin");
    const int tid = threadIdx.x;
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
        return res;
    }
    int cursor = 31 - __clz(diff);       // highest bit where keys differ
    const int lowest = __ffs(diff) - 1;  // lowest bit where keys differ
    uint32_t known = (cursor == 31) ? 0u : ~((2u << cursor) - 1u);
    known |= (1u << lowest) - 1u;        // common bits below the window
    uint32_t prefix = all_and & known;
    uint32_t remaining = (uint32_t)k;
    uint32_t *flat = &sm.hist[0][0];
    const int copy = tid & (kCopies - 1);

    while (cursor >= lowest) {
        const int span = cursor - lowest + 1;
        const int width = span < kDigit ? span : kDigit;
        const int shift = cursor + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        const int nb = 1 << width;
        for (int e = tid; e < kCopies * kBins; e += NT) flat[e] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < KPT; ++r)
            if (slot_index<KPT>(r) < n && (key[r] & known) == prefix)
                atomicAdd(&sm.hist[copy][(key[r] >> shift) & dmask], 1u);
        __syncthreads();
        // thread t < nb owns bin nb-1-t (descending digit order)
        uint32_t h = 0;
        const int bin = nb - 1 - tid;
        if (bin >= 0)
#pragma unroll
            for (int c = 0; c < kCopies; ++c) h += sm.hist[c][bin];
        uint32_t tot;
        const uint32_t above = block_excl_scan<NT>(h, sm.scratch, &tot);
        if (bin >= 0 && above < remaining && remaining <= above + h) {
            sm.found[0] = (uint32_t)bin;
            sm.found[1] = above;
        }
        __syncthreads();
        const uint32_t digit = sm.found[0];
        remaining -= sm.found[1];
        prefix |= digit << shift;
        known |= dmask << shift;
        cursor = shift - 1;
    }
    res.T = prefix;
    res.need_eq = remaining;
    return res;
}

// Selection of this thread's slots given the threshold: returns a bit mask
// (bit r = slot r selected) and, per selected slot, its rank among the
// selected indices in ascending index order (pos[r]).
template <int NT, int KPT>
__device__ uint64_t block_select_flags(const uint32_t (&key)[KPT], int n, SelectResult sr, SelectSmem &sm,
                                       uint32_t (&pos)[KPT])
{
    uint64_t eqm[KPT];
    uint32_t eq_wave = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        eqm[r] = __ballot(slot_index<KPT>(r) < n && key[r] == sr.T);
        eq_wave += (uint32_t)__popcll(eqm[r]);
    }
    uint32_t eq_tot;
    uint32_t eq_before = waves_excl_scan<NT>(eq_wave, sm.scratch, &eq_tot);
    uint64_t selm[KPT];
    uint32_t sel_wave = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const bool valid = slot_index<KPT>(r) < n;
        bool s = valid && key[r] > sr.T;
        if (valid && key[r] == sr.T) s = (eq_before + lanes_below(eqm[r])) < sr.need_eq;
        eq_before += (uint32_t)__popcll(eqm[r]);
        selm[r] = __ballot(s);
        sel_wave += (uint32_t)__popcll(selm[r]);
    }
    uint32_t sel_tot;
    uint32_t sel_before = waves_excl_scan<NT>(sel_wave, sm.scratch, &sel_tot);
    uint64_t flags = 0;
    const uint64_t me = 1ull << (threadIdx.x & 63);
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        if (selm[r] & me) {
            flags |= 1ull << r;
            pos[r] = sel_before + lanes_below(selm[r]);
        }
        sel_before += (uint32_t)__popcll(selm[r]);
    }
    return flags;
}

}  // namespace prox
