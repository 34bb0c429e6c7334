// Block-wide exact top-k selection over uint32 keys (larger key first, ties
// to the lower index), used for Stage 1's input sparsification and for the
// channel mask.  Keys are magnitudes' IEEE bit patterns, whose unsigned order
// is the order of the magnitudes.
//
// Each thread holds KPT keys for the contiguous index run [tid*KPT, tid*KPT+KPT)
// in registers.  The k-th largest key T is found by MSB-first radix select
// in LDS; digit passes start below the bits all keys share (AND/OR reduction),
// so peaked score distributions do not pile their LDS atomics on a few bins.
// The caller then selects key > T, plus the first `need_eq` keys == T in index
// order.
#pragma once

#include "common.h"

namespace prox {

struct SelectResult {
    uint32_t T;        // k-th largest key
    uint32_t need_eq;  // how many keys equal to T are selected (lowest indices)
};

struct SelectSmem {
    uint32_t hist[2048];
    uint32_t scratch[64];
    uint32_t found[2];
};

// n valid keys in total; keys beyond n (idx >= n) are ignored.  1 <= k <= n.
template <int NT, int KPT, int DIGIT>
__device__ SelectResult block_select_kth(const uint32_t (&key)[KPT], int n, int k, SelectSmem &sm)
{
    static_assert((1 << DIGIT) % NT == 0 || NT % (1 << DIGIT) == 0, "digit/thread mismatch");
    constexpr int NBINS = 1 << DIGIT;
    const int tid = threadIdx.x;
    const int base = tid * KPT;

    uint32_t a = 0xFFFFFFFFu, o = 0u;
#pragma unroll
    for (int r = 0; r < KPT; ++r)
        if (base + r < n) {
            a &= key[r];
            o |= key[r];
        }
    uint32_t all_or;
    uint32_t all_and = block_and_or<NT>(a, o, sm.scratch, &all_or);
    uint32_t diff = all_and ^ all_or;
    SelectResult res;
    if (diff == 0u) {  // every key equal
        res.T = all_and;
        res.need_eq = (uint32_t)k;
        return res;
    }
    int cursor = 31 - __clz(diff);  // highest bit that is not common
    uint32_t known_mask = (cursor == 31) ? 0u : ~((2u << cursor) - 1u);
    uint32_t prefix = all_and & known_mask;
    uint32_t remaining = (uint32_t)k;

    while (cursor >= 0) {
        const int width = (cursor + 1 < DIGIT) ? cursor + 1 : DIGIT;
        const int shift = cursor + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        const int nb = 1 << width;
        for (int b = tid; b < nb; b += NT) sm.hist[b] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < KPT; ++r)
            if (base + r < n && (key[r] & known_mask) == prefix)
                atomicAdd(&sm.hist[(key[r] >> shift) & dmask], 1u);
        __syncthreads();
        // bins in descending digit order: thread t owns bins [nb-1-t*BPT, nb-t*BPT)
        constexpr int BPT = (NBINS + NT - 1) / NT;
        uint32_t local = 0;
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            int bin = nb - 1 - (tid * BPT + q);
            if (bin >= 0) local += sm.hist[bin];
        }
        uint32_t tot;
        uint32_t above = block_excl_scan<NT>(local, sm.scratch, &tot);
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            int bin = nb - 1 - (tid * BPT + q);
            if (bin >= 0) {
                uint32_t h = sm.hist[bin];
                if (above < remaining && remaining <= above + h) {
                    sm.found[0] = (uint32_t)bin;
                    sm.found[1] = above;
                }
                above += h;
            }
        }
        __syncthreads();
        const uint32_t digit = sm.found[0];
        remaining -= sm.found[1];
        prefix |= digit << shift;
        known_mask |= dmask << shift;
        cursor = shift - 1;
        __syncthreads();
    }
    res.T = prefix;
    res.need_eq = remaining;
    return res;
}

// Selection flags for this thread's KPT keys, in index order, given the
// threshold.  Returns a bit mask (bit r = key r selected).
template <int NT, int KPT>
__device__ uint64_t block_select_flags(const uint32_t (&key)[KPT], int n, SelectResult sr, SelectSmem &sm,
                                       uint32_t *n_selected_before, uint32_t *n_selected_total)
{
    const int base = threadIdx.x * KPT;
    uint32_t eq = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) eq += (base + r < n && key[r] == sr.T) ? 1u : 0u;
    uint32_t eq_tot;
    uint32_t eq_before = block_excl_scan<NT>(eq, sm.scratch, &eq_tot);
    uint64_t flags = 0;
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        if (base + r >= n) continue;
        bool s = key[r] > sr.T;
        if (key[r] == sr.T) {
            s = eq_before < sr.need_eq;
            ++eq_before;
        }
        if (s) {
            flags |= 1ull << r;
            ++cnt;
        }
    }
    *n_selected_before = block_excl_scan<NT>(cnt, sm.scratch, n_selected_total);
    return flags;
}

}  // namespace prox
