// Block-wide exact top-k selection over uint32 keys (larger key first, ties
// to the lower index), used for Stage 1's input sparsification and for the
// channel mask.  Keys are magnitudes' IEEE bit patterns (sign bit clear),
// whose unsigned order is the order of the magnitudes.
//
// A workgroup retires about one wave64 instruction per clock, so the cost of
// a selection is the number of instructions spent per key plus the fixed
// cost of each pass (LDS clears, barriers).  The design keeps both small:
//  - keys stay in registers, wave-contiguous: wave w holds the indices
//    [w*64*KPT, (w+1)*64*KPT), lane l's slot r being index
//    w*64*KPT + r*64 + l, so a row r of a wave is 64 consecutive indices;
//  - the k-th largest key T is found by MSB-first radix passes of at most
//    11 bits (2048 counters, 8 KB of LDS) over the bit window where the
//    keys differ, stopping as soon as the keys of the crossing bin are
//    exactly the ones still needed;
//  - the selection ({key > T} and the lowest-index keys equal to T) is
//    written as a bitmap, one ballot per row, and compacted in index order
//    from the bitmap (one scan over words instead of one per key).
#pragma once

#include "common.h"

namespace prox {

constexpr int kPassBits = 11;
constexpr int kPassBins = 1 << kPassBits;
// Workgroups of 1024 threads count each bin in two words, lane l adding to
// copy l mod 2: keys of a wave that share a bin then often hit different
// words, and the LDS serializes fewer of its atomics.  Measured: the
// stand-alone selections of 4 tokens' inputs and of the mask 1.0 us faster
// together; in the 512-thread single-token kernel, whose two workgroups per
// CU share the LDS, two copies cost 0.6 us and four 2.7 us, so it keeps one.
constexpr int kHistCopiesMax = 2;
template <int NT>
__host__ __device__ constexpr int hist_copies()
{
    return NT >= 1024 ? 2 : 1;
}

struct SelectResult {
    uint32_t T;         // threshold key
    uint32_t need_eq;   // keys equal to T to select (lowest indices)
    uint32_t count_eq;  // keys equal to T; need_eq == count_eq: select key >= T
};

// MAXN: the largest key count (a multiple of 64).
template <int MAXN>
struct alignas(16) SelectSmem {
    static constexpr int W = MAXN / 32;  // bitmap words
    static_assert(MAXN % 64 == 0 && W <= kPassBins * (kHistCopiesMax - 1), "bitmap sizes");
    // radix counters; afterwards, from word kPassBins, the bitmap of keys
    // equal to T (above the bins a narrow last pass reads)
    uint32_t hist[kPassBins * kHistCopiesMax];
    uint32_t bits[W];          // selection bitmap: bit i of word i/32 = index i selected
    alignas(16) uint32_t scratch[64];
    uint32_t found[4];
};

template <int KPT>
__device__ __forceinline__ int slot_index(int r)
{
    return (threadIdx.x >> 6) * 64 * KPT + r * 64 + (threadIdx.x & 63);
}

// A value every lane holds alike, moved to a scalar register so that the
// branches on it are scalar.
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

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
    uint32_t sw[NW];
    lds_words<NW>(scratch, sw);
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        before += (w < wid) ? sw[w] : 0u;
        tot += sw[w];
    }
    __syncthreads();
    *total = tot;
    return before;
}

// Bin counts owned in thread order (thread t: bins [t*BPT, (t+1)*BPT)).
// Finds the bin holding the remaining-th largest key, counting from the top
// bin down: found[0] = bin, found[1] = keys in higher bins, found[2] = keys
// in the bin.  Requires 1 <= remaining <= total.  Two barriers.
template <int NT, int BPT>
__device__ __forceinline__ void find_crossing(const uint32_t (&h)[BPT], uint32_t remaining, uint32_t *scratch,
                                              uint32_t *found)
{
    constexpr int NW = NT / kWave;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) local += h[i];
    const uint32_t incl = wave_incl_scan(local);
    const uint32_t wtot = __builtin_amdgcn_readlane(incl, 63);
    if (lane == 0) scratch[wv] = wtot;
    __syncthreads();
    uint32_t a = wtot - incl;  // keys in this wave's higher threads
    uint32_t sw[NW];
    lds_words<NW>(scratch, sw);
#pragma unroll
    for (int w = 0; w < NW; ++w) a += (w > wv) ? sw[w] : 0u;
    if (a < remaining && remaining <= a + local) {
        bool done = false;
#pragma unroll
        for (int i = BPT - 1; i >= 0; --i) {
            if (!done && a < remaining && remaining <= a + h[i]) {
                found[0] = (uint32_t)(tid * BPT + i);
                found[1] = a;
                found[2] = h[i];
                done = true;
            }
            a += h[i];
        }
    }
    __syncthreads();
}

// One radix pass: counts the `width` (<= 11) bits at `shift` of the keys
// whose `known` bits equal `prefix`, finds the crossing bin and narrows the
// state to it.  Returns the number of keys in that bin.
template <int NT, int KPT, int MAXN>
__device__ __forceinline__ uint32_t radix_pass(const uint32_t (&key)[KPT], int n, int width, int shift,
                                               uint32_t &prefix, uint32_t &known, uint32_t &remaining,
                                               SelectSmem<MAXN> &sm)
{
    constexpr int BPT = kPassBins / NT;
    static_assert(BPT == 1 || BPT == 2 || BPT == 4, "bins per thread");
    constexpr int kHistCopies = hist_copies<NT>();
    static_assert(kHistCopies <= kHistCopiesMax, "histogram copies");
    constexpr int W = BPT * kHistCopies;  // this thread's words: its bins' copies
    const int tid = threadIdx.x;
    uint32_t *mine = &sm.hist[tid * W];
#pragma unroll
    for (int i = 0; i < W; i += 4) *reinterpret_cast<u32x4 *>(mine + i) = u32x4{0u, 0u, 0u, 0u};
    if (W == 2) *reinterpret_cast<u32x2 *>(mine) = u32x2{0u, 0u};
    if (W == 1) mine[0] = 0u;
    __syncthreads();
    const uint32_t dmask = (1u << width) - 1u;
    const uint32_t copy = (uint32_t)(tid & (kHistCopies - 1));
#pragma unroll
    for (int r = 0; r < KPT; ++r)
        if (slot_index<KPT>(r) < n && (key[r] & known) == prefix)
            atomicAdd(&sm.hist[((key[r] >> shift) & dmask) * kHistCopies + copy], 1u);
    __syncthreads();
    uint32_t bin, above, in_bin;
    if (width <= 6) {  // uniform
        // a narrow pass (always the last): every wave finds the crossing
        // itself, without a barrier.  Lane l takes bin nb - 1 - l, so the
        // inclusive scan over lanes counts the keys in that bin and above;
        // the first lane where that reaches `remaining` holds the crossing.
        const int lane = tid & 63, b = (1 << width) - 1 - lane;
        uint32_t hv = 0u;
        if (b >= 0) {
#pragma unroll
            for (int c = 0; c < kHistCopies; ++c) hv += sm.hist[b * kHistCopies + c];
        }
        const uint32_t incl = wave_incl_scan(hv);
        const uint64_t m = __ballot(b >= 0 && incl >= remaining);
        const int L = uniform(m ? (int)__builtin_ctzll(m) : 0);  // m != 0 when remaining <= total
        const uint32_t hl = (uint32_t)__builtin_amdgcn_readlane((int)hv, L);
        bin = (uint32_t)((1 << width) - 1 - L);
        above = (uint32_t)__builtin_amdgcn_readlane((int)incl, L) - hl;
        in_bin = hl;
    } else {
        uint32_t h[BPT];
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            h[i] = 0u;
#pragma unroll
            for (int c = 0; c < kHistCopies; ++c) h[i] += mine[i * kHistCopies + c];
        }
        find_crossing<NT, BPT>(h, remaining, sm.scratch, sm.found);
        bin = uniform_u32(sm.found[0]);
        above = uniform_u32(sm.found[1]);
        in_bin = uniform_u32(sm.found[2]);
    }
    remaining -= above;
    prefix |= bin << shift;
    known |= dmask << shift;
    return in_bin;
}

// Radix passes over the bits [lowest, cursor] below a known prefix, until
// the crossing bin holds exactly the keys still needed or every bit is known.
template <int NT, int KPT, int MAXN>
__device__ SelectResult radix_select_from(const uint32_t (&key)[KPT], int n, uint32_t prefix, uint32_t known,
                                          uint32_t remaining, int cursor, int lowest, SelectSmem<MAXN> &sm)
{
    uint32_t in_bin = 0;
    while (cursor >= lowest) {
        const int span = cursor - lowest + 1;
        const int width = span < kPassBits ? span : kPassBits;
        const int shift = cursor + 1 - width;
        in_bin = radix_pass<NT, KPT, MAXN>(key, n, width, shift, prefix, known, remaining, sm);
        cursor = shift - 1;
        if (remaining == in_bin) break;  // the whole bin is selected
    }
    // the bin's keys are >= prefix (unknown bits zero), lower keys < prefix,
    // higher keys > prefix; when every bit is known they all equal prefix
    SelectResult s;
    s.T = prefix;
    s.need_eq = remaining;
    s.count_eq = in_bin;
    return s;
}

// The k-th largest of n keys (1 <= k <= n; slots with index >= n ignored).
template <int NT, int KPT, int MAXN>
__device__ SelectResult block_select(const uint32_t (&key)[KPT], int n, int k, SelectSmem<MAXN> &sm)
{
    uint32_t a = 0xFFFFFFFFu, o = 0u;
#pragma unroll
    for (int r = 0; r < KPT; ++r)
        if (slot_index<KPT>(r) < n) {
            a &= key[r];
            o |= key[r];
        }
    uint32_t all_or;
    const uint32_t all_and = uniform_u32(block_and_or<NT>(a, o, sm.scratch, &all_or));
    const uint32_t diff = all_and ^ uniform_u32(all_or);
    if (diff == 0u) {  // every key equal: the k lowest indices
        SelectResult s;
        s.T = all_and;
        s.need_eq = (uint32_t)k;
        s.count_eq = (uint32_t)n;
        return s;
    }
    const int cursor = 31 - __clz(diff);  // highest bit where keys differ
    const int lowest = __ffs(diff) - 1;   // lowest bit where keys differ
    uint32_t known = (cursor == 31) ? 0u : ~((2u << cursor) - 1u);
    known |= (1u << lowest) - 1u;  // common bits below the window
    return radix_select_from<NT, KPT, MAXN>(key, n, all_and & known, known, (uint32_t)k, cursor, lowest, sm);
}

// The k-th largest of n keys when the bits outside [lowest, cursor] are known
// to be zero in every key (sign-free keys: bit 31; keys of bf16 values: bits
// 0..15), without first reducing the keys to find the window.
template <int NT, int KPT, int MAXN>
__device__ SelectResult block_select_window(const uint32_t (&key)[KPT], int n, int k, int cursor, int lowest,
                                            SelectSmem<MAXN> &sm)
{
    uint32_t known = (cursor == 31) ? 0u : ~((2u << cursor) - 1u);
    known |= (1u << lowest) - 1u;
    return radix_select_from<NT, KPT, MAXN>(key, n, 0u, known, (uint32_t)k, cursor, lowest, sm);
}

// Keeps the lowest `keep` set bits of m.
__device__ __forceinline__ uint32_t lowest_set_bits(uint32_t m, uint32_t keep)
{
    if (keep == 0u) return 0u;
    while ((uint32_t)__popc(m) > keep) m &= ~(0x80000000u >> __clz(m));
    return m;
}

// Writes the selection {key > T} and the need_eq lowest-index keys equal to
// T into sm.bits (words [0, ceil(NT*KPT/32)), every one written).  Lane r
// keeps row r's ballot and one store per lane writes them all.  Ends with a
// barrier.
template <int NT, int KPT, int MAXN>
__device__ void selection_bitmap(const uint32_t (&key)[KPT], int n, SelectResult s, SelectSmem<MAXN> &sm)
{
    static_assert(NT * KPT <= MAXN && KPT <= 64, "rows beyond the bitmap");
    constexpr int W = SelectSmem<MAXN>::W;
    const int lane = threadIdx.x & 63;
    const int row0 = (threadIdx.x >> 6) * 64 * KPT;  // this wave's first index
    const uint32_t T = uniform_u32(s.T), need_eq = uniform_u32(s.need_eq);
    const bool all = need_eq == uniform_u32(s.count_eq);
    // all: key >= T; else key > T here and the equal keys below
    const uint64_t T1 = all ? (uint64_t)T : (uint64_t)T + 1u;
    uint64_t mine = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const uint64_t gt = __ballot((slot_index<KPT>(r) < n) & ((uint64_t)key[r] >= T1));
        mine = (lane == r) ? gt : mine;
    }
    if (lane < KPT) *reinterpret_cast<uint64_t *>(&sm.bits[(row0 >> 5) + 2 * lane]) = mine;
    if (!all) {
        mine = 0;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const uint64_t eq = __ballot((slot_index<KPT>(r) < n) & (key[r] == T));
            mine = (lane == r) ? eq : mine;
        }
        if (lane < KPT) *reinterpret_cast<uint64_t *>(&sm.hist[kPassBins + (row0 >> 5) + 2 * lane]) = mine;
    }
    __syncthreads();
    if (!all) {  // of the keys equal to T, the need_eq first in index order
        constexpr int WPT = (W + NT - 1) / NT;
        const int nw = (n + 31) >> 5;  // words the rows wrote
        const int w0 = threadIdx.x * WPT;
        uint32_t m[WPT], cnt = 0;
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            m[j] = (w0 + j < nw) ? sm.hist[kPassBins + w0 + j] : 0u;
            cnt += (uint32_t)__popc(m[j]);
        }
        uint32_t tot;
        uint32_t before = block_excl_scan<NT>(cnt, sm.scratch, &tot);
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            const uint32_t keep = before < need_eq ? need_eq - before : 0u;
            if (m[j] && keep) sm.bits[w0 + j] |= lowest_set_bits(m[j], keep);
            before += (uint32_t)__popc(m[j]);
        }
        __syncthreads();
    }
}

// Calls emit(i, pos) for every index i < n set in sm.bits, pos being its
// rank in ascending index order.
template <int NT, int MAXN, typename Emit>
__device__ void emit_bitmap(int n, SelectSmem<MAXN> &sm, Emit emit)
{
    constexpr int W = SelectSmem<MAXN>::W;
    constexpr int WPT = (W + NT - 1) / NT;
    const int nw = (n + 31) >> 5;
    const int w0 = threadIdx.x * WPT;
    uint32_t m[WPT], cnt = 0;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int wj = w0 + j;
        m[j] = (wj < nw) ? sm.bits[wj] : 0u;
        if (wj == nw - 1 && (n & 31)) m[j] &= (1u << (n & 31)) - 1u;
        cnt += (uint32_t)__popc(m[j]);
    }
    uint32_t tot;
    uint32_t pos = block_excl_scan<NT>(cnt, sm.scratch, &tot);
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        uint32_t b = m[j];
        while (b) {
            emit(32 * (w0 + j) + (__ffs(b) - 1), pos++);
            b &= b - 1u;
        }
    }
}

__device__ __forceinline__ bool bitmap_test(const uint32_t *bits, int i) { return (bits[i >> 5] >> (i & 31)) & 1u; }

// out[pos] = i for every slot i whose key is >= T, pos its rank in index
// order, for pos < k.  Keys of slots past the end must be 0xFFFFFFFF: as
// int32 they are negative, below every threshold (T < 2^31).  No branch per
// row: a lane that stores nothing, or whose position is >= k, gives the
// store the buffer's end as offset and the range check drops it.
template <int NT, int KPT, int MAXN>
__device__ void emit_at_least(const uint32_t (&key)[KPT], uint32_t T, int32_t *out, uint32_t k,
                              SelectSmem<MAXN> &sm)
{
    const int32_t Ts = (int32_t)T;
    const uint32_t slot0 = (uint32_t)slot_index<KPT>(0);
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) cnt += (uint32_t)__popcll(__ballot((int32_t)key[r] >= Ts));
    uint32_t tot;
    uint32_t pos = uniform_u32(waves_excl_scan<NT>(cnt, sm.scratch, &tot));
    const OutBuf ob(out, k * 4u);
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const bool c = (int32_t)key[r] >= Ts;
        const uint64_t m = __ballot(c);
        const uint32_t off = (pos + lanes_below(m)) * 4u;
        ob.store(c ? off : ob.end, slot0 + (uint32_t)(r * 64));
        pos += (uint32_t)__popcll(m);
    }
}

}  // namespace prox
