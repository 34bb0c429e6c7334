// Internal launch interface between the C-ABI layer (api.hip) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prox {

// Longest input range one proxy workgroup compacts in LDS.
constexpr int kMaxSplitRange = 512;

// Launch shape of the proxy GEMV (K1).
struct ProxyPlan {
    int qbits;      // 8 or 4
    int cpl;        // channels per lane
    int nb;         // tokens held in registers (>= batch)
    int n_cblocks;  // ceil(F / (64 * cpl))
    int R;          // inputs per split (multiple of 128 for int4)
    int S;          // number of input splits
};

// Waves per down-projection workgroup (single token; half for 4-token
// passes) and selected rows each wave holds in flight (256 ranks per
// workgroup).  Measured on 4096 x 14336 bf16 at k = 4301: fewer, longer
// workgroups beat more, shorter ones, whose extra partials lengthen the
// split reduction.
constexpr int kDownWaves = 8;
constexpr int kDownRowsPerWave = 32;

// Launch shape of the down projection (K4).
struct DownPlan {
    int vec;        // columns per lane (16-byte loads)
    int cols;       // columns per workgroup slice = 64 * vec
    int n_slices;   // ceil(d / cols)
    int S;          // channel-rank splits
    int nb;         // tokens per pass
};

// Stage 2 for batches of 2..16 tokens, bf16 activations, on the matrix
// cores (stage2_batch.hip).
struct BatchPlan {
    int n_tiles;  // gate/up tiles of 16 channels
    int n_full;   // gate/up tiles run whole, one workgroup each (a multiple of the CU count)
    int SK;       // input chunks of each other tile
    int KW;       // inputs per chunk (a multiple of 1024)
    int KP;       // k rounded up to 32 (ranks of the s pieces)
    int n_ct;     // down column tiles (128 bytes of a row: 64 bf16 or 128 FP8 columns)
    int S;        // down rank splits
    int kps;      // down K-steps (32 ranks) per split
};

// Single-token Stage 1 in one kernel (stage1_fused.hip).
constexpr int kFusedMaxD = 8192;       // inputs (d_model)
constexpr int kFusedMaxF = 16384;      // channels whose top-k the kernel runs itself (scores in one workgroup)
constexpr int kFusedGemvMaxF = 65520;  // channels it scores (larger d_ff: the top-k is a second launch)
constexpr int kFusedScoreSlot = 511;   // counter of finished channel blocks

struct FusedPlan {
    int n_cblocks;  // ceil(F / channels per workgroup)
    int R;          // inputs per split
    int S;          // number of input splits
};

FusedPlan fused_plan(int qbits, int64_t d, int64_t F);
// Floats of `part` the kernel uses: the split partials (S x 2 x F), then 256
// 16-bit score counts per channel block (the first radix pass of the top-k,
// inside the kernel up to kFusedMaxF channels, else in a second launch).
int64_t fused_part_floats(int qbits, int64_t d, int64_t F);
bool fused_supported(int64_t B, int64_t d, int64_t F, int qbits);
// act: the gate activation (0 silu, 1 gelu tanh form); signal: the
// selection signal (0 |act(g~) u~|, 1 |act(g~)|, 2 |u~|).
// norm_eps >= 0: x is the residual stream h and every workgroup uses
// RMSNorm(h) = h / sqrt(mean(h^2) + norm_eps) in x's dtype, bitwise as
// rmsnorm_kernel computes it; the first workgroup also writes it to xn_out.
hipError_t launch_stage1_fused(int dtype, int qbits, const void *x, int d, int F, int k_in, int k,
                               const uint8_t *codes, const float *scales, float *part, float *score, int32_t *sel,
                               uint32_t *counters, int act, int signal, hipStream_t st, float norm_eps = -1.0f,
                               void *xn_out = nullptr);

hipError_t launch_xselect(int dtype, const void *x, int B, int d, int k_in, float *xh, uint32_t *counters,
                          int n_counters, hipStream_t st, float norm_eps = -1.0f,
                          void *xn_out = nullptr);
hipError_t launch_proxy(const ProxyPlan &pl, const float *xh, int B, int d, int F, const uint8_t *codes,
                        const float *scales, float *part, float *score, uint32_t *counters, int act, int signal,
                        hipStream_t st);
// The exact-state signal: score[j] = sum_b |s[b][j]| over s [B][F], and the
// selected channels' values s_sel[b][r] = s[b][sel[r]].
hipError_t launch_score_from_s(const float *s, int B, int F, float *score, hipStream_t st);
hipError_t launch_gather_s(const float *s, int B, int F, const int32_t *sel, int k, float *s_sel, hipStream_t st);
hipError_t launch_topk(const float *score, int n, int k, int32_t *sel, hipStream_t st);
// The top-k after stage1_fused_kernel's scores, from its channel blocks' score
// counts (blk_cnt: n_blocks x 128 words of 16-bit fields, n_blocks <= 128).
hipError_t launch_topk_counts(const float *score, int n, int k, int32_t *sel, const uint32_t *blk_cnt,
                              int n_blocks, hipStream_t st);

// Stage-2 weights as the kernels read them.  fmt 0: w_gu [F][2][d] and
// w_down_t [F][d] in the activation dtype.  fmt 1: the same layouts in FP8
// E4M3 codes, with fp32 scales per output row: gu_scales [F][2] (gate, up of
// channel j), down_scales [d] (row m of W_down).
struct S2Weights {
    int fmt;
    const void *w_gu;
    const float *gu_scales;
    const void *w_down_t;
    const float *down_scales;
    int act;  // gate activation: 0 silu, 1 gelu (tanh form)
};

// Stage 2 clamps every mask entry into [0, F): a malformed mask gives wrong
// values, never an access outside the weights.
hipError_t launch_gateup(int dtype, const S2Weights &w, const void *x, int B, int d, int F, const int32_t *sel,
                         int k, float *s_sp, int32_t *iota_out, hipStream_t st);
hipError_t launch_down(int dtype, const S2Weights &w, const DownPlan &pl, const float *s_sp, int B, int k,
                       const int32_t *sel, int d, int F, float *part, const void *residual, void *out,
                       uint32_t *counters, hipStream_t st);
// The proxy for batches of 2..16 bf16 tokens with int8 codes, on the matrix
// cores (stage1_batch.hip): scores from xh[B][d] (the kept inputs, zeros
// elsewhere).  part: proxy_batch_splits(d)*B*2*F floats; counters [0, F/128)
// zero on entry and left zero.
int proxy_batch_splits(int d);
hipError_t launch_proxy_batch(const float *xh, int B, int d, int F, const uint8_t *codes, const float *scales,
                              float *part, float *score, uint32_t *counters, int act, int signal, hipStream_t st);
// Stage 2 for batches (stage2_batch.hip).
BatchPlan batch_plan(int d, int k, int B, int fp8);
int batch_max_splits(int d, int F);         // the largest BatchPlan::S over k <= F
size_t batch_gu_part_floats(int d, int F);  // the largest gate/up chunk-sum count over k <= F
// gu_part: (n_tiles - n_full)*SK*512 floats; s_pieces: 3*16*KP bf16; dn_part: S*B*d
// floats; gu_counters: n_tiles words, dn_counters: n_ct words, zero on entry
// and left zero.
hipError_t launch_stage2_batch(const S2Weights &w, const void *x, int B, int d, int F, const int32_t *sel, int k,
                               const BatchPlan &pl, float *gu_part, uint16_t *s_pieces, float *dn_part,
                               const void *residual, void *out, uint32_t *gu_counters, uint32_t *dn_counters,
                               int32_t *iota_out, hipStream_t st);
// Stage 2 for one token in one launch (stage2.hip).  Counter slots:
// [kDownSliceBase, kDownSliceEnd) slice tickets, [kDownPassBase, +511)
// slice-tail counts, [kDownClaimBase, +511) slice-tail group claims, and from
// kS2SyncBase one 128-byte line per split holding its arrival count (gate/up
// workgroups add 1, down workgroups 1 << 16 once past their wait).  Split s
// sits in 4 KB page s % 64, line s / 64: the lines being polled at one time
// are 4 KB apart, so the polls spread over the memory channels instead of
// queueing on one (one packed run of counters slowed every gate/up row on
// that channel about 3x).  kFallbackSlot counts bounded waits that gave up
// (each then completed its work without the awaited data); unlike the others
// it is not reset by the kernels, only by a zero fill of the workspace.
constexpr int kDownSliceBase = 512;
constexpr int kDownSliceEnd = 1023;
constexpr int kDownPassBase = 1024;
constexpr int kDownClaimBase = 1536;
constexpr int kLayerBarrierSlot = 2045;  // the single-launch layer's grid-barrier arrivals
constexpr int kLayerErrorSlot = 2046;    // its grid-barrier waits that gave up (not reset by kernels)
constexpr int kLayerBlockSyncBase = 2048;  // its per-block barriers: arrivals, passes; one pair per 64 words
constexpr int kLayerBlockSyncStride = 64;
constexpr int kFallbackSlot = 2047;
constexpr int kS2SyncBase = 4096;
constexpr int kS2SyncPages = 64;
constexpr int kS2PageWords = 1024;
constexpr int kS2LineWords = 32;
constexpr int kS2MaxSplits = kS2SyncPages * (kS2PageWords / kS2LineWords);
constexpr int kS2SyncWords = kS2SyncPages * kS2PageWords;
__host__ __device__ constexpr int s2_sync_line(int s)
{
    return kS2SyncBase + (s % kS2SyncPages) * kS2PageWords + (s / kS2SyncPages) * kS2LineWords;
}
// Bounded cross-workgroup waits give up after spin_ticks of the 100 MHz
// real-time counter (0: kDefaultSpinTicks, half a second).
constexpr uint64_t kDefaultSpinTicks = 50000000ull;
hipError_t launch_stage2_fused(int dtype, const S2Weights &w, const void *x, int d, int F, const int32_t *sel, int k,
                               float *s_sp, float *part, const void *residual, void *out, uint32_t *counters,
                               int32_t *iota_out, hipStream_t st, uint64_t spin_ticks = 0);
hipError_t launch_fill_out(int dtype, int B, int d, const void *residual, void *out, hipStream_t st);
// Stage 2 for one bf16 token with bf16 or FP8 weights, d_model 4096 or 8192,
// in one launch of G workgroups, one per CU (stage2_rows.hip).  ypart: G * d floats.
// Counter words: the 64-bit arrival count at kRowsArriveSlot and the release
// words at s2_sync_line(kRowsReleaseBase + i), i < G; they hold launch numbers
// (they only grow), so they are not zero between calls; a zero fill restarts
// them.  sel null: channel r at rank r (k == F), written to iota_out if given.
constexpr int kRowsMaxGroups = 256;
constexpr int kRowsMaxChan = 128;      // channels per workgroup
constexpr int kRowsArriveSlot = 3072;  // two words, 8-byte aligned
constexpr int kRowsReleaseBase = 1024; // sync lines 1024.. (the single-token Stage 2 uses < 1024)
bool rows_supported(int64_t d, int64_t F, int64_t k, int G);
hipError_t launch_stage2_rows(const void *x, int d, int F, const int32_t *sel, int k, const S2Weights &w,
                              const void *residual, void *out, int32_t *iota_out, float *ypart, uint32_t *counters,
                              uint64_t spin_ticks, int G, hipStream_t st);
// Workgroups the rows kernel uses on the current device (one per CU, at most
// kRowsMaxGroups), or 0 if a CU cannot hold one of its workgroups.
int rows_groups();

// The whole forward for one bf16 token (bf16 weights, int8 proxy) in one
// launch of G workgroups, one per CU, all resident at once (layer.hip).  G
// <= kLayerMaxGroups sizes the workspace areas: part G*2048 floats, selw
// 1024 words, ypart G*d floats.  Counter slots: the per-block barrier words
// at kLayerBlockSyncBase + kLayerBlockSyncStride * c (c < 16),
// kFusedScoreSlot, kLayerBarrierSlot, kLayerErrorSlot and the release words
// at s2_sync_line(w), w < G.  residual may alias out.
constexpr int kLayerMaxGroups = 256;
bool layer_supported(int64_t B, int64_t d, int64_t F, int64_t k_in, int64_t k, int G);
hipError_t launch_layer(const void *x, int d, int F, int k_in, int k, const uint8_t *codes, const float *qscales,
                        const void *w_gu, const void *w_dt, const void *residual, void *out, int32_t *sel_out,
                        float *part, float *score, uint32_t *selw, float *ypart, uint32_t *counters, int act,
                        int signal, uint64_t spin_ticks, int G, hipStream_t st);
// Workgroups the single-launch layer uses on the current device (one per
// CU, at most kLayerMaxGroups), or 0 if it cannot run there (a CU does not
// hold one of its 1024-thread workgroups).
int layer_groups();
hipError_t launch_zero_u32(uint32_t *p, int n, hipStream_t st);
// Stream-read probe (probe.hip): reads bytes/16 16-byte vectors, XORs every
// 32-bit word read into *sink (device-scope atomics).
hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st);

hipError_t launch_pack(int dtype, const void *w_gate, const void *w_up, const void *w_down, int d, int F,
                       void *w_gu, void *w_down_t, hipStream_t st);
hipError_t launch_pack_fp8(int dtype, const void *w_gate, const void *w_up, const void *w_down, int d, int F,
                           uint8_t *w_gu8, float *gu_scales, uint8_t *w_down_t8, float *down_scales, hipStream_t st);
// proxy quantization from w_gu in the activation dtype (wfmt 0) or FP8 (wfmt 1, with gu_scales)
hipError_t launch_quantize(int dtype, int wfmt, const void *w_gu, const float *gu_scales, int qbits, int d, int F,
                           uint8_t *codes, float *scales, hipStream_t st);
hipError_t launch_rmsnorm(int dtype, const void *h, int B, int d, float eps, void *out, hipStream_t st);

}  // namespace prox
