// C ABI of the Prox library: argument validation, counts, workspace layout
// and the launch sequence of the two stages.  See include/prox.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/prox.h"
#include "kernels.h"

using namespace prox;

// The workspace of prox_ffn_forward_noalloc: one copy per device, held until
// the process ends.  Host code never uses this name as an address (on the
// host it stands for the symbol, not for device memory): the device address
// comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[PROX_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxBatch = 16;
constexpr int kMaxBatchInt4 = 4;
// The workspace starts with counters that must be zero between calls:
// [0,511) proxy channel blocks, 511 the single-token Stage 1's score ticket,
// [512,1023) down slices, [1024,1535) the single-token Stage 2's finished
// slice tails, [1536,2047) its slice-tail claims, 2045 and [2048,3072) the
// single-launch layer's barriers, 2046 its failed waits and 2047 the count
// of bounded waits that gave up (neither reset by a call), then from 4096
// the single-token Stage 2's per-split lines (64 pages of 4 KB).  Each other
// word is reset by the last workgroup to use it, except the rows Stage 2's
// arrival count (3072, 64 bits) and release lines (lines 1024.. of the
// per-split pages), which hold launch numbers.
constexpr int kCounters = kS2SyncBase + kS2SyncWords;
constexpr int kZeroWords = kCounters;
// The channel-block and slice ticket words: the batched Stage 1 clears them
// again on entry, inside its first kernel.
constexpr int kTicketWords = kDownSliceEnd;
constexpr int kTargetProxyBlocks = 1024;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// An enum the caller passed (a field or a parameter) read as the int it is
// in the C interface: a caller may hand over any int, and loading a C++
// enum object holding a value outside the enumeration is undefined.
template <typename E>
int enum_int(const E &e)
{
    static_assert(sizeof(E) == sizeof(int), "C enums are ints");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

prox_status hip_status(hipError_t e) { return e == hipSuccess ? PROX_OK : PROX_ERR_HIP; }

bool bad_ptr(const void *p) { return p == nullptr || ((uintptr_t)p & 15u) != 0; }
bool bad_ptr_opt(const void *p) { return p != nullptr && ((uintptr_t)p & 15u) != 0; }

int elem_bytes(int t) { return t == PROX_F32 ? 4 : 2; }

prox_status check_shape(int64_t d, int64_t F)
{
    if (d < 8 || d > 16384 || F < 16 || F > 65520) return PROX_ERR_UNSUPPORTED;
    if (d % 8 != 0 || F % 16 != 0) return PROX_ERR_UNSUPPORTED;
    return PROX_OK;
}

prox_status check_mode_shape(int64_t d, int64_t F, int mode)
{
    prox_status s = check_shape(d, F);
    if (s != PROX_OK) return s;
    if (mode != PROX_Q_INT8_ROW && mode != PROX_Q_INT4_G128) return PROX_ERR_UNSUPPORTED;
    if (mode == PROX_Q_INT4_G128 && d % 128 != 0) return PROX_ERR_UNSUPPORTED;
    return PROX_OK;
}

prox_status check_weights(const prox_weights *w)
{
    if (!w) return PROX_ERR_INVALID_ARG;
    if (enum_int(w->dtype) != PROX_F32 && enum_int(w->dtype) != PROX_BF16) return PROX_ERR_UNSUPPORTED;
    prox_status s = check_shape(w->d_model, w->d_ff);
    if (s != PROX_OK) return s;
    if (bad_ptr(w->w_gu) || bad_ptr(w->w_down_t)) return PROX_ERR_INVALID_ARG;
    if (enum_int(w->wformat) == PROX_W_FP8_E4M3) {
        if (w->d_model % 16 != 0) return PROX_ERR_UNSUPPORTED;
        if (bad_ptr(w->gu_scales) || bad_ptr(w->down_scales)) return PROX_ERR_INVALID_ARG;
    } else if (enum_int(w->wformat) != PROX_W_NATIVE) {
        return PROX_ERR_UNSUPPORTED;
    }
    return PROX_OK;
}

// Forward options (prox_options, validated): gate activation and selection signal.
struct Opts {
    int act = PROX_ACT_SILU;
    int signal = PROX_SIGNAL_S;
    uint64_t spin_ticks = 0;  // 0: the kernels' default bound
    int flags = 0;
};

prox_status check_options(const prox_options *o, Opts *out)
{
    if (!o) return PROX_OK;
    if (enum_int(o->activation) != PROX_ACT_SILU && enum_int(o->activation) != PROX_ACT_GELU_TANH) return PROX_ERR_UNSUPPORTED;
    if (enum_int(o->signal) < PROX_SIGNAL_S || enum_int(o->signal) > PROX_SIGNAL_EXACT_S) return PROX_ERR_UNSUPPORTED;
    if (o->wait_limit_ticks < 0) return PROX_ERR_INVALID_ARG;
    if (o->flags & ~PROX_FLAG_SINGLE_LAUNCH) return PROX_ERR_UNSUPPORTED;
    out->act = enum_int(o->activation);
    out->signal = enum_int(o->signal);
    out->spin_ticks = (uint64_t)o->wait_limit_ticks;
    out->flags = o->flags;
    return PROX_OK;
}

S2Weights s2_weights(const prox_weights *w, int act)
{
    const bool fp8 = enum_int(w->wformat) == PROX_W_FP8_E4M3;
    return S2Weights{fp8 ? 1 : 0, w->w_gu, fp8 ? w->gu_scales : nullptr, w->w_down_t,
                     fp8 ? w->down_scales : nullptr, act};
}

prox_status check_proxy(const prox_proxy *p, const prox_weights *w)
{
    if (!p) return PROX_ERR_INVALID_ARG;
    if (p->d_model != w->d_model || p->d_ff != w->d_ff) return PROX_ERR_INVALID_ARG;
    prox_status s = check_mode_shape(p->d_model, p->d_ff, enum_int(p->mode));
    if (s != PROX_OK) return s;
    if (bad_ptr(p->codes) || bad_ptr(p->scales)) return PROX_ERR_INVALID_ARG;
    return PROX_OK;
}

prox_status check_batch(int64_t B, int mode)
{
    if (B < 1) return PROX_ERR_INVALID_ARG;
    if (B > kMaxBatch) return PROX_ERR_UNSUPPORTED;
    if (mode == PROX_Q_INT4_G128 && B > kMaxBatchInt4) return PROX_ERR_UNSUPPORTED;
    return PROX_OK;
}

prox_status counts(int64_t d, int64_t F, float keep, float sp, int64_t *k_in, int64_t *k)
{
    if (isnan(keep) || !(keep > 0.0f) || keep > 1.0f) return PROX_ERR_INVALID_ARG;
    if (isnan(sp) || sp < 0.0f || sp > 1.0f) return PROX_ERR_INVALID_ARG;
    double a = floor((double)keep * (double)d + 0.5);
    if (a < 1.0) a = 1.0;
    if (a > (double)d) a = (double)d;
    double b = floor((1.0 - (double)sp) * (double)F + 0.5);
    if (b < 0.0) b = 0.0;
    if (b > (double)F) b = (double)F;
    *k_in = (int64_t)a;
    *k = (int64_t)b;
    return PROX_OK;
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

ProxyPlan proxy_plan(int64_t d, int64_t F, int64_t B, int mode)
{
    ProxyPlan p;
    p.qbits = mode == PROX_Q_INT4_G128 ? 4 : 8;
    p.cpl = p.qbits == 8 ? 4 : 8;  // one 32-bit code word per lane per half
    if (p.qbits == 8)
        p.nb = B == 1 ? 1 : (B <= 4 ? 4 : 16);
    else
        p.nb = B == 1 ? 1 : 4;
    p.n_cblocks = ceil_div(F, 64 * p.cpl);
    const int gran = p.qbits == 4 ? 128 : 32;
    const int s_min = ceil_div(d, kMaxSplitRange);
    int s = ceil_div(kTargetProxyBlocks, p.n_cblocks);
    const int s_max = ceil_div(d, 128);
    if (s > s_max) s = s_max;
    if (s < s_min) s = s_min;
    int R = ceil_div(ceil_div(d, s), gran) * gran;
    if (R > kMaxSplitRange) R = kMaxSplitRange;
    p.R = R;
    p.S = ceil_div(d, R);
    return p;
}

DownPlan down_plan(int64_t d, int64_t k, int64_t B, const prox_weights *w)
{
    DownPlan p;
    p.vec = enum_int(w->wformat) == PROX_W_FP8_E4M3 ? 8 : 16 / elem_bytes(enum_int(w->dtype));  // FP8: 8-byte loads
    p.cols = 64 * p.vec;
    p.n_slices = ceil_div(d, p.cols);
    p.S = ceil_div(k > 0 ? k : 1, kDownRowsPerWave * kDownWaves);
    p.nb = B >= 4 ? 4 : (int)B;
    return p;
}

struct Workspace {
    uint32_t *counters;
    float *lk_part;   // single-launch layer: proxy block partials
    uint32_t *lk_selw; // single-launch layer: the published selection
    float *ypart;     // one token's per-workgroup partial outputs (rows Stage 2, single-launch layer)
    float *xh;
    float *proxy_part;
    float *score;
    int32_t *sel;
    float *s_sp;
    float *down_part;
    float *gu_part;       // batches: gate/up chunk sums
    uint16_t *s_pieces;   // batches: s as three bf16 pieces
    float *bdn_part;      // batches: down split partials
    size_t bytes;
};

// Offsets depend only on (d, F, B, mode); the down partials are sized for the
// largest split count any k can use (the bf16 slicing, which has fewer slices).
Workspace layout(int64_t d, int64_t F, int64_t B, int mode, void *base)
{
    const ProxyPlan pp = proxy_plan(d, F, B, mode);
    size_t part_rows = (size_t)pp.S * B;
    if ((size_t)proxy_batch_splits((int)d) * B > part_rows) part_rows = (size_t)proxy_batch_splits((int)d) * B;
    size_t part_floats = part_rows * 2 * F;
    if (fused_supported(B, d, F, mode == PROX_Q_INT4_G128 ? 4 : 8)) {
        const size_t f = (size_t)fused_part_floats(mode == PROX_Q_INT4_G128 ? 4 : 8, d, F);
        if (f > part_floats) part_floats = f;
    }
    const int down_s_max = 2 * ceil_div(F, kDownRowsPerWave * kDownWaves);  // 4-token passes: half-size workgroups
    size_t off = 0;
    Workspace w;
    char *b = (char *)base;
    auto take = [&](size_t n) { char *p = b ? b + off : nullptr; off += align256(n); return p; };
    w.counters = (uint32_t *)take(sizeof(uint32_t) * kZeroWords);
    w.xh = (float *)take(sizeof(float) * B * d);
    w.proxy_part = (float *)take(sizeof(float) * part_floats);
    w.score = (float *)take(sizeof(float) * F);
    w.sel = (int32_t *)take(sizeof(int32_t) * F);
    w.s_sp = (float *)take(sizeof(float) * B * F);
    w.down_part = (float *)take(sizeof(float) * (size_t)down_s_max * 4 * d);
    if (B > 1) {  // the matrix-core Stage 2 (bf16 activations)
        w.gu_part = (float *)take(sizeof(float) * batch_gu_part_floats((int)d, (int)F));
        w.s_pieces = (uint16_t *)take(sizeof(uint16_t) * 3 * 16 * (size_t)(ceil_div(F, 32) * 32));
        w.bdn_part = (float *)take(sizeof(float) * (size_t)batch_max_splits((int)d, (int)F) * B * d);
    } else {
        w.gu_part = nullptr;
        w.s_pieces = nullptr;
        w.bdn_part = nullptr;
    }
    w.lk_part = w.ypart = nullptr;
    w.lk_selw = nullptr;
    if (B == 1 && (d == 4096 || d == 8192)) {  // the rows Stage 2 and the single-launch layer
        w.ypart = (float *)take(sizeof(float) * (size_t)kRowsMaxGroups * d);
        if (F <= kFusedMaxF) {
            w.lk_part = (float *)take(sizeof(float) * (size_t)kLayerMaxGroups * 2048);
            w.lk_selw = (uint32_t *)take(sizeof(uint32_t) * 1024);  // the published selection
        }
    }
    w.bytes = off;
    return w;
}

// The single-launch layer serves bf16 tokens with bf16 weights and an int8
// proxy where the device runs it (layer_groups) and the shape fits.
int layer_path(int64_t B, const prox_weights *w, const prox_proxy *p, int64_t k_in, int64_t k, const Opts &o)
{
    if (!(o.flags & PROX_FLAG_SINGLE_LAUNCH)) return 0;
    if (B != 1 || enum_int(w->dtype) != PROX_BF16 || enum_int(w->wformat) != PROX_W_NATIVE || !p || enum_int(p->mode) != PROX_Q_INT8_ROW) return 0;
    if (o.signal == PROX_SIGNAL_EXACT_S) return 0;
    const int G = layer_groups();
    return layer_supported(B, w->d_model, w->d_ff, k_in, k, G) ? G : 0;
}

prox_status run_layer(const void *x, const prox_weights *w, const prox_proxy *p, int64_t k_in, int64_t k,
                      const void *residual, void *out, int32_t *sel_out, const Workspace &ws, hipStream_t st,
                      const Opts &o, int G)
{
    return hip_status(launch_layer(x, (int)w->d_model, (int)w->d_ff, (int)k_in, (int)k, (const uint8_t *)p->codes,
                                   (const float *)p->scales, w->w_gu, w->w_down_t, residual, out, sel_out, ws.lk_part,
                                   ws.score, ws.lk_selw, ws.ypart, ws.counters, o.act, o.signal, o.spin_ticks,
                                   G, st));
}


#define TRY_HIP(expr)                                           \
    do {                                                        \
        hipError_t e_ = (expr);                                 \
        if (e_ != hipSuccess) return PROX_ERR_HIP;              \
    } while (0)

// Records ev[i] on the stream when timing events were supplied.
hipError_t mark(hipEvent_t *ev, int i, hipStream_t st) { return ev ? hipEventRecord(ev[i], st) : hipSuccess; }

// Stage 1 into `sel` (k entries), scores into `score`.
// norm_eps >= 0: x is h; Stage 1 uses RMSNorm(h) and writes it to xn (see
// launch_stage1_fused and launch_xselect).
prox_status run_stage1(const void *x, int64_t B, const prox_weights *w, const prox_proxy *p, int64_t k_in,
                       int64_t k, int32_t *sel, float *score, const Workspace &ws, hipStream_t st,
                       hipEvent_t *ev = nullptr, const Opts &o = Opts(), float norm_eps = -1.0f,
                       void *xn = nullptr)
{
    const int64_t d = w->d_model, F = w->d_ff;
    const int dt = enum_int(w->dtype) == PROX_F32 ? 0 : 1;
    if (fused_supported(B, d, F, enum_int(p->mode) == PROX_Q_INT4_G128 ? 4 : 8)) {  // its counters are zero on entry
        TRY_HIP(mark(ev, 0, st));
        TRY_HIP(launch_stage1_fused(dt, enum_int(p->mode) == PROX_Q_INT4_G128 ? 4 : 8, x, (int)d, (int)F, (int)k_in, (int)k,
                                    (const uint8_t *)p->codes, (const float *)p->scales, ws.proxy_part, score, sel,
                                    ws.counters, o.act, o.signal, st, norm_eps, xn));
        TRY_HIP(mark(ev, 1, st));
        return hip_status(mark(ev, 2, st));
    }
    const ProxyPlan pp = proxy_plan(d, F, B, enum_int(p->mode));
    TRY_HIP(mark(ev, 0, st));
    TRY_HIP(launch_xselect(dt, x, (int)B, (int)d, (int)k_in, ws.xh, ws.counters,
                           kTicketWords, st, norm_eps, xn));
    TRY_HIP(mark(ev, 1, st));
    // bf16 batches above 4 tokens, int8 codes: the matrix cores (at 4 tokens
    // the vector-ALU kernel is faster, 32.6 against 35.3 us at 4096 x 14336)
    if (dt == 1 && enum_int(p->mode) == PROX_Q_INT8_ROW && B > 4)
        TRY_HIP(launch_proxy_batch(ws.xh, (int)B, (int)d, (int)F, (const uint8_t *)p->codes,
                                   (const float *)p->scales, ws.proxy_part, score, ws.counters, o.act, o.signal, st));
    else
        TRY_HIP(launch_proxy(pp, ws.xh, (int)B, (int)d, (int)F, (const uint8_t *)p->codes,
                             (const float *)p->scales, ws.proxy_part, score, ws.counters, o.act, o.signal, st));
    TRY_HIP(mark(ev, 2, st));
    if (k > 0) TRY_HIP(launch_topk(score, (int)F, (int)k, sel, st));
    return PROX_OK;
}

// Stage 2 on `sel` (nullptr = every channel).  Counters must be zero.
prox_status run_stage2(const void *x, int64_t B, const prox_weights *w, const int32_t *sel, int64_t k,
                       const void *residual, void *out, int32_t *iota_out, const Workspace &ws, hipStream_t st,
                       hipEvent_t *ev = nullptr, const Opts &o = Opts())
{
    const int dt = enum_int(w->dtype) == PROX_F32 ? 0 : 1;
    const int64_t d = w->d_model;
    const S2Weights sw = s2_weights(w, o.act);
    TRY_HIP(mark(ev, 3, st));
    if (k == 0) {
        TRY_HIP(launch_fill_out(dt, (int)B, (int)d, residual, out, st));
        TRY_HIP(mark(ev, 4, st));
        return hip_status(mark(ev, 5, st));
    }
    if (B == 1 && dt == 1 && ws.ypart) {  // bf16 token: one workgroup per CU streams whole channels
        const int G = rows_groups();
        if (G && rows_supported(d, w->d_ff, k, G)) {
            TRY_HIP(launch_stage2_rows(x, (int)d, (int)w->d_ff, sel, (int)k, sw, residual, out, iota_out, ws.ypart,
                                       ws.counters, o.spin_ticks, G, st));
            TRY_HIP(mark(ev, 4, st));
            return hip_status(mark(ev, 5, st));
        }
    }
    if (B == 1) {  // one launch: the down projection starts while gate/up drains
        TRY_HIP(launch_stage2_fused(dt, sw, x, (int)d, (int)w->d_ff, sel, (int)k, ws.s_sp, ws.down_part, residual,
                                    out, ws.counters, iota_out, st, o.spin_ticks));
        TRY_HIP(mark(ev, 4, st));
        return hip_status(mark(ev, 5, st));
    }
    if (dt == 1) {  // bf16 activations: gate/up and down on the matrix cores
        const BatchPlan bp = batch_plan((int)d, (int)k, (int)B, sw.fmt);
        TRY_HIP(launch_stage2_batch(sw, x, (int)B, (int)d, (int)w->d_ff, sel, (int)k, bp, ws.gu_part, ws.s_pieces,
                                    ws.bdn_part, residual, out, ws.counters + kS2SyncBase,
                                    ws.counters + kDownSliceBase, iota_out, st));
        TRY_HIP(mark(ev, 4, st));
        return hip_status(mark(ev, 5, st));
    }
    TRY_HIP(launch_gateup(dt, sw, x, (int)B, (int)d, (int)w->d_ff, sel, (int)k, ws.s_sp, iota_out, st));
    TRY_HIP(mark(ev, 4, st));
    const DownPlan dp = down_plan(d, k, B, w);
    TRY_HIP(launch_down(dt, sw, dp, ws.s_sp, (int)B, (int)k, sel, (int)d, (int)w->d_ff, ws.down_part, residual, out,
                        ws.counters + kDownSliceBase, st));
    return hip_status(mark(ev, 5, st));
}

// The exact-state signal (no proxy, 0 < k < F): exact gate/up of every
// channel with the dense x, score_j = sum_b |s_bj|, the top-k, then the down
// projection on the selected channels' s values (gathered in rank order
// into the proxy-partials area, unused on this path).
prox_status run_exact_signal(const void *x, int64_t B, const prox_weights *w, int64_t k, int32_t *sel,
                             const void *residual, void *out, const Workspace &ws, hipStream_t st, const Opts &o)
{
    const int dt = enum_int(w->dtype) == PROX_F32 ? 0 : 1;
    const int64_t d = w->d_model, F = w->d_ff;
    const S2Weights sw = s2_weights(w, o.act);
    TRY_HIP(launch_gateup(dt, sw, x, (int)B, (int)d, (int)F, nullptr, (int)F, ws.s_sp, nullptr, st));
    TRY_HIP(launch_score_from_s(ws.s_sp, (int)B, (int)F, ws.score, st));
    TRY_HIP(launch_topk(ws.score, (int)F, (int)k, sel, st));
    TRY_HIP(launch_gather_s(ws.s_sp, (int)B, (int)F, sel, (int)k, ws.proxy_part, st));
    const DownPlan dp = down_plan(d, k, B, w);
    return hip_status(launch_down(dt, sw, dp, ws.proxy_part, (int)B, (int)k, sel, (int)d, (int)F, ws.down_part,
                                  residual, out, ws.counters + kDownSliceBase, st));
}

prox_status forward_impl(const void *x, int64_t B, const prox_weights *w, const prox_proxy *p, float keep,
                         float sp, const void *residual, void *out, int32_t *sel_out, void *workspace,
                         size_t ws_bytes, hipStream_t st, hipEvent_t *ev = nullptr,
                         const prox_options *opt = nullptr)
{
    Opts o;
    prox_status s = check_options(opt, &o);
    if (s != PROX_OK) return s;
    if (o.signal == PROX_SIGNAL_EXACT_S && ev) return PROX_ERR_UNSUPPORTED;
    s = check_weights(w);
    if (s != PROX_OK) return s;
    const bool exact = o.signal == PROX_SIGNAL_EXACT_S;  // no proxy is read
    const int mode = exact ? (p ? (int)enum_int(p->mode) : (int)PROX_Q_INT8_ROW) : -1;
    if (!exact || p) {
        s = check_proxy(p, w);
        if (s != PROX_OK) return s;
    }
    s = check_batch(B, exact ? mode : enum_int(p->mode));
    if (s != PROX_OK) return s;
    if (bad_ptr(x) || bad_ptr(out) || bad_ptr_opt(sel_out) || bad_ptr_opt(residual) || bad_ptr(workspace))
        return PROX_ERR_INVALID_ARG;
    if (x == out || x == residual) return PROX_ERR_INVALID_ARG;
    int64_t k_in, k;
    s = counts(w->d_model, w->d_ff, keep, sp, &k_in, &k);
    if (s != PROX_OK) return s;
    const Workspace ws = layout(w->d_model, w->d_ff, B, exact ? mode : enum_int(p->mode), workspace);
    if (ws_bytes < ws.bytes) return PROX_ERR_WORKSPACE;
    const int64_t F = w->d_ff;
    if (k == 0 || k == F) {  // no Stage 1
        TRY_HIP(mark(ev, 0, st));
        TRY_HIP(mark(ev, 1, st));
        TRY_HIP(mark(ev, 2, st));
        return run_stage2(x, B, w, nullptr, k, residual, out, k ? sel_out : nullptr, ws, st, ev, o);
    }
    int32_t *sel = sel_out ? sel_out : ws.sel;
    if (exact) return run_exact_signal(x, B, w, k, sel, residual, out, ws, st, o);
    if (const int G = layer_path(B, w, p, k_in, k, o)) {  // both stages in one launch
        TRY_HIP(mark(ev, 0, st));
        s = run_layer(x, w, p, k_in, k, residual, out, sel_out, ws, st, o, G);
        if (s != PROX_OK) return s;
        for (int i = 1; i < 6; ++i) TRY_HIP(mark(ev, i, st));
        return PROX_OK;
    }
    s = run_stage1(x, B, w, p, k_in, k, sel, ws.score, ws, st, ev, o);
    if (s != PROX_OK) return s;
    return run_stage2(x, B, w, sel, k, residual, out, nullptr, ws, st, ev, o);
}

// The device address of `scratch` on the current device, its counters
// cleared on the stream the first time (after that every call leaves them
// at zero).  Thread-safe; the table holds one address per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

prox_status static_scratch(hipStream_t st, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PROX_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PROX_ERR_HIP;
        TRY_HIP(launch_zero_u32((uint32_t *)ptr, kZeroWords, st));  // a kernel: capturable
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PROX_OK;
}

}  // namespace

extern "C" {

const char *prox_status_string(int status)
{
    switch (status) {
    case PROX_OK: return "PROX_OK";
    case PROX_ERR_INVALID_ARG: return "PROX_ERR_INVALID_ARG: invalid argument";
    case PROX_ERR_UNSUPPORTED: return "PROX_ERR_UNSUPPORTED: unsupported shape, dtype, mode or batch";
    case PROX_ERR_WORKSPACE: return "PROX_ERR_WORKSPACE: workspace too small";
    case PROX_ERR_HIP: return "PROX_ERR_HIP: HIP launch failed";
    case PROX_ERR_SCRATCH_LIMIT:
        return "PROX_ERR_SCRATCH_LIMIT: the layer's workspace exceeds PROX_STATIC_SCRATCH_BYTES (use a workspace)";
    default: return "unknown prox status";
    }
}

const char *prox_version(void) { return "prox-gfx950 0.2"; }

prox_status prox_counts(int64_t d, int64_t F, float keep, float sp, int64_t *k_in, int64_t *k)
{
    if (!k_in || !k) return PROX_ERR_INVALID_ARG;
    prox_status s = check_shape(d, F);
    if (s != PROX_OK) return s;
    return counts(d, F, keep, sp, k_in, k);
}

prox_status prox_effective_sparsity(const prox_cost_model *m, double keep, double sp, double *effective)
{
    if (!m || !effective || !(m->dense_us > 0.0)) return PROX_ERR_INVALID_ARG;
    if (!(keep >= 0.0 && keep <= 1.0) || !(sp >= 0.0 && sp <= 1.0)) return PROX_ERR_INVALID_ARG;
    const double t = m->stage1_fixed_us + m->stage1_per_keep_us * keep + m->stage2_fixed_us +
                     m->stage2_per_kept_us * (1.0 - sp);
    *effective = 1.0 - t / m->dense_us;
    return PROX_OK;
}

prox_status prox_allocate_sparsity(const prox_cost_model *m, double target, double anchor, double min_keep,
                                   double *keep_out, double *sp_out)
{
    if (!m || !keep_out || !sp_out) return PROX_ERR_INVALID_ARG;
    const double a1 = m->stage1_fixed_us, b1 = m->stage1_per_keep_us;
    const double a2 = m->stage2_fixed_us, b2 = m->stage2_per_kept_us;
    if (!(a1 >= 0.0 && b1 >= 0.0 && a2 >= 0.0 && b2 > 0.0 && m->dense_us > 0.0)) return PROX_ERR_INVALID_ARG;
    if (!(anchor >= 0.0 && anchor <= 1.0) || !(min_keep > 0.0 && min_keep <= 1.0) || !(target < 1.0))
        return PROX_ERR_INVALID_ARG;
    const double budget = (1.0 - target) * m->dense_us;  // the time the layer may take
    double keep = 1.0;
    if (b1 > 0.0) {
        // the anchor held: Stage 1 gets what Stage 2 at the anchor leaves
        keep = (budget - a1 - a2 - b2 * (1.0 - anchor)) / b1;
        if (keep >= min_keep && keep <= 1.0) {
            *keep_out = keep;
            *sp_out = anchor;
            return PROX_OK;
        }
        keep = keep > 1.0 ? 1.0 : min_keep;
    }
    // keep at its bound: Stage 2 gets the rest
    const double kappa = (budget - a1 - b1 * keep - a2) / b2;
    if (kappa < 0.0) return PROX_ERR_UNSUPPORTED;
    *keep_out = keep;
    *sp_out = 1.0 - (kappa < 1.0 ? kappa : 1.0);
    return PROX_OK;
}

prox_status prox_pack_weights(const void *w_gate, const void *w_up, const void *w_down, int64_t d, int64_t F,
                              prox_dtype dtype, void *w_gu_out, void *w_down_t_out, hipStream_t stream)
{
    const int dtype_i = enum_int(dtype);
    if (dtype_i != PROX_F32 && dtype_i != PROX_BF16) return PROX_ERR_UNSUPPORTED;
    prox_status s = check_shape(d, F);
    if (s != PROX_OK) return s;
    if (bad_ptr(w_gate) || bad_ptr(w_up) || bad_ptr(w_down) || bad_ptr(w_gu_out) || bad_ptr(w_down_t_out))
        return PROX_ERR_INVALID_ARG;
    return hip_status(launch_pack(dtype_i == PROX_F32 ? 0 : 1, w_gate, w_up, w_down, (int)d, (int)F, w_gu_out,
                                  w_down_t_out, stream));
}

prox_status prox_pack_weights_fp8(const void *w_gate, const void *w_up, const void *w_down, int64_t d, int64_t F,
                                  prox_dtype dtype, void *w_gu_out, float *gu_scales_out, void *w_down_t_out,
                                  float *down_scales_out, hipStream_t stream)
{
    const int dtype_i = enum_int(dtype);
    if (dtype_i != PROX_F32 && dtype_i != PROX_BF16) return PROX_ERR_UNSUPPORTED;
    prox_status s = check_shape(d, F);
    if (s != PROX_OK) return s;
    if (d % 16 != 0) return PROX_ERR_UNSUPPORTED;
    if (bad_ptr(w_gate) || bad_ptr(w_up) || bad_ptr(w_down) || bad_ptr(w_gu_out) || bad_ptr(gu_scales_out) ||
        bad_ptr(w_down_t_out) || bad_ptr(down_scales_out))
        return PROX_ERR_INVALID_ARG;
    return hip_status(launch_pack_fp8(dtype_i == PROX_F32 ? 0 : 1, w_gate, w_up, w_down, (int)d, (int)F,
                                      (uint8_t *)w_gu_out, gu_scales_out, (uint8_t *)w_down_t_out, down_scales_out,
                                      stream));
}

prox_status prox_proxy_sizes(int64_t d, int64_t F, prox_qmode mode, size_t *codes_bytes, size_t *scales_bytes)
{
    const int mode_i = enum_int(mode);
    if (!codes_bytes || !scales_bytes) return PROX_ERR_INVALID_ARG;
    prox_status s = check_mode_shape(d, F, mode_i);
    if (s != PROX_OK) return s;
    if (mode_i == PROX_Q_INT8_ROW) {
        *codes_bytes = (size_t)d * 2 * F;
        *scales_bytes = sizeof(float) * 2 * F;
    } else {
        *codes_bytes = (size_t)d * F;
        *scales_bytes = sizeof(float) * (d / 128) * 2 * F;
    }
    return PROX_OK;
}

prox_status prox_quantize_proxy(const prox_weights *w, prox_qmode mode, void *codes, void *scales,
                                hipStream_t stream)
{
    const int mode_i = enum_int(mode);
    prox_status s = check_weights(w);
    if (s != PROX_OK) return s;
    s = check_mode_shape(w->d_model, w->d_ff, mode_i);
    if (s != PROX_OK) return s;
    if (bad_ptr(codes) || bad_ptr(scales)) return PROX_ERR_INVALID_ARG;
    return hip_status(launch_quantize(enum_int(w->dtype) == PROX_F32 ? 0 : 1, enum_int(w->wformat) == PROX_W_FP8_E4M3 ? 1 : 0, w->w_gu,
                                      w->gu_scales, mode_i == PROX_Q_INT4_G128 ? 4 : 8, (int)w->d_model, (int)w->d_ff,
                                      (uint8_t *)codes, (float *)scales, stream));
}

prox_status prox_workspace_size(int64_t d, int64_t F, int64_t B, prox_qmode mode, size_t *bytes)
{
    const int mode_i = enum_int(mode);
    if (!bytes) return PROX_ERR_INVALID_ARG;
    prox_status s = check_mode_shape(d, F, mode_i);
    if (s != PROX_OK) return s;
    s = check_batch(B, mode_i);
    if (s != PROX_OK) return s;
    *bytes = layout(d, F, B, mode_i, nullptr).bytes;
    return PROX_OK;
}

prox_status prox_workspace_init(void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (bad_ptr(workspace)) return PROX_ERR_INVALID_ARG;
    if (workspace_bytes < sizeof(uint32_t) * kZeroWords) return PROX_ERR_WORKSPACE;
    return hip_status(launch_zero_u32((uint32_t *)workspace, kZeroWords, stream));
}

prox_status prox_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (bad_ptr(buf) || !sink || ((uintptr_t)sink & 3u)) return PROX_ERR_INVALID_ARG;
    if (bytes == 0 || bytes % 16 != 0) return PROX_ERR_INVALID_ARG;
    return hip_status(launch_read_probe(buf, bytes, sink, stream));
}

prox_status prox_workspace_check(const void *workspace, size_t workspace_bytes, uint32_t *fallbacks,
                                 hipStream_t stream)
{
    if (bad_ptr(workspace) || !fallbacks) return PROX_ERR_INVALID_ARG;
    if (workspace_bytes < sizeof(uint32_t) * kZeroWords) return PROX_ERR_WORKSPACE;
    uint32_t *h = (uint32_t *)malloc(sizeof(uint32_t) * kZeroWords);  // host memory
    if (!h) return PROX_ERR_HIP;
    hipError_t e = hipMemcpyAsync(h, workspace, sizeof(uint32_t) * kZeroWords, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        free(h);
        return PROX_ERR_HIP;
    }
    // the rows Stage 2's words hold launch numbers: its arrival count must be
    // a whole number of launches
    bool clean = true;
    for (int i = 0; i < kRowsMaxGroups; ++i) h[s2_sync_line(kRowsReleaseBase + i)] = 0u;
    const uint64_t arrivals = (uint64_t)h[kRowsArriveSlot] | ((uint64_t)h[kRowsArriveSlot + 1] << 32);
    h[kRowsArriveSlot] = h[kRowsArriveSlot + 1] = 0u;
    const int G = arrivals ? rows_groups() : 0;
    if (arrivals && (G == 0 || arrivals % (uint64_t)G != 0)) clean = false;
    for (int i = 0; i < kZeroWords; ++i)
        if (i != kFallbackSlot && i != kLayerErrorSlot && h[i] != 0u) clean = false;
    *fallbacks = h[kFallbackSlot];
    const bool failed = h[kLayerErrorSlot] != 0u;
    free(h);
    if (failed) return PROX_ERR_HIP;
    return clean ? PROX_OK : PROX_ERR_WORKSPACE;
}

prox_status prox_ffn_forward(const void *x, int64_t batch, const prox_weights *w, const prox_proxy *p,
                             float input_keep, float ffn_sparsity, void *out, int32_t *sel_idx_out,
                             void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return forward_impl(x, batch, w, p, input_keep, ffn_sparsity, nullptr, out, sel_idx_out, workspace,
                        workspace_bytes, stream);
}

prox_status prox_ffn_forward_residual(const void *x, int64_t batch, const prox_weights *w, const prox_proxy *p,
                                      float input_keep, float ffn_sparsity, const void *residual, void *out,
                                      int32_t *sel_idx_out, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream)
{
    if (bad_ptr(residual)) return PROX_ERR_INVALID_ARG;
    return forward_impl(x, batch, w, p, input_keep, ffn_sparsity, residual, out, sel_idx_out, workspace,
                        workspace_bytes, stream);
}

prox_status prox_ffn_forward_ex(const void *x, int64_t batch, const prox_weights *w, const prox_proxy *p,
                                float input_keep, float ffn_sparsity, const prox_options *opt, const void *residual,
                                void *out, int32_t *sel_idx_out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream)
{
    return forward_impl(x, batch, w, p, input_keep, ffn_sparsity, residual, out, sel_idx_out, workspace,
                        workspace_bytes, stream, nullptr, opt);
}

prox_status prox_ffn_forward_noalloc(const void *x, int64_t batch, const prox_weights *w, const prox_proxy *p,
                                     float input_keep, float ffn_sparsity, const void *residual, void *out,
                                     int32_t *sel_idx_out, hipStream_t stream)
{
    // the size limit first, on the host: nothing touches the device for a
    // layer whose workspace the static array cannot hold
    if (!w || !p) return PROX_ERR_INVALID_ARG;
    size_t need = 0;
    prox_status s = prox_workspace_size(w->d_model, w->d_ff, batch, p->mode, &need);
    if (s != PROX_OK) return s;
    if (need > (size_t)PROX_STATIC_SCRATCH_BYTES) return PROX_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    s = static_scratch(stream, &ws);
    if (s != PROX_OK) return s;
    return forward_impl(x, batch, w, p, input_keep, ffn_sparsity, residual, out, sel_idx_out, ws,
                        (size_t)PROX_STATIC_SCRATCH_BYTES, stream);
}

prox_status prox_ffn_forward_timed(const void *x, int64_t batch, const prox_weights *w, const prox_proxy *p,
                                   float input_keep, float ffn_sparsity, void *out, int32_t *sel_idx_out,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t *events)
{
    if (!events) return PROX_ERR_INVALID_ARG;
    for (int i = 0; i < 6; ++i)
        if (!events[i]) return PROX_ERR_INVALID_ARG;
    return forward_impl(x, batch, w, p, input_keep, ffn_sparsity, nullptr, out, sel_idx_out, workspace,
                        workspace_bytes, stream, events);
}

prox_status prox_stage1_select(const void *x, int64_t batch, const prox_weights *w, const prox_proxy *p,
                               float input_keep, float ffn_sparsity, int32_t *sel_idx_out, float *scores_out,
                               void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    prox_status s = check_weights(w);
    if (s != PROX_OK) return s;
    s = check_proxy(p, w);
    if (s != PROX_OK) return s;
    s = check_batch(batch, enum_int(p->mode));
    if (s != PROX_OK) return s;
    if (bad_ptr(x) || bad_ptr(sel_idx_out) || bad_ptr_opt(scores_out) || bad_ptr(workspace))
        return PROX_ERR_INVALID_ARG;
    int64_t k_in, k;
    s = counts(w->d_model, w->d_ff, input_keep, ffn_sparsity, &k_in, &k);
    if (s != PROX_OK) return s;
    if (k == w->d_ff) return PROX_ERR_INVALID_ARG;
    const Workspace ws = layout(w->d_model, w->d_ff, batch, enum_int(p->mode), workspace);
    if (workspace_bytes < ws.bytes) return PROX_ERR_WORKSPACE;
    return run_stage1(x, batch, w, p, k_in, k, sel_idx_out, scores_out ? scores_out : ws.score, ws, stream);
}

prox_status prox_topk(const float *scores, int64_t n, int64_t k, int32_t *sel_idx_out, void *workspace,
                      size_t workspace_bytes, hipStream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    if (n < 1 || n > 65535 || k < 0 || k > n) return PROX_ERR_INVALID_ARG;
    if (bad_ptr(scores) || bad_ptr(sel_idx_out)) return PROX_ERR_INVALID_ARG;
    if (k == 0) return PROX_OK;
    return hip_status(launch_topk(scores, (int)n, (int)k, sel_idx_out, stream));
}

prox_status prox_stage2_exact(const void *x, int64_t batch, const prox_weights *w, const int32_t *sel_idx,
                              int64_t k, void *out, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return prox_stage2_exact_ex(x, batch, w, sel_idx, k, nullptr, out, workspace, workspace_bytes, stream);
}

prox_status prox_stage2_exact_ex(const void *x, int64_t batch, const prox_weights *w, const int32_t *sel_idx,
                                 int64_t k, const prox_options *opt, void *out, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream)
{
    Opts o;
    prox_status s = check_options(opt, &o);
    if (s != PROX_OK) return s;
    s = check_weights(w);
    if (s != PROX_OK) return s;
    s = check_batch(batch, PROX_Q_INT8_ROW);
    if (s != PROX_OK) return s;
    if (k < 0 || k > w->d_ff) return PROX_ERR_INVALID_ARG;
    if (bad_ptr(x) || bad_ptr(out) || bad_ptr(workspace) || (k > 0 && bad_ptr(sel_idx))) return PROX_ERR_INVALID_ARG;
    if (x == out) return PROX_ERR_INVALID_ARG;
    const Workspace ws = layout(w->d_model, w->d_ff, batch, PROX_Q_INT8_ROW, workspace);
    if (workspace_bytes < ws.bytes) return PROX_ERR_WORKSPACE;
    return run_stage2(x, batch, w, sel_idx, k, nullptr, out, nullptr, ws, stream, nullptr, o);
}

prox_status prox_rmsnorm(const void *h, int64_t batch, int64_t d, prox_dtype dtype, float eps, void *out,
                         hipStream_t stream)
{
    const int dtype_i = enum_int(dtype);
    if (dtype_i != PROX_F32 && dtype_i != PROX_BF16) return PROX_ERR_UNSUPPORTED;
    if (batch < 1 || batch > 4096 || isnan(eps) || eps < 0.0f) return PROX_ERR_INVALID_ARG;
    // the kernel holds a row in 16-byte vectors, at most 16384 elements
    if (d < 8 || d > 16384 || d % 8 != 0) return PROX_ERR_UNSUPPORTED;
    if (bad_ptr(h) || bad_ptr(out)) return PROX_ERR_INVALID_ARG;
    return hip_status(launch_rmsnorm(dtype_i == PROX_F32 ? 0 : 1, h, (int)batch, (int)d, eps, out, stream));
}

prox_status prox_chain_forward(void *h, int64_t batch, const prox_weights *layers, const prox_proxy *proxies,
                               int64_t n_layers, float eps, float input_keep, float ffn_sparsity, void *workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    if (!layers || !proxies || n_layers < 1) return PROX_ERR_INVALID_ARG;
    if (isnan(eps) || eps < 0.0f) return PROX_ERR_INVALID_ARG;
    if (bad_ptr(h) || bad_ptr(workspace)) return PROX_ERR_INVALID_ARG;
    const prox_weights &w0 = layers[0];
    for (int64_t l = 0; l < n_layers; ++l) {
        prox_status s = check_weights(&layers[l]);
        if (s != PROX_OK) return s;
        s = check_proxy(&proxies[l], &layers[l]);
        if (s != PROX_OK) return s;
        if (layers[l].d_model != w0.d_model || layers[l].d_ff != w0.d_ff || enum_int(layers[l].dtype) != enum_int(w0.dtype) ||
            enum_int(proxies[l].mode) != enum_int(proxies[0].mode))
            return PROX_ERR_INVALID_ARG;
    }
    prox_status s = check_batch(batch, enum_int(proxies[0].mode));
    if (s != PROX_OK) return s;
    int64_t k_in, k;
    s = counts(w0.d_model, w0.d_ff, input_keep, ffn_sparsity, &k_in, &k);
    if (s != PROX_OK) return s;
    size_t ffn_bytes = 0;
    s = prox_workspace_size(w0.d_model, w0.d_ff, batch, proxies[0].mode, &ffn_bytes);  // checked valid above
    if (s != PROX_OK) return s;
    const size_t need = ffn_bytes + 256 + (size_t)batch * w0.d_model * 4;
    if (workspace_bytes < need) return PROX_ERR_WORKSPACE;
    void *xn = (char *)workspace + align256(ffn_bytes);
    const int dt = enum_int(w0.dtype) == PROX_F32 ? 0 : 1;
    if (k > 0 && k < w0.d_ff) {
        // Stage 1's first kernel (the single-token kernel, or the input
        // selection of a batch) normalizes h itself, bitwise as the RMSNorm
        // kernel, and hands RMSNorm(h) to Stage 2 in xn: no RMSNorm launch
        const Workspace ws = layout(w0.d_model, w0.d_ff, batch, enum_int(proxies[0].mode), workspace);
        const bool fused =
            batch == 1 && fused_supported(1, w0.d_model, w0.d_ff, enum_int(proxies[0].mode) == PROX_Q_INT4_G128 ? 4 : 8);
        for (int64_t l = 0; l < n_layers; ++l) {
            const prox_proxy &p = proxies[l];
            if (fused) {
                TRY_HIP(launch_stage1_fused(dt, enum_int(p.mode) == PROX_Q_INT4_G128 ? 4 : 8, h, (int)w0.d_model,
                                            (int)w0.d_ff, (int)k_in, (int)k, (const uint8_t *)p.codes,
                                            (const float *)p.scales, ws.proxy_part, ws.score, ws.sel, ws.counters,
                                            PROX_ACT_SILU, PROX_SIGNAL_S, stream, eps, xn));
            } else {
                s = run_stage1(h, batch, &layers[l], &p, k_in, k, ws.sel, ws.score, ws, stream, nullptr, Opts(), eps,
                               xn);
                if (s != PROX_OK) return s;
            }
            s = run_stage2(xn, batch, &layers[l], ws.sel, k, h, h, nullptr, ws, stream);
            if (s != PROX_OK) return s;
        }
        return PROX_OK;
    }
    for (int64_t l = 0; l < n_layers; ++l) {
        TRY_HIP(launch_rmsnorm(dt, h, (int)batch, (int)w0.d_model, eps, xn, stream));
        s = forward_impl(xn, batch, &layers[l], &proxies[l], input_keep, ffn_sparsity, h, h, nullptr, workspace,
                         ffn_bytes, stream);
        if (s != PROX_OK) return s;
    }
    return PROX_OK;
}

}  // extern "C"
