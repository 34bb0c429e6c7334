/*
 * Prox CPU oracle -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * A plain, slow, binary64 implementation of what the Prox two-stage sparse
 * SwiGLU FFN forward computes, written from the Prox pages ("Prox:
 * Training-Free FFN Activation Sparsity via Approximate Intermediate-Channel
 * Salience in LLMs": the original abstract, and the technical summary's
 * Problem Statement, Stage 1: Lightweight Proxy Construction, and Stage 2:
 * Exact Sparse Computation).  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or helper with the HIP library; the two meet only on the seeded
 * inputs.
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function.  Plain loops, no BLAS, no blocking; an OpenMP parallel-for over
 * independent output elements (each still summed by one thread in index
 * order, so results do not depend on the thread count).
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* threads (for the CPU-baseline timing only; results do not change)  */
/* ------------------------------------------------------------------ */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* SwiGLU activation.                                                  */
/* Problem Statement: the intermediate state is s = u (.) h with h the  */
/* gate activation.  Reading: h = silu(W_gate x) as in the SwiGLU FFNs */
/* of the Llama / Mistral / Qwen families the pages evaluate, and      */
/* silu(z) = z / (1 + exp(-z)).                                        */
/* ------------------------------------------------------------------ */
double oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* GELU-gated FFNs (GeGLU) in the tanh form of the Gemma family the pages */
/* also evaluate (technical summary, Key Contributions: Gemma-3 among the */
/* six families): gelu(z) = z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))). */
double oracle_gelu_tanh(double z)
{
    return 0.5 * z * (1.0 + tanh(sqrt(2.0 / acos(-1.0)) * (z + 0.044715 * z * z * z)));
}

/* the gate activation h = act(g): 0 = silu (SwiGLU), 1 = gelu_tanh (GeGLU) */
double oracle_act(int act, double z)
{
    return act == 1 ? oracle_gelu_tanh(z) : oracle_silu(z);
}

/* ------------------------------------------------------------------ */
/* Counts.  The pages give input sparsity as a fraction of retained    */
/* input entries (Sparsity Allocation: keep at least 30%) and Stage-2  */
/* sparsity as a fraction of intermediate channels dropped (~70%).     */
/* Reading: round half up in binary64, clamped.                        */
/* ------------------------------------------------------------------ */
int64_t oracle_input_count(double keep, int64_t d)
{
    double t = floor(keep * (double)d + 0.5);
    if (t < 1.0) t = 1.0;
    if (t > (double)d) t = (double)d;
    return (int64_t)t;
}

int64_t oracle_channel_count(double sparsity, int64_t F)
{
    double t = floor((1.0 - sparsity) * (double)F + 0.5);
    if (t < 0.0) t = 0.0;
    if (t > (double)F) t = (double)F;
    return (int64_t)t;
}

/* ------------------------------------------------------------------ */
/* Quantized proxy weights (Stage 1: quantized proxy copies of W_gate   */
/* and W_up).  The pages say only "INT4".  Reading: symmetric absmax,   */
/* binary32 arithmetic with round-to-nearest-even, binary32 scales;    */
/* an all-zero segment gets scale 0 and codes 0.  int8: one scale per  */
/* output row (qmax 127).  int4: one scale per (row, 128 consecutive   */
/* inputs) (qmax 7).  Codes are returned unpacked, one int8 per weight. */
/* ------------------------------------------------------------------ */
static void quantize_segment(const float *w, int64_t n, int qmax, int8_t *q, float *scale)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float m = fabsf(w[i]);
        if (m > a) a = m;
    }
    float s = a / (float)qmax;
    *scale = s;
    for (int64_t i = 0; i < n; ++i) {
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        float t = rintf(w[i] / s);
        if (t > (float)qmax) t = (float)qmax;
        if (t < (float)-qmax) t = (float)-qmax;
        q[i] = (int8_t)t;
    }
}

/* w: [rows][cols] binary32; q: [rows][cols]; scale: [rows] */
void oracle_quantize_int8_row(const float *w, int64_t rows, int64_t cols, int8_t *q, float *scale)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        quantize_segment(w + r * cols, cols, 127, q + r * cols, scale + r);
}

/* w: [rows][cols] binary32 with cols % 128 == 0; q: [rows][cols] in [-7,7];
 * scale: [rows][cols/128] */
void oracle_quantize_int4_g128(const float *w, int64_t rows, int64_t cols, int8_t *q, float *scale)
{
    int64_t groups = cols / 128;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        for (int64_t g = 0; g < groups; ++g)
            quantize_segment(w + r * cols + g * 128, 128, 7, q + r * cols + g * 128,
                             scale + r * groups + g);
}

/* ------------------------------------------------------------------ */
/* Magnitude ranking.  The mask is built from the magnitude ranking of  */
/* the (proxy) intermediate state (abstract; Stage 1: Mask Generation).*/
/* Reading for ties: a precedes b iff |a| > |b|, or |a| == |b| and a's  */
/* index is lower.  Full sort, then the first k indices in ascending   */
/* index order.                                                        */
/* ------------------------------------------------------------------ */
typedef struct {
    double mag;
    int64_t idx;
} ranked;

static int ranked_cmp(const void *pa, const void *pb)
{
    const ranked *a = (const ranked *)pa, *b = (const ranked *)pb;
    if (a->mag > b->mag) return -1;
    if (a->mag < b->mag) return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx) ? 1 : 0;
}

static int idx_cmp(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    return (a < b) ? -1 : (a > b) ? 1 : 0;
}

/* v: [n] finite values; out: [k] indices of the k first under the order,
 * sorted ascending.  Returns the k-th magnitude (the threshold T) through
 * *kth (0 if k == 0). */
void oracle_topk_ascending(const double *v, int64_t n, int64_t k, int64_t *out, double *kth)
{
    ranked *r = (ranked *)malloc((size_t)(n > 0 ? n : 1) * sizeof(ranked));
    for (int64_t i = 0; i < n; ++i) {
        r[i].mag = fabs(v[i]);
        r[i].idx = i;
    }
    qsort(r, (size_t)n, sizeof(ranked), ranked_cmp);
    for (int64_t i = 0; i < k; ++i) out[i] = r[i].idx;
    if (kth) *kth = (k > 0) ? r[k - 1].mag : 0.0;
    qsort(out, (size_t)k, sizeof(int64_t), idx_cmp);
    free(r);
}

/* ------------------------------------------------------------------ */
/* Stage 1, input sparsity (Stage 1: Input Sparsity & Quantization).   */
/* Reading: per token, keep the k_in entries of x that come first in   */
/* the magnitude order above; zero the others.                         */
/* x, xhat: [B][d]                                                     */
/* ------------------------------------------------------------------ */
void oracle_input_select(const double *x, int64_t B, int64_t d, int64_t k_in, double *xhat)
{
    int64_t *kept = (int64_t *)malloc((size_t)(k_in > 0 ? k_in : 1) * sizeof(int64_t));
    for (int64_t b = 0; b < B; ++b) {
        const double *xb = x + b * d;
        double *ob = xhat + b * d;
        oracle_topk_ascending(xb, d, k_in, kept, NULL);
        for (int64_t i = 0; i < d; ++i) ob[i] = 0.0;
        for (int64_t t = 0; t < k_in; ++t) ob[kept[t]] = xb[kept[t]];
    }
    free(kept);
}

/* ------------------------------------------------------------------ */
/* Stage 1, proxy activations and salience (Stage 1: Proxy Activation,  */
/* Mask Generation).  Dequantized proxy weight W~ = scale * code, exact */
/* in binary64.  g~ = W~_gate x^, u~ = W~_up x^, s~ = silu(g~) * u~.   */
/* Reading for a batch of B tokens (the pages target B = 1): one mask   */
/* for the batch, scored by score_j = sum_b |s~_{b,j}|.                */
/* mode 0 = int8 per row (scale [F]); 1 = int4 per 128-group (scale    */
/* [F][d/128]).  qg, qu: [F][d] codes.  gt, ut: [B][F]; score: [F].    */
/* ------------------------------------------------------------------ */
static double dequant(const int8_t *q, const float *scale, int mode, int64_t d, int64_t j, int64_t i)
{
    double s = (mode == 0) ? (double)scale[j] : (double)scale[j * (d / 128) + i / 128];
    return s * (double)q[j * d + i];
}

/* The per-token salience term of a channel for the selection signal.    */
/* Problem Statement: the exact intermediate state s = u (.) h is the      */
/* ideal signal; prior methods use one branch, the gate activation h or    */
/* the up activation u.  signal 0 = |h~ u~| (Prox), 1 = |h~| (gate branch  */
/* only), 2 = |u~| (up branch only), with h~ = act(g~).                    */
static double salience_term(int signal, int act, double g, double u)
{
    double h = oracle_act(act, g);
    if (signal == 1) return fabs(h);
    if (signal == 2) return fabs(u);
    return fabs(h * u);
}

void oracle_proxy(const double *xhat, int64_t B, int64_t d, int64_t F, int mode,
                  const int8_t *qg, const float *scg, const int8_t *qu, const float *scu,
                  int act, int signal, double *gt, double *ut, double *score)
{
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < F; ++j) {
        double sc = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            const double *xb = xhat + b * d;
            double g = 0.0, u = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                g += xb[i] * dequant(qg, scg, mode, d, j, i);
                u += xb[i] * dequant(qu, scu, mode, d, j, i);
            }
            gt[b * F + j] = g;
            ut[b * F + j] = u;
            sc += salience_term(signal, act, g, u);
        }
        score[j] = sc;
    }
}

/* ------------------------------------------------------------------ */
/* Stage 2, exact sparse computation (Stage 2: Exact Projections, Final */
/* Output).  For each selected channel j, with the original weights and */
/* the dense input x (reading: the proxy values and the sparsified x    */
/* are not propagated downstream): g = W_gate[j] . x, u = W_up[j] . x,  */
/* s = act(g) * u; then y = sum over selected j of W_down[:, j] * s_j   */
/* (the down projection restricted to the same mask).                  */
/* x: [B][d]; wg, wu: [F][d]; wd: [d][F] (nn.Linear orientation);       */
/* sel: [k] ascending; s: [B][k] (nullable); y: [B][d].                */
/* ------------------------------------------------------------------ */
void oracle_ffn_masked(const double *x, int64_t B, int64_t d, int64_t F,
                       const float *wg, const float *wu, const float *wd,
                       const int64_t *sel, int64_t k, int act, double *s_out, double *y)
{
    double *s = (double *)malloc((size_t)(B * k > 0 ? B * k : 1) * sizeof(double));
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < k; ++r) {
        int64_t j = sel[r];
        for (int64_t b = 0; b < B; ++b) {
            const double *xb = x + b * d;
            double g = 0.0, u = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                g += (double)wg[j * d + i] * xb[i];
                u += (double)wu[j * d + i] * xb[i];
            }
            s[b * k + r] = oracle_act(act, g) * u;
        }
    }
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < d; ++m) {
        for (int64_t b = 0; b < B; ++b) {
            double acc = 0.0;
            for (int64_t t = 0; t < k; ++t)
                acc += (double)wd[m * F + sel[t]] * s[b * k + t];
            y[b * d + m] = acc;
        }
    }
    if (s_out) memcpy(s_out, s, (size_t)(B * k) * sizeof(double));
    free(s);
}

/* ------------------------------------------------------------------ */
/* FP8 exact weights.  The pages claim Prox composes with FP8 model     */
/* quantization (technical summary, Experimental Results and            */
/* Significance and Claims) but give no scheme.  Reading: OCP E4M3 --   */
/* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 */
/* holds the subnormals m * 2^-9; no infinities; S.1111.111 is NaN; the */
/* largest finite magnitude is 448 -- with one binary32 scale per output */
/* row: scale = fl32(amax / 448); code = the E4M3 value nearest to      */
/* fl32(w / scale), ties to the even code, magnitudes above 448         */
/* saturating to 448; the code's sign is the quotient's sign bit.  An   */
/* all-zero row gets scale 0 and codes 0.                               */
/* ------------------------------------------------------------------ */
double oracle_e4m3_decode(int c)
{
    int sgn = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* The finite magnitudes 0x00..0x7E increase with the code, so the nearest */
/* one is found by searching that ordered table.                           */
int oracle_e4m3_encode(float v)
{
    int sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0, hi = 0x7E; /* largest code whose magnitude is <= a */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (oracle_e4m3_decode(mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo; /* decode(c) <= a < decode(c + 1), c + 1 <= 0x7E */
    double below = a - oracle_e4m3_decode(c), above = oracle_e4m3_decode(c + 1) - a;
    if (above < below || (above == below && ((c + 1) & 1) == 0)) c = c + 1;
    return sign | c;
}

/* w: [rows][cols] binary32; q: [rows][cols] E4M3 codes; scale: [rows] */
void oracle_quantize_fp8_row(const float *w, int64_t rows, int64_t cols, uint8_t *q, float *scale)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const float *wr = w + r * cols;
        float a = 0.0f;
        for (int64_t i = 0; i < cols; ++i)
            if (fabsf(wr[i]) > a) a = fabsf(wr[i]);
        float sc = a / 448.0f;
        scale[r] = sc;
        for (int64_t i = 0; i < cols; ++i) q[r * cols + i] = (uint8_t)(sc == 0.0f ? 0 : oracle_e4m3_encode(wr[i] / sc));
    }
}

/* The binary32 weights an FP8 layer stands for, as its proxy is built     */
/* from them: w = fl32(scale[r] * decode(q)).                              */
void oracle_dequant_fp8_f32(const uint8_t *q, const float *scale, int64_t rows, int64_t cols, float *w)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < cols; ++i) w[r * cols + i] = scale[r] * (float)oracle_e4m3_decode(q[r * cols + i]);
}

/* Stage 2 on FP8 weights: the masked SwiGLU of oracle_ffn_masked with each */
/* weight taken as scale * decode(code), exact in binary64 (24 + 4          */
/* significant bits).  qg, qu: [F][d], scales [F]; qd: [d][F] (W_down,      */
/* nn.Linear orientation), scales [d].                                      */
void oracle_ffn_masked_fp8(const double *x, int64_t B, int64_t d, int64_t F,
                           const uint8_t *qg, const float *sg, const uint8_t *qu, const float *su,
                           const uint8_t *qd, const float *sd, const int64_t *sel, int64_t k, int act,
                           double *s_out, double *y)
{
    double *s = (double *)malloc((size_t)(B * k > 0 ? B * k : 1) * sizeof(double));
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < k; ++r) {
        int64_t j = sel[r];
        for (int64_t b = 0; b < B; ++b) {
            const double *xb = x + b * d;
            double g = 0.0, u = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                g += (double)sg[j] * oracle_e4m3_decode(qg[j * d + i]) * xb[i];
                u += (double)su[j] * oracle_e4m3_decode(qu[j * d + i]) * xb[i];
            }
            s[b * k + r] = oracle_act(act, g) * u;
        }
    }
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < d; ++m) {
        for (int64_t b = 0; b < B; ++b) {
            double acc = 0.0;
            for (int64_t t = 0; t < k; ++t)
                acc += (double)sd[m] * oracle_e4m3_decode(qd[m * F + sel[t]]) * s[b * k + t];
            y[b * d + m] = acc;
        }
    }
    if (s_out) memcpy(s_out, s, (size_t)(B * k) * sizeof(double));
    free(s);
}

/* ------------------------------------------------------------------ */
/* RMSNorm with unit gain, for a stack of FFN layers (the pages do not  */
/* describe the layer glue): r = h / sqrt(mean(h^2) + eps).            */
/* ------------------------------------------------------------------ */
void oracle_rmsnorm(const double *h, int64_t B, int64_t d, double eps, double *r)
{
    for (int64_t b = 0; b < B; ++b) {
        double ss = 0.0;
        for (int64_t i = 0; i < d; ++i) ss += h[b * d + i] * h[b * d + i];
        double rms = sqrt(ss / (double)d + eps);
        for (int64_t i = 0; i < d; ++i) r[b * d + i] = h[b * d + i] / rms;
    }
}
