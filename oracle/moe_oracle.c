/*
 * CPU oracle for the sparse Mixture-of-Experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes, per token (the "eager" expert backend that the page
 * "Transformer中的混合专家架构详解" (MoEs in Transformers), section on the
 * experts backends, names as the correctness reference: loop over the
 * selected experts and apply each one's projections):
 *
 *   1. router logits  l[e] = <x, Wr[e]> (+ b[e])          (PhiMoE page, sec. 6:
 *                                                          a bias-free linear
 *                                                          router; bias optional)
 *   2. top-k experts by logit, ties to the lower index    (PhiMoE page, sec. 6:
 *                                                          greedy top-1, mask,
 *                                                          next; eval path)
 *   3. weights = softmax over the k selected logits, times the routed scale
 *                                                          (PhiMoE page, sec. 6;
 *                                                          Instella page: scale 2.5)
 *   4. expert SwiGLU: g = Wgu[e][0:I] x, u = Wgu[e][I:2I] x, h = silu(g)*u,
 *      y = Wd[e] h                                         (PhiMoE page, sec. 2,
 *                                                          item 3: packed gate_up,
 *                                                          chunk(2), act(gate)*up)
 *   5. out = sum_j w_j y_j  (+ every shared expert's SwiGLU output, unscaled)
 *                                                          (GraniteMoeSWA page,
 *                                                          decoder-layer section;
 *                                                          Instella page, FarSkipMoE)
 *   6. routing metadata: per-expert counts, exclusive offsets, and the stable
 *      expert-major permutation of flat assignments a = t*k + j
 *                                                          (MoEs in Transformers
 *                                                          page: grouped_mm sorts
 *                                                          tokens by expert id and
 *                                                          groups them; PhiMoE
 *                                                          page sec. 2 item 4:
 *                                                          no token is dropped)
 *
 * Precision: inputs are bf16 bit patterns (dtype 0) widened exactly to fp32,
 * or fp32 (dtype 1). Every sum accumulates in fp32 with fmaf in ascending
 * index order. The router logit is the one exception to "ascending": the
 * pages fix no summation order, yet the expert ids must be reproducible bit
 * for bit, so the logit is DEFINED as the fp32 sum taken in this order:
 * 64 partial sums P[0..63]; element i = 512*c + 8*L + v (v = 0..7) goes to
 * P[L], visiting c ascending then v ascending; then, for d = 32, 16, 8, 4,
 * 2, 1, every P[L] becomes P[L] + P[L ^ d]; the logit is P[0]. Softmax
 * weights and SiLU are evaluated in fp64 and rounded to fp32.
 *
 * Build: gcc -O2 -mfma -ffp-contract=off -fopenmp -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_BAD -1

static float widen(const void *base, int dtype, size_t i)
{
    if (dtype == 0) {
        uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return f;
    }
    return ((const float *)base)[i];
}

/* Logit of one (token, expert) pair in the order stated in the header. */
static float router_dot(const void *X, const void *Wr, int dtype, int64_t t, int64_t e, int64_t H)
{
    float P[64];
    for (int L = 0; L < 64; L++)
        P[L] = 0.0f;
    for (int64_t c = 0; c * 512 < H; c++)
        for (int L = 0; L < 64; L++)
            for (int v = 0; v < 8; v++) {
                int64_t i = 512 * c + 8 * L + v;
                if (i < H)
                    P[L] = fmaf(widen(X, dtype, (size_t)(t * H + i)),
                                widen(Wr, dtype, (size_t)(e * H + i)), P[L]);
            }
    for (int d = 32; d >= 1; d /= 2) {
        float Q[64];
        for (int L = 0; L < 64; L++)
            Q[L] = P[L] + P[L ^ d];
        memcpy(P, Q, sizeof P);
    }
    return P[0];
}

int oracle_router_logits(const void *X, const void *Wr, const float *bias, int dtype,
                         int64_t T, int64_t H, int64_t E, float *logits)
{
    if (!X || !Wr || !logits || T < 0 || H <= 0 || E <= 0 || (dtype != 0 && dtype != 1))
        return OR_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int64_t e = 0; e < E; e++) {
            float l = router_dot(X, Wr, dtype, t, e, H);
            if (bias)
                l = l + bias[e];
            logits[t * E + e] = l;
        }
    return OR_OK;
}

/* Ranking value of a key: a NaN ranks below every number (as -inf). */
static float rank_value(float x)
{
    return x != x ? -INFINITY : x;
}

/* Expert a ranks before expert b iff l[a] > l[b], or l[a] == l[b] and a < b
 * (NaN taken as -inf). */
static int ranks_before(const float *l, int64_t a, int64_t b)
{
    const float va = rank_value(l[a]), vb = rank_value(l[b]);
    return va > vb || (va == vb && a < b);
}

int oracle_select_topk(const float *logits, int64_t T, int64_t E, int k, float routed_scale,
                       int32_t *ids, float *weights)
{
    if (!logits || !ids || !weights || T < 0 || E <= 0 || k < 1 || k > E || k > 256)
        return OR_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        /* greedy: take the best remaining expert k times */
        for (int j = 0; j < k; j++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++) {
                int taken = 0;
                for (int q = 0; q < j; q++)
                    if (ids[t * k + q] == e)
                        taken = 1;
                if (taken)
                    continue;
                if (best < 0 || ranks_before(l, e, best))
                    best = e;
            }
            ids[t * k + j] = (int32_t)best;
        }
        /* softmax over the selected logits (shifted by the largest), renormalised */
        double m = (double)l[ids[t * k]];
        double p[256], s = 0.0;
        for (int j = 0; j < k; j++) {
            p[j] = exp((double)l[ids[t * k + j]] - m);
            s += p[j];
        }
        for (int j = 0; j < k; j++)
            weights[t * k + j] = (float)((double)routed_scale * p[j] / s);
    }
    return OR_OK;
}

int oracle_route(const int32_t *ids, int64_t T, int k, int64_t E, int32_t *counts,
                 int32_t *offsets, int32_t *perm, int32_t *inv)
{
    if (!ids || !counts || !offsets || !perm || !inv || T < 0 || k < 1 || E <= 0)
        return OR_BAD;
    int64_t TK = T * k;
    for (int64_t e = 0; e < E; e++)
        counts[e] = 0;
    for (int64_t a = 0; a < TK; a++) {
        if (ids[a] < 0 || ids[a] >= E)
            return OR_BAD;
        counts[ids[a]]++;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    /* stable counting sort: assignments of one expert keep ascending a */
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!next)
        return OR_BAD;
    for (int64_t e = 0; e < E; e++)
        next[e] = offsets[e];
    for (int64_t a = 0; a < TK; a++) {
        int32_t p = next[ids[a]]++;
        perm[p] = (int32_t)a;
        inv[a] = p;
    }
    free(next);
    return OR_OK;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* y = Wd h with h = silu(Wg x) * (Wu x); weights rows [0,I) gate, [I,2I) up. */
static void swiglu_expert(const float *x, const void *gate_up, const void *down, int dtype,
                          int64_t H, int64_t I, float *h, float *y)
{
    for (int64_t n = 0; n < I; n++) {
        float g = 0.0f, u = 0.0f;
        for (int64_t i = 0; i < H; i++) {
            g = fmaf(widen(gate_up, dtype, (size_t)(n * H + i)), x[i], g);
            u = fmaf(widen(gate_up, dtype, (size_t)((I + n) * H + i)), x[i], u);
        }
        h[n] = (float)(silu((double)g) * (double)u);
    }
    for (int64_t m = 0; m < H; m++) {
        float acc = 0.0f;
        for (int64_t n = 0; n < I; n++)
            acc = fmaf(widen(down, dtype, (size_t)(m * I + n)), h[n], acc);
        y[m] = acc;
    }
}

/*
 * Layer output for the listed tokens: out[r] = sum_j w[t,j] * FFN_{ids[t,j]}(x_t)
 * (j ascending, fp32 fmaf) + sum_s SharedFFN_s(x_t), with t = tokens[r].
 * gate_up is [E, 2I, H], down is [E, H, I]; shared expert s has gate_up
 * [2*shared_I[s], H] and down [H, shared_I[s]].
 */
int oracle_moe_tokens(const void *X, const void *gate_up, const void *down, int dtype,
                      int64_t H, int64_t I, const int32_t *ids, const float *weights, int k,
                      int n_shared, const void *const *shared_gate_up,
                      const void *const *shared_down, const int64_t *shared_I,
                      const int32_t *tokens, int64_t n_tokens, float *out)
{
    if (!X || !gate_up || !down || !ids || !weights || !tokens || !out || H <= 0 || I <= 0 ||
        k < 1 || n_shared < 0)
        return OR_BAD;
    int64_t Imax = I;
    for (int s = 0; s < n_shared; s++)
        if (shared_I[s] > Imax)
            Imax = shared_I[s];
    int bad = 0;
#pragma omp parallel
    {
        float *x = (float *)malloc(sizeof(float) * (size_t)H);
        float *y = (float *)malloc(sizeof(float) * (size_t)H);
        float *h = (float *)malloc(sizeof(float) * (size_t)Imax);
        if (!x || !y || !h) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_tokens; r++) {
                int64_t t = tokens[r];
                for (int64_t i = 0; i < H; i++)
                    x[i] = widen(X, dtype, (size_t)(t * H + i));
                float *o = out + r * H;
                for (int64_t m = 0; m < H; m++)
                    o[m] = 0.0f;
                for (int j = 0; j < k; j++) {
                    int64_t e = ids[t * k + j];
                    float w = weights[t * k + j];
                    size_t gu_off = (size_t)e * (size_t)(2 * I * H);
                    size_t dn_off = (size_t)e * (size_t)(H * I);
                    const void *gu = dtype == 0 ? (const void *)((const uint16_t *)gate_up + gu_off)
                                                : (const void *)((const float *)gate_up + gu_off);
                    const void *dn = dtype == 0 ? (const void *)((const uint16_t *)down + dn_off)
                                                : (const void *)((const float *)down + dn_off);
                    swiglu_expert(x, gu, dn, dtype, H, I, h, y);
                    for (int64_t m = 0; m < H; m++)
                        o[m] = fmaf(w, y[m], o[m]);
                }
                for (int s = 0; s < n_shared; s++) {
                    swiglu_expert(x, shared_gate_up[s], shared_down[s], dtype, H, shared_I[s], h, y);
                    for (int64_t m = 0; m < H; m++)
                        o[m] = o[m] + y[m];
                }
            }
        }
        free(x);
        free(y);
        free(h);
    }
    return bad ? OR_BAD : OR_OK;
}

/*
 * Router statistics for the load-balancing auxiliary loss (PhiMoE page,
 * section 6: the Switch Transformer loss over the router logits, scaled by
 * router_aux_loss_coef = 0.001, padding tokens excluded). The pages cite the
 * Switch paper's equations without printing them; its form is used: with n
 * counted tokens (mask[t] != 0, or all tokens when mask is NULL),
 *   P[e] = (1/n) sum_t softmax(logits[t, :])[e]   (all E experts),
 *   f[e] = (1/n) #{(t, j) : ids[t, j] = e}        (the top-k assignments),
 *   aux  = E * sum_e f[e] * P[e];
 * everything zero when n = 0. Evaluated in fp64. Against the pages this is
 * partly unpinned (they print no equation); the tests pin it to the loss's
 * closed forms (uniform logits, certain and balanced routing) and to a
 * separate numpy evaluation.
 */
int oracle_router_stats(const float *logits, const int32_t *ids, const int32_t *mask, int64_t T, int64_t E,
                        int k, double *prob_mean, double *load, double *aux)
{
    if (!logits || !ids || !prob_mean || !load || !aux || T < 0 || E < 1 || k < 1)
        return OR_BAD;
    for (int64_t e = 0; e < E; e++)
        prob_mean[e] = load[e] = 0.0;
    int64_t n = 0;
    for (int64_t t = 0; t < T; t++) {
        if (mask && mask[t] == 0)
            continue;
        n++;
        const float *l = logits + t * E;
        double m = l[0];
        for (int64_t e = 1; e < E; e++)
            if (l[e] > m)
                m = l[e];
        double z = 0.0;
        for (int64_t e = 0; e < E; e++)
            z += exp((double)l[e] - m);
        for (int64_t e = 0; e < E; e++)
            prob_mean[e] += exp((double)l[e] - m) / z;
        for (int j = 0; j < k; j++)
            load[ids[t * k + j]] += 1.0;
    }
    double a = 0.0;
    for (int64_t e = 0; e < E; e++) {
        prob_mean[e] = n ? prob_mean[e] / (double)n : 0.0;
        load[e] = n ? load[e] / (double)n : 0.0;
        a += load[e] * prob_mean[e];
    }
    *aux = (double)E * a;
    return OR_OK;
}

/*
 * FP8 expert weights (the low-precision decode storage: the MoEs in
 * Transformers page, section on why MoEs are fast, prices decode at memory
 * bandwidth over the bytes of the active weights and notes that a native
 * low-precision format is faster still; its weight-loading section ties
 * per-expert quantisation to packed experts). The pages fix no format; the
 * reading taken here is OCP FP8 E4M3 with one fp32 scale per weight row.
 *
 * E4M3 byte b: sign = bit 7, exponent field e = bits 6..3 (bias 7), mantissa
 * m = bits 2..0; e = 0 holds the subnormals m * 2^-9, otherwise the value is
 * (1 + m/8) * 2^(e-7); e = 15 with m = 7 is NaN. Largest finite: 448.
 */
static double e4m3_value(uint8_t b)
{
    int sgn = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return sgn ? -v : v;
}

/* The value table of all 256 codes (NaN for the two NaN codes). */
int oracle_e4m3_values(double *out256)
{
    if (!out256)
        return OR_BAD;
    for (int b = 0; b < 256; b++)
        out256[b] = e4m3_value((uint8_t)b);
    return OR_OK;
}

/*
 * Per-row quantisation of bf16 rows: a = max |w|, scale = a / 448 (fp32
 * division), q = the code whose value is nearest to w / scale (fp32
 * division), ties to the even code, saturating at 448; zero -> 0x00. A row
 * with a < 448 * 2^-126 (its scale would be subnormal) is stored as zeros
 * with scale 1. The nearest code is found by bisection over the 127
 * non-negative finite values, which increase with the code.
 */
int oracle_quantize_e4m3_rows(const uint16_t *w, int64_t rows, int64_t cols, uint8_t *q, float *scale)
{
    if (!w || !q || !scale || rows < 0 || cols < 1)
        return OR_BAD;
    double pos[127];
    for (int c = 0; c < 127; c++)
        pos[c] = e4m3_value((uint8_t)c);
    const float min_row_max = 448.0f * ldexpf(1.0f, -126);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float a = 0.0f;
        for (int64_t i = 0; i < cols; i++) {
            float x = fabsf(widen(w, 0, (size_t)(r * cols + i)));
            if (x > a)
                a = x;
        }
        int zero_row = !(a >= min_row_max);
        float sc = zero_row ? 1.0f : a / 448.0f;
        scale[r] = sc;
        for (int64_t i = 0; i < cols; i++) {
            uint8_t code = 0;
            if (!zero_row) {
                float v = widen(w, 0, (size_t)(r * cols + i)) / sc;
                double av = fabs((double)v);
                int c;
                if (av >= pos[126]) {
                    c = 126;
                } else {
                    int lo = 0, hi = 126; /* pos[lo] <= av < pos[hi] */
                    while (hi - lo > 1) {
                        int mid = (lo + hi) / 2;
                        if (pos[mid] <= av)
                            lo = mid;
                        else
                            hi = mid;
                    }
                    double dlo = av - pos[lo], dhi = pos[hi] - av;
                    c = dlo < dhi ? lo : dhi < dlo ? hi : ((lo & 1) ? hi : lo);
                }
                code = c == 0 ? 0 : (uint8_t)((v < 0 ? 0x80 : 0) | c);
            }
            q[r * cols + i] = code;
        }
    }
    return OR_OK;
}

/* The expert SwiGLU with E4M3 weights: each weight is fl32(value(q) * row
 * scale) (the product of a 4-bit and a 24-bit significand is exact in fp64,
 * so this is one rounding); tab[] holds value(q) for every code. */
static void swiglu_expert_e4m3(const double *tab, const float *x, const uint8_t *gate_up,
                               const float *gu_scale, const uint8_t *down, const float *dn_scale,
                               int64_t H, int64_t I, float *h, float *y)
{
    for (int64_t n = 0; n < I; n++) {
        float g = 0.0f, u = 0.0f;
        for (int64_t i = 0; i < H; i++) {
            float wg = (float)(tab[gate_up[n * H + i]] * (double)gu_scale[n]);
            float wu = (float)(tab[gate_up[(I + n) * H + i]] * (double)gu_scale[I + n]);
            g = fmaf(wg, x[i], g);
            u = fmaf(wu, x[i], u);
        }
        h[n] = (float)(silu((double)g) * (double)u);
    }
    for (int64_t m = 0; m < H; m++) {
        float acc = 0.0f;
        for (int64_t n = 0; n < I; n++)
            acc = fmaf((float)(tab[down[m * I + n]] * (double)dn_scale[m]), h[n], acc);
        y[m] = acc;
    }
}

/*
 * Same layer as oracle_moe_tokens with the routed experts stored as E4M3
 * bytes gate_up [E, 2I, H], down [E, H, I] and fp32 row scales
 * gu_scale [E, 2I], dn_scale [E, H]; activations and shared experts bf16.
 */
int oracle_moe_tokens_e4m3(const uint16_t *X, const uint8_t *gate_up, const float *gu_scale,
                           const uint8_t *down, const float *dn_scale, int64_t H, int64_t I,
                           const int32_t *ids, const float *weights, int k, int n_shared,
                           const void *const *shared_gate_up, const void *const *shared_down,
                           const int64_t *shared_I, const int32_t *tokens, int64_t n_tokens, float *out)
{
    if (!X || !gate_up || !gu_scale || !down || !dn_scale || !ids || !weights || !tokens || !out ||
        H <= 0 || I <= 0 || k < 1 || n_shared < 0)
        return OR_BAD;
    double tab[256];
    for (int b = 0; b < 256; b++)
        tab[b] = e4m3_value((uint8_t)b);
    int64_t Imax = I;
    for (int s = 0; s < n_shared; s++)
        if (shared_I[s] > Imax)
            Imax = shared_I[s];
    int bad = 0;
#pragma omp parallel
    {
        float *x = (float *)malloc(sizeof(float) * (size_t)H);
        float *y = (float *)malloc(sizeof(float) * (size_t)H);
        float *h = (float *)malloc(sizeof(float) * (size_t)Imax);
        if (!x || !y || !h) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_tokens; r++) {
                int64_t t = tokens[r];
                for (int64_t i = 0; i < H; i++)
                    x[i] = widen(X, 0, (size_t)(t * H + i));
                float *o = out + r * H;
                for (int64_t m = 0; m < H; m++)
                    o[m] = 0.0f;
                for (int j = 0; j < k; j++) {
                    int64_t e = ids[t * k + j];
                    float w = weights[t * k + j];
                    swiglu_expert_e4m3(tab, x, gate_up + (size_t)e * (size_t)(2 * I * H), gu_scale + e * 2 * I,
                                       down + (size_t)e * (size_t)(H * I), dn_scale + e * H, H, I, h, y);
                    for (int64_t m = 0; m < H; m++)
                        o[m] = fmaf(w, y[m], o[m]);
                }
                for (int s = 0; s < n_shared; s++) {
                    swiglu_expert(x, shared_gate_up[s], shared_down[s], 0, H, shared_I[s], h, y);
                    for (int64_t m = 0; m < H; m++)
                        o[m] = o[m] + y[m];
                }
            }
        }
        free(x);
        free(y);
        free(h);
    }
    return bad ? OR_BAD : OR_OK;
}

/* Number of OpenMP threads the oracle runs on (reported beside its timings). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/*
 * Scoring variants of the router. The Instella page gives its top-k method as
 * "noaux_tc" on a DeepSeek-V3 base (64 routed experts, 6 per token, routed
 * scale 2.5) without defining it; the definition taken is DeepSeek-V3's
 * published router:
 *   score   s[e] = sigmoid(l[e])           (the logit itself for softmax),
 *   key     c[e] = s[e] + bias[e]          (the bias steers selection only),
 *   groups  (n_group = G > 1) G groups of E/G consecutive experts; a group's
 *           score is the sum of its two largest keys (its only key when
 *           E/G = 1); the topk_group best groups are kept (ties to the lower
 *           group) and only their experts may be selected,
 *   top-k   greedy by key, ties to the lower expert index,
 *   weights the selected scores over their sum (sigmoid) or the softmax of
 *           the selected logits (softmax), times the routed scale.
 * Keys decide integers (the ids), so they are computed in fp32 with the
 * operation sequence the library's contract states: clamp to [-80, 80],
 * exp(x) = 2^n e^r with n = rint(x / ln2) and ln2 split into a short high
 * part and a rounded low part, e^r by its degree-8 Taylor polynomial in
 * Horner form with fused multiply-adds, then 1 / (1 + exp(-c)); the key and
 * the group sums (best key first, from 0) are fp32 additions. Weights are
 * evaluated in fp64 from the fp32 scores.
 * Parity unpinned against the pages, which name the rule without defining
 * it; the tests pin these functions to the mathematics (exp and sigmoid
 * against fp64, symmetry, the clamp) and to the published rule's
 * consequences (bias that only moves selection, groups, ties).
 */
static float exp_by_reduction(float x)
{
    const double ln2 = log(2.0);
    const float inv_ln2 = (float)(1.0 / ln2);
    const float ln2_hi = 0.693145751953125f; /* 15 significant bits: n * ln2_hi is exact */
    const float ln2_lo = (float)(ln2 - (double)ln2_hi);
    const float n = rintf(x * inv_ln2);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    double fact[9];
    fact[0] = 1.0;
    for (int j = 1; j <= 8; j++)
        fact[j] = fact[j - 1] * j;
    float p = (float)(1.0 / fact[8]);
    for (int j = 7; j >= 0; j--)
        p = fmaf(p, r, (float)(1.0 / fact[j]));
    return ldexpf(p, (int)n);
}

static float sigmoid_score(float l)
{
    /* fmaxf / fminf return the number when the other operand is NaN: a NaN
       logit scores as -80 */
    const float c = fminf(fmaxf(l, -80.0f), 80.0f);
    return 1.0f / (1.0f + exp_by_reduction(-c));
}

int oracle_exp_f32(const float *x, int64_t n, float *y)
{
    if (!x || !y || n < 0)
        return OR_BAD;
    for (int64_t i = 0; i < n; i++)
        y[i] = exp_by_reduction(x[i]);
    return OR_OK;
}

int oracle_sigmoid_scores(const float *x, int64_t n, float *y)
{
    if (!x || !y || n < 0)
        return OR_BAD;
    for (int64_t i = 0; i < n; i++)
        y[i] = sigmoid_score(x[i]);
    return OR_OK;
}

/* a ranks before b: larger value, then lower index (NaN taken as -inf) */
static int before(float va, int64_t a, float vb, int64_t b)
{
    va = rank_value(va);
    vb = rank_value(vb);
    return va > vb || (va == vb && a < b);
}

int oracle_select_scored(const float *logits, int64_t T, int64_t E, int k, float routed_scale,
                         int score_func, const float *bias, int n_group, int topk_group,
                         int32_t *ids, float *weights)
{
    if (!logits || !ids || !weights || T < 0 || E <= 0 || E > 4096 || k < 1 || k > E || k > 256 ||
        (score_func != 0 && score_func != 1))
        return OR_BAD;
    const int grouped = n_group > 1;
    if (grouped && (E % n_group || topk_group < 1 || topk_group > n_group ||
                    (int64_t)k > (int64_t)topk_group * (E / n_group)))
        return OR_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        float s[4096], key[4096];
        unsigned char allowed[4096];
        for (int64_t e = 0; e < E; e++) {
            s[e] = score_func == 1 ? sigmoid_score(l[e]) : l[e];
            key[e] = bias ? s[e] + bias[e] : s[e];
            allowed[e] = 1;
        }
        if (grouped) {
            const int64_t gsz = E / n_group;
            float gscore[4096];
            for (int g = 0; g < n_group; g++) {
                /* the group's best key, then its best other key */
                int64_t b1 = -1, b2 = -1;
                for (int64_t e = g * gsz; e < (g + 1) * gsz; e++)
                    if (b1 < 0 || before(key[e], e, key[b1], b1))
                        b1 = e;
                for (int64_t e = g * gsz; e < (g + 1) * gsz; e++)
                    if (e != b1 && (b2 < 0 || before(key[e], e, key[b2], b2)))
                        b2 = e;
                float sum = 0.0f + key[b1];
                if (b2 >= 0)
                    sum = sum + key[b2];
                gscore[g] = sum;
            }
            unsigned char kept[4096];
            for (int g = 0; g < n_group; g++)
                kept[g] = 0;
            for (int r = 0; r < topk_group; r++) {
                int best = -1;
                for (int g = 0; g < n_group; g++)
                    if (!kept[g] && (best < 0 || before(gscore[g], g, gscore[best], best)))
                        best = g;
                kept[best] = 1;
            }
            for (int64_t e = 0; e < E; e++)
                allowed[e] = kept[e / gsz];
        }
        for (int j = 0; j < k; j++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++)
                if (allowed[e] && (best < 0 || before(key[e], e, key[best], best)))
                    best = e;
            ids[t * k + j] = (int32_t)best;
            allowed[best] = 0;
        }
        double num[256], den = 0.0;
        if (score_func == 1) {
            for (int j = 0; j < k; j++)
                num[j] = (double)s[ids[t * k + j]];
        } else {
            double m = -INFINITY;
            for (int j = 0; j < k; j++)
                if ((double)l[ids[t * k + j]] > m)
                    m = (double)l[ids[t * k + j]];
            for (int j = 0; j < k; j++)
                num[j] = exp((double)l[ids[t * k + j]] - m);
        }
        for (int j = 0; j < k; j++)
            den += num[j];
        for (int j = 0; j < k; j++)
            weights[t * k + j] = (float)((double)routed_scale * num[j] / den);
    }
    return OR_OK;
}

/*
 * PhiMoE's sparsemixer router at inference (PhiMoE page, section 6: greedy
 * top-1, mask the chosen expert, take the next; each chosen expert's weight
 * comes out of a softmax; config table, section 3: router_jitter_noise 0.01
 * is the epsilon handed to sparsemixer). The page does not print which
 * experts enter each softmax; the published sparsemixer takes, in round j
 * with winner logit m over the experts not chosen before, the experts whose
 * relative gap (m - l[e]) / max(|l[e]|, m) is NOT above 2 * jitter_eps, and
 * the weight is that softmax's value at the winner. k rounds generalise the
 * page's two. The gap test decides membership, so it is taken in fp32 (a
 * 0/0 gap is NaN, which is not above the threshold: the expert stays); the
 * softmax is evaluated in fp64.
 * The membership rule is the published one, not the page's: parity of that
 * detail is unpinned against the pages; the tests pin the page's threshold
 * value, the greedy ids, and the limits (well separated logits, an unbounded
 * threshold giving the textbook softmax).
 */
int oracle_select_sparsemixer(const float *logits, int64_t T, int64_t E, int k, float routed_scale,
                              float jitter_eps, int32_t *ids, float *weights)
{
    if (!logits || !ids || !weights || T < 0 || E <= 0 || E > 4096 || k < 1 || k > E || !(jitter_eps >= 0.0f))
        return OR_BAD;
    const float thr = 2.0f * jitter_eps;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        unsigned char chosen[4096];
        for (int64_t e = 0; e < E; e++)
            chosen[e] = 0;
        for (int j = 0; j < k; j++) {
            int64_t w = -1;
            for (int64_t e = 0; e < E; e++)
                if (!chosen[e] && (w < 0 || before(l[e], e, l[w], w)))
                    w = e;
            const float m = l[w];
            double z = 0.0;
            for (int64_t e = 0; e < E; e++) {
                if (chosen[e])
                    continue;
                const float a = fabsf(l[e]);
                const float gap = (m - l[e]) / (a > m ? a : m);
                if (!(gap > thr))
                    z += exp((double)l[e] - (double)m);
            }
            ids[t * k + j] = (int32_t)w;
            weights[t * k + j] = (float)((double)routed_scale / z);
            chosen[w] = 1;
        }
    }
    return OR_OK;
}

/*
 * MXFP4 expert weights (OCP Microscaling Formats v1.0, MXFP4: the pages' "mxfp4
 * with block scales", the MoEs in Transformers page, sections on why MoEs are
 * fast and on weight loading). Each row of a weight matrix is cut into blocks
 * of 32 consecutive elements sharing one power-of-two factor 2^x, x stored
 * as the E8M0 byte x + 127; each element is an FP4 E2M1 code: bit 3 sign,
 * bits 2..1 exponent field e (bias 1), bit 0 mantissa m; e = 0 gives m * 0.5,
 * otherwise 2^(e-1) * (1 + m/2) -- magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 * Quantisation follows the specification's conversion: x = floor(log2 a) - 2
 * for the block's largest magnitude a (2 = the largest E2M1 exponent),
 * clamped to [-127, 127] (a = 0 or below 2^-126 gives -127); each element
 * becomes the E2M1 value nearest to w / 2^x, ties to the even code (m = 0),
 * magnitudes past 6 saturating to 6; the sign bit is w's. Packing: element 2i
 * in the low nibble of byte i, element 2i+1 in the high nibble.
 */
static double e2m1_value(int code)
{
    const int e = (code >> 1) & 3, m = code & 1;
    const double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (code & 8) ? -v : v;
}

int oracle_e2m1_values(double *out)
{
    if (!out)
        return OR_BAD;
    for (int c = 0; c < 16; c++)
        out[c] = e2m1_value(c);
    return OR_OK;
}

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* x of a block whose largest magnitude is a */
static int mx_block_exponent(double a)
{
    if (!(a >= ldexp(1.0, -126)))
        return -127;
    int x;
    frexp(a, &x); /* a = f * 2^x, f in [0.5, 1): floor(log2 a) = x - 1 */
    int s = x - 1 - 2;
    return s < -127 ? -127 : (s > 127 ? 127 : s);
}

int oracle_quantize_mxfp4_rows(const uint16_t *w, int64_t rows, int64_t cols, uint8_t *q, uint8_t *scale)
{
    if (!w || !q || !scale || rows < 0 || cols <= 0 || cols % 32)
        return OR_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < cols / 32; b++) {
            const uint16_t *blk = w + r * cols + b * 32;
            double a = 0.0;
            for (int i = 0; i < 32; i++)
                a = fmax(a, fabs(bf16_value(blk[i])));
            const int x = mx_block_exponent(a);
            scale[r * (cols / 32) + b] = (uint8_t)(x + 127);
            for (int i = 0; i < 32; i++) {
                const double y = fabs(bf16_value(blk[i])) / ldexp(1.0, x); /* exact in fp64 */
                /* brute force: the nearest of the 8 magnitudes, ties to the even code */
                int best = 0;
                for (int c = 1; c < 8; c++) {
                    const double dc = fabs(y - e2m1_value(c)), db = fabs(y - e2m1_value(best));
                    if (dc < db || (dc == db && (c & 1) == 0))
                        best = c;
                }
                const int code = best | ((blk[i] >> 15) ? 8 : 0);
                uint8_t *dst = q + r * (cols / 2) + b * 16 + i / 2;
                if (i % 2 == 0)
                    *dst = (uint8_t)code;
                else
                    *dst = (uint8_t)(*dst | (code << 4));
            }
        }
    return OR_OK;
}

/* w = e2m1(q) * 2^(scale - 127) as bf16 bits (exact: three significant bits) */
int oracle_dequantize_mxfp4_rows(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols, uint16_t *w)
{
    if (!q || !scale || !w || rows < 0 || cols <= 0 || cols % 32)
        return OR_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t i = 0; i < cols; i++) {
            const uint8_t byte = q[r * (cols / 2) + i / 2];
            const int code = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
            const int x = (int)scale[r * (cols / 32) + i / 32] - 127;
            const float f = (float)(e2m1_value(code) * ldexp(1.0, x));
            uint32_t u;
            memcpy(&u, &f, sizeof u);
            w[r * cols + i] = (uint16_t)(u >> 16);
        }
    return OR_OK;
}
