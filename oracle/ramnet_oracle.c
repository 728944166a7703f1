/*
 * RAM-Net layer recurrence: plain CPU oracle.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The product path (the HIP library and its
 * Python binding) never links, loads or calls it, and it shares no code,
 * header or table with that path.
 *
 * What it computes, and where the pages say so.  "Project page" below is the
 * RAM-Net project page (muoncat.github.io/ramnet_web, "RAM-Net: Linear-Time
 * Sequence Modeling with Sparsely Addressable State"); paragraph names are the
 * topics of its paragraphs, since the extracted text lost the headings.
 *
 *   - Product Softmax (project page, "Product Softmax" and "Soft Radix
 *     Address"): M = d_p^U slots; the logits are split into U blocks of d_p;
 *     a softmax over each block gives one digit's distribution; a slot's
 *     weight is the product of the probabilities of its U digits.
 *   - Top-K (project page, "exact Top-K" paragraph after "Waveform
 *     Modulation"; AI Radio episode: "Top-K truncation"): the K heaviest
 *     slots.  The plain definition (score all M, keep the K best) is the
 *     authority; the level-by-level prefix search is a second, separately
 *     written routine that the tests check against it.
 *   - CAPE (project page, "Cyclic Address Positional Embedding"): addresses
 *     are moved along the slot array by the token position, cyclically; the
 *     move only permutes slot indices.
 *   - Gated Sparse Update (project page, "Gated Sparse Update", four steps):
 *     retention, mass, rate, content, for the addressed slots only.
 *   - Read (project page, "three stages"): the read slots are combined by
 *     their weights, normalized and gated.
 *
 * Readings taken where the pages leave a step open (each also in the design
 * notes): block u is digit u counted from the most significant; weights are
 * the raw products (no renormalisation); ties go to the smaller slot index;
 * CAPE adds (P mod d_p) to every digit, cyclically in d_p; retention is
 * alpha = (1 - w)^(exp(gamma)) (the "power decay" of the AI Radio episode);
 * lambda = w / (m + eps) with the stored mass; all K writes of a token happen
 * before its read; RMSNorm over d_v with eps_norm; the gate is sigmoid(g).
 *
 * Arithmetic is fp64.  Storage follows the layer's dtypes: slot content S and
 * the output are rounded to the state dtype (fp32 or bf16, nearest-even) every
 * time they are stored, the mass to fp32; every read uses the stored value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_VERSION 1

int oracle_version(void) { return ORACLE_VERSION; }

/* ------------------------------------------------------------------ */
/* Storage rounding                                                   */
/* ------------------------------------------------------------------ */

/* Nearest fp32 value (ties to even: C's conversion in the default mode). */
static double store_f32(double x) { return (double)(float)x; }

/* Nearest bf16 value (8 significant bits, fp32 exponent range), ties to even,
 * rounded once from the fp64 value. */
static double store_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);                        /* |x| in [2^(e-1), 2^e) */
    int qexp = e - 8;                    /* spacing of 8-bit significands */
    if (qexp < -133) qexp = -133;        /* bf16 subnormal spacing 2^-133 */
    double q = ldexp(1.0, qexp);
    double r = rint(x / q) * q;          /* exact scaling by a power of two */
    const double bf16_max = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > bf16_max) r = copysign(INFINITY, x);
    return r;
}

static double store_state(int bf16, double x) {
    return bf16 ? store_bf16(x) : store_f32(x);
}

double oracle_round_bf16(double x) { return store_bf16(x); }

/* ------------------------------------------------------------------ */
/* Product Softmax                                                    */
/* ------------------------------------------------------------------ */

static long ipow_l(int base, int e) {
    long p = 1;
    for (int i = 0; i < e; i++) p *= base;
    return p;
}

/* Softmax over each of the U blocks of d_p logits (max subtracted).
 * probs[u*d_p + a] is the probability that digit u takes value a.
 * Adds the number of exponentials evaluated to *n_exp when given. */
static void digit_softmax(const float *logits, int U, int d_p, double *probs,
                          long *n_exp) {
    for (int u = 0; u < U; u++) {
        const float *l = logits + (long)u * d_p;
        double mx = l[0];
        for (int a = 1; a < d_p; a++)
            if (l[a] > mx) mx = l[a];
        double sum = 0.0;
        for (int a = 0; a < d_p; a++) {
            double e = exp((double)l[a] - mx);
            probs[u * d_p + a] = e;
            sum += e;
        }
        for (int a = 0; a < d_p; a++) probs[u * d_p + a] /= sum;
        if (n_exp) *n_exp += d_p;
    }
}

/* Digit u of slot i in base d_p; u = 0 is the most significant digit, so the
 * last block changes fastest along the slot index (project page, "Waveform
 * Modulation": low-order digits change at every slot). */
static int digit_of(long i, int u, int U, int d_p) {
    long place = ipow_l(d_p, U - 1 - u);
    return (int)((i / place) % d_p);
}

/* Weight of slot i: product of its digit probabilities, multiplied from the
 * most significant digit down (the tree's root-to-leaf order). */
static double slot_weight(const double *probs, long i, int U, int d_p) {
    double w = 1.0;
    for (int u = 0; u < U; u++) w *= probs[u * d_p + digit_of(i, u, U, d_p)];
    return w;
}

/* Heavier first; equal weights: smaller index first. */
static int ranks_before(double wa, long ia, double wb, long ib) {
    return wa > wb || (wa == wb && ia < ib);
}

/* All M slot weights for one address (test helper). */
int oracle_slot_weights(const float *logits, int U, int d_p, double *W) {
    if (U < 1 || d_p < 2) return -1;
    double *probs = (double *)malloc(sizeof(double) * U * d_p);
    if (!probs) return -2;
    digit_softmax(logits, U, d_p, probs, NULL);
    long M = ipow_l(d_p, U);
    for (long i = 0; i < M; i++) W[i] = slot_weight(probs, i, U, d_p);
    free(probs);
    return 0;
}

int oracle_digit_probs(const float *logits, int U, int d_p, double *probs,
                       long *n_exp) {
    if (U < 1 || d_p < 2) return -1;
    digit_softmax(logits, U, d_p, probs, n_exp);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Top-K                                                              */
/* ------------------------------------------------------------------ */

/* Plain definition: score every slot and keep the K that rank first.
 * idx/wt receive the K slots in rank order.  gap (if given) receives
 * (W_K - W_{K+1}) / W_K, the relative margin between the K-th and the
 * (K+1)-th weight: +inf when K = M, 0 when W_K = 0. */
static int topk_brute(const double *probs, int U, int d_p, int K, int32_t *idx,
                      double *wt, double *gap) {
    long M = ipow_l(d_p, U);
    if (K < 1 || K > M) return -1;
    int cap = K + 1;                       /* keep one extra for the gap */
    double *bw = (double *)malloc(sizeof(double) * cap);
    long *bi = (long *)malloc(sizeof(long) * cap);
    if (!bw || !bi) { free(bw); free(bi); return -2; }
    int n = 0;
    for (long i = 0; i < M; i++) {
        double w = slot_weight(probs, i, U, d_p);
        if (n == cap && !ranks_before(w, i, bw[n - 1], bi[n - 1])) continue;
        int p = (n < cap) ? n++ : n - 1;   /* slot to overwrite */
        while (p > 0 && ranks_before(w, i, bw[p - 1], bi[p - 1])) {
            bw[p] = bw[p - 1];
            bi[p] = bi[p - 1];
            p--;
        }
        bw[p] = w;
        bi[p] = i;
    }
    for (int j = 0; j < K; j++) {
        idx[j] = (int32_t)bi[j];
        wt[j] = bw[j];
    }
    if (gap) {
        if (K == M) *gap = INFINITY;
        else if (bw[K - 1] == 0.0) *gap = 0.0;
        else *gap = (bw[K - 1] - bw[K]) / bw[K - 1];
    }
    free(bw);
    free(bi);
    return 0;
}

typedef struct { double w; long prefix; } cand_t;

static int cand_cmp(const void *pa, const void *pb) {
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (ranks_before(a->w, a->prefix, b->w, b->prefix)) return -1;
    if (ranks_before(b->w, b->prefix, a->w, a->prefix)) return 1;
    return 0;
}

/* Level-by-level prefix search (project page, "Multilevel Decision Tree" and
 * the exact Top-K paragraph): fix one digit per level, most significant
 * first; at each level extend every kept partial address by the d_p values of
 * the next digit and keep the K best partial addresses.  cand_per_level[u]
 * (if given) receives the number of candidates scored at level u. */
static int topk_tree(const double *probs, int U, int d_p, int K, int32_t *idx,
                     double *wt, long *cand_per_level) {
    long M = ipow_l(d_p, U);
    if (K < 1 || K > M) return -1;
    cand_t *beam = (cand_t *)malloc(sizeof(cand_t) * K);
    cand_t *cand = (cand_t *)malloc(sizeof(cand_t) * (size_t)K * d_p);
    if (!beam || !cand) { free(beam); free(cand); return -2; }
    int nb = 1;
    beam[0].w = 1.0;
    beam[0].prefix = 0;
    for (int u = 0; u < U; u++) {
        int nc = 0;
        for (int e = 0; e < nb; e++)
            for (int a = 0; a < d_p; a++) {
                cand[nc].w = beam[e].w * probs[u * d_p + a];
                cand[nc].prefix = beam[e].prefix * d_p + a;
                nc++;
            }
        if (cand_per_level) cand_per_level[u] = nc;
        qsort(cand, nc, sizeof(cand_t), cand_cmp);
        nb = nc < K ? nc : K;
        memcpy(beam, cand, sizeof(cand_t) * nb);
    }
    for (int j = 0; j < K; j++) {
        idx[j] = (int32_t)beam[j].prefix;
        wt[j] = beam[j].w;
    }
    free(beam);
    free(cand);
    return 0;
}

/* ------------------------------------------------------------------ */
/* CAPE                                                               */
/* ------------------------------------------------------------------ */

/* Move slot i by token position P (project page, CAPE: addresses shift
 * cyclically along the slot array with the position).  The pages leave the
 * exact shift open; three readings, each a permutation of the M slots:
 *   form 1 (A): every digit advances by (P mod d_p), wrapping within its d_p
 *               values;
 *   form 2 (B): digit u advances by digit u of P written in base d_p (most
 *               significant first, U digits), each wrapping on its own (no
 *               carry);
 *   form 3 (C): the slot index advances by P, wrapping over all M slots. */
static long cape_move(long i, long P, int U, int d_p, int form) {
    const long M = ipow_l(d_p, U);
    if (form == 3) return (long)((((unsigned long)i + (unsigned long)(((P % M) + M) % M))) % (unsigned long)M);
    long j = 0;
    for (int u = 0; u < U; u++) {
        long a = digit_of(i, u, U, d_p);
        long s;
        if (form == 2)
            s = digit_of(((P % M) + M) % M, u, U, d_p);
        else
            s = ((P % d_p) + d_p) % d_p;
        j = j * d_p + (a + s) % d_p;
    }
    return j;
}

int oracle_cape(const int32_t *idx, long n, long P, int U, int d_p, int form,
                int32_t *out) {
    if (form < 1 || form > 3) return -1;
    for (long j = 0; j < n; j++) out[j] = (int32_t)cape_move(idx[j], P, U, d_p, form);
    return 0;
}

/* CAPE form a head uses: 0 (content-only) when its bit of content_heads is
 * set (heads 63 and above share bit 63), else `cape`. */
static int head_cape(int cape, uint64_t content_heads, long h) {
    const int bit = h < 63 ? (int)h : 63;
    return ((content_heads >> bit) & 1u) ? 0 : cape;
}

/* ------------------------------------------------------------------ */
/* One address: softmax -> Top-K -> CAPE                              */
/* ------------------------------------------------------------------ */

enum { TOPK_BRUTE = 0, TOPK_TREE = 1 };

/* Decodes one key or query.  idx receives post-CAPE slots (CAPE applied when
 * cape != 0), in the rank order of their content indices; wt the raw product
 * weights; gap the brute-force margin (NaN in tree mode). */
static int decode_one(const float *logits, int U, int d_p, int K, int mode,
                      int cape, long P, double *probs, int32_t *idx,
                      double *wt, double *gap, long *n_exp, long *cand) {
    digit_softmax(logits, U, d_p, probs, n_exp);
    int rc;
    if (mode == TOPK_TREE) {
        rc = topk_tree(probs, U, d_p, K, idx, wt, cand);
        if (gap) *gap = NAN;
    } else {
        rc = topk_brute(probs, U, d_p, K, idx, wt, gap);
    }
    if (rc) return rc;
    if (cape)
        for (int j = 0; j < K; j++) idx[j] = (int32_t)cape_move(idx[j], P, U, d_p, cape);
    return 0;
}

int oracle_decode_one(const float *logits, int U, int d_p, int K, int mode,
                      int cape, long P, int32_t *idx, double *wt, double *gap,
                      long *n_exp, long *cand_per_level) {
    if (U < 1 || d_p < 2 || K < 1 || K > ipow_l(d_p, U) || cape < 0 || cape > 3) return -1;
    double *probs = (double *)malloc(sizeof(double) * U * d_p);
    if (!probs) return -2;
    int rc = decode_one(logits, U, d_p, K, mode, cape, P, probs, idx, wt, gap,
                        n_exp, cand_per_level);
    free(probs);
    return rc;
}

/* Decodes every address of a [B,T,H,U*d_p] logit tensor at positions
 * pos0[b] + t (pos0 NULL means 0).  idx/wt are [B,T,H,K], gap [B,T,H]. */
int oracle_decode_all(int B, int T, int H, int U, int d_p, int K, int mode,
                      int cape, uint64_t content_heads, const int32_t *pos0,
                      const float *logits, int32_t *idx, double *wt,
                      double *gap, int nthreads) {
    long M = ipow_l(d_p, U);
    if (B < 0 || T < 0 || H < 0 || U < 1 || d_p < 2 || K < 1 || K > M || cape < 0 ||
        cape > 3)
        return -1;
    long n = (long)B * T * H;
    int L = U * d_p;
    int rc_all = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *probs = (double *)malloc(sizeof(double) * L);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (long a = 0; a < n; a++) {
            long b = a / ((long)T * H);
            long t = (a / H) % T;
            long P = (pos0 ? pos0[b] : 0) + t;
            int rc = decode_one(logits + a * L, U, d_p, K, mode,
                                head_cape(cape, content_heads, a % H), P, probs,
                                idx + a * K, wt + a * K, gap ? gap + a : NULL,
                                NULL, NULL);
            if (rc) rc_all = rc;
        }
        free(probs);
    }
    return rc_all;
}

/* ------------------------------------------------------------------ */
/* Gated Sparse Update, read, norm, gate                              */
/* ------------------------------------------------------------------ */

/* Retention of a slot written with weight w at a token with gate gamma
 * (project page, GSU step 1; AI Radio: "Power Decay Moving Average"):
 * alpha = (1 - w)^(exp(gamma)).  Smaller for a stronger write and for a
 * larger gamma; 1 as gamma -> -inf; 0 as gamma -> +inf; 0 at w = 1. */
static double retention(double w, double gamma) {
    if (w >= 1.0) return 0.0;
    return exp(exp(gamma) * log1p(-w));
}

typedef struct {
    int T, H, M_is_set;
    int U, d_p, K, d_v;
    long M;
    int state_bf16, cape, topk_mode;
    double eps_gsu, eps_norm;
} layer_cfg;

/* The recurrence of one (batch, head) unit over T tokens.
 *   addresses: either decoded here from q/k logits (q, k non-NULL), or taken
 *   as given from gw_idx/gw_wt/gr_idx/gr_wt (post-CAPE slots).
 * Pointers address the unit's first element; token stride is H*width. */
static int run_unit(const layer_cfg *c, long P0,
                    const float *q, const float *k,
                    const int32_t *gw_idx, const double *gw_wt,
                    const int32_t *gr_idx, const double *gr_wt,
                    const float *v, const float *gamma, const float *g,
                    const float *norm_w, float *S, float *mass, float *out,
                    int32_t *ow_idx, double *ow_wt, int32_t *or_idx,
                    double *or_wt, double *ow_gap, double *or_gap) {
    const int K = c->K, d_v = c->d_v, H = c->H, U = c->U, d_p = c->d_p;
    const int L = U * d_p;
    double *probs = (double *)malloc(sizeof(double) * L);
    int32_t *wi = (int32_t *)malloc(sizeof(int32_t) * K);
    int32_t *ri = (int32_t *)malloc(sizeof(int32_t) * K);
    double *ww = (double *)malloc(sizeof(double) * K);
    double *rw = (double *)malloc(sizeof(double) * K);
    double *r = (double *)malloc(sizeof(double) * d_v);
    int rc = 0;
    if (!probs || !wi || !ri || !ww || !rw || !r) { rc = -2; goto done; }

    for (int t = 0; t < c->T; t++) {
        const long P = P0 + t;
        const long th = (long)t * H;   /* token-head offset from the unit's origin */
        double wgap = NAN, rgap = NAN;

        /* Stage 1 + 2: addresses for this token. */
        if (q && k) {
            rc = decode_one(k + th * L, U, d_p, K, c->topk_mode, c->cape, P,
                            probs, wi, ww, &wgap, NULL, NULL);
            if (!rc)
                rc = decode_one(q + th * L, U, d_p, K, c->topk_mode, c->cape, P,
                                probs, ri, rw, &rgap, NULL, NULL);
            if (rc) goto done;
        } else {
            for (int j = 0; j < K; j++) {
                wi[j] = gw_idx[th * K + j];
                ww[j] = gw_wt[th * K + j];
                ri[j] = gr_idx[th * K + j];
                rw[j] = gr_wt[th * K + j];
            }
        }

        /* Stage 3: Gated Sparse Update of the K write slots. */
        const double gm = gamma[th];
        const float *vt = v + th * d_v;
        for (int j = 0; j < K; j++) {
            const double w = ww[j];
            if (!(w > 0.0)) continue;       /* w = 0: alpha = 1, lambda = 0 */
            const long i = wi[j];
            const double alpha = retention(w, gm);                 /* step 1 */
            const double m = store_f32(alpha * (double)mass[i] + w); /* step 2 */
            mass[i] = (float)m;
            const double lam = w / (m + c->eps_gsu);               /* step 3 */
            float *Si = S + i * d_v;
            for (int ch = 0; ch < d_v; ch++) {                      /* step 4 */
                const double s = Si[ch];
                Si[ch] = (float)store_state(c->state_bf16,
                                            s + lam * ((double)vt[ch] - s));
            }
        }

        /* Read: the K read slots combined by their weights (stored values). */
        for (int ch = 0; ch < d_v; ch++) r[ch] = 0.0;
        for (int j = 0; j < K; j++) {
            const float *Sj = S + (long)ri[j] * d_v;
            for (int ch = 0; ch < d_v; ch++) r[ch] += rw[j] * (double)Sj[ch];
        }

        /* RMSNorm over d_v, then the sigmoid output gate. */
        double ms = 0.0;
        for (int ch = 0; ch < d_v; ch++) ms += r[ch] * r[ch];
        ms /= d_v;
        /* An all-zero read with eps_norm = 0 is 0/0; its output is taken as
         * zero, the value every eps_norm > 0 gives for a zero read. */
        const double den = ms + c->eps_norm;
        const double inv = den > 0.0 ? 1.0 / sqrt(den) : 0.0;
        const float *gt = g + th * d_v;
        float *ot = out + th * d_v;
        for (int ch = 0; ch < d_v; ch++) {
            const double om = norm_w ? (double)norm_w[ch] : 1.0;
            const double gate = 1.0 / (1.0 + exp(-(double)gt[ch]));
            ot[ch] = (float)store_state(c->state_bf16, r[ch] * inv * om * gate);
        }

        if (ow_idx) for (int j = 0; j < K; j++) ow_idx[th * K + j] = wi[j];
        if (ow_wt) for (int j = 0; j < K; j++) ow_wt[th * K + j] = ww[j];
        if (or_idx) for (int j = 0; j < K; j++) or_idx[th * K + j] = ri[j];
        if (or_wt) for (int j = 0; j < K; j++) or_wt[th * K + j] = rw[j];
        if (ow_gap) ow_gap[th] = wgap;
        if (or_gap) or_gap[th] = rgap;
    }
done:
    free(probs); free(wi); free(ri); free(ww); free(rw); free(r);
    return rc;
}

static int check_cfg(int B, int T, int H, int d_p, int U, int K, int d_v) {
    if (B < 0 || T < 0 || H < 0 || d_p < 2 || U < 1 || d_v < 1) return -1;
    long M = ipow_l(d_p, U);
    if (M > (1L << 30) || K < 1 || K > M) return -1;
    return 0;
}

/* Shared driver: units (b, h) are independent and run in parallel. */
static int layer_driver(int B, int T, int H, int d_p, int U, int K, int d_v,
                        int state_bf16, int cape, uint64_t content_heads, double eps_gsu,
                        double eps_norm, int topk_mode,
                        const float *q, const float *k,
                        const int32_t *gw_idx, const double *gw_wt,
                        const int32_t *gr_idx, const double *gr_wt,
                        const float *v, const float *gamma, const float *g,
                        const float *norm_w, const int32_t *pos0, float *S,
                        float *mass, float *out, int32_t *w_idx, double *w_wt,
                        int32_t *r_idx, double *r_wt, double *w_gap,
                        double *r_gap, int nthreads) {
    if (check_cfg(B, T, H, d_p, U, K, d_v) || cape < 0 || cape > 3) return -1;
    layer_cfg c;
    memset(&c, 0, sizeof c);
    c.T = T; c.H = H; c.U = U; c.d_p = d_p; c.K = K; c.d_v = d_v;
    c.M = ipow_l(d_p, U);
    c.state_bf16 = state_bf16; c.cape = cape; c.topk_mode = topk_mode;
    c.eps_gsu = eps_gsu; c.eps_norm = eps_norm;
    const int L = U * d_p;
    const long units = (long)B * H;
    int rc_all = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (long uidx = 0; uidx < units; uidx++) {
        const long b = uidx / H, h = uidx % H;
        const long o = b * T * H + h;             /* first token-head of unit */
        const long P0 = pos0 ? pos0[b] : 0;
        layer_cfg cu = c;
        cu.cape = head_cape(cape, content_heads, h);
        int rc = run_unit(&cu, P0,
                          q ? q + o * L : NULL, k ? k + o * L : NULL,
                          gw_idx ? gw_idx + o * K : NULL,
                          gw_wt ? gw_wt + o * K : NULL,
                          gr_idx ? gr_idx + o * K : NULL,
                          gr_wt ? gr_wt + o * K : NULL,
                          v + o * d_v, gamma + o, g + o * d_v, norm_w,
                          S + uidx * c.M * d_v, mass + uidx * c.M,
                          out + o * d_v,
                          w_idx ? w_idx + o * K : NULL,
                          w_wt ? w_wt + o * K : NULL,
                          r_idx ? r_idx + o * K : NULL,
                          r_wt ? r_wt + o * K : NULL,
                          w_gap ? w_gap + o : NULL, r_gap ? r_gap + o : NULL);
        if (rc) rc_all = rc;
    }
    return rc_all;
}

/* The layer over [B,T,H]: decode both addresses of every token, then the
 * recurrence.  Layouts (contiguous, row-major):
 *   q, k [B,T,H,U*d_p]; v, g, out [B,T,H,d_v]; gamma [B,T,H];
 *   S [B,H,M,d_v] and mass [B,H,M], updated in place; norm_w [d_v] or NULL;
 *   pos0 [B] or NULL (position of token t is pos0[b] + t).
 * Optional outputs (NULL to skip): the post-CAPE addresses used,
 *   w_idx/w_wt/r_idx/r_wt [B,T,H,K], and the Top-K margins w_gap/r_gap
 *   [B,T,H] (brute mode only).
 * Returns 0, or a negative code for bad sizes / allocation failure. */
int oracle_layer(int B, int T, int H, int d_p, int U, int K, int d_v,
                 int state_bf16, int cape, uint64_t content_heads,
                 double eps_gsu, double eps_norm,
                 int topk_mode, const float *q, const float *k, const float *v,
                 const float *gamma, const float *g, const float *norm_w,
                 const int32_t *pos0, float *S, float *mass, float *out,
                 int32_t *w_idx, double *w_wt, int32_t *r_idx, double *r_wt,
                 double *w_gap, double *r_gap, int nthreads) {
    if (!q || !k) return -1;
    return layer_driver(B, T, H, d_p, U, K, d_v, state_bf16, cape, content_heads,
                        eps_gsu, eps_norm, topk_mode, q, k, NULL, NULL, NULL, NULL, v,
                        gamma, g, norm_w, pos0, S, mass, out, w_idx, w_wt,
                        r_idx, r_wt, w_gap, r_gap, nthreads);
}

/* The recurrence with the addresses given (post-CAPE slots and weights,
 * [B,T,H,K] each); no decoding and no CAPE.  Used by tests that construct
 * write/read patterns directly. */
int oracle_scan_given(int B, int T, int H, int d_p, int U, int K, int d_v,
                      int state_bf16, double eps_gsu, double eps_norm,
                      const int32_t *w_idx, const double *w_wt,
                      const int32_t *r_idx, const double *r_wt,
                      const float *v, const float *gamma, const float *g,
                      const float *norm_w, float *S, float *mass, float *out,
                      int nthreads) {
    if (!w_idx || !w_wt || !r_idx || !r_wt) return -1;
    long M = ipow_l(d_p, U);
    long n = (long)B * T * H * K;
    for (long j = 0; j < n; j++)
        if (w_idx[j] < 0 || w_idx[j] >= M || r_idx[j] < 0 || r_idx[j] >= M)
            return -1;
    return layer_driver(B, T, H, d_p, U, K, d_v, state_bf16, 0, 0, eps_gsu,
                        eps_norm, TOPK_BRUTE, NULL, NULL, w_idx, w_wt, r_idx,
                        r_wt, v, gamma, g, norm_w, NULL, S, mass, out, NULL,
                        NULL, NULL, NULL, NULL, NULL, nthreads);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
