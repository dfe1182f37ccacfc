/*
 * kve_oracle.c -- plain CPU oracle of the per-token KV-cache eviction step.
 *
 * TEST INFRASTRUCTURE ONLY (see kve_oracle.h).  Written for clarity, not
 * speed: double-precision logits and softmax, one loop per step of the
 * method, no blocking, no fusion, no reordering.  Build with
 * -ffp-contract=off so that every float operation written below is rounded
 * on its own, as the comments say.
 *
 * Page abbreviations used in the comments:
 *   [KF] "veloxquant_mlx.quantizers.keyformer module"
 *   [PK] "PyramidKV -- Layer-Adaptive Budget Attention-Mass Eviction"
 */
#include "kve_oracle.h"

#include <math.h>
#include <stddef.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE binary16 conversions, written from the format's definition:         */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds */
/* zero and the subnormals (fraction * 2^-24); exponent 31 holds inf / NaN.  */
/* ------------------------------------------------------------------------ */

float oracle_f16_to_f32(uint16_t h)
{
    /* Every binary16 value is a binary32 value, so the result is exact.      */
    /* Normal numbers (1.f) * 2^(e-15) keep their fraction bits (shifted to   */
    /* the top of binary32's 23) under the exponent re-biased from 15 to 127; */
    /* zero and the subnormals f * 2^-24 are an integer times a power of two, */
    /* exact in binary32; exponent 31 is infinity (f = 0) or NaN.             */
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t e = (h >> 10) & 0x1f;
    uint32_t f = h & 0x3ff;
    uint32_t bits;
    if (e == 0x1f) {
        bits = sign | 0x7f800000u | (f << 13);          /* inf / NaN          */
    } else if (e == 0) {
        float m = (float)f * 0x1p-24f;                  /* zero or subnormal  */
        memcpy(&bits, &m, sizeof bits);
        bits |= sign;
    } else {
        bits = sign | ((e - 15 + 127) << 23) | (f << 13);
    }
    float out;
    memcpy(&out, &bits, sizeof out);
    return out;
}

/* Round a binary32 value to the nearest binary16 value, ties to even.
 * The value is exact in double; the binary16 grid spacing at magnitude
 * |x| in [2^E, 2^(E+1)) is 2^(E-10) (E >= -14), and 2^-24 below 2^-14.
 * Scaling by a power of two is exact, and rint() rounds half to even. */
uint16_t oracle_f32_to_f16(float f)
{
    double x = (double)f;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7e00);
    if (isinf(a)) return (uint16_t)(sign | 0x7c00);
    if (a == 0.0) return sign;

    int E;
    frexp(a, &E);          /* a = m * 2^E with m in [0.5, 1)  ->  a in [2^(E-1), 2^E) */
    E -= 1;                /* now a in [2^E, 2^(E+1))                                 */
    if (E < -14) E = -14;  /* subnormal range shares the spacing of the lowest binade */
    double q = ldexp(1.0, E - 10);
    double r = rint(a / q) * q;         /* nearest multiple of the spacing, ties even */
    if (r > 65504.0) return (uint16_t)(sign | 0x7c00);  /* beyond the largest finite: inf */
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -14)) {                          /* subnormal result */
        long m = lrint(r / ldexp(1.0, -24));
        return (uint16_t)(sign | (uint16_t)m);
    }
    int Er;
    frexp(r, &Er);
    Er -= 1;                                            /* r in [2^Er, 2^(Er+1)) */
    long m = lrint(r / ldexp(1.0, Er - 10));            /* 1024..2047 */
    return (uint16_t)(sign | (uint16_t)((Er + 15) << 10) | (uint16_t)(m - 1024));
}

/* ------------------------------------------------------------------------ */
/* Frozen Gumbel noise.  [KF] THE HONESTY CRUX, item 2, and KeyformerState   */
/* (gumbel, pos, seed): one deterministic value per inserted token, derived  */
/* from a base seed and the head's running position, drawn once and never   */
/* redrawn.  [KF] keyformer_update_batched: each B*H row has its own stream. */
/* The pages do not name the generator.  Reading taken: the SplitMix64       */
/* output function (Steele, Lea & Flood 2014) chained over (seed, hh, pos),  */
/* 53 high bits to a uniform strictly inside (0,1), then the standard Gumbel */
/* inverse CDF  g = -log(-log u)  in double, rounded once to float.          */
/* ------------------------------------------------------------------------ */

uint64_t oracle_splitmix64_mix(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t oracle_splitmix64_next(uint64_t *state)
{
    uint64_t out = oracle_splitmix64_mix(*state);
    *state += 0x9E3779B97F4A7C15ULL;
    return out;
}

double oracle_gumbel_uniform(uint64_t seed, int64_t hh, int64_t pos)
{
    uint64_t h = oracle_splitmix64_mix(seed);
    h = oracle_splitmix64_mix(h ^ (uint64_t)hh);
    h = oracle_splitmix64_mix(h ^ (uint64_t)pos);
    /* (integer in [0, 2^53) + 1/2) / 2^53 : never 0, never 1 */
    return ((double)(h >> 11) + 0.5) * ldexp(1.0, -53);
}

float oracle_gumbel(uint64_t seed, int64_t hh, int64_t pos)
{
    double u = oracle_gumbel_uniform(seed, hh, pos);
    return (float)(-log(-log(u)));
}

/* ------------------------------------------------------------------------ */
/* Annealed temperature.  [KF] FIXED GAP #1 and KeyformerState (tau_init,   */
/* tau_end, anneal_steps): tau = tau_init + min(pos, T) * delta_tau with     */
/* delta_tau = (tau_end - tau_init) / T; constant tau_init when T == 0 or    */
/* tau_init == tau_end.  `pos` is the running position of the token being   */
/* inserted by this step (tau equals tau_init at pos 0).  Computed in double */
/* and rounded to float once.                                                */
/* ------------------------------------------------------------------------ */

float oracle_tau(double tau_init, double tau_end, int32_t anneal_steps, int64_t pos)
{
    if (anneal_steps <= 0 || tau_init == tau_end) return (float)tau_init;
    int64_t t = pos < (int64_t)anneal_steps ? pos : (int64_t)anneal_steps;
    double delta = (tau_end - tau_init) / (double)anneal_steps;
    return (float)(tau_init + (double)t * delta);
}

/* ------------------------------------------------------------------------ */
/* [PK] The budget schedule: a linear taper from a largest budget at layer 0 */
/* to a smallest at the last layer, centred so that the mean is avg_budget,  */
/* every entry floored at n_sink + 1; beta = 1 is flat; beta < 1 is an       */
/* error ([PK] Evidence).  Reading taken for the end points: the smallest is */
/* (2 - beta) * avg floored at n_sink + 1, the largest mirrors it about avg. */
/* This reproduces the page's 12-layer example exactly.  Entries are rounded */
/* to the nearest integer, halves to even.  One layer keeps avg; zero layers */
/* give an empty schedule.                                                   */
/* ------------------------------------------------------------------------ */

int oracle_pyramid_budgets(int32_t n_layers, int32_t avg_budget, int32_t n_sink,
                           double beta, int32_t *out)
{
    if (n_layers < 0 || n_sink < 0 || !(beta >= 1.0)) return -1;
    if (avg_budget < n_sink + 1) return -1;
    if (n_layers == 0) return 0;
    if (out == NULL) return -1;
    if (n_layers == 1) { out[0] = avg_budget; return 0; }

    double floor_b = (double)(n_sink + 1);
    double lo = (2.0 - beta) * (double)avg_budget;
    if (lo < floor_b) lo = floor_b;
    double hi = 2.0 * (double)avg_budget - lo;
    for (int32_t l = 0; l < n_layers; ++l) {
        double x = hi + ((lo - hi) * (double)l) / (double)(n_layers - 1);
        double r = rint(x);
        if (r < floor_b) r = floor_b;
        out[l] = (int32_t)r;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RoPE remap.  [KF] FIXED GAP #2 and KeyformerState (positions, rope_base): */
/* a key stored at position p and moved to position q is de-rotated and      */
/* re-rotated, which is one rotation by delta = q - p.  [KF] FUSED METAL     */
/* KERNEL: the rotation is done in fp32 on fp16 storage.  Readings taken:    */
/* the half-split pairing (element j with element j + d/2) and frequency     */
/* base^(-2j/d); the angle delta * freq and its cosine and sine in double,   */
/* each rounded to float; every fp32 product and sum rounded on its own (no  */
/* fused multiply-add); the result rounded to fp16, ties to even.            */
/* ------------------------------------------------------------------------ */

void oracle_rope_rotate(uint16_t *row, int32_t d, int64_t delta, double base)
{
    int32_t half = d / 2;
    for (int32_t j = 0; j < half; ++j) {
        double freq = pow(base, -(2.0 * (double)j) / (double)d);
        double theta = (double)delta * freq;
        float c = (float)cos(theta);
        float s = (float)sin(theta);
        float x1 = oracle_f16_to_f32(row[j]);
        float x2 = oracle_f16_to_f32(row[j + half]);
        float a = x1 * c;
        float b = x2 * s;
        float y1 = a - b;
        float e = x2 * c;
        float f = x1 * s;
        float y2 = e + f;
        row[j] = oracle_f32_to_f16(y1);
        row[j + half] = oracle_f32_to_f16(y2);
    }
}

/* ------------------------------------------------------------------------ */
/* One token through one cache.                                             */
/* ------------------------------------------------------------------------ */

static void copy_row(uint16_t *dst, const uint16_t *src, int32_t d)
{
    for (int32_t j = 0; j < d; ++j) dst[j] = src[j];
}

int oracle_step(oracle_cache *c, const uint16_t *k, const uint16_t *v,
                const oracle_params *prm, double min_margin_rel,
                int32_t *evicted, double *margin)
{
    const int32_t d = c->d;
    const int32_t n = c->n;            /* rows stored before this token */
    /* [KF] init_keyformer_state: the protected rows (sinks and the recent   */
    /* window) must leave room to evict within the budget.                    */
    if (d <= 0 || (d & 1) || n < 0 || prm->n_sink < 0 || prm->recent < 0 ||
        prm->budget <= prm->n_sink + prm->recent ||
        c->cap < prm->budget + 1 || n > prm->budget || n + 1 > c->cap)
        return -1;

    /* 1. Proxy attention.  [KF] keyformer_update step 1 and THE HONESTY     */
    /*    CRUX item 1; [PK] How it works steps 1-2: the incoming key is the  */
    /*    query, softmax(K_stored . k / sqrt(d)) over every row stored before */
    /*    this token (sinks included), and that mass is added to each row's  */
    /*    cumulative score.  Logits, max, exponentials and the normaliser in  */
    /*    double; each row's increment rounded to float once, then added to   */
    /*    the float score.                                                    */
    double *x = c->work;
    double *w = c->work + c->cap;
    if (n > 0) {
        double q[512];                  /* the query (the incoming key) */
        if (d > 512) return -1;
        for (int32_t j = 0; j < d; ++j) q[j] = (double)oracle_f16_to_f32(k[j]);
        double scale = sqrt((double)d);
        double mx = -INFINITY;
        for (int32_t i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < d; ++j)
                acc += (double)oracle_f16_to_f32(c->k[(size_t)i * d + j]) * q[j];
            x[i] = acc / scale;
            if (x[i] > mx) mx = x[i];
        }
        double z = 0.0;
        for (int32_t i = 0; i < n; ++i) {
            w[i] = exp(x[i] - mx);
            z += w[i];
        }
        /* TOVA-adapted ([PK] table of eviction axes): the score is the        */
        /* current step's weight alone.                                        */
        for (int32_t i = 0; i < n; ++i) {
            float inc = (float)(w[i] / z);
            c->snew[i] = prm->current_score ? inc : c->s[i] + inc;
        }
    }

    /* 2. The new row: cumulative score 0, its absolute position next_pos,   */
    /*    and its frozen Gumbel value.  [KF] keyformer_update step 2;         */
    /*    [PK] How it works step 2 (new tokens start at 0).                   */
    c->snew[n] = 0.0f;
    float g_new = prm->use_gumbel ? oracle_gumbel(prm->seed, prm->hh, c->pos) : 0.0f;

    /* 3. Over budget: evict the non-protected row with the smallest         */
    /*    score + tau * gumbel; at tau == 0 (and for PyramidKV, which carries */
    /*    no noise) the key is the raw score.  Protected: the n_sink leading  */
    /*    rows and the `recent` trailing rows of the n + 1 rows after the     */
    /*    append, so the new row is a candidate only when recent == 0.        */
    /*    [KF] keyformer_update step 3, KeyformerState (recent) and FUSED     */
    /*    METAL KERNEL; [PK] How it works step 3 (sinks count as +inf).       */
    /*    Readings: exactly one eviction once the token makes n + 1 > budget; */
    /*    the key is one fused multiply-add in float; ties go to the lowest   */
    /*    index.                                                              */
    int32_t e = -1;
    double gap = INFINITY;
    if (n + 1 > prm->budget) {
        float tau = prm->use_gumbel ? oracle_tau(prm->tau_init, prm->tau_end,
                                                 prm->anneal_steps, c->pos) : 0.0f;
        float best = INFINITY, second = INFINITY;
        double best_mag = 0.0, second_mag = 0.0;
        const int32_t last = n - prm->recent;     /* last candidate row */
        for (int32_t i = prm->n_sink; i <= last; ++i) {
            float gi = (i == n) ? g_new : c->g[i];
            float key = prm->use_gumbel ? fmaf(tau, gi, c->snew[i]) : c->snew[i];
            double mag = fabs((double)c->snew[i]) +
                         (prm->use_gumbel ? fabs((double)tau * (double)gi) : 0.0);
            if (e < 0 || key < best) {
                second = best; second_mag = best_mag;
                best = key; best_mag = mag; e = i;
            } else if (key < second) {
                second = key; second_mag = mag;
            }
        }
        gap = (double)second - (double)best;
        if (min_margin_rel >= 0.0) {
            double m = best_mag > second_mag ? best_mag : second_mag;
            if (!(gap > min_margin_rel * m)) {
                if (evicted) *evicted = e;
                if (margin) *margin = gap;
                return 1;                      /* rejected: nothing changed */
            }
        }
    }

    /* Commit: scores of the stored rows, then the append. */
    for (int32_t i = 0; i < n; ++i) c->s[i] = c->snew[i];
    copy_row(c->k + (size_t)n * d, k, d);
    copy_row(c->v + (size_t)n * d, v, d);
    c->s[n] = 0.0f;
    c->g[n] = g_new;
    c->p[n] = c->next_pos;
    c->tid[n] = c->next_pos;
    int32_t live = n + 1;

    /* 4. Compaction and RoPE remap.  [KF] keyformer_update step 3, and      */
    /*    KeyformerState (keys, positions): the rows after the evicted one    */
    /*    move down by one, keeping temporal order; afterwards positions are  */
    /*    the contiguous range 0..live-1, and each moved key is re-rotated    */
    /*    from the position it was rotated at to its new index.               */
    if (e >= 0) {
        for (int32_t j = e; j < live - 1; ++j) {
            int32_t src = j + 1;
            copy_row(c->k + (size_t)j * d, c->k + (size_t)src * d, d);
            copy_row(c->v + (size_t)j * d, c->v + (size_t)src * d, d);
            int64_t delta = (int64_t)j - (int64_t)c->p[src];
            if (delta != 0)
                oracle_rope_rotate(c->k + (size_t)j * d, d, delta, prm->rope_base);
            c->s[j] = c->s[src];
            c->g[j] = c->g[src];
            c->tid[j] = c->tid[src];
            c->p[j] = j;
        }
        live -= 1;
    }
    c->n = live;

    /* 5. Counters.  [KF] KeyformerState (pos, next_pos). */
    c->next_pos += 1;
    c->pos += 1;
    if (evicted) *evicted = e;
    if (margin) *margin = gap;
    return 0;
}

int oracle_run(oracle_cache *c, const uint16_t *ks, const uint16_t *vs, int32_t T,
               const oracle_params *prm, int32_t *evicted_out)
{
    for (int32_t t = 0; t < T; ++t) {
        int32_t e = -1;
        double m = 0.0;
        int rc = oracle_step(c, ks + (size_t)t * c->d, vs + (size_t)t * c->d, prm,
                             -1.0, &e, &m);
        if (rc != 0) return -1;
        if (evicted_out) evicted_out[t] = e;
    }
    return 0;
}
