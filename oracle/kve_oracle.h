/*
 * kve_oracle.h -- plain, slow, single-threaded CPU oracle of the per-token
 * KV-cache eviction step (Keyformer-adapted and PyramidKV/H2O-adapted).
 *
 * TEST INFRASTRUCTURE ONLY.  This directory is the independent checker of the
 * GPU library.  Only the test suite, the smoke entry point and the benchmark's
 * CPU-baseline leg may load or call it.  It shares no code, header, table or
 * constant with the GPU path, and the GPU path never calls it.
 *
 * Sources (the documentation pages of the VeloxQuant-MLX library):
 *   [KF]  "veloxquant_mlx.quantizers.keyformer module" -- sections
 *         KeyformerState, init_keyformer_state, keyformer_update,
 *         keyformer_update_batched, FIXED GAP #1 (annealing), FIXED GAP #2
 *         (RoPE position tracking), THE HONESTY CRUX.
 *   [PK]  "PyramidKV -- Layer-Adaptive Budget Attention-Mass Eviction" --
 *         sections "The budget schedule", "How it works", "Relationship to
 *         H2O", "Evidence", and the table of eviction axes (TOVA-adapted:
 *         current-step attention weight as the score signal).
 * Where those pages leave a step open, the reading taken is stated next to
 * the function that implements it.
 */
#ifndef KVE_ORACLE_H
#define KVE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One cache: the K/V store of one (batch, layer, kv-head).  All arrays are
 * owned by the caller and hold `cap` rows.  Rows [0, n) are live. */
typedef struct oracle_cache {
    int32_t   d;          /* head dimension                                   */
    int32_t   cap;        /* rows allocated (must be >= budget + 1)            */
    uint16_t *k;          /* fp16 bit patterns [cap][d], RoPE'd keys           */
    uint16_t *v;          /* fp16 bit patterns [cap][d]                        */
    float    *s;          /* cumulative proxy-attention mass [cap]            */
    float    *g;          /* frozen Gumbel value of each row [cap]             */
    int32_t  *p;          /* position each key is currently rotated at [cap]   */
    int64_t  *tid;        /* original token position of each row [cap] (bookkeeping only) */
    double   *work;       /* scratch [2*cap] (logits, then exp weights)         */
    float    *snew;       /* scratch [cap + 1] (candidate scores)              */
    int32_t   n;          /* live rows                                        */
    int32_t   next_pos;   /* absolute position of the next incoming token      */
    int32_t   pos;        /* running insertion count (Gumbel counter, tau)     */
} oracle_cache;

typedef struct oracle_params {
    int32_t  budget;        /* max rows kept, sinks included                  */
    int32_t  n_sink;        /* leading rows never evicted                     */
    int32_t  use_gumbel;    /* 1 = Keyformer-adapted, 0 = H2O / PyramidKV     */
    int32_t  anneal_steps;  /* T of the temperature ramp                      */
    double   tau_init;
    double   tau_end;
    double   rope_base;
    uint64_t seed;          /* base seed of the Gumbel stream                 */
    int64_t  hh;            /* row of this cache within its layer's B*H set   */
    int32_t  recent;        /* trailing rows never evicted (0 = off)          */
    int32_t  current_score; /* 1 = TOVA-adapted: a row's score is this step's
                               proxy attention weight alone (not accumulated) */
} oracle_params;

/* SplitMix64 output function applied to state value z (state advanced by
 * the golden-ratio increment first). */
uint64_t oracle_splitmix64_mix(uint64_t z);
/* One step of the SplitMix64 generator: advances *state, returns the output. */
uint64_t oracle_splitmix64_next(uint64_t *state);
/* The uniform variate in (0,1) behind the Gumbel draw of (seed, hh, pos). */
double   oracle_gumbel_uniform(uint64_t seed, int64_t hh, int64_t pos);
/* The frozen Gumbel value of the token inserted at running position pos. */
float    oracle_gumbel(uint64_t seed, int64_t hh, int64_t pos);
/* Annealed temperature of the step that inserts running position pos. */
float    oracle_tau(double tau_init, double tau_end, int32_t anneal_steps, int64_t pos);
/* Per-layer budgets; returns 0, or -1 on invalid arguments. */
int      oracle_pyramid_budgets(int32_t n_layers, int32_t avg_budget, int32_t n_sink,
                                double beta, int32_t *out);
/* IEEE binary16 <-> binary32, round to nearest even, subnormals kept. */
float    oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float f);
/* Rotate one stored fp16 key row by delta positions (half-split RoPE). */
void     oracle_rope_rotate(uint16_t *row, int32_t d, int64_t delta, double base);

/* One token through one cache.
 *   k, v          : the incoming fp16 key (already RoPE'd at next_pos) and value
 *   min_margin_rel: < 0 disables the guard; otherwise, when the step evicts and
 *                   the gap between the two smallest eviction keys is not above
 *                   min_margin_rel * (|s|+|tau*g| of the larger of the two), the
 *                   step is rejected and the cache is left untouched
 *   evicted       : out, the evicted row index (pre-compaction numbering) or -1
 *   margin        : out, that gap (or +inf when nothing is evicted)
 * Returns 0 when committed, 1 when rejected by the guard, -1 on bad input. */
int      oracle_step(oracle_cache *c, const uint16_t *k, const uint16_t *v,
                     const oracle_params *prm, double min_margin_rel,
                     int32_t *evicted, double *margin);

/* Convenience: run T tokens through one cache with the guard off.
 * ks, vs: [T][d]; evicted_out: [T]. Returns 0 or -1. */
int      oracle_run(oracle_cache *c, const uint16_t *ks, const uint16_t *vs, int32_t T,
                    const oracle_params *prm, int32_t *evicted_out);

#ifdef __cplusplus
}
#endif
#endif /* KVE_ORACLE_H */
