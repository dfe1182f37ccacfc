/*
 * kve.h -- C ABI of the MI355X (gfx950) KV-cache eviction step.
 *
 * One call steps one token into every cache of one layer: for each of the
 * layer's B*H caches (one per batch element and kv-head) it
 *   1. scores the stored keys with the incoming key as the query,
 *      softmax(K_stored . k_new / sqrt(d)), and adds that mass to each stored
 *      row's fp32 cumulative score;
 *   2. appends the new fp16 key/value row with score 0, position next_pos and
 *      (Keyformer) its frozen Gumbel value;
 *   3. if the cache now holds budget + 1 rows, evicts the non-sink row with
 *      the smallest  score + tau * gumbel  (ties: lowest index), moves the
 *      later rows down one slot, and re-rotates the moved keys' RoPE in fp32
 *      so that positions are again the contiguous range 0 .. n_kept-1.
 *
 * Sources (VeloxQuant-MLX documentation pages):
 *   "veloxquant_mlx.quantizers.keyformer module": keyformer_update (steps
 *     1-3), keyformer_update_batched (one call over the B*H rows, per-row
 *     noise streams), KeyformerState (field meanings), init_keyformer_state
 *     (argument checks), FIXED GAP #1 (annealed temperature), FIXED GAP #2
 *     (position tracking and RoPE remap), FUSED METAL KERNEL (fp32 rotation).
 *   "PyramidKV -- Layer-Adaptive Budget Attention-Mass Eviction": How it
 *     works (the H2O step per layer), The budget schedule, Parameters,
 *     Relationship to H2O.
 *
 * Conventions
 *   - Every tensor pointer is DEVICE memory owned by the caller (for example
 *     torch.Tensor.data_ptr() of a contiguous tensor on the current device).
 *     The library keeps no pointer after a call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising.  Results are visible to
 *     later work on the same stream; synchronise before reading elsewhere.
 *   - The calls allocate nothing, never synchronise, keep no state between
 *     calls (on the host or the device) and are reentrant.  The batched forms
 *     pass their layer descriptors by value with the launch.  Every call can
 *     be captured into a graph and replayed (the host counters advance at
 *     capture, not at replay).
 *   - Compaction is done in place by each cache's workgroup.  Large
 *     single-token launches run faster when their long compactions are
 *     spread over the GPU by a second kernel; that needs scratch memory, which
 *     only kve_step_ws uses, from a workspace the caller owns.
 *   - Arguments are checked on the host before anything is enqueued.  A
 *     failing check returns KVE_EINVAL and leaves the counters and every
 *     tensor untouched.  A device fault is asynchronous and surfaces at the
 *     caller's next synchronisation.
 */
#ifndef KVE_H
#define KVE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVE_OK        0
#define KVE_EINVAL   -1   /* an argument failed a host-side check            */
#define KVE_ELAUNCH  -2   /* the HIP runtime rejected the kernel launch       */
#define KVE_ENODEV   -3   /* no HIP device, or no gfx950 code for the current one */
#define KVE_ENOSPACE -4   /* kve_step_noalloc: more scratch needed than its buffer holds */

/* One layer's B*H caches.  Rows of a cache are contiguous, caches follow
 * each other:  element (hh, row, j) of k lives at k[(hh*cap + row)*d + j].
 * Rows [0, n_kept) are live and in temporal order; rows >= n_kept hold
 * unspecified data after a call. */
typedef struct kve_layer {
    void    *k;          /* fp16 [bh][cap][d]  keys, RoPE'd at `positions`          */
    void    *v;          /* fp16 [bh][cap][d]  values                               */
    float   *scores;     /* f32  [bh][cap]     cumulative proxy-attention mass       */
    float   *gumbel;     /* f32  [bh][cap]     frozen Gumbel value of each row;
                            required by keyformer_step, unused (may be NULL) by
                            pyramid_step                                             */
    int32_t *positions;  /* i32  [bh][cap]     position each key is rotated at; the
                            library writes it.  Precondition (true of any state
                            built by these calls from an empty cache):
                            positions[hh][i] == i for every live row i            */
    int32_t  bh;         /* number of caches (batch * kv-heads), >= 1              */
    int32_t  cap;        /* rows allocated per cache, >= budget + 1                */
    int32_t  d;          /* head dimension: 64 or 128                             */
    int32_t  hh_base;    /* index of row 0 of this call in the Gumbel stream
                            numbering (0 unless the B*H set is split across calls
                            or devices); cache hh draws from stream hh_base + hh  */
} kve_layer;

/* HOST memory, read and updated by each successful call; shared by every
 * cache of the layer (keyformer_update_batched shares them across rows). */
typedef struct kve_counters {
    int32_t n_kept;      /* live rows before the call (uniform across the bh caches) */
    int32_t next_pos;    /* absolute position of the incoming token                  */
    int32_t pos;         /* running insertion count: the Gumbel counter and the
                            annealing clock                                          */
} kve_counters;

/*
 * keyformer_step -- Keyformer-adapted step (keyformer_update_batched with one
 * token, return_indices replaced by `evicted`).
 *
 *   L          layer tensors (see kve_layer); L->gumbel must not be NULL
 *   new_k      fp16 [bh][d] device: incoming keys, already RoPE'd at next_pos
 *   new_v      fp16 [bh][d] device: incoming values
 *   ctr        host counters; on success n_kept = min(n_kept + 1, budget),
 *              next_pos += 1, pos += 1
 *   budget     rows kept at most, sinks included; n_sink < budget <= 12288
 *   n_sink     leading rows never evicted; >= 0
 *   tau_init, tau_end, anneal_steps
 *              temperature tau = tau_init + min(pos, anneal_steps) *
 *              (tau_end - tau_init) / anneal_steps, evaluated in double on the
 *              device and rounded to float; constant tau_init when
 *              anneal_steps == 0 or tau_init == tau_end.  Both >= 0,
 *              anneal_steps >= 0.  tau == 0 gives H2O exactly.
 *   rope_base  RoPE frequency base (> 0) used to re-rotate moved keys
 *   seed       base seed of the Gumbel streams: the value of the row inserted
 *              at running position pos in cache hh is
 *              g = -log(-log u), u = ((h >> 11) + 1/2) / 2^53,
 *              h = mix(mix(mix(seed) ^ (hh_base + hh)) ^ pos), mix = the
 *              SplitMix64 output function
 *   evicted    optional device i32 [bh]: the evicted row index (counted before
 *              compaction, the new row being index n_kept) or -1; may be NULL
 *   stream     hipStream_t or NULL
 * Returns KVE_OK, KVE_EINVAL (bad argument; also when no eviction happens but
 * next_pos != n_kept, which would break the contiguous-position invariant,
 * e.g. a budget raised after evictions), KVE_ENODEV or KVE_ELAUNCH.
 */
int keyformer_step(const kve_layer *L, const void *new_k, const void *new_v,
                   kve_counters *ctr, int32_t budget, int32_t n_sink,
                   double tau_init, double tau_end, int32_t anneal_steps,
                   double rope_base, uint64_t seed, int32_t *evicted, void *stream);

/*
 * pyramid_step -- H2O-adapted step at one layer's budget (PyramidKV-adapted
 * when `budget` comes from pyramid_budgets).  Same as keyformer_step with
 * tau == 0 and no noise: the eviction key is the raw score and L->gumbel is
 * neither read nor written.
 */
int pyramid_step(const kve_layer *L, const void *new_k, const void *new_v,
                 kve_counters *ctr, int32_t budget, int32_t n_sink, double rope_base,
                 int32_t *evicted, void *stream);

/*
 * keyformer_step_layers / pyramid_step_layers -- the same step for several
 * layers of one token in ONE launch: equivalent, bit for bit, to calling
 * keyformer_step / pyramid_step once per layer (in any order; the layers are
 * independent, as the PyramidKV page's "How it works" notes that layers never
 * exchange data).  One launch over all layers keeps every compute unit busy
 * while some caches finish their compaction, which per-layer launches of a
 * few hundred caches cannot.
 *
 *   n_layers   1 .. 128
 *   layers     HOST array [n_layers] of layer descriptors (all with the same d;
 *              bh, cap and hh_base may differ); the layers must not overlap
 *   new_k,new_v  HOST arrays [n_layers] of device pointers, fp16 [bh_l][d]
 *   ctrs       HOST array [n_layers] of counters, each updated as by the
 *              per-layer call
 *   budgets    HOST array [n_layers]: budget of each layer (for example from
 *              pyramid_budgets)
 *   evicted    HOST array [n_layers] of device i32 [bh_l] outputs (entries may
 *              be NULL), or NULL
 *   n_sink, tau_*, anneal_steps, rope_base, seed, stream: as per layer, shared
 * Every layer is checked before anything is enqueued; on KVE_EINVAL no
 * counter changes.  The descriptors of up to 32 layers travel by value with
 * a launch; a call over more layers is one launch per group of 32, in order
 * on `stream` (the same bits, since layers are independent).  On
 * KVE_ELAUNCH the groups launched before the failure have been stepped and
 * their counters advanced; the rest are untouched.
 */
int keyformer_step_layers(int32_t n_layers, const kve_layer *layers, const void *const *new_k,
                          const void *const *new_v, kve_counters *ctrs, const int32_t *budgets,
                          int32_t n_sink, double tau_init, double tau_end,
                          int32_t anneal_steps, double rope_base, uint64_t seed,
                          int32_t *const *evicted, void *stream);

int pyramid_step_layers(int32_t n_layers, const kve_layer *layers, const void *const *new_k,
                        const void *const *new_v, kve_counters *ctrs, const int32_t *budgets,
                        int32_t n_sink, double rope_base, int32_t *const *evicted,
                        void *stream);

/*
 * keyformer_step_tokens / pyramid_step_tokens -- S consecutive tokens into
 * every cache of one layer in ONE launch (keyformer_update absorbs S tokens
 * one after the other): bit for bit the same as S calls of keyformer_step /
 * pyramid_step.  Each cache's workgroup steps through the S tokens on its
 * own, so a cache that must move many rows for one token does not hold up
 * the others.
 *
 *   n_tokens   S, 1 .. 128
 *   new_k,new_v  device fp16 [S][bh][d]: token t's incoming rows at
 *              new_k + t*bh*d (already RoPE'd at next_pos + t)
 *   evicted    optional device i32 [S][bh]: token t's evicted index per cache
 *   ctr        advanced by S tokens on success
 *   other arguments as keyformer_step / pyramid_step.
 * Checked as one per-layer call (the first token's counters), plus
 * 1 <= n_tokens <= 128; launched as keyformer_step_layers_tokens with one
 * layer.
 */
int keyformer_step_tokens(const kve_layer *L, int32_t n_tokens, const void *new_k,
                          const void *new_v, kve_counters *ctr, int32_t budget, int32_t n_sink,
                          double tau_init, double tau_end, int32_t anneal_steps,
                          double rope_base, uint64_t seed, int32_t *evicted, void *stream);

int pyramid_step_tokens(const kve_layer *L, int32_t n_tokens, const void *new_k,
                        const void *new_v, kve_counters *ctr, int32_t budget, int32_t n_sink,
                        double rope_base, int32_t *evicted, void *stream);

/*
 * keyformer_step_layers_tokens / pyramid_step_layers_tokens -- both of the
 * above at once: S consecutive tokens into every cache of n_layers layers in
 * ONE launch, bit for bit the same as S calls of the *_step_layers form (or
 * n_layers * S per-layer calls).  Each layer's workgroups walk its caches
 * through the S tokens; layers never wait for one another.  This is the form
 * that fills the device when each layer has few caches (small batch).
 *
 *   n_layers   1 .. 128;  n_tokens  S, 1 .. 128
 *   layers, ctrs, budgets, n_sink, tau_*, anneal_steps, rope_base, seed,
 *   stream     as keyformer_step_layers; each ctrs[l] advances by S tokens
 *   new_k,new_v  HOST arrays [n_layers] of device pointers, fp16
 *              [S][bh_l][d]: token t's incoming rows of layer l at
 *              new_k[l] + t*bh_l*d
 *   evicted    HOST array [n_layers] of device i32 [S][bh_l] (entries may be
 *              NULL), or NULL
 * Checked and launched as keyformer_step_layers.
 */
int keyformer_step_layers_tokens(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                                 const void *const *new_k, const void *const *new_v,
                                 kve_counters *ctrs, const int32_t *budgets, int32_t n_sink,
                                 double tau_init, double tau_end, int32_t anneal_steps,
                                 double rope_base, uint64_t seed, int32_t *const *evicted,
                                 void *stream);

int pyramid_step_layers_tokens(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                               const void *const *new_k, const void *const *new_v,
                               kve_counters *ctrs, const int32_t *budgets, int32_t n_sink,
                               double rope_base, int32_t *const *evicted, void *stream);

/*
 * kve_step -- the general form of every call above, with the two extensions
 * the pages describe beyond the plain step:
 *   - a trailing protected window (Keyformer page, KeyformerState `recent`
 *     and init_keyformer_state: an extension, off by default): the last
 *     `recent` rows of the budget + 1 rows present after the append are
 *     never evicted, so the candidates are rows n_sink .. budget - recent and
 *     the incoming row is one only when recent == 0;
 *   - TOVA-adapted scoring (PyramidKV page, table of eviction axes: the
 *     current step's attention weight is the score signal): with
 *     KVE_SCORE_CURRENT a stored row's score becomes this step's proxy
 *     weight softmax(K.k/sqrt(d)) instead of accumulating it; the incoming
 *     row still enters with 0, so without a window TOVA always evicts it.
 * keyformer_step(...) is kve_step with n_layers = n_tokens = 1 and the policy
 * {n_sink, 0, KVE_SCORE_CUMULATIVE, 1, tau_init, tau_end, anneal_steps,
 * rope_base, seed}; pyramid_step the same with gumbel = 0.
 */
#define KVE_SCORE_CUMULATIVE 0   /* H2O / Keyformer / PyramidKV: score += weight */
#define KVE_SCORE_CURRENT    1   /* TOVA-adapted: score = weight                 */

typedef struct kve_policy {
    int32_t  n_sink;        /* leading rows never evicted, >= 0                       */
    int32_t  recent;        /* trailing rows never evicted, >= 0 (0 = off); every
                               layer's budget must exceed n_sink + recent              */
    int32_t  score;         /* KVE_SCORE_CUMULATIVE or KVE_SCORE_CURRENT              */
    int32_t  gumbel;        /* 1: Keyformer noise tau * g in the eviction key (every
                               layer needs its gumbel tensor); 0: no noise, and the
                               three fields below and `seed` are ignored             */
    double   tau_init;      /* as keyformer_step                                       */
    double   tau_end;
    int32_t  anneal_steps;
    int32_t  reserved;      /* unused                                                  */
    double   rope_base;     /* > 0                                                     */
    uint64_t seed;          /* Gumbel base seed, as keyformer_step                     */
} kve_policy;

/*
 *   n_layers   1 .. 128;  n_tokens  1 .. 128
 *   layers, new_k, new_v, ctrs, budgets, evicted, stream
 *              as keyformer_step_layers_tokens (with n_tokens == 1 the rows of
 *              token 0 are simply [bh_l][d])
 *   policy     HOST pointer, read during the call only
 * Returns as keyformer_step; KVE_EINVAL also for a NULL policy, an unknown
 * score rule, gumbel not 0 or 1, recent < 0 or budget <= n_sink + recent.
 * One layer and one token launch as keyformer_step does; otherwise as the
 * batched calls.
 */
int kve_step(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
             const void *const *new_k, const void *const *new_v, kve_counters *ctrs,
             const int32_t *budgets, const kve_policy *policy, int32_t *const *evicted,
             void *stream);

/*
 * kve_step_ws -- kve_step with a caller-owned device workspace, for the
 * large single-token launches whose long compactions dominate them (the
 * batched call keyformer_update_batched of the Keyformer page, one token,
 * with the moves of keyformer_update step 3 spread over the GPU).
 *
 * A single-token launch of at least 256 caches whose policy makes long
 * interior evictions routine (Keyformer noise, TOVA scoring, or a window
 * longer than 128 rows) hands every move of more than 128 rows to a second
 * kernel enqueued right after the step on `stream`: the step reserves one
 * workspace item per 64-row chunk of the move and parks the few rows the
 * chunks would otherwise race on, and the move kernel shifts the chunks on
 * many compute units at once.  The results are the same bits as kve_step's;
 * other launches (several tokens, fewer caches, other policies) ignore the
 * workspace.  A cache whose reservation does not fit in the workspace
 * compacts in place, so any size of at least one item is correct, and
 * kve_workspace_size gives the size at which every move can be handed over.
 *
 *   workspace        device memory owned by the caller, 256-byte aligned,
 *                    or NULL (then workspace_bytes must be 0 and the call is
 *                    kve_step)
 *   workspace_bytes  its size
 *   other arguments  as kve_step
 * Contract: the workspace must be all zero bytes before its first use (for
 * example torch.zeros).  Its first 16 bytes then hold two reservation
 * counters and a phase that the calls keep consistent: each call reserves on
 * the counter of the current phase, and its second kernel zeroes the other
 * counter and advances the phase, so every call leaves the workspace ready
 * for the next one and nothing needs clearing between calls (graph replays
 * included).  Calls that use one workspace must be ordered (the same stream,
 * or events): overlapping calls race.  After a KVE_ELAUNCH the layers'
 * tensors and the workspace are undefined: zero the workspace before using
 * it again.
 * Returns as kve_step; KVE_EINVAL also for a misaligned workspace or one
 * too small to hold a single item.
 */
int kve_step_ws(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                const void *const *new_k, const void *const *new_v, kve_counters *ctrs,
                const int32_t *budgets, const kve_policy *policy, int32_t *const *evicted,
                void *workspace, int64_t workspace_bytes, void *stream);

/*
 * kve_workspace_size -- bytes of workspace with which kve_step_ws hands over
 * every long move of a single-token launch over `caches` caches (the sum of
 * bh over its layers) whose budgets are at most max_budget, at head
 * dimension d: one 32-byte item and one parked 4*d-byte row per 64-row chunk
 * of each cache's longest possible move (max_budget - 1 rows), plus a
 * 256-byte header (counters and phase), each part 256-byte aligned.  Returns -1 for caches < 1,
 * max_budget outside 1 .. 12288, d not 64 or 128, or a size past 2^30 items.
 * Pure host arithmetic; needs no device.
 */
int64_t kve_workspace_size(int64_t caches, int32_t max_budget, int32_t d);

/*
 * kve_step_noalloc -- for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * allocation): kve_step_ws with the workspace in a fixed array of
 * KVE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on,
 * from its load until the process ends.  The call allocates nothing.
 *
 * Arguments, results and errors as kve_step_ws without the workspace; the
 * results are the same bits.  A call that would hand moves over (one token,
 * at least 256 caches, Keyformer noise, TOVA scoring or a window of more
 * than 128 rows) needs kve_workspace_size(sum of bh, largest budget, d)
 * bytes; if that exceeds KVE_NOALLOC_SCRATCH_BYTES it returns KVE_ENOSPACE
 * before anything is enqueued (use kve_step_ws with a workspace of that size
 * instead).  Other calls need no scratch and run as kve_step.  Each call that
 * uses the array first clears its header with a small kernel on `stream`.
 * All calls on one GPU share its array: calls that overlap on one GPU (on
 * different streams or host threads, without ordering) race.  The device
 * address of the array is looked up once per device, on the first call that
 * needs it.
 */
#define KVE_NOALLOC_SCRATCH_BYTES (16 << 20)

int kve_step_noalloc(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                     const void *const *new_k, const void *const *new_v, kve_counters *ctrs,
                     const int32_t *budgets, const kve_policy *policy, int32_t *const *evicted,
                     void *stream);

/*
 * pyramid_budgets -- per-layer budgets ("The budget schedule"): a linear taper
 * from the largest budget at layer 0 to the smallest at the last layer, mean
 * avg_budget, every entry at least n_sink + 1.  The smallest is
 * max((2 - beta) * avg_budget, n_sink + 1), the largest 2 * avg_budget minus
 * the smallest; entry l is their linear interpolation rounded to nearest
 * (halves to even).  beta == 1 gives every layer avg_budget; n_layers == 1
 * gives {avg_budget}; n_layers == 0 writes nothing.
 *   out   HOST i32 [n_layers]
 * Returns KVE_OK, or KVE_EINVAL if beta < 1 (or NaN), n_layers < 0,
 * n_sink < 0, avg_budget < n_sink + 1, or out == NULL with n_layers > 0.
 * Pure host arithmetic; needs no device.
 */
int pyramid_budgets(int32_t n_layers, int32_t avg_budget, int32_t n_sink, double beta,
                    int32_t *out);

/*
 * kve_kept_indices -- return_indices of keyformer_update_batched: after a call
 * that stepped n_tokens tokens into a cache that held n_prev rows, the rows
 * now kept, as chronological indices into the prior rows followed by the new
 * ones (0 .. n_prev-1 the prior rows in their order, n_prev + t the t-th new
 * token).  Composed from that cache's `evicted` outputs of the call, in
 * token order (each an index into the rows present after that token's
 * append, or -1).
 *   evicted   HOST i32 [n_tokens]; out  HOST i32 [n_prev + n_tokens]
 * Returns the number of kept rows written to out, or KVE_EINVAL (n_prev < 0,
 * n_tokens < 0, NULL pointers with n_tokens or n_prev > 0, an evicted index
 * out of range).  Pure host arithmetic; needs no device.
 */
int32_t kve_kept_indices(int32_t n_prev, int32_t n_tokens, const int32_t *evicted, int32_t *out);

/*
 * kve_fp16_bytes / kve_full_fp16_bytes -- keyformer_fp16_bytes and
 * full_keyformer_fp16_bytes: the K + V payload in fp16 of n_kept stored rows,
 * or of all tokens_seen tokens had none been evicted, for one cache of head
 * dimension d: 2 * 2 * rows * d bytes.  Scores, Gumbel values and positions
 * are bookkeeping, not payload.  Returns -1 if a count is negative or d < 1.
 */
int64_t kve_fp16_bytes(int64_t n_kept, int32_t d);
int64_t kve_full_fp16_bytes(int64_t tokens_seen, int32_t d);

/* Text for a KVE_* code (static storage). */
const char *kve_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* KVE_H */
