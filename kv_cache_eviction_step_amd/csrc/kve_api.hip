// kve_api.hip -- host side of the C ABI declared in include/kve.h:
// argument checks, the eviction policy, fp64 rotation constants and
// frequencies, the launches on the caller's stream, the counter update, the
// caller-owned move workspace of large single-token launches, and the
// host-only helpers (pyramid budget schedule, kept indices, byte accounting).
// Nothing here allocates, synchronises or keeps state between calls.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstring>
#include <mutex>

#include "kve.h"
#include "kve_step.h"

#define KVE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// Largest budget a cache may have: the kernel keeps one fp32 logit per stored
// row in LDS and each thread's share of the scores in registers.
constexpr int32_t kMaxBudget = kve::kMaxRows;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Rotation frequencies base^(-2j/d) and the fp32 cosine / sine of a rotation
// by -1 position, evaluated per call with the host's fp64 libm (a few
// microseconds; only calls in which some cache can evict need them).
void rope_tables(int d, double base, double *freq, float *cos_m1, float *sin_m1) {
  for (int j = 0; j < d / 2; ++j) {
    freq[j] = std::pow(base, -(2.0 * (double)j) / (double)d);
    const double th = -1.0 * freq[j];
    cos_m1[j] = (float)std::cos(th);
    sin_m1[j] = (float)std::sin(th);
  }
}

// A HIP error of a launch as a KVE_* code: no device, or no gfx950 code for
// the current one, is KVE_ENODEV; anything else KVE_ELAUNCH.
int launch_error(hipError_t err) {
  if (err == hipSuccess) return KVE_OK;
  if (err == hipErrorNoDevice || err == hipErrorNoBinaryForGpu ||
      err == hipErrorInvalidDeviceFunction || err == hipErrorInvalidDevice)
    return KVE_ENODEV;
  return KVE_ELAUNCH;
}

// Everything about a call that is not per layer: the eviction rule and the
// noise, as the entry points receive them.
struct Policy {
  int32_t n_sink = 0;
  int32_t recent = 0;          // trailing rows protected (0 = off)
  bool current = false;        // TOVA-adapted: score = this step's weight
  bool gumbel = false;         // Keyformer-adapted noise in the eviction key
  double tau_init = 0.0;
  double tau_end = 0.0;
  int32_t anneal_steps = 0;
  double rope_base = 10000.0;
  uint64_t seed = 0;
};

Policy keyformer_policy(int32_t n_sink, double tau_init, double tau_end, int32_t anneal_steps,
                        double rope_base, uint64_t seed) {
  Policy p;
  p.n_sink = n_sink;
  p.gumbel = true;
  p.tau_init = tau_init;
  p.tau_end = tau_end;
  p.anneal_steps = anneal_steps;
  p.rope_base = rope_base;
  p.seed = seed;
  return p;
}

Policy pyramid_policy(int32_t n_sink, double rope_base) {
  Policy p;
  p.n_sink = n_sink;
  p.rope_base = rope_base;
  return p;
}

// Host-side checks shared by every entry point (init_keyformer_state's guards
// and the layout); returns KVE_OK or KVE_EINVAL.
int check_layer(const kve_layer *L, const void *new_k, const void *new_v,
                const kve_counters *ctr, int32_t budget, const Policy &p) {
  if (!L || !ctr || !new_k || !new_v) return KVE_EINVAL;
  if (!L->k || !L->v || !L->scores || !L->positions) return KVE_EINVAL;
  if (p.gumbel && !L->gumbel) return KVE_EINVAL;
  if (!aligned16(L->k) || !aligned16(L->v) || !aligned16(new_k) || !aligned16(new_v))
    return KVE_EINVAL;
  if (L->d != 64 && L->d != 128) return KVE_EINVAL;
  if (L->bh < 1 || L->hh_base < 0 || (int64_t)L->hh_base + L->bh > INT32_MAX) return KVE_EINVAL;
  // the protected rows (sinks and the recent window) must leave room to evict
  if ((int64_t)budget <= (int64_t)p.n_sink + p.recent || budget > kMaxBudget) return KVE_EINVAL;
  if (L->cap < budget + 1) return KVE_EINVAL;
  const int32_t n = ctr->n_kept;
  if (n < 0 || n > budget) return KVE_EINVAL;
  if (ctr->pos < 0 || ctr->next_pos < n || ctr->next_pos == INT32_MAX || ctr->pos == INT32_MAX)
    return KVE_EINVAL;
  // without an eviction the new row keeps next_pos, which must equal its slot
  if (n + 1 <= budget && ctr->next_pos != n) return KVE_EINVAL;
  return KVE_OK;
}

int check_policy(const Policy &p) {
  if (p.n_sink < 0 || p.recent < 0) return KVE_EINVAL;
  if (!(p.tau_init >= 0.0) || !(p.tau_end >= 0.0) || !std::isfinite(p.tau_init) ||
      !std::isfinite(p.tau_end) || p.anneal_steps < 0)
    return KVE_EINVAL;
  if (!(p.rope_base > 0.0) || !std::isfinite(p.rope_base)) return KVE_EINVAL;
  return KVE_OK;
}

kve::LayerArgs layer_args(const kve_layer *L, const void *new_k, const void *new_v,
                          const kve_counters *ctr, int32_t budget, int32_t *evicted,
                          bool gumbel) {
  kve::LayerArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k = L->k;
  a.v = L->v;
  a.scores = L->scores;
  a.gumbel = gumbel ? L->gumbel : nullptr;
  a.positions = L->positions;
  a.new_k = new_k;
  a.new_v = new_v;
  a.evicted = evicted;
  a.cap = L->cap;
  a.n_prev = ctr->n_kept;
  a.budget = budget;
  a.next_pos = ctr->next_pos;
  a.pos = ctr->pos;
  a.hh_base = L->hh_base;
  return a;
}

kve::SharedArgs shared_args(int d, const Policy &p, bool evicts) {
  kve::SharedArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  sa.n_sink = p.n_sink;
  sa.recent = p.recent;
  sa.current = p.current ? 1 : 0;
  sa.anneal_steps = p.anneal_steps;
  sa.tau_init = p.gumbel ? p.tau_init : 0.0;
  sa.tau_end = p.gumbel ? p.tau_end : 0.0;
  sa.seed = p.seed;
  sa.scale = (float)(1.0 / std::sqrt((double)d));
  // keyformer FIXED GAP #2: moved stored rows go back one position.  The
  // incoming row, if it survives an older row's eviction, goes from next_pos
  // to slot n-1: the device rotates it by (n-1-next_pos) * freq[j] with an
  // fp64 sincos rounded once to fp32.  Nothing moves in a call in which no
  // cache is at its budget, and such a call leaves the tables unset.
  if (evicts) rope_tables(d, p.rope_base, sa.freq, sa.back1.c, sa.back1.s);
  return sa;
}

void advance(kve_counters *ctr, int32_t budget) {
  ctr->n_kept = ctr->n_kept + 1 > budget ? budget : ctr->n_kept + 1;
  ctr->next_pos += 1;
  ctr->pos += 1;
}

// ---------------------------------------------------------------------------
// handed-over compactions: single-token launches given a workspace (the
// kve_step_ws form) hand their long moves to the move kernel (kve_step.h)
// ---------------------------------------------------------------------------

// Handed over in single-token launches whose policy makes long interior
// moves routine (Gumbel noise, current-step scores, a window longer than a
// step moves by itself) and that hold at least this many caches: there the
// longest move, done by one compute unit, sets the launch's length.  Smaller
// launches are bound by their latency chain, where a second launch would cost
// more than it saves.  (With cumulative scores and a window, the row evicted
// is nearly always the one just outside the window: a move of `recent` rows.)
constexpr int64_t kDeferMinCaches = 256;

bool defers(const Policy &p, int64_t caches) {
  return (p.gumbel || p.current || p.recent > kve::kDeferRows) && caches >= kDeferMinCaches;
}

// A caller's workspace, checked: null items when there is none (every cache
// then compacts in place).  Returns KVE_EINVAL for a misaligned workspace or a
// size that is negative or too small to hold one item.
int make_pool(void *ws, int64_t bytes, int d, kve::MovePool &pool) {
  pool = kve::MovePool{};
  if (!ws) return bytes == 0 ? KVE_OK : KVE_EINVAL;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return KVE_EINVAL;
  const int64_t cap = kve::pool_capacity(bytes, d);
  if (cap < 1) return KVE_EINVAL;
  char *base = static_cast<char *>(ws);
  const int64_t c = std::min<int64_t>(cap, INT32_MAX / 2);
  pool.count = reinterpret_cast<int32_t *>(base);
  pool.items = reinterpret_cast<kve::MoveItem *>(base + kve::kPoolHeaderBytes);
  pool.rows = base + kve::kPoolHeaderBytes + kve::pool_items_bytes(c);
  pool.cap = (int32_t)c;
  return KVE_OK;
}

// One layer, one token: the descriptor travels by value with the launch.
// With a pool (and a policy and size that hand moves over), long moves go to
// the move kernel that follows the step.
int step_impl(const kve_layer *L, const void *new_k, const void *new_v, kve_counters *ctr,
              int32_t budget, const Policy &p, int32_t *evicted, const kve::MovePool &pool,
              void *stream) {
  if (check_policy(p) != KVE_OK) return KVE_EINVAL;
  if (check_layer(L, new_k, new_v, ctr, budget, p) != KVE_OK) return KVE_EINVAL;

  const bool evicts = ctr->n_kept + 1 > budget;
  const kve::LayerArgs la = layer_args(L, new_k, new_v, ctr, budget, evicted, p.gumbel);
  kve::SharedArgs sa = shared_args(L->d, p, evicts);
  // a step under its budget evicts nothing, so it has no move to hand over
  const bool hand_over = pool.items && evicts && defers(p, L->bh);
  if (hand_over) sa.pool = pool;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();                     // report this call's launch, not an older error
  int rc = KVE_OK;
  if (hand_over && pool.clear_first) rc = launch_error(kve::launch_pool_clear(pool, s));
  if (rc != KVE_OK) return rc;
  rc = launch_error(kve::launch_step(la, sa, L->bh, L->d, p.gumbel, s));
  if (rc != KVE_OK) return rc;
  if (hand_over) {
    rc = launch_error(kve::launch_moves(pool, sa.back1, L->d, s));
    if (rc != KVE_OK) return rc;
  }
  advance(ctr, budget);
  return KVE_OK;
}

// ---------------------------------------------------------------------------
// batched calls: up to kLaunchLayers layer descriptors travel by value with
// each launch; a call over more layers is several launches (layers never
// exchange data, so any grouping gives the same bits)
// ---------------------------------------------------------------------------

// The host checks of a descriptor-driven call: n_layers layers, each stepped
// n_tokens tokens.  KVE_OK or KVE_EINVAL.
int check_batch(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                const void *const *new_k, const void *const *new_v, const kve_counters *ctrs,
                const int32_t *budgets, const Policy &p) {
  if (n_layers < 1 || n_layers > kve::kMaxBatchLayers) return KVE_EINVAL;
  if (n_tokens < 1 || n_tokens > kve::kMaxTokens) return KVE_EINVAL;
  if (!layers || !new_k || !new_v || !ctrs || !budgets) return KVE_EINVAL;
  if (check_policy(p) != KVE_OK) return KVE_EINVAL;
  const int d = layers[0].d;
  int64_t blocks = 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    if (check_layer(&layers[l], new_k[l], new_v[l], &ctrs[l], budgets[l], p) != KVE_OK)
      return KVE_EINVAL;
    if (layers[l].d != d) return KVE_EINVAL;
    if ((int64_t)ctrs[l].next_pos + n_tokens >= INT32_MAX ||
        (int64_t)ctrs[l].pos + n_tokens >= INT32_MAX)
      return KVE_EINVAL;
    blocks += layers[l].bh;
  }
  if (blocks > INT32_MAX) return KVE_EINVAL;
  // Two layers sharing cache memory (the same layer passed twice, say) would be
  // stepped by two workgroups at once: reject overlapping key buffers.
  if (n_layers > 1) {
    int32_t order[kve::kMaxBatchLayers];
    for (int32_t l = 0; l < n_layers; ++l) order[l] = l;
    auto start = [&](int32_t l) { return reinterpret_cast<uintptr_t>(layers[l].k); };
    std::sort(order, order + n_layers, [&](int32_t a, int32_t b) { return start(a) < start(b); });
    for (int32_t i = 1; i < n_layers; ++i) {
      const kve_layer &prev = layers[order[i - 1]];
      const uintptr_t prev_end =
          start(order[i - 1]) + (uintptr_t)prev.bh * (uintptr_t)prev.cap * (uintptr_t)prev.d * 2u;
      if (start(order[i]) < prev_end) return KVE_EINVAL;
    }
  }
  return KVE_OK;
}

// Descriptor-driven launches: n_layers layers, each stepped n_tokens tokens.
// Checks every layer first.
int batch_impl(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
               const void *const *new_k, const void *const *new_v, kve_counters *ctrs,
               const int32_t *budgets, const Policy &p, int32_t *const *evicted,
               const kve::MovePool &pool, void *stream) {
  if (check_batch(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets, p) != KVE_OK)
    return KVE_EINVAL;
  const int d = layers[0].d;
  bool any_evicts = false;                    // some layer is at its budget
  for (int32_t l = 0; l < n_layers; ++l) any_evicts = any_evicts || ctrs[l].n_kept + n_tokens > budgets[l];
  const kve::SharedArgs shared = shared_args(d, p, any_evicts);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int32_t g0 = 0; g0 < n_layers; g0 += kve::kLaunchLayers) {
    const int32_t g1 = std::min(n_layers, g0 + kve::kLaunchLayers);
    kve::LayerPack pack{};
    int32_t block0 = 0, max_n = 0;
    bool evicts = false;                      // some layer is at its budget
    for (int32_t l = g0; l < g1; ++l) {
      kve::LayerArgs &a = pack.l[l - g0];
      a = layer_args(&layers[l], new_k[l], new_v[l], &ctrs[l], budgets[l],
                     evicted ? evicted[l] : nullptr, p.gumbel);
      a.block0 = block0;
      a.n_tokens = n_tokens;
      block0 += layers[l].bh;
      max_n = std::max(max_n, std::min(ctrs[l].n_kept + n_tokens - 1, budgets[l]));
      evicts = evicts || ctrs[l].n_kept + 1 > budgets[l];
    }
    kve::SharedArgs sa = shared;
    const bool hand_over = pool.items && n_tokens == 1 && evicts && defers(p, block0);
    if (hand_over) sa.pool = pool;
    (void)hipGetLastError();                   // report this launch, not an older error
    int rc = KVE_OK;
    if (hand_over && pool.clear_first) rc = launch_error(kve::launch_pool_clear(pool, s));
    if (rc != KVE_OK) return rc;
    rc = launch_error(
        kve::launch_step_layers(pack, g1 - g0, block0, max_n, n_tokens, sa, d, p.gumbel, s));
    if (rc != KVE_OK) return rc;
    if (hand_over) {
      rc = launch_error(kve::launch_moves(pool, sa.back1, d, s));
      if (rc != KVE_OK) return rc;
    }
    for (int32_t l = g0; l < g1; ++l)
      for (int32_t t = 0; t < n_tokens; ++t) advance(&ctrs[l], budgets[l]);
  }
  return KVE_OK;
}

}  // namespace

KVE_EXPORT int keyformer_step(const kve_layer *L, const void *new_k, const void *new_v,
                              kve_counters *ctr, int32_t budget, int32_t n_sink,
                              double tau_init, double tau_end, int32_t anneal_steps,
                              double rope_base, uint64_t seed, int32_t *evicted,
                              void *stream) {
  return step_impl(L, new_k, new_v, ctr, budget,
                   keyformer_policy(n_sink, tau_init, tau_end, anneal_steps, rope_base, seed),
                   evicted, kve::MovePool{}, stream);
}

KVE_EXPORT int pyramid_step(const kve_layer *L, const void *new_k, const void *new_v,
                            kve_counters *ctr, int32_t budget, int32_t n_sink,
                            double rope_base, int32_t *evicted, void *stream) {
  return step_impl(L, new_k, new_v, ctr, budget, pyramid_policy(n_sink, rope_base), evicted,
                   kve::MovePool{}, stream);
}

KVE_EXPORT int keyformer_step_layers(int32_t n_layers, const kve_layer *layers,
                                     const void *const *new_k, const void *const *new_v,
                                     kve_counters *ctrs, const int32_t *budgets, int32_t n_sink,
                                     double tau_init, double tau_end, int32_t anneal_steps,
                                     double rope_base, uint64_t seed, int32_t *const *evicted,
                                     void *stream) {
  return batch_impl(n_layers, 1, layers, new_k, new_v, ctrs, budgets,
                    keyformer_policy(n_sink, tau_init, tau_end, anneal_steps, rope_base, seed),
                    evicted, kve::MovePool{}, stream);
}

KVE_EXPORT int pyramid_step_layers(int32_t n_layers, const kve_layer *layers,
                                   const void *const *new_k, const void *const *new_v,
                                   kve_counters *ctrs, const int32_t *budgets, int32_t n_sink,
                                   double rope_base, int32_t *const *evicted, void *stream) {
  return batch_impl(n_layers, 1, layers, new_k, new_v, ctrs, budgets,
                    pyramid_policy(n_sink, rope_base), evicted, kve::MovePool{}, stream);
}

KVE_EXPORT int keyformer_step_tokens(const kve_layer *L, int32_t n_tokens, const void *new_k,
                                     const void *new_v, kve_counters *ctr, int32_t budget,
                                     int32_t n_sink, double tau_init, double tau_end,
                                     int32_t anneal_steps, double rope_base, uint64_t seed,
                                     int32_t *evicted, void *stream) {
  if (!L) return KVE_EINVAL;
  int32_t *ev[1] = {evicted};
  return batch_impl(1, n_tokens, L, &new_k, &new_v, ctr, &budget,
                    keyformer_policy(n_sink, tau_init, tau_end, anneal_steps, rope_base, seed),
                    ev, kve::MovePool{}, stream);
}

KVE_EXPORT int pyramid_step_tokens(const kve_layer *L, int32_t n_tokens, const void *new_k,
                                   const void *new_v, kve_counters *ctr, int32_t budget,
                                   int32_t n_sink, double rope_base, int32_t *evicted,
                                   void *stream) {
  if (!L) return KVE_EINVAL;
  int32_t *ev[1] = {evicted};
  return batch_impl(1, n_tokens, L, &new_k, &new_v, ctr, &budget,
                    pyramid_policy(n_sink, rope_base), ev, kve::MovePool{}, stream);
}

KVE_EXPORT int keyformer_step_layers_tokens(int32_t n_layers, int32_t n_tokens,
                                            const kve_layer *layers, const void *const *new_k,
                                            const void *const *new_v, kve_counters *ctrs,
                                            const int32_t *budgets, int32_t n_sink,
                                            double tau_init, double tau_end,
                                            int32_t anneal_steps, double rope_base,
                                            uint64_t seed, int32_t *const *evicted,
                                            void *stream) {
  return batch_impl(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets,
                    keyformer_policy(n_sink, tau_init, tau_end, anneal_steps, rope_base, seed),
                    evicted, kve::MovePool{}, stream);
}

KVE_EXPORT int pyramid_step_layers_tokens(int32_t n_layers, int32_t n_tokens,
                                          const kve_layer *layers, const void *const *new_k,
                                          const void *const *new_v, kve_counters *ctrs,
                                          const int32_t *budgets, int32_t n_sink,
                                          double rope_base, int32_t *const *evicted,
                                          void *stream) {
  return batch_impl(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets,
                    pyramid_policy(n_sink, rope_base), evicted, kve::MovePool{}, stream);
}

namespace {

// The general entry points' policy, checked field by field.
int policy_from(const kve_policy *policy, Policy &p) {
  if (!policy) return KVE_EINVAL;
  if (policy->score != KVE_SCORE_CUMULATIVE && policy->score != KVE_SCORE_CURRENT)
    return KVE_EINVAL;
  if (policy->gumbel != 0 && policy->gumbel != 1) return KVE_EINVAL;
  p = Policy{};
  p.n_sink = policy->n_sink;
  p.recent = policy->recent;
  p.current = policy->score == KVE_SCORE_CURRENT;
  p.gumbel = policy->gumbel == 1;
  p.tau_init = p.gumbel ? policy->tau_init : 0.0;
  p.tau_end = p.gumbel ? policy->tau_end : 0.0;
  p.anneal_steps = p.gumbel ? policy->anneal_steps : 0;
  p.rope_base = policy->rope_base;
  p.seed = p.gumbel ? policy->seed : 0;
  return KVE_OK;
}

int general_step(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                 const void *const *new_k, const void *const *new_v, kve_counters *ctrs,
                 const int32_t *budgets, const kve_policy *policy, int32_t *const *evicted,
                 const kve::MovePool &pool, void *stream) {
  if (!layers || !new_k || !new_v || !ctrs || !budgets) return KVE_EINVAL;
  Policy p;
  if (policy_from(policy, p) != KVE_OK) return KVE_EINVAL;
  if (n_layers == 1 && n_tokens == 1)        // the per-layer kernel
    return step_impl(&layers[0], new_k[0], new_v[0], &ctrs[0], budgets[0], p,
                     evicted ? evicted[0] : nullptr, pool, stream);
  return batch_impl(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets, p, evicted, pool,
                    stream);
}

// general_step's host checks alone (nothing is enqueued).
int check_general(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                  const void *const *new_k, const void *const *new_v, const kve_counters *ctrs,
                  const int32_t *budgets, const Policy &p) {
  if (!layers || !new_k || !new_v || !ctrs || !budgets) return KVE_EINVAL;
  if (n_layers == 1 && n_tokens == 1)
    return check_policy(p) == KVE_OK &&
                   check_layer(&layers[0], new_k[0], new_v[0], &ctrs[0], budgets[0], p) == KVE_OK
               ? KVE_OK
               : KVE_EINVAL;
  return check_batch(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets, p);
}

}  // namespace

KVE_EXPORT int kve_step(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                        const void *const *new_k, const void *const *new_v, kve_counters *ctrs,
                        const int32_t *budgets, const kve_policy *policy,
                        int32_t *const *evicted, void *stream) {
  return general_step(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets, policy, evicted,
                      kve::MovePool{}, stream);
}

KVE_EXPORT int kve_step_ws(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                           const void *const *new_k, const void *const *new_v,
                           kve_counters *ctrs, const int32_t *budgets, const kve_policy *policy,
                           int32_t *const *evicted, void *workspace, int64_t workspace_bytes,
                           void *stream) {
  if (!layers || n_layers < 1) return KVE_EINVAL;
  kve::MovePool pool;
  if (make_pool(workspace, workspace_bytes, layers[0].d, pool) != KVE_OK) return KVE_EINVAL;
  return general_step(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets, policy, evicted,
                      pool, stream);
}

// The workspace that lets every move of a single-token launch over `caches`
// caches at budgets up to max_budget be handed over: one item and one parked
// row per chunk of the longest move of each cache.
KVE_EXPORT int64_t kve_workspace_size(int64_t caches, int32_t max_budget, int32_t d) {
  if (caches < 1 || caches > INT32_MAX || max_budget < 1 || max_budget > kMaxBudget ||
      (d != 64 && d != 128))
    return -1;
  const int64_t items = caches * (int64_t)kve::max_move_chunks(max_budget);
  if (items > INT32_MAX / 2) return -1;
  return kve::pool_bytes(items, d);
}

// ---------------------------------------------------------------------------
// the entry point that allocates nothing (kve_step_noalloc): the workspace
// of kve_step_ws in a fixed-size array of every device the library runs on
// ---------------------------------------------------------------------------

namespace {

// Device memory of this array exists once per GPU, from the library's load
// until the process ends.  Host code never uses its name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[KVE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 128;

struct ScratchAddress {
  std::once_flag once;
  void *ptr = nullptr;        // device address of `scratch` on this device, or null
};
ScratchAddress g_scratch[kMaxDevices];

// The device address of the scratch array on the current device, looked up on
// the first call on that device (with the device current).
void *scratch_address(int dev) {
  ScratchAddress &a = g_scratch[dev];
  std::call_once(a.once, [&a] {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) a.ptr = p;
    else (void)hipGetLastError();
  });
  return a.ptr;
}

}  // namespace

KVE_EXPORT int kve_step_noalloc(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                                const void *const *new_k, const void *const *new_v,
                                kve_counters *ctrs, const int32_t *budgets,
                                const kve_policy *policy, int32_t *const *evicted,
                                void *stream) {
  if (!layers || !budgets || n_layers < 1 || n_layers > kve::kMaxBatchLayers) return KVE_EINVAL;
  Policy p;
  if (policy_from(policy, p) != KVE_OK) return KVE_EINVAL;
  // the scratch the call would use: every long move handed over, as with
  // kve_workspace_size's workspace
  int64_t caches = 0;
  int32_t max_budget = 1;
  for (int32_t l = 0; l < n_layers; ++l) {
    caches += layers[l].bh > 0 ? layers[l].bh : 0;
    max_budget = std::max(max_budget, budgets[l]);
  }
  const bool hands_over = n_tokens == 1 && defers(p, caches);
  if (!hands_over)                             // needs no scratch: kve_step
    return general_step(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets, policy,
                        evicted, kve::MovePool{}, stream);
  // every argument is checked before the size and before any device call
  if (check_general(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets, p) != KVE_OK)
    return KVE_EINVAL;
  const int64_t need = kve_workspace_size(caches, max_budget, layers[0].d);
  if (need < 0) return KVE_EINVAL;
  if (need > (int64_t)KVE_NOALLOC_SCRATCH_BYTES) return KVE_ENOSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return KVE_ENODEV;
  }
  void *ptr = scratch_address(dev);
  if (!ptr) return KVE_ENODEV;
  kve::MovePool pool;
  if (make_pool(ptr, KVE_NOALLOC_SCRATCH_BYTES, layers[0].d, pool) != KVE_OK) return KVE_EINVAL;
  pool.clear_first = 1;                        // the last call on this device left it as it was
  return general_step(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets, policy, evicted,
                      pool, stream);
}

// "The budget schedule": linear taper, mean avg_budget, floor n_sink + 1.
KVE_EXPORT int pyramid_budgets(int32_t n_layers, int32_t avg_budget, int32_t n_sink,
                               double beta, int32_t *out) {
  if (n_layers < 0 || n_sink < 0 || !(beta >= 1.0)) return KVE_EINVAL;
  if (avg_budget < n_sink + 1 || 2.0 * (double)avg_budget > (double)INT32_MAX) return KVE_EINVAL;
  if (n_layers == 0) return KVE_OK;
  if (!out) return KVE_EINVAL;
  if (n_layers == 1) {
    out[0] = avg_budget;
    return KVE_OK;
  }
  const double floor_b = (double)n_sink + 1.0;
  double smallest = (2.0 - beta) * (double)avg_budget;
  if (smallest < floor_b) smallest = floor_b;
  const double largest = 2.0 * (double)avg_budget - smallest;
  for (int32_t l = 0; l < n_layers; ++l) {
    const double x = largest + ((smallest - largest) * (double)l) / (double)(n_layers - 1);
    double r = std::nearbyint(x);                 // default rounding: nearest, ties to even
    if (r < floor_b) r = floor_b;
    out[l] = (int32_t)r;
  }
  return KVE_OK;
}

// return_indices (keyformer_update_batched): replay the call's evictions on
// the chronological index list of prior + new rows.
KVE_EXPORT int32_t kve_kept_indices(int32_t n_prev, int32_t n_tokens, const int32_t *evicted,
                                    int32_t *out) {
  if (n_prev < 0 || n_tokens < 0 || (int64_t)n_prev + n_tokens > INT32_MAX) return KVE_EINVAL;
  if ((n_tokens > 0 && !evicted) || ((int64_t)n_prev + n_tokens > 0 && !out)) return KVE_EINVAL;
  int32_t n = n_prev;
  for (int32_t i = 0; i < n_prev; ++i) out[i] = i;
  for (int32_t t = 0; t < n_tokens; ++t) {
    out[n++] = n_prev + t;                    // the append
    const int32_t e = evicted[t];
    if (e < -1 || e >= n) return KVE_EINVAL;
    if (e >= 0) {                             // later rows move down one slot
      for (int32_t j = e; j < n - 1; ++j) out[j] = out[j + 1];
      --n;
    }
  }
  return n;
}

// keyformer_fp16_bytes / full_keyformer_fp16_bytes: K + V in fp16.
KVE_EXPORT int64_t kve_fp16_bytes(int64_t n_kept, int32_t d) {
  if (n_kept < 0 || d < 1 || n_kept > INT64_MAX / 4 / d) return -1;
  return 4 * n_kept * d;
}

KVE_EXPORT int64_t kve_full_fp16_bytes(int64_t tokens_seen, int32_t d) {
  return kve_fp16_bytes(tokens_seen, d);
}

KVE_EXPORT const char *kve_strerror(int code) {
  switch (code) {
    case KVE_OK: return "ok";
    case KVE_EINVAL: return "invalid argument";
    case KVE_ELAUNCH: return "kernel launch failed";
    case KVE_ENODEV: return "no gfx950 HIP device";
    case KVE_ENOSPACE:
      return "the call needs more scratch than kve_step_noalloc's fixed device buffer holds";
    default: return "unknown error";
  }
}
