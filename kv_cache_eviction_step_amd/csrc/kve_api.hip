// kve_api.hip -- host side of the C ABI declared in include/kve.h:
// argument checks, the eviction policy, fp64 rotation constants and
// frequencies, the launches on the caller's stream, the counter update, the
// move scratch of large single-token launches, and the host-only helpers
// (pyramid budget schedule, kept indices, byte accounting).
#include <hip/hip_runtime.h>

#include <atomic>
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
// by -1 position, for the last (d, base) seen on this thread.
struct FreqCache {
  int d = 0;
  double base = 0.0;
  double freq[kve::kMaxHalfD];
  float cos_m1[kve::kMaxHalfD];
  float sin_m1[kve::kMaxHalfD];
};
thread_local FreqCache tl_freq;

const FreqCache &freqs(int d, double base) {
  FreqCache &c = tl_freq;
  if (c.d != d || c.base != base) {
    for (int j = 0; j < d / 2; ++j) {
      c.freq[j] = std::pow(base, -(2.0 * (double)j) / (double)d);
      const double th = -1.0 * c.freq[j];
      c.cos_m1[j] = (float)std::cos(th);
      c.sin_m1[j] = (float)std::sin(th);
    }
    c.d = d;
    c.base = base;
  }
  return c;
}

int check_device() {
  static std::atomic<int> state[128];        // 0 unknown, 1 gfx950, -1 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 128) return KVE_ENODEV;
  int s = state[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KVE_ENODEV;
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    state[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? KVE_OK : KVE_ENODEV;
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

kve::SharedArgs shared_args(int d, const Policy &p) {
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
  // keyformer FIXED GAP #2: moved stored rows go back one position
  const FreqCache &fc = freqs(d, p.rope_base);
  for (int j = 0; j < d / 2; ++j) {
    sa.back1.c[j] = fc.cos_m1[j];
    sa.back1.s[j] = fc.sin_m1[j];
    // The incoming row, if it survives an older row's eviction, goes from
    // next_pos to slot n-1: the device rotates it by (n-1-next_pos) * freq[j]
    // with an fp64 sincos rounded once to fp32.
    sa.freq[j] = fc.freq[j];
  }
  return sa;
}

void advance(kve_counters *ctr, int32_t budget) {
  ctr->n_kept = ctr->n_kept + 1 > budget ? budget : ctr->n_kept + 1;
  ctr->next_pos += 1;
  ctr->pos += 1;
}

// ---------------------------------------------------------------------------
// deferred compactions: single-token launches that hand their long moves to
// the move kernel (kve_step.h) park rows in a per-device scratch
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

// Parked rows per workgroup for budgets up to `budget`: the chunks of the
// longest move (at most budget - 1 rows).
int defer_slots(int32_t budget) {
  return std::max(1, (budget - 1 + kve::kMoveChunk - 1) / kve::kMoveChunk);
}

struct MoveScratch {
  std::mutex mu;
  void *rows = nullptr;
  kve::MoveItem *items = nullptr;
  int32_t *count = nullptr;      // [2], zero when allocated
  int64_t rows_cap = 0;          // bytes
  int64_t items_cap = 0;         // items
  int parity = 0;                // the counter the next launch appends to
  hipEvent_t done = nullptr;     // the last move kernel that used the scratch has finished
  hipStream_t last = nullptr;    // ... on this stream
  bool used = false;
  // A launch that queued moves without its move kernel (a failed launch or
  // event record) leaves a count that no kernel clears: the device then never
  // hands moves over again.
  bool broken = false;
};

void free_moves(MoveScratch &s) {
  (void)hipFree(s.rows);
  (void)hipFree(s.items);
  (void)hipFree(s.count);
  s.rows = nullptr;
  s.items = nullptr;
  s.count = nullptr;
  s.rows_cap = s.items_cap = 0;
  s.parity = 0;
  s.used = false;
}

MoveScratch g_moves[128];

// The scratch for `blocks` workgroups with `slots` parked rows of dimension d,
// ordered after its previous user; false if none can be had (the launch then
// compacts every cache itself).  s.mu must be held until finish_moves.
bool move_scratch(MoveScratch &s, int64_t blocks, int slots, int d, hipStream_t stream,
                  kve::DeferArgs &out) {
  const int64_t rows_bytes = blocks * slots * 4 * (int64_t)d;
  const int64_t items = blocks * slots;
  if (!s.done && hipEventCreateWithFlags(&s.done, hipEventDisableTiming) != hipSuccess) {
    s.done = nullptr;
    return false;
  }
  if (rows_bytes > s.rows_cap || items > s.items_cap) {
    const int64_t nr = std::max(rows_bytes, 2 * s.rows_cap);
    const int64_t ni = std::max(items, 2 * s.items_cap);
    if (s.rows) {                               // launches in flight may still read them
      if (hipDeviceSynchronize() != hipSuccess) return false;
      free_moves(s);
    }
    if (hipMalloc(&s.rows, nr) != hipSuccess ||
        hipMalloc(reinterpret_cast<void **>(&s.items), ni * sizeof(kve::MoveItem)) !=
            hipSuccess ||
        hipMalloc(reinterpret_cast<void **>(&s.count), 2 * sizeof(int32_t)) != hipSuccess ||
        hipMemset(s.count, 0, 2 * sizeof(int32_t)) != hipSuccess) {
      free_moves(s);
      return false;
    }
    s.rows_cap = nr;
    s.items_cap = ni;
  }
  if (s.used && s.last != stream && hipStreamWaitEvent(stream, s.done, 0) != hipSuccess)
    return false;
  out.rows = s.rows;
  out.items = s.items;
  out.count = s.count;
  out.slots = slots;
  out.parity = s.parity;
  return true;
}

// The move kernel after a launch that handed moves over, and the record that
// later users of the scratch wait for.
int finish_moves(MoveScratch &s, const kve::SharedArgs &sa, int64_t blocks, int d,
                 hipStream_t stream) {
  if (kve::launch_moves(sa.defer, (int)blocks, sa.back1, d, stream) != hipSuccess ||
      hipEventRecord(s.done, stream) != hipSuccess) {
    s.broken = true;
    return KVE_ELAUNCH;
  }
  s.last = stream;
  s.used = true;
  s.parity ^= 1;
  return KVE_OK;
}

// The scratch of the current device for a launch of `blocks` workgroups at
// budgets up to `budget`, taken (lock held) when the launch hands moves over.
// A stream under capture never hands moves over: the queue counter's parity
// alternates on the host per call, and a replayed graph would keep reusing
// one parity, so its count would never be cleared.  Such launches compact in
// place, as launches below the threshold always do.
MoveScratch *take_moves(const Policy &p, int64_t blocks, int32_t budget, int d,
                        hipStream_t stream, std::unique_lock<std::mutex> &lock,
                        kve::SharedArgs &sa) {
  int dev = 0;
  if (!defers(p, blocks) || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 128)
    return nullptr;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess ||
      capture != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();                  // so the launch check does not report it
    return nullptr;
  }
  lock = std::unique_lock<std::mutex>(g_moves[dev].mu);
  if (!g_moves[dev].broken &&
      move_scratch(g_moves[dev], blocks, defer_slots(budget), d, stream, sa.defer))
    return &g_moves[dev];
  sa.defer = kve::DeferArgs{};
  lock.unlock();
  return nullptr;
}

// One layer, one token: the descriptor travels by value with the launch.
int step_impl(const kve_layer *L, const void *new_k, const void *new_v, kve_counters *ctr,
              int32_t budget, const Policy &p, int32_t *evicted, void *stream) {
  if (check_policy(p) != KVE_OK) return KVE_EINVAL;
  if (check_layer(L, new_k, new_v, ctr, budget, p) != KVE_OK) return KVE_EINVAL;
  const int dev_state = check_device();
  if (dev_state != KVE_OK) return dev_state;

  const kve::LayerArgs la = layer_args(L, new_k, new_v, ctr, budget, evicted, p.gumbel);
  kve::SharedArgs sa = shared_args(L->d, p);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::unique_lock<std::mutex> lock;
  // a step under its budget evicts nothing, so it has no move to hand over
  MoveScratch *ms =
      ctr->n_kept + 1 > budget ? take_moves(p, L->bh, budget, L->d, s, lock, sa) : nullptr;
  if (kve::launch_step(la, sa, L->bh, L->d, p.gumbel, s) != hipSuccess) return KVE_ELAUNCH;
  if (ms && finish_moves(*ms, sa, L->bh, L->d, s) != KVE_OK) return KVE_ELAUNCH;
  advance(ctr, budget);
  return KVE_OK;
}

// ---------------------------------------------------------------------------
// batched calls: up to kLaunchLayers layer descriptors travel by value with
// each launch; a call over more layers is several launches (layers never
// exchange data, so any grouping gives the same bits)
// ---------------------------------------------------------------------------

// Descriptor-driven launches: n_layers layers, each stepped n_tokens tokens.
// Checks every layer first.
int batch_impl(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
               const void *const *new_k, const void *const *new_v, kve_counters *ctrs,
               const int32_t *budgets, const Policy &p, int32_t *const *evicted, void *stream) {
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
  const int dev_state = check_device();
  if (dev_state != KVE_OK) return dev_state;

  const kve::SharedArgs shared = shared_args(d, p);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int32_t g0 = 0; g0 < n_layers; g0 += kve::kLaunchLayers) {
    const int32_t g1 = std::min(n_layers, g0 + kve::kLaunchLayers);
    kve::LayerPack pack{};
    int32_t block0 = 0, max_n = 0, max_budget = 1;
    bool evicts = false;                      // some layer is at its budget
    for (int32_t l = g0; l < g1; ++l) {
      kve::LayerArgs &a = pack.l[l - g0];
      a = layer_args(&layers[l], new_k[l], new_v[l], &ctrs[l], budgets[l],
                     evicted ? evicted[l] : nullptr, p.gumbel);
      a.block0 = block0;
      a.n_tokens = n_tokens;
      block0 += layers[l].bh;
      max_n = std::max(max_n, std::min(ctrs[l].n_kept + n_tokens - 1, budgets[l]));
      max_budget = std::max(max_budget, budgets[l]);
      evicts = evicts || ctrs[l].n_kept + 1 > budgets[l];
    }
    kve::SharedArgs sa = shared;
    std::unique_lock<std::mutex> move_lock;
    MoveScratch *ms = n_tokens == 1 && evicts
                          ? take_moves(p, block0, max_budget, d, s, move_lock, sa)
                          : nullptr;
    if (kve::launch_step_layers(pack, g1 - g0, block0, max_n, n_tokens, sa, d, p.gumbel, s) !=
        hipSuccess)
      return KVE_ELAUNCH;
    if (ms && finish_moves(*ms, sa, block0, d, s) != KVE_OK) return KVE_ELAUNCH;
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
                   evicted, stream);
}

KVE_EXPORT int pyramid_step(const kve_layer *L, const void *new_k, const void *new_v,
                            kve_counters *ctr, int32_t budget, int32_t n_sink,
                            double rope_base, int32_t *evicted, void *stream) {
  return step_impl(L, new_k, new_v, ctr, budget, pyramid_policy(n_sink, rope_base), evicted,
                   stream);
}

KVE_EXPORT int keyformer_step_layers(int32_t n_layers, const kve_layer *layers,
                                     const void *const *new_k, const void *const *new_v,
                                     kve_counters *ctrs, const int32_t *budgets, int32_t n_sink,
                                     double tau_init, double tau_end, int32_t anneal_steps,
                                     double rope_base, uint64_t seed, int32_t *const *evicted,
                                     void *stream) {
  return batch_impl(n_layers, 1, layers, new_k, new_v, ctrs, budgets,
                    keyformer_policy(n_sink, tau_init, tau_end, anneal_steps, rope_base, seed),
                    evicted, stream);
}

KVE_EXPORT int pyramid_step_layers(int32_t n_layers, const kve_layer *layers,
                                   const void *const *new_k, const void *const *new_v,
                                   kve_counters *ctrs, const int32_t *budgets, int32_t n_sink,
                                   double rope_base, int32_t *const *evicted, void *stream) {
  return batch_impl(n_layers, 1, layers, new_k, new_v, ctrs, budgets,
                    pyramid_policy(n_sink, rope_base), evicted, stream);
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
                    ev, stream);
}

KVE_EXPORT int pyramid_step_tokens(const kve_layer *L, int32_t n_tokens, const void *new_k,
                                   const void *new_v, kve_counters *ctr, int32_t budget,
                                   int32_t n_sink, double rope_base, int32_t *evicted,
                                   void *stream) {
  if (!L) return KVE_EINVAL;
  int32_t *ev[1] = {evicted};
  return batch_impl(1, n_tokens, L, &new_k, &new_v, ctr, &budget,
                    pyramid_policy(n_sink, rope_base), ev, stream);
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
                    evicted, stream);
}

KVE_EXPORT int pyramid_step_layers_tokens(int32_t n_layers, int32_t n_tokens,
                                          const kve_layer *layers, const void *const *new_k,
                                          const void *const *new_v, kve_counters *ctrs,
                                          const int32_t *budgets, int32_t n_sink,
                                          double rope_base, int32_t *const *evicted,
                                          void *stream) {
  return batch_impl(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets,
                    pyramid_policy(n_sink, rope_base), evicted, stream);
}

KVE_EXPORT int kve_step(int32_t n_layers, int32_t n_tokens, const kve_layer *layers,
                        const void *const *new_k, const void *const *new_v, kve_counters *ctrs,
                        const int32_t *budgets, const kve_policy *policy,
                        int32_t *const *evicted, void *stream) {
  if (!policy || !layers || !new_k || !new_v || !ctrs || !budgets) return KVE_EINVAL;
  if (policy->score != KVE_SCORE_CUMULATIVE && policy->score != KVE_SCORE_CURRENT)
    return KVE_EINVAL;
  if (policy->gumbel != 0 && policy->gumbel != 1) return KVE_EINVAL;
  Policy p;
  p.n_sink = policy->n_sink;
  p.recent = policy->recent;
  p.current = policy->score == KVE_SCORE_CURRENT;
  p.gumbel = policy->gumbel == 1;
  p.tau_init = p.gumbel ? policy->tau_init : 0.0;
  p.tau_end = p.gumbel ? policy->tau_end : 0.0;
  p.anneal_steps = p.gumbel ? policy->anneal_steps : 0;
  p.rope_base = policy->rope_base;
  p.seed = p.gumbel ? policy->seed : 0;
  if (n_layers == 1 && n_tokens == 1)        // the per-layer kernel
    return step_impl(&layers[0], new_k[0], new_v[0], &ctrs[0], budgets[0], p,
                     evicted ? evicted[0] : nullptr, stream);
  return batch_impl(n_layers, n_tokens, layers, new_k, new_v, ctrs, budgets, p, evicted, stream);
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
    default: return "unknown error";
  }
}
