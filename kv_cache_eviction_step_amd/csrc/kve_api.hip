// kve_api.hip -- host side of the C ABI declared in include/kve.h:
// argument checks, fp64 rotation tables, the launch on the caller's stream,
// the counter update, and the pyramid budget schedule.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kve.h"
#include "kve_step.h"

#define KVE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// Largest budget a cache may have: the kernel keeps two fp32 values per
// stored row in LDS (at most 128 KiB of gfx950's 160 KiB).
constexpr int32_t kMaxBudget = 16384;

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

int step_impl(const kve_layer *L, const void *new_k, const void *new_v, kve_counters *ctr,
              int32_t budget, int32_t n_sink, double tau_init, double tau_end,
              int32_t anneal_steps, double rope_base, uint64_t seed, int32_t *evicted,
              void *stream, bool gumbel) {
  // ---- host-side checks (init_keyformer_state's guards and the layout) ----
  if (!L || !ctr || !new_k || !new_v) return KVE_EINVAL;
  if (!L->k || !L->v || !L->scores || !L->positions) return KVE_EINVAL;
  if (gumbel && !L->gumbel) return KVE_EINVAL;
  if (!aligned16(L->k) || !aligned16(L->v) || !aligned16(new_k) || !aligned16(new_v))
    return KVE_EINVAL;
  if (L->d != 64 && L->d != 128) return KVE_EINVAL;
  if (L->bh < 1 || L->hh_base < 0 || (int64_t)L->hh_base + L->bh > INT32_MAX) return KVE_EINVAL;
  if (n_sink < 0 || budget <= n_sink || budget > kMaxBudget) return KVE_EINVAL;
  if (L->cap < budget + 1) return KVE_EINVAL;
  if (!(tau_init >= 0.0) || !(tau_end >= 0.0) || !std::isfinite(tau_init) ||
      !std::isfinite(tau_end) || anneal_steps < 0)
    return KVE_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return KVE_EINVAL;
  const int32_t n = ctr->n_kept;
  if (n < 0 || n > budget) return KVE_EINVAL;
  if (ctr->pos < 0 || ctr->next_pos < n || ctr->next_pos == INT32_MAX || ctr->pos == INT32_MAX)
    return KVE_EINVAL;
  const bool over = n + 1 > budget;
  // without an eviction the new row keeps next_pos, which must equal its slot
  if (!over && ctr->next_pos != n) return KVE_EINVAL;

  const int dev = check_device();
  if (dev != KVE_OK) return dev;

  kve::StepArgs a;
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
  a.n_prev = n;
  a.budget = budget;
  a.n_sink = n_sink;
  a.next_pos = ctr->next_pos;
  a.pos = ctr->pos;
  a.anneal_steps = anneal_steps;
  a.hh_base = L->hh_base;
  a.tau_init = gumbel ? tau_init : 0.0;
  a.tau_end = gumbel ? tau_end : 0.0;
  a.seed = seed;
  a.scale = (float)(1.0 / std::sqrt((double)L->d));
  if (over) {
    // keyformer FIXED GAP #2: moved rows go back one position; the incoming
    // row, if it survives an older row's eviction, goes from next_pos to n-1
    const FreqCache &fc = freqs(L->d, rope_base);
    const double delta_new = (double)(n - 1) - (double)ctr->next_pos;
    for (int j = 0; j < L->d / 2; ++j) {
      a.rope.cos_m1[j] = fc.cos_m1[j];
      a.rope.sin_m1[j] = fc.sin_m1[j];
      const double th = delta_new * fc.freq[j];
      a.rope.cos_new[j] = (float)std::cos(th);
      a.rope.sin_new[j] = (float)std::sin(th);
    }
  }

  const hipError_t err =
      kve::launch_step(a, L->bh, L->d, gumbel, reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) return KVE_ELAUNCH;

  ctr->n_kept = over ? budget : n + 1;
  ctr->next_pos += 1;
  ctr->pos += 1;
  return KVE_OK;
}

}  // namespace

KVE_EXPORT int keyformer_step(const kve_layer *L, const void *new_k, const void *new_v,
                              kve_counters *ctr, int32_t budget, int32_t n_sink,
                              double tau_init, double tau_end, int32_t anneal_steps,
                              double rope_base, uint64_t seed, int32_t *evicted,
                              void *stream) {
  return step_impl(L, new_k, new_v, ctr, budget, n_sink, tau_init, tau_end, anneal_steps,
                   rope_base, seed, evicted, stream, true);
}

KVE_EXPORT int pyramid_step(const kve_layer *L, const void *new_k, const void *new_v,
                            kve_counters *ctr, int32_t budget, int32_t n_sink,
                            double rope_base, int32_t *evicted, void *stream) {
  return step_impl(L, new_k, new_v, ctr, budget, n_sink, 0.0, 0.0, 0, rope_base, 0, evicted,
                   stream, false);
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

KVE_EXPORT const char *kve_strerror(int code) {
  switch (code) {
    case KVE_OK: return "ok";
    case KVE_EINVAL: return "invalid argument";
    case KVE_ELAUNCH: return "kernel launch failed";
    case KVE_ENODEV: return "no gfx950 HIP device";
    default: return "unknown error";
  }
}
