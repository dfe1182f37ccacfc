// kve_step.h -- internal interface between the C ABI (kve_api.hip) and the
// gfx950 kernel (kve_step.hip).  Not installed; callers use include/kve.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kve {

constexpr int kMaxHalfD = 64;   // d <= 128

// fp32 cosine / sine of the rotation angles the step may need, computed on
// the host in fp64 and rounded once: rotating a moved row back by one
// position, and rotating the incoming row from next_pos to its final slot.
struct RopeTables {
  float cos_m1[kMaxHalfD];
  float sin_m1[kMaxHalfD];
  float cos_new[kMaxHalfD];
  float sin_new[kMaxHalfD];
};

struct StepArgs {
  void *k;                 // fp16 [bh][cap][d]
  void *v;                 // fp16 [bh][cap][d]
  float *scores;           // [bh][cap]
  float *gumbel;           // [bh][cap] (keyformer only)
  int32_t *positions;      // [bh][cap]
  const void *new_k;       // fp16 [bh][d]
  const void *new_v;       // fp16 [bh][d]
  int32_t *evicted;        // [bh] or null
  int32_t cap;
  int32_t n_prev;
  int32_t budget;
  int32_t n_sink;
  int32_t next_pos;
  int32_t pos;
  int32_t anneal_steps;
  int32_t hh_base;
  double tau_init;
  double tau_end;
  uint64_t seed;
  float scale;             // 1 / sqrt(d) in fp32
  RopeTables rope;
};

hipError_t launch_step(const StepArgs &a, int bh, int d, bool gumbel, hipStream_t stream);

}  // namespace kve
