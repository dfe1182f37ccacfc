// kve_step.h -- internal interface between the C ABI (kve_api.hip) and the
// gfx950 kernels (kve_step.hip).  Not installed; callers use include/kve.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kve_move_plan.h"

namespace kve {

constexpr int kMaxHalfD = 64;        // d <= 128
constexpr int kMaxBatchLayers = 128; // layers in one batched call
constexpr int kMaxTokens = 128;      // tokens in one multi-token call
constexpr int kMaxRows = 12288;      // largest budget: rows a cache may hold before a step

// fp32 cosine / sine of one rotation angle per RoPE pair, computed in fp64
// and rounded once.
struct RopeTable {
  float c[kMaxHalfD];
  float s[kMaxHalfD];
};

// Workgroups of the move kernel that share a queue longer than its grid.
#ifndef KVE_MOVE_STREAMS
#define KVE_MOVE_STREAMS 256
#endif
constexpr int kMoveStreams = KVE_MOVE_STREAMS;

// One chunk of a compaction handed from a step to the move kernel that
// follows it: of the cache whose rows e+1 .. n-1 move down one slot, chunk j
// (destination rows e + j*kMoveChunk .. up to n-2).  k == nullptr marks an
// item reserved by a step that then found the pool full (skipped).
struct MoveItem {
  void *k;                 // the cache's row 0 (keys)
  void *v;                 // the cache's row 0 (values)
  int32_t e;               // evicted row
  int32_t n;               // rows stored before the step
  int32_t base;            // the cache's first item: its parked rows are base .. base+chunks-1
  int32_t j;               // chunk
};

// The caller-owned workspace of a single-token launch that hands its long
// compactions to the move kernel.  A step that moves more than kDeferRows
// rows reserves one item per chunk with a vector atomic on count[0]: item
// base + j holds chunk j, and parked row base + j holds what the move would
// otherwise race on -- row 0 the incoming row (its key already rotated to
// its final slot), row j >= 1 row e + j*kMoveChunk as it was before the move
// (the first destination of chunk j, read by chunk j-1).  A reservation that
// does not fit in `cap` items compacts in place instead.  The move kernel
// works through the items; the header's counters and phase (the move plan)
// leave the next call's counter at zero, so nothing is cleared between
// calls and no host state is kept.
struct MovePool {
  int32_t *count;          // header words: counters, phase, launch phase (the move plan)
  MoveItem *items;         // [cap]; null pointer: every step compacts its own cache
  void *rows;              // fp16 [cap][2][d]: parked key then value of each item
  int32_t cap;             // items (and parked rows) the workspace holds
  int32_t clear_first;     // host only: zero the header before the step launch
};

// Workspace layout for `cap` items of head dimension d: counters, items,
// parked rows, each part 256-byte aligned.
constexpr int64_t kPoolHeaderBytes = 256;
inline int64_t pool_items_bytes(int64_t cap) { return (cap * (int64_t)sizeof(MoveItem) + 255) & ~(int64_t)255; }
inline int64_t pool_bytes(int64_t cap, int d) { return kPoolHeaderBytes + pool_items_bytes(cap) + cap * 4 * (int64_t)d; }
// The largest item count a workspace of `bytes` bytes holds (0 if none).
inline int64_t pool_capacity(int64_t bytes, int d) {
  if (bytes < kPoolHeaderBytes) return 0;
  int64_t cap = (bytes - kPoolHeaderBytes) / ((int64_t)sizeof(MoveItem) + 4 * (int64_t)d);
  while (cap > 0 && pool_bytes(cap, d) > bytes) --cap;
  return cap;
}

// One layer of a step: its B*H caches and where the incoming rows are.
struct LayerArgs {
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
  int32_t next_pos;
  int32_t pos;
  int32_t hh_base;         // Gumbel stream of cache 0
  int32_t block0;          // first workgroup of this layer in a batched launch
  int32_t n_tokens;        // tokens stepped by this launch (descriptor-driven kernel)
};

// What every layer of a launch shares.
struct SharedArgs {
  int32_t n_sink;
  int32_t recent;          // trailing rows never evicted (0 = off)
  int32_t current;         // 1: score = this step's weight (TOVA), 0: += (H2O / Keyformer)
  int32_t anneal_steps;
  int32_t early;           // 1: load the old scores before the key pass (set per launch)
  MovePool pool;           // long compactions handed to the move kernel (single tokens)
  double tau_init;
  double tau_end;
  uint64_t seed;
  float scale;             // 1 / sqrt(d) in fp32
  RopeTable back1;         // rotation by -1 position (moved stored rows)
  double freq[kMaxHalfD];  // RoPE pair frequencies base^(-2j/d), fp64 from the host; the
                           // incoming row's rotation is evaluated from them on the device
};

// One layer per launch: everything by value.
hipError_t launch_step(const LayerArgs &la, const SharedArgs &sa, int bh, int d, bool gumbel,
                       hipStream_t stream);

// Up to kLaunchLayers layer descriptors, passed by value with a launch (in
// the kernel-argument segment: no copy of its own, nothing to allocate).
constexpr int kLaunchLayers = 32;
struct LayerPack {
  LayerArgs l[kLaunchLayers];
};

// Several layers and/or several tokens per launch: `layers` is device memory;
// layer l steps layers[l].n_tokens tokens (n_tokens, the same for every
// layer), token t reading its incoming rows at new_k + t*bh*d and writing
// evicted + t*bh.
hipError_t launch_step_layers(const LayerPack &layers, int n_layers, int total_blocks,
                              int max_n_prev, int n_tokens, const SharedArgs &sa, int d,
                              bool gumbel, hipStream_t stream);

// Whether such a launch reads the keys with ordinary (cached) loads rather
// than non-temporal ones.
bool reuse_keys(int total_blocks, int max_n_prev, int n_tokens, int d);

// The move kernel: finishes the compactions that a single-token launch with
// sa.pool.items set handed over, and zeroes the pool's counters.  Must run
// after it on the same stream.
hipError_t launch_moves(const MovePool &pool, const RopeTable &back1, int d, hipStream_t stream);

// Zeroes the pool's header words (a scratch whose contents are unknown), in
// stream order before a step launch that uses it.
hipError_t launch_pool_clear(const MovePool &pool, hipStream_t stream);

}  // namespace kve
