// kve_step.h -- internal interface between the C ABI (kve_api.hip) and the
// gfx950 kernels (kve_step.hip).  Not installed; callers use include/kve.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Rows per chunk of a deferred compaction (one workgroup of the move kernel
// each), and the longest move a step still does itself.
// (Tuning builds may override the second with -D.)
constexpr int kMoveChunk = 64;
#ifndef KVE_DEFER_ROWS
#define KVE_DEFER_ROWS (2 * kMoveChunk)
#endif
constexpr int kDeferRows = KVE_DEFER_ROWS;
// Workgroups of the move kernel that share a queue longer than its grid.
#ifndef KVE_MOVE_STREAMS
#define KVE_MOVE_STREAMS 256
#endif
constexpr int kMoveStreams = KVE_MOVE_STREAMS;

// One chunk of a compaction handed from a step to the move kernel that
// follows it: of the cache whose rows e+1 .. n-1 move down one slot, chunk j
// (destination rows e + j*kMoveChunk .. up to n-2).
struct MoveItem {
  void *k;                 // the cache's row 0 (keys)
  void *v;                 // the cache's row 0 (values)
  int32_t e;               // evicted row
  int32_t n;               // rows stored before the step
  int32_t b;               // workgroup of the step (its scratch rows)
  int32_t j;               // chunk
};

// Deferred compactions of one launch: per workgroup `slots` rows of key +
// value (2d fp16 each) -- slot 0 the incoming row (its key already rotated to
// its final position), slot j >= 1 row e + j*kMoveChunk as it was before the
// move (the first destination of move chunk j, read by chunk j-1) -- and the
// queue of chunks, appended at count[parity].  The move kernel works through
// them and zeroes count[1 - parity], which the launch before it used, so the
// next launch (the other parity) starts from zero.
struct DeferArgs {
  MoveItem *items;         // [workgroups * slots]; null: every step compacts its own cache
  void *rows;              // fp16 [workgroups][slots][2][d]
  int32_t *count;          // [2]: items queued, by parity
  int32_t slots;           // >= the chunks of the longest possible move
  int32_t parity;          // 0 or 1, alternating between launches
};

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
  DeferArgs defer;         // long compactions handed to the move kernel (single tokens)
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
// sa.defer.items set handed over (`blocks` = that launch's workgroups).  Must
// run after it on the same stream.
hipError_t launch_moves(const DeferArgs &defer, int blocks, const RopeTable &back1, int d,
                        hipStream_t stream);

}  // namespace kve
