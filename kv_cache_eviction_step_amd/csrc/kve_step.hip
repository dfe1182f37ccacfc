// kve_step.hip -- gfx950 kernel of the per-token KV-cache eviction step.
//
// One workgroup owns one cache (one (batch, kv-head) of the layer) for the
// whole step, so no workgroup ever waits for another.  Phases inside the
// workgroup:
//   A  score pass: coalesced 128-bit loads of the stored keys (non-temporal,
//      or cached in a token loop whose keys fit the last-level cache), fp16
//      dot2 products against the incoming key, a DPP reduction over each
//      row's lanes, logits to LDS (a matrix-vector product: bandwidth bound,
//      no MFMA);
//   B  softmax: block max, exponentials and an exact (fixed-point) block sum;
//      each thread holds the old scores / gumbel of its rows in registers,
//      loaded before the score pass in latency-bound launches, else here;
//   C  new scores (fp32 add of the normalised mass, or the mass itself for
//      TOVA) and, when over budget, the eviction key  fma(tau, gumbel, score)
//      over the non-protected rows with a block argmin that breaks ties
//      towards the lowest index;
//   D  write-back: scores / gumbel / positions of the rows after the evicted
//      one move down one slot; keys and values of those rows move in
//      ascending chunks (load all, barrier, store), keys re-rotated by -1
//      position in fp32; the new row lands at its final slot.
//
// Two entry kernels share the body: one layer and one token per launch
// (everything passed by value), or several layers and/or tokens per launch
// (descriptors in device memory, the workgroups of each layer contiguous in
// the grid, each walking its cache through the tokens).  A third kernel
// finishes the long compactions that large single-token launches queue for
// it in a scratch buffer, spreading them over the GPU.
//
// Method (VeloxQuant-MLX pages): "veloxquant_mlx.quantizers.keyformer
// module" -- keyformer_update steps 1-3, KeyformerState, FIXED GAP #1/#2,
// FUSED METAL KERNEL; "PyramidKV -- Layer-Adaptive Budget Attention-Mass
// Eviction" -- How it works.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kve_step.h"

namespace kve {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte chunk
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Global-memory pointer.  The layer descriptors of the batched kernel are read
// from memory, so the compiler cannot tell on its own that their pointers are
// global; without this every access would be a flat one (64-bit address per
// lane, and counted against the LDS wait counter too).
template <typename T>
using gptr = __attribute__((address_space(1))) T *;

template <typename T>
__device__ __forceinline__ gptr<T> global(T *p) {
  return (gptr<T>)p;
}

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// SplitMix64 output function (Steele, Lea & Flood 2014) of state value z.
__device__ __forceinline__ uint64_t splitmix64_out(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Frozen Gumbel value of the row inserted at running position `pos` of
// stream `stream`: counter hash -> uniform in (0,1) -> -log(-log u) in fp64.
// Inlined where it should overlap loads in flight (a call would wait for
// them); called where inlining would put its constants in a loop's registers.
__device__ __forceinline__ float gumbel_value(uint64_t seed, uint64_t stream, uint64_t pos) {
  uint64_t h = splitmix64_out(splitmix64_out(splitmix64_out(seed) ^ stream) ^ pos);
  double u = ((double)(h >> 11) + 0.5) * 0x1p-53;
  return (float)(-log(-log(u)));
}
__device__ __noinline__ float gumbel_at(uint64_t seed, uint64_t stream, uint64_t pos) {
  return gumbel_value(seed, stream, pos);
}

// cos and sin of delta * freq: fp64 sincos, each rounded once to fp32 (the
// incoming row's rotation, keyformer FIXED GAP #2).  Not inlined: its
// polynomial constants would otherwise be hoisted out of the token loop of
// the batched kernel and held in registers for the whole launch.
__device__ __noinline__ f32x2 rotation_at(int32_t delta, double freq) {
  double sv, cv;
  sincos((double)delta * freq, &sv, &cv);
  f32x2 r;
  r.x = (float)cv;
  r.y = (float)sv;
  return r;
}

// Annealed temperature (keyformer FIXED GAP #1), fp64, rounded once.
__device__ __forceinline__ float tau_value(double tau_init, double tau_end, int32_t steps,
                                           int32_t pos) {
#pragma clang fp contract(off)
  if (steps <= 0 || tau_init == tau_end) return (float)tau_init;
  int32_t t = pos < steps ? pos : steps;
  double delta = (tau_end - tau_init) / (double)steps;
  double prod = (double)t * delta;
  return (float)(tau_init + prod);
}
__device__ __noinline__ float anneal_tau(double tau_init, double tau_end, int32_t steps,
                                         int32_t pos) {
  return tau_value(tau_init, tau_end, steps, pos);
}

// One RoPE pair rotated in fp32 with every product and sum rounded on its own.
__device__ __forceinline__ void rotate_pair(float x1, float x2, float c, float s, float &y1,
                                            float &y2) {
#pragma clang fp contract(off)
  float a = x1 * c;
  float b = x2 * s;
  y1 = a - b;
  float e = x2 * c;
  float f = x1 * s;
  y2 = e + f;
}

// A row's new score: its normalised weight w * (1/Z), rounded to fp32 on its
// own, added to the old score (TOVA-adapted: the weight alone).  No fused
// multiply-add: the increment is one rounded value, as the method's
// definition of the accumulated mass reads.
__device__ __forceinline__ float score_update(bool current, float old, float w, float rz) {
#pragma clang fp contract(off)
  const float p = w * rz;
  return current ? p : old + p;
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Rotate the two fp16 elements held in word w1 (first half of the row) with
// their partners in word w2 (second half); angles c[0..1], s[0..1].
__device__ __forceinline__ void rotate_word(uint32_t &w1, uint32_t &w2, const float *c,
                                            const float *s) {
  const half2_t x1 = as_h2(w1), x2 = as_h2(w2);
  float a0, b0, a1, b1;
  rotate_pair((float)x1[0], (float)x2[0], c[0], s[0], a0, b0);
  rotate_pair((float)x1[1], (float)x2[1], c[1], s[1], a1, b1);
  half2_t y1, y2;
  y1[0] = (_Float16)a0;
  y1[1] = (_Float16)a1;
  y2[0] = (_Float16)b0;
  y2[1] = (_Float16)b1;
  w1 = as_u32(y1);
  w2 = as_u32(y2);
}

// Rotate 8 pairs: chunk x1 holds elements j0..j0+7, x2 holds j0+d/2..j0+d/2+7.
__device__ __forceinline__ void rotate_chunk(u32x4 &x1, u32x4 &x2, const float *c,
                                             const float *s) {
  u32x4 y1, y2;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t a = x1[w], b = x2[w];
    rotate_word(a, b, c + 2 * w, s + 2 * w);
    y1[w] = a;
    y2[w] = b;
  }
  x1 = y1;
  x2 = y2;
}

// 8 fp16 products of one 16-byte chunk accumulated in fp32 (v_dot2_f32_f16).
__device__ __forceinline__ float dot8(const u32x4 a, const u32x4 b) {
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2(as_h2(a[w]), as_h2(b[w]), acc, false);
  return acc;
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, x)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// In-row butterfly of the reductions below, one DPP move per step (a VALU
// operation, no LDS traffic): quad_perm [1,0,3,2] and [2,3,0,1] (0xB1, 0x4E:
// partners 1 and 2 lanes away), then half-row mirror (0x141: lane i <-> 7-i of
// each 8) and row mirror (0x140: lane i <-> 15-i of each 16).  After the
// first k steps every lane holds the combination over its aligned group of
// 2^k lanes (k <= 4), for any associative and commutative combination.

// Sum over aligned groups of LANES lanes (4, 8 or 16); every lane gets the sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group");
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  if constexpr (LANES >= 8) x += dpp<0x141>(x);
  if constexpr (LANES == 16) x += dpp<0x140>(x);
  return x;
}

__device__ __forceinline__ float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t x, int l) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
}

// Whole-wave reductions, result uniform across the wave: the in-row butterfly
// (every lane of a row of 16 then holds its row's result), then the four row
// results read from lanes 0, 16, 32, 48 and combined.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
  x += dpp_u64<0xB1>(x);
  x += dpp_u64<0x4E>(x);
  x += dpp_u64<0x141>(x);
  x += dpp_u64<0x140>(x);
  return lane_u64(x, 0) + lane_u64(x, 16) + lane_u64(x, 32) + lane_u64(x, 48);
}

// (value, index) pairs as one 64-bit key whose unsigned order is the pairs'
// order: smaller value first, equal values by the lower index.  The value's
// bits map to an unsigned integer of the same order (non-negative floats get
// the sign bit set, negative ones have every bit flipped); -0 is made +0
// first, so that it ties with +0 as the float comparison has it.  Values are
// never NaN.
__device__ __forceinline__ uint64_t argkey(float v, int i) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)i;
}
__device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return b < a ? b : a; }
template <int CTRL>
__device__ __forceinline__ uint64_t min_dpp_u64(uint64_t x) {
  return min_u64(x, dpp_u64<CTRL>(x));
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
  x = min_dpp_u64<0xB1>(x);
  x = min_dpp_u64<0x4E>(x);
  x = min_dpp_u64<0x141>(x);
  x = min_dpp_u64<0x140>(x);
  return min_u64(min_u64(lane_u64(x, 0), lane_u64(x, 16)),
                 min_u64(lane_u64(x, 32), lane_u64(x, 48)));
}

// Reductions of the W per-wave partials held by lanes 0..W-1 (identity
// elsewhere), done by every wave on its own: the first log2(W) steps of the
// in-row butterfly, then lane 0's value, uniform across the wave.
template <int W>
__device__ __forceinline__ float partials_max(float x) {
  static_assert(W >= 1 && W <= 16 && (W & (W - 1)) == 0, "partials");
  if constexpr (W > 1) x = fmaxf(x, dpp<0xB1>(x));
  if constexpr (W > 2) x = fmaxf(x, dpp<0x4E>(x));
  if constexpr (W > 4) x = fmaxf(x, dpp<0x141>(x));
  if constexpr (W > 8) x = fmaxf(x, dpp<0x140>(x));
  return lane_f(x, 0);
}
template <int W>
__device__ __forceinline__ uint64_t partials_sum(uint64_t x) {
  static_assert(W >= 1 && W <= 16 && (W & (W - 1)) == 0, "partials");
  if constexpr (W > 1) x += dpp_u64<0xB1>(x);
  if constexpr (W > 2) x += dpp_u64<0x4E>(x);
  if constexpr (W > 4) x += dpp_u64<0x141>(x);
  if constexpr (W > 8) x += dpp_u64<0x140>(x);
  return lane_u64(x, 0);
}
template <int W>
__device__ __forceinline__ uint64_t partials_min_u64(uint64_t x) {
  static_assert(W >= 1 && W <= 16 && (W & (W - 1)) == 0, "partials");
  if constexpr (W > 1) x = min_dpp_u64<0xB1>(x);
  if constexpr (W > 2) x = min_dpp_u64<0x4E>(x);
  if constexpr (W > 4) x = min_dpp_u64<0x141>(x);
  if constexpr (W > 8) x = min_dpp_u64<0x140>(x);
  return lane_u64(x, 0);
}

// The softmax normaliser is summed exactly: each weight w in [0, 1] as the
// integer w * 2^40 (exact for w >= 2^-16, rounded to nearest below), so the
// total does not depend on how rows are grouped over lanes and waves (the
// workgroup size), and carries no float rounding of its own.
constexpr float kZScale = 0x1p40f;

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// 16-byte chunks per lane in the score pass of 512-thread workgroups
// (tuning builds may override with -D).
#ifndef KVE_CPL512
#define KVE_CPL512 2
#endif

// Rows each thread moves per chunk of the compaction where two workgroups
// share a compute unit (tuning builds may override with -D); a launch of at
// most one workgroup per compute unit moves two (step_kernel_solo).
#ifndef KVE_MOVE_UNROLL
#define KVE_MOVE_UNROLL 1
#endif

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (gfx9 encoding; expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// x, unchanged, through an empty asm: the optimiser can no longer treat it
// as loop-invariant (wave-uniform values only: the asm takes a scalar register).
template <typename T>
__device__ __forceinline__ T opaque(T x) {
  asm volatile("" : "+s"(x));
  return x;
}

// The same for a per-lane value (vector register).
__device__ __forceinline__ int opaque_lane(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Rotation constants shared by every token of a launch, copied from the
// kernel arguments into LDS once per workgroup by wave 0.  Reading them from
// LDS (not from the argument segment, which the compiler treats as invariant
// and would keep in registers across the token loop) keeps register use low.
__shared__ float lds_back_c[kMaxHalfD];      // rotation by -1 position
__shared__ float lds_back_s[kMaxHalfD];
__shared__ double lds_freq[kMaxHalfD];       // RoPE pair frequencies (fp64)

template <int D>
__device__ __forceinline__ void stage_tables(const SharedArgs &sa) {
  const int tid = threadIdx.x;
  if (tid < D / 2) {                            // wave 0 (readers wait for a barrier)
    lds_back_c[tid] = sa.back1.c[tid];
    lds_back_s[tid] = sa.back1.s[tid];
    lds_freq[tid] = sa.freq[tid];
  }
}

// Per-token values a launch over several tokens evaluates ahead, kTokChunk
// tokens at a time, into LDS: per token, the incoming row's rotation
// (cos[D/2], sin[D/2]), its Gumbel value and tau.
constexpr int kTokChunk = 16;

// The whole step for cache `hh` of layer `la` (one workgroup).  stage_tables
// has run in this workgroup.  PRE: `pre` holds this token's per-token values
// (above); otherwise the step evaluates them itself, each where no memory
// access is in flight (a call there would wait for every outstanding load).
template <int D, int NT, int U, bool GUMBEL, bool PRE, int R, bool REUSE, int UM = KVE_MOVE_UNROLL>
__device__ __forceinline__ void step_body(const LayerArgs &la, const SharedArgs &sa,
                                          const int hh, const float *pre) {
  constexpr int V16 = D / 8;        // 16-byte chunks per row
  // Score pass: CPL chunks of a row per lane -- two, one RoPE pair, at 512
  // threads (less reduction work per byte, which a latency-bound workgroup
  // feels); one at 1024 threads (measured faster there) -- LPR lanes per row.
  // Either way a logit is the same sum, so results do not depend on it: the
  // 8-product partial of every chunk, each pair's two partials added (chunks
  // c and c + D/16), then the pairs combined by the in-row butterfly.  With
  // one chunk per lane (lane c reads chunk c), a first step adds the partner
  // lane c ^ (D/16), and the butterfly over the pairs follows.
  constexpr int CPL = NT >= 1024 ? 1 : KVE_CPL512;
  constexpr int LPR = V16 / CPL;
  constexpr int RPS = NT / LPR;     // score pass: rows per sweep
  constexpr int UR = U / CPL;       // score pass: rows per lane per batch
  constexpr int ROWS_IT = RPS * UR; // score pass: rows per batch of loads
  constexpr int LPM = D / 16;       // move pass: lanes per row (one chunk of each half)
  constexpr int RPM = NT / LPM;     // move pass: rows per sweep
  constexpr int NWAVE = NT / 64;
  static_assert(NT % 64 == 0 && RPS * LPR == NT && RPM * LPM == NT && U % CPL == 0,
                "launch shape");

  // LDS: the logits [np] (then, past 8 slots per thread, the weights).
  // Scores and Gumbel values of the rows i = tid + k*NT, k < R (R*NT >= n),
  // live in this thread's registers.
  extern __shared__ float lds[];
  // one slot per wave for each reduction of the step (written once per step)
  __shared__ float red_m[NWAVE];
  __shared__ uint64_t red_z[NWAVE];
  __shared__ uint64_t red_k[NWAVE];
  __shared__ float rn_c[kMaxHalfD];          // incoming row's rotation (wave 0 only)
  __shared__ float rn_s[kMaxHalfD];

  // In the token loop, per-row offsets derived from the lane index would be
  // hoisted out of the loop and held for the whole launch; re-derive them.
  const int tid = PRE ? opaque_lane(threadIdx.x) : (int)threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = la.n_prev;
  const bool over = n + 1 > la.budget;
  const size_t row0 = (size_t)hh * (size_t)la.cap;     // first row of this cache
  float *__restrict__ lds_x = lds;
  const gptr<float> __restrict__ scores = global(la.scores);
  const gptr<float> __restrict__ gumbel = global(la.gumbel);

  // With the current-step score (TOVA) the old scores are not needed.
  const bool current = sa.current != 0;

  // ---- A: logits of every stored row against the incoming key -------------
  // Lane lr of a row's LPR lanes holds the 16-byte chunks chunk_of(c), c <
  // CPL (each load instruction reads whole 128-byte lines).  Two batches of U
  // loads in flight: batch it+1 is issued before batch it is consumed.  Rows
  // past n are clamped to row n-1 (a cache hit) and dropped.
  const gptr<const u32x4> __restrict__ K4 =
      global(reinterpret_cast<const u32x4 *>(la.k)) + row0 * V16;
  const int lr = tid % LPR;
  const int rr = tid / LPR;
  auto chunk_of = [&](int c) { return lr + c * LPR; };
  const gptr<const u32x4> nk4 =
      global(reinterpret_cast<const u32x4 *>(la.new_k)) + (size_t)hh * V16;
  u32x4 q[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) q[c] = nk4[chunk_of(c)];
  // The incoming row's value chunk `tid` (lanes 0..V16-1 store the row at the
  // end of the step): loaded now, so that no load is left for the step's end.
  u32x4 v_new = {};
  if (tid < V16) v_new = global(reinterpret_cast<const u32x4 *>(la.new_v))[(size_t)hh * V16 + tid];
  // With a workspace: its phase, written by the previous call's move kernel
  // and by nothing during this launch; loaded now (an ordinary load: the
  // workgroups of a compute die share one fetch of it), used only in phase D.
  int pool_phase_in = 0;
  if (!PRE && sa.pool.items != nullptr) pool_phase_in = global(sa.pool.count)[kPoolPhase];
  const float scale = sa.scale;
  float mx = -INFINITY;
  const int iters = (n + ROWS_IT - 1) / ROWS_IT;
  u32x4 bufa[U], bufb[U];
  // A single step reads the key stream once: non-temporal loads keep it from
  // pushing the scores (written back at the end of the step) out of the
  // caches.  When the same caches are stepped through several tokens and
  // their keys fit in the last-level cache (REUSE), ordinary loads let the
  // next token's pass hit there instead of HBM.
  auto load_batch = [&](int it, u32x4 *buf) {
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int r = min(it * ROWS_IT + u * RPS + rr, n - 1);
      const gptr<const u32x4> p = K4 + (size_t)r * V16;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        if constexpr (REUSE)
          buf[u * CPL + c] = p[chunk_of(c)];
        else
          buf[u * CPL + c] = __builtin_nontemporal_load(p + chunk_of(c));
      }
    }
  };
  auto consume = [&](int it, const u32x4 *buf) {
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int r = it * ROWS_IT + u * RPS + rr;
      float part = dot8(buf[u * CPL], q[0]);
      if constexpr (CPL == 2) {
        part += dot8(buf[u * CPL + 1], q[1]);
      } else if constexpr (V16 == 16) {
        part += dpp<0x128>(part);                  // row_ror:8 -- lane c ^ 8 of the row
      } else {
        part += __shfl_xor(part, V16 / 2);
      }
      const float x = group_sum<V16 / 2>(part) * scale;
      if (r < n) {
        if (lr == 0) lds_x[r] = x;
        mx = fmaxf(mx, x);
      }
    }
  };
  // tau and the new row's Gumbel value (one token, not precomputed): inlined
  // here so that they overlap the first key batch's loads.
  float tau = 0.f, g_new = 0.f;
  auto noise = [&]() {
    if constexpr (!PRE) {
      if (GUMBEL && over) tau = tau_value(sa.tau_init, sa.tau_end, sa.anneal_steps, la.pos);
      if (GUMBEL)
        g_new = gumbel_value(sa.seed, (uint64_t)(int64_t)(la.hh_base + hh),
                             (uint64_t)(int64_t)la.pos);
    }
  };
  // The old scores (and, when evicting, Gumbel values) of this thread's rows.
  // In a launch whose workgroups each have a compute unit to themselves the
  // step is a latency chain, and loading them before the key pass hides their
  // latency (with at most 8 slots per thread: larger caches need the registers
  // for the key pass).  Otherwise they are loaded after it, overlapping the
  // normaliser: a launch that streams HBM at full rate runs no faster for the
  // early loads, and measured 1.7 % slower with the key stream cached.  A slot
  // is read only for i < n (and only under the condition it was loaded under).
  const bool early = R <= 8 && sa.early != 0;
  float sreg[R], greg[R];
  auto load_state = [&]() {
    if (!current) {
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int i = tid + k * NT;
        if (i < n) sreg[k] = scores[row0 + i];
      }
    }
    if (GUMBEL && over) {
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int i = tid + k * NT;
        if (i < n) greg[k] = gumbel[row0 + i];
      }
    }
  };
  if (early) load_state();
  if (iters > 0) load_batch(0, bufa);
  __builtin_amdgcn_sched_barrier(0);            // issue the loads before the fp64 work
  noise();
  if constexpr (!PRE) asm volatile("" ::"v"(tau), "v"(g_new));   // evaluate here, not at the use
  // Two register buffers take turns (no copies, so the compiler waits only
  // for the batch being consumed while the next one is in flight).
  if (iters > 0) {
    int it = 0;
    for (; it + 2 < iters; it += 2) {
      load_batch(it + 1, bufb);
      consume(it, bufa);
      load_batch(it + 2, bufa);
      consume(it + 1, bufb);
    }
    if (it + 1 < iters) {
      load_batch(it + 1, bufb);
      consume(it, bufa);
      consume(it + 1, bufb);
    } else {
      consume(it, bufa);
    }
  }

  if (!early) load_state();

  // ---- B: softmax normaliser ------------------------------------------------
  mx = wave_max(mx);
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();                              // also: every logit is in LDS
  mx = partials_max<NWAVE>(lane < NWAVE ? red_m[lane] : -INFINITY);
  // The weights stay in this thread's registers (rows i = tid + k*NT, as the
  // scores) when the slots are few; large caches, whose registers the score
  // slots already fill, keep them in LDS in place of the logits.
  constexpr bool WREG = R <= 8;
  float wreg[WREG ? R : 1];
  uint64_t sum = 0;
  if constexpr (WREG) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int i = tid + k * NT;
      if (i < n) {
        const float w = expf(lds_x[i] - mx);
        wreg[k] = w;
        sum += (uint64_t)rintf(w * kZScale);
      }
    }
  } else {
    for (int i = tid; i < n; i += NT) {
      const float w = expf(lds_x[i] - mx);
      lds_x[i] = w;
      sum += (uint64_t)rintf(w * kZScale);
    }
  }
  sum = wave_sum_u64(sum);
  if (lane == 0) red_z[wave] = sum;
  __syncthreads();
  const uint64_t z = partials_sum<NWAVE>(lane < NWAVE ? red_z[lane] : (uint64_t)0);
  const float rz = 1.0f / (float)((double)z * (1.0 / (double)kZScale));

  // ---- C: new scores and the eviction choice --------------------------------
  if constexpr (PRE) {
    if (GUMBEL) g_new = pre[D];
    if (GUMBEL && over) tau = pre[D + 1];
  }
  // Candidates: rows n_sink .. n - recent of the n + 1 rows after the append
  // (sinks and the trailing window protected); the new row (index n) is one
  // only without a window.  The host guarantees the range is not empty.
  const int n_sink = sa.n_sink;
  const int last = n - sa.recent;
  float bv = INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = tid + k * NT;
    if (i < n) {
      const float s = score_update(current, sreg[k], WREG ? wreg[k] : lds_x[i], rz);
      sreg[k] = s;
      if (over && i >= n_sink && i <= last) {
        const float key = GUMBEL ? fmaf(tau, greg[k], s) : s;
        if (key < bv) {                    // rows visited in increasing order
          bv = key;
          bi = i;
        }
      }
    }
  }
  uint64_t best = argkey(bv, bi);
  if (over && tid == 0 && last == n) {     // the new row: score 0
    const float key = GUMBEL ? fmaf(tau, g_new, 0.0f) : 0.0f;
    best = min_u64(best, argkey(key, n));
  }
  best = wave_min_u64(best);
  if (lane == 0) red_k[wave] = best;
  __syncthreads();
  const int arg =
      (int)(uint32_t)partials_min_u64<NWAVE>(lane < NWAVE ? red_k[lane] : ~(uint64_t)0);
  const int e = over ? arg : -1;
  // The incoming row moves (from next_pos to slot n-1) only when an older row
  // was evicted; only then is its rotation needed.
  const float *rot_c = rn_c, *rot_s = rn_s;
  if constexpr (PRE) {
    rot_c = pre;
    rot_s = pre + D / 2;
  } else if (e >= 0 && e < n && wave == 0 && lane < D / 2) {
    const f32x2 r = rotation_at(n - 1 - la.next_pos, lds_freq[lane]);   // staged by this lane
    rn_c[lane] = r.x;
    rn_s[lane] = r.y;
  }
  if (tid == 0 && la.evicted) global(la.evicted)[hh] = e;

  const int pool_phase = __builtin_amdgcn_readfirstlane(pool_phase_in);

  // ---- D: write-back ----------------------------------------------------------
  // A single step writes its state through the L2 (agent-scope relaxed atomic
  // stores, which the L2 writes through at once): written as ordinary stores,
  // the lines stay dirty in the L2 until the key streams of other caches
  // evict them one by one, and each of those lone writes turns an HBM channel
  // around in the middle of the reads.  A token loop re-reads its state on
  // the next token and keeps ordinary stores.
  auto st_state = [](auto x, auto p) {
    if constexpr (REUSE)
      *p = x;
    else
      __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  const gptr<int32_t> __restrict__ positions = global(la.positions);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = tid + k * NT;
    if (i < n) {
      if (e < 0 || i < e) {
        st_state(sreg[k], scores + (row0 + i));
      } else if (i > e) {
        st_state(sreg[k], scores + (row0 + i - 1));
        if constexpr (GUMBEL) st_state(greg[k], gumbel + (row0 + i - 1));
        st_state(i - 1, positions + (row0 + i - 1));
      }
    }
  }

  const gptr<u32x4> __restrict__ Kw = global(reinterpret_cast<u32x4 *>(la.k)) + row0 * V16;
  const gptr<u32x4> __restrict__ Vw = global(reinterpret_cast<u32x4 *>(la.v)) + row0 * V16;
  const int lm = tid % LPM;                     // chunk lm of the first half, lm of the second
  const int rm = tid / LPM;

  // A single-token launch followed by the move kernel hands it every move
  // longer than kDeferRows (the move plan): the step reserves one pool item
  // per chunk, parks the rows that chunks would otherwise race on (each
  // chunk's first destination) and the incoming row, queues the chunks, and
  // the move kernel shifts them in parallel over the GPU instead of one
  // compute unit doing them in turn.  A reservation that does not fit in the
  // pool marks its items empty and compacts in place.
  bool defer = !PRE && sa.pool.items != nullptr && move_handed_over(e, n);
  gptr<u32x4> slot = nullptr;                   // this move's parked rows
  if (!PRE && sa.pool.items != nullptr && blockIdx.x == 0 && tid == 0)
    global(sa.pool.count)[kPoolLaunchPhase] = pool_phase;     // the launch's phase
  if (defer) {
    __shared__ int item_base;
    constexpr int PIECES_EARLY = 2;             // parked 16-byte pieces loaded per thread
    const int chunks = move_chunks(e, n);       //   while the reservation is in flight
    const int pieces = (chunks - 1) * 2 * V16;
    u32x4 pk[PIECES_EARLY];
    auto parked_piece = [&](int i) {            // piece i of parked rows 1 .. chunks-1
      const int j = 1 + i / (2 * V16), w = i % (2 * V16);
      const size_t row = (size_t)parked_row(e, j) * V16;
      return w < V16 ? Kw[row + w] : Vw[row + w - V16];
    };
#pragma unroll
    for (int u = 0; u < PIECES_EARLY; ++u)
      if (tid + u * NT < pieces) pk[u] = parked_piece(tid + u * NT);
    if (tid == 0) item_base = atomicAdd(sa.pool.count + pool_counter(pool_phase), chunks);
    __syncthreads();                            // item_base
    const int base = __builtin_amdgcn_readfirstlane(item_base);
    MoveItem *const items = sa.pool.items;
    if (!reservation_fits(base, chunks, sa.pool.cap)) {
      for (int i = tid; i < chunks; i += NT) {  // the part of the reservation inside the pool
        const int64_t it = (int64_t)base + i;
        if (it >= 0 && it < sa.pool.cap) items[it].k = nullptr;
      }
      defer = false;
    } else {
      slot = global(reinterpret_cast<u32x4 *>(sa.pool.rows)) + (size_t)base * (2 * V16);
      // slot row 0 is the incoming row, rows 1 .. chunks-1 the parked ones
#pragma unroll
      for (int u = 0; u < PIECES_EARLY; ++u)
        if (tid + u * NT < pieces) slot[2 * V16 + tid + u * NT] = pk[u];
      for (int i = tid + PIECES_EARLY * NT; i < pieces; i += NT) slot[2 * V16 + i] = parked_piece(i);
      if (tid < chunks) {
        MoveItem it;
        it.k = static_cast<char *>(la.k) + row0 * (size_t)(2 * D);
        it.v = static_cast<char *>(la.v) + row0 * (size_t)(2 * D);
        it.e = e;
        it.n = n;
        it.base = base;
        it.j = tid;
        items[base + tid] = it;
      }
    }
  }

  // old rows e+1 .. n-1 move to e .. n-2, keys rotated by one position back.
  // Chunks of CH destination rows, software-pipelined: chunk c+1's loads are
  // in flight while chunk c is rotated and stored.  In place and safe: chunk
  // c+1 reads only rows after every row chunk c writes, and chunk c is stored
  // only after every wave's loads of chunk c have landed (wait + barrier).
  // Loads are issued unconditionally (row index clamped to the last source
  // row) so that the explicit wait counts are exact.  The vector-memory
  // counter retires loads and stores in issue order, so once chunk c-1's
  // stores sit between chunk c's loads and chunk c+1's, waiting for chunk c
  // leaves those stores (and chunk c+1's loads) in flight: a chunk never
  // waits for the previous chunk's stores to be acknowledged.
  if (!defer && e >= 0 && e < n - 1) {
    constexpr int CH = RPM * UM;
    constexpr int LOADS = 4 * UM;               // per thread per chunk
    constexpr int STORES = 4 * UM;              // per thread per full chunk
    const int last = n - 2;                     // last destination row
    float cs[8], sn[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cs[j] = lds_back_c[lm * 8 + j];
      sn[j] = lds_back_s[lm * 8 + j];
    }
    u32x4 ak1[UM], ak2[UM], av1[UM], av2[UM];
    u32x4 bk1[UM], bk2[UM], bv1[UM], bv2[UM];
    // 32-bit byte offsets from the cache's first row (a cache is at most
    // kMaxRows + 1 rows of 2D bytes): one address register per access, on
    // top of the cache's uniform base.
    gptr<char> const Kc = reinterpret_cast<gptr<char>>(Kw);
    gptr<char> const Vc = reinterpret_cast<gptr<char>>(Vw);
    auto at = [](gptr<char> base, uint32_t off) {
      return reinterpret_cast<gptr<u32x4>>(base + off);
    };
    // Moved rows are next read by the next step's key pass.  Unless that
    // pass can find them in the last-level cache (REUSE), the move streams
    // them non-temporally, like the key pass itself (measured: 3 % faster
    // launches where interior evictions are common).
    auto ld = [](gptr<u32x4> p) {
      if constexpr (REUSE)
        return *p;
      else
        return __builtin_nontemporal_load(p);
    };
    auto st = [](u32x4 x, gptr<u32x4> p) {
      if constexpr (REUSE)
        *p = x;
      else
        __builtin_nontemporal_store(x, p);
    };
    auto load_chunk = [&](int d0, u32x4 *k1, u32x4 *k2, u32x4 *v1, u32x4 *v2) {
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        const uint32_t src = (uint32_t)(min(d0 + rm + u * RPM, last) + 1) * (2 * D) + lm * 16;
        k1[u] = ld(at(Kc, src));
        k2[u] = ld(at(Kc, src + D));
        v1[u] = ld(at(Vc, src));
        v2[u] = ld(at(Vc, src + D));
      }
    };
    // `full`: every row of the chunk is a destination (all chunks but the
    // last), so the stores need no guard; an unguarded store is never skipped,
    // which keeps the count of stores in flight exact for the wait above it.
    auto store_chunk = [&](int d0, u32x4 *k1, u32x4 *k2, const u32x4 *v1, const u32x4 *v2,
                           bool full) {
#pragma unroll
      for (int u = 0; u < UM; ++u) rotate_chunk(k1[u], k2[u], cs, sn);
      __syncthreads();                          // every wave's loads of this chunk landed
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        const int dst = d0 + rm + u * RPM;
        if (full || dst <= last) {
          const uint32_t o = (uint32_t)dst * (2 * D) + lm * 16;
          st(k1[u], at(Kc, o));
          st(k2[u], at(Kc, o + D));
          st(v1[u], at(Vc, o));
          st(v2[u], at(Vc, o + D));
        }
      }
    };
    int d0 = e;
    load_chunk(d0, ak1, ak2, av1, av2);
    // first chunk: nothing stored yet, only the next chunk's loads stay
    const bool more = d0 + CH <= last;
    if (more) {
      load_chunk(d0 + CH, bk1, bk2, bv1, bv2);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));     // chunk d0 landed, next in flight
      store_chunk(d0, ak1, ak2, av1, av2, true);
      d0 += CH;
    } else {
      __builtin_amdgcn_s_waitcnt(0);
      store_chunk(d0, ak1, ak2, av1, av2, false);
    }
    // later chunks (every chunk before the last is full, so every wave issued
    // STORES stores for it): the previous chunk's stores may stay in flight
    while (more) {
      if (d0 + CH <= last) {
        load_chunk(d0 + CH, ak1, ak2, av1, av2);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(STORES + LOADS));
        store_chunk(d0, bk1, bk2, bv1, bv2, true);
      } else {
        __builtin_amdgcn_s_waitcnt(0);
        store_chunk(d0, bk1, bk2, bv1, bv2, false);
        break;
      }
      d0 += CH;
      if (d0 + CH <= last) {
        load_chunk(d0 + CH, bk1, bk2, bv1, bv2);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(STORES + LOADS));
        store_chunk(d0, ak1, ak2, av1, av2, true);
      } else {
        __builtin_amdgcn_s_waitcnt(0);
        store_chunk(d0, ak1, ak2, av1, av2, false);
        break;
      }
      d0 += CH;
    }
  }

  // the new row at its final slot: n (no eviction), n-1 (an older row left),
  // or nowhere (it was the one evicted).  Lane c < LPM stores key chunks c
  // and c + LPM, a RoPE pair (with two chunks per lane the pair it holds in
  // q, lr == c), rotated when the row moved; lane c < V16 stores value chunk
  // c, loaded at the start.
  const int f = e < 0 ? n : (e < n ? n - 1 : -1);
  if (f >= 0 && tid < V16) {
    const size_t o = (size_t)f * V16;
    // handed over: the row goes to scratch slot 0 (keys, then values), and
    // the move kernel writes it once it has read row n-1
    const gptr<u32x4> dk = defer ? slot : Kw + o;
    const gptr<u32x4> dv = defer ? slot + V16 : Vw + o;
    if (tid < LPM) {
      u32x4 k1, k2;
      if constexpr (CPL == 2) {
        k1 = q[0];
        k2 = q[CPL - 1];
      } else {
        k1 = nk4[tid];
        k2 = nk4[tid + LPM];
      }
      if (e >= 0) {                              // moved: rotate to position f
        float cs[8], sn[8];      // written above by this same wave, or before the token
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          cs[j] = rot_c[tid * 8 + j];
          sn[j] = rot_s[tid * 8 + j];
        }
        rotate_chunk(k1, k2, cs, sn);
      }
      dk[tid] = k1;
      dk[tid + LPM] = k2;
    }
    dv[tid] = v_new;
    if (tid == 0) {
      st_state(0.0f, scores + (row0 + f));
      if constexpr (GUMBEL) st_state(g_new, gumbel + (row0 + f));
      st_state(e < 0 ? la.next_pos : f, positions + (row0 + f));
    }
  }
}

// One layer per launch: workgroup hh owns cache hh.
template <int D, int NT, int U, bool GUMBEL, int R>
__global__ __launch_bounds__(NT) void step_kernel(LayerArgs la, SharedArgs sa) {
  stage_tables<D>(sa);
  step_body<D, NT, U, GUMBEL, false, R, false>(la, sa, blockIdx.x, nullptr);
}

// The same, for a layer of at most as many caches as compute units, where no
// compute unit runs more than one workgroup: the compaction moves two sweeps
// of rows per chunk, twice the bytes in flight, with registers that two
// workgroups on one compute unit could not share.  A long interior move is
// then the end of the launch, done by one compute unit (measured on the
// 8B-shaped per-layer launch with moves in place: 0.981 -> 0.936 ms per
// token).
template <int D, int NT, int U, bool GUMBEL, int R>
__global__ __launch_bounds__(NT) void step_kernel_solo(LayerArgs la, SharedArgs sa) {
  stage_tables<D>(sa);
  step_body<D, NT, U, GUMBEL, false, R, false, 2>(la, sa, blockIdx.x, nullptr);
}

// Several layers and/or tokens per launch: the workgroups of layer l are
// block0(l) .. block0(l+1)-1; layer descriptors live in device memory.  A
// workgroup steps its cache through the layer's tokens one after the other
// (keyformer_update absorbs S tokens as S steps); between tokens every store
// of the workgroup has landed and every wave has arrived, so the next token
// reads the state the previous one left.
template <int D, int NT, int U, bool GUMBEL, int R, bool REUSE>
__global__ __launch_bounds__(NT) void step_layers_kernel(LayerPack pack, int n_layers,
                                                         SharedArgs sa) {
  const LayerArgs *__restrict__ layers = pack.l;    // in the kernel-argument segment
  // layer of this workgroup: the number of layers starting at or before it,
  // counted with one load per lane and a ballot (at most 128 layers)
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  int count = 0;
  for (int base = 0; base < n_layers; base += 64) {
    const int i = base + lane;
    const bool starts = i < n_layers && layers[i].block0 <= b;
    count += __popcll(__ballot(starts));
  }
  const LayerArgs &la = layers[count - 1];
  const int hh = b - la.block0;
  const int n_tokens = la.n_tokens;
  const int bh = (count < n_layers ? layers[count].block0 : (int)gridDim.x) - la.block0;
  stage_tables<D>(sa);
  if (!REUSE && n_tokens == 1) {               // nothing to share between tokens
    step_body<D, NT, U, GUMBEL, false, R, false>(la, sa, hh, nullptr);
    return;
  }
  __syncthreads();                              // every wave reads lds_freq below
  // The per-token values, kTokChunk tokens at a time, in dynamic LDS past the
  // step's own arrays at their largest over this launch's tokens.
  extern __shared__ float lds_dyn[];
  constexpr int TAB = D + 2;
  const int n_last = min(la.n_prev + n_tokens - 1, la.budget);
  float *const tab = lds_dyn + ((n_last + 63) & ~63) + 64;
  LayerArgs lt = la;
  for (int t = 0; t < n_tokens; ++t) {
    if (t % kTokChunk == 0) {                   // nothing is in flight here
      const int cnt = min(kTokChunk, n_tokens - t);
      for (int k = threadIdx.x; k < cnt * (D / 2); k += NT) {
        const int i = k / (D / 2), j = k - i * (D / 2);
        const int tok = t + i;
        const int n_i = min(la.n_prev + tok, la.budget);
        const f32x2 r = rotation_at(n_i - 1 - (la.next_pos + tok), lds_freq[j]);
        tab[i * TAB + j] = r.x;
        tab[i * TAB + D / 2 + j] = r.y;
      }
      if (GUMBEL && (int)threadIdx.x >= NT - cnt) {
        const int i = threadIdx.x - (NT - cnt);
        const int32_t pos = la.pos + t + i;
        tab[i * TAB + D] = gumbel_at(sa.seed, (uint64_t)(int64_t)(la.hh_base + hh),
                                     (uint64_t)(int64_t)pos);
        tab[i * TAB + D + 1] = anneal_tau(sa.tau_init, sa.tau_end, sa.anneal_steps, pos);
      }
      __syncthreads();
    }
    // Re-derive every per-cache address on each token (the asm hides these
    // values from the optimiser): hoisting them out of the loop would hold
    // them in registers for the whole launch.
    lt.k = opaque(la.k);
    lt.v = opaque(la.v);
    lt.scores = opaque(la.scores);
    lt.gumbel = opaque(la.gumbel);
    lt.positions = opaque(la.positions);
    lt.cap = opaque(la.cap);
    const int hh_t = opaque(hh);
    lt.n_prev = min(la.n_prev + t, la.budget);
    lt.next_pos = la.next_pos + t;
    lt.pos = la.pos + t;
    lt.new_k = reinterpret_cast<const char *>(la.new_k) + (size_t)t * bh * D * 2;
    lt.new_v = reinterpret_cast<const char *>(la.new_v) + (size_t)t * bh * D * 2;
    lt.evicted = la.evicted ? la.evicted + (size_t)t * bh : nullptr;
    step_body<D, NT, U, GUMBEL, true, R, REUSE>(lt, sa, hh_t, tab + (t % kTokChunk) * TAB);
    __builtin_amdgcn_s_waitcnt(0);              // this token's stores have landed
    __syncthreads();
  }
}

// Finishes the compactions a single-token launch handed over, one queued
// chunk at a time, following the move plan (kve_move_plan.h): chunk j fills
// its destination rows from the rows one below, keys rotated by -1 position,
// reading every source from the cache except its next chunk's first
// destination, which comes from the parked copy.  So no two chunks touch the
// same row, and each chunk reads everything before it writes.  The last
// chunk then writes the incoming row at n-1.  The grid strides over the
// queued items.  Workgroup 0 also prepares the pool for the next call: it
// zeroes the counter that call will reserve on and advances the phase (the
// move plan's header protocol), so the next launch finds its counter at zero
// without any clearing on the host.
template <int D>
__global__ __launch_bounds__(256) void move_kernel(MovePool pool, RopeTable back1) {
  constexpr int NT = 256;
  constexpr int V16 = D / 8;
  constexpr int LPM = D / 16;                   // lanes per row: chunks lm and lm + LPM
  constexpr int RPM = NT / LPM;                 // rows per sweep
  constexpr int SW = kMoveChunk / RPM;          // sweeps per chunk
  static_assert(SW * RPM == kMoveChunk, "move chunk");
  // Everything the first chunk depends on is loaded at once, so that the
  // launch waits for one round trip before its row loads, not three: the
  // phase, both reservation counters (the phase picks one), and the item this
  // workgroup takes first if the queue reaches it (items[blockIdx.x] is inside
  // the pool: the grid is never larger than its capacity).  Ordinary loads:
  // the phase and the counter it picks were last written before this launch
  // began (the counter by the step's atomics, the phase by its workgroup 0),
  // and workgroup 0's updates below change neither of them (the other
  // counter, which it zeroes, is read here but not used).
  const int phase = global(pool.count)[kPoolLaunchPhase];
  const int count_even = global(pool.count)[kPoolCount];
  const int count_odd = global(pool.count)[kPoolCount + 1];
  const MoveItem first_item = pool.items[blockIdx.x];
  const int reserved = pool_counter(phase) == kPoolCount ? count_even : count_odd;
  const int queued = items_queued(reserved, pool.cap);
  if (blockIdx.x == 0 && threadIdx.x == 0) {    // the next call's counter, then its phase
    atomicExch(pool.count + pool_counter(pool_next_phase(phase)), 0);
    atomicExch(pool.count + kPoolPhase, pool_next_phase(phase));
  }
  const int tid = threadIdx.x, lm = tid % LPM, rm = tid / LPM;
  float cs[8], sn[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    cs[i] = back1.c[lm * 8 + i];
    sn[i] = back1.s[lm * 8 + i];
  }
  // Up to a grid's worth of chunks, each gets a workgroup of its own (the
  // launch is one round trip long).  A longer queue is shared by fewer
  // workgroups, each taking many chunks in turn: fewer streams in flight
  // move more bytes per second.
  const int active = queued > (int)gridDim.x ? min((int)gridDim.x, kMoveStreams)
                                             : (int)gridDim.x;
  const int first = (int)blockIdx.x < active ? (int)blockIdx.x : queued;
  // The next item's descriptor is loaded while this chunk moves, so that a
  // workgroup taking chunks in turn waits for one round trip per chunk (its
  // rows), not two.
  MoveItem next_item = first_item;
  for (int item = first; item < queued; item += active) {
    const MoveItem md = next_item;
    if (item + active < queued) next_item = pool.items[item + active];
    if (md.k == nullptr) continue;              // reserved by a step that found no room
    const int j = md.j, e = md.e, n = md.n, last = move_last_dst(n);
    const int chunks = move_chunks(e, n);
    const int d0 = chunk_first_dst(e, j);
    const gptr<u32x4> K = global(reinterpret_cast<u32x4 *>(md.k));
    const gptr<u32x4> V = global(reinterpret_cast<u32x4 *>(md.v));
    const gptr<const u32x4> P = global(reinterpret_cast<const u32x4 *>(pool.rows)) +
                                (size_t)md.base * (2 * V16);     // the cache's parked rows
    u32x4 k1[SW], k2[SW], v1[SW], v2[SW];
#pragma unroll
    for (int w = 0; w < SW; ++w) {
      const int dst = d0 + rm + w * RPM;
      if (dst <= last) {
        const int src = chunk_source_row(e, j, chunks, dst);
        if (src < 0) {                          // the next chunk's first row: parked
          const gptr<const u32x4> r = P + (size_t)(j + 1) * 2 * V16;
          k1[w] = r[lm];
          k2[w] = r[lm + LPM];
          v1[w] = r[V16 + lm];
          v2[w] = r[V16 + lm + LPM];
        } else {
          const size_t o = (size_t)src * V16;
          k1[w] = __builtin_nontemporal_load(K + o + lm);
          k2[w] = __builtin_nontemporal_load(K + o + lm + LPM);
          v1[w] = __builtin_nontemporal_load(V + o + lm);
          v2[w] = __builtin_nontemporal_load(V + o + lm + LPM);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();                            // every row of the chunk has been read
#pragma unroll
    for (int w = 0; w < SW; ++w) {
      const int dst = d0 + rm + w * RPM;
      if (dst <= last) {
        rotate_chunk(k1[w], k2[w], cs, sn);
        const size_t o = (size_t)dst * V16;
        __builtin_nontemporal_store(k1[w], K + o + lm);
        __builtin_nontemporal_store(k2[w], K + o + lm + LPM);
        __builtin_nontemporal_store(v1[w], V + o + lm);
        __builtin_nontemporal_store(v2[w], V + o + lm + LPM);
      }
    }
    if (j == chunks - 1 && tid < 2 * V16) {     // the incoming row (parked row 0) at n-1
      const u32x4 x = P[tid];
      const size_t o = (size_t)(n - 1) * V16;
      if (tid < V16)
        K[o + tid] = x;
      else
        V[o + tid - V16] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

// Launch shapes (tuning builds may override these with -D).
#ifndef KVE_THREADS
#define KVE_THREADS 512
#endif
#ifndef KVE_UNROLL
#define KVE_UNROLL 8
#endif
#ifndef KVE_MOVE_WGS
#define KVE_MOVE_WGS (4 * kComputeUnits)
#endif
constexpr int kThreads = KVE_THREADS;
constexpr int kWideThreads = 2 * KVE_THREADS;
constexpr int kUnroll = KVE_UNROLL;
// MI355X: 256 compute units, each holding two of these workgroups at once.  A
// launch is a latency chain per cache when no compute unit holds more than
// one of its workgroups.
constexpr int kComputeUnits = 256;

static size_t lds_bytes_for(int n_prev) {
  const size_t np = (size_t)((n_prev + 63) & ~63) + 64;
  return np * sizeof(float);
}

template <typename K>
static hipError_t allow_lds(K kern, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Register slots per thread for the scores of a cache of n rows: the
// smallest of three sizes that covers ceil(n / NT).
template <int NT>
struct Slots {
  static constexpr int r0 = 2, r1 = 8, r2 = (kMaxRows + NT - 1) / NT;
  static_assert(r1 <= r2, "row slots");
};

template <int NT, int D, bool GUMBEL, int R>
static hipError_t launch_d_r(const LayerArgs &la, const SharedArgs &sa, int bh,
                             hipStream_t stream) {
  auto go = [&](auto kern) {
    const size_t lds = lds_bytes_for(la.n_prev);
    hipError_t err = allow_lds(kern, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(bh), dim3(NT), lds, stream, la, sa);
    return hipGetLastError();
  };
  return bh <= kComputeUnits ? go(step_kernel_solo<D, NT, kUnroll, GUMBEL, R>)
                             : go(step_kernel<D, NT, kUnroll, GUMBEL, R>);
}

template <int NT, int D, bool GUMBEL>
static hipError_t launch_d(const LayerArgs &la, const SharedArgs &sa, int bh,
                           hipStream_t stream) {
  using S = Slots<NT>;
  const int r = (la.n_prev + NT - 1) / NT;
  if (r <= S::r0) return launch_d_r<NT, D, GUMBEL, S::r0>(la, sa, bh, stream);
  if (r <= S::r1) return launch_d_r<NT, D, GUMBEL, S::r1>(la, sa, bh, stream);
  return launch_d_r<NT, D, GUMBEL, S::r2>(la, sa, bh, stream);
}

template <int NT, int D, bool GUMBEL, int R, bool REUSE>
static hipError_t launch_layers_d_r(const LayerPack &layers, int n_layers, int total_blocks,
                                    int max_n_prev, const SharedArgs &sa, hipStream_t stream) {
  auto kern = step_layers_kernel<D, NT, kUnroll, GUMBEL, R, REUSE>;
  const size_t lds = lds_bytes_for(max_n_prev) + (size_t)kTokChunk * (D + 2) * sizeof(float);
  hipError_t err = allow_lds(kern, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(total_blocks), dim3(NT), lds, stream, layers, n_layers, sa);
  return hipGetLastError();
}

template <int NT, int D, bool GUMBEL, bool REUSE>
static hipError_t launch_layers_d(const LayerPack &layers, int n_layers, int total_blocks,
                                  int max_n_prev, const SharedArgs &sa, hipStream_t stream) {
  using S = Slots<NT>;
  const int r = (max_n_prev + NT - 1) / NT;
  if (r <= S::r0)
    return launch_layers_d_r<NT, D, GUMBEL, S::r0, REUSE>(layers, n_layers, total_blocks,
                                                          max_n_prev, sa, stream);
  if (r <= S::r1)
    return launch_layers_d_r<NT, D, GUMBEL, S::r1, REUSE>(layers, n_layers, total_blocks,
                                                          max_n_prev, sa, stream);
  return launch_layers_d_r<NT, D, GUMBEL, S::r2, REUSE>(layers, n_layers, total_blocks,
                                                        max_n_prev, sa, stream);
}

template <int NT>
static hipError_t launch_step_nt(const LayerArgs &la, const SharedArgs &sa, int bh, int d,
                                 bool gumbel, hipStream_t stream) {
  if (d == 128)
    return gumbel ? launch_d<NT, 128, true>(la, sa, bh, stream)
                  : launch_d<NT, 128, false>(la, sa, bh, stream);
  return gumbel ? launch_d<NT, 64, true>(la, sa, bh, stream)
                : launch_d<NT, 64, false>(la, sa, bh, stream);
}

template <int NT, bool REUSE>
static hipError_t launch_layers_nt(const LayerPack &layers, int n_layers, int total_blocks,
                                   int max_n_prev, const SharedArgs &sa, int d, bool gumbel,
                                   hipStream_t stream) {
  if (d == 128)
    return gumbel ? launch_layers_d<NT, 128, true, REUSE>(layers, n_layers, total_blocks,
                                                          max_n_prev, sa, stream)
                  : launch_layers_d<NT, 128, false, REUSE>(layers, n_layers, total_blocks,
                                                           max_n_prev, sa, stream);
  return gumbel ? launch_layers_d<NT, 64, true, REUSE>(layers, n_layers, total_blocks, max_n_prev,
                                                       sa, stream)
                : launch_layers_d<NT, 64, false, REUSE>(layers, n_layers, total_blocks,
                                                        max_n_prev, sa, stream);
}

// Whether a launch that steps its caches through several tokens should keep
// their keys cached between tokens: the keys of the caches resident at once
// (two workgroups on each of the 256 compute units) must fit in three
// quarters of the 256 MB last-level (Infinity) cache, so that a cache's next
// pass finds them there.  Larger footprints stream them non-temporally, as a
// single token does.
bool reuse_keys(int total_blocks, int max_n_prev, int n_tokens, int d) {
  constexpr int64_t kResidentBlocks = 2 * kComputeUnits;
  constexpr int64_t kReuseBytes = (int64_t)192 << 20;
  if (n_tokens < 2) return false;
  const int64_t resident = total_blocks < kResidentBlocks ? total_blocks : kResidentBlocks;
  return resident * (int64_t)max_n_prev * d * 2 <= kReuseBytes;
}

hipError_t launch_step(const LayerArgs &la, const SharedArgs &sa_in, int bh, int d, bool gumbel,
                       hipStream_t stream) {
  SharedArgs sa = sa_in;
  sa.early = bh <= kComputeUnits;
  return launch_step_nt<kThreads>(la, sa, bh, d, gumbel, stream);
}

hipError_t launch_step_layers(const LayerPack &layers, int n_layers, int total_blocks,
                              int max_n_prev, int n_tokens, const SharedArgs &sa_in, int d,
                              bool gumbel, hipStream_t stream) {
  SharedArgs sa = sa_in;
  sa.early = total_blocks <= kComputeUnits;
  const bool reuse = reuse_keys(total_blocks, max_n_prev, n_tokens, d);
  // A token loop that fills the GPU (at least as many workgroups as it holds
  // of 512 threads) walks its caches' tokens faster with 1024-thread
  // workgroups: one per compute unit, twice the key bytes in flight per
  // cache.  Fewer, latency-bound workgroups, and single tokens, keep 512
  // threads, whose reductions are shorter.
  if (n_tokens > 1 && total_blocks >= 2 * kComputeUnits)
    return reuse ? launch_layers_nt<kWideThreads, true>(layers, n_layers, total_blocks,
                                                        max_n_prev, sa, d, gumbel, stream)
                 : launch_layers_nt<kWideThreads, false>(layers, n_layers, total_blocks,
                                                         max_n_prev, sa, d, gumbel, stream);
  return reuse ? launch_layers_nt<kThreads, true>(layers, n_layers, total_blocks, max_n_prev, sa,
                                                  d, gumbel, stream)
               : launch_layers_nt<kThreads, false>(layers, n_layers, total_blocks, max_n_prev, sa,
                                                   d, gumbel, stream);
}

// One wave writes zeros over the header's words (a fill kernel rather than a
// memset: it may be captured into a graph and replayed).
__global__ __launch_bounds__(64) void pool_clear_kernel(int32_t *header) {
  const int i = threadIdx.x;
  if (i < (int)(kPoolHeaderBytes / sizeof(int32_t))) global(header)[i] = 0;
}

hipError_t launch_pool_clear(const MovePool &pool, hipStream_t stream) {
  hipLaunchKernelGGL(pool_clear_kernel, dim3(1), dim3(64), 0, stream, pool.count);
  return hipGetLastError();
}

hipError_t launch_moves(const MovePool &pool, const RopeTable &back1, int d,
                        hipStream_t stream) {
  // enough workgroups to spread the longest moves of a launch over the GPU;
  // each strides over the queued chunks
  const dim3 grid((unsigned)std::min<int64_t>(pool.cap, KVE_MOVE_WGS));
  if (d == 128)
    hipLaunchKernelGGL(move_kernel<128>, grid, dim3(256), 0, stream, pool, back1);
  else
    hipLaunchKernelGGL(move_kernel<64>, grid, dim3(256), 0, stream, pool, back1);
  return hipGetLastError();
}

}  // namespace kve
