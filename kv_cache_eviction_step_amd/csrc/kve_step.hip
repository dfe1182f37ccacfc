// kve_step.hip -- gfx950 kernel of the per-token KV-cache eviction step.
//
// One workgroup owns one cache (one (batch, kv-head) of the layer) for the
// whole step, so no cross-workgroup synchronisation or scratch memory is
// needed.  Phases inside the workgroup:
//   A  score pass: coalesced 128-bit loads of the stored keys, fp16 dot2
//      products against the incoming key, 16-lane DPP reduction per row,
//      logits to LDS (a matrix-vector product: bandwidth bound, no MFMA);
//   B  softmax: block max, exponentials and block sum over LDS;
//   C  new scores (fp32 add of the normalised mass) and, when over budget,
//      the eviction key  fma(tau, gumbel, score)  with a block argmin that
//      breaks ties towards the lowest index;
//   D  write-back: scores / gumbel / positions of the rows after the evicted
//      one move down one slot; keys and values of those rows move in
//      ascending chunks (load all, barrier, store), keys re-rotated by -1
//      position in fp32; the new row lands at its final slot.
//
// Method (VeloxQuant-MLX pages): "veloxquant_mlx.quantizers.keyformer
// module" -- keyformer_update steps 1-3, KeyformerState, FIXED GAP #1/#2,
// FUSED METAL KERNEL; "PyramidKV -- Layer-Adaptive Budget Attention-Mass
// Eviction" -- How it works.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kve_step.h"

namespace kve {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte chunk

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
__device__ __noinline__ float gumbel_at(uint64_t seed, uint64_t stream, uint64_t pos) {
  uint64_t h = splitmix64_out(splitmix64_out(splitmix64_out(seed) ^ stream) ^ pos);
  double u = ((double)(h >> 11) + 0.5) * 0x1p-53;
  return (float)(-log(-log(u)));
}

// Annealed temperature (keyformer FIXED GAP #1), fp64, rounded once.
__device__ __noinline__ float anneal_tau(double tau_init, double tau_end, int32_t steps,
                                         int32_t pos) {
#pragma clang fp contract(off)
  if (steps <= 0 || tau_init == tau_end) return (float)tau_init;
  int32_t t = pos < steps ? pos : steps;
  double delta = (tau_end - tau_init) / (double)steps;
  double prod = (double)t * delta;
  return (float)(tau_init + prod);
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

// 8 fp16 products accumulated in fp32 (v_dot2_f32_f16).
__device__ __forceinline__ float dot8(const u32x4 a, const u32x4 b) {
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2(as_h2(a[w]), as_h2(b[w]), acc, false);
  return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LANES lanes (8 or 16); every lane gets the sum.
// quad_perm [1,0,3,2] and [2,3,0,1], then half-row mirror, then row mirror.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  if constexpr (LANES == 16) x += dpp<0x140>(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// (value, index) pairs: smaller value wins, equal values go to the lower index.
__device__ __forceinline__ void argmin_merge(float &v, int &i, float v2, int i2) {
  if (v2 < v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ __forceinline__ void wave_argmin(float &v, int &i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v2 = __shfl_xor(v, o);
    int i2 = __shfl_xor(i, o);
    argmin_merge(v, i, v2, i2);
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

template <int D, int NT, int U, bool GUMBEL>
__global__ __launch_bounds__(NT) void step_kernel(StepArgs a) {
  constexpr int V16 = D / 8;        // 16-byte chunks per row
  constexpr int LPR = D / 8;        // score pass: lanes per row (one chunk each)
  constexpr int RPS = NT / LPR;     // score pass: rows per sweep
  constexpr int HALF = D / 2;
  constexpr int LPM = D / 16;       // move pass: lanes per row (one chunk of each half)
  constexpr int RPM = NT / LPM;     // move pass: rows per sweep
  constexpr int UM = 2;             // move pass: sweeps per chunk
  constexpr int NWAVE = NT / 64;
  static_assert(NT % 64 == 0 && RPS * LPR == NT && RPM * LPM == NT, "launch shape");

  extern __shared__ float lds[];    // [n] logits -> weights -> new scores ; [n] gumbel
  __shared__ float red_v[NWAVE];
  __shared__ int red_i[NWAVE];
  __shared__ float bc_v;
  __shared__ int bc_e;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = blockIdx.x;
  const int n = a.n_prev;
  const size_t row0 = (size_t)hh * (size_t)a.cap;     // first row of this cache

  const u32x4 *__restrict__ K4 = reinterpret_cast<const u32x4 *>(a.k) + row0 * V16;
  float *__restrict__ lds_s = lds;
  float *__restrict__ lds_g = lds + n;

  // ---- A: logits of every stored row against the incoming key -------------
  const int lr = tid % LPR;
  const int rr = tid / LPR;
  const u32x4 q = reinterpret_cast<const u32x4 *>(a.new_k)[(size_t)hh * V16 + lr];
  float mx = -INFINITY;
  for (int base = 0; base < n; base += RPS * U) {
    u32x4 kr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = base + rr + u * RPS;
      kr[u] = r < n ? K4[(size_t)r * V16 + lr] : u32x4(0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = base + rr + u * RPS;
      const float x = group_sum<LPR>(dot8(kr[u], q)) * a.scale;
      if (r < n) {
        if (lr == 0) lds_s[r] = x;
        mx = fmaxf(mx, x);
      }
    }
  }

  // ---- B: softmax normaliser ------------------------------------------------
  mx = wave_max(mx);
  if (lane == 0) red_v[wave] = mx;
  __syncthreads();
  if (wave == 0) {
    float m = lane < NWAVE ? red_v[lane] : -INFINITY;
    m = wave_max(m);
    if (lane == 0) bc_v = m;
  }
  __syncthreads();
  mx = bc_v;
  float sum = 0.f;
  for (int i = tid; i < n; i += NT) {
    const float w = expf(lds_s[i] - mx);
    lds_s[i] = w;
    sum += w;
  }
  sum = wave_sum(sum);
  __syncthreads();                              // every wave has read bc_v / red_v
  if (lane == 0) red_v[wave] = sum;
  __syncthreads();
  if (wave == 0) {
    float z = lane < NWAVE ? red_v[lane] : 0.f;
    z = wave_sum(z);
    if (lane == 0) bc_v = z;
  }
  __syncthreads();
  const float rz = 1.0f / bc_v;

  // ---- C: new scores and the eviction choice --------------------------------
  const bool over = n + 1 > a.budget;
  const float tau = (GUMBEL && over) ? anneal_tau(a.tau_init, a.tau_end, a.anneal_steps, a.pos)
                                     : 0.f;
  const float g_new = GUMBEL ? gumbel_at(a.seed, (uint64_t)(int64_t)(a.hh_base + hh),
                                         (uint64_t)(int64_t)a.pos)
                             : 0.f;
  float bv = INFINITY;
  int bi = 0x7fffffff;
  for (int i = tid; i < n; i += NT) {
    const float s = a.scores[row0 + i] + lds_s[i] * rz;
    lds_s[i] = s;
    if (over && i >= a.n_sink) {
      float key = s;
      if constexpr (GUMBEL) {
        const float g = a.gumbel[row0 + i];
        lds_g[i] = g;
        key = fmaf(tau, g, s);
      }
      if (key < bv) {                      // rows visited in increasing order
        bv = key;
        bi = i;
      }
    }
  }
  if (over && tid == 0) {                  // the new row: score 0
    const float key = GUMBEL ? fmaf(tau, g_new, 0.0f) : 0.0f;
    argmin_merge(bv, bi, key, n);
  }
  wave_argmin(bv, bi);
  __syncthreads();                              // bc_v consumed by every wave
  if (lane == 0) {
    red_v[wave] = bv;
    red_i[wave] = bi;
  }
  __syncthreads();
  if (wave == 0) {
    float v = lane < NWAVE ? red_v[lane] : INFINITY;
    int i = lane < NWAVE ? red_i[lane] : 0x7fffffff;
    wave_argmin(v, i);
    if (lane == 0) bc_e = over ? i : -1;
  }
  __syncthreads();
  const int e = bc_e;
  if (tid == 0 && a.evicted) a.evicted[hh] = e;

  // ---- D: write-back ----------------------------------------------------------
  for (int i = tid; i < n; i += NT) {
    if (e < 0 || i < e) {
      a.scores[row0 + i] = lds_s[i];
    } else if (i > e) {
      a.scores[row0 + i - 1] = lds_s[i];
      if constexpr (GUMBEL) a.gumbel[row0 + i - 1] = lds_g[i];
      a.positions[row0 + i - 1] = i - 1;
    }
  }

  u32x4 *__restrict__ Kw = reinterpret_cast<u32x4 *>(a.k) + row0 * V16;
  u32x4 *__restrict__ Vw = reinterpret_cast<u32x4 *>(a.v) + row0 * V16;
  const int lm = tid % LPM;                     // chunk lm of the first half, lm of the second
  const int rm = tid / LPM;

  // old rows e+1 .. n-1 move to e .. n-2, keys rotated by one position back
  if (e >= 0 && e < n - 1) {
    float cs[8], sn[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cs[j] = a.rope.cos_m1[lm * 8 + j];
      sn[j] = a.rope.sin_m1[lm * 8 + j];
    }
    for (int d0 = e; d0 < n - 1; d0 += RPM * UM) {
      u32x4 k1[UM], k2[UM], v1[UM], v2[UM];
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        const int dst = d0 + rm + u * RPM;
        if (dst < n - 1) {
          const size_t src = (size_t)(dst + 1) * V16;
          k1[u] = Kw[src + lm];
          k2[u] = Kw[src + lm + V16 / 2];
          v1[u] = Vw[src + lm];
          v2[u] = Vw[src + lm + V16 / 2];
        }
      }
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        const int dst = d0 + rm + u * RPM;
        if (dst < n - 1) rotate_chunk(k1[u], k2[u], cs, sn);
      }
      __builtin_amdgcn_s_waitcnt(0);            // every load of this chunk has landed
      __syncthreads();
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        const int dst = d0 + rm + u * RPM;
        if (dst < n - 1) {
          const size_t o = (size_t)dst * V16;
          Kw[o + lm] = k1[u];
          Kw[o + lm + V16 / 2] = k2[u];
          Vw[o + lm] = v1[u];
          Vw[o + lm + V16 / 2] = v2[u];
        }
      }
    }
  }

  // the new row at its final slot: n (no eviction), n-1 (an older row left),
  // or nowhere (it was the one evicted)
  const int f = e < 0 ? n : (e < n ? n - 1 : -1);
  if (f >= 0 && tid < LPM) {
    const u32x4 *nk = reinterpret_cast<const u32x4 *>(a.new_k) + (size_t)hh * V16;
    const u32x4 *nv = reinterpret_cast<const u32x4 *>(a.new_v) + (size_t)hh * V16;
    u32x4 k1 = nk[lm], k2 = nk[lm + V16 / 2];
    if (e >= 0) {                                // moved: rotate to position f
      float cs[8], sn[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        cs[j] = a.rope.cos_new[lm * 8 + j];
        sn[j] = a.rope.sin_new[lm * 8 + j];
      }
      rotate_chunk(k1, k2, cs, sn);
    }
    const size_t o = (size_t)f * V16;
    Kw[o + lm] = k1;
    Kw[o + lm + V16 / 2] = k2;
    Vw[o + lm] = nv[lm];
    Vw[o + lm + V16 / 2] = nv[lm + V16 / 2];
    if (tid == 0) {
      a.scores[row0 + f] = 0.0f;
      if constexpr (GUMBEL) a.gumbel[row0 + f] = g_new;
      a.positions[row0 + f] = e < 0 ? a.next_pos : f;
    }
  }
  (void)HALF;
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

template <int D, bool GUMBEL>
static hipError_t launch_d(const StepArgs &a, int bh, hipStream_t stream) {
  constexpr int NT = 512;
  constexpr int U = 8;
  auto kern = step_kernel<D, NT, U, GUMBEL>;
  const size_t lds_bytes = (size_t)2 * (size_t)(a.n_prev > 0 ? a.n_prev : 1) * sizeof(float);
  if (lds_bytes > 64 * 1024) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)lds_bytes);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3(bh), dim3(NT), lds_bytes, stream, a);
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, int bh, int d, bool gumbel, hipStream_t stream) {
  if (d == 128) return gumbel ? launch_d<128, true>(a, bh, stream) : launch_d<128, false>(a, bh, stream);
  return gumbel ? launch_d<64, true>(a, bh, stream) : launch_d<64, false>(a, bh, stream);
}

}  // namespace kve
