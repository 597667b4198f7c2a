// Device-side building blocks shared by the WKV kernels (gfx950 only).
//
// The operator is the one defined on the page "Linear attention without
// writing a CUDA kernel", section "The recurrence": per channel, the output
// at position t is a weighted mean of the values, where a past token i < t
// weighs exp(k_i - (t-1-i) w) and the current token weighs exp(u + k_t). The
// same section carries it forward as a state (num, den, max_exp) rescaled
// against a running maximum exponent.
//
// Conventions inside the kernels:
//   * every exponential is one v_exp_f32 of a difference scaled by log2 e;
//   * the running maximum is index-tracked (see Lane below);
//   * of the two weights rescaled against a common maximum one is exactly 1,
//     so each mix costs a single exp2 of minus an absolute difference.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------- element I/O
//
// k, v and out hold V consecutive channels per thread, loaded as 1, 2 or 4
// dwords. NT selects non-temporal (streaming) accesses for data touched once.

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int NW, bool NT>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    w[0] = NT ? __builtin_nontemporal_load(p) : *p;
  } else if constexpr (NW == 2) {
    const u32x2* q = reinterpret_cast<const u32x2*>(p);
    u32x2 t = NT ? __builtin_nontemporal_load(q) : *q;
    w[0] = t.x;
    w[1] = t.y;
  } else {
    static_assert(NW == 4, "1, 2 or 4 dwords");
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    u32x4 t = NT ? __builtin_nontemporal_load(q) : *q;
    w[0] = t.x;
    w[1] = t.y;
    w[2] = t.z;
    w[3] = t.w;
  }
}

template <int NW, bool NT>
__device__ __forceinline__ void store_words(uint32_t* __restrict__ p, const uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    if (NT) __builtin_nontemporal_store(w[0], p); else *p = w[0];
  } else if constexpr (NW == 2) {
    u32x2 t = {w[0], w[1]};
    u32x2* q = reinterpret_cast<u32x2*>(p);
    if (NT) __builtin_nontemporal_store(t, q); else *q = t;
  } else {
    static_assert(NW == 4, "1, 2 or 4 dwords");
    u32x4 t = {w[0], w[1], w[2], w[3]};
    u32x4* q = reinterpret_cast<u32x4*>(p);
    if (NT) __builtin_nontemporal_store(t, q); else *q = t;
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 t = {a, b};
  bf16x2 h = __builtin_convertvector(t, bf16x2);  // v_cvt_pk_bf16_f32: nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// fp32 I/O: V in {1, 2, 4}.
struct IoF32 {
  using elem = float;
  template <int V, bool NT>
  static __device__ __forceinline__ void load(const float* __restrict__ p, float (&x)[V]) {
    uint32_t w[V];
    load_words<V, NT>(reinterpret_cast<const uint32_t*>(p), w);
#pragma unroll
    for (int i = 0; i < V; ++i) x[i] = __uint_as_float(w[i]);
  }
  template <int V, bool NT>
  static __device__ __forceinline__ void store(float* __restrict__ p, const float (&x)[V]) {
    uint32_t w[V];
#pragma unroll
    for (int i = 0; i < V; ++i) w[i] = __float_as_uint(x[i]);
    store_words<V, NT>(reinterpret_cast<uint32_t*>(p), w);
  }
};

// bf16 I/O (values upcast exactly to fp32; outputs rounded to nearest even):
// V = 1 (one 16-bit access) or V in {2, 4, 8} (two channels per dword).
struct IoBf16 {
  using elem = uint16_t;
  template <int V, bool NT>
  static __device__ __forceinline__ void load(const uint16_t* __restrict__ p, float (&x)[V]) {
    if constexpr (V == 1) {
      const uint32_t h = NT ? __builtin_nontemporal_load(p) : *p;
      x[0] = __uint_as_float(h << 16);
      return;
    } else {
    static_assert(V % 2 == 0, "bf16 channels come in pairs");
    uint32_t w[V / 2];
    load_words<V / 2, NT>(reinterpret_cast<const uint32_t*>(p), w);
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    }
  }
  template <int V, bool NT>
  static __device__ __forceinline__ void store(uint16_t* __restrict__ p, const float (&x)[V]) {
    if constexpr (V == 1) {
      const uint16_t h = static_cast<uint16_t>(pack_bf16x2(x[0], 0.0f) & 0xffffu);
      if (NT) __builtin_nontemporal_store(h, p); else *p = h;
    } else {
      static_assert(V % 2 == 0, "bf16 channels come in pairs");
      uint32_t w[V / 2];
#pragma unroll
      for (int i = 0; i < V / 2; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
      store_words<V / 2, NT>(reinterpret_cast<uint32_t*>(p), w);
    }
  }
};

// ------------------------------------------------------------ the recurrence
//
// Exponents stay in natural units. Every exponential is taken of a small
// difference that is formed first at full precision (key minus the key that
// set the maximum, plus an exact integer age times w) and only then scaled by
// log2 e for v_exp_f32; scaling a key by log2 e on its own would round at the
// key's magnitude and shift every weight by up to ulp(|k|).

// Running state of one channel. The true sums are n e^m and d e^m, with the
// running maximum exponent m = base - age * w kept index-tracked: base is the
// key of the token that set it (or the max_exp of the state loaded), age the
// whole number of steps it has decayed since. m is formed with one rounding
// whenever it is needed, instead of subtracting w once per token (that rounds
// the same way every step and drifts when w is far below the ulp of m).
struct Lane {
  float n;
  float d;
  float base;
  float age;
};

constexpr float kEmpty = -1.0e38f;  // max_exp of the empty state (finite on purpose)

__device__ __forceinline__ Lane lane_empty() { return Lane{0.0f, 0.0f, kEmpty, 0.0f}; }

__device__ __forceinline__ Lane lane_from_state(float n, float d, float m) {
  return Lane{n, d, m, 0.0f};
}

__device__ __forceinline__ float lane_max_exp(const Lane& s, float w) {
  return __builtin_fmaf(-s.age, w, s.base);
}

// One token. Output: the state as it stands mixed with the current token at
// weight e^(u + k); then the state is decayed by one step and the token is
// added at weight e^k. Of each pair of weights, taken against the larger
// exponent, one is exactly 1.
__device__ __forceinline__ float lane_step(Lane& s, float k, float v, float w, float u) {
  const float dk = k - s.base;
  // output: (u + k) - m
  const float s1 = __builtin_fmaf(s.age, w, dk + u);
  const float x = fast_exp2(__builtin_fabsf(s1) * -kLog2e);
  const bool cur_wins = s1 > 0.0f;
  const float fa = cur_wins ? x : 1.0f;  // factor on the state
  const float fb = cur_wins ? 1.0f : x;  // factor on the current token
  const float num = __builtin_fmaf(fa, s.n, fb * v);
  const float den = __builtin_fmaf(fa, s.d, fb);
  const float out = num * fast_rcp(den);
  // advance: k - (m - w)
  const float age1 = s.age + 1.0f;
  const float s2 = __builtin_fmaf(age1, w, dk);
  const float y = fast_exp2(__builtin_fabsf(s2) * -kLog2e);
  const bool tok_wins = s2 > 0.0f;
  const float ga = tok_wins ? y : 1.0f;
  const float gb = tok_wins ? 1.0f : y;
  s.n = __builtin_fmaf(ga, s.n, gb * v);
  s.d = __builtin_fmaf(ga, s.d, gb);
  s.base = tok_wins ? k : s.base;
  s.age = tok_wins ? 0.0f : age1;
  return out;
}

// The state advance alone (the second half of lane_step): decay by one step,
// add the token at weight e^k.
__device__ __forceinline__ void lane_advance(Lane& s, float k, float v, float w) {
  const float age1 = s.age + 1.0f;
  const float s2 = __builtin_fmaf(age1, w, k - s.base);  // k - (m - w)
  const float y = fast_exp2(__builtin_fabsf(s2) * -kLog2e);
  const bool tok_wins = s2 > 0.0f;
  const float ga = tok_wins ? y : 1.0f;
  const float gb = tok_wins ? 1.0f : y;
  s.n = __builtin_fmaf(ga, s.n, gb * v);
  s.d = __builtin_fmaf(ga, s.d, gb);
  s.base = tok_wins ? k : s.base;
  s.age = tok_wins ? 0.0f : age1;
}

// The same step with one exponential instead of two. Both the update and the
// output are taken against the state's maximum after the step,
// m' = max(m - w, k): the decayed state then weighs F = e^(m - w - m') and the
// token G = e^(k - m'), one of them exactly 1 and the other one exp2 of minus
// an absolute difference. The output's weights, e^m for the state and
// e^(u + k) for the token, are the same two scaled by e^w and e^u, so
//   out = (F n + G c v) / (F d + G c),   c = e^(u - w) per channel.
// Valid while c and 1/c are far inside the fp32 range (|u - w| <= kFastGap);
// otherwise the kernels use lane_step.
constexpr float kFastGap = 32.0f;

__device__ __forceinline__ bool fast_step_ok(float w, float u) {
  return __builtin_fabsf(u - w) <= kFastGap;  // false for NaN too
}

__device__ __forceinline__ float bonus_ratio(float w, float u) { return expf(u - w); }

__device__ __forceinline__ float lane_step_fast(Lane& s, float k, float v, float w, float c) {
  const float age1 = s.age + 1.0f;
  const float g = __builtin_fmaf(age1, w, k - s.base);  // k - (m - w)
  const float x = fast_exp2(__builtin_fabsf(g) * -kLog2e);
  const bool tok_wins = g > 0.0f;
  const float F = tok_wins ? x : 1.0f;
  const float G = tok_wins ? 1.0f : x;
  // every multiply-add is spelled out, so that the rounding does not depend
  // on how the compiler splits the surrounding code into blocks
  const float fn = F * s.n;
  const float gc = G * c;
  const float out = __builtin_fmaf(gc, v, fn) * fast_rcp(__builtin_fmaf(F, s.d, gc));
  s.n = __builtin_fmaf(G, v, fn);
  s.d = __builtin_fmaf(F, s.d, G);
  s.base = tok_wins ? k : s.base;
  s.age = tok_wins ? 0.0f : age1;
  return out;
}

// c = e^(u - w) of each of V channels, for lane_step_fast.
template <int V>
__device__ __forceinline__ void bonus_ratios(const float (&wd)[V], const float (&ub)[V],
                                             float (&cb)[V]) {
#pragma unroll
  for (int j = 0; j < V; ++j) cb[j] = bonus_ratio(wd[j], ub[j]);
}

// True when every channel of every active lane of the wave may take
// lane_step_fast: the same answer in all lanes, so a branch on it does not
// diverge.
template <int V>
__device__ __forceinline__ bool wave_fast_ok(const float (&wd)[V], const float (&ub)[V]) {
  bool ok = true;
#pragma unroll
  for (int j = 0; j < V; ++j) ok = ok && fast_step_ok(wd[j], ub[j]);
  return __all(ok) != 0;
}

template <bool FAST>
__device__ __forceinline__ float step_sel(Lane& s, float k, float v, float w, float u, float c) {
  if constexpr (FAST) {
    return lane_step_fast(s, k, v, w, c);
  } else {
    return lane_step(s, k, v, w, u);
  }
}

// The receptance gate sigmoid(r) = 1 / (1 + e^-r) on an output; e^-r
// overflows to +inf for r < -88, giving exactly 0, and underflows to 0 for
// r > 104, giving exactly 1.
__device__ __forceinline__ float gate(float r) {
  return fast_rcp(1.0f + fast_exp2(r * -kLog2e));
}

// ------------------------------------------------- segment summaries (chunks)

// The state produced by a run of `len` tokens from the empty state, with its
// maximum exponent m (natural units) taken at the end of the run.
struct Seg {
  float n, d, m, len;
};

__device__ __forceinline__ Seg seg_identity() { return Seg{0.0f, 0.0f, kEmpty, 0.0f}; }

// a then b: a is decayed by b.len steps while b passes, then the two add,
// relative to the larger exponent. When a's decayed maximum a.m - b.len w wins
// it is stored rounded to fp32 (by up to ulp(|m|)/2, 5e-4 at |m| = 1e4); the
// sums are scaled by e^delta, delta the rounding (formed exactly: the product
// inside the fma is exact and a.m minus its rounded decay is exact for nearby
// values), so they stay exact relative to the stored maximum.
__device__ __forceinline__ Seg seg_combine(const Seg& a, const Seg& b, float w) {
  const float t = __builtin_fmaf(-b.len, w, a.m - b.m);  // (a.m - b.len w) - b.m
  const float e = fast_exp2(__builtin_fabsf(t) * -kLog2e);
  const bool a_wins = t >= 0.0f;
  const float ma = __builtin_fmaf(-b.len, w, a.m);
  const float delta = __builtin_fmaf(-b.len, w, a.m - ma);  // (a.m - b.len w) - ma
  const float corr = a_wins ? fast_exp2(delta * kLog2e) : 1.0f;
  const float fa = a_wins ? corr : e;
  const float fb = a_wins ? e * corr : 1.0f;
  Seg r;
  r.n = __builtin_fmaf(fa, a.n, fb * b.n);
  r.d = __builtin_fmaf(fa, a.d, fb * b.d);
  r.m = a_wins ? ma : b.m;
  r.len = a.len + b.len;
  return r;
}

// Running lane state followed by a segment. If the lane's maximum still wins
// it stays index-tracked (its age grows by the segment length, exactly);
// otherwise the segment's maximum becomes the new base.
__device__ __forceinline__ void lane_absorb(Lane& s, const Seg& b, float w) {
  const float age2 = s.age + b.len;
  const float t = __builtin_fmaf(-age2, w, s.base - b.m);  // (base - age2 w) - b.m
  const float e = fast_exp2(__builtin_fabsf(t) * -kLog2e);
  const bool a_wins = t >= 0.0f;
  const float fa = a_wins ? 1.0f : e;
  const float fb = a_wins ? e : 1.0f;
  s.n = __builtin_fmaf(fa, s.n, fb * b.n);
  s.d = __builtin_fmaf(fa, s.d, fb * b.d);
  s.base = a_wins ? s.base : b.m;
  s.age = a_wins ? age2 : 0.0f;
}

}  // namespace wkv
