// Lane state and segment summaries of the per-token-decay operator, shared by
// its forward kernels and its backward pass (gfx950 only). With a decay rate
// per token the running maximum exponent cannot be index-tracked, so every
// exponent that accumulates rates is fp64 and differences are rounded to fp32
// only right before v_exp_f32; values and sums stay fp32.
#pragma once

#include "wkv_device.h"

namespace wkv {
namespace {

constexpr double kEmptyD = static_cast<double>(kEmpty);  // the fp32 empty max_exp, exactly

// e^(-|x|) of an fp64 exponent difference.
__device__ __forceinline__ float exp_neg_abs(double x) {
  return fast_exp2(__builtin_fabsf(static_cast<float>(x)) * -kLog2e);
}

// Running state of one channel: true sums n e^m and d e^m.
struct LaneD {
  float n, d;
  double m;
};

__device__ __forceinline__ LaneD laned_empty() { return LaneD{0.0f, 0.0f, kEmptyD}; }

// A checkpoint for the backward pass: the lane state in front of a chunk of
// kCkptTokens tokens, 16 bytes, stored at [chunk][b * C + c].
struct LaneCk {
  float n, d;
  double m;
};

// One token. Output: the state as it stands mixed with the token at weight
// e^(u + k); then the state decays by e^(-w) and the token is added at e^k.
// Of each pair of weights, taken against the larger exponent, one is 1.
__device__ __forceinline__ float laned_step(LaneD& s, float k, float v, float w, double ud) {
  const double kd = static_cast<double>(k);
  const double dk = kd - s.m;   // k - m
  const double s1 = dk + ud;    // (u + k) - m
  const float x = exp_neg_abs(s1);
  const bool cur_wins = s1 > 0.0;
  const float fa = cur_wins ? x : 1.0f;
  const float fb = cur_wins ? 1.0f : x;
  const float out = __builtin_fmaf(fa, s.n, fb * v) * fast_rcp(__builtin_fmaf(fa, s.d, fb));
  // the decayed state's exponent against the token's; the new maximum is one
  // v_max_f64 rather than a compare and a 64-bit select
  const double mw = s.m - static_cast<double>(w);
  const double s2 = kd - mw;
  const float y = exp_neg_abs(s2);
  const bool tok_wins = s2 > 0.0;
  const float ga = tok_wins ? y : 1.0f;
  const float gb = tok_wins ? 1.0f : y;
  s.n = __builtin_fmaf(ga, s.n, gb * v);
  s.d = __builtin_fmaf(ga, s.d, gb);
  s.m = __builtin_fmax(kd, mw);
  return out;
}

// A run of tokens from the empty state: (n, d) against the largest exponent
// m at the end of the run, and the run's total rate ws (what a state that
// enters the run decays by while it passes).
struct SegD {
  float n, d;
  double m, ws;
};

__device__ __forceinline__ SegD segd_identity() { return SegD{0.0f, 0.0f, kEmptyD, 0.0}; }

// a then b: a decays by b's total rate, then the two add against the larger
// exponent.
__device__ __forceinline__ SegD segd_combine(const SegD& a, const SegD& b) {
  const double am = a.m - b.ws;
  const double t = am - b.m;
  const float e = exp_neg_abs(t);
  const bool a_wins = t >= 0.0;
  const float fa = a_wins ? 1.0f : e;
  const float fb = a_wins ? e : 1.0f;
  return SegD{__builtin_fmaf(fa, a.n, fb * b.n), __builtin_fmaf(fa, a.d, fb * b.d),
              a_wins ? am : b.m, a.ws + b.ws};
}

// A running state followed by a run.
__device__ __forceinline__ void laned_absorb(LaneD& s, const SegD& b) {
  const double am = s.m - b.ws;
  const double t = am - b.m;
  const float e = exp_neg_abs(t);
  const bool a_wins = t >= 0.0;
  const float fa = a_wins ? 1.0f : e;
  const float fb = a_wins ? e : 1.0f;
  s.n = __builtin_fmaf(fa, s.n, fb * b.n);
  s.d = __builtin_fmaf(fa, s.d, fb * b.d);
  s.m = a_wins ? am : b.m;
}

}  // namespace
}  // namespace wkv
