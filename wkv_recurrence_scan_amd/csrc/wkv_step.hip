// Batched decode step: one token for every (b, c) lane, state updated in
// place. This is the constant-cost step of the page "Linear attention without
// writing a CUDA kernel" (section "The recurrence"): the output mixes the
// state as it stands with the current token at the bonus weight exp(u + k);
// then the state is decayed by exp(-w) and the token added at weight exp(k),
// both mixes taken against the larger of their two exponents.
//
// The state crosses the interface with a plain max_exp, so the decay has to be
// applied to it once per call; the exponent stays in natural units here (only
// the argument of each exp2 is scaled by log2 e) so that a call adds no
// conversion rounding to the state it hands back.
#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

constexpr int kStepThreads = 256;

template <typename IoT, int V, bool G>
__global__ __launch_bounds__(kStepThreads) void wkv_step_kernel(
    int64_t B, int64_t C, const float* __restrict__ w, const float* __restrict__ u,
    const typename IoT::elem* __restrict__ k, const typename IoT::elem* __restrict__ v,
    const typename IoT::elem* __restrict__ rg, float* __restrict__ state,
    typename IoT::elem* __restrict__ out) {
  const int64_t groups_per_row = C / V;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kStepThreads + threadIdx.x;
  if (gid >= B * groups_per_row) return;
  const int64_t b = gid / groups_per_row;
  const int64_t c0 = (gid - b * groups_per_row) * V;
  const int64_t lane0 = b * C + c0;
  const int64_t plane = B * C;

  float ww[V], uu[V], kk[V], vv[V], rr[V], n[V], d[V], m[V], o[V];
  IoF32::load<V, false>(w + c0, ww);
  IoF32::load<V, false>(u + c0, uu);
  IoT::template load<V, true>(k + lane0, kk);
  IoT::template load<V, true>(v + lane0, vv);
  if constexpr (G) IoT::template load<V, true>(rg + lane0, rr);
  IoF32::load<V, false>(state + lane0, n);
  IoF32::load<V, false>(state + plane + lane0, d);
  IoF32::load<V, false>(state + 2 * plane + lane0, m);
#pragma unroll
  for (int j = 0; j < V; ++j) {
    // output: state against the current token with the bonus
    const float t1 = (uu[j] + kk[j]) - m[j];
    const float x = fast_exp2(-__builtin_fabsf(t1) * kLog2e);
    const bool cur_wins = t1 > 0.0f;
    const float fa = cur_wins ? x : 1.0f;
    const float fb = cur_wins ? 1.0f : x;
    o[j] = __builtin_fmaf(fa, n[j], fb * vv[j]) * fast_rcp(__builtin_fmaf(fa, d[j], fb));
    if constexpr (G) o[j] *= gate(rr[j]);
    // advance: decayed state against the current token without the bonus
    const float md = m[j] - ww[j];
    const float t2 = kk[j] - md;
    const float y = fast_exp2(-__builtin_fabsf(t2) * kLog2e);
    const bool tok_wins = t2 > 0.0f;
    const float ga = tok_wins ? y : 1.0f;
    const float gb = tok_wins ? 1.0f : y;
    n[j] = __builtin_fmaf(ga, n[j], gb * vv[j]);
    d[j] = __builtin_fmaf(ga, d[j], gb);
    m[j] = tok_wins ? kk[j] : md;
  }
  IoT::template store<V, true>(out + lane0, o);
  IoF32::store<V, false>(state + lane0, n);
  IoF32::store<V, false>(state + plane + lane0, d);
  IoF32::store<V, false>(state + 2 * plane + lane0, m);
}

template <typename IoT, int V>
hipError_t launch_step_t(const StepArgs& a, hipStream_t st) {
  const int64_t threads = a.B * (a.C / V);
  const int64_t blocks = (threads + kStepThreads - 1) / kStepThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const auto* k = static_cast<const typename IoT::elem*>(a.k);
  const auto* v = static_cast<const typename IoT::elem*>(a.v);
  const auto* r = static_cast<const typename IoT::elem*>(a.r);
  auto* out = static_cast<typename IoT::elem*>(a.out);
  if (r != nullptr) {
    hipLaunchKernelGGL((wkv_step_kernel<IoT, V, true>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kStepThreads), 0, st, a.B, a.C, a.w, a.u, k, v, r, a.state, out);
  } else {
    hipLaunchKernelGGL((wkv_step_kernel<IoT, V, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kStepThreads), 0, st, a.B, a.C, a.w, a.u, k, v, r, a.state, out);
  }
  return hipGetLastError();
}

// T == 0 forward: copy the state through (or write the empty state).
__global__ __launch_bounds__(256) void wkv_state_copy_kernel(int64_t n, const float* __restrict__ src,
                                                             float* __restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= 3 * n) return;
  if (src != nullptr) {
    dst[i] = src[i];
  } else {
    dst[i] = i < 2 * n ? 0.0f : -1.0e38f;
  }
}

bool aligned(const void* p, int bytes) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

}  // namespace

// fp32: one channel per thread. A step is one short pass over a few MB, so
// what counts is spreading it over the chip: at B=256 C=768 four channels per
// thread make 192 blocks of 256 for 256 CUs, and one channel per thread was
// faster at every block size measured (in a HIP graph of 256 steps, 2.44-2.53
// against 2.64-2.79 us per step, of which an empty launch takes 1.59 us).
// bf16 keeps the widest width the pointers allow (2-byte accesses otherwise).
int step_vec_width(int io, int64_t C, const StepArgs& a) {
  if (io == kF32) return 1;
  const int elem = 2;
  for (int V : {4, 2, 1}) {
    if (C % V) continue;
    if (!aligned(a.k, V * elem) || !aligned(a.v, V * elem) || !aligned(a.out, V * elem)) continue;
    if (!aligned(a.r, V * elem)) continue;
    if (!aligned(a.w, V * 4) || !aligned(a.u, V * 4) || !aligned(a.state, V * 4)) continue;
    return V;
  }
  return 1;
}

hipError_t launch_step(const StepArgs& a, int io, int vec, hipStream_t s) {
  if (io == kF32) return launch_step_t<IoF32, 1>(a, s);
  if (vec == 4) return launch_step_t<IoBf16, 4>(a, s);
  if (vec == 2) return launch_step_t<IoBf16, 2>(a, s);
  return launch_step_t<IoBf16, 1>(a, s);
}

hipError_t launch_state_copy(int64_t B, int64_t C, const float* state_in, float* state_out,
                             hipStream_t s) {
  const int64_t n = B * C;
  const int64_t blocks = (3 * n + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(wkv_state_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     n, state_in, state_out);
  return hipGetLastError();
}

}  // namespace wkv
