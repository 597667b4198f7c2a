// Token shift: the input of each projection of a time-mixing block is the
// current token vector moved towards the one before it by a per-channel
// fraction, x'_p,t = x_t + (x_{t-1} - x_t) * mu_p (page "RWKV-v6
// Architecture: Attention-Free Linear Transformers", section "The Core
// Components of the RWKV-v6 Time-Mixing Block", item 1, Data-Dependent Token
// Shift; page "RWKV: Merging Transformer Training with RNN Speed",
// Time-Mixing block). It produces the WKV operator's inputs, ahead of the
// projections, so it is a kernel of its own rather than fused into the scan.
//
// Elementwise and bound by HBM: x is read once (plus one token per run of
// 8 or 16 tokens, the token before the run), and P mixes are written. A
// thread owns V adjacent channels (16 bytes) of one batch row for a run of
// tokens and keeps the previous token in registers; the 64 lanes of a wave
// cover 64 consecutive 16-byte pieces of a row, so every load and store
// instruction of a wave touches one contiguous 1 KiB. The token before a
// call's first one is x_prev (zeros when absent); the thread of each row's
// first run also writes the row's last token to x_last, after it has read
// x_prev, so x_last may be x_prev itself (decode in place).
#include "wkv_device.h"
#include "wkv_internal.h"

#include <type_traits>

namespace wkv {
namespace {

constexpr int kShiftThreads = 256;
// tokens per thread: 16 (8 for bf16's 8-channel pieces, whose run would
// otherwise take 128 registers)
template <int V>
constexpr int shift_run() { return V > 4 ? 8 : 16; }

template <typename IoT, int V, int P>
__global__ __launch_bounds__(kShiftThreads) void wkv_shift_kernel(
    int64_t B, int64_t T, int64_t C, const float* __restrict__ mu,
    const typename IoT::elem* __restrict__ x, const typename IoT::elem* x_prev,
    typename IoT::elem* __restrict__ out, typename IoT::elem* x_last) {
  using E = typename IoT::elem;
  constexpr int kShiftRun = shift_run<V>();
  const int64_t nvec = C / V;
  const int64_t runs = (T + kShiftRun - 1) / kShiftRun;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * kShiftThreads + threadIdx.x;
  if (id >= B * runs * nvec) return;
  const int64_t cv = id % nvec;  // channel piece, fastest: a wave covers consecutive pieces
  const int64_t rest = id / nvec;
  const int64_t j = rest % runs;
  const int64_t b = rest / runs;
  const int64_t c0 = cv * V;
  const int64_t t0 = j * kShiftRun;
  const int64_t n = T - t0 < kShiftRun ? T - t0 : kShiftRun;

  float m[P][V];
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int i = 0; i < V; ++i) m[p][i] = mu[p * C + c0 + i];
  }

  const E* xr = x + b * T * C + c0;
  float prev[V];
  if (t0 > 0) {
    IoT::template load<V, false>(xr + (t0 - 1) * C, prev);
  } else if (x_prev != nullptr) {
    IoT::template load<V, false>(x_prev + b * C + c0, prev);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) prev[i] = 0.0f;
  }
  if (t0 == 0 && x_last != nullptr) {
    // read before written: x_last may be x_prev
    float last[V];
    IoT::template load<V, true>(xr + (T - 1) * C, last);
    IoT::template store<V, false>(x_last + b * C + c0, last);
  }

  // the run's tokens, all loads first (full runs unconditionally)
  float cur[kShiftRun][V];
  if (n == kShiftRun) {
#pragma unroll
    for (int t = 0; t < kShiftRun; ++t) IoT::template load<V, true>(xr + (t0 + t) * C, cur[t]);
  } else {
#pragma unroll
    for (int t = 0; t < kShiftRun; ++t)
      if (t < n) IoT::template load<V, true>(xr + (t0 + t) * C, cur[t]);
  }
  const int64_t plane = B * T * C;
  E* orow = out + b * T * C + c0;
#pragma unroll
  for (int t = 0; t < kShiftRun; ++t) {
    if (t < n) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float o[V];
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = __builtin_fmaf(m[p][i], prev[i] - cur[t][i], cur[t][i]);
        IoT::template store<V, true>(orow + p * plane + (t0 + t) * C, o);
      }
#pragma unroll
      for (int i = 0; i < V; ++i) prev[i] = cur[t][i];
    }
  }
}

// T == 0: x_last <- x_prev (or zeros).
template <typename E>
__global__ __launch_bounds__(kShiftThreads) void wkv_shift_carry_kernel(int64_t n, const E* src,
                                                                        E* dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kShiftThreads + threadIdx.x;
  if (i < n) dst[i] = src != nullptr ? src[i] : E(0);
}

template <typename IoT, int V, int P>
hipError_t launch_shift_vp(const ShiftArgs& a, hipStream_t st) {
  using E = typename IoT::elem;
  constexpr int kShiftRun = shift_run<V>();
  const int64_t runs = (a.T + kShiftRun - 1) / kShiftRun;
  const int64_t items = a.B * runs * (a.C / V);
  const int64_t blocks = (items + kShiftThreads - 1) / kShiftThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((wkv_shift_kernel<IoT, V, P>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kShiftThreads), 0, st, a.B, a.T, a.C, a.mu,
                     static_cast<const E*>(a.x), static_cast<const E*>(a.x_prev),
                     static_cast<E*>(a.out), static_cast<E*>(a.x_last));
  return hipGetLastError();
}

template <typename IoT, int V>
hipError_t launch_shift_v(const ShiftArgs& a, hipStream_t st) {
  switch (a.P) {
    case 1: return launch_shift_vp<IoT, V, 1>(a, st);
    case 2: return launch_shift_vp<IoT, V, 2>(a, st);
    case 3: return launch_shift_vp<IoT, V, 3>(a, st);
    case 4: return launch_shift_vp<IoT, V, 4>(a, st);
    case 5: return launch_shift_vp<IoT, V, 5>(a, st);
    case 6: return launch_shift_vp<IoT, V, 6>(a, st);
    case 7: return launch_shift_vp<IoT, V, 7>(a, st);
    case 8: return launch_shift_vp<IoT, V, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

bool aligned(const void* p, int bytes) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

}  // namespace

hipError_t launch_shift(const ShiftArgs& a, int io, hipStream_t st) {
  if (a.T == 0) {
    if (a.x_last == nullptr || a.x_last == a.x_prev) return hipSuccess;
    const int64_t n = a.B * a.C;
    const int64_t blocks = (n + kShiftThreads - 1) / kShiftThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (io == kBf16) {
      hipLaunchKernelGGL(wkv_shift_carry_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kShiftThreads), 0, st, n, static_cast<const uint16_t*>(a.x_prev),
                         static_cast<uint16_t*>(a.x_last));
    } else {
      hipLaunchKernelGGL(wkv_shift_carry_kernel<float>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kShiftThreads), 0, st, n, static_cast<const float*>(a.x_prev),
                         static_cast<float*>(a.x_last));
    }
    return hipGetLastError();
  }
  // 16-byte pieces when C and every pointer allow them, else one channel
  const int es = io == kBf16 ? 2 : 4;
  const int wide = 16 / es;
  const bool ok = a.C % wide == 0 && aligned(a.x, 16) && aligned(a.x_prev, 16) &&
                  aligned(a.out, 16) && aligned(a.x_last, 16) && aligned(a.mu, 16);
  if (io == kBf16) {
    return ok ? launch_shift_v<IoBf16, 8>(a, st) : launch_shift_v<IoBf16, 1>(a, st);
  }
  return ok ? launch_shift_v<IoF32, 4>(a, st) : launch_shift_v<IoF32, 1>(a, st);
}

}  // namespace wkv
