// Single-pass time-parallel prefill with decoupled look-back.
//
// The time-parallel form of RWKV is an associative prefix scan over time
// (page "RWKV-v6 Architecture: Attention-Free Linear Transformers", section on
// architectural duality; page "RWKV: Merging Transformer Training with RNN
// Speed", paragraph on the time-parallel mode). Here the sequence is cut into
// segments of one tile each, and every (segment, channel group) pair is one
// workgroup, so a problem with few (b, c) lanes still fills the GPU; k and v
// are read from HBM once.
//
// A workgroup:
//   1. serves channel group blockIdx % G and takes that group's next segment
//      from the group's own ticket counter, so every segment it will wait for
//      was taken by a workgroup that has already started: no co-residency or
//      dispatch order is assumed and no wait can deadlock (per-group counters
//      also keep the counter atomics off a single address);
//   2. loads its tile (L tokens of k and v per thread), summarises each
//      sub-chunk and scans the sub-chunks (lane shuffles in a wave, LDS
//      across waves) into the tile's aggregate;
//   3. publishes its aggregate, then looks back: every K-th segment (an
//      anchor; K = 8 for fp32) publishes its inclusive prefix, and a segment
//      starts from the inclusive prefix of the last anchor before it and folds
//      in the aggregates of the segments in between, oldest first. The
//      workgroup's threads fetch those K words groups side by side (one per
//      thread), so the look-back costs one round trip; the fold order is
//      fixed, so results do not depend on timing (the kernel is
//      deterministic), and anchors chain only T / (K tiles) deep;
//   4. every thread re-runs the recurrence over its registers from its
//      sub-chunk's start state and writes the outputs.
//
// Publication uses 64-bit words tagged with a per-launch epoch in their high
// half and written/read with device-scope relaxed atomics: a value is
// accepted only when its tag is the current epoch, so the words need no
// fences and nothing has to be cleared between launches. The epoch lives in
// the workspace (a launch counter that the last channel group to finish
// advances), so a launch replayed from a HIP graph still gets a fresh one;
// tags are never 0, so a zero-filled workspace holds no valid word. The
// workspace's layout depends on the problem's sizes: reusing it for other
// sizes needs it zero-filled again. Inclusive prefixes
// keep their maximum index-tracked (base, age), so chains of segments do not
// accumulate rounding. Every wait is bounded: past the limit a workgroup
// flags an error word in the workspace and proceeds, so the kernel always
// finishes.
#include "wkv_device.h"
#include "wkv_internal.h"
#include "wkv_tile.h"

#include <type_traits>

namespace wkv {
namespace {

constexpr int kLbLC = 32, kLbPS = 2;
// Every K-th segment publishes its inclusive prefix, K = (threads per
// workgroup) / (channels per workgroup). A segment needs its anchor's prefix
// and the aggregates in between: one word group per (slot, channel), fetched
// by one thread each, so a workgroup's threads cover all of them at once.
template <int V, int W>
constexpr int64_t anchor_spacing() { return (64 * W) / (kLbLC * V); }
// Bound on every wait, in polls (~1 us each): far above any wait a correct
// launch sees (microseconds), small enough that a broken one still ends fast.
constexpr uint32_t kSpinLimit = 1u << 14;

__device__ __forceinline__ void put(uint64_t* p, float x, uint32_t epoch) {
  const uint64_t word = (static_cast<uint64_t>(epoch) << 32) | __float_as_uint(x);
  __hip_atomic_store(p, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool get(uint64_t* p, uint32_t epoch, float& x) {
  const uint64_t word = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  x = __uint_as_float(static_cast<uint32_t>(word));
  return static_cast<uint32_t>(word >> 32) == epoch;
}

struct LbArgs {
  int64_t groups;       // G: channel groups (B * groups_per_row)
  int64_t segments;     // S: segments per lane
  int64_t gpr;          // channel groups per batch row
  uint32_t* ctrl;       // [0] error flag, [1] launch count, [2] finished groups;
                        // per group g at [4 + 4g]: ticket, finished workgroups
  uint64_t* agg;        // [S][G][CH][3] tile aggregates (n, d, m)
  uint64_t* inc;        // [S][G][CH][4] inclusive prefixes (n, d, base, age)
  uint32_t epoch;       // tag of this launch's words: launch count + 1 (never 0)
};

// Wait (bounded) until the n tagged words at p carry this launch's epoch and
// return their values. Past the limit the error word is set and zeros are
// returned, so the kernel still finishes.
template <int N>
__device__ __forceinline__ void wait_words(const LbArgs& a, uint64_t* p, float (&x)[N]) {
  for (uint32_t spin = 0;; ++spin) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = get(p + i, a.epoch, x[i]) && ok;
    if (ok) return;
    if (spin >= kSpinLimit) {
      __hip_atomic_fetch_or(a.ctrl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int i = 0; i < N; ++i) x[i] = 0.0f;
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

template <typename IoT, int V, int W, int L, bool MASKED>
__device__ __forceinline__ void lb_tile(const LbArgs& a, int64_t s, int64_t g, int64_t B, int64_t T,
                                        int64_t C, const float* __restrict__ w,
                                        const float* __restrict__ u,
                                        const typename IoT::elem* __restrict__ k,
                                        const typename IoT::elem* __restrict__ v,
                                        const float* __restrict__ state_in,
                                        typename IoT::elem* __restrict__ out,
                                        float* __restrict__ state_out, Seg (*tot)[kLbLC * V],
                                        Lane* xs, Seg (*fetched)[kLbLC * V]) {
  constexpr int LC = kLbLC, PS = kLbPS, CH = LC * V, TL = W * PS * L;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int cl = lane % LC;
  const int sl = lane / LC;
  const int sub = wave * PS + sl;

  const int64_t b = g / a.gpr;
  const int64_t c0 = (g - b * a.gpr) * CH + cl * V;
  const bool cvalid = c0 < C;
  const int64_t cc = cvalid ? c0 : C - V;
  const int64_t plane = B * C;
  const int64_t lane0 = b * C + cc;

  float wd[V], ub[V];
  IoF32::load<V, false>(w + cc, wd);
  IoF32::load<V, false>(u + cc, ub);

  const int64_t first = s * TL + static_cast<int64_t>(sub) * L;
  const int64_t left = T - first;
  const int nvalid = MASKED ? (left <= 0 ? 0 : (left >= L ? L : static_cast<int>(left))) : L;
  const int64_t base = b * T * C + cc + first * C;
  ChunkRegs<V, L> r;
  chunk_load<IoT, V, L, MASKED>(r, k + base, v + base, C, nvalid);

  // sub-chunk summaries, scan inside the wave, wave totals through LDS
  Seg inc[V], exc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    float kk[L], vv[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      kk[i] = r.k[i][j];
      vv[i] = r.v[i][j];
    }
    inc[j] = summarize<L, MASKED>(kk, vv, wd[j], nvalid);
  }
#pragma unroll
  for (int off = 1; off < PS; off <<= 1) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const Seg p = shfl_up_seg(inc[j], off * LC);
      if (sl >= off) inc[j] = seg_combine(p, inc[j], wd[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const Seg p = shfl_up_seg(inc[j], LC);
    exc[j] = sl > 0 ? p : seg_identity();
  }
  if (sl == PS - 1) {
#pragma unroll
    for (int j = 0; j < V; ++j) tot[wave][cl * V + j] = inc[j];
  }
  __syncthreads();
  Seg before[V], whole[V];  // waves before this one; the whole tile
#pragma unroll
  for (int j = 0; j < V; ++j) whole[j] = seg_identity();
#pragma unroll
  for (int jj = 0; jj < W; ++jj) {
    if (jj == wave) {
#pragma unroll
      for (int j = 0; j < V; ++j) before[j] = whole[j];
    }
#pragma unroll
    for (int j = 0; j < V; ++j) whole[j] = seg_combine(whole[j], tot[jj][cl * V + j], wd[j]);
  }

  // Look-back. Segment s > 0 starts from the inclusive prefix of the last
  // anchor before it and folds in, oldest first, the aggregates of the
  // segments in between; that fold order is fixed, so the kernel is
  // deterministic. Non-anchor segments publish their aggregate first (later
  // segments fold it in); anchors publish their inclusive prefix at the end.
  constexpr int64_t K = anchor_spacing<V, W>();
  const bool is_anchor = s % K == 0;
  const int64_t anchor = s == 0 ? 0 : ((s - 1) / K) * K;
  if (s > 0 && !is_anchor && wave == 0 && sl == 0) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      uint64_t* pa = a.agg + ((s * a.groups + g) * CH + cl * V + j) * 3;
      put(pa, whole[j].n, a.epoch);
      put(pa + 1, whole[j].d, a.epoch);
      put(pa + 2, whole[j].m, a.epoch);
    }
  }
  if (s > 0) {
    // thread (slot r, channel c): slot 0 is the anchor's prefix, slot r > 0
    // the aggregate of segment anchor + r; all waits run side by side
    const int c = tid % CH;
    const int rslot = tid / CH;
    const int64_t seg = anchor + rslot;
    if (rslot == 0) {
      float x[4];
      wait_words<4>(a, a.inc + ((seg * a.groups + g) * CH + c) * 4, x);
      fetched[0][c] = Seg{x[0], x[1], x[2], x[3]};
    } else if (seg < s) {
      float x[3];
      wait_words<3>(a, a.agg + ((seg * a.groups + g) * CH + c) * 3, x);
      fetched[rslot][c] = Seg{x[0], x[1], x[2], static_cast<float>(TL)};
    }
  }
  __syncthreads();
  if (wave == 0 && sl == 0) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int idx = cl * V + j;
      Lane x;
      if (s == 0) {
        x = state_in != nullptr ? lane_from_state(state_in[lane0 + j], state_in[plane + lane0 + j],
                                                  state_in[2 * plane + lane0 + j])
                                : lane_empty();
      } else {
        const Seg& p = fetched[0][idx];  // (n, d, base, age) of the anchor's prefix
        x = Lane{p.n, p.d, p.m, p.len};
        for (int64_t r = 1; anchor + r < s; ++r) lane_absorb(x, fetched[r][idx], wd[j]);
      }
      Lane incl = x;
      lane_absorb(incl, whole[j], wd[j]);
      if (is_anchor) {
        uint64_t* pi = a.inc + ((s * a.groups + g) * CH + idx) * 4;
        put(pi, incl.n, a.epoch);
        put(pi + 1, incl.d, a.epoch);
        put(pi + 2, incl.base, a.epoch);
        put(pi + 3, incl.age, a.epoch);
      }
      xs[idx] = x;
      if (s == a.segments - 1 && state_out != nullptr && cvalid) {
        state_out[lane0 + j] = incl.n;
        state_out[plane + lane0 + j] = incl.d;
        state_out[2 * plane + lane0 + j] = lane_max_exp(incl, wd[j]);
      }
    }
  }
  __syncthreads();

  // every thread: state in front of its sub-chunk, then the rescan
  Lane pre[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    pre[j] = xs[cl * V + j];
    lane_absorb(pre[j], before[j], wd[j]);
    lane_absorb(pre[j], exc[j], wd[j]);
  }
  typename IoT::elem* op = out + base;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (!MASKED || i < nvalid) {
      float o[V];
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] = lane_step(pre[j], r.k[i][j], r.v[i][j], wd[j], ub[j]);
      if (cvalid) IoT::template store<V, true>(op + i * C, o);
    }
  }
}

template <typename IoT, int V, int W, int L>
__global__ __launch_bounds__(64 * W) void wkv_lookback_kernel(
    int64_t B, int64_t T, int64_t C, const float* __restrict__ w, const float* __restrict__ u,
    const typename IoT::elem* __restrict__ k, const typename IoT::elem* __restrict__ v,
    const float* __restrict__ state_in, typename IoT::elem* __restrict__ out,
    float* __restrict__ state_out, LbArgs a) {
  // (state_in is read by segment 0's workgroups before state_out is written
  // by the last segment's, which waited on segment 0 through the published
  // prefixes, so the two may be the same buffer)
  constexpr int CH = kLbLC * V, TL = W * kLbPS * L;
  __shared__ Seg tot[W][CH];
  __shared__ Lane xs[CH];
  __shared__ Seg fetched[anchor_spacing<V, W>()][CH];
  __shared__ uint32_t seg_s, epoch_s;

  // Work assignment per channel group: block i serves group i % G and takes
  // the group's next segment from the group's own ticket counter, so within a
  // group segments are handed out in start order (every segment a workgroup
  // waits for belongs to a workgroup that has already started) and the
  // counters' atomics are spread over G addresses.
  const int64_t g = blockIdx.x % a.groups;
  uint32_t* gc = a.ctrl + 4 + 4 * g;  // ticket, finished workgroups
  if (threadIdx.x == 0) {
    seg_s = __hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t launches = __hip_atomic_load(a.ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    epoch_s = launches % 0xffffffffu + 1u;
  }
  __syncthreads();
  a.epoch = epoch_s;
  const int64_t s = seg_s;
  if (s >= a.segments) {
    // only possible with a workspace that was not zero-filled: do no work
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_or(a.ctrl, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if ((s + 1) * TL <= T) {
    lb_tile<IoT, V, W, L, false>(a, s, g, B, T, C, w, u, k, v, state_in, out, state_out, tot,
                                 xs, fetched);
  } else {
    lb_tile<IoT, V, W, L, true>(a, s, g, B, T, C, w, u, k, v, state_in, out, state_out, tot, xs,
                                fetched);
  }
  // The group's last workgroup returns the group's counters to zero; the last
  // group to finish (every workgroup of the launch has then read the launch
  // count) advances the launch count, so the next launch, replayed from a
  // graph or not, tags its words differently.
  if (threadIdx.x == 0) {
    const uint32_t done =
        __hip_atomic_fetch_add(gc + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
    if (done == static_cast<uint32_t>(a.segments)) {
      __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(gc + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t groups_done =
          __hip_atomic_fetch_add(a.ctrl + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
      if (groups_done == static_cast<uint32_t>(a.groups)) {
        __hip_atomic_store(a.ctrl + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(a.ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Workgroup shape by sequence length (measured on MI355X): W waves of two
// 32-channel sub-chunk rows, L tokens per sub-chunk, so a segment (one tile)
// is 2*W*L tokens. One function decides; sizing and launching both go
// through it, so they cannot disagree.
constexpr int64_t kLbShortT = 512, kLbMidT = 2048;

template <class F>
auto lb_dispatch(int64_t T, F&& f) {
  if (T <= kLbShortT) return f(std::integral_constant<int, 4>{}, std::integral_constant<int, 4>{});
  if (T <= kLbMidT) return f(std::integral_constant<int, 8>{}, std::integral_constant<int, 16>{});
  return f(std::integral_constant<int, 4>{}, std::integral_constant<int, 32>{});
}

// Control words: an error word and launch counters, then four words per
// channel group, rounded up to 256 bytes so the tagged words after them stay
// aligned.
int64_t lookback_ctrl_bytes(int64_t groups) { return ((16 + 16 * groups + 255) / 256) * 256; }

template <int V, int W, int L>
int64_t lb_bytes(int64_t B, int64_t T, int64_t C) {
  constexpr int64_t CH = kLbLC * V, TL = W * kLbPS * L;
  const int64_t groups = B * ((C + CH - 1) / CH);
  const int64_t segments = (T + TL - 1) / TL;
  return lookback_ctrl_bytes(groups) +
         groups * segments * CH * 7 * static_cast<int64_t>(sizeof(uint64_t));
}

template <typename IoT, int V, int W, int L>
hipError_t launch_lb_t(const FwdArgs& a, const LbWorkspace& ws, hipStream_t st) {
  constexpr int CH = kLbLC * V, TL = W * kLbPS * L;
  // the slots this launch indexes must lie inside the workspace it was given
  if (ws.bytes < lb_bytes<V, W, L>(a.B, a.T, a.C)) return hipErrorInvalidValue;
  const int64_t gpr = (a.C + CH - 1) / CH;
  const int64_t groups = a.B * gpr;
  const int64_t segments = (a.T + TL - 1) / TL;
  const int64_t items = groups * segments;
  if (items > 0x7fffffff) return hipErrorInvalidConfiguration;
  LbArgs la;
  la.groups = groups;
  la.segments = segments;
  la.gpr = gpr;
  la.ctrl = ws.ctrl;
  uint64_t* slots = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws.ctrl) +
                                                lookback_ctrl_bytes(groups));
  la.agg = slots;
  la.inc = slots + items * CH * 3;
  la.epoch = 0;  // read from the workspace by the kernel
  hipLaunchKernelGGL((wkv_lookback_kernel<IoT, V, W, L>), dim3(static_cast<unsigned>(items)),
                     dim3(64 * W), 0, st, a.B, a.T, a.C, a.w, a.u,
                     static_cast<const typename IoT::elem*>(a.k),
                     static_cast<const typename IoT::elem*>(a.v), a.state_in,
                     static_cast<typename IoT::elem*>(a.out), a.state_out, la);
  return hipGetLastError();
}

template <typename IoT, int V>
hipError_t launch_lb_v(const FwdArgs& a, const LbWorkspace& ws, hipStream_t st) {
  return lb_dispatch(a.T, [&](auto w, auto l) {
    return launch_lb_t<IoT, V, decltype(w)::value, decltype(l)::value>(a, ws, st);
  });
}

}  // namespace

int lookback_vec_width(int io, int64_t C, const FwdArgs& a) { return chunk_vec_width(io, C, a); }

int64_t lookback_workspace_bytes(int vec, int64_t B, int64_t T, int64_t C) {
  return lb_dispatch(T, [&](auto w, auto l) {
    return vec == 2 ? lb_bytes<2, decltype(w)::value, decltype(l)::value>(B, T, C)
                    : lb_bytes<1, decltype(w)::value, decltype(l)::value>(B, T, C);
  });
}

hipError_t launch_lookback(const FwdArgs& a, int io, int vec, const LbWorkspace& ws,
                           hipStream_t s) {
  if (io == kF32) return launch_lb_v<IoF32, 1>(a, ws, s);
  if (vec == 2) return launch_lb_v<IoBf16, 2>(a, ws, s);
  return launch_lb_v<IoBf16, 1>(a, ws, s);
}

}  // namespace wkv
