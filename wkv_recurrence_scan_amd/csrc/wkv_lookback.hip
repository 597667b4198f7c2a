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
//   1. serves a channel group (one block per group in every row of G blocks;
//      a group keeps its XCD, and every XCD serves a mix of column offsets)
//      and takes that group's next segment
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
// fences and nothing has to be cleared between launches. Each channel group's
// ticket counter is never reset: every launch advances it by exactly S (the
// segments per group), so ticket t means segment t mod S of launch t / S, and
// the launch number gives the epoch (a launch replayed from a HIP graph gets
// a fresh one too, and nothing has to run before or after the scan to keep
// the counters in step). That holds while a workspace keeps its layout (the
// number of channel groups G and of segments S): the first launch on a
// zero-filled workspace claims it for its (G, S) (one workgroup stores the
// claim; the others only load it), and a launch with another (G, S) on the
// same workspace finds the claim,
// flags the error word and produces NaN instead of mixing with the other
// layout's words. Tags are never 0, so a zero-filled workspace holds no valid
// word. Inclusive prefixes keep their maximum index-tracked (base, age), so
// chains of segments do not accumulate rounding. Every wait is bounded: past
// the limit a workgroup sets the workspace's sticky error word and carries on
// with a NaN prefix, so the kernel always finishes and the outputs that
// depended on the missing words are NaN, never plausible values; the host
// reads the error word back with wkv_workspace_status.
//
// While its ticket is in flight a workgroup already loads the tile of the
// segment it will most likely get (blocks of a group start in index order),
// and loads again only if the ticket says otherwise; the guess only decides
// what is prefetched, never which segment is processed.
#include "wkv_device.h"
#include "wkv_internal.h"
#include "wkv_tile.h"

#include <type_traits>

namespace wkv {
namespace {

// Lane layouts: LC lanes of adjacent channels by PS = 64 / LC sub-chunk rows
// per wave (LC = 32: two 128-byte row pieces per load instruction; LC = 64:
// one 256-byte piece).
// Every K-th segment publishes its inclusive prefix, K = (threads per
// workgroup) / (channels per workgroup). A segment needs its anchor's prefix
// and the aggregates in between: one word group per (slot, channel), fetched
// by one thread each, so a workgroup's threads cover all of them at once.
template <int V, int W, int LC>
constexpr int64_t anchor_spacing() { return (64 * W) / (LC * V); }
// Bound on every wait, in polls (~1 us each): far above any wait a correct
// launch sees (microseconds), small enough that a broken one still ends fast.
constexpr uint32_t kSpinLimit = 1u << 14;

// Control words at the start of the workspace (32-bit each): [0] the sticky
// error word (bit 0: a wait ran out, as when overlapping launches share the
// workspace; bit 2: the workspace is claimed by another layout), [1] a word
// only tests write (bit 0: publish nothing, so that every wait runs out;
// bits 8-31: a replacement for kSpinLimit, 0 for none), [2..3] the 64-bit
// claim (G << 32 | S, 0 while unclaimed). Then per channel group a 64-bit
// ticket counter, 16 bytes apart.
constexpr int kCtrlErr = 0, kCtrlTest = 1, kCtrlClaim = 2;
constexpr uint32_t kTestNoPublish = 1u;
constexpr int kTicketStride = 4;  // in 32-bit words

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
  uint32_t* ctrl;       // control words (kCtrl*), then the ticket counters
  uint64_t* agg;        // [S][G][CH][3] tile aggregates (n, d, m)
  uint64_t* inc;        // [S][G][CH][4] inclusive prefixes (n, d, base, age)
  uint32_t epoch;       // tag of this launch's words (never 0), read by the kernel
  uint32_t spin_limit;  // polls before a wait gives up, read by the kernel
  bool publish;         // false only when a test asked for it, read by the kernel
  bool claimed;         // false: the workspace belongs to another layout (read nothing)
};

// Wait (bounded) until the n tagged words at p carry this launch's epoch and
// return their values. Past the limit the error word is set and NaNs are
// returned, so the kernel still finishes and what depends on them is NaN.
template <int N>
__device__ __forceinline__ void wait_words(const LbArgs& a, uint64_t* p, float (&x)[N]) {
  if (!a.claimed) {  // another layout's words: none may be read (already flagged)
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = __builtin_nanf("");
    return;
  }
  for (uint32_t spin = 0;; ++spin) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = get(p + i, a.epoch, x[i]) && ok;
    if (ok) return;
    if (spin >= a.spin_limit) {
      __hip_atomic_fetch_or(a.ctrl + kCtrlErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int i = 0; i < N; ++i) x[i] = __builtin_nanf("");
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Offset of thread (wave, lane)'s first token of segment s in k, v and out.
template <int V, int W, int L, int LC>
__device__ __forceinline__ int64_t lb_offset(int64_t s, int64_t g, int64_t gpr, int64_t T,
                                             int64_t C) {
  constexpr int PS = 64 / LC, CH = LC * V, TL = W * PS * L;
  const int lane = threadIdx.x & 63;
  const int sub = (threadIdx.x >> 6) * PS + lane / LC;
  const int64_t b = g / gpr;
  const int64_t c0 = (g - b * gpr) * CH + (lane % LC) * V;
  const int64_t cc = c0 < C ? c0 : C - V;
  return b * T * C + cc + (s * TL + static_cast<int64_t>(sub) * L) * C;
}

// One segment of one channel group; r holds this thread's tokens of it
// (loaded by the caller), the first nvalid of them valid.
template <typename IoT, int V, int W, int L, int LC, bool MASKED, bool G>
__device__ __forceinline__ void lb_tile(const LbArgs& a, int64_t s, int64_t g, int64_t B, int64_t T,
                                        int64_t C, const float* __restrict__ w,
                                        const float* __restrict__ u,
                                        const ChunkRegs<V, L, G>& r, int nvalid,
                                        const float* __restrict__ state_in,
                                        typename IoT::elem* __restrict__ out,
                                        float* __restrict__ state_out, Seg (*tot)[LC * V],
                                        Lane* xs, Seg (*fetched)[LC * V]) {
  constexpr int PS = 64 / LC, CH = LC * V, TL = W * PS * L;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int cl = lane % LC;
  const int sl = lane / LC;

  const int64_t b = g / a.gpr;
  const int64_t c0 = (g - b * a.gpr) * CH + cl * V;
  const bool cvalid = c0 < C;
  const int64_t cc = cvalid ? c0 : C - V;
  const int64_t plane = B * C;
  const int64_t lane0 = b * C + cc;
  const int64_t base = lb_offset<V, W, L, LC>(s, g, a.gpr, T, C);

  float wd[V], ub[V];
  IoF32::load<V, false>(w + cc, wd);
  IoF32::load<V, false>(u + cc, ub);

  // sub-chunk summaries, scan inside the wave, wave totals through LDS
  Seg exc[V], before[V], whole[V];
  tile_scan<V, LC, PS, W, L, MASKED>(r, wd, nvalid, tot, exc, before, whole);

  // Look-back. Segment s > 0 starts from the inclusive prefix of the last
  // anchor before it and folds in, oldest first, the aggregates of the
  // segments in between; that fold order is fixed, so the kernel is
  // deterministic. Non-anchor segments publish their aggregate first (later
  // segments fold it in); anchors publish their inclusive prefix at the end.
  constexpr int64_t K = anchor_spacing<V, W, LC>();
  const bool is_anchor = s % K == 0;
  const int64_t anchor = s == 0 ? 0 : ((s - 1) / K) * K;
  if (a.publish && s > 0 && !is_anchor && wave == 0 && sl == 0) {
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
      if (is_anchor && a.publish) {
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
  float cb[V];
  bonus_ratios(wd, ub, cb);
  rescan_sel<IoT, V, L, MASKED, G>(wave_fast_ok(wd, ub), pre, r, wd, ub, cb, nvalid, cvalid,
                                   out + base, C);
}

template <typename IoT, int V, int W, int L, int LC, bool G>
__global__ __launch_bounds__(64 * W) void wkv_lookback_kernel(
    int64_t B, int64_t T, int64_t C, const float* __restrict__ w, const float* __restrict__ u,
    const typename IoT::elem* __restrict__ k, const typename IoT::elem* __restrict__ v,
    const typename IoT::elem* __restrict__ rg, const float* __restrict__ state_in,
    typename IoT::elem* __restrict__ out, float* __restrict__ state_out, LbArgs a) {
  // (state_in is read by segment 0's workgroups before state_out is written
  // by the last segment's, which waited on segment 0 through the published
  // prefixes, so the two may be the same buffer)
  constexpr int PS = 64 / LC, CH = LC * V, TL = W * PS * L;
  __shared__ Seg tot[W][CH];
  __shared__ Lane xs[CH];
  __shared__ Seg fetched[anchor_spacing<V, W, LC>()][CH];
  __shared__ uint32_t seg_s, epoch_s, test_s, ours_s;

  // Work assignment per channel group: block i = q G + o (row q, offset o)
  // serves group g(o), the same group in every row, and takes the group's
  // next segment from the group's own ticket counter, so within a group
  // segments are handed out in start order (every segment a workgroup waits
  // for belongs to a workgroup that has already started) and the counters'
  // atomics are spread over G addresses.
  // Blocks are dealt to the 8 XCDs round-robin. When G is a multiple of 8 a
  // group's blocks therefore all run on one XCD and start in row order, which
  // keeps the prefetch guess below right (a group whose blocks hop between
  // XCDs gets its tickets out of row order whenever one XCD runs ahead, and
  // every wrong guess fetches a tile twice). g(o) then permutes each run of
  // 8 offsets by its run index, so that every XCD serves every residue of g
  // mod 8, i.e. every 128-byte column offset within 1 KiB: measured on
  // MI355X, some column offsets stream more slowly than others, and an XCD
  // holding only those falls behind the rest.
  const int64_t row = blockIdx.x / a.groups;
  const int64_t o = blockIdx.x - row * a.groups;
  const int64_t g = (a.groups % kNumXcd) != 0
                        ? o
                        : (o & ~int64_t{kNumXcd - 1}) | (((o & (kNumXcd - 1)) + (o / kNumXcd)) &
                                                         (kNumXcd - 1));
  // thread 0 issues its ticket, the layout claim and the test word together
  // (one round trip); their values are needed only after the tile's prefetch
  // is issued
  uint64_t ticket = 0, claim = 0, words = 0;
  const uint64_t layout =
      (static_cast<uint64_t>(a.groups) << 32) | static_cast<uint64_t>(a.segments);
  if (threadIdx.x == 0) {
    // (the ticket last: the compiler waits for its value at once, and then
    // the two loads are in flight already)
    claim = __hip_atomic_load(reinterpret_cast<uint64_t*>(a.ctrl + kCtrlClaim), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    words = __hip_atomic_load(reinterpret_cast<uint64_t*>(a.ctrl + kCtrlErr), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    ticket = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(a.ctrl + kTicketStride) +
                                        2 * g,
                                    uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // prefetch the likely segment's tile while the ticket is in flight: the
  // group's blocks are one per row, so this block is most likely its row-th
  const int64_t guess = row;
  const bool guess_full = (guess + 1) * TL <= T;
  ChunkRegs<V, L, G> r;
  auto rat = [&](int64_t off) { return G ? rg + off : rg; };
  if (guess_full) {
    const int64_t off = lb_offset<V, W, L, LC>(guess, g, a.gpr, T, C);
    chunk_load<IoT, V, L, false, G>(r, k + off, v + off, rat(off), C, L);
  }
  const uint64_t S = static_cast<uint64_t>(a.segments);
  if (threadIdx.x == 0) {
    // an unclaimed (zero-filled) workspace holds no valid word, so every
    // workgroup of its first launch may go ahead; the one with group 0's
    // first ticket records the claim for the launches after it (a store by
    // one workgroup, not an atomic update by all)
    const bool ours = claim == 0 || claim == layout;
    if (claim == 0 && ticket == 0 && g == 0)
      __hip_atomic_store(reinterpret_cast<uint64_t*>(a.ctrl + kCtrlClaim), layout,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!ours)
      __hip_atomic_fetch_or(a.ctrl + kCtrlErr, 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    seg_s = static_cast<uint32_t>(ticket % S);
    epoch_s = static_cast<uint32_t>((ticket / S) % 0xffffffffull) + 1u;
    test_s = static_cast<uint32_t>(words >> 32);
    ours_s = ours ? 1u : 0u;
  }
  __syncthreads();
  a.epoch = epoch_s;
  a.spin_limit = (test_s >> 8) != 0u ? (test_s >> 8) : kSpinLimit;
  a.claimed = ours_s != 0u;
  a.publish = a.claimed && (test_s & kTestNoPublish) == 0u;
  const int64_t s = seg_s;
  const int64_t off = lb_offset<V, W, L, LC>(s, g, a.gpr, T, C);
  if ((s + 1) * TL <= T) {
    if (!guess_full || s != guess) {
      chunk_load<IoT, V, L, false, G>(r, k + off, v + off, rat(off), C, L);
    }
    lb_tile<IoT, V, W, L, LC, false, G>(a, s, g, B, T, C, w, u, r, L, state_in, out, state_out,
                                        tot, xs, fetched);
  } else {
    const int sub = (threadIdx.x >> 6) * PS + (threadIdx.x & 63) / LC;
    const int64_t left = T - (s * TL + static_cast<int64_t>(sub) * L);
    const int nvalid = left <= 0 ? 0 : (left >= L ? L : static_cast<int>(left));
    chunk_load<IoT, V, L, true, G>(r, k + off, v + off, rat(off), C, nvalid);
    lb_tile<IoT, V, W, L, LC, true, G>(a, s, g, B, T, C, w, u, r, nvalid, state_in, out,
                                       state_out, tot, xs, fetched);
  }
}

// Workgroup shape by sequence length and form (measured on MI355X): V
// channels per thread (at most VMAX, what the pointers allow), W waves of
// PS = 64 / LC sub-chunk rows of LC channel lanes, L tokens per sub-chunk,
// so a segment (one tile) is W PS L tokens. Past 2048 tokens every form
// takes one channel per thread: ungated in one 64-channel row per wave (8
// waves of 32 tokens; the plain copy pattern of one 256-byte piece per load
// instruction streams at 0.75 of the HBM peak against 0.67 for two 128-byte
// pieces): B=4 T=16384 C=2048 fp32 304-306 against 310-320 us, bf16 209-215
// against 226-249 (two channels per thread held 209 registers there);
// gated, where 147 registers would leave one such 8-wave workgroup per CU,
// in 32-channel pairs of 4 waves: fp32 354-366 against 414-424 us, bf16
// 319-321 against 391 with two channels per thread. One function decides;
// sizing and launching both go through it, so they cannot disagree.
constexpr int64_t kLbShortT = 512, kLbMidT = 2048;

template <int N>
using Int = std::integral_constant<int, N>;

// f(V, W, L, LC) as integral constants
template <int VMAX, class F>
auto lb_dispatch(bool gated, int64_t T, F&& f) {
  if (T <= kLbShortT) return f(Int<VMAX>{}, Int<4>{}, Int<4>{}, Int<32>{});
  if (T <= kLbMidT) return f(Int<VMAX>{}, Int<8>{}, Int<16>{}, Int<32>{});
  if (!gated) return f(Int<1>{}, Int<8>{}, Int<32>{}, Int<64>{});
  return f(Int<1>{}, Int<4>{}, Int<32>{}, Int<32>{});
}

// Control words (16 bytes), then one 64-bit ticket counter per channel group
// (16 bytes apart), rounded up to 256 bytes so the tagged words after them
// stay aligned.
int64_t lookback_ctrl_bytes(int64_t groups) {
  return ((16 + 4 * kTicketStride * groups + 255) / 256) * 256;
}

template <int V, int W, int L, int LC>
int64_t lb_bytes(int64_t B, int64_t T, int64_t C) {
  constexpr int64_t CH = LC * V, TL = W * (64 / LC) * L;
  const int64_t groups = B * ((C + CH - 1) / CH);
  const int64_t segments = (T + TL - 1) / TL;
  return lookback_ctrl_bytes(groups) +
         groups * segments * CH * 7 * static_cast<int64_t>(sizeof(uint64_t));
}

template <typename IoT, int V, int W, int L, int LC>
hipError_t launch_lb_t(const FwdArgs& a, const LbWorkspace& ws, hipStream_t st) {
  constexpr int CH = LC * V, TL = W * (64 / LC) * L;
  // the slots this launch indexes must lie inside the workspace it was given
  if (ws.bytes < lb_bytes<V, W, L, LC>(a.B, a.T, a.C)) return hipErrorInvalidValue;
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
  la.epoch = 0;          // these three are read from the control words by the kernel
  la.spin_limit = kSpinLimit;
  la.publish = true;
  la.claimed = true;
  const auto* kk = static_cast<const typename IoT::elem*>(a.k);
  const auto* vv = static_cast<const typename IoT::elem*>(a.v);
  const auto* rr = static_cast<const typename IoT::elem*>(a.r);
  auto* oo = static_cast<typename IoT::elem*>(a.out);
  if (rr != nullptr) {
    hipLaunchKernelGGL((wkv_lookback_kernel<IoT, V, W, L, LC, true>),
                       dim3(static_cast<unsigned>(items)), dim3(64 * W), 0, st, a.B, a.T, a.C,
                       a.w, a.u, kk, vv, rr, a.state_in, oo, a.state_out, la);
  } else {
    hipLaunchKernelGGL((wkv_lookback_kernel<IoT, V, W, L, LC, false>),
                       dim3(static_cast<unsigned>(items)), dim3(64 * W), 0, st, a.B, a.T, a.C,
                       a.w, a.u, kk, vv, rr, a.state_in, oo, a.state_out, la);
  }
  return hipGetLastError();
}

template <typename IoT, int VMAX>
hipError_t launch_lb_io(const FwdArgs& a, const LbWorkspace& ws, hipStream_t st) {
  return lb_dispatch<VMAX>(a.r != nullptr, a.T, [&](auto v, auto w, auto l, auto lc) {
    return launch_lb_t<IoT, decltype(v)::value, decltype(w)::value, decltype(l)::value,
                       decltype(lc)::value>(a, ws, st);
  });
}

template <int VMAX>
int64_t lb_bytes_any(int64_t B, int64_t T, int64_t C) {
  // the larger of the gated and the plain layout: one workspace serves a
  // call whichever it takes
  int64_t most = 0;
  for (bool gated : {false, true}) {
    const int64_t n = lb_dispatch<VMAX>(gated, T, [&](auto v, auto w, auto l, auto lc) {
      return lb_bytes<decltype(v)::value, decltype(w)::value, decltype(l)::value,
                      decltype(lc)::value>(B, T, C);
    });
    most = n > most ? n : most;
  }
  return most;
}

}  // namespace

namespace {
__global__ __launch_bounds__(256) void wkv_zero_fill(uint4* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t{256} + threadIdx.x; i < n; i += int64_t{gridDim.x} * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}
}  // namespace

hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(wkv_zero_fill, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<uint4*>(p), n);
  return hipGetLastError();
}

int lookback_vec_width(int io, int64_t C, const FwdArgs& a) { return chunk_vec_width(io, C, a); }

int64_t lookback_workspace_bytes(int vec, int64_t B, int64_t T, int64_t C) {
  return vec == 2 ? lb_bytes_any<2>(B, T, C) : lb_bytes_any<1>(B, T, C);
}

hipError_t launch_lookback(const FwdArgs& a, int io, int vec, const LbWorkspace& ws,
                           hipStream_t s) {
  if (io == kF32) return launch_lb_io<IoF32, 1>(a, ws, s);
  if (vec == 2) return launch_lb_io<IoBf16, 2>(a, ws, s);
  return launch_lb_io<IoBf16, 1>(a, ws, s);
}

}  // namespace wkv
