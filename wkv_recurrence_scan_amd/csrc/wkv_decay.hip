// WKV with a per-token (data-dependent) decay rate.
//
// The page "RWKV-v6 Architecture: Attention-Free Linear Transformers"
// (section "The Core Components of the RWKV-v6 Time-Mixing Block", the items
// on the dynamic data-dependent decay and on the matrix-valued state) computes
// the decay from every token and applies step t's decay to the state carried
// in from step t-1 before step t's own term is added. Here the vector-state
// operator of the page "Linear attention without writing a CUDA kernel"
// (section "The recurrence") takes a positive rate w[b][t][c] per token and
// channel: step t multiplies the state by e^(-w_t). A constant rate gives the
// constant-decay operator.
//
// Precision. With a rate per token the running maximum can no longer be kept
// as (key, whole number of steps); instead every exponent that accumulates
// rates -- the running maximum, a segment's total rate and the decay behind
// each token of a sub-chunk -- is fp64, and differences are rounded to fp32
// only right before v_exp_f32. Values, numerators and denominators stay fp32.
// The fp64 work is a handful of adds and conversions per token, small next to
// the 16 bytes per channel-token these kernels move.
//
// Kernels: a channel-parallel sequential scan (large B*C), a chunked scan
// over time (small B*C) with the layout of the constant-decay chunked scan --
// a segment summary carries its total rate where that one carries a length --
// and the batched decode step.
#include "wkv_device.h"
#include "wkv_internal.h"
#include "wkv_tile.h"
#include "wkv_decay_lane.h"

#include <type_traits>

namespace wkv {
namespace {

__device__ __forceinline__ SegD shfl_up_segd(const SegD& x, int delta) {
  SegD r;
  r.n = __shfl_up(x.n, delta, 64);
  r.d = __shfl_up(x.d, delta, 64);
  r.m = __shfl_up(x.m, delta, 64);
  r.ws = __shfl_up(x.ws, delta, 64);
  return r;
}

// Summary of one thread's sub-chunk. Token i has decayed by the rates of the
// sub-chunk's later steps (accumulated in fp64, newest first); its exponent
// k_i minus that stays fp64, and so does the maximum, so each weight's
// exponent difference is rounded to fp32 only once, right before v_exp_f32
// (rounding k_i minus the decay to fp32 first would move every weight by up
// to ulp(|k|): 5e-4 at |k| = 1e4). MASKED: only the first nvalid tokens exist.
template <int L, bool MASKED>
__device__ __forceinline__ SegD summarize_d(const float (&kk)[L], const float (&vv)[L],
                                            const float (&ww)[L], int nvalid) {
  double z[L];
  double suf = 0.0;
  double top = kEmptyD;
#pragma unroll
  for (int i = L - 1; i >= 0; --i) {
    z[i] = kEmptyD;
    if (!MASKED || i < nvalid) {
      z[i] = static_cast<double>(kk[i]) - suf;
      suf += static_cast<double>(ww[i]);
      top = __builtin_fmax(top, z[i]);
    }
  }
  float n = 0.0f, d = 0.0f;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    float e = fast_exp2(static_cast<float>(z[i] - top) * kLog2e);
    if (MASKED && i >= nvalid) e = 0.0f;
    d += e;
    n = __builtin_fmaf(e, vv[i], n);
  }
  return SegD{n, d, top, suf};
}

template <int V>
__device__ __forceinline__ void load_state_d(const float* __restrict__ state_in, int64_t lane0,
                                             int64_t plane, LaneD (&s)[V]) {
  if (state_in != nullptr) {
    float n[V], d[V], m[V];
    IoF32::load<V, false>(state_in + lane0, n);
    IoF32::load<V, false>(state_in + plane + lane0, d);
    IoF32::load<V, false>(state_in + 2 * plane + lane0, m);
#pragma unroll
    for (int j = 0; j < V; ++j) s[j] = LaneD{n[j], d[j], static_cast<double>(m[j])};
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) s[j] = laned_empty();
  }
}

template <int V>
__device__ __forceinline__ void store_state_d(float* __restrict__ state_out, int64_t lane0,
                                              int64_t plane, const LaneD (&s)[V]) {
  float n[V], d[V], m[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    n[j] = s[j].n;
    d[j] = s[j].d;
    m[j] = static_cast<float>(s[j].m);
  }
  IoF32::store<V, false>(state_out + lane0, n);
  IoF32::store<V, false>(state_out + plane + lane0, d);
  IoF32::store<V, false>(state_out + 2 * plane + lane0, m);
}

// ------------------------------------------------------ sequential scan

constexpr int kDdSeqThreads = 256;

template <int V, int U>
struct DdBlock {
  float k[U][V];
  float v[U][V];
  float w[U][V];
};

template <typename IoT, int V, int U>
__device__ __forceinline__ void dd_seq_load(DdBlock<V, U>& blk,
                                            const typename IoT::elem* __restrict__ kp,
                                            const typename IoT::elem* __restrict__ vp,
                                            const typename IoT::elem* __restrict__ wp, int64_t C) {
#pragma unroll
  for (int i = 0; i < U; ++i) {
    IoT::template load<V, true>(kp + i * C, blk.k[i]);
    IoT::template load<V, true>(vp + i * C, blk.v[i]);
    IoT::template load<V, true>(wp + i * C, blk.w[i]);
  }
}

template <typename IoT, int V, int U>
__device__ __forceinline__ void dd_seq_compute(const DdBlock<V, U>& blk, LaneD (&s)[V],
                                               const double (&ud)[V],
                                               typename IoT::elem* __restrict__ op, int64_t C) {
#pragma unroll
  for (int i = 0; i < U; ++i) {
    float o[V];
#pragma unroll
    for (int j = 0; j < V; ++j) o[j] = laned_step(s[j], blk.k[i][j], blk.v[i][j], blk.w[i][j], ud[j]);
    IoT::template store<V, true>(op + i * C, o);
  }
}

// CK: also save the backward's checkpoints (one channel per thread; the
// blocks of U = kCkptTokens tokens are the checkpoint chunks).
template <typename IoT, int V, int U, bool CK>
__global__ __launch_bounds__(kDdSeqThreads) void wkv_dd_seq_kernel(
    int64_t B, int64_t T, int64_t C, const typename IoT::elem* __restrict__ w,
    const float* __restrict__ u, const typename IoT::elem* __restrict__ k,
    const typename IoT::elem* __restrict__ v, const float* __restrict__ state_in,
    typename IoT::elem* __restrict__ out, float* __restrict__ state_out,
    LaneCk* __restrict__ ckpt) {
  static_assert(!CK || (V == 1 && U == kCkptTokens), "checkpoints: one channel, 8-token blocks");
  const int64_t groups_per_row = C / V;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kDdSeqThreads + threadIdx.x;
  if (gid >= B * groups_per_row) return;
  const int64_t b = gid / groups_per_row;
  const int64_t c0 = (gid - b * groups_per_row) * V;
  const int64_t plane = B * C;
  const int64_t lane0 = b * C + c0;

  float uu[V];
  IoF32::load<V, false>(u + c0, uu);
  double ud[V];
#pragma unroll
  for (int j = 0; j < V; ++j) ud[j] = static_cast<double>(uu[j]);
  LaneD s[V];
  load_state_d<V>(state_in, lane0, plane, s);

  const int64_t row = b * T * C + c0;
  const typename IoT::elem* kp = k + row;
  const typename IoT::elem* vp = v + row;
  const typename IoT::elem* wp = w + row;
  typename IoT::elem* op = out + row;

  // two register buffers; the next block's loads are issued before the
  // current block is computed, unconditionally inside the loop, so the
  // counter-based waits stop at the block about to be used; the last one or
  // two blocks are computed after the loop, so no block is read twice
  DdBlock<V, U> A, Bf;
  auto load = [&](DdBlock<V, U>& x, int64_t blk) {
    const int64_t t = blk * U;
    dd_seq_load<IoT, V, U>(x, kp + t * C, vp + t * C, wp + t * C, C);
  };
  auto run = [&](const DdBlock<V, U>& x, int64_t blk) {
    if constexpr (CK) ckpt[blk * plane + lane0] = LaneCk{s[0].n, s[0].d, s[0].m};
    dd_seq_compute<IoT, V, U>(x, s, ud, op + blk * U * C, C);
  };
  const int64_t nblk = T / U;
  if (nblk > 0) load(A, 0);
  int64_t blk = 0;
  for (; blk + 2 < nblk; blk += 2) {
    load(Bf, blk + 1);
    run(A, blk);
    load(A, blk + 2);
    run(Bf, blk + 1);
  }
  if (blk + 1 < nblk) {  // two left
    load(Bf, blk + 1);
    run(A, blk);
    run(Bf, blk + 1);
  } else if (blk < nblk) {  // one left
    run(A, blk);
  }
  if constexpr (CK) {
    if (nblk * U < T) ckpt[nblk * plane + lane0] = LaneCk{s[0].n, s[0].d, s[0].m};
  }
  for (int64_t t = nblk * U; t < T; ++t) {
    float kk[V], vv[V], ww[V], o[V];
    IoT::template load<V, true>(kp + t * C, kk);
    IoT::template load<V, true>(vp + t * C, vv);
    IoT::template load<V, true>(wp + t * C, ww);
#pragma unroll
    for (int j = 0; j < V; ++j) o[j] = laned_step(s[j], kk[j], vv[j], ww[j], ud[j]);
    IoT::template store<V, true>(op + t * C, o);
  }
  if (state_out != nullptr) store_state_d<V>(state_out, lane0, plane, s);
}

// ------------------------------------------------------ chunked scan

constexpr int kDdLC = 32, kDdPS = 2;

template <int V, int L>
struct DdRegs {
  float k[L][V];
  float v[L][V];
  float w[L][V];
};

template <typename IoT, int V, int L, bool MASKED>
__device__ __forceinline__ void dd_chunk_load(DdRegs<V, L>& r,
                                              const typename IoT::elem* __restrict__ kp,
                                              const typename IoT::elem* __restrict__ vp,
                                              const typename IoT::elem* __restrict__ wp, int64_t C,
                                              int nvalid) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (!MASKED || i < nvalid) {
      IoT::template load<V, false>(kp + i * C, r.k[i]);
      IoT::template load<V, false>(vp + i * C, r.v[i]);
      IoT::template load<V, false>(wp + i * C, r.w[i]);
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) r.k[i][j] = r.v[i][j] = r.w[i][j] = 0.0f;
    }
  }
}

// One tile: summaries, scan inside the wave, wave totals through LDS, the
// state in front of every sub-chunk, then the rescan of each thread's tokens.
// CK: the re-scan also saves the state in front of every token whose index
// is a multiple of kCkptTokens to ck[(index / kCkptTokens) * lanes + lane]
// (one channel per thread); tok0 is the index of the thread's first token.
template <typename IoT, int V, int LC, int PS, int W, int L, bool MASKED, bool CK>
__device__ __forceinline__ void dd_chunk_tile(const DdRegs<V, L>& r, int nvalid, LaneD (&carry)[V],
                                              const double (&ud)[V], SegD (*tot)[LC * V],
                                              typename IoT::elem* __restrict__ op, int64_t C,
                                              bool cvalid, int wave, int sl, int cl,
                                              LaneCk* __restrict__ ck, int64_t lanes,
                                              int64_t lane, int64_t tok0) {
  static_assert(!CK || V == 1, "checkpoints are saved by one-channel threads");
  SegD inc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    float kk[L], vv[L], ww[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      kk[i] = r.k[i][j];
      vv[i] = r.v[i][j];
      ww[i] = r.w[i][j];
    }
    inc[j] = summarize_d<L, MASKED>(kk, vv, ww, nvalid);
  }
#pragma unroll
  for (int off = 1; off < PS; off <<= 1) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const SegD p = shfl_up_segd(inc[j], off * LC);
      if (sl >= off) inc[j] = segd_combine(p, inc[j]);
    }
  }
  SegD exc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const SegD p = shfl_up_segd(inc[j], LC);
    exc[j] = sl > 0 ? p : segd_identity();
  }
  if (sl == PS - 1) {
#pragma unroll
    for (int j = 0; j < V; ++j) tot[wave][cl * V + j] = inc[j];
  }
  __syncthreads();
  LaneD pre[V];
#pragma unroll
  for (int jj = 0; jj < W; ++jj) {
    if (jj == wave) {
#pragma unroll
      for (int j = 0; j < V; ++j) pre[j] = carry[j];
    }
#pragma unroll
    for (int j = 0; j < V; ++j) laned_absorb(carry[j], tot[jj][cl * V + j]);
  }
#pragma unroll
  for (int j = 0; j < V; ++j) laned_absorb(pre[j], exc[j]);
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (!MASKED || i < nvalid) {
      if constexpr (CK) {
        const int64_t t = tok0 + i;
        if (cvalid && (t % kCkptTokens) == 0)
          ck[(t / kCkptTokens) * lanes + lane] = LaneCk{pre[0].n, pre[0].d, pre[0].m};
      }
      float o[V];
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] = laned_step(pre[j], r.k[i][j], r.v[i][j], r.w[i][j], ud[j]);
      if (cvalid) IoT::template store<V, true>(op + i * C, o);
    }
  }
}

template <typename IoT, int V, int LC, int PS, int W, int L, bool CK>
__global__ __launch_bounds__(64 * W) void wkv_dd_chunk_kernel(
    int64_t B, int64_t T, int64_t C, const typename IoT::elem* __restrict__ w,
    const float* __restrict__ u, const typename IoT::elem* __restrict__ k,
    const typename IoT::elem* __restrict__ v, const float* __restrict__ state_in,
    typename IoT::elem* __restrict__ out, float* __restrict__ state_out, int64_t groups_per_row,
    LaneCk* __restrict__ ckpt) {
  static_assert(LC * PS == 64, "a wave is LC channel groups by PS sub-chunks");
  constexpr int CH = LC * V;
  constexpr int TL = W * PS * L;
  __shared__ SegD tot[2][W][CH];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int cl = lane % LC;
  const int sl = lane / LC;
  const int sub = wave * PS + sl;

  const int64_t g = xcd_swizzle(blockIdx.x, B * groups_per_row);
  const int64_t b = g / groups_per_row;
  const int64_t c0 = (g - b * groups_per_row) * CH + cl * V;
  const bool cvalid = c0 < C;
  const int64_t cc = cvalid ? c0 : C - V;  // idle tail threads mirror the last channels
  const int64_t plane = B * C;
  const int64_t lane0 = b * C + cc;

  float uu[V];
  IoF32::load<V, false>(u + cc, uu);
  double ud[V];
#pragma unroll
  for (int j = 0; j < V; ++j) ud[j] = static_cast<double>(uu[j]);
  LaneD carry[V];
  load_state_d<V>(state_in, lane0, plane, carry);

  const int64_t base = b * T * C + cc + static_cast<int64_t>(sub) * L * C;
  const typename IoT::elem* kp = k + base;
  const typename IoT::elem* vp = v + base;
  const typename IoT::elem* wp = w + base;
  typename IoT::elem* op = out + base;
  const int64_t step = static_cast<int64_t>(TL) * C;

  const int64_t full = T / TL;
  auto tok0 = [&](int64_t tile) { return tile * TL + static_cast<int64_t>(sub) * L; };
  DdRegs<V, L> A, Bf;
  if (full > 0) dd_chunk_load<IoT, V, L, false>(A, kp, vp, wp, C, L);
  for (int64_t tile = 0; tile < full; tile += 2) {
    const int64_t nb = tile + 1 < full ? tile + 1 : full - 1;
    dd_chunk_load<IoT, V, L, false>(Bf, kp + nb * step, vp + nb * step, wp + nb * step, C, L);
    dd_chunk_tile<IoT, V, LC, PS, W, L, false, CK>(A, L, carry, ud, tot[tile & 1],
                                                   op + tile * step, C, cvalid, wave, sl, cl,
                                                   ckpt, plane, lane0, tok0(tile));
    if (tile + 1 >= full) break;
    const int64_t na = tile + 2 < full ? tile + 2 : full - 1;
    dd_chunk_load<IoT, V, L, false>(A, kp + na * step, vp + na * step, wp + na * step, C, L);
    dd_chunk_tile<IoT, V, LC, PS, W, L, false, CK>(Bf, L, carry, ud, tot[(tile + 1) & 1],
                                                   op + (tile + 1) * step, C, cvalid, wave, sl,
                                                   cl, ckpt, plane, lane0, tok0(tile + 1));
  }
  if (full * TL < T) {  // last, partial tile
    const int64_t first = full * TL + static_cast<int64_t>(sub) * L;
    const int64_t left = T - first;
    const int nvalid = left <= 0 ? 0 : (left >= L ? L : static_cast<int>(left));
    DdRegs<V, L> last;
    dd_chunk_load<IoT, V, L, true>(last, kp + full * step, vp + full * step, wp + full * step, C,
                                   nvalid);
    dd_chunk_tile<IoT, V, LC, PS, W, L, true, CK>(last, nvalid, carry, ud, tot[full & 1],
                                                  op + full * step, C, cvalid, wave, sl, cl, ckpt,
                                                  plane, lane0, tok0(full));
  }
  if (state_out != nullptr && sub == 0 && cvalid) store_state_d<V>(state_out, lane0, plane, carry);
}

// ------------------------------------------------------ decode step

constexpr int kDdStepThreads = 256;

template <typename IoT, int V>
__global__ __launch_bounds__(kDdStepThreads) void wkv_dd_step_kernel(
    int64_t B, int64_t C, const typename IoT::elem* __restrict__ w, const float* __restrict__ u,
    const typename IoT::elem* __restrict__ k, const typename IoT::elem* __restrict__ v,
    float* __restrict__ state, typename IoT::elem* __restrict__ out) {
  const int64_t groups_per_row = C / V;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kDdStepThreads + threadIdx.x;
  if (gid >= B * groups_per_row) return;
  const int64_t b = gid / groups_per_row;
  const int64_t c0 = (gid - b * groups_per_row) * V;
  const int64_t lane0 = b * C + c0;
  const int64_t plane = B * C;

  float ww[V], uu[V], kk[V], vv[V], o[V];
  IoT::template load<V, true>(w + lane0, ww);
  IoF32::load<V, false>(u + c0, uu);
  IoT::template load<V, true>(k + lane0, kk);
  IoT::template load<V, true>(v + lane0, vv);
  LaneD s[V];
  load_state_d<V>(state, lane0, plane, s);
#pragma unroll
  for (int j = 0; j < V; ++j) o[j] = laned_step(s[j], kk[j], vv[j], ww[j], static_cast<double>(uu[j]));
  IoT::template store<V, true>(out + lane0, o);
  store_state_d<V>(state, lane0, plane, s);
}

// ------------------------------------------------------ launchers

template <typename T>
const T* cp(const void* p) {
  return static_cast<const T*>(p);
}

template <typename IoT, int V>
hipError_t launch_dd_seq_t(const DdArgs& a, hipStream_t st) {
  constexpr int U = 8;
  const int64_t threads = a.B * (a.C / V);
  const int64_t blocks = (threads + kDdSeqThreads - 1) / kDdSeqThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  using E = typename IoT::elem;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kDdSeqThreads);
  auto* ck = static_cast<LaneCk*>(a.ckpt);
  if constexpr (std::is_same<IoT, IoF32>::value && V == 1) {
    if (ck != nullptr) {
      hipLaunchKernelGGL((wkv_dd_seq_kernel<IoT, V, U, true>), grid, block, 0, st, a.B, a.T, a.C,
                         cp<E>(a.w), a.u, cp<E>(a.k), cp<E>(a.v), a.state_in,
                         static_cast<E*>(a.out), a.state_out, ck);
      return hipGetLastError();
    }
  } else {
    if (ck != nullptr) return hipErrorInvalidValue;  // checkpoints: fp32 only
  }
  hipLaunchKernelGGL((wkv_dd_seq_kernel<IoT, V, U, false>), grid, block, 0, st, a.B, a.T, a.C,
                     cp<E>(a.w), a.u, cp<E>(a.k), cp<E>(a.v), a.state_in, static_cast<E*>(a.out),
                     a.state_out, nullptr);
  return hipGetLastError();
}

template <typename IoT, int V, int W, int L>
hipError_t launch_dd_chunk_t(const DdArgs& a, hipStream_t st) {
  constexpr int CH = kDdLC * V;
  const int64_t gpr = (a.C + CH - 1) / CH;
  const int64_t blocks = a.B * gpr;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  using E = typename IoT::elem;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * W);
  auto* ck = static_cast<LaneCk*>(a.ckpt);
  if constexpr (std::is_same<IoT, IoF32>::value && V == 1) {
    if (ck != nullptr) {
      hipLaunchKernelGGL((wkv_dd_chunk_kernel<IoT, V, kDdLC, kDdPS, W, L, true>), grid, block, 0,
                         st, a.B, a.T, a.C, cp<E>(a.w), a.u, cp<E>(a.k), cp<E>(a.v), a.state_in,
                         static_cast<E*>(a.out), a.state_out, gpr, ck);
      return hipGetLastError();
    }
  } else {
    if (ck != nullptr) return hipErrorInvalidValue;  // checkpoints: fp32 only
  }
  hipLaunchKernelGGL((wkv_dd_chunk_kernel<IoT, V, kDdLC, kDdPS, W, L, false>), grid, block, 0, st,
                     a.B, a.T, a.C, cp<E>(a.w), a.u, cp<E>(a.k), cp<E>(a.v), a.state_in,
                     static_cast<E*>(a.out), a.state_out, gpr, nullptr);
  return hipGetLastError();
}

// Tile shapes: short sequences want few serial tiles; longer ones two waves
// per SIMD. The rate array makes the register tile half as large again as the
// constant-decay scan's, so tiles hold fewer tokens per thread (no spills at
// these shapes).
constexpr int64_t kDdShortT = 256, kDdLongT = 2048;

template <typename IoT, int V>
hipError_t launch_dd_chunk_v(const DdArgs& a, hipStream_t st) {
  // measured on MI355X (fp32; bf16 pairs take half the tokens per thread):
  // B=8 T=1024 C=768 26.4 us with 8 waves of 8 tokens against 29.8 us with
  // 16 waves; B=4 T=16384 C=2048 450 us with 4 waves of 16 against 468-488
  if (a.T <= kDdShortT) return launch_dd_chunk_t<IoT, V, 8, 4>(a, st);
  if (a.T <= kDdLongT) return launch_dd_chunk_t<IoT, V, 8, V == 1 ? 8 : 4>(a, st);
  return launch_dd_chunk_t<IoT, V, 4, V == 1 ? 16 : 8>(a, st);
}

template <typename IoT, int V>
hipError_t launch_dd_step_t(const DdStepArgs& a, hipStream_t st) {
  const int64_t threads = a.B * (a.C / V);
  const int64_t blocks = (threads + kDdStepThreads - 1) / kDdStepThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  using E = typename IoT::elem;
  hipLaunchKernelGGL((wkv_dd_step_kernel<IoT, V>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kDdStepThreads), 0, st, a.B, a.C, cp<E>(a.w), a.u, cp<E>(a.k),
                     cp<E>(a.v), a.state, static_cast<E*>(a.out));
  return hipGetLastError();
}

bool aligned(const void* p, int bytes) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

}  // namespace

int dd_vec_width(int io, int64_t C, const DdArgs& a) {
  if (io != kBf16) return 1;
  const bool ok = C % 2 == 0 && aligned(a.k, 4) && aligned(a.v, 4) && aligned(a.w, 4) &&
                  aligned(a.out, 4) && aligned(a.u, 8) && aligned(a.state_in, 8) &&
                  aligned(a.state_out, 8);
  return ok ? 2 : 1;
}

// fp32: one channel per thread, as the constant-decay step (more blocks for
// a short pass); bf16: the widest width the pointers allow.
int dd_step_vec_width(int io, int64_t C, const DdStepArgs& a) {
  if (io == kF32) return 1;
  const int elem = 2;
  for (int V : {4, 2, 1}) {
    if (C % V) continue;
    if (!aligned(a.k, V * elem) || !aligned(a.v, V * elem) || !aligned(a.w, V * elem) ||
        !aligned(a.out, V * elem))
      continue;
    if (!aligned(a.u, V * 4) || !aligned(a.state, V * 4)) continue;
    return V;
  }
  return 1;
}

hipError_t launch_dd_seq(const DdArgs& a, int io, int vec, hipStream_t s) {
  if (io == kF32) return launch_dd_seq_t<IoF32, 1>(a, s);
  if (vec == 2) return launch_dd_seq_t<IoBf16, 2>(a, s);
  return launch_dd_seq_t<IoBf16, 1>(a, s);
}

hipError_t launch_dd_chunk(const DdArgs& a, int io, int vec, int cus, hipStream_t s) {
  if (io == kF32) return launch_dd_chunk_v<IoF32, 1>(a, s);
  // Two bf16 channels per thread halve the workgroups; while that leaves CUs
  // idle, one channel per thread is faster (measured on MI355X, bf16: B=8
  // T=1024 C=768 24.5 against 49.2 us, B=4 T=2048 C=2048 55.9 against 94.8;
  // B=32 T=512 C=1024, 512 two-channel workgroups, 54.4 against 53.9).
  const int64_t two_ch_blocks = a.B * ((a.C + 2 * kDdLC - 1) / (2 * kDdLC));
  if (vec == 2 && two_ch_blocks >= cus) return launch_dd_chunk_v<IoBf16, 2>(a, s);
  return launch_dd_chunk_v<IoBf16, 1>(a, s);
}

hipError_t launch_dd_step(const DdStepArgs& a, int io, int vec, hipStream_t s) {
  if (io == kF32) return launch_dd_step_t<IoF32, 1>(a, s);
  if (vec == 4) return launch_dd_step_t<IoBf16, 4>(a, s);
  if (vec == 2) return launch_dd_step_t<IoBf16, 2>(a, s);
  return launch_dd_step_t<IoBf16, 1>(a, s);
}

}  // namespace wkv
