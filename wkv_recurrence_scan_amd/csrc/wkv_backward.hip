// Backward pass of the WKV operator: gradients of a loss with respect to w,
// u, k, v and the initial state, given the loss's gradient with respect to
// the outputs (and, optionally, to the final state).
//
// The operator is the wkv_t equation of the page "Linear attention without
// writing a CUDA kernel", section "The recurrence": out_t = Num_t / Den_t,
// sums over the initial state, the past tokens i < t (weight
// e^{k_i - (t-1-i) w}) and the current token (weight e^{u + k_t}). Its
// derivatives follow from the quotient rule; with a_t = g_t / Den_t
// (g_t = dL/dout_t) and, for each position i, the suffix sums over later
// positions t > i
//   P_i  = sum a_t e^{-(t-1-i) w},          Q_i  = sum a_t out_t e^{-(t-1-i) w},
//   R_i  = sum (t-1-i) a_t e^{-(t-1-i) w},  Rq_i = sum (t-1-i) a_t out_t e^{-(t-1-i) w},
// they are
//   dL/dv_i = g_i E_i / Den_i + e^{k_i} P_i                      (E_i = e^{u + k_i})
//   dL/dk_i = g_i E_i (v_i - out_i) / Den_i + e^{k_i} (v_i P_i - Q_i)
//   dL/du   = sum_i g_i E_i (v_i - out_i) / Den_i
//   dL/dw   = -sum_i e^{k_i} (v_i R_i - Rq_i)   (+ the initial state's term)
// and the suffix sums run backwards in time as a scan with the same decay:
//   P_{i-1} = a_i + e^{-w} P_i,  Q_{i-1} = a_i out_i + e^{-w} Q_i,
//   R_{i-1} = e^{-w} (R_i + P_i), Rq_{i-1} = e^{-w} (Rq_i + Q_i).
// A gradient of the final state enters as P_{T-1} = dL/dN_T, Q_{T-1} =
// -dL/dD_T; the initial state's gradients are e^{m0} P_{-1}, -e^{m0} Q_{-1}.
// The float64 oracle computes the same derivatives term by term.
//
// One thread owns one (b, c) lane (the channel-parallel layout of the
// sequential forward scan) and makes two passes over its sequence:
//   1. forward, state advance only, storing the state every kLc tokens
//      (a checkpoint, 16 bytes) in the workspace;
//   2. backward over the chunks: reload a chunk's checkpoint, k, v and g,
//      rerun the forward over the chunk's kLc tokens in registers (recording
//      out_t, Den_t and the current token's weight), then walk the chunk
//      backwards, emitting dL/dk and dL/dv and carrying the four suffix sums.
// The suffix sums are kept relative to a common exponent z = zb - za w,
// index-tracked like the forward state's maximum, and every mix takes one
// exp2 of minus an absolute difference, so nothing overflows. Per-lane partial
// sums of dL/dw and dL/du go to the workspace and a second kernel adds them
// over the batch in a fixed order (deterministic).
//
// HBM traffic per channel-token (fp32): pass 1 reads k, v (8 B); pass 2 reads
// k, v, g (12 B) and writes dL/dk, dL/dv (8 B); checkpoints add 2 x 16 / kLc B.
// When the forward saved the checkpoints pass 1 is skipped; for small B*C a
// one-pass chunked kernel (further down) then replaces the segmented ones.
#include "wkv_device.h"
#include "wkv_internal.h"
#include "wkv_tile.h"

#include <type_traits>

namespace wkv {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kLc = kCkptTokens;  // tokens per checkpoint chunk

// Suffix sums of one lane, relative to e^z with z = zb - za * w.
struct Suffix {
  float p, q, r, rq, zb, za;
};

// One forward step that also records what the backward walk needs: the
// output, the log-scale M and reciprocal rho of the output's denominator
// (Den = e^M / rho) and the current token's share om = E / Den.
__device__ __forceinline__ float lane_step_rec(Lane& s, float k, float v, float w, float u,
                                               float& M, float& rho, float& om) {
  const float dk = k - s.base;
  const float s1 = __builtin_fmaf(s.age, w, dk + u);  // (u + k) - m
  const float x = fast_exp2(__builtin_fabsf(s1) * -kLog2e);
  const bool cur_wins = s1 > 0.0f;
  const float fa = cur_wins ? x : 1.0f;
  const float fb = cur_wins ? 1.0f : x;
  rho = fast_rcp(__builtin_fmaf(fa, s.d, fb));
  const float out = __builtin_fmaf(fa, s.n, fb * v) * rho;
  M = cur_wins ? k + u : lane_max_exp(s, w);
  om = fb * rho;
  lane_advance(s, k, v, w);
  return out;
}

// L tokens' k, v, dL/dout and, for a gated output (G), the receptance.
template <int L, bool G>
struct ChunkL {
  float k[L], v[L], g[L], r[G ? L : 1];
};
template <bool G>
using Chunk = ChunkL<kLc, G>;

template <bool MASKED, bool G, int L>
__device__ __forceinline__ void load_chunk(ChunkL<L, G>& c, const float* __restrict__ kp,
                                           const float* __restrict__ vp,
                                           const float* __restrict__ gp,
                                           const float* __restrict__ rp, int64_t C, int n) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (!MASKED || i < n) {
      c.k[i] = __builtin_nontemporal_load(kp + i * C);
      c.v[i] = __builtin_nontemporal_load(vp + i * C);
      c.g[i] = __builtin_nontemporal_load(gp + i * C);
      if constexpr (G) c.r[i] = __builtin_nontemporal_load(rp + i * C);
    } else {
      c.k[i] = 0.0f;
      c.v[i] = 0.0f;
      c.g[i] = 0.0f;
      if constexpr (G) c.r[i] = 0.0f;
    }
  }
}

// dL/d(wkv_t) from dL/dout_t: the gate's share when the output is gated.
template <bool G, int L>
__device__ __forceinline__ float wkv_grad(const ChunkL<L, G>& c, int i) {
  if constexpr (G) return c.g[i] * gate(c.r[i]);
  return c.g[i];
}

// What the backward walk needs of each token of a chunk, from a forward run
// over it: the output y, the log-scale M and reciprocal rho of its
// denominator, and the current token's share om (see lane_step_rec).
template <int L>
struct FwdRec {
  float y[L], M[L], rho[L], om[L];
};

// The forward over a chunk of n tokens (all L unless MASKED) from state st.
template <int L, bool MASKED, bool G>
__device__ __forceinline__ void chunk_record(const ChunkL<L, G>& c, int n, Lane st, float w,
                                             float u, FwdRec<L>& f) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (!MASKED || i < n) f.y[i] = lane_step_rec(st, c.k[i], c.v[i], w, u, f.M[i], f.rho[i], f.om[i]);
  }
}

// Backward walk over a recorded chunk, last token first, from the suffix
// sums a at its end (left at the position before it); gk, gv (and gr when G)
// point at the chunk's first token and are written only when `store`. With a
// gate, dL/dr_t = dL/dout_t wkv_t s (1 - s), s = sigmoid(r_t), and the WKV
// sees dL/dout_t s.
template <int L, bool MASKED, bool G>
__device__ __forceinline__ void chunk_walk(const ChunkL<L, G>& c, const FwdRec<L>& f, int n,
                                           Suffix& a, float w, float& gw_acc, float& gu_acc,
                                           float* __restrict__ gkp, float* __restrict__ gvp,
                                           float* __restrict__ grp, int64_t C, bool store) {
#pragma unroll
  for (int i = L - 1; i >= 0; --i) {
    if (!MASKED || i < n) {
      // gradients of token i from the suffix sums over t > i
      float gi = c.g[i];
      if constexpr (G) {
        const float sg = gate(c.r[i]);
        if (store) __builtin_nontemporal_store(gi * f.y[i] * sg * (1.0f - sg), grp + i * C);
        gi *= sg;
      }
      const float e_cur = gi * f.om[i];
      const float ex = fast_exp2(__builtin_fmaf(-a.za, w, c.k[i] + a.zb) * kLog2e);  // e^(k_i+z)
      const float gv = __builtin_fmaf(a.p, ex, e_cur);
      const float gk = __builtin_fmaf(c.v[i], gv, -__builtin_fmaf(a.q, ex, e_cur * f.y[i]));
      gu_acc = __builtin_fmaf(e_cur, c.v[i] - f.y[i], gu_acc);
      gw_acc = __builtin_fmaf(-ex, __builtin_fmaf(c.v[i], a.r, -a.rq), gw_acc);
      if (store) {
        __builtin_nontemporal_store(gk, gkp + i * C);
        __builtin_nontemporal_store(gv, gvp + i * C);
      }
      // token i joins the suffix sums: a new term g_i rho_i e^{-M_i} against
      // the old sums decayed by one step
      const float sg = __builtin_fmaf(a.za + 1.0f, w, -f.M[i] - a.zb);  // -M_i - (z - w)
      const float x = fast_exp2(__builtin_fabsf(sg) * -kLog2e);
      const bool new_wins = sg > 0.0f;
      const float fo = new_wins ? x : 1.0f;
      const float fn = new_wins ? 1.0f : x;
      const float ai = gi * f.rho[i] * fn;
      a.r = fo * (a.r + a.p);
      a.rq = fo * (a.rq + a.q);
      a.p = __builtin_fmaf(fo, a.p, ai);
      a.q = __builtin_fmaf(fo, a.q, ai * f.y[i]);
      a.zb = new_wins ? -f.M[i] : a.zb;
      a.za = new_wins ? 0.0f : a.za + 1.0f;
    }
  }
}

// Backward walk over one chunk of n tokens (all kLc unless MASKED) starting
// from checkpoint state st.
template <bool MASKED, bool G>
__device__ __forceinline__ void chunk_backward(const Chunk<G>& c, int n, Lane st, Suffix& a,
                                               float w, float u, float& gw_acc, float& gu_acc,
                                               float* __restrict__ gkp, float* __restrict__ gvp,
                                               float* __restrict__ grp, int64_t C) {
  FwdRec<kLc> f;
  chunk_record<kLc, MASKED, G>(c, n, st, w, u, f);
  chunk_walk<kLc, MASKED, G>(c, f, n, a, w, gw_acc, gu_acc, gkp, gvp, grp, C, true);
}

// A chunk's own suffix sums at the position before it: the sum over its
// tokens (j = 0, 1, ... from its first) of a_j e^{-j w} times (1, out_j, j,
// j out_j), a_j = dL/dwkv_j / Den_j, relative to the largest exponent
// -M_j - j w.
template <int L, bool MASKED, bool G>
__device__ __forceinline__ Suffix chunk_own_sums(const ChunkL<L, G>& c, const FwdRec<L>& f, int n,
                                                 float w) {
  float p = 0.0f, q = 0.0f, r = 0.0f, rq = 0.0f, zl = kEmpty;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (!MASKED || i < n) {
      const float jj = static_cast<float>(i);
      const float xe = __builtin_fmaf(-jj, w, -f.M[i]);
      const float d = xe - zl;
      const float e = fast_exp2(__builtin_fabsf(d) * -kLog2e);
      const bool nw = d > 0.0f;
      const float fo = nw ? e : 1.0f;
      const float fn = (nw ? 1.0f : e) * wkv_grad<G>(c, i) * f.rho[i];
      p = __builtin_fmaf(fo, p, fn);
      q = __builtin_fmaf(fo, q, fn * f.y[i]);
      r = __builtin_fmaf(fo, r, fn * jj);
      rq = __builtin_fmaf(fo, rq, fn * jj * f.y[i]);
      zl = nw ? xe : zl;
    }
  }
  return Suffix{p, q, r, rq, zl, 0.0f};
}

// Suffix sums across a span X of len tokens: acc holds the sums at the end
// of X (from the tokens after it) and leaves with the sums at the position
// before X: decayed by len steps (their distance-weighted parts gain len times
// the plain ones) plus X's own sums, taken against the larger exponent.
__device__ __forceinline__ void suffix_absorb(Suffix& acc, const Suffix& X, float len, float w) {
  // X's exponent minus acc's once decayed: (X.zb - X.za w) - (acc.zb - (acc.za + len) w)
  const float sg = __builtin_fmaf(acc.za + len - X.za, w, X.zb - acc.zb);
  const float e = fast_exp2(__builtin_fabsf(sg) * -kLog2e);
  const bool xw = sg > 0.0f;
  const float fo = xw ? e : 1.0f;
  const float fx = xw ? 1.0f : e;
  acc.r = __builtin_fmaf(fo, __builtin_fmaf(len, acc.p, acc.r), fx * X.r);
  acc.rq = __builtin_fmaf(fo, __builtin_fmaf(len, acc.q, acc.rq), fx * X.rq);
  acc.p = __builtin_fmaf(fo, acc.p, fx * X.p);
  acc.q = __builtin_fmaf(fo, acc.q, fx * X.q);
  acc.zb = xw ? X.zb : acc.zb;
  acc.za = xw ? X.za : acc.za + len;
}

// Where one lane's tokens are: k, v, g and the gradients at row + t * C.
struct LaneIo {
  const float* k;
  const float* v;
  const float* g;
  const float* r;  // receptance (gated output) or nullptr
  float* gk;
  float* gv;
  float* gr;       // dL/dr or nullptr
  int64_t row, C, step;  // step = kLc * C
  int64_t nfull;         // chunks of kLc tokens that are full
  int rest;              // tokens in the last, partial chunk (0: none)
};

__device__ __forceinline__ Suffix suffix_init(const float* __restrict__ state_out,
                                              const float* __restrict__ gstate_out,
                                              int64_t lanes, int64_t lane) {
  if (gstate_out != nullptr) {
    // dL/dN_T = g_num e^{-m_out}: p = g_num, q = -g_den relative to z = -m_out
    return Suffix{gstate_out[lane], -gstate_out[lanes + lane], 0.0f, 0.0f,
                  -state_out[2 * lanes + lane], 0.0f};
  }
  return Suffix{0.0f, 0.0f, 0.0f, 0.0f, kEmpty, 0.0f};
}

// Forward state advance over chunks [j0, j1) (all full), storing the state in
// front of each chunk when CKPT. Two register buffers used alternately: the
// next chunk's loads are issued before the current one is consumed,
// unconditionally inside the loop so that the compiler's counter waits stay
// exact; the last one or two chunks are consumed after it, so no chunk is
// read twice.
template <bool CKPT>
__device__ __forceinline__ void forward_chunks(Lane& s, const LaneIo& io, int64_t j0, int64_t j1,
                                               float w, float4* __restrict__ ckpt,
                                               int64_t lanes, int64_t lane) {
  float ka[kLc], va[kLc], kb[kLc], vb[kLc];
  auto load2 = [&](float (&kk)[kLc], float (&vv)[kLc], int64_t j) {
#pragma unroll
    for (int i = 0; i < kLc; ++i) {
      kk[i] = __builtin_nontemporal_load(io.k + io.row + j * io.step + i * io.C);
      vv[i] = __builtin_nontemporal_load(io.v + io.row + j * io.step + i * io.C);
    }
  };
  auto advance = [&](const float (&kk)[kLc], const float (&vv)[kLc], int64_t j) {
    if (CKPT) ckpt[j * lanes + lane] = make_float4(s.n, s.d, s.base, s.age);
#pragma unroll
    for (int i = 0; i < kLc; ++i) lane_advance(s, kk[i], vv[i], w);
  };
  if (j0 < j1) load2(ka, va, j0);
  int64_t j = j0;
  for (; j + 2 < j1; j += 2) {
    load2(kb, vb, j + 1);
    advance(ka, va, j);
    load2(ka, va, j + 2);
    advance(kb, vb, j + 1);
  }
  if (j + 1 < j1) {  // two left
    load2(kb, vb, j + 1);
    advance(ka, va, j);
    advance(kb, vb, j + 1);
  } else if (j < j1) {  // one left
    advance(ka, va, j);
  }
}

// The partial last chunk (io.rest tokens) forward, state advance only.
__device__ __forceinline__ void forward_rest(Lane& s, const LaneIo& io, float w) {
  const int64_t off = io.row + io.nfull * io.step;
#pragma unroll
  for (int i = 0; i < kLc; ++i) {
    if (i < io.rest) {
      lane_advance(s, __builtin_nontemporal_load(io.k + off + i * io.C),
                   __builtin_nontemporal_load(io.v + off + i * io.C), w);
    }
  }
}

// Backward walk over chunks [j0, j1) of one lane, last first, from their
// checkpoints; chunk io.nfull (if inside the range) is the partial one.
template <bool G>
__device__ __forceinline__ void backward_chunks(const LaneIo& io, int64_t j0, int64_t j1,
                                                const float4* __restrict__ ckpt, int64_t lanes,
                                                int64_t lane, float w, float u, Suffix& a,
                                                float& gw_acc, float& gu_acc) {
  // r and gr only exist for a gated output
  auto rp = [&](int64_t off) { return G ? io.r + off : io.r; };
  auto grp = [&](int64_t off) { return G ? io.gr + off : io.gr; };
  if (j1 > io.nfull) {  // the partial chunk comes last in time, so first here
    const int64_t off = io.row + io.nfull * io.step;
    Chunk<G> ch;
    load_chunk<true, G>(ch, io.k + off, io.v + off, io.g + off, rp(off), io.C, io.rest);
    const float4 cp = ckpt[io.nfull * lanes + lane];
    chunk_backward<true, G>(ch, io.rest, Lane{cp.x, cp.y, cp.z, cp.w}, a, w, u, gw_acc, gu_acc,
                            io.gk + off, io.gv + off, grp(off), io.C);
    j1 = io.nfull;
  }
  if (j0 >= j1) return;
  auto at = [&](int64_t j) { return io.row + j * io.step; };
  Chunk<G> A, Bf;
  load_chunk<false, G>(A, io.k + at(j1 - 1), io.v + at(j1 - 1), io.g + at(j1 - 1), rp(at(j1 - 1)),
                       io.C, kLc);
  for (int64_t j = j1 - 1; j >= j0; j -= 2) {
    const int64_t jb = j - 1 >= j0 ? j - 1 : j0;
    load_chunk<false, G>(Bf, io.k + at(jb), io.v + at(jb), io.g + at(jb), rp(at(jb)), io.C,
                         kLc);
    float4 cp = ckpt[j * lanes + lane];
    chunk_backward<false, G>(A, kLc, Lane{cp.x, cp.y, cp.z, cp.w}, a, w, u, gw_acc, gu_acc,
                             io.gk + at(j), io.gv + at(j), grp(at(j)), io.C);
    if (j - 1 < j0) break;
    const int64_t ja = j - 2 >= j0 ? j - 2 : j0;
    load_chunk<false, G>(A, io.k + at(ja), io.v + at(ja), io.g + at(ja), rp(at(ja)), io.C, kLc);
    cp = ckpt[(j - 1) * lanes + lane];
    chunk_backward<false, G>(Bf, kLc, Lane{cp.x, cp.y, cp.z, cp.w}, a, w, u, gw_acc, gu_acc,
                             io.gk + at(j - 1), io.gv + at(j - 1), grp(at(j - 1)), io.C);
  }
}

// Gradients of the initial state from the suffix sums at position -1
// (e^{m0} P, -e^{m0} Q) and its share of dL/dw; zeros without one.
__device__ __forceinline__ void initial_state_grad(const Lane& s0, bool have, const Suffix& a,
                                                   float w, float& gw_acc,
                                                   float* __restrict__ gstate_in, int64_t lanes,
                                                   int64_t lane) {
  if (have) {
    const float n0 = s0.n, d0 = s0.d, m0 = s0.base;
    const float e0 = fast_exp2(__builtin_fmaf(-a.za, w, m0 + a.zb) * kLog2e);
    const float gn0 = a.p * e0;
    const float gd0 = -a.q * e0;
    gw_acc = __builtin_fmaf(-e0, __builtin_fmaf(n0, a.r, -d0 * a.rq), gw_acc);
    if (gstate_in != nullptr) {
      gstate_in[lane] = gn0;
      gstate_in[lanes + lane] = gd0;
      gstate_in[2 * lanes + lane] = __builtin_fmaf(n0, gn0, d0 * gd0);
    }
  } else if (gstate_in != nullptr) {
    gstate_in[lane] = 0.0f;
    gstate_in[lanes + lane] = 0.0f;
    gstate_in[2 * lanes + lane] = 0.0f;
  }
}

struct BwdKernelArgs {
  int64_t B, T, C;
  const float* w;
  const float* u;
  const float* k;
  const float* v;
  const float* gout;
  const float* state_in;
  const float* state_out;
  const float* gstate_out;
  const float* r;    // receptance of a gated output, or nullptr
  float* gk;
  float* gv;
  float* gr;         // dL/dr (gated output only)
  float* gstate_in;
  float4* ckpt;      // [chunks][lanes] state in front of each chunk
  float* gw_part;    // [segments][lanes]
  float* gu_part;
  float4* seg_fwd;   // [segments][lanes] forward summary of each segment from empty
  float4* seg_rev;   // [segments][lanes] the segment's own suffix sums (p, q, r, rq)
  float* seg_rev_z;  // [segments][lanes] their exponent
  int64_t segments;  // S
  int64_t seg_chunks;  // chunks per segment (all but the last one full)
};

__device__ __forceinline__ LaneIo lane_io(const BwdKernelArgs& a, int64_t lane) {
  const int64_t b = lane / a.C;
  const int64_t c = lane - b * a.C;
  LaneIo io;
  io.k = a.k;
  io.v = a.v;
  io.g = a.gout;
  io.r = a.r;
  io.gk = a.gk;
  io.gv = a.gv;
  io.gr = a.gr;
  io.row = b * a.T * a.C + c;
  io.C = a.C;
  io.step = static_cast<int64_t>(kLc) * a.C;
  io.nfull = a.T / kLc;
  io.rest = static_cast<int>(a.T - io.nfull * kLc);
  return io;
}

__device__ __forceinline__ Lane initial_lane(const BwdKernelArgs& a, int64_t lanes, int64_t lane) {
  return a.state_in != nullptr ? lane_from_state(a.state_in[lane], a.state_in[lanes + lane],
                                                 a.state_in[2 * lanes + lane])
                               : lane_empty();
}

// Large B*C: one thread per lane, both passes over the whole sequence
// (GIVEN: the forward saved the checkpoints, pass 1 is skipped).
template <bool G, bool GIVEN>
__global__ __launch_bounds__(kBwdThreads) void wkv_backward_kernel(BwdKernelArgs a) {
  const int64_t lanes = a.B * a.C;
  const int64_t lane = static_cast<int64_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (lane >= lanes) return;
  const int64_t c = lane % a.C;
  const float wc = a.w[c], uc = a.u[c];
  const LaneIo io = lane_io(a, lane);
  const int64_t nch = io.nfull + (io.rest > 0 ? 1 : 0);

  // pass 1: forward state advance, a checkpoint in front of every chunk
  const Lane s_init = initial_lane(a, lanes, lane);
  if constexpr (!GIVEN) {
    Lane s = s_init;
    forward_chunks<true>(s, io, 0, io.nfull, wc, a.ckpt, lanes, lane);
    if (io.rest > 0) a.ckpt[io.nfull * lanes + lane] = make_float4(s.n, s.d, s.base, s.age);
  }
  // pass 2: backward over the chunks, last first
  Suffix acc = suffix_init(a.state_out, a.gstate_out, lanes, lane);
  float gw_acc = 0.0f, gu_acc = 0.0f;
  backward_chunks<G>(io, 0, nch, a.ckpt, lanes, lane, wc, uc, acc, gw_acc, gu_acc);
  initial_state_grad(s_init, a.state_in != nullptr, acc, wc, gw_acc, a.gstate_in, lanes, lane);
  a.gw_part[lane] = gw_acc;
  a.gu_part[lane] = gu_acc;
}

// Small B*C: the sequence is cut into S segments of seg_chunks chunks and
// every (segment, lane) pair is one thread, in three launches.
//   A: the forward summary of each segment from the empty state;
//   B: each segment's start state (the initial state and the summaries of the
//      segments before it, folded in order), the forward over the segment
//      storing checkpoints, and the segment's own suffix sums (its tokens'
//      contributions to P, Q, R, Rq at the position before it);
//   C: each segment's suffix sums at its end (the final state's gradient and
//      the later segments' own sums, folded from the last one down), then the
//      backward walk over the segment's chunks.
// Thread i is lane i % lanes of segment i / lanes.
constexpr int kFoldBatch = 8;  // earlier/later segment sums fetched together

__device__ __forceinline__ void seg_bounds(const BwdKernelArgs& a, const LaneIo& io, int64_t s,
                                           int64_t& j0, int64_t& j1) {
  const int64_t nch = io.nfull + (io.rest > 0 ? 1 : 0);
  j0 = s * a.seg_chunks;
  j1 = j0 + a.seg_chunks < nch ? j0 + a.seg_chunks : nch;
}

__global__ __launch_bounds__(kBwdThreads) void wkv_bwd_seg_forward_kernel(BwdKernelArgs a) {
  const int64_t lanes = a.B * a.C;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (id >= lanes * a.segments) return;
  const int64_t s = id / lanes, lane = id - s * lanes;
  const float wc = a.w[lane % a.C];
  const LaneIo io = lane_io(a, lane);
  int64_t j0, j1;
  seg_bounds(a, io, s, j0, j1);
  Lane x = lane_empty();
  forward_chunks<false>(x, io, j0, j1 < io.nfull ? j1 : io.nfull, wc, nullptr, lanes, lane);
  if (j1 > io.nfull) forward_rest(x, io, wc);
  a.seg_fwd[s * lanes + lane] = make_float4(x.n, x.d, lane_max_exp(x, wc), 0.0f);
}

template <bool G, bool GIVEN>
__global__ __launch_bounds__(kBwdThreads) void wkv_bwd_seg_sums_kernel(BwdKernelArgs a) {
  const int64_t lanes = a.B * a.C;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (id >= lanes * a.segments) return;
  const int64_t s = id / lanes, lane = id - s * lanes;
  const int64_t c = lane % a.C;
  const float wc = a.w[c], uc = a.u[c];
  const LaneIo io = lane_io(a, lane);
  int64_t j0, j1;
  seg_bounds(a, io, s, j0, j1);
  // start state: the forward's checkpoint (GIVEN), else the initial state,
  // then every earlier segment (all full)
  Lane x;
  if constexpr (GIVEN) {
    const float4 cp = a.ckpt[j0 * lanes + lane];
    x = Lane{cp.x, cp.y, cp.z, cp.w};
  } else {
    x = initial_lane(a, lanes, lane);
    const float seg_len = static_cast<float>(a.seg_chunks * kLc);
    // (summaries fetched kFoldBatch at a time so that their loads overlap;
    // the fold order is unchanged)
    int64_t sr = 0;
    for (; sr + kFoldBatch <= s; sr += kFoldBatch) {
      float4 f[kFoldBatch];
#pragma unroll
      for (int m = 0; m < kFoldBatch; ++m) f[m] = a.seg_fwd[(sr + m) * lanes + lane];
#pragma unroll
      for (int m = 0; m < kFoldBatch; ++m)
        lane_absorb(x, Seg{f[m].x, f[m].y, f[m].z, seg_len}, wc);
    }
    for (; sr < s; ++sr) {
      const float4 f = a.seg_fwd[sr * lanes + lane];
      lane_absorb(x, Seg{f.x, f.y, f.z, seg_len}, wc);
    }
  }
  // forward over the segment: checkpoints, and the segment's own suffix sums
  // at the position before it, sum over its tokens t (j = t - first) of
  // a_t e^{-j w} times (1, out_t, j, j out_t), a_t = g_t / Den_t, accumulated
  // relative to the largest exponent -M_t - j w seen so far
  float p = 0.0f, q = 0.0f, r = 0.0f, rq = 0.0f, zl = kEmpty;
  float jj = 0.0f;
  // chunks with their loads double-buffered; only a partial last chunk is
  // compiled with a test per token
  auto process = [&](const Chunk<G>& ch, int n, auto full) {
#pragma unroll
    for (int i = 0; i < kLc; ++i) {
      if (decltype(full)::value || i < n) {
        float M, rho, om;
        const float y = lane_step_rec(x, ch.k[i], ch.v[i], wc, uc, M, rho, om);
        const float xe = __builtin_fmaf(-jj, wc, -M);  // exponent of a_t e^{-j w}
        const float d = xe - zl;
        const float e = fast_exp2(__builtin_fabsf(d) * -kLog2e);
        const bool nw = d > 0.0f;
        const float fo = nw ? e : 1.0f;
        const float fn = (nw ? 1.0f : e) * wkv_grad<G>(ch, i) * rho;
        p = __builtin_fmaf(fo, p, fn);
        q = __builtin_fmaf(fo, q, fn * y);
        r = __builtin_fmaf(fo, r, fn * jj);
        rq = __builtin_fmaf(fo, rq, fn * jj * y);
        zl = nw ? xe : zl;
        jj += 1.0f;
      }
    }
  };
  auto load = [&](Chunk<G>& ch, int64_t j, int n) {
    const int64_t off = io.row + j * io.step;
    const float* rp = G ? io.r + off : io.r;
    if (n == kLc) {
      load_chunk<false, G>(ch, io.k + off, io.v + off, io.g + off, rp, io.C, kLc);
    } else {
      load_chunk<true, G>(ch, io.k + off, io.v + off, io.g + off, rp, io.C, n);
    }
  };
  auto save = [&](int64_t j) {
    if constexpr (!GIVEN) a.ckpt[j * lanes + lane] = make_float4(x.n, x.d, x.base, x.age);
  };
  // full chunks through two buffers with no branch around their loads inside
  // the loop (the last one or two after it, so none is read twice), then the
  // sequence's partial last chunk on its own
  const int64_t jf = j1 < io.nfull ? j1 : io.nfull;
  if (j0 < jf) {
    Chunk<G> A, Bf;
    load(A, j0, kLc);
    int64_t j = j0;
    for (; j + 2 < jf; j += 2) {
      load(Bf, j + 1, kLc);
      save(j);
      process(A, kLc, std::true_type{});
      load(A, j + 2, kLc);
      save(j + 1);
      process(Bf, kLc, std::true_type{});
    }
    if (j + 1 < jf) {  // two left
      load(Bf, j + 1, kLc);
      save(j);
      process(A, kLc, std::true_type{});
      save(j + 1);
      process(Bf, kLc, std::true_type{});
    } else if (j < jf) {  // one left
      save(j);
      process(A, kLc, std::true_type{});
    }
  }
  if (j1 > jf) {
    Chunk<G> last;
    load(last, jf, io.rest);
    save(jf);
    process(last, io.rest, std::false_type{});
  }
  a.seg_rev[s * lanes + lane] = make_float4(p, q, r, rq);
  a.seg_rev_z[s * lanes + lane] = zl;
}

template <bool G>
__global__ __launch_bounds__(kBwdThreads) void wkv_bwd_seg_backward_kernel(BwdKernelArgs a) {
  const int64_t lanes = a.B * a.C;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (id >= lanes * a.segments) return;
  const int64_t s = id / lanes, lane = id - s * lanes;
  const int64_t c = lane % a.C;
  const float wc = a.w[c], uc = a.u[c];
  const LaneIo io = lane_io(a, lane);
  int64_t j0, j1;
  seg_bounds(a, io, s, j0, j1);
  // suffix sums at this segment's end: the final state's gradient, then each
  // later segment X (last first): the sums decay across X's L tokens (their
  // age-weighted parts gain L times the plain ones) and X's own sums are added
  Suffix acc = suffix_init(a.state_out, a.gstate_out, lanes, lane);
  const int64_t nch = io.nfull + (io.rest > 0 ? 1 : 0);
  auto absorb_later = [&](int64_t x, const float4& X, float zx) {
    const int64_t xj0 = x * a.seg_chunks;
    const int64_t xj1 = xj0 + a.seg_chunks < nch ? xj0 + a.seg_chunks : nch;
    const float L = static_cast<float>((xj1 - xj0) * kLc - (xj1 > io.nfull && io.rest > 0
                                                                ? kLc - io.rest
                                                                : 0));
    suffix_absorb(acc, Suffix{X.x, X.y, X.z, X.w, zx, 0.0f}, L, wc);
  };
  // later segments, last first, their sums fetched kFoldBatch at a time
  int64_t x = a.segments - 1;
  for (; x - kFoldBatch >= s; x -= kFoldBatch) {
    float4 X[kFoldBatch];
    float zx[kFoldBatch];
#pragma unroll
    for (int m = 0; m < kFoldBatch; ++m) {
      X[m] = a.seg_rev[(x - m) * lanes + lane];
      zx[m] = a.seg_rev_z[(x - m) * lanes + lane];
    }
#pragma unroll
    for (int m = 0; m < kFoldBatch; ++m) absorb_later(x - m, X[m], zx[m]);
  }
  for (; x > s; --x) absorb_later(x, a.seg_rev[x * lanes + lane], a.seg_rev_z[x * lanes + lane]);
  float gw_acc = 0.0f, gu_acc = 0.0f;
  backward_chunks<G>(io, j0, j1, a.ckpt, lanes, lane, wc, uc, acc, gw_acc, gu_acc);
  if (s == 0) {
    initial_state_grad(initial_lane(a, lanes, lane), a.state_in != nullptr, acc, wc, gw_acc,
                       a.gstate_in, lanes, lane);
  }
  a.gw_part[s * lanes + lane] = gw_acc;
  a.gu_part[s * lanes + lane] = gu_acc;
}

// Small B*C with the forward's checkpoints: one pass. One workgroup owns
// kBcLC adjacent channels of one batch row and walks the sequence from its
// end in tiles of P = 2W sub-chunks of L tokens (whole checkpoint chunks);
// lane (sl, cl) of wave `wave` holds sub-chunk 2 wave + sl of channel cl.
// Per tile:
//   1. each thread loads its sub-chunk's k, v, dL/dout (and r) and the
//      checkpoint in front of it, re-runs the forward over it in registers
//      and forms the sub-chunk's own suffix sums;
//   2. the two sub-chunks of a wave combine through a lane shuffle, the wave
//      totals go through LDS; every thread folds the carry (the sums at the
//      tile's end) with the totals of the waves after its own, last first,
//      then with the later sub-chunk of its wave: the sums at its sub-chunk's
//      end;
//   3. each thread walks its sub-chunk backwards from there, writing dL/dk,
//      dL/dv; the carry moves to the tile's start.
// k, v and dL/dout are read once. The per-thread partial sums of dL/dw and
// dL/du are added per channel in a fixed order at the end.
constexpr int kBcLC = 32, kBcPS = 2;
constexpr int kBcW = 8, kBcL = 8;  // waves per workgroup, tokens per sub-chunk

template <int W, int L, bool MASKED, bool G>
__device__ __forceinline__ void bwd_tile(const ChunkL<L, G>& ch, const float4& cp, int n,
                                         int64_t t0, int64_t T, Suffix& carry,
                                         Suffix (*tot)[kBcLC], float wc, float uc,
                                         float& gw_acc, float& gu_acc, const BwdKernelArgs& a,
                                         int64_t off, bool cvalid, int wave, int sl, int cl) {
  constexpr int TL = W * kBcPS * L;
  // 1. forward from the checkpoint, own sums
  FwdRec<L> f;
  const Lane st = n > 0 ? Lane{cp.x, cp.y, cp.z, cp.w} : lane_empty();
  chunk_record<L, MASKED, G>(ch, n, st, wc, uc, f);
  const Suffix own = chunk_own_sums<L, MASKED, G>(ch, f, n, wc);
  // 2. the wave's later sub-chunk, the wave total
  Suffix later;
  later.p = __shfl_down(own.p, kBcLC, 64);
  later.q = __shfl_down(own.q, kBcLC, 64);
  later.r = __shfl_down(own.r, kBcLC, 64);
  later.rq = __shfl_down(own.rq, kBcLC, 64);
  later.zb = __shfl_down(own.zb, kBcLC, 64);
  later.za = __shfl_down(own.za, kBcLC, 64);
  // tokens of sub-chunk s of this tile (all L in a full tile)
  const int64_t tile0 = t0 - static_cast<int64_t>(wave * kBcPS + sl) * L;
  auto sub_len = [&](int s) -> float {
    if constexpr (!MASKED) {
      return static_cast<float>(L);
    } else {
      const int64_t left = T - (tile0 + static_cast<int64_t>(s) * L);
      return static_cast<float>(left <= 0 ? 0 : (left >= L ? L : left));
    }
  };
  if (sl == 0) {
    Suffix t = later;
    suffix_absorb(t, own, static_cast<float>(n), wc);
    tot[wave][cl] = t;
  }
  __syncthreads();
  Suffix mine = carry;
#pragma unroll
  for (int jj = W - 1; jj >= 0; --jj) {
    if (jj == wave) mine = carry;
    suffix_absorb(carry, tot[jj][cl], sub_len(kBcPS * jj) + sub_len(kBcPS * jj + 1), wc);
  }
  if (sl == 0) suffix_absorb(mine, later, sub_len(kBcPS * wave + 1), wc);
  static_assert(TL % kLc == 0, "tiles are whole checkpoint chunks");
  // 3. walk back over the sub-chunk
  float* grp = G ? a.gr + off : a.gr;
  chunk_walk<L, MASKED, G>(ch, f, n, mine, wc, gw_acc, gu_acc, a.gk + off, a.gv + off, grp, a.C,
                           cvalid);
}

template <int W, int L, bool G>
__global__ __launch_bounds__(64 * W) void wkv_bwd_chunk_kernel(BwdKernelArgs a,
                                                               int64_t groups_per_row) {
  static_assert(L % kLc == 0, "a sub-chunk starts at a checkpoint");
  constexpr int TL = W * kBcPS * L;  // tokens per tile
  constexpr int SUBS = W * kBcPS;
  __shared__ Suffix tot[2][W][kBcLC];
  __shared__ float red[2][SUBS][kBcLC];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int cl = lane % kBcLC;
  const int sl = lane / kBcLC;
  const int sub = wave * kBcPS + sl;

  const int64_t g = xcd_swizzle(blockIdx.x, a.B * groups_per_row);
  const int64_t b = g / groups_per_row;
  const int64_t c0 = (g - b * groups_per_row) * kBcLC + cl;
  const bool cvalid = c0 < a.C;
  const int64_t c = cvalid ? c0 : a.C - 1;  // idle tail threads mirror the last channel
  const int64_t lanes = a.B * a.C;
  const int64_t lane_id = b * a.C + c;
  const float wc = a.w[c], uc = a.u[c];
  const int64_t T = a.T, C = a.C;
  const int64_t row = b * T * C + c;
  const int64_t full = T / TL;  // tiles with every token present

  Suffix carry = suffix_init(a.state_out, a.gstate_out, lanes, lane_id);
  float gw_acc = 0.0f, gu_acc = 0.0f;
  auto first = [&](int64_t tile) { return tile * TL + static_cast<int64_t>(sub) * L; };
  auto rp = [&](int64_t o) { return G ? a.r + o : a.r; };
  auto load = [&](ChunkL<L, G>& ch, float4& cp, int64_t tile) {
    const int64_t o = row + first(tile) * C;
    load_chunk<false, G>(ch, a.k + o, a.v + o, a.gout + o, rp(o), C, L);
    cp = a.ckpt[(first(tile) / kLc) * lanes + lane_id];
  };
  int parity = 0;
  if (full * TL < T) {  // the last, partial tile comes first here
    const int64_t t0 = first(full);
    const int64_t left = T - t0;
    const int n = left <= 0 ? 0 : (left >= L ? L : static_cast<int>(left));
    ChunkL<L, G> last;
    const int64_t o = row + (n > 0 ? t0 : 0) * C;
    load_chunk<true, G>(last, a.k + o, a.v + o, a.gout + o, rp(o), C, n);
    const float4 cp = n > 0 ? a.ckpt[(t0 / kLc) * lanes + lane_id] : make_float4(0, 0, 0, 0);
    bwd_tile<W, L, true, G>(last, cp, n, t0, T, carry, tot[parity], wc, uc, gw_acc, gu_acc, a, o,
                            cvalid, wave, sl, cl);
    parity ^= 1;
  }
  // full tiles, last first; the next one's loads are issued before the
  // current one is processed, unconditionally inside the loop. Ungated, the
  // last one or two tiles are processed after the loop, so no tile is read
  // twice. Gated, those extra inlined tiles would push the kernel (256 VGPRs)
  // into 256 bytes of spills per lane and take 2.7x as long (measured on
  // MI355X, B=8 T=1024 C=768: 142.6 against 52.2 us), so the loop runs to
  // the end and its last prefetch re-reads tile 0 instead.
  ChunkL<L, G> A, Bf;
  float4 ca, cb;
  auto run = [&](ChunkL<L, G>& ch, const float4& cp, int64_t tile) {
    bwd_tile<W, L, false, G>(ch, cp, L, first(tile), T, carry, tot[parity], wc, uc, gw_acc,
                             gu_acc, a, row + first(tile) * C, cvalid, wave, sl, cl);
    parity ^= 1;
  };
  if (full > 0) load(A, ca, full - 1);
  if constexpr (G) {
    for (int64_t tile = full - 1; tile >= 0; tile -= 2) {
      load(Bf, cb, tile >= 1 ? tile - 1 : 0);
      run(A, ca, tile);
      if (tile < 1) break;
      load(A, ca, tile >= 2 ? tile - 2 : 0);
      run(Bf, cb, tile - 1);
    }
  } else {
    int64_t tile = full - 1;
    for (; tile >= 2; tile -= 2) {
      load(Bf, cb, tile - 1);
      run(A, ca, tile);
      load(A, ca, tile - 2);
      run(Bf, cb, tile - 1);
    }
    if (tile == 1) {  // two left
      load(Bf, cb, 0);
      run(A, ca, 1);
      run(Bf, cb, 0);
    } else if (tile == 0) {  // one left
      run(A, ca, 0);
    }
  }
  // carry: the sums at position -1 (every thread holds the same)
  if (sub == 0) {
    initial_state_grad(initial_lane(a, lanes, lane_id), a.state_in != nullptr, carry, wc, gw_acc,
                       cvalid ? a.gstate_in : nullptr, lanes, lane_id);
  }
  red[0][sub][cl] = gw_acc;
  red[1][sub][cl] = gu_acc;
  __syncthreads();
  if (sub == 0 && cvalid) {
    float tw = 0.0f, tu = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < SUBS; ++s2) {
      tw += red[0][s2][cl];
      tu += red[1][s2][cl];
    }
    a.gw_part[lane_id] = tw;
    a.gu_part[lane_id] = tu;
  }
}

// dL/dw and dL/du: the per-lane partial sums added over the batch. A
// workgroup owns 32 channels (128-byte row pieces); its 32 row slices each add
// the rows b = slice, slice + 32, ... in order (eight rows' loads issued
// together, rows past the end read as zero), then the slice totals are added
// in order through LDS: the result does not depend on timing.
constexpr int kRedCh = 32, kRedSlices = 32, kRedBatch = 8;

__global__ __launch_bounds__(kRedCh * kRedSlices) void wkv_grad_reduce_kernel(
    int64_t B, int64_t C, const float* __restrict__ gw_part, const float* __restrict__ gu_part,
    float* __restrict__ gw, float* __restrict__ gu) {
  __shared__ float sw[kRedSlices][kRedCh], su[kRedSlices][kRedCh];
  const int ch = threadIdx.x % kRedCh;
  const int slice = threadIdx.x / kRedCh;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kRedCh + ch;
  float aw = 0.0f, au = 0.0f;
  if (c < C) {
    for (int64_t b0 = slice; b0 < B; b0 += kRedBatch * kRedSlices) {
      float xw[kRedBatch], xu[kRedBatch];
#pragma unroll
      for (int m = 0; m < kRedBatch; ++m) {
        const int64_t b = b0 + m * kRedSlices;
        xw[m] = b < B && gw_part != nullptr ? gw_part[b * C + c] : 0.0f;
        xu[m] = b < B ? gu_part[b * C + c] : 0.0f;
      }
#pragma unroll
      for (int m = 0; m < kRedBatch; ++m) {
        aw += xw[m];
        au += xu[m];
      }
    }
  }
  sw[slice][ch] = aw;
  su[slice][ch] = au;
  __syncthreads();
  if (slice == 0 && c < C) {
    float tw = 0.0f, tu = 0.0f;
#pragma unroll
    for (int i = 0; i < kRedSlices; ++i) {
      tw += sw[i][ch];
      tu += su[i][ch];
    }
    if (gw != nullptr) gw[c] = tw;
    gu[c] = tu;
  }
}

constexpr int64_t align256(int64_t n) { return ((n + 255) / 256) * 256; }

// Segments per lane: one when B*C alone gives the GPU enough threads (2^16
// lanes: 1024 waves), otherwise enough for about 2^17 threads, each segment
// at least 32 tokens and a whole number of checkpoint chunks (measured on
// MI355X at B=8 T=1024 C=768: 22 segments of 48 tokens, 69.8 us, against
// 72.4 us for 2^18 threads and 77-95 us for 2^16 or 2^19).
struct SegPlan {
  int64_t segments, seg_chunks;
};

SegPlan seg_plan(int64_t lanes, int64_t T) {
  const int64_t nch = (T + kLc - 1) / kLc;
  SegPlan p{1, nch > 0 ? nch : 1};
  if (lanes <= 0 || lanes >= (int64_t(1) << 16) || T < 64) return p;
  int64_t want = ((int64_t(1) << 17) + lanes - 1) / lanes;
  const int64_t most = T / 32;
  if (want > most) want = most;
  if (want <= 1) return p;
  p.seg_chunks = (nch + want - 1) / want;
  p.segments = (nch + p.seg_chunks - 1) / p.seg_chunks;
  return p;
}

struct WsLayout {
  int64_t part, ckpt, seg_fwd, seg_rev, seg_rev_z, total;
};

WsLayout ws_layout(int64_t B, int64_t T, int64_t C) {
  const int64_t lanes = B * C;
  const SegPlan sp = seg_plan(lanes, T);
  const int64_t nch = (T + kLc - 1) / kLc;
  WsLayout l;
  l.part = 0;
  l.ckpt = align256(2 * 4 * sp.segments * lanes);
  l.seg_fwd = l.ckpt + align256(16 * nch * lanes);
  const int64_t seg = sp.segments > 1 ? sp.segments : 0;
  l.seg_rev = l.seg_fwd + align256(16 * seg * lanes);
  l.seg_rev_z = l.seg_rev + align256(16 * seg * lanes);
  l.total = l.seg_rev_z + align256(4 * seg * lanes);
  return l;
}

}  // namespace

int64_t backward_segments(int64_t lanes, int64_t T, int64_t* seg_chunks) {
  const SegPlan p = seg_plan(lanes, T);
  *seg_chunks = p.seg_chunks;
  return p.segments;
}

hipError_t launch_grad_reduce(int64_t rows, int64_t C, const float* gw_part, const float* gu_part,
                              float* gw, float* gu, hipStream_t st) {
  const int64_t rblocks = (C + kRedCh - 1) / kRedCh;
  if (rblocks == 0) return hipSuccess;
  if (rblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(wkv_grad_reduce_kernel, dim3(static_cast<unsigned>(rblocks)),
                     dim3(kRedCh * kRedSlices), 0, st, rows, C, gw_part, gu_part, gw, gu);
  return hipGetLastError();
}

int64_t backward_workspace_bytes(int64_t B, int64_t T, int64_t C) {
  return B * C > 0 ? ws_layout(B, T, C).total : 0;
}

hipError_t launch_backward(const BwdArgs& a, void* ws, hipStream_t st) {
  const int64_t lanes = a.B * a.C;
  const SegPlan sp = seg_plan(lanes, a.T);
  const WsLayout l = ws_layout(a.B, a.T, a.C);
  char* base = static_cast<char*>(ws);
  // the forward's checkpoints when given (read only: the kernels that write
  // checkpoints are not launched then), else the workspace's
  const bool given = a.ckpt != nullptr;
  // small B*C with the forward's checkpoints: the one-pass chunked kernel
  // (one partial-sum row per batch row) while its workgroups fill at least
  // three quarters of the CUs. It walks the whole sequence per workgroup, so
  // with fewer the segmented kernels, which split time as well, are faster.
  // Measured on MI355X, with checkpoints: B=8 T=1024 C=768 (192 workgroups)
  // 45 against 53 us, B=16 T=2048 C=1024 164 against 220, B=4 T=16384
  // C=2048 668 against 895; B=1 T=4096 C=768 (24 workgroups) 129 against 52.
  const int64_t groups = a.B * ((a.C + kBcLC - 1) / kBcLC);
  const bool one_pass = given && sp.segments > 1 && 4 * groups >= 3 * static_cast<int64_t>(a.cus);
  const int64_t rows = one_pass ? 1 : sp.segments;
  float4* ck = given ? const_cast<float4*>(reinterpret_cast<const float4*>(a.ckpt))
                     : reinterpret_cast<float4*>(base + l.ckpt);
  BwdKernelArgs k{a.B, a.T, a.C, a.w, a.u, a.k, a.v, a.gout, a.state_in, a.state_out,
                  a.gstate_out, a.r, a.gk, a.gv, a.gr, a.gstate_in,
                  ck,
                  reinterpret_cast<float*>(base + l.part),
                  reinterpret_cast<float*>(base + l.part) + rows * lanes,
                  reinterpret_cast<float4*>(base + l.seg_fwd),
                  reinterpret_cast<float4*>(base + l.seg_rev),
                  reinterpret_cast<float*>(base + l.seg_rev_z), sp.segments, sp.seg_chunks};
  if (lanes > 0) {
    const int64_t threads = lanes * sp.segments;
    const int64_t blocks = (threads + kBwdThreads - 1) / kBwdThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kBwdThreads);
    const bool gated = a.r != nullptr;
    if (one_pass) {
      const int64_t gpr = (a.C + kBcLC - 1) / kBcLC;
      const int64_t wgs = a.B * gpr;
      if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
      const dim3 cgrid(static_cast<unsigned>(wgs)), cblock(64 * kBcW);
      if (gated) {
        hipLaunchKernelGGL((wkv_bwd_chunk_kernel<kBcW, kBcL, true>), cgrid, cblock, 0, st, k, gpr);
      } else {
        hipLaunchKernelGGL((wkv_bwd_chunk_kernel<kBcW, kBcL, false>), cgrid, cblock, 0, st, k,
                           gpr);
      }
    } else if (sp.segments == 1) {
      if (gated) {
        if (given) {
          hipLaunchKernelGGL((wkv_backward_kernel<true, true>), grid, block, 0, st, k);
        } else {
          hipLaunchKernelGGL((wkv_backward_kernel<true, false>), grid, block, 0, st, k);
        }
      } else {
        if (given) {
          hipLaunchKernelGGL((wkv_backward_kernel<false, true>), grid, block, 0, st, k);
        } else {
          hipLaunchKernelGGL((wkv_backward_kernel<false, false>), grid, block, 0, st, k);
        }
      }
    } else {
      // with the forward's checkpoints every segment starts from its own: no
      // summaries to fold
      if (!given) hipLaunchKernelGGL(wkv_bwd_seg_forward_kernel, grid, block, 0, st, k);
      if (gated) {
        if (given) {
          hipLaunchKernelGGL((wkv_bwd_seg_sums_kernel<true, true>), grid, block, 0, st, k);
        } else {
          hipLaunchKernelGGL((wkv_bwd_seg_sums_kernel<true, false>), grid, block, 0, st, k);
        }
        hipLaunchKernelGGL(wkv_bwd_seg_backward_kernel<true>, grid, block, 0, st, k);
      } else {
        if (given) {
          hipLaunchKernelGGL((wkv_bwd_seg_sums_kernel<false, true>), grid, block, 0, st, k);
        } else {
          hipLaunchKernelGGL((wkv_bwd_seg_sums_kernel<false, false>), grid, block, 0, st, k);
        }
        hipLaunchKernelGGL(wkv_bwd_seg_backward_kernel<false>, grid, block, 0, st, k);
      }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rblocks = (a.C + kRedCh - 1) / kRedCh;
  if (rblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(wkv_grad_reduce_kernel, dim3(static_cast<unsigned>(rblocks)),
                     dim3(kRedCh * kRedSlices), 0, st, a.B * rows, a.C, k.gw_part,
                     k.gu_part, a.gw, a.gu);
  return hipGetLastError();
}

}  // namespace wkv
