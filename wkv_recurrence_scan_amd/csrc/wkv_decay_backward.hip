// Backward pass of the WKV operator with a per-token decay rate (fp32): the
// gradients of a loss with respect to w[b][t][c], u, k, v and the initial
// state, given dL/dout (and, optionally, dL/dstate_out).
//
// The operator is the per-token-decay form described on the page "RWKV-v6
// Architecture: Attention-Free Linear Transformers" (section "The Core
// Components of the RWKV-v6 Time-Mixing Block", item on the dynamic
// data-dependent decay) applied to the recurrence of the page "Linear
// attention without writing a CUDA kernel" (section "The recurrence"): step t
// outputs from the state as it stands plus the current token at e^(u + k_t),
// then decays the state by e^(-w_t) and adds the token at e^(k_t). Token i thus
// reaches output t > i with weight e^(k_i) W(i, t), W(i, t) = e^(-(w_{i+1} +
// ... + w_{t-1})). With a_t = g_t / Den_t and the suffix sums over later
// positions
//   P_i = sum_{t>i} a_t W(i, t),   Q_i = sum_{t>i} a_t out_t W(i, t),
// which run backwards as P_{i-1} = a_i + e^(-w_i) P_i (Q likewise), the
// quotient rule gives the constant-decay operator's dL/dv, dL/dk and dL/du
// unchanged, and for a rate, whose step separates every earlier token from
// every later output,
//   dL/dw_j = -e^(-w_j) (N_j P_j - D_j Q_j),
// with (N_j, D_j) the true sums of the state in front of step j (the initial
// state included). Derived here; the float64 oracle differentiates the
// defining sums term by term instead.
//
// Layout as in the constant-decay backward: every (segment, lane) pair is a
// thread; one segment per lane when B*C alone fills the GPU. When the forward
// saved the checkpoints, A and the checkpoint writes are skipped (B runs only
// with several segments, each starting from its first checkpoint). Launches:
//   A (several segments only): each segment's forward summary from the empty
//     state (sums, maximum exponent, total rate);
//   B: each segment's start state (the initial state, then the earlier
//     summaries in order), its checkpoints (the state in front of every
//     8-token chunk) and, with several segments, its own suffix sums at the
//     position in front of it;
//   C: the suffix sums at the segment's end (dL/dstate_out, then the later
//     segments' own sums, last first: crossing a segment decays them by its
//     total rate), then the walk back over its chunks: re-run a chunk's
//     forward from its checkpoint in registers, emit dL/dk, dL/dv and dL/dw
//     token by token, carry P and Q.
// Exponents that accumulate rates are fp64, as in the forward kernels; P and
// Q are fp32 relative to an fp64 exponent z, and every mix takes one exp2 of
// minus an absolute difference. dL/du is added over the batch and segments in
// a fixed order by the batch reduction.
#include "wkv_decay_lane.h"
#include "wkv_device.h"
#include "wkv_internal.h"

#include <type_traits>

namespace wkv {
namespace {

constexpr int kDbThreads = 256;
constexpr int kDbLc = kCkptTokens;  // tokens per checkpoint chunk

// Suffix sums P = p e^z, Q = q e^z.
struct SufD {
  float p, q;
  double z;
};

struct DdBwdKernelArgs {
  int64_t B, T, C;
  const float* w;
  const float* u;
  const float* k;
  const float* v;
  const float* gout;
  const float* state_in;
  const float* state_out;
  const float* gstate_out;
  float* gk;
  float* gv;
  float* gw;
  float* gstate_in;
  float* gu_part;   // [segments][lanes]
  LaneCk* ckpt;        // [chunks][lanes]
  float2* seg_nd;   // [segments][lanes] forward summary: sums,
  double* seg_m;    //   maximum exponent,
  double* seg_ws;   //   total rate
  float2* own_pq;   // [segments][lanes] the segment's own suffix sums,
  double* own_z;    //   their exponent
  int64_t segments, seg_chunks;
};

// The state advance of laned_step alone.
__device__ __forceinline__ void laned_advance(LaneD& s, float k, float v, float w) {
  const double kd = static_cast<double>(k);
  const double mw = s.m - static_cast<double>(w);
  const double s2 = kd - mw;  // k - (m - w)
  const float y = exp_neg_abs(s2);
  const bool tok_wins = s2 > 0.0;
  const float ga = tok_wins ? y : 1.0f;
  const float gb = tok_wins ? 1.0f : y;
  s.n = __builtin_fmaf(ga, s.n, gb * v);
  s.d = __builtin_fmaf(ga, s.d, gb);
  s.m = __builtin_fmax(kd, mw);
}

// laned_step recording the output's denominator as e^M / rho and the current
// token's share om = e^(u + k) / Den.
__device__ __forceinline__ float laned_step_rec(LaneD& s, float k, float v, float w, double ud,
                                                double& M, float& rho, float& om) {
  const double kd = static_cast<double>(k);
  const double s1 = (kd - s.m) + ud;  // (u + k) - m
  const float x = exp_neg_abs(s1);
  const bool cur_wins = s1 > 0.0;
  const float fa = cur_wins ? x : 1.0f;
  const float fb = cur_wins ? 1.0f : x;
  rho = fast_rcp(__builtin_fmaf(fa, s.d, fb));
  const float out = __builtin_fmaf(fa, s.n, fb * v) * rho;
  M = cur_wins ? kd + ud : s.m;
  om = fb * rho;
  laned_advance(s, k, v, w);
  return out;
}

// e^x of an fp64 exponent that is known not to overflow.
__device__ __forceinline__ float exp_d(double x) {
  return fast_exp2(static_cast<float>(x) * kLog2e);
}

// n tokens (at most kDbLc) of one lane from row offset o; G: dL/dout too.
template <bool G>
struct DbChunk {
  float k[kDbLc], v[kDbLc], w[kDbLc], g[G ? kDbLc : 1];
};

template <bool G, bool MASKED>
__device__ __forceinline__ void db_load(DbChunk<G>& c, const DdBwdKernelArgs& a, int64_t o,
                                        int n) {
#pragma unroll
  for (int i = 0; i < kDbLc; ++i) {
    // MASKED (a sequence's partial last chunk, n >= 1 tokens): the tokens
    // past the end re-read the last one and are replaced by zeros, so every
    // load stays unconditional (conditional loads into the array put it in
    // scratch memory)
    const bool live = !MASKED || i < n;
    const int64_t at = o + static_cast<int64_t>(live ? i : n - 1) * a.C;
    const float k = __builtin_nontemporal_load(a.k + at);
    const float v = __builtin_nontemporal_load(a.v + at);
    const float w = __builtin_nontemporal_load(a.w + at);
    c.k[i] = live ? k : 0.0f;
    c.v[i] = live ? v : 0.0f;
    c.w[i] = live ? w : 0.0f;
    if constexpr (G) {
      const float g = __builtin_nontemporal_load(a.gout + at);
      c.g[i] = live ? g : 0.0f;
    }
  }
}

struct DbThread {
  int64_t s, lane, c, row, lanes, j0, j1;
};

__device__ __forceinline__ bool db_thread(const DdBwdKernelArgs& a, DbThread& th) {
  th.lanes = a.B * a.C;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * kDbThreads + threadIdx.x;
  if (id >= th.lanes * a.segments) return false;
  th.s = id / th.lanes;
  th.lane = id - th.s * th.lanes;
  const int64_t b = th.lane / a.C;
  th.c = th.lane - b * a.C;
  th.row = b * a.T * a.C + th.c;
  const int64_t nch = (a.T + kDbLc - 1) / kDbLc;
  th.j0 = th.s * a.seg_chunks;
  th.j1 = th.j0 + a.seg_chunks < nch ? th.j0 + a.seg_chunks : nch;
  return true;
}

__device__ __forceinline__ int chunk_tokens(const DdBwdKernelArgs& a, int64_t j) {
  const int64_t left = a.T - j * kDbLc;
  return left >= kDbLc ? kDbLc : static_cast<int>(left);
}

// Calls body(chunk, j, tokens, full) for the thread's chunks j0 .. j1-1 in
// order (REV: last first). `full` is a compile-time flag: only the
// sequence's last chunk can be partial; it is loaded and processed on its own
// (first when REV), with a test per token. The full chunks run through two
// register buffers with no branch around their loads inside the loop: the
// next chunk's loads are issued before the current one is processed, so the
// compiler's counter waits stop at the chunk about to be used; the last one
// or two chunks are processed after the loop, so none is read twice.
template <bool G, bool REV, typename F>
__device__ __forceinline__ void db_walk(const DdBwdKernelArgs& a, const DbThread& th, F&& body) {
  const int64_t jf = th.j1 < a.T / kDbLc ? th.j1 : a.T / kDbLc;  // end of the full chunks
  const bool partial = th.j1 > jf;                               // chunk jf is partial
  auto partial_chunk = [&]() {
    const int nt = chunk_tokens(a, jf);
    DbChunk<G> c;
    db_load<G, true>(c, a, th.row + jf * kDbLc * a.C, nt);
    body(c, jf, nt, std::false_type{});
  };
  if (REV && partial) partial_chunk();
  const int64_t n = jf - th.j0;
  if (n > 0) {
    auto chunk = [&](int64_t q) { return REV ? jf - 1 - q : th.j0 + q; };
    auto load = [&](DbChunk<G>& c, int64_t q) {
      db_load<G, false>(c, a, th.row + chunk(q) * kDbLc * a.C, kDbLc);
    };
    DbChunk<G> A, Bf;
    load(A, 0);
    int64_t q = 0;
    for (; q + 2 < n; q += 2) {
      load(Bf, q + 1);
      body(A, chunk(q), kDbLc, std::true_type{});
      load(A, q + 2);
      body(Bf, chunk(q + 1), kDbLc, std::true_type{});
    }
    if (q + 1 < n) {  // two left
      load(Bf, q + 1);
      body(A, chunk(q), kDbLc, std::true_type{});
      body(Bf, chunk(q + 1), kDbLc, std::true_type{});
    } else if (q < n) {  // one left
      body(A, chunk(q), kDbLc, std::true_type{});
    }
  }
  if (!REV && partial) partial_chunk();
}

// A: forward summary of every segment but the last from the empty state.
__global__ __launch_bounds__(kDbThreads) void wkv_dd_bwd_seg_forward_kernel(DdBwdKernelArgs a) {
  DbThread th;
  if (!db_thread(a, th)) return;
  LaneD x = laned_empty();
  double ws = 0.0;
  db_walk<false, false>(a, th, [&](const DbChunk<false>& ch, int64_t, int n, auto full) {
#pragma unroll
    for (int i = 0; i < kDbLc; ++i) {
      if (decltype(full)::value || i < n) {
        laned_advance(x, ch.k[i], ch.v[i], ch.w[i]);
        ws += static_cast<double>(ch.w[i]);
      }
    }
  });
  const int64_t at = th.s * th.lanes + th.lane;
  a.seg_nd[at] = make_float2(x.n, x.d);
  a.seg_m[at] = x.m;
  a.seg_ws[at] = ws;
}

// B: start state, checkpoints and (OWN) the segment's own suffix sums: the sum
// over its tokens t of a_t W(first - 1, t) (1, out_t), relative to the largest
// exponent -M_t - (rates of the segment's steps before t). GIVEN: the forward
// saved the checkpoints; the segment starts from its first one and writes none.
template <bool OWN, bool GIVEN>
__global__ __launch_bounds__(kDbThreads) void wkv_dd_bwd_seg_sums_kernel(DdBwdKernelArgs a) {
  DbThread th;
  if (!db_thread(a, th)) return;
  const double ud = static_cast<double>(a.u[th.c]);
  LaneD x = laned_empty();
  if constexpr (GIVEN) {
    const LaneCk cp = a.ckpt[th.j0 * th.lanes + th.lane];
    x = LaneD{cp.n, cp.d, cp.m};
  } else {
    if (a.state_in != nullptr) {
      x = LaneD{a.state_in[th.lane], a.state_in[th.lanes + th.lane],
                static_cast<double>(a.state_in[2 * th.lanes + th.lane])};
    }
    for (int64_t sr = 0; sr < th.s; ++sr) {
      const int64_t at = sr * th.lanes + th.lane;
      const float2 nd = a.seg_nd[at];
      laned_absorb(x, SegD{nd.x, nd.y, a.seg_m[at], a.seg_ws[at]});
    }
  }
  float p = 0.0f, q = 0.0f;
  double zl = kEmptyD, cw = 0.0;
  db_walk<OWN, false>(a, th, [&](const DbChunk<OWN>& ch, int64_t j, int n, auto full) {
    if constexpr (!GIVEN) a.ckpt[j * th.lanes + th.lane] = LaneCk{x.n, x.d, x.m};
#pragma unroll
    for (int i = 0; i < kDbLc; ++i) {
      if (decltype(full)::value || i < n) {
        if constexpr (OWN) {
          double M;
          float rho, om;
          const float y = laned_step_rec(x, ch.k[i], ch.v[i], ch.w[i], ud, M, rho, om);
          const double xe = -M - cw;
          const double dd = xe - zl;
          const float e = exp_neg_abs(dd);
          const bool nw = dd > 0.0;
          const float fo = nw ? e : 1.0f;
          const float fn = (nw ? 1.0f : e) * ch.g[i] * rho;
          p = __builtin_fmaf(fo, p, fn);
          q = __builtin_fmaf(fo, q, fn * y);
          zl = nw ? xe : zl;
          cw += static_cast<double>(ch.w[i]);
        } else {
          laned_advance(x, ch.k[i], ch.v[i], ch.w[i]);
        }
      }
    }
  });
  if constexpr (OWN) {
    const int64_t at = th.s * th.lanes + th.lane;
    a.own_pq[at] = make_float2(p, q);
    a.own_z[at] = zl;
    // the segment's total rate, which the walk back needs to cross it (A,
    // which also writes it, does not run when the checkpoints are given;
    // otherwise this launch reads the earlier segments' totals and leaves them)
    if constexpr (GIVEN) a.seg_ws[at] = cw;
  }
}

// C: the suffix sums at the segment's end, then the walk back over its chunks.
__global__ __launch_bounds__(kDbThreads) void wkv_dd_bwd_seg_backward_kernel(DdBwdKernelArgs a) {
  DbThread th;
  if (!db_thread(a, th)) return;
  const double ud = static_cast<double>(a.u[th.c]);
  SufD acc{0.0f, 0.0f, kEmptyD};
  if (a.gstate_out != nullptr) {
    // dL/dN_T = g_num e^(-m_out), dL/dD_T = g_den e^(-m_out)
    acc = SufD{a.gstate_out[th.lane], -a.gstate_out[th.lanes + th.lane],
               -static_cast<double>(a.state_out[2 * th.lanes + th.lane])};
  }
  for (int64_t x = a.segments - 1; x > th.s; --x) {
    const int64_t at = x * th.lanes + th.lane;
    const double zd = acc.z - a.seg_ws[at];  // decayed across segment x
    const float2 own = a.own_pq[at];
    const double sg = a.own_z[at] - zd;
    const float e = exp_neg_abs(sg);
    const bool xw = sg > 0.0;
    const float fo = xw ? e : 1.0f;
    const float fx = xw ? 1.0f : e;
    acc.p = __builtin_fmaf(fo, acc.p, fx * own.x);
    acc.q = __builtin_fmaf(fo, acc.q, fx * own.y);
    acc.z = xw ? a.own_z[at] : zd;
  }
  float gu_acc = 0.0f;
  db_walk<true, true>(a, th, [&](const DbChunk<true>& ch, int64_t j, int n, auto full) {
    const int64_t o = th.row + j * kDbLc * a.C;
    const LaneCk cp = a.ckpt[j * th.lanes + th.lane];
    LaneD st{cp.n, cp.d, cp.m};
    float y[kDbLc], rho[kDbLc], om[kDbLc], pn[kDbLc], pd[kDbLc];
    double M[kDbLc], pm[kDbLc];
#pragma unroll
    for (int i = 0; i < kDbLc; ++i) {
      if (decltype(full)::value || i < n) {
        pn[i] = st.n;
        pd[i] = st.d;
        pm[i] = st.m;
        y[i] = laned_step_rec(st, ch.k[i], ch.v[i], ch.w[i], ud, M[i], rho[i], om[i]);
      }
    }
#pragma unroll
    for (int i = kDbLc - 1; i >= 0; --i) {
      if (decltype(full)::value || i < n) {
        // token i from the sums over t > i
        const float e_cur = ch.g[i] * om[i];
        const float ex = exp_d(static_cast<double>(ch.k[i]) + acc.z);  // e^(k_i + z)
        const float gv = __builtin_fmaf(acc.p, ex, e_cur);
        const float gk = __builtin_fmaf(ch.v[i], gv, -__builtin_fmaf(acc.q, ex, e_cur * y[i]));
        gu_acc = __builtin_fmaf(e_cur, ch.v[i] - y[i], gu_acc);
        // the rate of step i: -(N_i P_i - D_i Q_i) e^(-w_i)
        const float er = exp_d(pm[i] - static_cast<double>(ch.w[i]) + acc.z);
        const float gw = -(pn[i] * acc.p - pd[i] * acc.q) * er;
        __builtin_nontemporal_store(gk, a.gk + o + i * a.C);
        __builtin_nontemporal_store(gv, a.gv + o + i * a.C);
        __builtin_nontemporal_store(gw, a.gw + o + i * a.C);
        // token i joins: a_i = g_i rho_i e^(-M_i) against the sums decayed by w_i
        const double zd = acc.z - static_cast<double>(ch.w[i]);
        const double sg = -M[i] - zd;
        const float e = exp_neg_abs(sg);
        const bool nw = sg > 0.0;
        const float fo = nw ? e : 1.0f;
        const float ai = ch.g[i] * rho[i] * (nw ? 1.0f : e);
        acc.p = __builtin_fmaf(fo, acc.p, ai);
        acc.q = __builtin_fmaf(fo, acc.q, ai * y[i]);
        acc.z = nw ? -M[i] : zd;
      }
    }
  });
  if (th.s == 0 && a.gstate_in != nullptr) {
    float gn0 = 0.0f, gd0 = 0.0f, gm0 = 0.0f;
    if (a.state_in != nullptr) {
      const float n0 = a.state_in[th.lane], d0 = a.state_in[th.lanes + th.lane];
      const double m0 = static_cast<double>(a.state_in[2 * th.lanes + th.lane]);
      const float e0 = exp_d(m0 + acc.z);
      gn0 = acc.p * e0;
      gd0 = -acc.q * e0;
      gm0 = __builtin_fmaf(n0, gn0, d0 * gd0);
    }
    a.gstate_in[th.lane] = gn0;
    a.gstate_in[th.lanes + th.lane] = gd0;
    a.gstate_in[2 * th.lanes + th.lane] = gm0;
  }
  a.gu_part[th.s * th.lanes + th.lane] = gu_acc;
}

constexpr int64_t align256(int64_t n) { return ((n + 255) / 256) * 256; }

struct DbLayout {
  int64_t gu_part, ckpt, seg_nd, seg_m, seg_ws, own_pq, own_z, total;
};

DbLayout db_layout(int64_t B, int64_t T, int64_t C, int64_t S) {
  const int64_t lanes = B * C;
  const int64_t nch = (T + kDbLc - 1) / kDbLc;
  const int64_t s2 = S > 1 ? S : 0;
  DbLayout l;
  l.gu_part = 0;
  l.ckpt = align256(4 * S * lanes);
  l.seg_nd = l.ckpt + align256(16 * nch * lanes);
  l.seg_m = l.seg_nd + align256(8 * s2 * lanes);
  l.seg_ws = l.seg_m + align256(8 * s2 * lanes);
  l.own_pq = l.seg_ws + align256(8 * s2 * lanes);
  l.own_z = l.own_pq + align256(8 * s2 * lanes);
  l.total = l.own_z + align256(8 * s2 * lanes);
  return l;
}

}  // namespace

int64_t dd_backward_workspace_bytes(int64_t B, int64_t T, int64_t C) {
  if (B * C <= 0) return 0;
  int64_t chunks = 0;
  const int64_t S = backward_segments(B * C, T, &chunks);
  return db_layout(B, T, C, S).total;
}

hipError_t launch_dd_backward(const DdBwdArgs& a, void* ws, hipStream_t st) {
  const int64_t lanes = a.B * a.C;
  int64_t seg_chunks = 1;
  const int64_t S = backward_segments(lanes, a.T, &seg_chunks);
  const DbLayout l = db_layout(a.B, a.T, a.C, S);
  char* base = static_cast<char*>(ws);
  // the forward's checkpoints when given (read only: nothing that writes
  // checkpoints is launched then), else the workspace's
  const bool given = a.ckpt != nullptr;
  LaneCk* ck = given ? const_cast<LaneCk*>(static_cast<const LaneCk*>(a.ckpt))
                     : reinterpret_cast<LaneCk*>(base + l.ckpt);
  DdBwdKernelArgs k{a.B, a.T, a.C, a.w, a.u, a.k, a.v, a.gout, a.state_in, a.state_out,
                    a.gstate_out, a.gk, a.gv, a.gw, a.gstate_in,
                    reinterpret_cast<float*>(base + l.gu_part),
                    ck,
                    reinterpret_cast<float2*>(base + l.seg_nd),
                    reinterpret_cast<double*>(base + l.seg_m),
                    reinterpret_cast<double*>(base + l.seg_ws),
                    reinterpret_cast<float2*>(base + l.own_pq),
                    reinterpret_cast<double*>(base + l.own_z), S, seg_chunks};
  const int64_t threads = lanes * S;
  const int64_t blocks = (threads + kDbThreads - 1) / kDbThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (blocks > 0) {
    const dim3 grid(static_cast<unsigned>(blocks)), block(kDbThreads);
    if (S > 1) {
      if (given) {
        hipLaunchKernelGGL((wkv_dd_bwd_seg_sums_kernel<true, true>), grid, block, 0, st, k);
      } else {
        hipLaunchKernelGGL(wkv_dd_bwd_seg_forward_kernel, grid, block, 0, st, k);
        hipLaunchKernelGGL((wkv_dd_bwd_seg_sums_kernel<true, false>), grid, block, 0, st, k);
      }
    } else if (!given) {
      hipLaunchKernelGGL((wkv_dd_bwd_seg_sums_kernel<false, false>), grid, block, 0, st, k);
    }
    hipLaunchKernelGGL(wkv_dd_bwd_seg_backward_kernel, grid, block, 0, st, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_grad_reduce(a.B * S, a.C, nullptr, k.gu_part, nullptr, a.gu, st);
}

}  // namespace wkv
