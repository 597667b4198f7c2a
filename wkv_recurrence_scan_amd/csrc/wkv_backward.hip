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
#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kLc = 8;  // tokens per checkpoint chunk

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

struct Chunk {
  float k[kLc], v[kLc], g[kLc];
};

template <bool MASKED>
__device__ __forceinline__ void load_chunk(Chunk& c, const float* __restrict__ kp,
                                           const float* __restrict__ vp,
                                           const float* __restrict__ gp, int64_t C, int n) {
#pragma unroll
  for (int i = 0; i < kLc; ++i) {
    if (!MASKED || i < n) {
      c.k[i] = __builtin_nontemporal_load(kp + i * C);
      c.v[i] = __builtin_nontemporal_load(vp + i * C);
      c.g[i] = __builtin_nontemporal_load(gp + i * C);
    } else {
      c.k[i] = 0.0f;
      c.v[i] = 0.0f;
      c.g[i] = 0.0f;
    }
  }
}

// Backward walk over one chunk of n tokens (all kLc unless MASKED) starting
// from checkpoint state st; gk, gv point at the chunk's first token.
template <bool MASKED>
__device__ __forceinline__ void chunk_backward(const Chunk& c, int n, Lane st, Suffix& a,
                                               float w, float u, float& gw_acc, float& gu_acc,
                                               float* __restrict__ gkp, float* __restrict__ gvp,
                                               int64_t C) {
  float y[kLc], M[kLc], rho[kLc], om[kLc];
#pragma unroll
  for (int i = 0; i < kLc; ++i) {
    if (!MASKED || i < n) y[i] = lane_step_rec(st, c.k[i], c.v[i], w, u, M[i], rho[i], om[i]);
  }
#pragma unroll
  for (int i = kLc - 1; i >= 0; --i) {
    if (!MASKED || i < n) {
      // gradients of token i from the suffix sums over t > i
      const float e_cur = c.g[i] * om[i];
      const float ex = fast_exp2(__builtin_fmaf(-a.za, w, c.k[i] + a.zb) * kLog2e);  // e^(k_i+z)
      const float gv = __builtin_fmaf(a.p, ex, e_cur);
      const float gk = __builtin_fmaf(c.v[i], gv, -__builtin_fmaf(a.q, ex, e_cur * y[i]));
      gu_acc = __builtin_fmaf(e_cur, c.v[i] - y[i], gu_acc);
      gw_acc = __builtin_fmaf(-ex, __builtin_fmaf(c.v[i], a.r, -a.rq), gw_acc);
      __builtin_nontemporal_store(gk, gkp + i * C);
      __builtin_nontemporal_store(gv, gvp + i * C);
      // token i joins the suffix sums: a new term g_i rho_i e^{-M_i} against
      // the old sums decayed by one step
      const float sg = __builtin_fmaf(a.za + 1.0f, w, -M[i] - a.zb);  // -M_i - (z - w)
      const float x = fast_exp2(__builtin_fabsf(sg) * -kLog2e);
      const bool new_wins = sg > 0.0f;
      const float fo = new_wins ? x : 1.0f;
      const float fn = new_wins ? 1.0f : x;
      const float ai = c.g[i] * rho[i] * fn;
      a.r = fo * (a.r + a.p);
      a.rq = fo * (a.rq + a.q);
      a.p = __builtin_fmaf(fo, a.p, ai);
      a.q = __builtin_fmaf(fo, a.q, ai * y[i]);
      a.zb = new_wins ? -M[i] : a.zb;
      a.za = new_wins ? 0.0f : a.za + 1.0f;
    }
  }
}

__global__ __launch_bounds__(kBwdThreads) void wkv_backward_kernel(
    int64_t B, int64_t T, int64_t C, const float* __restrict__ w, const float* __restrict__ u,
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ gout,
    const float* __restrict__ state_in, const float* __restrict__ state_out,
    const float* __restrict__ gstate_out, float* __restrict__ gk, float* __restrict__ gv,
    float* __restrict__ gstate_in, float4* __restrict__ ckpt, float* __restrict__ gw_part,
    float* __restrict__ gu_part) {
  const int64_t lanes = B * C;
  const int64_t lane = static_cast<int64_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (lane >= lanes) return;
  const int64_t b = lane / C;
  const int64_t c = lane - b * C;
  const float wc = w[c], uc = u[c];
  const int64_t row = b * T * C + c;
  const int64_t nfull = T / kLc;
  const int rest = static_cast<int>(T - nfull * kLc);
  const int64_t step = static_cast<int64_t>(kLc) * C;

  // pass 1: forward state advance, a checkpoint in front of every chunk
  const Lane s_init = state_in != nullptr
                          ? lane_from_state(state_in[lane], state_in[lanes + lane],
                                            state_in[2 * lanes + lane])
                          : lane_empty();
  {
    Lane s = s_init;
    // two register buffers used alternately; the next chunk's loads are
    // issued before the current chunk is consumed (the last chunk re-reads
    // itself, so the loads are unconditional and the compiler's counter
    // waits stay exact)
    float ka[kLc], va[kLc], kb[kLc], vb[kLc];
    auto load2 = [&](float (&kk)[kLc], float (&vv)[kLc], int64_t j) {
#pragma unroll
      for (int i = 0; i < kLc; ++i) {
        kk[i] = __builtin_nontemporal_load(k + row + j * step + i * C);
        vv[i] = __builtin_nontemporal_load(v + row + j * step + i * C);
      }
    };
    auto advance = [&](const float (&kk)[kLc], const float (&vv)[kLc], int64_t j) {
      ckpt[j * lanes + lane] = make_float4(s.n, s.d, s.base, s.age);
#pragma unroll
      for (int i = 0; i < kLc; ++i) lane_advance(s, kk[i], vv[i], wc);
    };
    if (nfull > 0) load2(ka, va, 0);
    for (int64_t j = 0; j < nfull; j += 2) {
      load2(kb, vb, j + 1 < nfull ? j + 1 : j);
      advance(ka, va, j);
      if (j + 1 >= nfull) break;
      load2(ka, va, j + 2 < nfull ? j + 2 : j + 1);
      advance(kb, vb, j + 1);
    }
    if (rest > 0) ckpt[nfull * lanes + lane] = make_float4(s.n, s.d, s.base, s.age);
  }

  // pass 2: backward over the chunks, last first
  Suffix a;
  if (gstate_out != nullptr) {
    // dL/dN_T = g_num e^{-m_out}: p = g_num, q = -g_den relative to z = -m_out
    a = Suffix{gstate_out[lane], -gstate_out[lanes + lane], 0.0f, 0.0f,
               -state_out[2 * lanes + lane], 0.0f};
  } else {
    a = Suffix{0.0f, 0.0f, 0.0f, 0.0f, kEmpty, 0.0f};
  }
  float gw_acc = 0.0f, gu_acc = 0.0f;
  if (rest > 0) {
    const int64_t off = row + nfull * step;
    Chunk ch;
    load_chunk<true>(ch, k + off, v + off, gout + off, C, rest);
    const float4 cp = ckpt[nfull * lanes + lane];
    chunk_backward<true>(ch, rest, Lane{cp.x, cp.y, cp.z, cp.w}, a, wc, uc, gw_acc, gu_acc,
                         gk + off, gv + off, C);
  }
  if (nfull > 0) {
    Chunk A, Bf;
    load_chunk<false>(A, k + row + (nfull - 1) * step, v + row + (nfull - 1) * step,
                      gout + row + (nfull - 1) * step, C, kLc);
    for (int64_t j = nfull - 1; j >= 0; j -= 2) {
      const int64_t jb = j - 1 >= 0 ? j - 1 : 0;
      load_chunk<false>(Bf, k + row + jb * step, v + row + jb * step, gout + row + jb * step, C,
                        kLc);
      float4 cp = ckpt[j * lanes + lane];
      chunk_backward<false>(A, kLc, Lane{cp.x, cp.y, cp.z, cp.w}, a, wc, uc, gw_acc, gu_acc,
                            gk + row + j * step, gv + row + j * step, C);
      if (j - 1 < 0) break;
      const int64_t ja = j - 2 >= 0 ? j - 2 : 0;
      load_chunk<false>(A, k + row + ja * step, v + row + ja * step, gout + row + ja * step, C,
                        kLc);
      cp = ckpt[(j - 1) * lanes + lane];
      chunk_backward<false>(Bf, kLc, Lane{cp.x, cp.y, cp.z, cp.w}, a, wc, uc, gw_acc, gu_acc,
                            gk + row + (j - 1) * step, gv + row + (j - 1) * step, C);
    }
  }

  // the initial state: e^{m0} P_{-1}, -e^{m0} Q_{-1}, and its share of dL/dw
  if (state_in != nullptr) {
    const float n0 = s_init.n, d0 = s_init.d, m0 = s_init.base;
    const float e0 = fast_exp2(__builtin_fmaf(-a.za, wc, m0 + a.zb) * kLog2e);
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
  gw_part[lane] = gw_acc;
  gu_part[lane] = gu_acc;
}

// dL/dw and dL/du: the per-lane partial sums added over the batch, in order.
__global__ __launch_bounds__(256) void wkv_grad_reduce_kernel(int64_t B, int64_t C,
                                                              const float* __restrict__ gw_part,
                                                              const float* __restrict__ gu_part,
                                                              float* __restrict__ gw,
                                                              float* __restrict__ gu) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= C) return;
  float sw = 0.0f, su = 0.0f;
  for (int64_t b = 0; b < B; ++b) {
    sw += gw_part[b * C + c];
    su += gu_part[b * C + c];
  }
  gw[c] = sw;
  gu[c] = su;
}

int64_t part_bytes(int64_t lanes) { return ((8 * lanes + 255) / 256) * 256; }

}  // namespace

int64_t backward_workspace_bytes(int64_t B, int64_t T, int64_t C) {
  const int64_t lanes = B * C;
  const int64_t chunks = (T + kLc - 1) / kLc;
  return part_bytes(lanes) + chunks * lanes * static_cast<int64_t>(sizeof(float4));
}

hipError_t launch_backward(const BwdArgs& a, void* ws, hipStream_t st) {
  const int64_t lanes = a.B * a.C;
  float* gw_part = static_cast<float*>(ws);
  float* gu_part = gw_part + lanes;
  float4* ckpt = reinterpret_cast<float4*>(static_cast<char*>(ws) + part_bytes(lanes));
  if (lanes > 0) {
    const int64_t blocks = (lanes + kBwdThreads - 1) / kBwdThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(wkv_backward_kernel, dim3(static_cast<unsigned>(blocks)),
                       dim3(kBwdThreads), 0, st, a.B, a.T, a.C, a.w, a.u, a.k, a.v, a.gout,
                       a.state_in, a.state_out, a.gstate_out, a.gk, a.gv, a.gstate_in, ckpt,
                       gw_part, gu_part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rblocks = (a.C + 255) / 256;
  if (rblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(wkv_grad_reduce_kernel, dim3(static_cast<unsigned>(rblocks)), dim3(256), 0,
                     st, a.B, a.C, gw_part, gu_part, a.gw, a.gu);
  return hipGetLastError();
}

}  // namespace wkv
