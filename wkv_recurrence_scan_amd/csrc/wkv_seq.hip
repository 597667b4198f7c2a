// Channel-parallel sequential scan: one thread owns V adjacent channels of one
// batch row and walks all T tokens in order, carrying the (num, den, max_exp)
// state of the page "Linear attention without writing a CUDA kernel"
// (section "The recurrence") in registers.
//
// Memory: k, v and out are [B][T][C] with C fastest. At every token the 64
// lanes of a wave touch 64*V adjacent channels, so each load/store
// instruction covers one contiguous run of 64*V elements. Tokens are fetched
// in blocks of U, and the next block's loads are issued before the current
// block is computed (two register buffers, no copies), so U tokens of k and v
// per thread are always in flight behind the arithmetic.
//
// This is the path for large B*C (every lane already gives the GPU enough
// independent work); the chunked scan covers small B*C.
#include "wkv_device.h"
#include "wkv_internal.h"

#include <type_traits>

namespace wkv {
namespace {

constexpr int kSeqThreads = 256;

// U tokens of k, v and, for gated calls (G), the receptance r.
template <typename IoT, int V, int U, bool G>
struct SeqBlock {
  float k[U][V];
  float v[U][V];
  float r[G ? U : 1][V];
};

template <typename IoT, int V, int U, bool G>
__device__ __forceinline__ void seq_load(SeqBlock<IoT, V, U, G>& blk,
                                         const typename IoT::elem* __restrict__ kp,
                                         const typename IoT::elem* __restrict__ vp,
                                         const typename IoT::elem* __restrict__ rp, int64_t C) {
#pragma unroll
  for (int i = 0; i < U; ++i) {
    IoT::template load<V, true>(kp + i * C, blk.k[i]);
    IoT::template load<V, true>(vp + i * C, blk.v[i]);
    if constexpr (G) IoT::template load<V, true>(rp + i * C, blk.r[i]);
  }
}

template <typename IoT, int V, int U, bool FAST, bool G>
__device__ __forceinline__ void seq_compute(const SeqBlock<IoT, V, U, G>& blk, Lane (&s)[V],
                                            const float (&wd)[V], const float (&ub)[V],
                                            const float (&cb)[V],
                                            typename IoT::elem* __restrict__ op, int64_t C) {
#pragma unroll
  for (int i = 0; i < U; ++i) {
    float o[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      o[j] = step_sel<FAST>(s[j], blk.k[i][j], blk.v[i][j], wd[j], ub[j], cb[j]);
      if constexpr (G) o[j] *= gate(blk.r[i][j]);
    }
    IoT::template store<V, true>(op + i * C, o);
  }
}

// All T tokens of one thread's channels, in order. CK (fp32, one channel per
// thread, U = kCkptTokens): the state in front of every block of U tokens
// also goes to ckpt[block * lanes + lane] as (n, d, base, age), the
// checkpoints of the backward pass.
template <typename IoT, int V, int U, bool FAST, bool G, bool CK>
__device__ __forceinline__ void seq_walk(Lane (&s)[V], const float (&wd)[V], const float (&ub)[V],
                                         const float (&cb)[V],
                                         const typename IoT::elem* __restrict__ kp,
                                         const typename IoT::elem* __restrict__ vp,
                                         const typename IoT::elem* __restrict__ rp,
                                         typename IoT::elem* __restrict__ op, int64_t T,
                                         int64_t C, float4* __restrict__ ckpt, int64_t lanes,
                                         int64_t lane) {
  static_assert(!CK || (V == 1 && U == kCkptTokens), "checkpoint blocks are kCkptTokens tokens");
  auto save = [&](int64_t blk) {
    if constexpr (CK) ckpt[blk * lanes + lane] = make_float4(s[0].n, s[0].d, s[0].base, s[0].age);
  };
  // Two register buffers, alternating; the loads for the block after the one
  // being computed are issued first, on every path (the last full block
  // re-reads itself, a cache hit), so that the compiler's counter-based waits
  // only ever wait for the block about to be used.
  SeqBlock<IoT, V, U, G> A, Bf;
  auto at = [&](int64_t t) { return G ? rp + t * C : rp; };
  const int64_t nblk = T / U;
  if (nblk > 0) seq_load<IoT, V, U, G>(A, kp, vp, rp, C);
  for (int64_t blk = 0; blk < nblk; blk += 2) {
    const int64_t nb = (blk + 1 < nblk ? blk + 1 : nblk - 1) * U;
    seq_load<IoT, V, U, G>(Bf, kp + nb * C, vp + nb * C, at(nb), C);
    save(blk);
    seq_compute<IoT, V, U, FAST, G>(A, s, wd, ub, cb, op + blk * U * C, C);
    if (blk + 1 >= nblk) break;
    const int64_t na = (blk + 2 < nblk ? blk + 2 : nblk - 1) * U;
    seq_load<IoT, V, U, G>(A, kp + na * C, vp + na * C, at(na), C);
    save(blk + 1);
    seq_compute<IoT, V, U, FAST, G>(Bf, s, wd, ub, cb, op + (blk + 1) * U * C, C);
  }
  if (nblk * U < T) save(nblk);
  for (int64_t t = nblk * U; t < T; ++t) {
    float kk[V], vv[V], rr[V], o[V];
    IoT::template load<V, true>(kp + t * C, kk);
    IoT::template load<V, true>(vp + t * C, vv);
    if constexpr (G) IoT::template load<V, true>(rp + t * C, rr);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      o[j] = step_sel<FAST>(s[j], kk[j], vv[j], wd[j], ub[j], cb[j]);
      if constexpr (G) o[j] *= gate(rr[j]);
    }
    IoT::template store<V, true>(op + t * C, o);
  }
}

template <typename IoT, int V, int U, bool G, bool CK>
__global__ __launch_bounds__(kSeqThreads) void wkv_seq_kernel(
    int64_t B, int64_t T, int64_t C, const float* __restrict__ w, const float* __restrict__ u,
    const typename IoT::elem* __restrict__ k, const typename IoT::elem* __restrict__ v,
    const typename IoT::elem* __restrict__ rg, const float* __restrict__ state_in,
    typename IoT::elem* __restrict__ out, float* __restrict__ state_out,
    float4* __restrict__ ckpt) {
  const int64_t groups_per_row = C / V;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kSeqThreads + threadIdx.x;
  if (gid >= B * groups_per_row) return;
  const int64_t b = gid / groups_per_row;
  const int64_t c0 = (gid - b * groups_per_row) * V;
  const int64_t plane = B * C;
  const int64_t lane0 = b * C + c0;

  float wd[V], ub[V];  // decay w and bonus u of the V channels
  IoF32::load<V, false>(w + c0, wd);
  IoF32::load<V, false>(u + c0, ub);

  Lane s[V];
  if (state_in != nullptr) {
    float n[V], d[V], m[V];
    IoF32::load<V, false>(state_in + lane0, n);
    IoF32::load<V, false>(state_in + plane + lane0, d);
    IoF32::load<V, false>(state_in + 2 * plane + lane0, m);
#pragma unroll
    for (int j = 0; j < V; ++j) s[j] = lane_from_state(n[j], d[j], m[j]);
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) s[j] = lane_empty();
  }

  const int64_t row = b * T * C + c0;
  const typename IoT::elem* kp = k + row;
  const typename IoT::elem* vp = v + row;
  const typename IoT::elem* rp = G ? rg + row : nullptr;
  typename IoT::elem* op = out + row;

  float cb[V];
  bonus_ratios(wd, ub, cb);
  if (wave_fast_ok(wd, ub)) {
    seq_walk<IoT, V, U, true, G, CK>(s, wd, ub, cb, kp, vp, rp, op, T, C, ckpt, plane, lane0);
  } else {
    seq_walk<IoT, V, U, false, G, CK>(s, wd, ub, cb, kp, vp, rp, op, T, C, ckpt, plane, lane0);
  }

  if (state_out != nullptr) {
    float n[V], d[V], m[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      n[j] = s[j].n;
      d[j] = s[j].d;
      m[j] = lane_max_exp(s[j], wd[j]);
    }
    IoF32::store<V, false>(state_out + lane0, n);
    IoF32::store<V, false>(state_out + plane + lane0, d);
    IoF32::store<V, false>(state_out + 2 * plane + lane0, m);
  }
}

template <typename IoT, int V, bool G, bool CK>
hipError_t launch_seq_g(const FwdArgs& a, hipStream_t st) {
  constexpr int U = 8;
  const int64_t threads = a.B * (a.C / V);
  const int64_t blocks = (threads + kSeqThreads - 1) / kSeqThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((wkv_seq_kernel<IoT, V, U, G, CK>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kSeqThreads), 0, st, a.B, a.T, a.C, a.w, a.u,
                     static_cast<const typename IoT::elem*>(a.k),
                     static_cast<const typename IoT::elem*>(a.v),
                     static_cast<const typename IoT::elem*>(a.r), a.state_in,
                     static_cast<typename IoT::elem*>(a.out), a.state_out,
                     reinterpret_cast<float4*>(a.ckpt));
  return hipGetLastError();
}

template <typename IoT, int V>
hipError_t launch_seq_t(const FwdArgs& a, hipStream_t st) {
  if constexpr (std::is_same<IoT, IoF32>::value && V == 1) {
    if (a.ckpt != nullptr) {
      return a.r != nullptr ? launch_seq_g<IoT, V, true, true>(a, st)
                            : launch_seq_g<IoT, V, false, true>(a, st);
    }
  } else {
    if (a.ckpt != nullptr) return hipErrorInvalidValue;  // checkpoints: fp32 only
  }
  return a.r != nullptr ? launch_seq_g<IoT, V, true, false>(a, st)
                        : launch_seq_g<IoT, V, false, false>(a, st);
}

bool aligned(const void* p, int bytes) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

}  // namespace

int seq_vec_width(int io, int64_t C, const FwdArgs& a) {
  // fp32: one dword per channel; bf16: pairs of channels share a dword.
  const int cands_f32[] = {1};
  const int cands_bf16[] = {2, 1};
  const int elem = io == kBf16 ? 2 : 4;
  const int* c = io == kBf16 ? cands_bf16 : cands_f32;
  const int nc = io == kBf16 ? 2 : 1;
  for (int i = 0; i < nc; ++i) {
    const int V = c[i];
    if (C % V) continue;
    if (!aligned(a.k, V * elem) || !aligned(a.v, V * elem) || !aligned(a.out, V * elem)) continue;
    if (!aligned(a.r, V * elem)) continue;
    if (!aligned(a.w, V * 4) || !aligned(a.u, V * 4)) continue;
    if (!aligned(a.state_in, V * 4) || !aligned(a.state_out, V * 4)) continue;
    return V;
  }
  return 1;
}

hipError_t launch_seq(const FwdArgs& a, int io, int vec, hipStream_t s) {
  if (io == kF32) return launch_seq_t<IoF32, 1>(a, s);
  if (vec == 2) return launch_seq_t<IoBf16, 2>(a, s);
  return launch_seq_t<IoBf16, 1>(a, s);
}

}  // namespace wkv
