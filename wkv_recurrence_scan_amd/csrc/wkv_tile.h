// Tile-level building blocks shared by the two time-parallel prefill kernels
// (the chunked scan and the look-back scan): XCD-aware work placement, the
// sub-chunk summary, lane shuffles of summaries and the register tile loader.
#pragma once

#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

constexpr int kNumXcd = 8;

// Block index -> work index such that consecutive work indices land on the
// same XCD when blocks are dealt to XCDs round-robin. A bijection on [0, n).
__device__ __forceinline__ int64_t xcd_swizzle(int64_t bid, int64_t n) {
  const int64_t q = n / kNumXcd, r = n % kNumXcd;
  const int64_t xcd = bid % kNumXcd, slot = bid / kNumXcd;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

__device__ __forceinline__ Seg shfl_up_seg(const Seg& x, int delta) {
  Seg r;
  r.n = __shfl_up(x.n, delta, 64);
  r.d = __shfl_up(x.d, delta, 64);
  r.m = __shfl_up(x.m, delta, 64);
  r.len = __shfl_up(x.len, delta, 64);
  return r;
}

// Summary of one sub-chunk: its own state from empty, maximum taken at the
// end of the sub-chunk. MASKED: only the first nvalid tokens exist.
// The maximum `top` is found on the rounded exponents k_i - (last - i) w, but
// each weight's exponent is then formed against it as (k_i - top) - (last - i) w:
// the key difference is exact for keys near the maximum, so the sums are exact
// relative to the stored `top`, however coarse the keys' own grid (at |k| = 1e4
// rounding k_i - (last - i) w first would move every weight by up to ulp(1e4)).
template <int L, bool MASKED>
__device__ __forceinline__ Seg summarize(const float (&kk)[L], const float (&vv)[L], float wd,
                                         int nvalid) {
  float top = kEmpty;
  const float last = MASKED ? static_cast<float>(nvalid - 1) : static_cast<float>(L - 1);
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (!MASKED || i < nvalid)
      top = __builtin_fmaxf(top, __builtin_fmaf(static_cast<float>(i) - last, wd, kk[i]));
  }
  float n = 0.0f, d = 0.0f;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    float e = fast_exp2(__builtin_fmaf(static_cast<float>(i) - last, wd, kk[i] - top) * kLog2e);
    if (MASKED && i >= nvalid) e = 0.0f;
    d += e;
    n = __builtin_fmaf(e, vv[i], n);
  }
  return Seg{n, d, top, MASKED ? static_cast<float>(nvalid) : static_cast<float>(L)};
}

// One thread's tokens of a tile: k, v and, for gated calls (G), the
// receptance r.
template <int V, int L, bool G = false>
struct ChunkRegs {
  float k[L][V];
  float v[L][V];
  float r[G ? L : 1][V];
};

// rp is read only when G. The loads are non-temporal: a tile is read once
// (measured on MI355X: B=8 T=1024 C=768 22.9 against 23.5 us per layer,
// B=4 T=16384 C=2048 look-back 315 against 337 us).
template <typename IoT, int V, int L, bool MASKED, bool G>
__device__ __forceinline__ void chunk_load(ChunkRegs<V, L, G>& r,
                                           const typename IoT::elem* __restrict__ kp,
                                           const typename IoT::elem* __restrict__ vp,
                                           const typename IoT::elem* __restrict__ rp, int64_t C,
                                           int nvalid) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (!MASKED || i < nvalid) {
      IoT::template load<V, true>(kp + i * C, r.k[i]);
      IoT::template load<V, true>(vp + i * C, r.v[i]);
      if constexpr (G) IoT::template load<V, true>(rp + i * C, r.r[i]);
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        r.k[i][j] = 0.0f;
        r.v[i][j] = 0.0f;
        if constexpr (G) r.r[i][j] = 0.0f;
      }
    }
  }
}

// The scan of one tile held in registers, W waves of 2 x 32 lanes: lane
// (sl, cl) of wave `wave` holds sub-chunk wave*PS + sl of channel group cl.
// Returns per thread the segments before its sub-chunk inside its wave (exc),
// the totals of the waves before its own (before) and the whole tile
// (whole). tot is LDS scratch of W x CH segments. In two halves around one
// workgroup barrier, which the caller places (tile_scan does both): the first
// summarises, scans inside the wave and posts the wave's total; the second
// reads the totals of all W waves.
template <int V, int LC, int PS, int L, bool MASKED, bool G>
__device__ __forceinline__ void tile_scan_post(const ChunkRegs<V, L, G>& r, const float (&wd)[V],
                                               int nvalid, Seg (*tot)[LC * V], int wave,
                                               Seg (&exc)[V]) {
  const int lane = threadIdx.x & 63;
  const int cl = lane % LC;
  const int sl = lane / LC;
  Seg inc[V];
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
}

template <int V, int LC, int W>
__device__ __forceinline__ void tile_scan_totals(const float (&wd)[V], Seg (*tot)[LC * V], int wave,
                                                 Seg (&before)[V], Seg (&whole)[V]) {
  const int cl = (threadIdx.x & 63) % LC;
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
}

template <int V, int LC, int PS, int W, int L, bool MASKED, bool G>
__device__ __forceinline__ void tile_scan(const ChunkRegs<V, L, G>& r, const float (&wd)[V], int nvalid,
                                          Seg (*tot)[LC * V], Seg (&exc)[V], Seg (&before)[V],
                                          Seg (&whole)[V]) {
  const int wave = threadIdx.x >> 6;
  tile_scan_post<V, LC, PS, L, MASKED, G>(r, wd, nvalid, tot, wave, exc);
  __syncthreads();
  tile_scan_totals<V, LC, W>(wd, tot, wave, before, whole);
}

// Where a prefill saves the backward pass's checkpoints (fp32, one channel
// per thread): the lane state in front of every token whose index is a
// multiple of kCkptTokens goes to p[(token / kCkptTokens) * lanes + lane] as
// (n, d, base, age); tok0 is the index of the thread's first token here.
struct CkOut {
  float4* p;
  int64_t lanes, lane, tok0;
};

// Re-runs the recurrence over one thread's sub-chunk from the state in front
// of it and writes the outputs (gated by sigmoid(r) when G). FAST selects
// lane_step_fast; CK also saves checkpoints (see CkOut).
template <typename IoT, int V, int L, bool MASKED, bool FAST, bool G, bool CK = false>
__device__ __forceinline__ void rescan(Lane (&pre)[V], const ChunkRegs<V, L, G>& r,
                                       const float (&wd)[V], const float (&ub)[V],
                                       const float (&cb)[V], int nvalid, bool cvalid,
                                       typename IoT::elem* __restrict__ op, int64_t C,
                                       const CkOut& ck = CkOut{}) {
  static_assert(!CK || V == 1, "checkpoints are saved by one-channel threads");
#pragma unroll
  for (int i = 0; i < L; ++i) {
    // a guard, not a break, so that the loop stays fully unrolled and the
    // register arrays keep static indices
    if (!MASKED || i < nvalid) {
      if constexpr (CK) {
        const int64_t t = ck.tok0 + i;
        if (cvalid && (t % kCkptTokens) == 0)
          ck.p[(t / kCkptTokens) * ck.lanes + ck.lane] =
              make_float4(pre[0].n, pre[0].d, pre[0].base, pre[0].age);
      }
      float o[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        o[j] = step_sel<FAST>(pre[j], r.k[i][j], r.v[i][j], wd[j], ub[j], cb[j]);
        if constexpr (G) o[j] *= gate(r.r[i][j]);
      }
      if (cvalid) IoT::template store<V, true>(op + i * C, o);
    }
  }
}

// Two re-runs side by side, token i of tile a then token i of tile b: the
// two recurrences are independent, so their latency chains overlap. Tile a
// is complete; tile b has nvalid_b tokens when MASKED_B (its missing tokens
// were loaded as zeros and are stepped over without being stored: the state
// they leave is not used).
template <typename IoT, int V, int L, bool MASKED_B, bool FAST, bool G, bool CK = false>
__device__ __forceinline__ void rescan2(Lane (&pa)[V], const ChunkRegs<V, L, G>& ra,
                                        typename IoT::elem* __restrict__ opa, const CkOut& cka,
                                        Lane (&pb)[V], const ChunkRegs<V, L, G>& rb, int nvalid_b,
                                        typename IoT::elem* __restrict__ opb, const CkOut& ckb,
                                        const float (&wd)[V], const float (&ub)[V],
                                        const float (&cb)[V], bool cvalid, int64_t C) {
  static_assert(!CK || V == 1, "checkpoints are saved by one-channel threads");
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool bvalid = !MASKED_B || i < nvalid_b;
    if constexpr (CK) {
      const int64_t ta = cka.tok0 + i, tb = ckb.tok0 + i;
      if (cvalid && (ta % kCkptTokens) == 0)
        cka.p[(ta / kCkptTokens) * cka.lanes + cka.lane] =
            make_float4(pa[0].n, pa[0].d, pa[0].base, pa[0].age);
      if (cvalid && bvalid && (tb % kCkptTokens) == 0)
        ckb.p[(tb / kCkptTokens) * ckb.lanes + ckb.lane] =
            make_float4(pb[0].n, pb[0].d, pb[0].base, pb[0].age);
    }
    float oa[V], ob[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      oa[j] = step_sel<FAST>(pa[j], ra.k[i][j], ra.v[i][j], wd[j], ub[j], cb[j]);
      ob[j] = step_sel<FAST>(pb[j], rb.k[i][j], rb.v[i][j], wd[j], ub[j], cb[j]);
      if constexpr (G) {
        oa[j] *= gate(ra.r[i][j]);
        ob[j] *= gate(rb.r[i][j]);
      }
    }
    if (cvalid) IoT::template store<V, true>(opa + i * C, oa);
    if (cvalid && bvalid) IoT::template store<V, true>(opb + i * C, ob);
  }
}

template <typename IoT, int V, int L, bool MASKED, bool G, bool CK = false>
__device__ __forceinline__ void rescan_sel(bool fast, Lane (&pre)[V], const ChunkRegs<V, L, G>& r,
                                           const float (&wd)[V], const float (&ub)[V],
                                           const float (&cb)[V], int nvalid, bool cvalid,
                                           typename IoT::elem* __restrict__ op, int64_t C,
                                           const CkOut& ck = CkOut{}) {
  if (fast) {
    rescan<IoT, V, L, MASKED, true, G, CK>(pre, r, wd, ub, cb, nvalid, cvalid, op, C, ck);
  } else {
    rescan<IoT, V, L, MASKED, false, G, CK>(pre, r, wd, ub, cb, nvalid, cvalid, op, C, ck);
  }
}

}  // namespace
}  // namespace wkv
