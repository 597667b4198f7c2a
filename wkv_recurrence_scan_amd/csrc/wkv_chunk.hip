// Chunked associative scan over time, for problems whose B*C alone cannot
// fill the GPU.
//
// The pages describe the time-parallel form of RWKV as an associative prefix
// scan (page "RWKV-v6 Architecture: Attention-Free Linear Transformers",
// section on architectural duality; page "RWKV: Merging Transformer Training
// with RNN Speed", paragraph on the time-parallel mode). For this operator the
// scan element is a segment summary (num, den, max_exp, length): the state a
// run of tokens produces from the empty state. Two adjacent segments combine
// by decaying the earlier one by the later one's length and adding.
//
// One workgroup owns LC*V adjacent channels of one batch row for the whole
// sequence. Time is cut into tiles of P = W*PS sub-chunks of L tokens; thread
// (sub-chunk s, channel group cl) holds its L tokens of k and v in registers.
// Per tile:
//   1. each thread summarises its sub-chunk (exact maximum first, then one
//      exp2 per token);
//   2. the PS sub-chunks inside a wave are scanned with lane shuffles;
//   3. each wave's total goes through LDS; every thread folds the carry from
//      the previous tile with the totals of the waves before its own, then
//      with its in-wave exclusive prefix: that is the state in front of its
//      sub-chunk;
//   4. each thread re-runs the recurrence over its registers from that state
//      and writes the outputs. k and v are read from HBM once.
// The carry across tiles keeps its maximum index-tracked (exact integer age),
// so long sequences do not accumulate rounding in the running maximum.
//
// Wave layout: lane = cl + LC*sl, so one load instruction reads PS rows of
// LC*V contiguous channels. Workgroups for neighbouring channel groups are
// placed on the same XCD (blocks are dealt round-robin over the 8 XCDs), so
// lines shared by two groups (bf16 tails, odd C) are fetched through one L2.
#include "wkv_device.h"
#include "wkv_internal.h"
#include "wkv_tile.h"

#include <type_traits>

namespace wkv {
namespace {

template <typename IoT, int V, int LC, int PS, int W, int L, bool MASKED, bool G, bool CK>
__device__ __forceinline__ void chunk_tile(const ChunkRegs<V, L, G>& r, int nvalid, Lane (&carry)[V],
                                           const float (&wd)[V], const float (&ub)[V],
                                           const float (&cb)[V], bool fast, Seg (*tot)[LC * V],
                                           typename IoT::elem* __restrict__ op, int64_t C,
                                           bool cvalid, int wave, int sl, int cl,
                                           const CkOut& ck) {
  // 1. own summary, 2. inclusive scan over the wave's sub-chunks
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
  Seg exc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const Seg p = shfl_up_seg(inc[j], LC);
    exc[j] = sl > 0 ? p : seg_identity();
  }
  // 3. wave totals through LDS, fold carry -> prefix of this wave -> own prefix
  if (sl == PS - 1) {
#pragma unroll
    for (int j = 0; j < V; ++j) tot[wave][cl * V + j] = inc[j];
  }
  __syncthreads();
  Lane pre[V];
#pragma unroll
  for (int jj = 0; jj < W; ++jj) {
    if (jj == wave) {
#pragma unroll
      for (int j = 0; j < V; ++j) pre[j] = carry[j];
    }
#pragma unroll
    for (int j = 0; j < V; ++j) lane_absorb(carry[j], tot[jj][cl * V + j], wd[j]);
  }
#pragma unroll
  for (int j = 0; j < V; ++j) lane_absorb(pre[j], exc[j], wd[j]);
  // 4. rescan own tokens from the prefix
  rescan_sel<IoT, V, L, MASKED, G, CK>(fast, pre, r, wd, ub, cb, nvalid, cvalid, op, C, ck);
}

template <typename IoT, int V, int LC, int PS, int W, int L, bool G, bool CK>
__global__ __launch_bounds__(64 * W) void wkv_chunk_kernel(
    int64_t B, int64_t T, int64_t C, const float* __restrict__ w, const float* __restrict__ u,
    const typename IoT::elem* __restrict__ k, const typename IoT::elem* __restrict__ v,
    const typename IoT::elem* __restrict__ rg, const float* __restrict__ state_in,
    typename IoT::elem* __restrict__ out, float* __restrict__ state_out,
    int64_t groups_per_row, float4* __restrict__ ckpt) {
  static_assert(LC * PS == 64, "a wave is LC channel groups by PS sub-chunks");
  constexpr int CH = LC * V;          // channels per workgroup
  constexpr int TL = W * PS * L;      // tokens per tile
  __shared__ Seg tot[2][W][CH];

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

  float wd[V], ub[V];  // decay w and bonus u of the V channels
  IoF32::load<V, false>(w + cc, wd);
  IoF32::load<V, false>(u + cc, ub);
  float cb[V];
  bonus_ratios(wd, ub, cb);
  const bool fast = wave_fast_ok(wd, ub);
  Lane carry[V];
  if (state_in != nullptr) {
    float n[V], d[V], m[V];
    IoF32::load<V, false>(state_in + lane0, n);
    IoF32::load<V, false>(state_in + plane + lane0, d);
    IoF32::load<V, false>(state_in + 2 * plane + lane0, m);
#pragma unroll
    for (int j = 0; j < V; ++j) carry[j] = lane_from_state(n[j], d[j], m[j]);
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) carry[j] = lane_empty();
  }

  const int64_t base = b * T * C + cc + static_cast<int64_t>(sub) * L * C;
  const typename IoT::elem* kp = k + base;
  const typename IoT::elem* vp = v + base;
  const typename IoT::elem* rp = G ? rg + base : nullptr;
  typename IoT::elem* op = out + base;
  const int64_t step = static_cast<int64_t>(TL) * C;
  // checkpoints (CK): this thread's first token of a tile
  auto ck_at = [&](int64_t tile) {
    return CkOut{ckpt, plane, lane0, tile * TL + static_cast<int64_t>(sub) * L};
  };

  const int64_t full = T / TL;  // tiles with every token present
  // Software pipeline over two register buffers: the loads of the next tile
  // are issued before the current one is processed. Inside the loop every
  // load is a real one and unconditional, so the compiler's counter-based
  // waits stop at the current tile's loads instead of draining the prefetch;
  // the last one or two tiles are processed after it (two: both loaded up
  // front), so no tile is read twice.
  ChunkRegs<V, L, G> A, Bf;
  auto at = [&](const typename IoT::elem* p, int64_t t) { return G ? p + t * step : p; };
  auto load = [&](ChunkRegs<V, L, G>& r, int64_t t) {
    chunk_load<IoT, V, L, false, G>(r, kp + t * step, vp + t * step, at(rp, t), C, L);
  };
  auto tile_of = [&](const ChunkRegs<V, L, G>& r, int64_t t) {
    chunk_tile<IoT, V, LC, PS, W, L, false, G, CK>(r, L, carry, wd, ub, cb, fast, tot[t & 1],
                                                   op + t * step, C, cvalid, wave, sl, cl,
                                                   ck_at(t));
  };
  if (full > 0) load(A, 0);
  int64_t tile = 0;
  for (; tile + 2 < full; tile += 2) {
    load(Bf, tile + 1);
    tile_of(A, tile);
    load(A, tile + 2);
    tile_of(Bf, tile + 1);
  }
  if (tile + 1 < full) {  // two left
    load(Bf, tile + 1);
    tile_of(A, tile);
    tile_of(Bf, tile + 1);
  } else if (tile < full) {  // one left
    tile_of(A, tile);
  }
  if (full * TL < T) {  // last, partial tile
    const int64_t first = full * TL + static_cast<int64_t>(sub) * L;
    const int64_t left = T - first;
    const int nvalid = left <= 0 ? 0 : (left >= L ? L : static_cast<int>(left));
    ChunkRegs<V, L, G> last;
    chunk_load<IoT, V, L, true, G>(last, kp + full * step, vp + full * step, at(rp, full), C,
                                   nvalid);
    chunk_tile<IoT, V, LC, PS, W, L, true, G, CK>(last, nvalid, carry, wd, ub, cb, fast,
                                                  tot[full & 1], op + full * step, C, cvalid,
                                                  wave, sl, cl, ck_at(full));
  }

  if (state_out != nullptr && sub == 0 && cvalid) {
    float n[V], d[V], m[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      n[j] = carry[j].n;
      d[j] = carry[j].d;
      m[j] = lane_max_exp(carry[j], wd[j]);
    }
    IoF32::store<V, false>(state_out + lane0, n);
    IoF32::store<V, false>(state_out + plane + lane0, d);
    IoF32::store<V, false>(state_out + 2 * plane + lane0, m);
  }
}

// Channel threads per wave: 32 lanes x 4 bytes = one 128-byte line per row
// (fp32), so a load instruction reads whole lines from two rows.
constexpr int kLC = 32, kPS = 2;

// Workgroup shape by sequence length (measured on MI355X): short sequences
// want the fewest serial tiles (B=8 T=1024 C=768: 8 waves of 16 tokens, 24.6
// us, against 25.7-27.2 for 8 x 8, 4 x 16, 16 x 8 and 4 x 32); long ones
// smaller tiles (B=4 T=16384 C=2048: 8 x 8, 346 us, against 370-402 for
// 16 x 8, 8 x 16, 4 x 16 and 4 x 32).
template <typename IoT, int V, int W, int L, bool G, bool CK>
hipError_t launch_chunk_g(const FwdArgs& a, hipStream_t st) {
  constexpr int CH = kLC * V;
  const int64_t gpr = (a.C + CH - 1) / CH;
  const int64_t blocks = a.B * gpr;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((wkv_chunk_kernel<IoT, V, kLC, kPS, W, L, G, CK>),
                     dim3(static_cast<unsigned>(blocks)), dim3(64 * W), 0, st, a.B, a.T, a.C,
                     a.w, a.u, static_cast<const typename IoT::elem*>(a.k),
                     static_cast<const typename IoT::elem*>(a.v),
                     static_cast<const typename IoT::elem*>(a.r), a.state_in,
                     static_cast<typename IoT::elem*>(a.out), a.state_out, gpr,
                     reinterpret_cast<float4*>(a.ckpt));
  return hipGetLastError();
}

template <typename IoT, int V, int W, int L>
hipError_t launch_chunk_t(const FwdArgs& a, hipStream_t st) {
  if constexpr (std::is_same<IoT, IoF32>::value && V == 1) {
    if (a.ckpt != nullptr) {
      return a.r != nullptr ? launch_chunk_g<IoT, V, W, L, true, true>(a, st)
                            : launch_chunk_g<IoT, V, W, L, false, true>(a, st);
    }
  } else {
    if (a.ckpt != nullptr) return hipErrorInvalidValue;  // checkpoints: fp32 only
  }
  return a.r != nullptr ? launch_chunk_g<IoT, V, W, L, true, false>(a, st)
                        : launch_chunk_g<IoT, V, W, L, false, false>(a, st);
}

constexpr int64_t kShortT = 256, kLongT = 2048;

template <typename IoT, int V>
hipError_t launch_chunk_v(const FwdArgs& a, hipStream_t st) {
  if (a.T <= kShortT) return launch_chunk_t<IoT, V, 8, 4>(a, st);
  if (a.T <= kLongT) return launch_chunk_t<IoT, V, 8, 16>(a, st);
  return launch_chunk_t<IoT, V, 8, 8>(a, st);
}

bool aligned(const void* p, int bytes) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

}  // namespace

int chunk_vec_width(int io, int64_t C, const FwdArgs& a) {
  if (io != kBf16) return 1;
  const bool ok = C % 2 == 0 && aligned(a.k, 4) && aligned(a.v, 4) && aligned(a.out, 4) &&
                  aligned(a.r, 4) && aligned(a.w, 8) && aligned(a.u, 8) &&
                  aligned(a.state_in, 8) && aligned(a.state_out, 8);
  return ok ? 2 : 1;
}

hipError_t launch_chunk(const FwdArgs& a, int io, int vec, hipStream_t s) {
  if (io == kF32) return launch_chunk_v<IoF32, 1>(a, s);
  if (vec == 2) return launch_chunk_v<IoBf16, 2>(a, s);
  return launch_chunk_v<IoBf16, 1>(a, s);
}

}  // namespace wkv
