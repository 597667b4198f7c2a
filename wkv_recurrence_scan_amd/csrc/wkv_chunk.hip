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

template <typename IoT, int V, int LC, int PS, int W, int L, bool G, bool CK, int PD>
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
  // Software pipeline over PD + 1 register buffers: the loads of the next PD
  // tiles are issued before the current one is processed. Inside the loop
  // every load is a real one and unconditional, so the compiler's
  // counter-based waits stop at the current tile's loads instead of draining
  // the prefetch; the last tiles are processed after it, so no tile is read
  // twice.
  static_assert(PD == 1 || PD == 2, "prefetch distance one or two tiles");
  ChunkRegs<V, L, G> A, Bf, Cr;  // Cr: the third buffer (PD == 2)
  auto at = [&](const typename IoT::elem* p, int64_t t) { return G ? p + t * step : p; };
  auto load = [&](ChunkRegs<V, L, G>& r, int64_t t) {
    chunk_load<IoT, V, L, false, G>(r, kp + t * step, vp + t * step, at(rp, t), C, L);
  };
  if (full > 0) load(A, 0);
  if constexpr (PD == 2) {
    if (full > 1) load(Bf, 1);
  }
  // what needs w, u and the initial state is worked out once the first
  // tile's loads are in flight (each of these waits for its loads)
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
  auto tile_of = [&](const ChunkRegs<V, L, G>& r, int64_t t) {
    chunk_tile<IoT, V, LC, PS, W, L, false, G, CK>(r, L, carry, wd, ub, cb, fast, tot[t & 1],
                                                   op + t * step, C, cvalid, wave, sl, cl,
                                                   ck_at(t));
  };
  int64_t tile = 0;
  if constexpr (PD == 1) {
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
  } else {
    // A holds tile `tile` and Bf tile + 1 (both in flight) at the top
    for (; tile + 4 < full; tile += 3) {
      load(Cr, tile + 2);
      tile_of(A, tile);
      load(A, tile + 3);
      tile_of(Bf, tile + 1);
      load(Bf, tile + 4);
      tile_of(Cr, tile + 2);
    }
    const int64_t left = full - tile;  // at most four, the first two loaded
    if (left >= 3) load(Cr, tile + 2);
    if (left >= 1) tile_of(A, tile);
    if (left == 4) load(A, tile + 3);
    if (left >= 2) tile_of(Bf, tile + 1);
    if (left >= 3) tile_of(Cr, tile + 2);
    if (left == 4) tile_of(A, tile + 3);
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

// ------------------------------------------------ two walkers per workgroup
//
// The kernel above walks a workgroup's tiles one after another, so its time
// is the sum of their latency chains (load wait, summary, scans, re-run).
// With at most four tiles per sequence the workgroup is split into two
// walkers of kSplitW waves, each loading both of its tiles at once: walker 0
// walks the first half of the tiles from the initial state as above; walker
// 1 summarises and scans the second half meanwhile. Walker 0 knows its final
// state as soon as its last tile is scanned, hands it to walker 1 through LDS
// and re-runs that tile while walker 1 re-runs its two tiles from it, side by
// side. Every tile is still read from HBM once, and the folds are the
// one-walker kernel's, in the same order, so both kernels give the same bits.
// Measured on MI355X at B=8 T=1024 C=768 fp32: 21.7-22.1 us per launch
// against 22.6; a per-workgroup trace shows the launch's loads arriving 3 to
// 9 us after the start and the last stores leaving at about 15 us, so what
// is left is the memory system's time for the loads and stores, not the
// chain of tiles.
constexpr int kSplitW = 8, kSplitL = 16, kSplitMaxTiles = 4;
constexpr int64_t kSplitTile = int64_t{kSplitW} * kPS * kSplitL;

template <typename IoT, int V, int L, bool G, bool CK>
__global__ __launch_bounds__(128 * kSplitW) void wkv_chunk_split_kernel(
    int64_t B, int64_t T, int64_t C, const float* __restrict__ w, const float* __restrict__ u,
    const typename IoT::elem* __restrict__ k, const typename IoT::elem* __restrict__ v,
    const typename IoT::elem* __restrict__ rg, const float* __restrict__ state_in,
    typename IoT::elem* __restrict__ out, float* __restrict__ state_out,
    int64_t groups_per_row, float4* __restrict__ ckpt) {
  constexpr int W = kSplitW, LC = kLC, PS = kPS;
  constexpr int CH = LC * V;      // channels per workgroup
  constexpr int TL = W * PS * L;  // tokens per tile
  __shared__ Seg tot[2][2][W][CH];  // [walker][tile slot]
  __shared__ Lane hand[CH];         // walker 0's final state, for walker 1

  const int tid = threadIdx.x;
  const int walker = tid / (64 * W);
  const int wave = (tid >> 6) % W;  // inside the walker
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

  float wd[V], ub[V];
  IoF32::load<V, false>(w + cc, wd);
  IoF32::load<V, false>(u + cc, ub);

  // tiles: walker 0 takes the first ceil(n / 2), walker 1 the rest (the
  // launcher guarantees 1 <= n <= kSplitMaxTiles)
  const int64_t n = (T + TL - 1) / TL;
  const int64_t n0 = (n + 1) / 2;
  const int64_t t0 = walker == 0 ? 0 : n0;
  const int cnt = static_cast<int>(walker == 0 ? n0 : n - n0);

  const int64_t base = b * T * C + cc + static_cast<int64_t>(sub) * L * C;
  const typename IoT::elem* kp = k + base;
  const typename IoT::elem* vp = v + base;
  const typename IoT::elem* rp = G ? rg + base : nullptr;
  typename IoT::elem* op = out + base;
  const int64_t step = static_cast<int64_t>(TL) * C;
  auto at = [&](const typename IoT::elem* p, int64_t t) { return G ? p + t * step : p; };
  auto full = [&](int64_t t) { return (t + 1) * TL <= T; };
  auto nvalid_of = [&](int64_t t) {
    const int64_t left = T - (t * TL + static_cast<int64_t>(sub) * L);
    return left <= 0 ? 0 : (left >= L ? L : static_cast<int>(left));
  };
  auto ck_at = [&](int64_t t) {
    return CkOut{ckpt, plane, lane0, t * TL + static_cast<int64_t>(sub) * L};
  };

  // A walker loads both of its tiles at once: walker 0 at the start, walker 1
  // after the first barrier (see below), so that walker 0's tiles are not
  // queued behind its.
  ChunkRegs<V, L, G> R[2];
  auto load_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t t = t0 + i;
      if (i < cnt) {
        if (full(t)) {
          chunk_load<IoT, V, L, false, G>(R[i], kp + t * step, vp + t * step, at(rp, t), C, L);
        } else {
          chunk_load<IoT, V, L, true, G>(R[i], kp + t * step, vp + t * step, at(rp, t), C,
                                         nvalid_of(t));
        }
      }
    }
  };
  load_tiles();

  // (what needs w, u and the initial state waits for their loads: after
  // the tiles' loads are issued)
  float cb[V];
  bonus_ratios(wd, ub, cb);
  const bool fast = wave_fast_ok(wd, ub);
  Lane carry[V];
  if (state_in != nullptr) {
    float nn[V], d[V], m[V];
    IoF32::load<V, false>(state_in + lane0, nn);
    IoF32::load<V, false>(state_in + plane + lane0, d);
    IoF32::load<V, false>(state_in + 2 * plane + lane0, m);
#pragma unroll
    for (int j = 0; j < V; ++j) carry[j] = lane_from_state(nn[j], d[j], m[j]);
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) carry[j] = lane_empty();
  }

  // The state in front of this thread's sub-chunk of a scanned tile: the
  // carry absorbs the tile's wave totals one by one (taken when its own wave
  // comes up), then the sub-chunks before it in its wave; the carry moves past
  // the tile. The same folds in the same order as the one-walker kernel, so
  // both give the same bits.
  auto enter = [&](Lane (&pre)[V], Seg (*totals)[CH], const Seg (&exc)[V]) {
#pragma unroll
    for (int jj = 0; jj < W; ++jj) {
      if (jj == wave) {
#pragma unroll
        for (int j = 0; j < V; ++j) pre[j] = carry[j];
      }
#pragma unroll
      for (int j = 0; j < V; ++j) lane_absorb(carry[j], totals[jj][cl * V + j], wd[j]);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) lane_absorb(pre[j], exc[j], wd[j]);
  };
  auto rerun = [&](Lane (&pre)[V], const ChunkRegs<V, L, G>& r, int64_t t) {
    if (full(t)) {
      rescan_sel<IoT, V, L, false, G, CK>(fast, pre, r, wd, ub, cb, L, cvalid, op + t * step, C,
                                          ck_at(t));
    } else {
      rescan_sel<IoT, V, L, true, G, CK>(fast, pre, r, wd, ub, cb, nvalid_of(t), cvalid,
                                         op + t * step, C, ck_at(t));
    }
  };

  // Three barriers. Walker 1 runs one barrier behind walker 0, so that walker
  // 0 never waits for walker 1's data:
  //   barrier 1: walker 0's first tile scanned (walker 1 posts nothing);
  //   barrier 2: walker 0's second tile (after re-running its first) and
  //              walker 1's first tile scanned;
  //   barrier 3: walker 1's second tile scanned; walker 0 has handed over its
  //              final state, worked out from its last tile's scan.
  // Then walker 0 re-runs its last tile and walker 1 its tiles, from the
  // state handed over, side by side. A tile's wave totals stay in LDS
  // (tot[walker][slot]) until the end.
  Seg exc[2][V];
  Lane pre_last[V];
  auto post = [&](int i) {
    const int64_t t = t0 + i;
    if (full(t)) {
      tile_scan_post<V, LC, PS, L, false, G>(R[i], wd, L, tot[walker][i], wave, exc[i]);
    } else {
      tile_scan_post<V, LC, PS, L, true, G>(R[i], wd, nvalid_of(t), tot[walker][i], wave,
                                            exc[i]);
    }
  };
  // walker 0's slot i is scanned: re-run it now unless it is its last, whose
  // state goes to walker 1 first
  auto w0_after = [&](int i) {
    if (i + 1 < cnt) {
      Lane pre[V];
      enter(pre, tot[0][i], exc[i]);
      rerun(pre, R[i], t0 + i);
    } else {
      enter(pre_last, tot[0][i], exc[i]);
      if (sub == 0) {
#pragma unroll
        for (int j = 0; j < V; ++j) hand[cl * V + j] = carry[j];
      }
    }
  };
  if (walker == 0) post(0);  // walker 0 always has a tile
  __syncthreads();
  if (walker == 0) {
    w0_after(0);
    if (cnt > 1) post(1);
  } else if (cnt > 0) {
    post(0);
  }
  __syncthreads();
  if (walker == 0) {
    if (cnt > 1) w0_after(1);
  } else if (cnt > 1) {
    post(1);
  }
  __syncthreads();
  if (walker == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i + 1 == cnt) rerun(pre_last, R[i], t0 + i);
    }
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) carry[j] = hand[cl * V + j];
    if (cnt == 2) {
      // both states first (each tile's carry-in comes from the scans), then
      // the two re-runs side by side; only the second tile can be partial
      Lane pa[V], pb[V];
      enter(pa, tot[1][0], exc[0]);
      enter(pb, tot[1][1], exc[1]);
      const int64_t ta = t0, tb = t0 + 1;
      auto both = [&](auto fast_c, auto masked_c) {
        rescan2<IoT, V, L, decltype(masked_c)::value, decltype(fast_c)::value, G, CK>(
            pa, R[0], op + ta * step, ck_at(ta), pb, R[1], nvalid_of(tb), op + tb * step,
            ck_at(tb), wd, ub, cb, cvalid, C);
      };
      const std::true_type yes{};
      const std::false_type no{};
      if (full(tb)) {
        if (fast) both(yes, no); else both(no, no);
      } else {
        if (fast) both(yes, yes); else both(no, yes);
      }
    } else if (cnt == 1) {
      Lane pre[V];
      enter(pre, tot[1][0], exc[0]);
      rerun(pre, R[0], t0);
    }
    // walker 1 ends with the final state (walker 0's when it has no tile)
    if (state_out != nullptr && sub == 0 && cvalid) {
      float nn[V], d[V], m[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        nn[j] = carry[j].n;
        d[j] = carry[j].d;
        m[j] = lane_max_exp(carry[j], wd[j]);
      }
      IoF32::store<V, false>(state_out + lane0, nn);
      IoF32::store<V, false>(state_out + plane + lane0, d);
      IoF32::store<V, false>(state_out + 2 * plane + lane0, m);
    }
  }
}


// Workgroup shape by sequence length (measured on MI355X): short sequences
// want the fewest serial tiles (B=8 T=1024 C=768: 8 waves of 16 tokens, 24.6
// us, against 25.7-27.2 for 8 x 8, 4 x 16, 16 x 8 and 4 x 32); long ones
// smaller tiles (B=4 T=16384 C=2048: 8 x 8, 346 us, against 370-402 for
// 16 x 8, 8 x 16, 4 x 16 and 4 x 32).
template <typename IoT, int V, int W, int L, bool G, bool CK, int PD>
hipError_t launch_chunk_g(const FwdArgs& a, hipStream_t st) {
  constexpr int CH = kLC * V;
  const int64_t gpr = (a.C + CH - 1) / CH;
  const int64_t blocks = a.B * gpr;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((wkv_chunk_kernel<IoT, V, kLC, kPS, W, L, G, CK, PD>),
                     dim3(static_cast<unsigned>(blocks)), dim3(64 * W), 0, st, a.B, a.T, a.C,
                     a.w, a.u, static_cast<const typename IoT::elem*>(a.k),
                     static_cast<const typename IoT::elem*>(a.v),
                     static_cast<const typename IoT::elem*>(a.r), a.state_in,
                     static_cast<typename IoT::elem*>(a.out), a.state_out, gpr,
                     reinterpret_cast<float4*>(a.ckpt));
  return hipGetLastError();
}

// PD: prefetch distance of ungated calls (gated ones keep one tile: a third
// buffer of k, v and r would cost a workgroup per CU)
template <typename IoT, int V, int W, int L, int PD = 1>
hipError_t launch_chunk_t(const FwdArgs& a, hipStream_t st) {
  if constexpr (std::is_same<IoT, IoF32>::value && V == 1) {
    if (a.ckpt != nullptr) {
      return a.r != nullptr ? launch_chunk_g<IoT, V, W, L, true, true, 1>(a, st)
                            : launch_chunk_g<IoT, V, W, L, false, true, PD>(a, st);
    }
  } else {
    if (a.ckpt != nullptr) return hipErrorInvalidValue;  // checkpoints: fp32 only
  }
  return a.r != nullptr ? launch_chunk_g<IoT, V, W, L, true, false, 1>(a, st)
                        : launch_chunk_g<IoT, V, W, L, false, false, PD>(a, st);
}

template <typename IoT, int V, bool G, bool CK>
hipError_t launch_chunk_split_g(const FwdArgs& a, hipStream_t st) {
  constexpr int CH = kLC * V;
  const int64_t gpr = (a.C + CH - 1) / CH;
  const int64_t blocks = a.B * gpr;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((wkv_chunk_split_kernel<IoT, V, kSplitL, G, CK>),
                     dim3(static_cast<unsigned>(blocks)), dim3(128 * kSplitW), 0, st, a.B, a.T,
                     a.C, a.w, a.u, static_cast<const typename IoT::elem*>(a.k),
                     static_cast<const typename IoT::elem*>(a.v),
                     static_cast<const typename IoT::elem*>(a.r), a.state_in,
                     static_cast<typename IoT::elem*>(a.out), a.state_out, gpr,
                     reinterpret_cast<float4*>(a.ckpt));
  return hipGetLastError();
}

constexpr int64_t kShortT = 256, kLongT = 2048;

template <typename IoT, int V>
hipError_t launch_chunk_v(const FwdArgs& a, int cus, hipStream_t st) {
  if constexpr (std::is_same<IoT, IoF32>::value && V == 1) {
    // ungated fp32 sequences of two to four 256-token tiles whose workgroups
    // each get a CU of their own: two walkers per workgroup (measured on
    // MI355X: B=8 T=1024 C=768, 192 workgroups, 22.0 against 22.6 us; with
    // more workgroups than CUs the one-walker kernel's two workgroups per CU
    // win, B=256 T=512 C=768 223 against 265 us). The gated form would not
    // fit its two tiles of k, v and r in the 128 registers a 1024-thread
    // workgroup allows.
    const int64_t blocks = a.B * ((a.C + kLC * V - 1) / (kLC * V));
    if (a.T > kShortT && a.T <= kSplitMaxTiles * kSplitTile && a.r == nullptr &&
        blocks <= cus) {
      return a.ckpt != nullptr ? launch_chunk_split_g<IoT, V, false, true>(a, st)
                               : launch_chunk_split_g<IoT, V, false, false>(a, st);
    }
  }
  if (a.T <= kShortT) return launch_chunk_t<IoT, V, 8, 4>(a, st);
  if (a.T <= kLongT) {
    // gated fp32 holds r as well: 8 tokens per thread (105 VGPRs) beat 16
    // (155) on MI355X, B=8 T=1024 C=768 26.1 against 27.1 us per layer
    const bool gated_f32 = std::is_same<IoT, IoF32>::value && a.r != nullptr;
    return gated_f32 ? launch_chunk_t<IoT, V, 8, 8>(a, st) : launch_chunk_t<IoT, V, 8, 16>(a, st);
  }
  // long sequences walk many tiles, one after another: with one channel per
  // thread the loads run two tiles ahead (84 -> 103 VGPRs, still two 8-wave
  // workgroups per CU; two channels per thread would drop to one)
  return launch_chunk_t<IoT, V, 8, 8, V == 1 ? 2 : 1>(a, st);
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

hipError_t launch_chunk(const FwdArgs& a, int io, int vec, int cus, hipStream_t s) {
  if (io == kF32) return launch_chunk_v<IoF32, 1>(a, cus, s);
  // Two bf16 channels per thread halve the workgroups (a workgroup walks the
  // whole sequence of its channels); while that leaves CUs idle, one channel
  // per thread is faster (measured on MI355X, bf16: B=8 T=1024 C=768 18.3
  // against 25.9 us, B=4 T=2048 C=2048 38.1 against 50.8; with as many
  // two-channel workgroups as CUs, B=16 T=1024 C=1024, two: 30.6 against
  // 37.8).
  const int64_t two_ch_blocks = a.B * ((a.C + 2 * kLC - 1) / (2 * kLC));
  if (vec == 2 && two_ch_blocks >= cus) return launch_chunk_v<IoBf16, 2>(a, cus, s);
  return launch_chunk_v<IoBf16, 1>(a, cus, s);
}

}  // namespace wkv
