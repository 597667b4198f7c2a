// Matrix-valued-state recurrence (head size 64, fp32).
//
// The page "RWKV-v6 Architecture: Attention-Free Linear Transformers"
// (section "The Core Components of the RWKV-v6 Time-Mixing Block", item
// "Matrix-Valued Hidden State", and the step function of its PyTorch
// listing): per head of D channels a D x D state; step t scales row i by the
// decay factor of channel i, adds the outer product of key and value, and
// outputs the new state applied to the key, gated by sigmoid of the
// receptance:
//   S_t[i][j] = e^(-lam_t[i]) S_{t-1}[i][j] + k_t[i] v_t[j]
//   y_t[i]    = sigmoid(r_t[i]) * sum_j S_t[i][j] k_t[j]
//
// Layout: r, k, v, lam, y are [B][T][C] with C = H * 64 (channel h*64 + i);
// a state is [B][H][64][64], row i then column j.
//
// Chunked form. The recurrence is linear in the state, so over a chunk of
// L = 16 tokens with decay factors w_t = e^-lam_t the state moves as
//   S_end = diag(E_15) S_start + sum_s diag(P_(s,15)) k_s v_s^T
// and the outputs are
//   y_t = sigmoid(r_t) (E_t (S_start k_t) + sum_(s<=t) P_(s,t) k_s (v_s . k_t)),
// where E_t is the product of the chunk's factors up to and including token
// t and P_(s,t) the product over the tokens after s up to t (elementwise per
// row i). Three 64-deep contractions per chunk run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32): the readout S_start k_t for the 16 tokens, the
// key-value products G[s][t] = v_s . k_t, and the state update V^T K^ with
// K^[s][i] = P_(s,15)[i] k_s[i]. The remaining causal sum over s <= t is
// elementwise per row and runs on the vector units.
//
// The factors are only ever multiplied, never divided, so a huge rate sends
// the affected terms to zero and nothing overflows: the chunk is cut into
// four blocks of four tokens, P_(s,t) for s and t in different blocks is
// (product over the rest of s's block) x (whole blocks in between) x
// (product over t's block up to t), and inside a block the products are taken
// directly.
//
// Work split. A workgroup of four waves owns one (batch, head) over one
// segment of the sequence; wave w owns state rows i = 16w .. 16w+15. Lane
// (n = lane % 16, q = lane / 16) holds, in the accumulator layout of the
// matrix instruction, S[16w + n][16m + 4q + e] for m, e = 0..3, so the state
// stays in registers across chunks and feeds the readout as its B operand
// with no data movement. The readout's token rows are permuted so that lane
// q's four tokens are q, 7 - q, 8 + q and 15 - q -- one in each block, with
// the same amount of causal-sum work on every lane. Each chunk's rows of k,
// v, lam and r (256 bytes per row) are staged once through LDS by the whole
// workgroup, double-buffered, with the next chunk's global loads in flight
// while the current one is computed; the staging threads turn lam into the
// factor e^-lam and r into its gate, and also store k, v and the factors
// transposed (channel-major) for the column reads of the causal sum. Every
// wave needs all of the key-value products; each forms the part of their
// 64-deep sum over its own 16 channels and the four parts are added through
// LDS (one barrier), 36 matrix instructions per wave and chunk instead of 48
// (measured on MI355X at B=256 T=512, 12 heads: 643 against 667 us).
//
// Segments. With few (batch, head) pairs the sequence is cut into P segments
// (of a whole number of chunks) so that there are enough workgroups: a first
// kernel runs every segment but the last from the zero state (state update
// only) and stores its final state and, per row, the product of its decay
// factors; the second kernel starts each segment from the state in front of
// it -- the initial state carried through the earlier segments in order,
// S <- diag(A_p) S + S_p (the recurrence itself, one step per segment) -- and
// runs it with the readout. No atomics, no waits; the result does not depend
// on P beyond rounding.
#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kMsD = 64;                    // head size
constexpr int kMsL = 16;                    // tokens per chunk
constexpr int kMsWaves = 4;                 // wave w owns state rows 16w ..
constexpr int kMsThreads = 64 * kMsWaves;
constexpr int kMsCol = kMsL + 4;            // padded row of a channel-major tile
constexpr int kMsFold = 4;                  // earlier segments folded per batch of loads

struct MsKernelArgs {
  int64_t B, T, H;
  int64_t P, SL;          // P segments of SL tokens (a multiple of kMsL; the last may be shorter)
  const float* lam;
  const float* k;
  const float* v;
  const float* r;
  const float* state_in;  // [B][H][64][64] or nullptr (zero state)
  float* out;
  float* state_out;       // or nullptr
  float* seg_state;       // [P-1][B*H][64][64]: final state of segment p from zero
  float* seg_decay;       // [P-1][B*H][64]: product of segment p's decay factors per row
};

// One staged chunk: one row per channel i holding, for the chunk's 16
// tokens, the decay factors e^-lam, the keys decayed to the end of their
// block of four, the values and the four block products of the factors;
// READ adds the keys and the gates sigmoid(r). A row is 52 floats (84 with
// READ), i.e. 52 (20) modulo the 64 banks, so the rows of 16 neighbouring
// channels start on distinct 4-bank groups and every access pattern below is
// conflict-free.
template <bool READ>
struct MsStage {
  static constexpr int kW = 0, kKD = 16, kV = 32, kBP = 48, kK = 52, kG = 68;
  static constexpr int kLen = READ ? 84 : 52;
  alignas(16) float row[kMsD][kLen];
  __device__ __forceinline__ f4 ld4(int i, int field, int t) const {
    return *reinterpret_cast<const f4*>(&row[i][field + t]);
  }
  __device__ __forceinline__ void st4(int i, int field, int t, f4 x) {
    *reinterpret_cast<f4*>(&row[i][field + t]) = x;
  }
};

// Thread x's share of a chunk: channel x % 64, tokens 4 (x / 64) .. + 3
// (every load instruction of a wave reads one 256-byte token row).
template <bool READ>
struct MsPrefetch {
  float k[4], v[4], lam[4], r[READ ? 4 : 1];
};

template <bool READ>
__device__ __forceinline__ void ms_fetch(MsPrefetch<READ>& f, const MsKernelArgs& a, int64_t row0,
                                         int64_t t0, int64_t tend) {
  // a uniform base at the chunk's first token and 32-bit per-thread offsets
  // (16 token rows of one sequence always fit)
  const int64_t C = a.H * kMsD;
  const int64_t base = row0 + t0 * C;
  const float* __restrict__ k = a.k + base;
  const float* __restrict__ v = a.v + base;
  const float* __restrict__ lam = a.lam + base;
  const float* __restrict__ r = a.r + base;
  const uint32_t u0 = 4 * (threadIdx.x >> 6);
  const uint32_t off0 = u0 * static_cast<uint32_t>(C) + (threadIdx.x & 63);
  const int64_t left = tend - t0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t off = off0 + e * static_cast<uint32_t>(C);
    if (left >= kMsL || static_cast<int64_t>(u0 + e) < left) {
      f.k[e] = k[off];
      f.v[e] = v[off];
      f.lam[e] = lam[off];
      if constexpr (READ) f.r[e] = r[off];
    } else {
      // a token past the end leaves the state as it is: no key, no value, factor 1
      f.k[e] = f.v[e] = f.lam[e] = 0.0f;
      if constexpr (READ) f.r[e] = 0.0f;
    }
  }
}

template <bool READ>
__device__ __forceinline__ void ms_put(MsStage<READ>& s, const MsPrefetch<READ>& f) {
  using St = MsStage<READ>;
  const int c = threadIdx.x & 63;
  const int b = threadIdx.x >> 6;
  float w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = fast_exp2(f.lam[e] * -kLog2e);
  const float s3 = w[3], s2 = w[2] * s3, s1 = w[1] * s2;
  s.st4(c, St::kW, 4 * b, f4{w[0], w[1], w[2], w[3]});
  s.st4(c, St::kKD, 4 * b, f4{f.k[0] * s1, f.k[1] * s2, f.k[2] * s3, f.k[3]});
  s.st4(c, St::kV, 4 * b, f4{f.v[0], f.v[1], f.v[2], f.v[3]});
  s.row[c][St::kBP + b] = w[0] * s1;
  if constexpr (READ) {
    s.st4(c, St::kK, 4 * b, f4{f.k[0], f.k[1], f.k[2], f.k[3]});
    s.st4(c, St::kG, 4 * b, f4{gate(f.r[0]), gate(f.r[1]), gate(f.r[2]), gate(f.r[3])});
  }
}

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Token of row m of the readout's A operand: lane q's accumulator rows
// 4q .. 4q+3 then hold tokens q, 7 - q, 8 + q, 15 - q.
__device__ __forceinline__ int ms_token(int m) {
  const int b = m & 3, o = m >> 2;
  return 4 * b + ((b & 1) ? 3 - o : o);
}

// 4-way select by q (q = 0..3).
__device__ __forceinline__ float sel4(int q, float x0, float x1, float x2, float x3) {
  const float lo = (q & 1) ? x1 : x0;
  const float hi = (q & 1) ? x3 : x2;
  return (q & 2) ? hi : lo;
}

// One chunk of one (batch, head) from the state S (this lane's 16 entries of
// row 16w + n): READ also forms the gated outputs of tokens [tb, tend) into
// out (FULL: all 16 of them, without guards). Returns the product of the
// chunk's decay factors of row 16w + n.
template <bool READ, bool FULL>
__device__ __forceinline__ float ms_chunk(const MsStage<READ>& st, float (*gt)[kMsCol],
                                          f4 (*gpart)[64], const MsKernelArgs& a, int64_t orow,
                                          int64_t tb, int64_t tend, f4 (&S)[4]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, q = lane >> 4;
  const int w = threadIdx.x >> 6;
  const int i = 16 * w + n;  // this lane's state row (channel of the head)

  using St = MsStage<READ>;
  const f4 bp = st.ld4(i, St::kBP, 0);
  const float pre1 = bp[0], pre2 = pre1 * bp[1], pre3 = pre2 * bp[2];
  const float total = pre3 * bp[3];

  // the state-update operands: values transposed (A) and the keys of tokens
  // s = 4q .. 4q+3 decayed to the end of the chunk (B)
  f4 vA[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) vA[m] = st.ld4(16 * m + n, St::kV, 4 * q);
  const float tail = sel4(q, bp[1] * bp[2] * bp[3], bp[2] * bp[3], bp[3], 1.0f);
  const f4 kh = tail * st.ld4(i, St::kKD, 4 * q);

  if constexpr (READ) {
    // token-major operands: token ms_token(n) of the keys at channels
    // 16m + 4q + e, and token n of the values at this wave's channels 16w +
    // 4q + e
    f4 kA[4], vG;
    const int tn = ms_token(n);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int e = 0; e < 4; ++e) kA[m][e] = st.row[16 * m + 4 * q + e][St::kK + tn];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) vG[e] = st.row[16 * w + 4 * q + e][St::kV + n];
    // G[s][ms_token(n)] for s = 4q + e is a 64-deep sum over the head's
    // channels: each wave forms the part over its own 16 (4 instead of 16
    // matrix instructions) and the four parts meet in LDS; the readout
    // X[ms_token(4q + e)][i] runs while the parts are exchanged
    f4 g = {0.0f, 0.0f, 0.0f, 0.0f}, x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) g = mfma4(vG[e], sel4(w, kA[0][e], kA[1][e], kA[2][e], kA[3][e]), g);
    gpart[w][lane] = g;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x = mfma4(kA[m][e], S[m][e], x);
    }
    __syncthreads();
    g = gpart[0][lane];
#pragma unroll
    for (int u = 1; u < kMsWaves; ++u) g += gpart[u][lane];
    // G to this wave's LDS tile, token-major: gt[t][s]
    *reinterpret_cast<f4*>(&gt[tn][4 * q]) = g;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    float* __restrict__ out = a.out + orow + tb * a.H * kMsD;  // the chunk's first token row
    const uint32_t C32 = static_cast<uint32_t>(a.H * kMsD);
    const int rem = tend - tb < kMsL ? static_cast<int>(tend - tb) : kMsL;  // tokens of this chunk
    // lane q's token in block j is t = 4j + o: o = q for even j, 3 - q for odd j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = (j & 1) ? 3 - q : q;
      const int t = 4 * j + o;
      // earlier blocks: sum_b (whole blocks between) * sum_(s in b) kd[s] G[s][t]
      float cross = 0.0f;
#pragma unroll
      for (int b = 0; b < j; ++b) {
        const f4 gs = *reinterpret_cast<const f4*>(&gt[t][4 * b]);
        const f4 kb = st.ld4(i, St::kKD, 4 * b);
        float yb = kb[0] * gs[0];
        yb = __builtin_fmaf(kb[1], gs[1], yb);
        yb = __builtin_fmaf(kb[2], gs[2], yb);
        yb = __builtin_fmaf(kb[3], gs[3], yb);
        cross = __builtin_fmaf(bp[b], cross, yb);
      }
      // t's own block, tokens 4j .. t: direct products
      const f4 gs = *reinterpret_cast<const f4*>(&gt[t][4 * j]);
      const f4 wj = st.ld4(i, St::kW, 4 * j);
      const f4 kj = st.ld4(i, St::kK, 4 * j);
      float inb = 0.0f, pb = 1.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (e <= o) {
          inb = __builtin_fmaf(wj[e], inb, kj[e] * gs[e]);
          pb *= wj[e];
        }
      }
      const float prej = j == 0 ? 1.0f : (j == 1 ? pre1 : (j == 2 ? pre2 : pre3));
      const float acc = __builtin_fmaf(prej, x[j], cross);
      const float y = st.row[i][St::kG + t] * __builtin_fmaf(pb, acc, inb);
      if (FULL || t < rem) __builtin_nontemporal_store(y, out + (t * C32 + i));
    }
  }

  // state update: S <- diag(total) S + V^T K^
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    S[m] *= total;
#pragma unroll
    for (int e = 0; e < 4; ++e) S[m] = mfma4(vA[m][e], kh[e], S[m]);
  }
  return total;
}

// Walks chunks [t0, tend) of one (batch, head) from the state in S.
// Returns the product of the decay factors of row 16w + n over the walk.
template <bool READ>
__device__ __forceinline__ float ms_walk(const MsKernelArgs& a, int64_t row0, int64_t t0,
                                         int64_t tend, f4 (&S)[4]) {
  __shared__ MsStage<READ> stage[2];
  __shared__ float gtile[READ ? kMsWaves : 1][kMsL][kMsCol];
  __shared__ f4 gparts[READ ? kMsWaves : 1][64];  // each wave's part of the key-value products
  float prod = 1.0f;
  const int64_t nch = (tend - t0 + kMsL - 1) / kMsL;
  if (nch <= 0) return prod;
  float (*gt)[kMsCol] = gtile[READ ? (threadIdx.x >> 6) : 0];
  MsPrefetch<READ> f;
  ms_fetch<READ>(f, a, row0, t0, tend);
  ms_put<READ>(stage[0], f);
  ms_fetch<READ>(f, a, row0, t0 + kMsL, tend);
  __syncthreads();
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t tb = t0 + c * kMsL;
    if (tb + kMsL <= tend) {
      prod *= ms_chunk<READ, true>(stage[c & 1], gt, gparts, a, row0, tb, tend, S);
    } else {
      prod *= ms_chunk<READ, false>(stage[c & 1], gt, gparts, a, row0, tb, tend, S);
    }
    // the next chunk goes into the other stage buffer, whose readers (chunk
    // c - 1) all passed the previous barrier
    if (c + 1 < nch) {
      ms_put<READ>(stage[(c + 1) & 1], f);
      ms_fetch<READ>(f, a, row0, tb + 2 * kMsL, tend);
    }
    __syncthreads();
  }
  return prod;
}

// This lane's state entries of (batch, head) bh: row 16w + n, columns
// 16m + 4q .. + 3 for m = 0..3 (float4 m at offset + 16m).
__device__ __forceinline__ int64_t ms_row_off(int64_t bh) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  return bh * kMsD * kMsD + static_cast<int64_t>(16 * w + (lane & 15)) * kMsD + 4 * (lane >> 4);
}

__device__ __forceinline__ void ms_load_state(const float* __restrict__ p, f4 (&S)[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) S[m] = *reinterpret_cast<const f4*>(p + 16 * m);
}

__device__ __forceinline__ void ms_store_state(float* __restrict__ p, const f4 (&S)[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) *reinterpret_cast<f4*>(p + 16 * m) = S[m];
}

// Segment p < P - 1 of (batch, head) bh from the zero state: its final state
// and the product of its decay factors per row.
__global__ __launch_bounds__(kMsThreads) void wkv6_seg_state_kernel(MsKernelArgs a) {
  const int64_t nbh = a.B * a.H;
  const int64_t bh = blockIdx.x % nbh;
  const int64_t p = blockIdx.x / nbh;
  const int64_t b = bh / a.H, h = bh - b * a.H;
  const int64_t row0 = b * a.T * a.H * kMsD + h * kMsD;
  const int64_t t0 = p * a.SL;
  const int64_t tend = t0 + a.SL < a.T ? t0 + a.SL : a.T;
  f4 S[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) S[m] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  const float prod = ms_walk<false>(a, row0, t0, tend, S);
  ms_store_state(a.seg_state + p * nbh * kMsD * kMsD + ms_row_off(bh), S);
  if ((threadIdx.x & 63) < 16)
    a.seg_decay[(p * nbh + bh) * kMsD + 16 * (threadIdx.x >> 6) + (threadIdx.x & 15)] = prod;
}

// Segment p of (batch, head) bh: the state in front of it, then the walk with
// the gated readout; the last segment writes the final state.
__global__ __launch_bounds__(kMsThreads, 3) void wkv6_scan_kernel(MsKernelArgs a) {
  const int64_t nbh = a.B * a.H;
  const int64_t bh = blockIdx.x % nbh;
  const int64_t p = blockIdx.x / nbh;
  const int64_t b = bh / a.H, h = bh - b * a.H;
  const int64_t row0 = b * a.T * a.H * kMsD + h * kMsD;
  const int64_t t0 = p * a.SL;
  const int64_t tend = t0 + a.SL < a.T ? t0 + a.SL : a.T;
  const int i = 16 * (threadIdx.x >> 6) + (threadIdx.x & 15);
  f4 S[4];
  if (a.state_in != nullptr) {
    ms_load_state(a.state_in + ms_row_off(bh), S);
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) S[m] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // carry the state through the earlier segments, oldest first; the loads of
  // kMsFold segments are issued together so that their latencies overlap
  for (int64_t p0 = 0; p0 < p; p0 += kMsFold) {
    f4 L[kMsFold][4];
    float A[kMsFold];
#pragma unroll
    for (int u = 0; u < kMsFold; ++u) {
      if (p0 + u < p) {
        ms_load_state(a.seg_state + (p0 + u) * nbh * kMsD * kMsD + ms_row_off(bh), L[u]);
        A[u] = a.seg_decay[((p0 + u) * nbh + bh) * kMsD + i];
      }
    }
#pragma unroll
    for (int u = 0; u < kMsFold; ++u) {
      if (p0 + u < p) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int e = 0; e < 4; ++e) S[m][e] = __builtin_fmaf(A[u], S[m][e], L[u][m][e]);
        }
      }
    }
  }
  ms_walk<true>(a, row0, t0, tend, S);
  if (p == a.P - 1 && a.state_out != nullptr) ms_store_state(a.state_out + ms_row_off(bh), S);
}

// One decode step for every (batch, head), the state read and written in
// place: a workgroup of 256 threads per (batch, head). Thread x owns the
// state's 16-byte pieces 256c + x (c = 0..3) in flat row-major order -- row
// i = 16c + x / 16, columns j = 4 (x % 16) .. + 3 -- so every load and store
// instruction of a wave covers 1 KiB of contiguous state; a row's readout
// sum_j S[i][j] k_j is reduced over the 16 lanes that hold it.
__global__ __launch_bounds__(256) void wkv6_step_kernel(
    int64_t H, const float* __restrict__ lam, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ r, float* __restrict__ state,
    float* __restrict__ out) {
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / H, h = bh - b * H;
  const int64_t row = b * H * kMsD + h * kMsD;  // this head's channels of batch row b
  const int x = threadIdx.x;
  const int j0 = 4 * (x & 15);
  float* __restrict__ S = state + bh * kMsD * kMsD;
  f4 st[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) st[c] = *reinterpret_cast<const f4*>(S + 4 * (256 * c + x));
  // every load is issued before the first use: columns' k, v, rows' k, rate, r
  float kj[4], vj[4], ki[4], li[4], ri[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kj[e] = k[row + j0 + e];
    vj[e] = v[row + j0 + e];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = 16 * c + (x >> 4);
    ki[c] = k[row + i];
    li[c] = lam[row + i];
    ri[c] = r[row + i];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float wf = fast_exp2(li[c] * -kLog2e);
    float p = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      st[c][e] = __builtin_fmaf(wf, st[c][e], ki[c] * vj[e]);
      p = __builtin_fmaf(st[c][e], kj[e], p);
    }
    *reinterpret_cast<f4*>(S + 4 * (256 * c + x)) = st[c];
    // butterfly: all 16 lanes of the row end with the full sum and store the
    // same value (no branch, so nothing is deferred behind one)
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) p += __shfl_xor(p, m, 16);
    out[row + 16 * c + (x >> 4)] = p * gate(ri[c]);
  }
}

// T == 0: state_out <- state_in, or zeros.
__global__ __launch_bounds__(256) void wkv6_state_copy_kernel(int64_t n, const float* __restrict__ src,
                                                              float* __restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = src != nullptr ? src[i] : 0.0f;
}

}  // namespace

hipError_t launch_matrix_state_copy(int64_t B, int64_t H, const float* src, float* dst,
                                    hipStream_t s) {
  const int64_t n = B * H * kMsD * kMsD;
  const int64_t blocks = (n + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(wkv6_state_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     n, src, dst);
  return hipGetLastError();
}

#ifndef WKV_MS_WG_PER_CU
#define WKV_MS_WG_PER_CU 3
#endif
#ifndef WKV_MS_MIN_SEG
#define WKV_MS_MIN_SEG 64
#endif

// Segments for a problem: enough workgroups to give every CU about
// WKV_MS_WG_PER_CU, but no segment shorter than WKV_MS_MIN_SEG tokens.
int64_t matrix_segments(int64_t B, int64_t T, int64_t H, int cus) {
  const int64_t nbh = B * H;
  if (nbh <= 0 || T <= 0) return 1;
  const int64_t want = (static_cast<int64_t>(WKV_MS_WG_PER_CU) * cus + nbh - 1) / nbh;
  const int64_t cap = T / WKV_MS_MIN_SEG > 1 ? T / WKV_MS_MIN_SEG : 1;
  const int64_t P = want < cap ? want : cap;
  return P > 1 ? P : 1;
}

int64_t matrix_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t P) {
  if (P <= 1) return 0;
  const int64_t nbh = B * H;
  const int64_t st = (P - 1) * nbh * kMsD * kMsD * 4;
  const int64_t dec = (P - 1) * nbh * kMsD * 4;
  return ((st + 255) / 256) * 256 + ((dec + 255) / 256) * 256;
}

hipError_t launch_matrix(const MatrixArgs& m, int64_t P, void* ws, hipStream_t s) {
  MsKernelArgs a{};
  a.B = m.B;
  a.T = m.T;
  a.H = m.H;
  // whole chunks per segment; rounding up may leave fewer segments than the
  // workspace was sized for
  a.SL = ((m.T + P - 1) / P + kMsL - 1) / kMsL * kMsL;
  if (a.SL <= 0) a.SL = kMsL;
  P = (m.T + a.SL - 1) / a.SL;
  if (P < 1) P = 1;
  a.P = P;
  a.lam = m.lam;
  a.k = m.k;
  a.v = m.v;
  a.r = m.r;
  a.state_in = m.state_in;
  a.out = m.out;
  a.state_out = m.state_out;
  const int64_t nbh = m.B * m.H;
  if (P > 1) {
    const int64_t st = (P - 1) * nbh * kMsD * kMsD * 4;
    a.seg_state = static_cast<float*>(ws);
    a.seg_decay = reinterpret_cast<float*>(static_cast<char*>(ws) + ((st + 255) / 256) * 256);
    const int64_t blocks1 = (P - 1) * nbh;
    if (blocks1 > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(wkv6_seg_state_kernel, dim3(static_cast<unsigned>(blocks1)),
                       dim3(kMsThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = P * nbh;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(wkv6_scan_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kMsThreads), 0,
                     s, a);
  return hipGetLastError();
}

hipError_t launch_matrix_step(const MatrixStepArgs& m, hipStream_t s) {
  const int64_t blocks = m.B * m.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(wkv6_step_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     m.H, m.lam, m.k, m.v, m.r, m.state, m.out);
  return hipGetLastError();
}

}  // namespace wkv
