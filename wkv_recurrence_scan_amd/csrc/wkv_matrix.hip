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
// Work split. A workgroup of 4 waves owns one (batch, head) over one segment
// of the sequence: lane i of every wave holds row i of the state, and wave q
// holds its columns 16q .. 16q+15, so every wave updates 64 x 16 entries and
// forms a partial readout over its 16 columns; the four partials of each
// token meet in LDS. Token rows (k, v, lam and r: 256 bytes each) are staged
// through LDS a block of 8 tokens at a time, double-buffered, with the next
// block's global loads in flight while the current one is computed; a wave
// reads its 16 key and value entries of a token as broadcast LDS reads.
//
// Segments. With few (batch, head) pairs the sequence is cut into P segments
// so that there are enough workgroups: a first kernel runs every segment but
// the last from the zero state and stores its final state and, per row, the
// product of its decay factors; the second kernel starts each segment from
// the state in front of it -- the initial state carried through the earlier
// segments in order, S <- diag(A_p) S + S_p (the recurrence itself, one step
// per segment) -- and re-runs it with the readout. No atomics, no waits; the
// result does not depend on P beyond rounding.
#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

constexpr int kMsD = 64;                    // head size
constexpr int kMsJW = 16;                   // state columns per wave
constexpr int kMsWaves = kMsD / kMsJW;      // 4 waves per workgroup
constexpr int kMsThreads = 64 * kMsWaves;
constexpr int kMsU = 8;                     // tokens per staged block

struct MsKernelArgs {
  int64_t B, T, H;
  int64_t P, SL;          // P segments of SL tokens (the last may be shorter)
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

// One staged block of token rows.
template <bool R>
struct MsStage {
  float k[kMsU][kMsD];
  float v[kMsU][kMsD];
  float lam[kMsU][kMsD];
  float r[R ? kMsU : 1][kMsD];
};

// Thread t's share of a block: token t / TPR, channels FV (t % TPR) and the
// FV - 1 after them (TPR threads per 64-channel row).
constexpr int kMsFV = kMsU * kMsD / kMsThreads;
constexpr int kMsTPR = kMsD / kMsFV;
typedef float msvec __attribute__((ext_vector_type(kMsFV)));

template <bool R>
struct MsPrefetch {
  msvec k, v, lam, r;
};

template <bool R>
__device__ __forceinline__ void ms_fetch(MsPrefetch<R>& f, const MsKernelArgs& a, int64_t row0,
                                         int64_t t0, int64_t tend) {
  const int u = threadIdx.x / kMsTPR;
  const int c = kMsFV * (threadIdx.x % kMsTPR);
  const int64_t t = t0 + u;
  if (t < tend) {
    const int64_t off = row0 + t * a.H * kMsD + c;
    f.k = *reinterpret_cast<const msvec*>(a.k + off);
    f.v = *reinterpret_cast<const msvec*>(a.v + off);
    f.lam = *reinterpret_cast<const msvec*>(a.lam + off);
    if constexpr (R) f.r = *reinterpret_cast<const msvec*>(a.r + off);
  } else {
    f.k = f.v = f.lam = f.r = msvec{};
  }
}

template <bool R>
__device__ __forceinline__ void ms_put(MsStage<R>& s, const MsPrefetch<R>& f) {
  const int u = threadIdx.x / kMsTPR;
  const int c = kMsFV * (threadIdx.x % kMsTPR);
  *reinterpret_cast<msvec*>(&s.k[u][c]) = f.k;
  *reinterpret_cast<msvec*>(&s.v[u][c]) = f.v;
  *reinterpret_cast<msvec*>(&s.lam[u][c]) = f.lam;
  if constexpr (R) *reinterpret_cast<msvec*>(&s.r[u][c]) = f.r;
}

// The first nt tokens of a staged block (FULL: all kMsU of them, without
// guards, so the state stays in place across tokens).
template <bool READ, bool FULL>
__device__ __forceinline__ void ms_tokens(const MsStage<READ>& st, float (*part)[kMsU][kMsD],
                                          int nt, float (&S)[kMsJW], float& prod) {
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < kMsU; ++u) {
    if (FULL || u < nt) {
      const float ki = st.k[u][lane];
      const float wf = fast_exp2(st.lam[u][lane] * -kLog2e);
      prod *= wf;
      float vj[kMsJW], kj[kMsJW];
#pragma unroll
      for (int c = 0; c < kMsJW; ++c) {
        vj[c] = st.v[u][q * kMsJW + c];
        kj[c] = st.k[u][q * kMsJW + c];
      }
      float p = 0.0f;
#pragma unroll
      for (int c = 0; c < kMsJW; ++c) {
        S[c] = __builtin_fmaf(wf, S[c], ki * vj[c]);
        if constexpr (READ) p = __builtin_fmaf(S[c], kj[c], p);
      }
      if constexpr (READ) part[q][u][lane] = p;
    }
  }
}

// Walks tokens [t0, tend) of one (batch, head) from the state in S (this
// thread's row i = lane, columns 16q ..). READ: also form the gated outputs.
// Returns the product of the decay factors of row i over the walk.
template <bool READ>
__device__ __forceinline__ float ms_walk(const MsKernelArgs& a, int64_t row0, int64_t t0,
                                         int64_t tend, float (&S)[kMsJW]) {
  __shared__ MsStage<READ> stage[2];
  __shared__ float part[2][kMsWaves][kMsU][kMsD];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  const int64_t C = a.H * kMsD;
  float prod = 1.0f;
  const int64_t nblk = (tend - t0 + kMsU - 1) / kMsU;
  if (nblk <= 0) return prod;
  MsPrefetch<READ> f;
  ms_fetch<READ>(f, a, row0, t0, tend);
  ms_put<READ>(stage[0], f);
  ms_fetch<READ>(f, a, row0, t0 + kMsU, tend);
  __syncthreads();
  for (int64_t n = 0; n < nblk; ++n) {
    const MsStage<READ>& st = stage[n & 1];
    const int64_t tb = t0 + n * kMsU;
    const int nt = tend - tb < kMsU ? static_cast<int>(tend - tb) : kMsU;
    if (nt == kMsU) {
      ms_tokens<READ, true>(st, part[n & 1], nt, S, prod);
    } else {
      ms_tokens<READ, false>(st, part[n & 1], nt, S, prod);
    }
    // wave q finishes tokens q and q + 4 of the block after the barrier; it
    // takes their receptance now, since the next block's data may overwrite
    // this stage buffer before a slower wave reaches that point
    float rg[kMsU / kMsWaves];
    if constexpr (READ) {
#pragma unroll
      for (int m = 0; m < kMsU / kMsWaves; ++m) {
        const int u = q + m * kMsWaves;
        rg[m] = u < nt ? st.r[u][lane] : 0.0f;
      }
    }
    // the next block goes into the other stage buffer, whose readers (block
    // n - 1) all passed the previous barrier
    if (n + 1 < nblk) {
      ms_put<READ>(stage[(n + 1) & 1], f);
      ms_fetch<READ>(f, a, row0, tb + 2 * kMsU, tend);
    }
    __syncthreads();
    if constexpr (READ) {
#pragma unroll
      for (int m = 0; m < kMsU / kMsWaves; ++m) {
        const int u = q + m * kMsWaves;
        if (u < nt) {
          float y = 0.0f;
#pragma unroll
          for (int qq = 0; qq < kMsWaves; ++qq) y += part[n & 1][qq][u][lane];
          y *= gate(rg[m]);
          __builtin_nontemporal_store(y, a.out + row0 + (tb + u) * C + lane);
        }
      }
    }
  }
  return prod;
}

// This thread's 16 state entries of (batch, head) bh: row = lane, columns 16q ..
__device__ __forceinline__ int64_t ms_state_off(int64_t bh) {
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  return bh * kMsD * kMsD + static_cast<int64_t>(lane) * kMsD + q * kMsJW;
}

__device__ __forceinline__ void ms_load16(const float* __restrict__ p, float (&S)[kMsJW]) {
#pragma unroll
  for (int c = 0; c < kMsJW; c += 4) {
    const float4 x = *reinterpret_cast<const float4*>(p + c);
    S[c] = x.x;
    S[c + 1] = x.y;
    S[c + 2] = x.z;
    S[c + 3] = x.w;
  }
}

__device__ __forceinline__ void ms_store16(float* __restrict__ p, const float (&S)[kMsJW]) {
#pragma unroll
  for (int c = 0; c < kMsJW; c += 4)
    *reinterpret_cast<float4*>(p + c) = float4{S[c], S[c + 1], S[c + 2], S[c + 3]};
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
  float S[kMsJW];
#pragma unroll
  for (int c = 0; c < kMsJW; ++c) S[c] = 0.0f;
  const float prod = ms_walk<false>(a, row0, t0, tend, S);
  ms_store16(a.seg_state + p * nbh * kMsD * kMsD + ms_state_off(bh), S);
  if ((threadIdx.x >> 6) == 0) a.seg_decay[(p * nbh + bh) * kMsD + threadIdx.x] = prod;
}

// Segment p of (batch, head) bh: the state in front of it, then the walk with
// the gated readout; the last segment writes the final state.
__global__ __launch_bounds__(kMsThreads) void wkv6_scan_kernel(MsKernelArgs a) {
  const int64_t nbh = a.B * a.H;
  const int64_t bh = blockIdx.x % nbh;
  const int64_t p = blockIdx.x / nbh;
  const int64_t b = bh / a.H, h = bh - b * a.H;
  const int64_t row0 = b * a.T * a.H * kMsD + h * kMsD;
  const int64_t t0 = p * a.SL;
  const int64_t tend = t0 + a.SL < a.T ? t0 + a.SL : a.T;
  const int lane = threadIdx.x & 63;
  float S[kMsJW];
  if (a.state_in != nullptr) {
    ms_load16(a.state_in + ms_state_off(bh), S);
  } else {
#pragma unroll
    for (int c = 0; c < kMsJW; ++c) S[c] = 0.0f;
  }
  // carry the state through the earlier segments, oldest first
  for (int64_t pp = 0; pp < p; ++pp) {
    float L[kMsJW];
    ms_load16(a.seg_state + pp * nbh * kMsD * kMsD + ms_state_off(bh), L);
    const float A = a.seg_decay[(pp * nbh + bh) * kMsD + lane];
#pragma unroll
    for (int c = 0; c < kMsJW; ++c) S[c] = __builtin_fmaf(A, S[c], L[c]);
  }
  ms_walk<true>(a, row0, t0, tend, S);
  if (p == a.P - 1 && a.state_out != nullptr) ms_store16(a.state_out + ms_state_off(bh), S);
}

// One decode step for every (batch, head): state read and written in place.
__global__ __launch_bounds__(kMsThreads) void wkv6_step_kernel(
    int64_t H, const float* __restrict__ lam, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ r, float* __restrict__ state,
    float* __restrict__ out) {
  __shared__ float kv[2][kMsD];
  __shared__ float part[kMsWaves][kMsD];
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / H, h = bh - b * H;
  const int64_t row = b * H * kMsD + h * kMsD;  // this head's channels of batch row b
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  if (q == 0) {
    kv[0][lane] = k[row + lane];
    kv[1][lane] = v[row + lane];
  }
  float S[kMsJW];
  ms_load16(state + ms_state_off(bh), S);
  const float ki = k[row + lane];
  const float wf = fast_exp2(lam[row + lane] * -kLog2e);
  __syncthreads();
  float p = 0.0f;
#pragma unroll
  for (int c = 0; c < kMsJW; ++c) {
    S[c] = __builtin_fmaf(wf, S[c], ki * kv[1][q * kMsJW + c]);
    p = __builtin_fmaf(S[c], kv[0][q * kMsJW + c], p);
  }
  part[q][lane] = p;
  ms_store16(state + ms_state_off(bh), S);
  __syncthreads();
  if (q == 0) {
    float y = 0.0f;
#pragma unroll
    for (int qq = 0; qq < kMsWaves; ++qq) y += part[qq][lane];
    out[row + lane] = y * gate(r[row + lane]);
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

// Segments for a problem: enough workgroups to give every CU about four, but
// no segment shorter than 64 tokens.
int64_t matrix_segments(int64_t B, int64_t T, int64_t H, int cus) {
  const int64_t nbh = B * H;
  if (nbh <= 0 || T <= 0) return 1;
  const int64_t want = (4LL * cus + nbh - 1) / nbh;
  const int64_t cap = T / 64 > 1 ? T / 64 : 1;
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
  a.P = P;
  a.SL = (m.T + P - 1) / P;
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
  hipLaunchKernelGGL(wkv6_step_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kMsThreads), 0, s,
                     m.H, m.lam, m.k, m.v, m.r, m.state, m.out);
  return hipGetLastError();
}

}  // namespace wkv
