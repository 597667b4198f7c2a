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
  // Two register buffers, alternating: the loads of the block after the one
  // being computed are issued first. Inside the loop every load is a real,
  // unconditional one, so that the compiler's counter-based waits only ever
  // wait for the block about to be used; the last one or two blocks are
  // computed after it (two: both loaded up front), so no block is read twice.
  SeqBlock<IoT, V, U, G> A, Bf;
  auto at = [&](int64_t t) { return G ? rp + t * C : rp; };
  auto load = [&](SeqBlock<IoT, V, U, G>& x, int64_t blk) {
    const int64_t t = blk * U;
    seq_load<IoT, V, U, G>(x, kp + t * C, vp + t * C, at(t), C);
  };
  const int64_t nblk = T / U;
  if (nblk > 0) load(A, 0);
  int64_t blk = 0;
  for (; blk + 2 < nblk; blk += 2) {
    load(Bf, blk + 1);
    save(blk);
    seq_compute<IoT, V, U, FAST, G>(A, s, wd, ub, cb, op + blk * U * C, C);
    load(A, blk + 2);
    save(blk + 1);
    seq_compute<IoT, V, U, FAST, G>(Bf, s, wd, ub, cb, op + (blk + 1) * U * C, C);
  }
  if (blk + 1 < nblk) {  // two left
    load(Bf, blk + 1);
    save(blk);
    seq_compute<IoT, V, U, FAST, G>(A, s, wd, ub, cb, op + blk * U * C, C);
    save(blk + 1);
    seq_compute<IoT, V, U, FAST, G>(Bf, s, wd, ub, cb, op + (blk + 1) * U * C, C);
  } else if (blk < nblk) {  // one left
    save(blk);
    seq_compute<IoT, V, U, FAST, G>(A, s, wd, ub, cb, op + blk * U * C, C);
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

// ------------------------------------------- bf16: tiles staged through LDS
//
// For bf16 the lane-per-channel walk above reads one dword (two channels) per
// lane and token, so every load instruction of a wave covers 256 bytes of one
// row. Here a workgroup of 256 threads owns a 1 KiB piece of a row (512
// channels, two per thread) and streams it in tiles of kTileTok tokens: each
// tile of k, v (and r) is fetched with 16-byte loads (a whole 1 KiB row per
// wave instruction) into LDS, each thread walks its two channels through the
// tile from LDS, and the outputs go back through LDS to 16-byte stores. The
// next tile is in flight (in registers) while the current one is computed;
// one barrier per tile. Measured on MI355X at B=64 T=4096 C=4096: 0.74 of the
// HBM roofline against 0.68 for the lane-per-channel walk.
constexpr int kTileThreads = 256, kTileV = 2, kTileTok = 8;
constexpr int kTileCh = kTileThreads * kTileV;         // 512 channels
constexpr int kTileRowVec = kTileCh * 2 / 16;          // 16-byte words per row piece
constexpr int kTileVec = kTileTok * kTileRowVec;       // per tile and tensor
constexpr int kTileNv = kTileVec / kTileThreads;       // per thread
static_assert(kTileNv * kTileThreads == kTileVec, "a tile splits evenly over the threads");

template <bool FAST, bool G>
__device__ __forceinline__ void tile_walk(const u32x4* kb, const u32x4* vb, const u32x4* rb,
                                          u32x4* ob, int nrows, Lane (&s)[kTileV],
                                          const float (&wd)[kTileV], const float (&ub)[kTileV],
                                          const float (&cb)[kTileV]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int r = 0; r < kTileTok; ++r) {
    if (r < nrows) {
      float kk[kTileV], vv[kTileV], rr[kTileV], o[kTileV];
      const int at = r * kTileCh + tid * kTileV;
      IoBf16::load<kTileV, false>(reinterpret_cast<const uint16_t*>(kb) + at, kk);
      IoBf16::load<kTileV, false>(reinterpret_cast<const uint16_t*>(vb) + at, vv);
      if constexpr (G) IoBf16::load<kTileV, false>(reinterpret_cast<const uint16_t*>(rb) + at, rr);
#pragma unroll
      for (int j = 0; j < kTileV; ++j) {
        o[j] = step_sel<FAST>(s[j], kk[j], vv[j], wd[j], ub[j], cb[j]);
        if constexpr (G) o[j] *= gate(rr[j]);
      }
      IoBf16::store<kTileV, false>(reinterpret_cast<uint16_t*>(ob) + at, o);
    }
  }
}

template <bool G>
__global__ __launch_bounds__(kTileThreads) void wkv_seq_tile_kernel(
    int64_t B, int64_t T, int64_t C, const float* __restrict__ w, const float* __restrict__ u,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ rg, const float* __restrict__ state_in,
    uint16_t* __restrict__ out, float* __restrict__ state_out) {
  __shared__ u32x4 kb[2][kTileVec];
  __shared__ u32x4 vb[2][kTileVec];
  __shared__ u32x4 rb[G ? 2 : 1][G ? kTileVec : 1];
  __shared__ u32x4 ob[2][kTileVec];
  const int tid = threadIdx.x;
  const int64_t gpr = C / kTileCh;  // C is a multiple of kTileCh here
  const int64_t b = blockIdx.x / gpr;
  const int64_t cw = (blockIdx.x - b * gpr) * kTileCh;  // the workgroup's first channel
  const int64_t c0 = cw + tid * kTileV;                  // this thread's
  const int64_t plane = B * C;
  const int64_t lane0 = b * C + c0;

  float wd[kTileV], ub[kTileV], cb[kTileV];
  IoF32::load<kTileV, false>(w + c0, wd);
  IoF32::load<kTileV, false>(u + c0, ub);
  bonus_ratios(wd, ub, cb);
  const bool fast = wave_fast_ok(wd, ub);
  Lane s[kTileV];
  if (state_in != nullptr) {
    float n[kTileV], d[kTileV], m[kTileV];
    IoF32::load<kTileV, false>(state_in + lane0, n);
    IoF32::load<kTileV, false>(state_in + plane + lane0, d);
    IoF32::load<kTileV, false>(state_in + 2 * plane + lane0, m);
#pragma unroll
    for (int j = 0; j < kTileV; ++j) s[j] = lane_from_state(n[j], d[j], m[j]);
  } else {
#pragma unroll
    for (int j = 0; j < kTileV; ++j) s[j] = lane_empty();
  }

  // byte addresses of the workgroup's row piece at token 0
  const int64_t row_bytes = C * 2;
  const char* kbase = reinterpret_cast<const char*>(k + b * T * C + cw);
  const char* vbase = reinterpret_cast<const char*>(v + b * T * C + cw);
  const char* rbase = G ? reinterpret_cast<const char*>(rg + b * T * C + cw) : nullptr;
  char* obase = reinterpret_cast<char*>(out + b * T * C + cw);
  u32x4 rk[kTileNv], rv[kTileNv], rr[G ? kTileNv : 1];
  // tile t's rows (only the first nrows when MASKED) into the registers
  auto gload = [&](int64_t t, int nrows, auto masked) {
#pragma unroll
    for (int i = 0; i < kTileNv; ++i) {
      const int j = tid + i * kTileThreads;
      const int row = j / kTileRowVec, col = j % kTileRowVec;
      if (!decltype(masked)::value || row < nrows) {
        const int64_t off = (t * kTileTok + row) * row_bytes + col * 16;
        rk[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off));
        rv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off));
        if constexpr (G) rr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rbase + off));
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kTileNv; ++i) {
      const int j = tid + i * kTileThreads;
      kb[buf][j] = rk[i];
      vb[buf][j] = rv[i];
      if constexpr (G) rb[buf][j] = rr[i];
    }
  };
  auto walk = [&](int buf, int nrows) {
    const u32x4* rbp = G ? rb[buf] : nullptr;
    if (fast) {
      tile_walk<true, G>(kb[buf], vb[buf], rbp, ob[buf], nrows, s, wd, ub, cb);
    } else {
      tile_walk<false, G>(kb[buf], vb[buf], rbp, ob[buf], nrows, s, wd, ub, cb);
    }
  };
  auto gstore = [&](int64_t t, int buf, int nrows, auto masked) {
#pragma unroll
    for (int i = 0; i < kTileNv; ++i) {
      const int j = tid + i * kTileThreads;
      const int row = j / kTileRowVec, col = j % kTileRowVec;
      if (!decltype(masked)::value || row < nrows) {
        const int64_t off = (t * kTileTok + row) * row_bytes + col * 16;
        __builtin_nontemporal_store(ob[buf][j], reinterpret_cast<u32x4*>(obase + off));
      }
    }
  };
  const std::false_type full{};
  const std::true_type part{};

  // Full tiles through the pipeline: tile t + 1 waits in registers and goes
  // to LDS after tile t is walked, then tile t + 2's loads are issued. Inside
  // the loop every load and store is unconditional (the compiler's counter
  // waits then stop at the data about to be used); the last two full tiles
  // are walked after it, then the partial tile on its own.
  const int64_t nfull = T / kTileTok;
  const int rest = static_cast<int>(T - nfull * kTileTok);
  if (nfull > 0) {
    gload(0, kTileTok, full);
    lstore(0);
    if (nfull > 1) gload(1, kTileTok, full);
    __syncthreads();
    int64_t t = 0;
    for (; t + 2 < nfull; ++t) {
      const int buf = static_cast<int>(t & 1);
      walk(buf, kTileTok);
      lstore(buf ^ 1);
      gload(t + 2, kTileTok, full);
      __syncthreads();
      gstore(t, buf, kTileTok, full);
    }
    if (t + 1 < nfull) {  // two left, the second in registers
      const int buf = static_cast<int>(t & 1);
      walk(buf, kTileTok);
      lstore(buf ^ 1);
      __syncthreads();
      gstore(t, buf, kTileTok, full);
      ++t;
    }
    {  // the last full tile, already in LDS
      const int buf = static_cast<int>(t & 1);
      walk(buf, kTileTok);
      __syncthreads();
      gstore(t, buf, kTileTok, full);
    }
  }
  if (rest > 0) {
    // the buffer after the last full tile's: no thread reads it any more
    const int buf = static_cast<int>(nfull & 1);
    gload(nfull, rest, part);
    lstore(buf);
    __syncthreads();
    walk(buf, rest);
    __syncthreads();
    gstore(nfull, buf, rest, part);
  }

  if (state_out != nullptr) {
    float n[kTileV], d[kTileV], m[kTileV];
#pragma unroll
    for (int j = 0; j < kTileV; ++j) {
      n[j] = s[j].n;
      d[j] = s[j].d;
      m[j] = lane_max_exp(s[j], wd[j]);
    }
    IoF32::store<kTileV, false>(state_out + lane0, n);
    IoF32::store<kTileV, false>(state_out + plane + lane0, d);
    IoF32::store<kTileV, false>(state_out + 2 * plane + lane0, m);
  }
}

hipError_t launch_seq_tile(const FwdArgs& a, hipStream_t st) {
  const int64_t blocks = a.B * (a.C / kTileCh);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const auto* kk = static_cast<const uint16_t*>(a.k);
  const auto* vv = static_cast<const uint16_t*>(a.v);
  const auto* rr = static_cast<const uint16_t*>(a.r);
  auto* oo = static_cast<uint16_t*>(a.out);
  if (rr != nullptr) {
    hipLaunchKernelGGL(wkv_seq_tile_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kTileThreads), 0, st, a.B, a.T, a.C, a.w, a.u, kk, vv, rr,
                       a.state_in, oo, a.state_out);
  } else {
    hipLaunchKernelGGL(wkv_seq_tile_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kTileThreads), 0, st, a.B, a.T, a.C, a.w, a.u, kk, vv, rr,
                       a.state_in, oo, a.state_out);
  }
  return hipGetLastError();
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

static bool tile_ok(const FwdArgs& a) {
  // whole 1 KiB row pieces, 16-byte aligned rows and pointers, no checkpoints
  return a.C % kTileCh == 0 && a.ckpt == nullptr && aligned(a.k, 16) && aligned(a.v, 16) &&
         aligned(a.out, 16) && aligned(a.r, 16) && aligned(a.w, 8) && aligned(a.u, 8) &&
         aligned(a.state_in, 8) && aligned(a.state_out, 8);
}

hipError_t launch_seq(const FwdArgs& a, int io, int vec, hipStream_t s) {
  if (io == kF32) return launch_seq_t<IoF32, 1>(a, s);
  if (tile_ok(a)) return launch_seq_tile(a, s);
  if (vec == 2) return launch_seq_t<IoBf16, 2>(a, s);
  return launch_seq_t<IoBf16, 1>(a, s);
}

}  // namespace wkv
