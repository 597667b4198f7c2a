// C interface of libwkv (declared in include/wkv.h): argument validation,
// kernel selection and launch on the caller's stream. No device memory is
// allocated here; the only state kept is a per-device compute-unit count,
// queried once.
#include "wkv.h"

#include <atomic>
#include <cstdint>
#include <mutex>

#include "wkv_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0: not yet queried

int cu_count(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

int fail(int status, hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return status;
}

bool mul3(int64_t a, int64_t b, int64_t c, int64_t* r) {
  int64_t ab;
  return !__builtin_mul_overflow(a, b, &ab) && !__builtin_mul_overflow(ab, c, r);
}

// [p, p + bytes) and [q, q + bytes2) share a byte (empty ranges never do).
bool overlaps(const void* p, int64_t bytes, const void* q, int64_t bytes2) {
  if (p == nullptr || q == nullptr || bytes <= 0 || bytes2 <= 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + static_cast<uintptr_t>(bytes2) && b < a + static_cast<uintptr_t>(bytes);
}

bool misaligned(const void* p, int bytes) {
  return p != nullptr && reinterpret_cast<uintptr_t>(p) % bytes != 0;
}

// Largest byte count a single tensor may span: keeps every index computation
// in the kernels inside int64.
constexpr int64_t kMaxBytes = int64_t(1) << 60;

// Kernel for AUTO. The sequential scan needs no cross-thread combine, so it
// wins whenever B*C lanes alone give every SIMD at least one wave (4 SIMDs per
// CU). Below that a time-parallel kernel creates the missing parallelism:
// up to kChunkMaxT tokens the chunked scan (it needs no workspace; the
// second exception below takes the look-back scan for some fp32 shapes),
// beyond it the look-back scan when a workspace is available.
//
// First exception, measured on MI355X: the sequential scan walks every batch
// row at the same token, and that access pattern streams at 0.71-0.75 of the
// HBM peak when a row's bytes (T * C * 4 for fp32) are a power of two but at
// only 0.64-0.66 otherwise (the same walk over rows padded from 1.5 to 2 MiB
// went from 0.66 to 0.71). The chunked scan keeps a few rows' tiles in
// flight instead and holds 0.66 there, so plain (ungated, constant-decay,
// no checkpoints) fp32 rows of another size with 512 to kChunkMaxT tokens
// take it. The other forms keep the sequential scan: their chunked kernels
// hold more registers (three waves per SIMD instead of four) and lose there
// (B=256 T=512 C=768: the checkpointing prefill 273 against 246 us, the
// per-token decay 341 against 313). bf16 keeps the sequential scan too,
// whose LDS-staged tiles stay ahead of the chunked scan at every measured
// size.
//
// Second exception, for fp32 with a workspace, measured on MI355X over
// 8-layer graphs: once the chunked scan's 32-channel groups (B * ceil(C / 32),
// one workgroup each) outnumber the CUs, but by at most four to one, the
// chunked scan leaves CUs unevenly loaded, and the look-back scan's 256-token
// segments win past 512 tokens (plain form, measured from T = 520: 3-38% on 19 shapes; B=16 T=2048
// C=768 64 against 79 us) and from T = 1280 up when gated (14-29% on 5; at
// T = 896-1152 the gated chunked scan still won by 7-10%). At up to one
// group per CU the chunked scan's two walkers win (B=8 T=1024 C=768: 22
// against 26 us); past four per CU neither wins everywhere (B=64 T=1536
// C=768: the chunked scan by 7%), nor does the bf16 look-back scan anywhere
// below T = 2048.
constexpr int64_t kChunkMaxT = 2048;
constexpr int64_t kLbMidMinT = 513, kLbMidMinTGated = 1280;

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int choose_path(int64_t B, int64_t T, int64_t C, int io, int dev, bool have_ws, bool plain) {
  const int64_t per_thread = io == wkv::kBf16 ? 2 : 1;
  const int64_t waves = (B * C / per_thread + 63) / 64;
  if (T < 32) return WKV_PATH_SEQ;
  if (waves >= 4LL * cu_count(dev)) {
    int64_t row_bytes = 0;
    const bool uneven_rows = plain && io == wkv::kF32 &&
                             (__builtin_mul_overflow(T * C, 4, &row_bytes) || !pow2(row_bytes));
    return uneven_rows && T >= 512 && T <= kChunkMaxT ? WKV_PATH_CHUNK : WKV_PATH_SEQ;
  }
  if (!have_ws) return WKV_PATH_CHUNK;
  if (T > kChunkMaxT) return WKV_PATH_LOOKBACK;
  const int64_t groups = B * ((C + 31) / 32), cus = cu_count(dev);
  const bool mid = io == wkv::kF32 && groups > cus && groups <= 4 * cus &&
                   T >= (plain ? kLbMidMinT : kLbMidMinTGated);
  return mid ? WKV_PATH_LOOKBACK : WKV_PATH_CHUNK;
}

// Workspace the look-back kernel needs, whichever channel width the pointers
// allow (the larger of the two candidates).
int64_t lookback_bytes(int io, int64_t B, int64_t T, int64_t C) {
  const int64_t a = wkv::lookback_workspace_bytes(1, B, T, C);
  if (io != wkv::kBf16) return a;
  const int64_t b = wkv::lookback_workspace_bytes(2, B, T, C);
  return a > b ? a : b;
}

// Bytes of the backward pass's checkpoints for these sizes: one float4 per
// lane and chunk of kCkptTokens tokens, or -1 past the size limit.
int64_t ckpt_bytes(int64_t B, int64_t T, int64_t C) {
  const int64_t nch = (T + wkv::kCkptTokens - 1) / wkv::kCkptTokens;
  int64_t n;
  if (!mul3(nch, B, C, &n) || __builtin_mul_overflow(n, 16, &n) || n > kMaxBytes) return -1;
  return n;
}

int forward_impl(int64_t B, int64_t T, int64_t C, const float* w, const float* u, const void* k,
                 const void* v, const void* r, bool gated, const float* state_in, void* out,
                 float* state_out, int io, int path, void* workspace, int64_t workspace_bytes,
                 hipStream_t stream, float* ckpt = nullptr, bool check_only = false) {
  if (io != WKV_IO_F32 && io != WKV_IO_BF16) return WKV_ERR_ARG;
  if (path < WKV_PATH_AUTO || path > WKV_PATH_LOOKBACK) return WKV_ERR_ARG;
  if (B < 0 || T < 0 || C < 0) return WKV_ERR_DIM;
  const int64_t es = io == WKV_IO_BF16 ? 2 : 4;
  int64_t seq_bytes, state_bytes;
  if (!mul3(B, T, C, &seq_bytes) || __builtin_mul_overflow(seq_bytes, es, &seq_bytes) ||
      seq_bytes > kMaxBytes)
    return WKV_ERR_DIM;
  if (!mul3(B, C, 12, &state_bytes) || state_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (B == 0 || C == 0) return WKV_OK;

  if (w == nullptr || u == nullptr) return WKV_ERR_NULL;
  if (T > 0 && (k == nullptr || v == nullptr || out == nullptr)) return WKV_ERR_NULL;
  if (gated && T > 0 && r == nullptr) return WKV_ERR_NULL;
  if (!gated || T == 0) r = nullptr;
  if (misaligned(w, 4) || misaligned(u, 4) || misaligned(state_in, 4) || misaligned(state_out, 4))
    return WKV_ERR_ALIGN;
  if (misaligned(k, es) || misaligned(v, es) || misaligned(out, es) || misaligned(r, es))
    return WKV_ERR_ALIGN;

  const int64_t pbytes = C * 4;
  const int64_t sbytes = T > 0 ? seq_bytes : 0;
  if (overlaps(out, sbytes, r, sbytes) || overlaps(state_out, state_bytes, r, sbytes))
    return WKV_ERR_ALIAS;
  // out must not touch anything else
  if (overlaps(out, sbytes, k, sbytes) || overlaps(out, sbytes, v, sbytes) ||
      overlaps(out, sbytes, w, pbytes) || overlaps(out, sbytes, u, pbytes) ||
      overlaps(out, sbytes, state_in, state_bytes) || overlaps(out, sbytes, state_out, state_bytes))
    return WKV_ERR_ALIAS;
  // state_out may be state_in exactly, and must not touch any other input
  if (overlaps(state_out, state_bytes, k, sbytes) || overlaps(state_out, state_bytes, v, sbytes) ||
      overlaps(state_out, state_bytes, w, pbytes) || overlaps(state_out, state_bytes, u, pbytes))
    return WKV_ERR_ALIAS;
  if (state_out != state_in && overlaps(state_out, state_bytes, state_in, state_bytes))
    return WKV_ERR_ALIAS;
  if (ckpt != nullptr && T > 0) {
    // checkpoints for the backward pass: fp32, the sequential or chunked scan
    const int64_t cb = ckpt_bytes(B, T, C);
    if (io != WKV_IO_F32) return WKV_ERR_ARG;
    if (cb < 0) return WKV_ERR_DIM;
    if (misaligned(ckpt, 16)) return WKV_ERR_ALIGN;
    if (overlaps(ckpt, cb, k, sbytes) || overlaps(ckpt, cb, v, sbytes) ||
        overlaps(ckpt, cb, r, sbytes) || overlaps(ckpt, cb, out, sbytes) ||
        overlaps(ckpt, cb, w, pbytes) || overlaps(ckpt, cb, u, pbytes) ||
        overlaps(ckpt, cb, state_in, state_bytes) || overlaps(ckpt, cb, state_out, state_bytes))
      return WKV_ERR_ALIAS;
    if (path == WKV_PATH_LOOKBACK) return WKV_ERR_ARG;
  } else {
    ckpt = nullptr;
  }
  if (workspace != nullptr && workspace_bytes < 0) return WKV_ERR_WORKSPACE;
  const bool have_ws = ckpt == nullptr && workspace != nullptr && workspace_bytes > 0;
  if (have_ws) {
    if (misaligned(workspace, 256)) return WKV_ERR_ALIGN;
    if (overlaps(workspace, workspace_bytes, k, sbytes) ||
        overlaps(workspace, workspace_bytes, v, sbytes) ||
        overlaps(workspace, workspace_bytes, out, sbytes) ||
        overlaps(workspace, workspace_bytes, r, sbytes) ||
        overlaps(workspace, workspace_bytes, w, pbytes) ||
        overlaps(workspace, workspace_bytes, u, pbytes) ||
        overlaps(workspace, workspace_bytes, state_in, state_bytes) ||
        overlaps(workspace, workspace_bytes, state_out, state_bytes))
      return WKV_ERR_ALIAS;
  }

  const wkv::FwdArgs a{B, T, C, w, u, k, v, state_in, out, state_out, r, ckpt};
  if (path == WKV_PATH_LOOKBACK && T > 0 &&
      (!have_ws || workspace_bytes < wkv::lookback_workspace_bytes(
                                         wkv::lookback_vec_width(io, C, a), B, T, C)))
    return WKV_ERR_WORKSPACE;

  if (check_only) return WKV_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, e);

  if (T == 0) {
    if (state_out == nullptr || state_out == state_in) return WKV_OK;
    e = wkv::launch_state_copy(B, C, state_in, state_out, stream);
    return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
  }

  if (path == WKV_PATH_AUTO)
    path = choose_path(B, T, C, io, dev, have_ws, !gated && ckpt == nullptr);
  if (path == WKV_PATH_SEQ) {
    e = wkv::launch_seq(a, io, wkv::seq_vec_width(io, C, a), stream);
  } else if (path == WKV_PATH_CHUNK) {
    e = wkv::launch_chunk(a, io, wkv::chunk_vec_width(io, C, a), cu_count(dev), stream);
  } else {
    const int vec = wkv::lookback_vec_width(io, C, a);
    if (!have_ws || workspace_bytes < wkv::lookback_workspace_bytes(vec, B, T, C))
      return WKV_ERR_WORKSPACE;
    const wkv::LbWorkspace ws{static_cast<uint32_t*>(workspace), workspace_bytes};
    e = wkv::launch_lookback(a, io, vec, ws, stream);
  }
  return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
}

// Device scratch of wkv_forward_noalloc, for callers that cannot allocate:
// the look-back scan's workspace, one copy per device (each device that loads
// the library holds it until the process ends). Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, once per device, and is
// kept in g_scratch.
constexpr int64_t kScratchBytes = int64_t{32} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch[kMaxDevices];

// This device's scratch (dev must be current), or nullptr with *e set.
void* scratch_on(int dev, hipError_t* e) {
  if (dev < 0 || dev >= kMaxDevices) {
    *e = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  *e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (*e != hipSuccess || p == nullptr) {
    if (*e == hipSuccess) *e = hipErrorInvalidSymbol;
    return nullptr;
  }
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

int shift_impl(int64_t B, int64_t T, int64_t C, int64_t P, const float* mu, const void* x,
               const void* x_prev, void* out, void* x_last, int io, hipStream_t stream) {
  if (io != WKV_IO_F32 && io != WKV_IO_BF16) return WKV_ERR_ARG;
  if (B < 0 || T < 0 || C < 0 || P < 1 || P > wkv::kShiftMaxP) return WKV_ERR_DIM;
  const int64_t es = io == WKV_IO_BF16 ? 2 : 4;
  int64_t seq_bytes, out_bytes, row_bytes, mu_bytes;
  if (!mul3(B, T, C, &seq_bytes) || __builtin_mul_overflow(seq_bytes, es, &seq_bytes) ||
      __builtin_mul_overflow(seq_bytes, P, &out_bytes) || out_bytes > kMaxBytes)
    return WKV_ERR_DIM;
  if (!mul3(B, C, es, &row_bytes) || !mul3(P, C, 4, &mu_bytes)) return WKV_ERR_DIM;
  if (B == 0 || C == 0) return WKV_OK;
  if (T > 0 && (mu == nullptr || x == nullptr || out == nullptr)) return WKV_ERR_NULL;
  if (misaligned(mu, 4) || misaligned(x, es) || misaligned(x_prev, es) || misaligned(out, es) ||
      misaligned(x_last, es))
    return WKV_ERR_ALIGN;
  const int64_t sb = T > 0 ? seq_bytes : 0, ob = T > 0 ? out_bytes : 0;
  if (overlaps(out, ob, x, sb) || overlaps(out, ob, x_prev, row_bytes) ||
      overlaps(out, ob, mu, mu_bytes) || overlaps(out, ob, x_last, row_bytes))
    return WKV_ERR_ALIAS;
  if (overlaps(x_last, row_bytes, x, sb) || overlaps(x_last, row_bytes, mu, mu_bytes))
    return WKV_ERR_ALIAS;
  if (x_last != x_prev && overlaps(x_last, row_bytes, x_prev, row_bytes)) return WKV_ERR_ALIAS;
  const wkv::ShiftArgs a{B, T, C, P, mu, x, x_prev, out, x_last};
  const hipError_t e = wkv::launch_shift(a, io, stream);
  return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
}

int step_impl(int64_t B, int64_t C, const float* w, const float* u, const void* k, const void* v,
              const void* r, bool gated, float* state, void* out, int io, hipStream_t stream) {
  if (B < 0 || C < 0) return WKV_ERR_DIM;
  const int64_t es = io == WKV_IO_BF16 ? 2 : 4;
  int64_t io_bytes, state_bytes;
  if (!mul3(B, C, es, &io_bytes) || io_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (!mul3(B, C, 12, &state_bytes) || state_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (B == 0 || C == 0) return WKV_OK;
  if (w == nullptr || u == nullptr || k == nullptr || v == nullptr || state == nullptr ||
      out == nullptr || (gated && r == nullptr))
    return WKV_ERR_NULL;
  if (!gated) r = nullptr;
  if (misaligned(w, 4) || misaligned(u, 4) || misaligned(state, 4)) return WKV_ERR_ALIGN;
  if (misaligned(k, es) || misaligned(v, es) || misaligned(out, es) || misaligned(r, es))
    return WKV_ERR_ALIGN;
  const int64_t pbytes = C * 4;
  if (overlaps(out, io_bytes, k, io_bytes) || overlaps(out, io_bytes, v, io_bytes) ||
      overlaps(out, io_bytes, w, pbytes) || overlaps(out, io_bytes, u, pbytes) ||
      overlaps(out, io_bytes, state, state_bytes) || overlaps(out, io_bytes, r, io_bytes))
    return WKV_ERR_ALIAS;
  if (overlaps(state, state_bytes, k, io_bytes) || overlaps(state, state_bytes, v, io_bytes) ||
      overlaps(state, state_bytes, w, pbytes) || overlaps(state, state_bytes, u, pbytes) ||
      overlaps(state, state_bytes, r, io_bytes))
    return WKV_ERR_ALIAS;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, e);
  const wkv::StepArgs a{B, C, w, u, k, v, state, out, r};
  e = wkv::launch_step(a, io, wkv::step_vec_width(io, C, a), stream);
  return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
}

// Per-token decay: w is a sequence like k (same element type), u per channel.
int forward_dd_impl(int64_t B, int64_t T, int64_t C, const void* w, const float* u, const void* k,
                    const void* v, const float* state_in, void* out, float* state_out, int io,
                    int path, hipStream_t stream, void* ckpt = nullptr, bool want_ckpt = false) {
  if (io != WKV_IO_F32 && io != WKV_IO_BF16) return WKV_ERR_ARG;
  if (path != WKV_PATH_AUTO && path != WKV_PATH_SEQ && path != WKV_PATH_CHUNK) return WKV_ERR_ARG;
  if (B < 0 || T < 0 || C < 0) return WKV_ERR_DIM;
  const int64_t es = io == WKV_IO_BF16 ? 2 : 4;
  int64_t seq_bytes, state_bytes;
  if (!mul3(B, T, C, &seq_bytes) || __builtin_mul_overflow(seq_bytes, es, &seq_bytes) ||
      seq_bytes > kMaxBytes)
    return WKV_ERR_DIM;
  if (!mul3(B, C, 12, &state_bytes) || state_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (B == 0 || C == 0) return WKV_OK;
  if (u == nullptr) return WKV_ERR_NULL;
  if (T > 0 && (w == nullptr || k == nullptr || v == nullptr || out == nullptr))
    return WKV_ERR_NULL;
  if (misaligned(u, 4) || misaligned(state_in, 4) || misaligned(state_out, 4))
    return WKV_ERR_ALIGN;
  if (misaligned(w, es) || misaligned(k, es) || misaligned(v, es) || misaligned(out, es))
    return WKV_ERR_ALIGN;
  const int64_t pbytes = C * 4;
  const int64_t sbytes = T > 0 ? seq_bytes : 0;
  if (want_ckpt) {
    // checkpoints for the backward: fp32 only, 16-byte records
    if (io != WKV_IO_F32) return WKV_ERR_ARG;
    if (T == 0) ckpt = nullptr;
    if (T > 0 && ckpt == nullptr) return WKV_ERR_NULL;
    if (misaligned(ckpt, 16)) return WKV_ERR_ALIGN;
    const int64_t cbytes = T > 0 ? ckpt_bytes(B, T, C) : 0;
    if (cbytes < 0) return WKV_ERR_DIM;
    const void* others[] = {w, u, k, v, out, state_in, state_out};
    const int64_t sizes[] = {sbytes, pbytes, sbytes, sbytes, sbytes, state_bytes, state_bytes};
    for (int i = 0; i < 7; ++i)
      if (overlaps(ckpt, cbytes, others[i], sizes[i])) return WKV_ERR_ALIAS;
  }
  if (overlaps(out, sbytes, w, sbytes) || overlaps(out, sbytes, k, sbytes) ||
      overlaps(out, sbytes, v, sbytes) || overlaps(out, sbytes, u, pbytes) ||
      overlaps(out, sbytes, state_in, state_bytes) || overlaps(out, sbytes, state_out, state_bytes))
    return WKV_ERR_ALIAS;
  if (overlaps(state_out, state_bytes, w, sbytes) || overlaps(state_out, state_bytes, k, sbytes) ||
      overlaps(state_out, state_bytes, v, sbytes) || overlaps(state_out, state_bytes, u, pbytes))
    return WKV_ERR_ALIAS;
  if (state_out != state_in && overlaps(state_out, state_bytes, state_in, state_bytes))
    return WKV_ERR_ALIAS;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, e);
  if (T == 0) {
    if (state_out == nullptr || state_out == state_in) return WKV_OK;
    e = wkv::launch_state_copy(B, C, state_in, state_out, stream);
    return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
  }
  const wkv::DdArgs a{B, T, C, w, u, k, v, state_in, out, state_out, ckpt};
  if (path == WKV_PATH_AUTO) path = choose_path(B, T, C, io, dev, false, false);
  const int vec = wkv::dd_vec_width(io, C, a);
  e = path == WKV_PATH_SEQ ? wkv::launch_dd_seq(a, io, vec, stream)
                           : wkv::launch_dd_chunk(a, io, vec, cu_count(dev), stream);
  return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
}

int step_dd_impl(int64_t B, int64_t C, const void* w, const float* u, const void* k,
                 const void* v, float* state, void* out, int io, hipStream_t stream) {
  if (io != WKV_IO_F32 && io != WKV_IO_BF16) return WKV_ERR_ARG;
  if (B < 0 || C < 0) return WKV_ERR_DIM;
  const int64_t es = io == WKV_IO_BF16 ? 2 : 4;
  int64_t io_bytes, state_bytes;
  if (!mul3(B, C, es, &io_bytes) || io_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (!mul3(B, C, 12, &state_bytes) || state_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (B == 0 || C == 0) return WKV_OK;
  if (w == nullptr || u == nullptr || k == nullptr || v == nullptr || state == nullptr ||
      out == nullptr)
    return WKV_ERR_NULL;
  if (misaligned(u, 4) || misaligned(state, 4)) return WKV_ERR_ALIGN;
  if (misaligned(w, es) || misaligned(k, es) || misaligned(v, es) || misaligned(out, es))
    return WKV_ERR_ALIGN;
  const int64_t pbytes = C * 4;
  if (overlaps(out, io_bytes, w, io_bytes) || overlaps(out, io_bytes, k, io_bytes) ||
      overlaps(out, io_bytes, v, io_bytes) || overlaps(out, io_bytes, u, pbytes) ||
      overlaps(out, io_bytes, state, state_bytes))
    return WKV_ERR_ALIAS;
  if (overlaps(state, state_bytes, w, io_bytes) || overlaps(state, state_bytes, k, io_bytes) ||
      overlaps(state, state_bytes, v, io_bytes) || overlaps(state, state_bytes, u, pbytes))
    return WKV_ERR_ALIAS;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, e);
  const wkv::DdStepArgs a{B, C, w, u, k, v, state, out};
  e = wkv::launch_dd_step(a, io, wkv::dd_step_vec_width(io, C, a), stream);
  return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
}

// Matrix-valued state: segments for these sizes on this device, limited to
// what the workspace holds (one segment, i.e. none, without a workspace).
int64_t matrix_plan(int64_t B, int64_t T, int64_t H, int dev, int64_t ws_bytes) {
  int64_t P = wkv::matrix_segments(B, T, H, cu_count(dev));
  while (P > 1 && wkv::matrix_workspace_bytes(B, T, H, P) > ws_bytes) --P;
  return P;
}

int matrix_forward_impl(int64_t B, int64_t T, int64_t H, int64_t D, const float* w,
                        const float* k, const float* v, const float* r, const float* state_in,
                        float* out, float* state_out, void* workspace, int64_t workspace_bytes,
                        hipStream_t stream) {
  if (B < 0 || T < 0 || H < 0 || D < 0) return WKV_ERR_DIM;
  if (D != wkv::kMatrixHead || H > wkv::kMatrixMaxHeads) return WKV_ERR_DIM;
  int64_t seq_bytes, state_bytes;
  if (!mul3(B, T, H * D, &seq_bytes) || __builtin_mul_overflow(seq_bytes, 4, &seq_bytes) ||
      seq_bytes > kMaxBytes)
    return WKV_ERR_DIM;
  if (!mul3(B, H, D * D * 4, &state_bytes) || state_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (B == 0 || H == 0) return WKV_OK;
  if (T > 0 && (w == nullptr || k == nullptr || v == nullptr || r == nullptr || out == nullptr))
    return WKV_ERR_NULL;
  const void* all[] = {w, k, v, r, out};
  for (const void* p : all)
    if (misaligned(p, 8)) return WKV_ERR_ALIGN;
  if (misaligned(state_in, 16) || misaligned(state_out, 16)) return WKV_ERR_ALIGN;
  const int64_t sbytes = T > 0 ? seq_bytes : 0;
  const void* ins[] = {w, k, v, r};
  for (const void* p : ins) {
    if (overlaps(out, sbytes, p, sbytes) || overlaps(state_out, state_bytes, p, sbytes))
      return WKV_ERR_ALIAS;
  }
  if (overlaps(out, sbytes, state_in, state_bytes) || overlaps(out, sbytes, state_out, state_bytes))
    return WKV_ERR_ALIAS;
  if (state_out != state_in && overlaps(state_out, state_bytes, state_in, state_bytes))
    return WKV_ERR_ALIAS;
  if (workspace_bytes < 0) return WKV_ERR_WORKSPACE;
  const int64_t wsb = workspace == nullptr ? 0 : workspace_bytes;
  if (wsb > 0) {
    if (misaligned(workspace, 256)) return WKV_ERR_ALIGN;
    const void* every[] = {w, k, v, r, out};
    for (const void* p : every)
      if (overlaps(workspace, wsb, p, sbytes)) return WKV_ERR_ALIAS;
    if (overlaps(workspace, wsb, state_in, state_bytes) ||
        overlaps(workspace, wsb, state_out, state_bytes))
      return WKV_ERR_ALIAS;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, e);
  if (T == 0) {
    if (state_out == nullptr || state_out == state_in) return WKV_OK;
    e = wkv::launch_matrix_state_copy(B, H, state_in, state_out, stream);
    return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
  }
  const int64_t P = matrix_plan(B, T, H, dev, wsb);
  const wkv::MatrixArgs a{B, T, H, w, k, v, r, state_in, out, state_out};
  e = wkv::launch_matrix(a, P, workspace, stream);
  return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
}

int matrix_step_impl(int64_t B, int64_t H, int64_t D, const float* w, const float* k,
                     const float* v, const float* r, float* state, float* out,
                     hipStream_t stream) {
  if (B < 0 || H < 0 || D < 0) return WKV_ERR_DIM;
  if (D != wkv::kMatrixHead) return WKV_ERR_DIM;
  int64_t io_bytes, state_bytes;
  if (!mul3(B, H, D * 4, &io_bytes) || io_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (!mul3(B, H, D * D * 4, &state_bytes) || state_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (B == 0 || H == 0) return WKV_OK;
  if (w == nullptr || k == nullptr || v == nullptr || r == nullptr || state == nullptr ||
      out == nullptr)
    return WKV_ERR_NULL;
  const void* all[] = {w, k, v, r, out};
  for (const void* p : all)
    if (misaligned(p, 4)) return WKV_ERR_ALIGN;
  if (misaligned(state, 16)) return WKV_ERR_ALIGN;
  const void* ins[] = {w, k, v, r};
  for (const void* p : ins) {
    if (overlaps(out, io_bytes, p, io_bytes) || overlaps(state, state_bytes, p, io_bytes))
      return WKV_ERR_ALIAS;
  }
  if (overlaps(out, io_bytes, state, state_bytes)) return WKV_ERR_ALIAS;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, e);
  const wkv::MatrixStepArgs a{B, H, w, k, v, r, state, out};
  e = wkv::launch_matrix_step(a, stream);
  return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
}

int backward_impl(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                  const float* k, const float* v, const float* r, const float* state_in,
                  const float* state_out, const float* gstate_out, const float* gout, float* gk,
                  float* gv, float* gr, float* gw, float* gu, float* gstate_in, void* workspace,
                  int64_t workspace_bytes, hipStream_t stream, const float* ckpt = nullptr) {
  if (B < 0 || T < 0 || C < 0) return WKV_ERR_DIM;
  int64_t seq_bytes, state_bytes;
  if (!mul3(B, T, C, &seq_bytes) || __builtin_mul_overflow(seq_bytes, 4, &seq_bytes) ||
      seq_bytes > kMaxBytes)
    return WKV_ERR_DIM;
  if (!mul3(B, C, 12, &state_bytes) || state_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (C == 0) return WKV_OK;
  const int64_t need = wkv::backward_workspace_bytes(B, T, C);
  if (need < 0 || need > kMaxBytes) return WKV_ERR_DIM;

  if (w == nullptr || u == nullptr || gw == nullptr || gu == nullptr) return WKV_ERR_NULL;
  const bool tokens = B > 0 && T > 0;
  if (tokens && (k == nullptr || v == nullptr || gout == nullptr || gk == nullptr || gv == nullptr))
    return WKV_ERR_NULL;
  if ((gstate_out == nullptr) != (state_out == nullptr)) return WKV_ERR_NULL;
  if (tokens && r != nullptr && gr == nullptr) return WKV_ERR_NULL;
  if (!tokens) r = nullptr, gr = nullptr;
  if (r == nullptr) gr = nullptr;
  const void* all[] = {w,    u,  k,  v,  r,  state_in, state_out, gstate_out,
                       gout, gk, gv, gr, gw, gu,       gstate_in};
  for (const void* p : all)
    if (misaligned(p, 4)) return WKV_ERR_ALIGN;
  if (!tokens) ckpt = nullptr;
  const int64_t cbytes = ckpt != nullptr ? ckpt_bytes(B, T, C) : 0;
  if (cbytes < 0) return WKV_ERR_DIM;
  if (misaligned(ckpt, 16)) return WKV_ERR_ALIGN;

  const int64_t pbytes = C * 4;
  const int64_t sbytes = tokens ? seq_bytes : 0;
  struct Range {
    const void* p;
    int64_t n;
  };
  const Range inputs[] = {{w, pbytes},        {u, pbytes},          {k, sbytes},
                          {v, sbytes},        {r, sbytes},          {gout, sbytes},
                          {state_in, state_bytes}, {state_out, state_bytes},
                          {gstate_out, state_bytes}, {ckpt, cbytes}};
  const Range outputs[] = {{gk, sbytes}, {gv, sbytes}, {gr, sbytes}, {gw, pbytes}, {gu, pbytes},
                           {gstate_in, state_bytes}};
  for (int i = 0; i < 6; ++i) {
    for (const Range& r : inputs)
      if (overlaps(outputs[i].p, outputs[i].n, r.p, r.n)) return WKV_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outputs[i].p, outputs[i].n, outputs[j].p, outputs[j].n)) return WKV_ERR_ALIAS;
  }
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return WKV_ERR_WORKSPACE;
    if (misaligned(workspace, 256)) return WKV_ERR_ALIGN;
    for (const Range& r : inputs)
      if (overlaps(workspace, workspace_bytes, r.p, r.n)) return WKV_ERR_ALIAS;
    for (const Range& r : outputs)
      if (overlaps(workspace, workspace_bytes, r.p, r.n)) return WKV_ERR_ALIAS;
  }

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, e);
  wkv::BwdArgs a{B,  T,  C,  w,  u,         k, v,  gout, state_in, state_out, gstate_out,
                 gk, gv, gw, gu, gstate_in, r, gr, ckpt};
  a.cus = cu_count(dev);
  e = wkv::launch_backward(a, workspace, stream);
  return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
}

// Backward of the per-token-decay operator (fp32; gw shaped like k).
int backward_dd_impl(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                     const float* k, const float* v, const float* state_in,
                     const float* state_out, const float* gstate_out, const float* gout,
                     float* gk, float* gv, float* gw, float* gu, float* gstate_in,
                     void* workspace, int64_t workspace_bytes, hipStream_t stream,
                     const void* ckpt = nullptr, bool want_ckpt = false) {
  if (B < 0 || T < 0 || C < 0) return WKV_ERR_DIM;
  int64_t seq_bytes, state_bytes;
  if (!mul3(B, T, C, &seq_bytes) || __builtin_mul_overflow(seq_bytes, 4, &seq_bytes) ||
      seq_bytes > kMaxBytes)
    return WKV_ERR_DIM;
  if (!mul3(B, C, 12, &state_bytes) || state_bytes > kMaxBytes) return WKV_ERR_DIM;
  if (C == 0) return WKV_OK;
  const int64_t need = wkv::dd_backward_workspace_bytes(B, T, C);
  if (need < 0 || need > kMaxBytes) return WKV_ERR_DIM;

  if (u == nullptr || gu == nullptr) return WKV_ERR_NULL;
  const bool tokens = B > 0 && T > 0;
  if (tokens && (w == nullptr || k == nullptr || v == nullptr || gout == nullptr ||
                 gk == nullptr || gv == nullptr || gw == nullptr))
    return WKV_ERR_NULL;
  if ((gstate_out == nullptr) != (state_out == nullptr)) return WKV_ERR_NULL;
  const void* all[] = {w, u, k, v, state_in, state_out, gstate_out, gout, gk, gv, gw, gu,
                       gstate_in};
  for (const void* p : all)
    if (misaligned(p, 4)) return WKV_ERR_ALIGN;
  if (!tokens) ckpt = nullptr;
  if (want_ckpt && tokens && ckpt == nullptr) return WKV_ERR_NULL;
  if (misaligned(ckpt, 16)) return WKV_ERR_ALIGN;
  const int64_t cbytes = ckpt != nullptr ? ckpt_bytes(B, T, C) : 0;
  if (cbytes < 0) return WKV_ERR_DIM;

  const int64_t pbytes = C * 4;
  const int64_t sbytes = tokens ? seq_bytes : 0;
  struct Range {
    const void* p;
    int64_t n;
  };
  const Range inputs[] = {{w, sbytes},        {u, pbytes},          {k, sbytes},
                          {v, sbytes},        {gout, sbytes},       {state_in, state_bytes},
                          {state_out, state_bytes}, {gstate_out, state_bytes}, {ckpt, cbytes}};
  const Range outputs[] = {{gk, sbytes}, {gv, sbytes}, {gw, sbytes}, {gu, pbytes},
                           {gstate_in, state_bytes}};
  for (int i = 0; i < 5; ++i) {
    for (const Range& r : inputs)
      if (overlaps(outputs[i].p, outputs[i].n, r.p, r.n)) return WKV_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outputs[i].p, outputs[i].n, outputs[j].p, outputs[j].n)) return WKV_ERR_ALIAS;
  }
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return WKV_ERR_WORKSPACE;
    if (misaligned(workspace, 256)) return WKV_ERR_ALIGN;
    for (const Range& r : inputs)
      if (overlaps(workspace, workspace_bytes, r.p, r.n)) return WKV_ERR_ALIAS;
    for (const Range& r : outputs)
      if (overlaps(workspace, workspace_bytes, r.p, r.n)) return WKV_ERR_ALIAS;
  }

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, e);
  const wkv::DdBwdArgs a{B, T, C, w, u, k, v, gout, state_in, state_out, gstate_out,
                         gk, gv, gw, gu, gstate_in, ckpt};
  e = wkv::launch_dd_backward(a, workspace, stream);
  return e == hipSuccess ? WKV_OK : fail(WKV_ERR_LAUNCH, e);
}

}  // namespace

extern "C" {

int wkv_backward(int64_t B, int64_t T, int64_t C, const float* w, const float* u, const float* k,
                 const float* v, const float* r, const float* state_in, const float* state_out,
                 const float* gstate_out, const float* gout, float* gk, float* gv, float* gr,
                 float* gw, float* gu, float* gstate_in, void* workspace,
                 int64_t workspace_bytes, hipStream_t stream) {
  return backward_impl(B, T, C, w, u, k, v, r, state_in, state_out, gstate_out, gout, gk, gv, gr,
                       gw, gu, gstate_in, workspace, workspace_bytes, stream);
}

int wkv_backward_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                      const float* k, const float* v, const float* r, const float* state_in,
                      const float* state_out, const float* gstate_out, const float* gout,
                      const float* ckpt, float* gk, float* gv, float* gr, float* gw, float* gu,
                      float* gstate_in, void* workspace, int64_t workspace_bytes,
                      hipStream_t stream) {
  if (ckpt == nullptr && B > 0 && T > 0 && C > 0) return WKV_ERR_NULL;
  return backward_impl(B, T, C, w, u, k, v, r, state_in, state_out, gstate_out, gout, gk, gv, gr,
                       gw, gu, gstate_in, workspace, workspace_bytes, stream, ckpt);
}

int64_t wkv_ckpt_bytes(int64_t B, int64_t T, int64_t C) {
  if (B < 0 || T < 0 || C < 0) return -WKV_ERR_DIM;
  const int64_t n = ckpt_bytes(B, T, C);
  return n < 0 ? -WKV_ERR_DIM : n;
}

int wkv_forward_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                     const float* k, const float* v, const float* r, const float* state_in,
                     float* out, float* state_out, float* ckpt, int path, hipStream_t stream) {
  if (path != WKV_PATH_AUTO && path != WKV_PATH_SEQ && path != WKV_PATH_CHUNK) return WKV_ERR_ARG;
  if (ckpt == nullptr && B > 0 && T > 0 && C > 0) return WKV_ERR_NULL;
  return forward_impl(B, T, C, w, u, k, v, r, r != nullptr, state_in, out, state_out, WKV_IO_F32,
                      path, nullptr, 0, stream, ckpt);
}

int64_t wkv_backward_workspace_size(int64_t B, int64_t T, int64_t C) {
  if (B < 0 || T < 0 || C < 0) return -WKV_ERR_DIM;
  int64_t cells;
  if (!mul3(B, T, C, &cells) || cells > kMaxBytes) return -WKV_ERR_DIM;
  if (C == 0) return 0;
  const int64_t n = wkv::backward_workspace_bytes(B, T, C);
  return n < 0 || n > kMaxBytes ? -WKV_ERR_DIM : n;
}

int wkv_backward_dd(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                    const float* k, const float* v, const float* state_in, const float* state_out,
                    const float* gstate_out, const float* gout, float* gk, float* gv, float* gw,
                    float* gu, float* gstate_in, void* workspace, int64_t workspace_bytes,
                    hipStream_t stream) {
  return backward_dd_impl(B, T, C, w, u, k, v, state_in, state_out, gstate_out, gout, gk, gv, gw,
                          gu, gstate_in, workspace, workspace_bytes, stream);
}

int wkv_forward_dd_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                        const float* k, const float* v, const float* state_in, float* out,
                        float* state_out, void* ckpt, int path, hipStream_t stream) {
  return forward_dd_impl(B, T, C, w, u, k, v, state_in, out, state_out, WKV_IO_F32, path, stream,
                         ckpt, true);
}

int wkv_backward_dd_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                         const float* k, const float* v, const float* state_in,
                         const float* state_out, const float* gstate_out, const float* gout,
                         const void* ckpt, float* gk, float* gv, float* gw, float* gu,
                         float* gstate_in, void* workspace, int64_t workspace_bytes,
                         hipStream_t stream) {
  return backward_dd_impl(B, T, C, w, u, k, v, state_in, state_out, gstate_out, gout, gk, gv, gw,
                          gu, gstate_in, workspace, workspace_bytes, stream, ckpt, true);
}

int64_t wkv_backward_dd_workspace_size(int64_t B, int64_t T, int64_t C) {
  if (B < 0 || T < 0 || C < 0) return -WKV_ERR_DIM;
  int64_t cells;
  if (!mul3(B, T, C, &cells) || cells > kMaxBytes) return -WKV_ERR_DIM;
  if (C == 0) return 0;
  const int64_t n = wkv::dd_backward_workspace_bytes(B, T, C);
  return n < 0 || n > kMaxBytes ? -WKV_ERR_DIM : n;
}


int wkv_forward(int64_t B, int64_t T, int64_t C, const float* w, const float* u, const float* k,
                const float* v, const float* state_in, float* out, float* state_out,
                hipStream_t stream) {
  return forward_impl(B, T, C, w, u, k, v, nullptr, false, state_in, out, state_out, WKV_IO_F32,
                      WKV_PATH_AUTO, nullptr, 0, stream);
}

int wkv_forward_bf16(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                     const uint16_t* k, const uint16_t* v, const float* state_in, uint16_t* out,
                     float* state_out, hipStream_t stream) {
  return forward_impl(B, T, C, w, u, k, v, nullptr, false, state_in, out, state_out, WKV_IO_BF16,
                      WKV_PATH_AUTO, nullptr, 0, stream);
}

int wkv_forward_ex(int64_t B, int64_t T, int64_t C, const float* w, const float* u, const void* k,
                   const void* v, const float* state_in, void* out, float* state_out, int io,
                   int path, hipStream_t stream) {
  return forward_impl(B, T, C, w, u, k, v, nullptr, false, state_in, out, state_out, io, path,
                      nullptr, 0, stream);
}

int wkv_forward_ws(int64_t B, int64_t T, int64_t C, const float* w, const float* u, const void* k,
                   const void* v, const float* state_in, void* out, float* state_out, int io,
                   int path, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return forward_impl(B, T, C, w, u, k, v, nullptr, false, state_in, out, state_out, io, path,
                      workspace, workspace_bytes, stream);
}

int wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                        const void* k, const void* v, const float* state_in, void* out,
                        float* state_out, int io, int path, hipStream_t stream) {
  if (io != WKV_IO_F32 && io != WKV_IO_BF16) return WKV_ERR_ARG;
  if (path < WKV_PATH_AUTO || path > WKV_PATH_LOOKBACK) return WKV_ERR_ARG;
  if (B < 0 || T < 0 || C < 0) return WKV_ERR_DIM;
  if (B == 0 || C == 0 || T == 0)
    return forward_impl(B, T, C, w, u, k, v, nullptr, false, state_in, out, state_out, io, path,
                        nullptr, 0, stream);
  // the scratch serves when the look-back scan runs and fits in it: an
  // explicit LOOKBACK beyond kScratchBytes is WKV_ERR_WORKSPACE, AUTO then
  // chooses among the kernels that need none
  int64_t seq;
  if (!mul3(B, T, C, &seq) || seq > kMaxBytes) return WKV_ERR_DIM;
  const int64_t need = lookback_bytes(io, B, T, C);
  if (path == WKV_PATH_LOOKBACK && need > kScratchBytes) return WKV_ERR_WORKSPACE;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, e);
  const bool fits = need <= kScratchBytes;
  const int chosen = path == WKV_PATH_AUTO ? choose_path(B, T, C, io, dev, fits, true) : path;
  if (chosen != WKV_PATH_LOOKBACK)
    return forward_impl(B, T, C, w, u, k, v, nullptr, false, state_in, out, state_out, io, chosen,
                        nullptr, 0, stream);
  void* ws = scratch_on(dev, &e);
  if (ws == nullptr) return fail(WKV_ERR_LAUNCH, e);
  // Calls may come with any sizes and in any order (HIP graph replays
  // included), so every look-back call starts from a zero-filled workspace:
  // the part of the array it uses is cleared first, in stream order, by a
  // kernel. Arguments are validated before anything is enqueued.
  const int pre = forward_impl(B, T, C, w, u, k, v, nullptr, false, state_in, out, state_out, io,
                               WKV_PATH_LOOKBACK, ws, kScratchBytes, stream, nullptr, true);
  if (pre != WKV_OK) return pre;
  e = wkv::launch_zero_fill(ws, (need + 15) / 16 * 16, stream);
  if (e != hipSuccess) return fail(WKV_ERR_LAUNCH, e);
  return forward_impl(B, T, C, w, u, k, v, nullptr, false, state_in, out, state_out, io,
                      WKV_PATH_LOOKBACK, ws, kScratchBytes, stream);
}

int wkv_forward_gated(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                      const void* k, const void* v, const void* r, const float* state_in,
                      void* out, float* state_out, int io, int path, void* workspace,
                      int64_t workspace_bytes, hipStream_t stream) {
  return forward_impl(B, T, C, w, u, k, v, r, true, state_in, out, state_out, io, path,
                      workspace, workspace_bytes, stream);
}

int wkv_forward_dd(int64_t B, int64_t T, int64_t C, const void* w, const float* u, const void* k,
                   const void* v, const float* state_in, void* out, float* state_out, int io,
                   int path, hipStream_t stream) {
  return forward_dd_impl(B, T, C, w, u, k, v, state_in, out, state_out, io, path, stream);
}

int wkv_step_dd(int64_t B, int64_t C, const void* w, const float* u, const void* k, const void* v,
                float* state, void* out, int io, hipStream_t stream) {
  return step_dd_impl(B, C, w, u, k, v, state, out, io, stream);
}

int wkv_matrix_forward(int64_t B, int64_t T, int64_t H, int64_t D, const float* w,
                       const float* k, const float* v, const float* r, const float* state_in,
                       float* out, float* state_out, void* workspace, int64_t workspace_bytes,
                       hipStream_t stream) {
  return matrix_forward_impl(B, T, H, D, w, k, v, r, state_in, out, state_out, workspace,
                             workspace_bytes, stream);
}

int64_t wkv_matrix_workspace_size(int64_t B, int64_t T, int64_t H, int64_t D) {
  if (B < 0 || T < 0 || H < 0 || D < 0) return -WKV_ERR_DIM;
  if (D != wkv::kMatrixHead || H > wkv::kMatrixMaxHeads) return -WKV_ERR_DIM;
  int64_t cells;
  if (!mul3(B, T, H * D, &cells) || cells > kMaxBytes) return -WKV_ERR_DIM;
  if (B == 0 || H == 0 || T == 0) return 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return -fail(WKV_ERR_DEVICE, e);
  const int64_t P = wkv::matrix_segments(B, T, H, cu_count(dev));
  return wkv::matrix_workspace_bytes(B, T, H, P);
}

int wkv_matrix_step(int64_t B, int64_t H, int64_t D, const float* w, const float* k,
                    const float* v, const float* r, float* state, float* out,
                    hipStream_t stream) {
  return matrix_step_impl(B, H, D, w, k, v, r, state, out, stream);
}

int64_t wkv_workspace_size(int64_t B, int64_t T, int64_t C, int io, int path) {
  if (io != WKV_IO_F32 && io != WKV_IO_BF16) return -WKV_ERR_ARG;
  if (path < WKV_PATH_AUTO || path > WKV_PATH_LOOKBACK) return -WKV_ERR_ARG;
  if (B < 0 || T < 0 || C < 0) return -WKV_ERR_DIM;
  int64_t cells;
  if (!mul3(B, T, C, &cells) || cells > kMaxBytes) return -WKV_ERR_DIM;
  if (B == 0 || C == 0 || T == 0) return 0;
  if (path == WKV_PATH_AUTO) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return -fail(WKV_ERR_DEVICE, e);
    path = choose_path(B, T, C, io, dev, true, true);
  }
  return path == WKV_PATH_LOOKBACK ? lookback_bytes(io, B, T, C) : 0;
}

int wkv_select_path(int64_t B, int64_t T, int64_t C, int io) {
  if (io != WKV_IO_F32 && io != WKV_IO_BF16) return -WKV_ERR_ARG;
  if (B < 0 || T < 0 || C < 0) return -WKV_ERR_DIM;
  int64_t n;
  if (!mul3(B, T, C, &n) || n > kMaxBytes / 4) return -WKV_ERR_DIM;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return -fail(WKV_ERR_DEVICE, e);
  return choose_path(B, T, C, io, dev, true, true);
}

int wkv_step(int64_t B, int64_t C, const float* w, const float* u, const float* k, const float* v,
             float* state, float* out, hipStream_t stream) {
  return step_impl(B, C, w, u, k, v, nullptr, false, state, out, WKV_IO_F32, stream);
}

int wkv_step_bf16(int64_t B, int64_t C, const float* w, const float* u, const uint16_t* k,
                  const uint16_t* v, float* state, uint16_t* out, hipStream_t stream) {
  return step_impl(B, C, w, u, k, v, nullptr, false, state, out, WKV_IO_BF16, stream);
}

int wkv_step_gated(int64_t B, int64_t C, const float* w, const float* u, const void* k,
                   const void* v, const void* r, float* state, void* out, int io,
                   hipStream_t stream) {
  if (io != WKV_IO_F32 && io != WKV_IO_BF16) return WKV_ERR_ARG;
  return step_impl(B, C, w, u, k, v, r, true, state, out, io, stream);
}

const char* wkv_status_string(int status) {
  switch (status) {
    case WKV_OK: return "WKV_OK";
    case WKV_ERR_NULL: return "WKV_ERR_NULL: a required pointer is NULL";
    case WKV_ERR_DIM: return "WKV_ERR_DIM: negative or too large size";
    case WKV_ERR_ALIGN: return "WKV_ERR_ALIGN: pointer not aligned to its element size";
    case WKV_ERR_ALIAS: return "WKV_ERR_ALIAS: an output overlaps another argument";
    case WKV_ERR_LAUNCH: return "WKV_ERR_LAUNCH: kernel launch failed";
    case WKV_ERR_DEVICE: return "WKV_ERR_DEVICE: no usable HIP device";
    case WKV_ERR_ARG: return "WKV_ERR_ARG: io or path out of range";
    case WKV_ERR_WORKSPACE: return "WKV_ERR_WORKSPACE: the kernel needs a (larger) workspace";
    case WKV_ERR_LOOKBACK:
      return "WKV_ERR_LOOKBACK: a look-back launch could not chain its segments; outputs past the "
             "failure are NaN or unwritten";
    default: return "unknown wkv_status";
  }
}

int wkv_workspace_status(void* workspace, int64_t workspace_bytes, int clear,
                         hipStream_t stream) {
  if (workspace == nullptr) return WKV_ERR_NULL;
  if (workspace_bytes < 16) return WKV_ERR_WORKSPACE;
  if (misaligned(workspace, 256)) return WKV_ERR_ALIGN;
  // the error word is the first 32-bit word of the workspace
  uint32_t err = 0;
  hipError_t e = hipMemcpyAsync(&err, workspace, sizeof(err), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(WKV_ERR_LAUNCH, e);
  if (err != 0 && clear != 0) {
    const uint32_t zero = 0;
    e = hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(WKV_ERR_LAUNCH, e);
  }
  return err != 0 ? WKV_ERR_LOOKBACK : WKV_OK;
}

int wkv_token_shift(int64_t B, int64_t T, int64_t C, int64_t P, const float* mu, const void* x,
                    const void* x_prev, void* out, void* x_last, int io, hipStream_t stream) {
  return shift_impl(B, T, C, P, mu, x, x_prev, out, x_last, io, stream);
}

int wkv_last_hip_error(void) { return g_last_hip_error; }

int wkv_abi_version(void) { return 1; }

}  // extern "C"
