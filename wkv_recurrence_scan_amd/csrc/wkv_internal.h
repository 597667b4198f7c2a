// Internal interface between the C-ABI layer (wkv_api.cpp) and the kernel
// translation units. Not installed; the public interface is include/wkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

enum Io : int { kF32 = 0, kBf16 = 1 };

// Tokens per checkpoint chunk of the backward pass (and of a prefill that
// saves its checkpoints for it).
constexpr int kCkptTokens = 8;

struct FwdArgs {
  int64_t B, T, C;
  const float* w;
  const float* u;
  const void* k;
  const void* v;
  const float* state_in;  // nullptr: empty state
  void* out;
  float* state_out;       // nullptr: not written
  const void* r = nullptr;  // receptance, like k; non-null: out = sigmoid(r) * wkv
  float* ckpt = nullptr;    // fp32 only: [ceil(T/8)][B*C] float4 states for the backward
};

struct StepArgs {
  int64_t B, C;
  const float* w;
  const float* u;
  const void* k;
  const void* v;
  float* state;
  void* out;
  const void* r = nullptr;  // receptance, like k; non-null: out = sigmoid(r) * wkv
};

// Channels per thread each kernel can be built for; the host picks the widest
// one that divides C and matches the pointers' alignment.
int seq_vec_width(int io, int64_t C, const FwdArgs& a);
int chunk_vec_width(int io, int64_t C, const FwdArgs& a);
int step_vec_width(int io, int64_t C, const StepArgs& a);

// Look-back scan: device workspace = control words, then the published
// per-(segment, channel) words. Zero-filled before first use; each launch
// leaves it ready for the next.
struct LbWorkspace {
  uint32_t* ctrl;  // start of the workspace
  int64_t bytes;   // its size
};
int lookback_vec_width(int io, int64_t C, const FwdArgs& a);
int64_t lookback_workspace_bytes(int vec, int64_t B, int64_t T, int64_t C);
hipError_t launch_lookback(const FwdArgs& a, int io, int vec, const LbWorkspace& ws, hipStream_t s);
// Zero-fills bytes (a multiple of 16) at p with a kernel on stream s.
hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t s);

// Backward pass (fp32): gradients for w, u, k, v and the initial state.
struct BwdArgs {
  int64_t B, T, C;
  const float* w;
  const float* u;
  const float* k;
  const float* v;
  const float* gout;
  const float* state_in;    // nullptr: empty initial state
  const float* state_out;   // with gstate_out: the forward's final state
  const float* gstate_out;  // nullptr: no gradient on the final state
  float* gk;
  float* gv;
  float* gw;                // [C], summed over the batch
  float* gu;                // [C]
  float* gstate_in;         // nullptr: not wanted
  const float* r = nullptr; // receptance of a gated output (out = sigmoid(r) * wkv)
  float* gr = nullptr;      // dL/dr, with r
  const float* ckpt = nullptr;  // the forward's checkpoints ([ceil(T/8)][B*C] float4), or nullptr
  int cus = 256;                // compute units of the device
};
// Workspace: per-lane partial sums and per-chunk checkpoints, written before
// they are read in every launch (no clearing needed).
int64_t backward_workspace_bytes(int64_t B, int64_t T, int64_t C);
hipError_t launch_backward(const BwdArgs& a, void* ws, hipStream_t s);

// Segments per lane of the backward passes for B*C lanes and T tokens (1: one
// thread per lane) and the checkpoint chunks per segment.
int64_t backward_segments(int64_t lanes, int64_t T, int64_t* seg_chunks);
// dL/du (and dL/dw when gw is not null) added over `rows` rows of C per-lane
// partial sums, in a fixed order; zero rows give zeros.
hipError_t launch_grad_reduce(int64_t rows, int64_t C, const float* gw_part, const float* gu_part,
                              float* gw, float* gu, hipStream_t s);

// Backward pass of the per-token-decay operator (fp32): w, k, v, gout, gk, gv
// and gw are [B][T][C]; gu is [C], summed over the batch.
struct DdBwdArgs {
  int64_t B, T, C;
  const float* w;
  const float* u;
  const float* k;
  const float* v;
  const float* gout;
  const float* state_in;    // nullptr: empty initial state
  const float* state_out;   // with gstate_out: the forward's final state
  const float* gstate_out;  // nullptr: no gradient on the final state
  float* gk;
  float* gv;
  float* gw;
  float* gu;
  float* gstate_in;         // nullptr: not wanted
  const void* ckpt = nullptr;  // the forward's checkpoints (see DdArgs), or nullptr
};
int64_t dd_backward_workspace_bytes(int64_t B, int64_t T, int64_t C);
hipError_t launch_dd_backward(const DdBwdArgs& a, void* ws, hipStream_t s);

// Per-token (data-dependent) decay: w has k's layout and element type.
struct DdArgs {
  int64_t B, T, C;
  const void* w;
  const float* u;
  const void* k;
  const void* v;
  const float* state_in;  // nullptr: empty state
  void* out;
  float* state_out;       // nullptr: not written
  void* ckpt = nullptr;   // fp32 only: [ceil(T/8)][B*C] states (n, d, fp64 m) for the backward
};
struct DdStepArgs {
  int64_t B, C;
  const void* w;          // this step's rates, [B][C]
  const float* u;
  const void* k;
  const void* v;
  float* state;
  void* out;
};
int dd_vec_width(int io, int64_t C, const DdArgs& a);
int dd_step_vec_width(int io, int64_t C, const DdStepArgs& a);
hipError_t launch_dd_seq(const DdArgs& a, int io, int vec, hipStream_t s);
hipError_t launch_dd_chunk(const DdArgs& a, int io, int vec, int cus, hipStream_t s);
hipError_t launch_dd_step(const DdStepArgs& a, int io, int vec, hipStream_t s);

// Matrix-valued state (head size 64, fp32): r, k, v, lam, out [B][T][H*64];
// states [B][H][64][64].
struct MatrixArgs {
  int64_t B, T, H;
  const float* lam;
  const float* k;
  const float* v;
  const float* r;
  const float* state_in;  // nullptr: zero state
  float* out;
  float* state_out;       // nullptr: not written
};
struct MatrixStepArgs {
  int64_t B, H;
  const float* lam;
  const float* k;
  const float* v;
  const float* r;
  float* state;
  float* out;
};
constexpr int64_t kMatrixHead = 64;
// the prefill kernels address 16 token rows of H * 64 channels with 32-bit offsets
constexpr int64_t kMatrixMaxHeads = int64_t{1} << 22;
int64_t matrix_segments(int64_t B, int64_t T, int64_t H, int cus);
int64_t matrix_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t P);
hipError_t launch_matrix(const MatrixArgs& m, int64_t P, void* ws, hipStream_t s);
hipError_t launch_matrix_step(const MatrixStepArgs& m, hipStream_t s);
// T == 0: state_out <- state_in, or zeros when state_in is null.
hipError_t launch_matrix_state_copy(int64_t B, int64_t H, const float* src, float* dst,
                                    hipStream_t s);

// Token shift: out[p][b][t][c] = x[b][t][c] + (x[b][t-1][c] - x[b][t][c]) * mu[p][c],
// x[b][-1] = x_prev[b] (zeros when null); x_last[b] <- x[b][T-1] (may be x_prev).
struct ShiftArgs {
  int64_t B, T, C, P;
  const float* mu;     // [P][C]
  const void* x;       // [B][T][C]
  const void* x_prev;  // [B][C] or nullptr
  void* out;           // [P][B][T][C]
  void* x_last;        // [B][C] or nullptr
};
constexpr int64_t kShiftMaxP = 8;
hipError_t launch_shift(const ShiftArgs& a, int io, hipStream_t s);

hipError_t launch_seq(const FwdArgs& a, int io, int vec, hipStream_t s);
// cus: compute units of the device (the two-walker kernel serves grids that
// give each workgroup a CU of its own)
hipError_t launch_chunk(const FwdArgs& a, int io, int vec, int cus, hipStream_t s);
hipError_t launch_step(const StepArgs& a, int io, int vec, hipStream_t s);
// T == 0: state_out <- state_in, or the empty state when state_in is null.
hipError_t launch_state_copy(int64_t B, int64_t C, const float* state_in, float* state_out,
                             hipStream_t s);

}  // namespace wkv
