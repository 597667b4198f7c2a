/*
 * wkv.h -- C interface of libwkv: the RWKV weighted-key-value (WKV) operator
 * on AMD MI355X (gfx950), prefill and decode.
 *
 * The operator
 * ------------
 * Defined on the page "Linear attention without writing a CUDA kernel",
 * section "The recurrence" (the wkv_t equation): for every channel c of every
 * sequence b independently, the output at position t is a weighted mean of the
 * values seen so far,
 *
 *     out_t = ( sum_{i<t} e^{k_i - (t-1-i) w} v_i + e^{u + k_t} v_t )
 *           / ( sum_{i<t} e^{k_i - (t-1-i) w}     + e^{u + k_t}     )
 *
 * where w > 0 is the channel's decay rate (each step back in time costs a
 * factor e^{-w}; the newest past token is not decayed) and u is the channel's
 * bonus for the current token. The same section carries the sums forward as a
 * state (num, den, max_exp): the true sums are num * e^{max_exp} and
 * den * e^{max_exp}, kept relative to a running maximum exponent the way a
 * stable softmax is. A step outputs from the state as it stands plus the bonus
 * term, then decays the state by e^{-w} and adds the current token (no bonus).
 *
 * Memory layout and ownership
 * ---------------------------
 * All array arguments are HIP device pointers owned by the caller; the library
 * allocates no device memory and keeps no state between calls apart from a
 * once-per-device property query. Row-major, C fastest:
 *   k, v, out : [B][T][C]  (wkv_step: [B][C])   fp32, or bf16 in the _bf16 calls
 *   w, u      : [C] fp32
 *   state     : [3][B][C] fp32, three planes num, den, max_exp.
 * The empty state (before any token) is num = den = 0, max_exp = -1e38; use
 * that, not -inf. A state passed in need not be normalised: any (n, d, m) with
 * d > 0 describes the sums n e^m, d e^m.
 *
 * Calls are asynchronous: they validate arguments, enqueue kernels on `stream`
 * (0 = the null stream) and return. Device-side faults surface at the caller's
 * next synchronisation. Every call is thread-safe. Inputs are not modified
 * except `state` of wkv_step, which is updated in place.
 *
 * Value preconditions (not checked on the device): w > 0 and finite; k, u
 * finite; v finite. Keys of any finite size are handled (the state is
 * rescaled against its running maximum); NaN/Inf inputs give unspecified
 * results.
 *
 * Errors
 * ------
 * Every entry point returns WKV_OK (0) or one of the wkv_status codes below;
 * on error nothing has been enqueued. wkv_status_string() names a code.
 */
#ifndef WKV_H_
#define WKV_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wkv_status {
  WKV_OK = 0,
  WKV_ERR_NULL = 1,   /* a required pointer is NULL                              */
  WKV_ERR_DIM = 2,    /* negative size, or B*T*C (in bytes) does not fit 63 bits  */
  WKV_ERR_ALIGN = 3,  /* a pointer is not aligned to its element size             */
  WKV_ERR_ALIAS = 4,  /* an output overlaps an input or another output            */
  WKV_ERR_LAUNCH = 5, /* the kernel launch failed (see wkv_last_hip_error)        */
  WKV_ERR_DEVICE = 6, /* no usable HIP device is current                          */
  WKV_ERR_ARG = 7,    /* an enumerated argument (io, path) is out of range        */
  WKV_ERR_WORKSPACE = 8, /* the kernel needs a workspace: missing or too small    */
  WKV_ERR_LOOKBACK = 9  /* reported by wkv_workspace_status only: a LOOKBACK launch
                           could not chain its segments (see there)                */
} wkv_status;

/* Element type of k, v and out (w, u and the state are always fp32). */
enum { WKV_IO_F32 = 0, WKV_IO_BF16 = 1 };

/* Prefill kernels; all compute the same function and may differ in the last
 * bits. SEQ: one lane per (b, c) walks the sequence (large B*C). CHUNK: one
 * workgroup per channel group walks the sequence in tiles, scanning
 * sub-chunks in parallel (small B*C, no workspace). LOOKBACK: every
 * (sequence segment, channel group) is its own workgroup, chained by a
 * decoupled look-back through a device workspace (small B*C, most
 * parallelism). AUTO picks SEQ when B*C alone fills the GPU, otherwise CHUNK
 * up to T = 2048 and, for longer sequences, LOOKBACK when a workspace is
 * given (CHUNK when not); the plain (ungated, no checkpoints) fp32 forward
 * also takes CHUNK where B*C fills the GPU, 512 <= T <= 2048 and a batch
 * row's T * C * 4 bytes are not a power of two; with a workspace, fp32 takes
 * LOOKBACK from T = 513 (gated: T = 1280) to 2048 where the 32-channel
 * groups, B * ceil(C / 32), number more than the CUs and at most four times
 * as many (see wkv_select_path). */
enum { WKV_PATH_AUTO = 0, WKV_PATH_SEQ = 1, WKV_PATH_CHUNK = 2, WKV_PATH_LOOKBACK = 3 };

/* Prefill / training form over a whole sequence (page "Linear attention
 * without writing a CUDA kernel", section "The recurrence", wkv_t equation).
 *
 *   B, T, C    sizes (>= 0). B == 0 or C == 0: nothing to do, WKV_OK.
 *              T == 0: state_out receives state_in (or the empty state).
 *   w, u       [C] fp32 decay rate (> 0) and current-token bonus.
 *   k, v       [B][T][C] fp32 keys and values.
 *   state_in   [3][B][C] state before token 0, or NULL for the empty state.
 *   out        [B][T][C] fp32 outputs, written for every position.
 *   state_out  [3][B][C] state after token T-1 (inclusive: the next step's
 *              output uses it as it stands), or NULL to skip it. May be the
 *              same pointer as state_in (read before written, per lane); any
 *              other overlap with an input is WKV_ERR_ALIAS, as is any overlap
 *              of out with another argument.
 *   stream     HIP stream to enqueue on (0: null stream).
 */
int wkv_forward(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                const float* k, const float* v, const float* state_in, float* out,
                float* state_out, hipStream_t stream);

/* As wkv_forward with k, v, out in bf16 (raw 16-bit patterns). Inputs are
 * widened exactly to fp32; all arithmetic and the state are fp32; outputs are
 * rounded to the nearest bf16 (ties to even). */
int wkv_forward_bf16(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                     const uint16_t* k, const uint16_t* v, const float* state_in,
                     uint16_t* out, float* state_out, hipStream_t stream);

/* As wkv_forward / wkv_forward_bf16 with the element type (WKV_IO_*) and the
 * prefill kernel (WKV_PATH_*) chosen by the caller; k, v, out point to
 * elements of that type. */
int wkv_forward_ex(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                   const void* k, const void* v, const float* state_in, void* out,
                   float* state_out, int io, int path, hipStream_t stream);

/* As wkv_forward_ex with a device workspace, which the LOOKBACK kernel needs
 * (and AUTO then may choose).
 *   workspace        device memory of at least wkv_workspace_size(...) bytes,
 *                    256-byte aligned, owned by the caller. It must be
 *                    zero-filled before its first use, and again before it
 *                    serves a call with another look-back layout (the layout
 *                    follows from B, T and C, the element type, whether the
 *                    bf16 pointers allow two channels per thread and, past
 *                    2048 tokens, whether the call is gated); every call
 *                    leaves it ready for the next call with the same layout
 *                    (no clearing in between, HIP graph replays included).
 *                    Under AUTO this applies to every call that takes
 *                    LOOKBACK (wkv_select_path), fp32 calls from 513 tokens
 *                    included: a caller that varies B, T or C with one
 *                    workspace zero-fills it when the layout changes, or
 *                    keeps one workspace per shape.
 *                    Calls that may run concurrently must not share a
 *                    workspace. It must not overlap any other argument.
 *   workspace_bytes  its size in bytes.
 * A call whose kernel needs no workspace ignores it (it may be NULL).
 *
 * Misuse is reported, never silent: the first LOOKBACK launch on a
 * zero-filled workspace claims it for its layout, and a later launch with
 * another layout (see above) on the same, uncleared workspace, or a wait
 * for an earlier segment that runs out (as when overlapping calls share a
 * workspace), sets the workspace's error word and writes NaN where the
 * missing data would have gone, so the affected outputs are NaN rather than
 * plausible values. wkv_workspace_status reads the word. Layout of the
 * first 16 bytes (32-bit words): [0] the error word (bit 0: a wait ran out;
 * bit 2: another layout's claim), [1] zero in normal use (tests set bit 0,
 * "publish nothing", and a smaller bound on each wait in bits 8-31, to force
 * the failure path), [2..3] the layout claim. */
int wkv_forward_ws(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                   const void* k, const void* v, const float* state_in, void* out,
                   float* state_out, int io, int path, void* workspace,
                   int64_t workspace_bytes, hipStream_t stream);

/* Reads the error word of a workspace used by wkv_forward_ws (and friends)
 * after the work enqueued on `stream` so far has finished: waits for the
 * stream, then returns WKV_OK if no LOOKBACK launch with this workspace ever
 * failed to chain its segments (since the word was last cleared), or
 * WKV_ERR_LOOKBACK if one did; with clear != 0 the word is then reset to 0.
 * Blocking (it synchronises the stream), so not for use under HIP graph
 * capture. WKV_ERR_NULL / WKV_ERR_WORKSPACE (fewer than 16 bytes) /
 * WKV_ERR_ALIGN (not 256-byte aligned) for a bad workspace argument,
 * WKV_ERR_LAUNCH if the copy or the synchronisation fails. */
int wkv_workspace_status(void* workspace, int64_t workspace_bytes, int clear,
                         hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): as
 * wkv_forward_ws without the workspace argument. The look-back scan's
 * workspace is instead a static device array inside the library, 32 MiB per
 * device (held from the library's load to the end of the process), found with
 * hipGetSymbolAddress on the first call on each device. No call allocates
 * memory. Since calls may come with any sizes and in any order (graph
 * replays included), every call that runs the look-back scan first enqueues
 * a kernel that zero-fills the part of the array it will use (the scan's
 * workspace size), then the scan.
 *   path LOOKBACK whose workspace (wkv_workspace_size) exceeds 32 MiB:
 *        WKV_ERR_WORKSPACE. AUTO uses the array when its choice is the
 *        look-back scan and it fits, and otherwise picks among the kernels
 *        that need no workspace; SEQ and CHUNK never touch it.
 * Every call on one device shares that device's array: calls that may
 * overlap in time on one device (other streams, other threads) race on it
 * and must not be made; calls in order on one stream are fine, with any
 * sizes. Other arguments, layout and errors as wkv_forward_ws. */
int wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                        const void* k, const void* v, const float* state_in, void* out,
                        float* state_out, int io, int path, hipStream_t stream);

/* As wkv_forward_ws with the output gated by the receptance:
 * out_t = sigmoid(r_t) * wkv_t per element (page "RWKV-v6 Architecture:
 * Attention-Free Linear Transformers", the output equation of its recurrence;
 * page "RWKV: Merging Transformer Training with RNN Speed", Time-Mixing
 * block). r: [B][T][C] of the element type io, required when T > 0; it must
 * not overlap out or state_out. state_out is the ungated state. */
int wkv_forward_gated(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                      const void* k, const void* v, const void* r, const float* state_in,
                      void* out, float* state_out, int io, int path, void* workspace,
                      int64_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace wkv_forward_ws (or wkv_forward_gated) needs for these
 * sizes and this path (0 when the kernel uses none; enough for either form
 * and either channel width the pointers may allow), or a negative
 * wkv_status on error. */
int64_t wkv_workspace_size(int64_t B, int64_t T, int64_t C, int io, int path);

/* The kernel WKV_PATH_AUTO uses for these sizes on the current device when a
 * workspace is available (WKV_PATH_SEQ, WKV_PATH_CHUNK or WKV_PATH_LOOKBACK;
 * without one, LOOKBACK becomes WKV_PATH_CHUNK), or a negative wkv_status on
 * error. This is the plain forward's choice; the gated, checkpointing and
 * per-token-decay forms differ in two cases: where B*C alone fills the GPU they
 * always take WKV_PATH_SEQ, while the plain fp32 forward takes WKV_PATH_CHUNK
 * for 512 <= T <= 2048 when a batch row's T * C * 4 bytes are not a power of
 * two; and where the plain fp32 forward with a workspace takes
 * WKV_PATH_LOOKBACK below T = 2049 (513 <= T, more 32-channel groups than
 * CUs, at most four per CU), the gated one does so from T = 1280 only, and
 * the checkpointing and per-token-decay forms, which have no look-back
 * kernel, take WKV_PATH_CHUNK. */
int wkv_select_path(int64_t B, int64_t T, int64_t C, int io);

/* One decode step for B sequences at once (page "Linear attention without
 * writing a CUDA kernel", section "The recurrence", the step function that
 * carries num, den and max_exp).
 *
 *   B, C       sizes (>= 0); zero is a no-op.
 *   w, u       [C] fp32.
 *   k, v       [B][C] fp32, the current token.
 *   state      [3][B][C] fp32, read and then overwritten with the state after
 *              this token.
 *   out        [B][C] fp32 output for this token. Must not overlap any other
 *              argument.
 */
int wkv_step(int64_t B, int64_t C, const float* w, const float* u, const float* k,
             const float* v, float* state, float* out, hipStream_t stream);

/* As wkv_step with k, v, out in bf16; state stays fp32. */
int wkv_step_bf16(int64_t B, int64_t C, const float* w, const float* u, const uint16_t* k,
                  const uint16_t* v, float* state, uint16_t* out, hipStream_t stream);

/* Backward pass of the prefill (fp32): gradients of a loss L with respect to
 * w, u, k, v, the receptance r of a gated output and the initial state, given
 * dL/dout and optionally dL/dstate_out. The derivatives are those of the
 * wkv_t ratio of the page "Linear attention without writing a CUDA kernel",
 * section "The recurrence" (quotient rule over its terms; the page trains its
 * model through this operator), times the gate sigmoid(r) when there is one.
 *
 *   B, T, C     sizes (>= 0). C == 0: nothing to do. B == 0: gw, gu zeroed.
 *   w, u        [C] the forward's decay and bonus.
 *   k, v        [B][T][C] the forward's keys and values.
 *   r           [B][T][C] the receptance of wkv_forward_gated, or NULL for an
 *               ungated output.
 *   state_in    [3][B][C] the forward's initial state, or NULL (empty state).
 *   state_out,  [3][B][C] the state the forward returned and dL/d(num, den,
 *   gstate_out  max_exp) of it, both or neither (NULL: no gradient on the final
 *               state). The final state's gradient is taken through num and
 *               den at the given max_exp; the max_exp plane of gstate_out is
 *               not read (for a loss of the state itself it equals
 *               num * g_num + den * g_den).
 *   gout        [B][T][C] dL/dout (of the gated output when r is given).
 *   gk, gv      [B][T][C] out: dL/dk, dL/dv.
 *   gr          [B][T][C] out: dL/dr; required with r, ignored without.
 *   gw, gu      [C] out: dL/dw, dL/du summed over the batch.
 *   gstate_in   [3][B][C] out: dL/d(num, den, max_exp) of state_in (zeros when
 *               state_in is NULL), or NULL to skip it.
 *   workspace   device memory of wkv_backward_workspace_size(B, T, C) bytes,
 *               256-byte aligned, owned by the caller; contents need no
 *               clearing (everything read is written first in the same
 *               call). Must not overlap any other argument; calls that may
 *               run concurrently must not share it.
 * Outputs must not overlap any input or each other (WKV_ERR_ALIAS). The
 * result is deterministic (fixed-order sums). */
int wkv_backward(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                 const float* k, const float* v, const float* r, const float* state_in,
                 const float* state_out, const float* gstate_out, const float* gout,
                 float* gk, float* gv, float* gr, float* gw, float* gu, float* gstate_in,
                 void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace wkv_backward needs for these sizes, or a negative
 * wkv_status on error. */
int64_t wkv_backward_workspace_size(int64_t B, int64_t T, int64_t C);

/* Training pair for the prefill (fp32): a forward that saves, and a backward
 * that takes, the state in front of every chunk of 8 tokens of every lane.
 * The backward then skips its own re-run of the forward to rebuild those
 * states (for large B*C one of its two passes over k and v; for small B*C its
 * segment summaries and their folds). Same operator, derivatives and
 * conventions as wkv_forward_gated / wkv_backward.
 *
 * wkv_ckpt_bytes: size of ckpt for these sizes, ceil(T / 8) * B * C * 16
 * bytes, or a negative wkv_status.
 *
 * wkv_forward_ckpt: as wkv_forward_gated (r NULL: ungated output) with
 *   ckpt   out: [ceil(T / 8)][B][C] float4 (num, den, base, age), the lane
 *          state in front of token 8j at [j][b][c], the maximum exponent kept
 *          as base - age * w; 16-byte aligned, wkv_ckpt_bytes bytes, owned by
 *          the caller; must not overlap any other argument. Required when
 *          B, T, C > 0 (WKV_ERR_NULL).
 *   path   WKV_PATH_AUTO, WKV_PATH_SEQ or WKV_PATH_CHUNK (the look-back scan
 *          saves no checkpoints: WKV_PATH_LOOKBACK gives WKV_ERR_ARG). The
 *          outputs equal those of the same kernel without checkpoints bit
 *          for bit.
 *
 * wkv_backward_ckpt: as wkv_backward with
 *   ckpt   [ceil(T / 8)][B][C] float4, what wkv_forward_ckpt wrote for the
 *          same w, u, k, v and state_in (checkpoints of other inputs give
 *          wrong gradients; this is not detected); 16-byte aligned, read
 *          only; required when B, T, C > 0. The workspace is as for
 *          wkv_backward (wkv_backward_workspace_size). */
int64_t wkv_ckpt_bytes(int64_t B, int64_t T, int64_t C);
int wkv_forward_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                     const float* k, const float* v, const float* r, const float* state_in,
                     float* out, float* state_out, float* ckpt, int path, hipStream_t stream);
int wkv_backward_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                      const float* k, const float* v, const float* r, const float* state_in,
                      const float* state_out, const float* gstate_out, const float* gout,
                      const float* ckpt, float* gk, float* gv, float* gr, float* gw, float* gu,
                      float* gstate_in, void* workspace, int64_t workspace_bytes,
                      hipStream_t stream);

/* One decode step with the gated output, out = sigmoid(r) * wkv (see
 * wkv_forward_gated); k, v, r, out of element type io ([B][C]); the state is
 * fp32 and ungated. */
int wkv_step_gated(int64_t B, int64_t C, const float* w, const float* u, const void* k,
                   const void* v, const void* r, float* state, void* out, int io,
                   hipStream_t stream);

/* Prefill with a per-token (data-dependent) decay (page "RWKV-v6
 * Architecture: Attention-Free Linear Transformers", section "The Core
 * Components of the RWKV-v6 Time-Mixing Block", items on the dynamic
 * data-dependent decay and the matrix-valued state: step t decays the state
 * carried in from step t-1 before its own term is added). Step t multiplies
 * the state by e^(-w[b][t][c]); the output uses the state before that decay
 * plus the current token at e^(u + k), as in wkv_forward. With w[b][t][c] = w[c]
 * for every t this is wkv_forward.
 *
 *   w          [B][T][C] positive rates, element type io (like k), required
 *              when T > 0. It must not overlap out or state_out.
 *   u, k, v, state_in, out, state_out, io, stream: as wkv_forward_ex.
 *   path       WKV_PATH_AUTO, WKV_PATH_SEQ or WKV_PATH_CHUNK (no look-back
 *              kernel for this operator: WKV_PATH_LOOKBACK gives WKV_ERR_ARG).
 * Running maxima and accumulated rates are carried in fp64 inside the
 * kernels (the per-token rate rules out the constant-decay kernels' exact
 * integer ages); everything else is fp32. */
int wkv_forward_dd(int64_t B, int64_t T, int64_t C, const void* w, const float* u,
                   const void* k, const void* v, const float* state_in, void* out,
                   float* state_out, int io, int path, hipStream_t stream);

/* One decode step with this step's own rates w ([B][C], element type io, like
 * k): out = the state mixed with the token at e^(u + k); then the state decays
 * by e^(-w) and the token is added at e^k. k, v, out of element type io; the
 * state is fp32, updated in place. Overlaps as wkv_step. */
int wkv_step_dd(int64_t B, int64_t C, const void* w, const float* u, const void* k,
                const void* v, float* state, void* out, int io, hipStream_t stream);

/* Gradients of the per-token-decay prefill (fp32): dL/dw for every rate,
 * dL/du, dL/dk, dL/dv and dL/dstate_in from dL/dout and optionally
 * dL/dstate_out. The derivatives are those of wkv_forward_dd's operator (the
 * per-token decay of the page "RWKV-v6 Architecture: Attention-Free Linear
 * Transformers", section "The Core Components of the RWKV-v6 Time-Mixing
 * Block", on the wkv_t ratio of the page "Linear attention without writing
 * a CUDA kernel", section "The recurrence"); a rate w[b][t][c] decays
 * every earlier token's term in the outputs after step t.
 *
 *   w           [B][T][C] fp32 the forward's rates; u [C] its bonus.
 *   k, v, gout  [B][T][C] fp32 keys, values and dL/dout.
 *   state_in, state_out, gstate_out, gstate_in: as wkv_backward.
 *   gk, gv, gw  [B][T][C] out: dL/dk, dL/dv, dL/dw.
 *   gu          [C] out: dL/du summed over the batch.
 *   workspace   wkv_backward_dd_workspace_size(B, T, C) bytes, 256-byte
 *               aligned, owned by the caller, no clearing needed; calls that
 *               may run concurrently must not share it.
 * Sizes, errors and overlap rules as wkv_backward; deterministic. */
int wkv_backward_dd(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                    const float* k, const float* v, const float* state_in, const float* state_out,
                    const float* gstate_out, const float* gout, float* gk, float* gv, float* gw,
                    float* gu, float* gstate_in, void* workspace, int64_t workspace_bytes,
                    hipStream_t stream);

/* Bytes of workspace wkv_backward_dd needs for these sizes, or a negative
 * wkv_status on error. */
int64_t wkv_backward_dd_workspace_size(int64_t B, int64_t T, int64_t C);

/* Training pair for the per-token-decay prefill (fp32), as wkv_forward_ckpt /
 * wkv_backward_ckpt for the constant decay: the forward saves the state in
 * front of every chunk of 8 tokens, and the backward starts from those
 * states instead of re-running the forward to rebuild them.
 *
 * wkv_forward_dd_ckpt: as wkv_forward_dd (fp32 only) with
 *   ckpt   out: [ceil(T / 8)][B][C] records of 16 bytes (float num, float
 *          den, double max_exp), the lane state in front of token 8j at
 *          [j][b][c]; wkv_ckpt_bytes(B, T, C) bytes, 16-byte aligned, owned
 *          by the caller; must not overlap any other argument. Required when
 *          B, T, C > 0 (WKV_ERR_NULL). The outputs equal those of
 *          wkv_forward_dd on the same path bit for bit.
 * wkv_backward_dd_ckpt: as wkv_backward_dd with ckpt, what
 *   wkv_forward_dd_ckpt wrote for the same w, u, k, v and state_in (other
 *   checkpoints give wrong gradients; this is not detected); read only. The
 *   workspace is as for wkv_backward_dd. */
int wkv_forward_dd_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                        const float* k, const float* v, const float* state_in, float* out,
                        float* state_out, void* ckpt, int path, hipStream_t stream);
int wkv_backward_dd_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                         const float* k, const float* v, const float* state_in,
                         const float* state_out, const float* gstate_out, const float* gout,
                         const void* ckpt, float* gk, float* gv, float* gw, float* gu,
                         float* gstate_in, void* workspace, int64_t workspace_bytes,
                         hipStream_t stream);

/* Matrix-valued-state recurrence (page "RWKV-v6 Architecture: Attention-Free
 * Linear Transformers", section "The Core Components of the RWKV-v6
 * Time-Mixing Block", item "Matrix-Valued Hidden State", and the step
 * function of its PyTorch listing). Per head of D channels a D x D state:
 *   S_t[i][j] = e^(-w_t[i]) S_{t-1}[i][j] + k_t[i] v_t[j]
 *   out_t[i]  = sigmoid(r_t[i]) * sum_j S_t[i][j] k_t[j]
 * with channel c = h * D + i. fp32 throughout.
 *
 *   B, T, H     sizes (>= 0); B == 0 or H == 0: nothing to do; H above
 *               2^22 heads: WKV_ERR_DIM.
 *   D           head size; only 64 is built (other values: WKV_ERR_DIM).
 *   w           [B][T][H*D] positive decay rates (the factor is e^(-w)).
 *   k, v, r     [B][T][H*D] key, value, receptance.
 *   state_in    [B][H][D][D] (row i, column j), or NULL for the zero state.
 *   out         [B][T][H*D].
 *   state_out   [B][H][D][D] state after the last token, or NULL; may equal
 *               state_in exactly.
 *   workspace   optional device memory, 256-byte aligned, of up to
 *               wkv_matrix_workspace_size(...) bytes; contents need no
 *               clearing. With less (or NULL) the kernel cuts the sequence
 *               into fewer segments (none without one): same result up to
 *               rounding, less parallelism. Must not overlap any other
 *               argument; concurrent calls must not share it.
 * Pointers to 8-byte-aligned sequences, 16-byte-aligned states. out and
 * state_out must not overlap an input (WKV_ERR_ALIAS). T == 0 copies the
 * state through (or zero-fills state_out). */
int wkv_matrix_forward(int64_t B, int64_t T, int64_t H, int64_t D, const float* w,
                       const float* k, const float* v, const float* r, const float* state_in,
                       float* out, float* state_out, void* workspace, int64_t workspace_bytes,
                       hipStream_t stream);

/* Bytes of workspace that lets wkv_matrix_forward use all the segments it
 * wants for these sizes on the current device (0: it needs none), or a
 * negative wkv_status. */
int64_t wkv_matrix_workspace_size(int64_t B, int64_t T, int64_t H, int64_t D);

/* One decode step of the matrix-valued-state recurrence for all (batch,
 * head) pairs: w, k, v, r, out [B][H*D] fp32 (one token), state [B][H][D][D]
 * fp32 updated in place; D == 64. */
int wkv_matrix_step(int64_t B, int64_t H, int64_t D, const float* w, const float* k,
                    const float* v, const float* r, float* state, float* out,
                    hipStream_t stream);

/* Static, NUL-terminated name of a wkv_status code. */
/* Token shift, the step in front of the projections whose outputs feed the
 * WKV operator (page "RWKV-v6 Architecture: Attention-Free Linear
 * Transformers", section "The Core Components of the RWKV-v6 Time-Mixing
 * Block", item 1, Data-Dependent Token Shift; page "RWKV: Merging
 * Transformer Training with RNN Speed", Time-Mixing block): for every
 * projection p, the input is the current token vector moved towards the one
 * before it by a per-channel fraction,
 *
 *     out[p][b][t][c] = x[b][t][c] + (x[b][t-1][c] - x[b][t][c]) * mu[p][c].
 *
 *   B, T, C    sizes (>= 0): batch rows, tokens, channels. B == 0 or C == 0:
 *              nothing to do. T == 0: x_last receives x_prev (or zeros).
 *   P          projections, 1 <= P <= 8 (WKV_ERR_DIM otherwise).
 *   mu         [P][C] fp32 mixing fractions, one vector per projection.
 *   x          [B][T][C] token vectors (fp32, or bf16 with io = WKV_IO_BF16).
 *   x_prev     [B][C] the token before x[b][0] (the previous call's last), or
 *              NULL for zeros (the start of a sequence).
 *   out        [P][B][T][C] the P mixes, one [B][T][C] block per projection,
 *              same element type as x (bf16: rounded to nearest even from the
 *              fp32 result of one fused multiply-add).
 *   x_last     [B][C] receives x[b][T-1], the next call's x_prev, or NULL to
 *              skip it. May be the same pointer as x_prev (decode: T = 1, the
 *              carried token updated in place); any other overlap of x_last or
 *              out with an argument is WKV_ERR_ALIAS.
 *   io         WKV_IO_F32 or WKV_IO_BF16 (WKV_ERR_ARG otherwise).
 * Asynchronous on `stream` like every call here. */
int wkv_token_shift(int64_t B, int64_t T, int64_t C, int64_t P, const float* mu, const void* x,
                    const void* x_prev, void* out, void* x_last, int io, hipStream_t stream);

const char* wkv_status_string(int status);

/* hipError_t of the last WKV_ERR_LAUNCH / WKV_ERR_DEVICE returned on the
 * calling thread (0 if none). */
int wkv_last_hip_error(void);

/* Interface version; bumped on any incompatible change of this header. */
int wkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WKV_H_ */
