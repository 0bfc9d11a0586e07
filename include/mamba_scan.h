/*
 * mamba_scan.h -- C ABI of libmamba_scan: Mamba's selective state-space scan (S6) and its
 * one-token recurrent step on AMD Instinct MI355X (gfx950).
 *
 * The operation (Mamba paper, Section 3 "Selective State Space Models" / Algorithm 2, as
 * restated on the Keras/TensorFlow Mamba tutorial page in its `selective_scan` and
 * `MambaBlock.ssm` code, and on the upstream mamba README under "Selective SSM"):
 * for every batch b, channel d and state n,
 *     delta_t   = softplus(delta_raw_t + delta_bias[d])        (or without softplus)
 *     Abar_t    = exp(delta_t * A[d, n])
 *     h_t[n]    = Abar_t * h_{t-1}[n] + delta_t * B[b, n, t] * u_t      (h_0 = 0)
 *     y_t       = sum_n C[b, n, t] * h_t[n] + D[d] * u_t
 *     out_t     = y_t * silu(z_t)                              (when z is given)
 * The input term is the Euler form delta * B * u, the form the tutorial's code computes;
 * silu(v) = v / (1 + e^-v).
 *
 * Conventions shared by every entry point
 *   - Tensors are passed as mss_tensor_t descriptors of DEVICE memory on the current HIP
 *     device.  The caller allocates and owns every buffer; the library never frees or
 *     keeps user memory.  Layout must be dense row-major (last stride 1, every other
 *     stride the product of the later extents), strides counted in elements, and data
 *     aligned to its element size.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream) and return
 *     as soon as the work is queued.  Kernel faults surface at the caller's next
 *     synchronisation.  Every argument is validated before any HIP call is made, so an
 *     invalid call never touches the device.
 *   - Return value: MSS_OK (0) or a negative mss_status_t; mss_status_string() names it.
 *     No C++ exception crosses the ABI.
 *   - The forward and backward scans split their work across wavefronts and carry state
 *     between the parts through a library-owned device workspace per (device, stream; for
 *     hipStreamPerThread also per host thread), allocated with hipMalloc on first need.  Calls
 *     on one stream are ordered, so they never share it concurrently.  When a later call needs
 *     more room, a larger buffer replaces it; the old one is kept (not freed) until
 *     mss_release_workspaces(), because a HIP graph captured earlier may still hold its address.
 *     Under stream capture nothing can be allocated: if the stream's workspace is too small the
 *     call returns MSS_ERR_UNSUPPORTED, so make one call of at least the same size on the
 *     capturing stream first.  A captured graph holds the workspace's address, so its replays
 *     must not overlap other calls on that stream.  No entry point records a memset: scratch is
 *     cleared by kernels.  (The forward's workspace does not depend on the problem size: 17
 *     floats per row of a 64-row wavefront, 4352 bytes per wavefront of one round of
 *     wavefronts, 13.4 MB on a 256-CU device.)
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSS_VERSION 20000 /* major * 10000 + minor * 100 + patch */

typedef enum { MSS_F32 = 0, MSS_BF16 = 1, MSS_I32 = 2 } mss_dtype_t;  /* I32: lengths only */

typedef enum {
    MSS_OK = 0,
    MSS_ERR_NULL_ARG = -1,    /* a required descriptor or its data pointer is NULL          */
    MSS_ERR_SHAPE = -2,       /* ndim or extents inconsistent with the other arguments      */
    MSS_ERR_DTYPE = -3,       /* dtype not allowed for that argument                         */
    MSS_ERR_LAYOUT = -4,      /* not dense row-major, or misaligned data pointer             */
    MSS_ERR_ALIAS = -5,       /* an output overlaps an input or another output               */
    MSS_ERR_UNSUPPORTED = -6, /* valid but not implemented (that d_state, sizes too large)    */
    MSS_ERR_HIP = -7          /* the HIP runtime reported an error while queuing the work    */
} mss_status_t;

/* A dense tensor in device memory.  Only the first `ndim` entries of shape/stride are read. */
typedef struct {
    void* data;        /* device pointer                                   */
    int32_t dtype;     /* mss_dtype_t                                      */
    int32_t ndim;      /* 1 to 4                                           */
    int64_t shape[4];
    int64_t stride[4]; /* in elements                                      */
} mss_tensor_t;

/*
 * Forward selective scan (the equations above) over a whole sequence, h_0 = 0.
 *   u, delta    (batch, d_inner, L)      f32 or bf16, same dtype; delta is the raw value
 *   A           (d_inner, d_state)       f32, real (callers pass A, e.g. -exp(A_log))
 *   B, C        (batch, d_state, L)      f32, one B and C per (batch, time) shared by all d
 *   D           (d_inner,)               f32, nullable (no skip)
 *   z           (batch, d_inner, L)      dtype of u, nullable (no gate)
 *   delta_bias  (d_inner,)               f32, nullable (bias 0)
 *   softplus_flag  nonzero: delta = softplus(delta_raw + bias); zero: delta_raw + bias
 *   out         (batch, d_inner, L)      dtype of u, written
 *   last_state  (batch, d_inner, d_state) f32, nullable; written with h_L (zeros if L = 0)
 * d_state is 16, 32, 64 or 128 (MSS_ERR_UNSUPPORTED otherwise; 16 runs the fast kernels, the
 * others the general ones, where d_state / 16 neighbouring lanes share a channel).  out must not
 * overlap any input or last_state.  A and last_state must be 16-byte aligned
 * (MSS_ERR_LAYOUT otherwise).  When every row of u / delta / z / out spans
 * a multiple of 16 bytes and those tensors and B / C start 16-byte aligned, the vectorised
 * kernels run with aligned 16-byte accesses; any other valid layout runs the same kernels with
 * element-aligned accesses (about 1.5x the time on the Mamba-2.8B layer shape).
 * Accuracy: fp32 arithmetic with an fp32 state.  Where every row of A is (n + 1) A[d, 0] exactly
 * (bf16 rows at d_state 16, any rows at d_state 128) the kernels keep the state scaled by
 * delta u and add (delta u + copysign(2^-40, delta u)) B in place of delta u B: at most
 * 2^-40 |B| per state and step away from the recurrence.
 */
int mss_selective_scan_fwd(const mss_tensor_t* u, const mss_tensor_t* delta,
                           const mss_tensor_t* A, const mss_tensor_t* B, const mss_tensor_t* C,
                           const mss_tensor_t* D, const mss_tensor_t* z,
                           const mss_tensor_t* delta_bias, int softplus_flag,
                           const mss_tensor_t* out, const mss_tensor_t* last_state,
                           void* stream);

/*
 * The same forward scan continued from a given state instead of h_0 = 0: the recurrence runs
 * unchanged with h_{t-1} at t = 1 taken from initial_state.  Cutting a sequence anywhere and
 * scanning the second part from the first part's last_state gives the outputs and final state
 * of one scan over the whole sequence (prefill in chunks, or a prompt appended to a cached
 * state), since each step depends on the past only through h_{t-1} (the tutorial page's
 * "Going from continuous spaces to discrete spaces" part: the hidden state is handed on to
 * the next input as in an RNN; the mamba-jax README's recurrent `--scan` generation).
 *   initial_state  (batch, d_inner, d_state) f32, nullable (then exactly mss_selective_scan_fwd)
 *   every other argument as for mss_selective_scan_fwd; with L = 0, last_state receives a copy
 *   of initial_state.
 * initial_state must be 16-byte aligned (MSS_ERR_LAYOUT otherwise) and must not overlap out or
 * last_state (MSS_ERR_ALIAS): the kernels of a split sequence read it while others write
 * last_state, so an in-place update needs a second buffer.
 */
int mss_selective_scan_fwd_with_state(const mss_tensor_t* u, const mss_tensor_t* delta,
                                      const mss_tensor_t* A, const mss_tensor_t* B,
                                      const mss_tensor_t* C, const mss_tensor_t* D,
                                      const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                      const mss_tensor_t* initial_state, int softplus_flag,
                                      const mss_tensor_t* out, const mss_tensor_t* last_state,
                                      void* stream);

/*
 * mss_selective_scan_fwd_with_state for a batch of sequences of different lengths (prompts of
 * different lengths prefilled together, each handing its own final state to decode): batch b's
 * sequence is steps [0, seq_lens[b]) of its rows.  Its steps stop there, last_state[b] is the
 * state after its own last step, and out[b, :, t] is 0 for t >= seq_lens[b].  Since step t
 * depends on the past only through h_{t-1}, these are the results of scanning each sequence on
 * its own (the tutorial page's recurrent view, "Going from continuous spaces to discrete spaces").
 *   seq_lens  (batch,)   MSS_I32 in device memory, nullable (then all L); values are clamped to
 *                        [0, L] on the device (they are not read on the host)
 *   every other argument as for mss_selective_scan_fwd_with_state.
 * The work done does not shrink with the lengths: steps past a sequence's end run as identity
 * steps.
 */
int mss_selective_scan_fwd_varlen(const mss_tensor_t* u, const mss_tensor_t* delta,
                                  const mss_tensor_t* A, const mss_tensor_t* B,
                                  const mss_tensor_t* C, const mss_tensor_t* D,
                                  const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                  const mss_tensor_t* initial_state, const mss_tensor_t* seq_lens,
                                  int softplus_flag, const mss_tensor_t* out,
                                  const mss_tensor_t* last_state, void* stream);

/*
 * mss_selective_scan_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments, checks and
 * results (bit-identical to mss_selective_scan_fwd whenever that call would split the work the
 * same way, which it does on devices of up to 320 CUs), but the carried segment aggregates live in
 * a fixed 16 MiB array of device memory that the library holds on each GPU for the life of the
 * process, so the call allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   - Limit: the aggregates take 4352 bytes per wavefront of the split, so at most 3855
 *     wavefronts; the automatic split is capped there, and a wavefront count forced through
 *     mss_set_plan_overrides beyond it returns MSS_ERR_UNSUPPORTED before any HIP call.  So do
 *     problems of 2^32 or more (64-channel group, time tile) pairs, which the other forward
 *     entry points hand to kernels that need row-sized scratch.
 *   - d_state must be 16 (MSS_ERR_UNSUPPORTED otherwise).
 *   - Every call on one GPU shares that GPU's array (nothing in it needs to start at zero; a
 *     call leaves its own aggregates behind): calls that overlap in time on one GPU (on two
 *     streams, or two host threads) race and may give wrong results.  Order them on one stream.
 *   - The first call on a device looks up that device's array (hipGetSymbolAddress); make it
 *     once outside graph capture if the capture mode forbids that lookup.
 */
int mss_selective_scan_fwd_noalloc(const mss_tensor_t* u, const mss_tensor_t* delta,
                                   const mss_tensor_t* A, const mss_tensor_t* B,
                                   const mss_tensor_t* C, const mss_tensor_t* D,
                                   const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                   int softplus_flag, const mss_tensor_t* out,
                                   const mss_tensor_t* last_state, void* stream);

/*
 * Gradients of mss_selective_scan_fwd (h_0 = 0) for training: given dout = dL/dout of a scalar
 * loss L, writes dL/d(every input).  The pages define only the forward; these are its exact
 * derivatives by the chain rule (reverse mode through the recurrence: with dy = dout silu(z),
 * G_t = dL/dh_t = dy_t C_t + Abar_{t+1} G_{t+1} is carried backward over t).  The forward
 * states are recomputed, not stored: the call needs only the forward's inputs.
 *   u, delta, A, B, C, D, z, delta_bias, softplus_flag   exactly as passed to the forward
 *   dout        (batch, d_inner, L)      dtype of u
 *   du, ddelta  (batch, d_inner, L)      dtype of u, written (ddelta is w.r.t. the raw delta)
 *   dA          (d_inner, d_state)       f32, written (sum over batch and time)
 *   dB, dC      (batch, d_state, L)      f32, written (sum over d_inner)
 *   dD          (d_inner,)               f32, nullable; written with sum dy u (also when D is
 *                                        NULL: the gradient at D = 0)
 *   dz          (batch, d_inner, L)      dtype of u, nullable; must be NULL when z is NULL
 *                                        (MSS_ERR_SHAPE otherwise)
 *   ddelta_bias (d_inner,)               f32, nullable; written (also when delta_bias is NULL)
 * Outputs are overwritten, not accumulated.  d_state must be 16; A must be 16-byte aligned;
 * no output may overlap an input or another output (MSS_ERR_ALIAS).  Sums are taken in a
 * fixed order: repeated calls give identical results.  Uses the library workspace (long
 * sequences: about 8 bytes per (batch, d_inner, step) of state checkpoints plus
 * 128 bytes per (64-channel group, batch, step) of partial dB / dC sums).
 */
int mss_selective_scan_bwd(const mss_tensor_t* u, const mss_tensor_t* delta,
                           const mss_tensor_t* A, const mss_tensor_t* B, const mss_tensor_t* C,
                           const mss_tensor_t* D, const mss_tensor_t* z,
                           const mss_tensor_t* delta_bias, int softplus_flag,
                           const mss_tensor_t* dout, const mss_tensor_t* du,
                           const mss_tensor_t* ddelta, const mss_tensor_t* dA,
                           const mss_tensor_t* dB, const mss_tensor_t* dC,
                           const mss_tensor_t* dD, const mss_tensor_t* dz,
                           const mss_tensor_t* ddelta_bias, void* stream);

/*
 * The backward of mss_selective_scan_fwd_varlen, for chunked training and batches of different
 * lengths: the forward started from initial_state and stopped at seq_lens (both nullable, as in
 * the forward), and the loss may also depend on the final state through dlast_state =
 * dL/d last_state (nullable: 0), which seeds the adjoint at each sequence's last step.
 * dinitial_state (nullable) receives dL/d initial_state, the adjoint left after step 0 (the
 * previous chunk's dlast_state).  Steps past a sequence's end take no part: du, ddelta, dz are 0
 * there.  State tensors (batch, d_inner, d_state) f32, 16-byte aligned; seq_lens (batch,) I32.
 * Every other argument as for mss_selective_scan_bwd; dinitial_state may not overlap any input
 * or output.
 */
int mss_selective_scan_bwd_varlen(const mss_tensor_t* u, const mss_tensor_t* delta,
                                  const mss_tensor_t* A, const mss_tensor_t* B,
                                  const mss_tensor_t* C, const mss_tensor_t* D,
                                  const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                  const mss_tensor_t* initial_state, const mss_tensor_t* seq_lens,
                                  int softplus_flag, const mss_tensor_t* dout,
                                  const mss_tensor_t* dlast_state, const mss_tensor_t* du,
                                  const mss_tensor_t* ddelta, const mss_tensor_t* dA,
                                  const mss_tensor_t* dB, const mss_tensor_t* dC,
                                  const mss_tensor_t* dD, const mss_tensor_t* dz,
                                  const mss_tensor_t* ddelta_bias,
                                  const mss_tensor_t* dinitial_state, void* stream);

/*
 * mss_selective_scan_fwd_varlen that also keeps the states its backward needs, so that
 * mss_selective_scan_bwd_saved need not recompute them: saved_states[k] receives h entering step
 * 8k (h_{8k-1} of the recurrence; initial_state, or 0, for k = 0) for every 8k < L.  Past a
 * sequence's end (seq_lens) the state is held, so the entries there repeat the final state.
 *   saved_states  (ceil(L / 8), d_state / 4, batch * d_inner * 4) f32, written: state n of row
 *                 r = b * d_inner + d entering step 8k is at [k][n / 4][4 r + n % 4] (planes of
 *                 four states, so that 64 rows' float4s are one contiguous 1 KiB run); dense,
 *                 16-byte aligned; may not overlap any input or output (MSS_ERR_ALIAS).
 *                 NULL: exactly mss_selective_scan_fwd_varlen.
 * Costs 64 / 8 = 8 bytes of extra writes per (batch, d_inner, step).  Every other argument as
 * for mss_selective_scan_fwd_varlen; out and last_state are bit-identical to it.  With
 * saved_states given, d_state must be 16 (the backward's; MSS_ERR_UNSUPPORTED otherwise).
 */
int mss_selective_scan_fwd_save(const mss_tensor_t* u, const mss_tensor_t* delta,
                                const mss_tensor_t* A, const mss_tensor_t* B,
                                const mss_tensor_t* C, const mss_tensor_t* D,
                                const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                const mss_tensor_t* initial_state, const mss_tensor_t* seq_lens,
                                int softplus_flag, const mss_tensor_t* out,
                                const mss_tensor_t* last_state, const mss_tensor_t* saved_states,
                                void* stream);

/*
 * mss_selective_scan_bwd_varlen from the states saved by mss_selective_scan_fwd_save (the same
 * inputs; the forward's initial_state is carried inside saved_states, so it is not passed):
 * the backward then skips its forward recomputation.  Results agree with
 * mss_selective_scan_bwd_varlen to rounding (the states come from the forward's own order of
 * operations), and need a smaller workspace (no checkpoints).
 *   saved_states  as written by mss_selective_scan_fwd_save for these inputs, read only; NULL
 *                 gives MSS_ERR_NULL_ARG; no output may overlap it (MSS_ERR_ALIAS).
 * Every other argument as for mss_selective_scan_bwd_varlen.
 */
int mss_selective_scan_bwd_saved(const mss_tensor_t* u, const mss_tensor_t* delta,
                                 const mss_tensor_t* A, const mss_tensor_t* B,
                                 const mss_tensor_t* C, const mss_tensor_t* D,
                                 const mss_tensor_t* z, const mss_tensor_t* delta_bias,
                                 const mss_tensor_t* seq_lens, int softplus_flag,
                                 const mss_tensor_t* saved_states, const mss_tensor_t* dout,
                                 const mss_tensor_t* dlast_state, const mss_tensor_t* du,
                                 const mss_tensor_t* ddelta, const mss_tensor_t* dA,
                                 const mss_tensor_t* dB, const mss_tensor_t* dC,
                                 const mss_tensor_t* dD, const mss_tensor_t* dz,
                                 const mss_tensor_t* ddelta_bias,
                                 const mss_tensor_t* dinitial_state, void* stream);

/*
 * One recurrent (decode) step: the same equations for a single token, continuing from
 * `state`, which is updated in place (the recurrent mode the mamba-jax README's `--scan`
 * generation loop and the upstream README's generation benchmark run token by token).
 * softplus is always applied to dt + dt_bias.
 *   state       (batch, d_inner, d_state) f32, read and written
 *   x, dt       (batch, d_inner)         f32 or bf16, same dtype
 *   A           (d_inner, d_state)       f32
 *   B, C        (batch, d_state)         f32
 *   D           (d_inner,)               f32, nullable
 *   z           (batch, d_inner)         dtype of x, nullable
 *   dt_bias     (d_inner,)               f32, nullable
 *   out         (batch, d_inner)         dtype of x, written
 * d_state must be 16, 32, 64 or 128.  out must not overlap any input or the state; the state
 * must not overlap any input.  state, A, B and C must be 16-byte aligned (MSS_ERR_LAYOUT otherwise).
 */
int mss_selective_state_update(const mss_tensor_t* state, const mss_tensor_t* x,
                               const mss_tensor_t* dt, const mss_tensor_t* A,
                               const mss_tensor_t* B, const mss_tensor_t* C,
                               const mss_tensor_t* D, const mss_tensor_t* z,
                               const mss_tensor_t* dt_bias, const mss_tensor_t* out,
                               void* stream);

/*
 * Causal depthwise conv1d (+ silu): the step in front of the scan in the tutorial page's
 * `MambaBlock` (a Conv1D with one filter per channel, kernel size 4, bias, channels-first data,
 * causal padding, then swish; the upstream README's d_conv = 4).  Per channel d and step t,
 *     y[t] = bias[d] + sum_{k=0}^{K-1} weight[d][k] * x[t - (K-1) + k],   out = silu(y) or y,
 * a cross-correlation whose last tap meets the current input; inputs before t = 0 come from
 * initial_state (zeros when NULL).
 *   x              (batch, d_inner, L)        f32 or bf16
 *   weight         (d_inner, K)               f32, 1 <= K <= 4 (MSS_ERR_UNSUPPORTED above)
 *   bias           (d_inner,)                 f32, nullable (0)
 *   initial_state  (batch, d_inner, K - 1)    dtype of x, nullable: the K - 1 inputs before t = 0,
 *                                             oldest first
 *   silu_flag      nonzero: out = silu(y)
 *   out            (batch, d_inner, L)        dtype of x, written
 *   final_state    (batch, d_inner, K - 1)    dtype of x, nullable: written with the last K - 1
 *                                             inputs (older ones from initial_state when L < K - 1)
 * Chunked prefill: pass one chunk's final_state as the next chunk's initial_state (a different
 * buffer: out and final_state may not overlap an input or each other, MSS_ERR_ALIAS).
 */
int mss_causal_conv1d_fwd(const mss_tensor_t* x, const mss_tensor_t* weight,
                          const mss_tensor_t* bias, const mss_tensor_t* initial_state,
                          int silu_flag, const mss_tensor_t* out,
                          const mss_tensor_t* final_state, void* stream);

/*
 * The same conv for one token per row, with the K - 1 previous inputs kept in `state`, which is
 * updated in place (the window moves by one: the oldest input drops out, x comes in).
 *   state   (batch, d_inner, K - 1)   dtype of x, read and written
 *   x       (batch, d_inner)          f32 or bf16
 *   weight  (d_inner, K) f32; bias (d_inner,) f32 nullable; silu_flag as above
 *   out     (batch, d_inner)          dtype of x, written
 * out and the state may not overlap an input or each other.
 */
int mss_causal_conv1d_update(const mss_tensor_t* state, const mss_tensor_t* x,
                             const mss_tensor_t* weight, const mss_tensor_t* bias, int silu_flag,
                             const mss_tensor_t* out, void* stream);

/*
 * Launch timing, for measurement only (the results of the calls above do not depend on it).
 * mss_profile_enable(1) clears the records and makes each later mss_selective_scan_fwd or
 * mss_selective_scan_fwd_with_state (up to 1024 calls) record three library-owned HIP events on its stream: before its first kernel,
 * between the carry stage (the per-segment aggregates of a split sequence) and the main
 * kernel, and after the main kernel.  mss_profile_enable(0) stops recording (the records stay).
 * mss_profile_fwd waits for the recorded calls to finish and returns their count and the
 * summed carry-stage and main-kernel times in milliseconds (a call that did not split its
 * sequence adds 0 carry time).  Events are created on the device current at the recording
 * call; record calls of one device at a time.
 * Returns MSS_OK; MSS_ERR_NULL_ARG for a NULL output pointer; MSS_ERR_HIP when the runtime
 * reports an error.
 */
int mss_profile_enable(int on);
int mss_profile_fwd(int* calls, double* carry_ms, double* main_ms);

/*
 * Mamba-2's SSD layer (the upstream README's Mamba-2 block, whose state size is usually 64 or 128): the
 * selective recurrence above with Mamba-2's tied parameters, for every batch b, head h (P
 * channels p) and state n:
 *     delta_t   = softplus(dt[b, t, h] + dt_bias[h])               (or without softplus)
 *     h_t[p, n] = exp(delta_t A[h]) h_{t-1}[p, n] + delta_t B[b, t, g, n] x[b, t, h, p]   (h_0 = 0)
 *     y_t[p]    = sum_n C[b, t, g, n] h_t[p, n] + D[h] x[b, t, h, p]
 *     out       = y silu(z[b, t, h, p])                            (when z is given)
 * with one scalar A per head, one delta per (batch, time, head) shared by its channels, and B, C per
 * (batch, time, group), heads in contiguous blocks of H / G per group (head h reads g = h / (H/G)).
 * Computed as a chunked scan (64-step chunks, dense products on the matrix cores); results agree
 * with the step-by-step recurrence to rounding.
 *   x, z, out   (batch, L, heads, headdim)    bf16 (z nullable: no gate)
 *   dt          (batch, L, heads)             bf16, raw (before bias and softplus)
 *   A           (heads,)                      f32, negative
 *   B, C        (batch, L, groups, d_state)   bf16; heads % groups == 0 (MSS_ERR_SHAPE otherwise)
 *   D, dt_bias  (heads,)                      f32, nullable
 *   last_state  (batch, heads, headdim, d_state) f32, nullable; written with h_L
 * headdim must be 64 and d_state 64 or 128; fp32 activations are not implemented (both
 * MSS_ERR_UNSUPPORTED).  x, z, out, B and C must be 16-byte aligned (MSS_ERR_LAYOUT).  out and
 * last_state may not overlap an input or each other.  Long sequences are cut into segments whose
 * local end states pass through the library workspace (headdim * d_state + 1 floats per batch,
 * head and segment but the last).
 */
int mss_ssd_scan_fwd(const mss_tensor_t* x, const mss_tensor_t* dt, const mss_tensor_t* A,
                     const mss_tensor_t* B, const mss_tensor_t* C, const mss_tensor_t* D,
                     const mss_tensor_t* z, const mss_tensor_t* dt_bias, int softplus_flag,
                     const mss_tensor_t* out, const mss_tensor_t* last_state, void* stream);

/*
 * Frees every workspace buffer the library holds, on every device (current ones and those
 * replaced by larger ones), after waiting for each device to finish its work.  HIP graphs that
 * captured library calls must not be replayed afterwards (their workspace is gone); later calls
 * allocate again.  Returns MSS_OK or MSS_ERR_HIP.
 */
int mss_release_workspaces(void);

/*
 * Test and tuning hook, not for production use: fixes choices the library otherwise makes by
 * itself, for every later call in the process (results agree to rounding with any setting).
 *   force_generic     nonzero: the forward runs the generic kernels (any layout; slower)
 *   generic_segments  > 0: segments per channel group of the generic forward
 *   fast_waves        > 0: wavefronts the fast forward spreads a call over (each takes an equal
 *                     share of the (64-channel group, time tile) work; more than the groups
 *                     splits sequences, fewer makes one wavefront scan several groups)
 *   bwd_segments      > 0: segments per channel group of the backward
 *   ssd_segments      > 0: segments each (batch, head) of mss_ssd_scan_fwd is cut into
 * Zeros restore the automatic plans.  Returns MSS_OK, or MSS_ERR_SHAPE for a negative count.
 */
int mss_set_plan_overrides(int force_generic, int generic_segments, int64_t fast_waves,
                           int bwd_segments, int ssd_segments);

/* Static, NUL-terminated name of a status code ("MSS_OK", "MSS_ERR_SHAPE", ...). */
const char* mss_status_string(int status);

/* MSS_VERSION of the loaded library. */
int mss_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
