/*
 * ssm66.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * Seven operations (and one measurement aid, ssm_alu_probe), defined on
 * "Mamba and selective state spaces"
 * (zerotofrontier.app/ssm/mamba):
 *
 *   ssm_scan_fwd : the selective state-space layer (S6) over whole sequences --
 *                  section "The selective state-space model", the S6 definition
 *                  box (Delta_t = softplus(raw_t + b_Delta); abar = exp(Delta A);
 *                  h_t = abar h_{t-1} + bbar x_t; y_t = C_t . h_t + D x_t), with
 *                  the two input-weight rules of "The discretization the code
 *                  actually uses" (zero-order hold, and the exponential-Euler
 *                  rule bbar = Delta B) and the SiLU(z) gate of "The Mamba
 *                  block".  Prefill keeps only the final state ("Decoding with
 *                  a constant-size cache"), returned in last_state.
 *   ssm_scan_fwd_ex : the same scan for sequences that do not start from zero
 *                  or do not fill the batch: an initial state (a later chunk
 *                  of a prefill starts from the state the earlier chunk
 *                  returned), per-sequence lengths with padding after them
 *                  (padding must be kept out of the state: "Where Mamba
 *                  implementations go wrong"), and document starts where the
 *                  state is forgotten ("What each parameter does": packed
 *                  documents should not see each other).
 *   ssm_scan_bwd : gradients of ssm_scan_fwd (with h0 and the gradient of
 *                  last_state), recomputing the states from the inputs instead
 *                  of storing them ("Why the scan must be fused": the backward
 *                  pass reloads x, Delta, B, C and recomputes the states; the
 *                  backward of a linear recurrence is a reverse recurrence).
 *                  For training, ssm_scan_fwd_ckpt also keeps the state every
 *                  16 tokens, and ssm_scan_bwd_ex recomputes from those
 *                  checkpoints instead of from the start of the sequence.
 *   ssm_step     : one token of that layer against a state cache, updated in
 *                  place ("Decoding with a constant-size cache").
 *   ssm_ssd_fwd  : the Mamba-2 / SSD layer, one scalar decay per head, as a
 *                  chunked masked matmul on the matrix cores (the first page on
 *                  what Mamba cannot do yet; "The Mamba CUDA kernel" on
 *                  "State-space models & Mamba", llm-tutorial.darvinyi.com).
 *   ssm_conv1d_fwd, ssm_conv1d_step : the short causal depthwise convolution
 *                  (+ SiLU) that feeds the scan in "The Mamba block", over
 *                  whole sequences and as one decoding step with its window of
 *                  the last k - 1 inputs; ssm_conv1d_bwd is its backward pass.
 *
 * Conventions shared by all calls
 *   - Every pointer is caller-owned DEVICE memory (HBM).  The library keeps no
 *     pointer after the call returns and allocates nothing.
 *   - Tensors are dense and row-major:
 *       u, delta, z, y    : (batch, seqlen, dim)   [ssm_step: (batch, dim)]
 *       B, C              : (batch, seqlen, dstate) [ssm_step: (batch, dstate)]
 *       A                 : (dim, dstate)            float32
 *       D, delta_bias     : (dim)                    float32
 *       last_state, state : (batch, dim, dstate)     float32
 *     u, delta, B, C, z and y share one I/O dtype (io_dtype: SSM_F32 or
 *     SSM_BF16); A, D, delta_bias and the states are float32 in every mode.
 *   - D, z, delta_bias and last_state may be NULL (no skip, no gate, zero bias,
 *     final state not returned).
 *   - softplus != 0 applies Delta = softplus(delta + bias); softplus == 0 uses
 *     Delta = delta + bias as given.  The bias is added exactly once.
 *   - dt_mode selects the input weight: SSM_DT_ZOH, bbar = (exp(Delta A) - 1)/A B
 *     (limit Delta B at A = 0), or SSM_DT_EULER, bbar = Delta B.
 *   - The gate multiplies the whole S6 output: y = (C.h + D u) * z * sigmoid(z).
 *   - 1 <= dstate <= 16; batch, seqlen, dim >= 0.  Zero batch or dim is a no-op;
 *     seqlen == 0 writes the initial state (zero, or h0) to last_state.
 *   - Pointers must be aligned to their element size.  y must not overlap an
 *     input; in ssm_step, y must not overlap state.
 *   - Values are not checked: negative Delta, A >= 0, NaN and Inf are computed
 *     as written.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work and return; nothing is synchronised.  On any error status nothing
 *     has been enqueued, except SSM_ERR_HIP, which reports a failed launch.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Thread-safe.  The only mutable global state is the per-device address
 *     of ssm_scan_bwd_noalloc's static scratch, set once under a lock.
 */
#ifndef SSM66_H
#define SSM66_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 10

/* status codes */
#define SSM_OK 0
#define SSM_ERR_NULL 1        /* a required pointer is NULL */
#define SSM_ERR_SHAPE 2       /* negative size, dstate outside [1, 16], width outside
                                 [1, 4], or size overflow */
#define SSM_ERR_DTYPE 3       /* io_dtype is not SSM_F32 or SSM_BF16 */
#define SSM_ERR_FLAG 4        /* softplus not 0/1, or dt_mode unknown */
#define SSM_ERR_ALIGN 5       /* a pointer is not aligned to its element size */
#define SSM_ERR_UNSUPPORTED 6 /* a size the kernels do not handle (e.g. > 2^31 rows) */
#define SSM_ERR_HIP 7         /* the HIP runtime rejected the launch */

/* io dtypes */
#define SSM_F32 0
#define SSM_BF16 1

/* discretization rules */
#define SSM_DT_ZOH 0
#define SSM_DT_EULER 1

/* scan kernel choices for ssm_scan_fwd_kernel */
#define SSM_SCAN_KERNEL_AUTO 0 /* the library's choice by shape (what ssm_scan_fwd runs) */
#define SSM_SCAN_KERNEL_SEQ1 1 /* sequential; 1 state per lane for 9..16 states */
#define SSM_SCAN_KERNEL_SEQ2 2 /* sequential; 2 states per lane for 9..16 states */
#define SSM_SCAN_KERNEL_SEQ4 3 /* sequential; 4 states per lane for 9..16 states */
#define SSM_SCAN_KERNEL_TPAR 4 /* time-parallel, four waves per (batch, channel) row */
#define SSM_SCAN_KERNEL_WAVE 5 /* time-parallel, one wave per row */
#define SSM_SCAN_KERNEL_WAVE4 6 /* time-parallel, 16 lanes per row (four rows per wave) */

/*
 * The selective scan over whole sequences.
 *
 * y[b,t,c] = gate(z[b,t,c]) * (sum_n C[b,t,n] h_t[b,c,n] + D[c] u[b,t,c]),
 * h_t[b,c,n] = exp(Delta A[c,n]) h_{t-1}[b,c,n] + bbar(Delta, A[c,n], B[b,t,n]) u[b,t,c],
 * Delta = softplus?(delta[b,t,c] + delta_bias[c]), h_{-1} = 0.
 * last_state (optional) receives h after the last token.
 * Three kernels compute it ("Mamba and selective state spaces", "Selection
 * breaks the convolution": the recurrence is an associative scan):
 *   - sequential: lanes hold (channel, state group) and run through time;
 *     for sequences under 256 tokens, and for 32768 or more (batch x
 *     channel) rows;
 *   - time-parallel, one wave per row: lanes hold four consecutive tokens,
 *     composed in the lane and across the wave by a parallel scan; for
 *     1024 to 32767 rows and 256 or more tokens;
 *   - time-parallel, four waves per row: lanes hold one token each; for
 *     fewer than 1024 rows and 128 or more tokens.
 * All give the same result up to fp32 rounding; ssm_scan_kernel_name()
 * names the one a call will run, and ssm_scan_fwd_kernel forces one.
 * Returns SSM_OK or an error status (see above).
 */
int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus,
                 int dt_mode, void* y, float* last_state, int64_t batch, int64_t seqlen,
                 int64_t dim, int64_t dstate, int io_dtype, void* stream);

/*
 * ssm_scan_fwd with three optional extras (any of them may be NULL; with all
 * three NULL it is ssm_scan_fwd):
 *   h0        (batch, dim, dstate) float32: the state before token 0
 *             (instead of zero).  last_state may be the same buffer as h0
 *             (the state is then advanced in place); no other overlap.
 *   seq_lens  (batch) int32: sequence b has seq_lens[b] real tokens followed
 *             by padding (values are clamped to [0, seqlen]).  Padded tokens
 *             do not touch the state, whatever their inputs hold (NaN
 *             included), and their y is 0; last_state is the state after the
 *             last real token.
 *   reset     (batch, seqlen) uint8: nonzero at t means a new document starts
 *             at token t: the state is set to zero before token t is written.
 *             Left padding is a reset at the first real token.
 * seq_lens must be 4-byte aligned; reset has no alignment requirement.
 * Returns SSM_OK or an error status.
 */
int ssm_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int softplus, int dt_mode, const float* h0, const int32_t* seq_lens,
                    const uint8_t* reset, void* y, float* last_state, int64_t batch,
                    int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* stream);

/*
 * ssm_scan_fwd_ex and ssm_scan_fwd_ckpt in one call, on a kernel chosen by the
 * caller: kernel is one of SSM_SCAN_KERNEL_* (SSM_SCAN_KERNEL_AUTO is the
 * library's own choice).  For tests that run every kernel on the same inputs,
 * and for measuring one kernel against another; every kernel computes the
 * same layer ("The selective state-space model"; the three compositions of
 * its recurrence are described at ssm_scan_fwd).  h0, seq_lens, reset and
 * ckpt are nullable and mean what they mean for ssm_scan_fwd_ex and
 * ssm_scan_fwd_ckpt.  The SEQ choices fix the states per lane only for 9..16
 * states (fewer states have one shape).  Returns SSM_ERR_FLAG for an unknown
 * kernel, SSM_ERR_UNSUPPORTED where the forced kernel cannot address the
 * shape (the time-parallel kernels need 1024 * dim < 2^32), else as
 * ssm_scan_fwd_ex.
 */
int ssm_scan_fwd_kernel(int kernel, const void* u, const void* delta, const float* A,
                        const void* B, const void* C, const float* D, const void* z,
                        const float* delta_bias, int softplus, int dt_mode, const float* h0,
                        const int32_t* seq_lens, const uint8_t* reset, void* y,
                        float* last_state, float* ckpt, int64_t batch, int64_t seqlen,
                        int64_t dim, int64_t dstate, int io_dtype, void* stream);

/*
 * Bytes of device workspace ssm_scan_bwd needs for these sizes (0 for invalid
 * sizes): per-chunk state checkpoints (batch x ceil(seqlen/16) x dim x dstate
 * floats) and the partial sums that are added in a fixed order at the end.
 */
size_t ssm_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * Backward pass of ssm_scan_fwd / ssm_scan_fwd_ex without lengths or resets
 * (ssm_scan_bwd_ex takes those).
 * Inputs: the forward's inputs (u, delta, A, B, C, D, z, delta_bias, softplus,
 * dt_mode, h0 -- D, z, delta_bias, h0 nullable), dy (batch, seqlen, dim) io
 * dtype, and dlast_state (batch, dim, dstate) float32, the gradient of
 * last_state (NULL = zero).
 * Outputs (overwritten, not accumulated into):
 *   du, ddelta (gradient of the RAW delta), dz : (batch, seqlen, dim) io dtype
 *     (dz is required when z is given and ignored otherwise);
 *   dB, dC : (batch, seqlen, dstate) io dtype;
 *   dA : (dim, dstate) float32;  dD, ddelta_bias : (dim) float32, or NULL;
 *   dh0 : (batch, dim, dstate) float32, or NULL.
 * workspace: device memory of at least ssm_scan_bwd_workspace_size(...) bytes,
 * 256-byte aligned, owned by the caller, contents not needed before or after.
 * Sums over channels (dB, dC) and over batch entries (dA, dD, ddelta_bias) are
 * added in a fixed order: repeated calls give identical bits.  Calls that share
 * a workspace must not overlap.  Returns SSM_OK or an error status
 * (SSM_ERR_SHAPE also when workspace_bytes is too small).
 */
int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus,
                 int dt_mode, const float* h0, const void* dy, const float* dlast_state,
                 void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                 float* ddelta_bias, float* dh0, void* workspace, size_t workspace_bytes,
                 int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 void* stream);

/*
 * Bytes of the training forward's checkpoints for these sizes (0 for invalid
 * sizes): the state before every 16th token, (batch, ceil(seqlen/16), dim,
 * dstate) float32, rounded up to 256 bytes.
 */
size_t ssm_scan_ckpt_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * The name of the kernel ssm_scan_fwd, ssm_scan_fwd_ex and ssm_scan_fwd_ckpt
 * run for these sizes, e.g.
 * "scan_wave_kernel (time-parallel, one wave per row)".  A static string
 * owned by the library; "invalid shape" for sizes the scan rejects.  Host
 * only: no device work.
 */
const char* ssm_scan_kernel_name(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * The training forward: ssm_scan_fwd with an initial state (h0, nullable, as
 * in ssm_scan_fwd_ex) that also writes the state before tokens 0, 16, 32, ...
 * of every sequence to ckpt (device memory of ssm_scan_ckpt_size(...) bytes,
 * float32, 4-byte aligned, owned by the caller; required when seqlen > 0):
 * the checkpoints the backward pass would otherwise rebuild with a forward
 * sweep ("Why the scan must be fused": only chunk boundaries are kept, the
 * states in between are recomputed).  y and last_state are the same as
 * ssm_scan_fwd_ex's.  Returns SSM_OK or an error status.
 */
int ssm_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      int softplus, int dt_mode, const float* h0, void* y, float* last_state,
                      float* ckpt, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                      int io_dtype, void* stream);

/*
 * ssm_scan_bwd for the whole ssm_scan_fwd_ex: seq_lens (batch) int32 and
 * reset (batch, seqlen) uint8, both nullable, mean what they mean there --
 * tokens at or past a length are padding (their du, ddelta, dz and their rows
 * of dB, dC come out zero; dlast_state reaches the last real token), and a
 * document starting at t sees a zero state, so no gradient flows from t back
 * to earlier tokens or to h0 ("Mamba and selective state spaces", "Why the
 * scan must be fused": the backward pass is the forward's linear recurrence
 * run in reverse, here with the forward's breaks).  ckpt (nullable) is what
 * the forward wrote for the same inputs, h0, lengths and resets
 * (ssm_scan_fwd_ckpt, or ssm_scan_fwd_kernel with a ckpt); with it the
 * backward skips its own forward sweep (the checkpoint part of the workspace
 * is then unused; checkpoints of chunks wholly in the padding are not read).
 * With all three NULL it is ssm_scan_bwd.  seq_lens must be 4-byte aligned.
 * Returns SSM_OK or an error status.
 */
int ssm_scan_bwd_ex(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int softplus, int dt_mode, const float* h0, const int32_t* seq_lens,
                    const uint8_t* reset, const void* dy, const float* dlast_state, void* du,
                    void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                    float* ddelta_bias, float* dh0, const float* ckpt, void* workspace,
                    size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim,
                    int64_t dstate, int io_dtype, void* stream);

/* size of the static device scratch behind ssm_scan_bwd_noalloc (64 MiB) */
#define SSM_NOALLOC_SCRATCH_BYTES 67108864

/*
 * ssm_scan_bwd_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without workspace and workspace_bytes, the same kernels
 * and the same results, with the workspace taken from a static array in
 * device memory of SSM_NOALLOC_SCRATCH_BYTES.  The library calls no allocator
 * for it: the array exists once per GPU it runs on and stays until the
 * process ends.  Sizes whose ssm_scan_bwd_workspace_size exceeds the array
 * return SSM_ERR_UNSUPPORTED before any HIP call.  Every call on one GPU
 * shares that GPU's array (nothing in it needs to start at zero; it keeps the
 * last call's partial sums): calls that overlap on one GPU -- on different
 * streams, or from different threads without ordering -- race and give wrong
 * results.  The first call on a device looks the array's address up on that
 * device (SSM_ERR_HIP if the runtime cannot).  Returns SSM_OK or an error
 * status as ssm_scan_bwd_ex.
 */
int ssm_scan_bwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D, const void* z, const float* delta_bias,
                         int softplus, int dt_mode, const float* h0, const int32_t* seq_lens,
                         const uint8_t* reset, const void* dy, const float* dlast_state,
                         void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                         void* dz, float* ddelta_bias, float* dh0, const float* ckpt,
                         int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         int io_dtype, void* stream);

/*
 * One decode step against the state cache `state` (batch, dim, dstate),
 * updated in place: the same body as one token of ssm_scan_fwd.
 * u, delta, z, y: (batch, dim); B, C: (batch, dstate).
 * Returns SSM_OK or an error status.
 */
int ssm_step(float* state, const void* u, const void* delta, const float* A, const void* B,
             const void* C, const float* D, const void* z, const float* delta_bias, int softplus,
             int dt_mode, void* y, int64_t batch, int64_t dim, int64_t dstate, int io_dtype,
             void* stream);

/*
 * The Mamba-2 / SSD layer: the S6 recurrence with one scalar decay A[h] and
 * one step size per (token, head) for each head of `headdim` channels, and B,
 * C shared by all heads:
 *   Delta = softplus?(dt[b,t,h] + dt_bias[h]),  alpha = exp(Delta A[h]),
 *   w = Delta (SSM_DT_EULER) or Delta (exp(Delta A) - 1)/(Delta A) (SSM_DT_ZOH),
 *   h_t[p,n] = alpha h_{t-1}[p,n] + w B[b,t,n] x[b,t,h,p],
 *   y[b,t,h,p] = (sum_n C[b,t,n] h_t[p,n] + D[h] x[b,t,h,p]) * silu(z)?
 * Layouts: x, z, y (batch, seqlen, nheads * headdim) io dtype; dt
 * (batch, seqlen, nheads) float32; A, D, dt_bias (nheads) float32; B, C
 * (batch, seqlen, dstate) io dtype; h0, last_state (batch, nheads * headdim,
 * dstate) float32 (the scan's state layout).  D, z, dt_bias, h0, last_state
 * may be NULL.  The kernel runs on the matrix cores with bf16 operands and
 * fp32 accumulation and state: io_dtype must be SSM_BF16, headdim a multiple
 * of 16, nheads * headdim at most 2^23 and dstate 64 or 128 (else
 * SSM_ERR_UNSUPPORTED); x, z, y, B, C must be 16-byte aligned.  Returns SSM_OK
 * or an error status.
 */
int ssm_ssd_fwd(const void* x, const float* dt, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, int softplus, int dt_mode,
                const float* h0, void* y, float* last_state, int64_t batch, int64_t seqlen,
                int64_t nheads, int64_t headdim, int64_t dstate, int io_dtype, void* stream);

/*
 * The block's causal depthwise convolution over whole sequences ("The Mamba
 * block": x_t = SiLU(sum_{i<k} w_i * xt_{t-i} + b_conv), inputs before the
 * sequence are zero, each channel has its own k taps).
 *   x, out      : (batch, seqlen, dim), io dtype
 *   weight      : (dim, width) float32; weight[c * width + i] multiplies the
 *                 input i steps back (i = 0 is the current token)
 *   bias        : (dim) float32, or NULL
 *   silu        : 1 applies SiLU to the sum, 0 returns the sum
 *   window_in   : (batch, width - 1, dim) io dtype, oldest first: the inputs
 *                 before token 0 (a later chunk of a prefill), or NULL (zeros)
 *   seq_lens    : (batch) int32 or NULL; tokens past a length output 0
 *   reset       : (batch, seqlen) uint8 or NULL; a document starting at t sees
 *                 zeros before t
 *   window_out  : (batch, width - 1, dim) io dtype, or NULL: the last width - 1
 *                 real inputs, oldest first (zeros before a document start) --
 *                 the decoding window after a prefill ("Decoding with a
 *                 constant-size cache").  Must not overlap window_in.
 * 1 <= width <= 4.  The io pointers must be aligned to their element size;
 * weight, bias and seq_lens to 4 bytes.  Returns SSM_OK or an error status.
 */
int ssm_conv1d_fwd(const void* x, const float* weight, const float* bias, int silu,
                   const void* window_in, const int32_t* seq_lens, const uint8_t* reset,
                   void* out, void* window_out, int64_t batch, int64_t seqlen, int64_t dim,
                   int64_t width, int io_dtype, void* stream);

/*
 * One decoding step of the convolution: out = SiLU?(w_0 x + sum_{i>=1} w_i
 * window[width - 1 - i] + b); then window (batch, width - 1, dim), oldest
 * first, drops its oldest input and appends x, in place (the window holds
 * inputs, not outputs: "Where Mamba implementations go wrong").
 * x, out: (batch, dim) io dtype; weight, bias as for ssm_conv1d_fwd.
 * Returns SSM_OK or an error status.
 */
int ssm_conv1d_step(void* window, const void* x, const float* weight, const float* bias,
                    int silu, void* out, int64_t batch, int64_t dim, int64_t width, int io_dtype,
                    void* stream);

/*
 * Bytes of device workspace ssm_conv1d_bwd needs for these sizes (0 for
 * invalid sizes): (width + 1) partial sums per channel for every 128 tokens
 * of every sequence.
 */
size_t ssm_conv1d_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t width);

/*
 * Backward pass of ssm_conv1d_fwd (the same x, weight, bias, silu, window_in,
 * seq_lens, reset): the chain rule through "The Mamba block"'s convolution
 * x_t = SiLU(sum_{i<k} w_i * xt_{t-i} + b_conv).  Given dout (batch, seqlen,
 * dim) io dtype and dwindow_out (batch, width - 1, dim) io dtype or NULL, the
 * gradient of window_out, it writes
 *   dx          : (batch, seqlen, dim) io dtype (zero past a length);
 *   dweight     : (dim, width) float32;  dbias : (dim) float32, or NULL;
 *   dwindow_in  : (batch, width - 1, dim) io dtype, the gradient of
 *                 window_in -- written only when window_in is given, and not
 *                 the same memory.
 * An input feeds the outputs of its document only (no gradient crosses a
 * document start) and of real tokens only.  workspace: device memory of at
 * least ssm_conv1d_bwd_workspace_size(...) bytes, 16-byte aligned, owned by
 * the caller; the sums over tokens and batch entries behind dweight and
 * dbias are added in a fixed order (repeated calls give identical bits).
 * 1 <= width <= 4; one sequence (seqlen * dim elements) must stay below
 * 2^31 bytes (else SSM_ERR_UNSUPPORTED).  Returns SSM_OK or an error status
 * (SSM_ERR_SHAPE also when workspace_bytes is too small).
 */
int ssm_conv1d_bwd(const void* x, const float* weight, const float* bias, int silu,
                   const void* window_in, const int32_t* seq_lens, const uint8_t* reset,
                   const void* dout, const void* dwindow_out, void* dx, float* dweight,
                   float* dbias, void* dwindow_in, void* workspace, size_t workspace_bytes,
                   int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int io_dtype,
                   void* stream);

/* issue-rate probes of ssm_alu_probe */
#define SSM_PROBE_FMA 0 /* per iteration 8 x v_fma_f32 per lane */
#define SSM_PROBE_EXP 1 /* per iteration 8 x v_exp_f32 per lane */
#define SSM_PROBE_MIX 2 /* per iteration 8 x (v_exp_f32 + 4 x v_fma_f32) per lane */

/*
 * A measurement aid, not part of the layer: the chip's fp32 FMA and v_exp_f32
 * issue rates, which bound the scan ("Mamba and selective state spaces", "Why
 * the scan must be fused": one exponential per state update, and a few
 * multiply-adds, set the scan's compute floor).  Launches blocks x 256 lanes
 * that each run iters iterations of the chosen body over 8 independent
 * chains and write one float per lane to sink (blocks * 256 floats, device
 * memory, 4-byte aligned, owned by the caller; the values have no meaning).
 * Time the launch on `stream` to get lane-operations per second.
 * Returns SSM_ERR_FLAG for an unknown op, SSM_ERR_SHAPE for blocks outside
 * [1, 2^31 - 1] or iters outside [0, 2^31 - 1], else as the other calls.
 */
int ssm_alu_probe(int op, float* sink, int64_t blocks, int64_t iters, void* stream);

/* A static, human-readable string for a status code. */
const char* ssm_status_string(int status);

/* SSM_ABI_VERSION of the built library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM66_H */
