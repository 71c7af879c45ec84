/*
 * libjscan -- selective state-space scan for AMD MI355X (gfx950).
 *
 * The operation is the recurrence of a state-space model with a fixed-size
 * state, made selective by per-token parameters ("AI Engineering from Scratch",
 * Jamba lesson, section "一页讲完 SSM", and its glossary entry for the selective
 * SSM): for every sequence b, channel d and state index n,
 *
 *     h[t][n] = exp(delta[t][d] * A[d][n]) * h[t-1][n] + delta[t][d] * B[t][n] * x[t][d]
 *     y[t][d] = (sum_n C[t][n] * h[t][n] + D[d] * x[t][d]) * SiLU(z[t][d])
 *
 * with SiLU(v) = v / (1 + exp(-v)).  A is real and diagonal per (channel,
 * state), as in the Mamba-1 layers that make up seven of every eight layers of
 * Jamba (Jamba lesson, sections "Jamba 块" and "Mamba-3"; the Jamba report by
 * zako-mio, section 2.1).  The decay exp(delta*A) and the input term
 * delta*B*x are the discretisation the pages call "Euler" for the input; the
 * gate multiplies the whole output, D skip included.  A prefill scans a whole
 * sequence; a decode step advances the state by one token, and the state is
 * carried from the prefill into decoding (ksqn.cn blog, section 4.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array argument is a DEVICE pointer into dense, row-major memory,
 *    owned by the caller.  The library keeps no pointer after a call returns.
 *  - `io` gives the element type of x, delta, z, B, C and y: JSCAN_IO_BF16
 *    (bfloat16 bit patterns, converted to fp32 exactly on load, rounded to
 *    nearest-even on store) or JSCAN_IO_F32.  A, D and every state array are
 *    always fp32; the arithmetic is fp32 throughout.
 *  - d_state must be 16 (the Mamba state width of the pages); other values
 *    return JSCAN_ERR_UNSUPPORTED.
 *  - Every pointer must be 16-byte aligned (JSCAN_ERR_ALIGN otherwise).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously on it; a call returns once the work is enqueued.
 *  - Arguments are validated on the host before anything is enqueued.  On an
 *    error nothing is launched and no output is written.  Faults during
 *    execution surface at the caller's next synchronisation, as for any HIP
 *    kernel.  NaN and Inf inputs are not checked: they propagate through the
 *    arithmetic of the channel they belong to.
 *  - Calls are thread-safe; concurrent calls on different streams must not
 *    share output buffers or workspace.
 */
#ifndef JSCAN_H
#define JSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JSCAN_OK = 0,
  JSCAN_ERR_NULL = 1,        /* a required pointer is NULL */
  JSCAN_ERR_SHAPE = 2,       /* a size is negative, or sizes overflow 64-bit byte counts */
  JSCAN_ERR_UNSUPPORTED = 3, /* d_state != 16, or unknown io */
  JSCAN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  JSCAN_ERR_ALIAS = 5,       /* an output overlaps an input or another output */
  JSCAN_ERR_WORKSPACE = 6,   /* workspace given but smaller than required */
  JSCAN_ERR_HIP = 7          /* a HIP runtime call failed (see jscan_last_error) */
} jscan_status;

typedef enum { JSCAN_IO_F32 = 0, JSCAN_IO_BF16 = 1 } jscan_io;

/*
 * Bytes of device workspace jscan_prefill needs for this problem.  It depends
 * only on the sizes.  Returns 0 for an invalid size combination.
 */
size_t jscan_prefill_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                                    jscan_io io);

/*
 * Prefill: the scan over L tokens of `batch` independent sequences.
 *
 *   x, delta, z : [batch][L][d_inner]   (io)   inputs; delta is used as given
 *                                              (no softplus or bias inside)
 *   B, C        : [batch][L][d_state]   (io)   per-token rows shared by all channels
 *   A           : [d_inner][d_state]    fp32   decay rates (any finite value)
 *   D           : [d_inner]             fp32   skip weights
 *   h0          : [batch][d_inner][d_state] fp32, or NULL for a zero initial state
 *   y           : [batch][L][d_inner]   (io)   output
 *   hT          : [batch][d_inner][d_state] fp32 final state, or NULL.  hT may be
 *                 the same pointer as h0 (in-place carry); any other overlap
 *                 with an input or with y is JSCAN_ERR_ALIAS.
 *   workspace   : device scratch of at least jscan_prefill_workspace_size()
 *                 bytes, or NULL (the library then allocates and frees
 *                 stream-ordered scratch itself).  Its contents on entry do
 *                 not matter; it must not overlap any other argument.
 *
 * batch, L or d_inner may be 0: then nothing is computed, and if L == 0 the
 * final state hT is h0 (or zeros).  Sizes must be >= 0 (JSCAN_ERR_SHAPE).
 * Calling the prefill on consecutive pieces of a sequence, passing each
 * piece's hT as the next piece's h0, computes the scan of the whole sequence.
 */
jscan_status jscan_prefill(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                           const void* x, const void* delta, const float* A, const void* B,
                           const void* C, const float* D, const void* z, const float* h0,
                           void* y, float* hT, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * jscan_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and results as jscan_prefill without a workspace; the
 * chunked plan's records (per sequence, forward chunk and channel: 16 fp32
 * end states, a delta sum, a flag and 16 fp32 starting states, 136 bytes;
 * per sequence, chunk and 64-channel group two 4-byte token indices; a 256-byte
 * tag; each region rounded up to 256 bytes) live in a scratch
 * array of 64 MiB that the library holds on each GPU it runs on until the
 * process ends: batch * chunks * d_inner up to about 493 000 (at batch 1 and
 * d_inner 8192, plans of up to 60 chunks; the automatic plan there takes 32;
 * a one-chunk plan needs no records at all).  A larger problem returns
 * JSCAN_ERR_WORKSPACE before any GPU work, and jscan_last_error names the
 * bytes it needs.
 * The call allocates nothing (no hipMalloc, no stream-ordered allocation);
 * its first call on a device looks up the array's device address.  Every
 * call on one GPU shares the array: calls that overlap in time on one GPU
 * (on different streams) race and give wrong results.  Nothing in the array
 * needs to start at zero.  A prefill workspace written here cannot be passed
 * to jscan_backward_saved (it holds no sub-chunk records).
 */
jscan_status jscan_prefill_noalloc(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                                   const void* x, const void* delta, const float* A, const void* B,
                                   const void* C, const float* D, const void* z, const float* h0, void* y,
                                   float* hT, void* stream);

/*
 * Decode step for one sequence: one token, state updated in place.
 *
 *   state : [d_inner][d_state] fp32, read and overwritten with the new state
 *   x, delta, z, y : [d_inner] (io);  B, C : [d_state] (io);  A, D as above.
 *   y must not overlap any input or the state.
 */
jscan_status jscan_step(int64_t d_inner, int64_t d_state, jscan_io io, float* state,
                        const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, void* y, void* stream);

/*
 * Decode step for n_seq independent sequences (one token each), states updated
 * in place.
 *
 *   state : [n_seq][d_inner][d_state] fp32
 *   x, delta, z, y : [n_seq][d_inner] (io);  B, C : [n_seq][d_state] (io)
 *   A, D shared by all sequences, as above.
 *
 * n_seq * d_inner may be at most 2^30 - 64 (a 64 GiB state): the step runs
 * four lanes per (sequence, channel) in a one-dimensional grid, which holds at
 * most 2^32 work-items.  Larger products, and negative sizes, return
 * JSCAN_ERR_SHAPE before any GPU work; so do the fused and trapezoidal steps.
 */
jscan_status jscan_step_batch(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io,
                              float* state, const void* x, const void* delta, const float* A,
                              const void* B, const void* C, const float* D, const void* z,
                              void* y, void* stream);

/*
 * Optional input prologue of a Mamba layer, fused into the scan: the steps
 * Mamba-1/2 apply to x and delta before the recurrence, and the RMSNorm Jamba
 * adds to Mamba-internal activations ("Jamba: A Hybrid Transformer-Mamba
 * Language Model — 深度解读报告", sections 3.1 and 4.9, which do not say which
 * activations; here the time step and the B, C rows).  The "AI Engineering
 * from Scratch" Jamba lesson (section "Mamba-3") contrasts Mamba-3's
 * in-recurrence form with the "outer convolution on x_t" of the earlier
 * models; the pages give no kernel width (1..4 here, Mamba's usual 4).
 *
 *  - Causal depthwise convolution of x over the sequence, then SiLU:
 *      xc[t][d] = SiLU(conv_bias[d] + sum_k conv_weight[d][k] * x[t - (conv_width-1) + k][d])
 *    where x before the first token comes from conv_state_in (the previous
 *    call's last conv_width-1 raw x, [nseq][conv_width-1][d_inner] fp32;
 *    NULL = zeros).  The scan then uses xc wherever it used x (input term
 *    and D skip).  conv_state_out receives the last conv_width-1 raw x of
 *    this call (NULL: not written; it may be the same buffer as
 *    conv_state_in, for an in-place carry).  conv_weight NULL: no
 *    convolution (conv_bias and the conv states must then be NULL).
 *  - dt_softplus != 0: delta := softplus(delta + dt_bias[d]) =
 *    log(1 + exp(delta + dt_bias[d])) (dt_bias NULL: no bias).
 *
 * All prologue arrays are fp32 device pointers, 16-byte aligned.  nseq is
 * the batch (prefill) or n_seq (decode step).
 */
typedef struct {
  const float* conv_weight;   /* [d_inner][conv_width] */
  const float* conv_bias;     /* [d_inner] */
  const float* conv_state_in; /* [nseq][conv_width-1][d_inner] */
  float* conv_state_out;      /* [nseq][conv_width-1][d_inner] */
  const float* dt_bias;       /* [d_inner] */
  int32_t conv_width;         /* 1..4 */
  int32_t dt_softplus;        /* nonzero: softplus(delta + dt_bias) */
  /* RMSNorm before everything above, v_i / sqrt(mean_j v_j^2 + rms_eps) * w_i:
   * of delta over its d_inner channels per token, and of the B and C rows
   * over their d_state entries per token (NULL weight: not normalised).  The
   * normalised values are not rounded to the I/O dtype: a pre-pass writes,
   * in fp32, each token's inverse root-mean-square of delta and its
   * normalised B and C rows (132 bytes per token), and the scan applies
   * delta * w[d] * s[t] as it loads delta.  The prefill keeps these in its
   * workspace (jscan_prefill_workspace_size counts them); the decode step
   * in the workspace of jscan_step_batch_fused_ws, or else in scratch it
   * allocates and frees stream-ordered.  Not combined with the trapezoidal
   * form (JSCAN_ERR_UNSUPPORTED). */
  const float* rms_dt_weight; /* [d_inner] */
  const float* rms_B_weight;  /* [d_state] */
  const float* rms_C_weight;  /* [d_state] */
  float rms_eps;
} jscan_prologue;

/*
 * jscan_prefill with the input prologue above applied to x and delta (NULL
 * prologue = jscan_prefill).  Same arguments, layouts and errors otherwise;
 * a bad conv_width returns JSCAN_ERR_UNSUPPORTED.  Runs the scan with one
 * wave per 64 channels whatever the plan override says.
 */
jscan_status jscan_prefill_fused(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                                 const void* x, const void* delta, const float* A, const void* B,
                                 const void* C, const float* D, const void* z, const float* h0,
                                 void* y, float* hT, const jscan_prologue* prologue, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * jscan_step_batch with the input prologue (conv state [n_seq][conv_width-1]
 * [d_inner], normally updated in place: conv_state_out == conv_state_in).
 */
jscan_status jscan_step_batch_fused(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io,
                                    float* state, const void* x, const void* delta, const float* A,
                                    const void* B, const void* C, const float* D, const void* z,
                                    void* y, const jscan_prologue* prologue, void* stream);

/*
 * Bytes of device workspace jscan_step_batch_fused_ws needs for this
 * prologue: the RMSNorm rows of n_seq sequences (132 bytes per sequence,
 * rounded up), or 0 when the prologue normalises nothing (or d_state != 16,
 * or n_seq is outside 1 .. 2^30 - 64).
 */
size_t jscan_step_workspace_size(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io,
                                 const jscan_prologue* prologue);

/*
 * jscan_step_batch_fused with a caller workspace (16-byte aligned, device
 * memory, owned by the caller, not overlapping any other argument): with
 * RMSNorm the step then calls no allocator and can be captured in a HIP
 * graph.  workspace NULL: as jscan_step_batch_fused.  A workspace smaller
 * than jscan_step_workspace_size() returns JSCAN_ERR_WORKSPACE.  The
 * workspace holds nothing between calls.
 */
jscan_status jscan_step_batch_fused_ws(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io,
                                       float* state, const void* x, const void* delta, const float* A,
                                       const void* B, const void* C, const float* D, const void* z, void* y,
                                       const jscan_prologue* prologue, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * Exponential-trapezoidal recurrence (Mamba-3's discretisation).  The "AI
 * Engineering from Scratch" Jamba lesson (section "Mamba-3" and its
 * glossary) describes it only in words: a more expressive recurrence that
 * contains the Euler rule above as a special case and applies a
 * convolution-like operation to the state input inside the recurrence.  The
 * reading implemented: the input integral of one step is a weighted
 * two-point rule with the exponential kernel on the earlier point,
 *   h_t = a_t h_{t-1} + delta_t ((1 - lam_t) a_t B_{t-1} x_{t-1} + lam_t B_t x_t),
 *   a_t = exp(delta_t A),  y_t as in jscan_prefill,
 * so lam_t = 1 is jscan_prefill's recurrence and lam_t = 1/2 the trapezoidal
 * rule.  All arrays are device pointers in the I/O dtype, 16-byte aligned:
 *   lam    [nseq][L][d_inner]  weight lam_t (NULL: 1/2 everywhere)
 *   x_prev [nseq][d_inner]     x of the token before the first (NULL: zero)
 *   B_prev [nseq][d_state]     B row of that token (NULL: zero)
 * To continue a sequence, pass the last row of the previous call's x and B
 * (or, when decoding, the previous step's x and B).
 */
typedef struct {
  const void* lam;
  const void* x_prev;
  const void* B_prev;
} jscan_trap;

/*
 * jscan_prefill with the exponential-trapezoidal recurrence (trap NULL: all
 * fields NULL).  prologue may add softplus(delta + dt_bias); a convolution
 * prologue returns JSCAN_ERR_UNSUPPORTED (Mamba-3 moves that operation inside
 * the recurrence).  Otherwise as jscan_prefill_fused.
 */
jscan_status jscan_prefill_trap(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                                const void* x, const void* delta, const float* A, const void* B, const void* C,
                                const float* D, const void* z, const float* h0, void* y, float* hT,
                                const jscan_trap* trap, const jscan_prologue* prologue, void* workspace,
                                size_t workspace_bytes, void* stream);

/* jscan_step_batch with the exponential-trapezoidal recurrence (lam is
 * [n_seq][d_inner]). */
jscan_status jscan_step_batch_trap(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io, float* state,
                                   const void* x, const void* delta, const float* A, const void* B,
                                   const void* C, const float* D, const void* z, void* y,
                                   const jscan_trap* trap, const jscan_prologue* prologue, void* stream);

/*
 * Backward (gradient) of jscan_prefill, for training.  The pages describe
 * training Jamba ("Jamba: A Hybrid Transformer-Mamba Language Model — 深度解读
 * 报告", section 3.3 on the training infrastructure) but
 * give no backward; this is the reverse-mode derivative of the recurrence
 * above.  Given the forward's inputs and the gradients of a scalar loss with
 * respect to its outputs,
 *   dy  [batch][L][d_inner]           (I/O dtype)
 *   dhT [batch][d_inner][d_state] fp32 (NULL: zero; hT was not used),
 * it writes the gradients with respect to every input:
 *   dx, ddelta, dz [batch][L][d_inner] (I/O dtype)
 *   dA [d_inner][d_state] fp32, dD [d_inner] fp32 (summed over batch, tokens)
 *   dB, dC [batch][L][d_state] fp32 (summed over channels)
 *   dh0 [batch][d_inner][d_state] fp32 (NULL: not written; h0 NULL is a zero
 *        initial state and dh0 is still its gradient)
 * Every output is overwritten, never accumulated.  The forward states are
 * recomputed from the inputs (nothing is saved by jscan_prefill).
 *
 * Gradients (per sequence b, channel d, state n, with a_t = exp(delta_t A),
 * the forward states h_t, p_t = C_t . h_t + D x_t and dp_t = dy_t SiLU(z_t)):
 * the adjoint lambda_t = dp_t C_t + a_{t+1} lambda_{t+1} (lambda_{L-1} gets
 * + dhT) gives dx_t = D dp_t + delta_t (lambda_t . B_t), ddelta_t =
 * sum_n lambda_tn (A_n a_tn h_{t-1,n} + B_tn x_t), dz_t = dy_t p_t SiLU'(z_t),
 * dA_n = sum lambda_tn delta_t a_tn h_{t-1,n}, dD = sum dp_t x_t,
 * dB_tn = sum_d lambda_tn delta_t x_t, dC_tn = sum_d dp_t h_tn,
 * dh0 = a_0 lambda_0.
 *
 * workspace: NULL (allocated and freed stream-ordered) or at least
 * jscan_backward_workspace_size() bytes; it holds recomputed states (about 8
 * bytes per channel-token) and partial sums.  Errors as for jscan_prefill;
 * no output may overlap an input or another output.  Results do not depend
 * on scheduling (every sum is taken in a fixed order).
 */
size_t jscan_backward_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                                     jscan_io io);

jscan_status jscan_backward(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                            const void* x, const void* delta, const float* A, const void* B, const void* C,
                            const float* D, const void* z, const float* h0, const void* dy, const float* dhT,
                            void* dx, void* ddelta, void* dz, float* dA, float* dB, float* dC, float* dD,
                            float* dh0, void* workspace, size_t workspace_bytes, void* stream);

/*
 * jscan_backward for a training step that kept the workspace of its forward
 * call: prefill_workspace is the workspace a jscan_prefill call used (the
 * plain prefill, not the fused or trapezoidal one) with the same x, delta, A,
 * B, h0 and sizes, on the same thread's launch plan, unchanged since.  The
 * backward runs its sweeps on sub-chunks of the sequence whenever the batch's
 * channel groups alone cannot fill the GPU (every chunked prefill plan and
 * some single-chunk ones).  The prefill then records, in that workspace, the
 * chunk-local state at every sub-chunk boundary and the true state before
 * every chunk, and the backward derives each sub-chunk's starting state from
 * them instead of running a state-only pass over the sequence.  Otherwise the
 * workspace is not read.  The gradients equal jscan_backward's bit for bit.
 *
 * prefill_workspace: at least jscan_prefill_workspace_size() bytes (read
 * only; JSCAN_ERR_NULL if it is needed and NULL).  workspace: NULL or at
 * least jscan_backward_workspace_size() - jscan_prefill_workspace_size()
 * bytes.  Otherwise as jscan_backward; nothing may overlap prefill_workspace.
 *
 * A chunked prefill writes a tag at the start of its workspace (sizes, plan,
 * and which recurrence and prologue).  The backward compares it on the GPU:
 * a workspace from a prefill of other sizes, under another plan, or from the
 * fused or trapezoidal prefill makes every gradient NaN.  One that a plain
 * prefill of the same sizes and plan wrote over other inputs cannot be told
 * apart and gives wrong gradients.
 */
jscan_status jscan_backward_saved(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                                  const void* x, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* h0, const void* dy,
                                  const float* dhT, void* dx, void* ddelta, void* dz, float* dA, float* dB,
                                  float* dC, float* dD, float* dh0, const void* prefill_workspace,
                                  size_t prefill_workspace_bytes, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Static name of a status code. */
const char* jscan_status_string(jscan_status status);

/* Text of the last error reported on the calling thread ("" if none). */
const char* jscan_last_error(void);

/*
 * Launch plan the prefill uses for these sizes (on the calling thread, after
 * any override): the number of waves that share one group of 64 channels
 * (always 1: one wave owns all 16 states of its 64 channels) and the number
 * of sequence chunks scanned in parallel.  One chunk is a single pass; more
 * is pass 1 (every chunk from a zero state, recording its end state), the
 * carry combine, and pass 2 (chunks after the first rescanned from their true
 * starting state until the carried-in part has decayed below fp32 resolution;
 * the recurrence's Ā = exp(Δ·A) is the "Jamba lesson" "一页讲完 SSM" step).
 * Returns JSCAN_ERR_SHAPE for invalid sizes.
 */
jscan_status jscan_prefill_plan(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                                int* waves_per_group, int* chunks);

/*
 * Override the launch plan for the prefill calls (and workspace sizes) of the
 * calling thread: waves_per_group must be 1 and chunks in [1, 4096] (chunks
 * longer than L - 1 tokens collapse to fewer); (0, 0) restores the automatic
 * plan.  Results do not depend on the plan beyond floating-point rounding;
 * this exists to test and tune every variant.  Any other pair returns
 * JSCAN_ERR_UNSUPPORTED.
 */
jscan_status jscan_set_plan_override(int waves_per_group, int chunks);

/*
 * How much of the work of a chunked prefill fell to which pass, read from the
 * records the last prefill of these sizes left in `workspace` (a workspace
 * passed to jscan_prefill or jscan_prefill_fused on this thread's current
 * plan).  Synchronous: it copies the records to the host on `stream` and
 * waits for them.  stats (host, 3 doubles): [0] the fraction of the tokens of
 * chunks after the first that pass 1 scanned without writing y (before its
 * predicted point of decay), [1] the fraction pass 2 rescanned, [2] the number
 * of chunks.  A single-chunk plan gives 0, 0, 1.  JSCAN_ERR_WORKSPACE when the
 * workspace is smaller than the plan's records or holds no records of a
 * prefill of these sizes and plan; JSCAN_ERR_NULL, JSCAN_ERR_SHAPE as usual.
 */
jscan_status jscan_prefill_stats(const void* workspace, size_t workspace_bytes, int64_t batch, int64_t L,
                                 int64_t d_inner, double* stats, void* stream);

/*
 * Measurement hook.  When both events are non-NULL, the next jscan_prefill
 * call on this thread records `before` on its stream immediately before
 * launching its main scan kernel and `after` immediately after it, then
 * forgets the events.  Arguments are hipEvent_t handles.
 */
void jscan_time_next_prefill(void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* JSCAN_H */
