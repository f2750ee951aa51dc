/*
 * ssm.h -- C ABI of the MI355X (gfx950) selective-scan library (libssm.so).
 *
 * The library computes the Mamba (S6) selective scan and its single-token
 * recurrent state update.  For every batch row b, channel d and state n:
 *
 *     dA      = exp(delta[b,t,d] * A[d,n])                  (discretised A)
 *     h[n]    = dA * h[n] + delta[b,t,d] * B[b,t,n] * x[b,t,d]
 *     y[b,t,d] = sum_n C[b,t,n] * h[n] + Dskip[d] * x[b,t,d]
 *     y[b,t,d] = y[b,t,d] * z * sigmoid(z),  z = z[b,t,d]   (optional gate)
 *
 * Sources: the "selective_scan(x, delta, A, B, C, D)" listing and the
 * MambaBlock listing (gate y * silu(z)) on managen.ai, "Mamba: State Space
 * Models Challenge Transformers"; the MambaBlock._selective_scan listing on the
 * "State Space Models Mamba" skill page (A_bar = exp(delta A), B_bar = delta
 * B, readout after the update, skip term D u); the inference-mode update on
 * brentwoodlivery, "State-space models (Mamba, S4)", section "Training vs
 * Inference Modes".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers (HIP global memory) on the
 *   current device, contiguous and row-major, 16-byte aligned.
 * - Layouts: x, delta, z, y are [batch, seqlen, dim] with dim fastest;
 *   B and C are [batch, seqlen, dstate] with dstate fastest; A is [dim, dstate];
 *   Dskip is [dim]; every state (h0, h_last, h) is [batch, dim, dstate] fp32.
 * - `dtype` applies to x, delta, z, B, C and y.  A, Dskip and all states are fp32.
 *   bf16 outputs are rounded to nearest-even from the fp32 accumulator.
 * - The caller owns and allocates all memory, including the scan workspace
 *   (size from ssm_scan_workspace_bytes).  The library never allocates,
 *   frees or synchronises (but see SSM_SYNC below).
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *   Argument checks run on the host before any launch; a rejected call
 *   launches nothing and writes nothing.  Faults inside a kernel surface at
 *   the caller's next synchronisation.
 * - Return value: an ssm_status.  On anything but SSM_OK a one-line reason is
 *   available from ssm_last_error() (per thread).  Nothing aborts, throws
 *   across the ABI or prints (but see SSM_LOG below).
 * - Debugging aids, read once from the environment: SSM_LOG=1 prints one line per
 *   call on stderr saying what the call launches (kernel path, plan, workspace);
 *   SSM_SYNC=1 makes every launch wait for its stream, so that a kernel that fails
 *   is reported as SSM_EHIP by the call that launched it.
 * - Thread safety: the library holds no global state beyond the per-thread
 *   error text; concurrent calls on different streams are independent.
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 7
#define SSM_MAX_DSTATE 256

typedef enum ssm_dtype {
    SSM_DTYPE_F32 = 0,
    SSM_DTYPE_BF16 = 1
} ssm_dtype;

typedef enum ssm_status {
    SSM_OK = 0,
    SSM_EINVAL = 1,        /* bad shape, null or misaligned pointer, overlapping output */
    SSM_EUNSUPPORTED = 2,  /* valid request the library does not implement (e.g. dstate > 16) */
    SSM_EWORKSPACE = 3,    /* workspace missing or smaller than ssm_scan_workspace_bytes() */
    SSM_EHIP = 4           /* the HIP runtime refused a launch */
} ssm_status;

/*
 * How the continuous parameters (A, B) become the discrete step (A_bar, B_bar)
 * for step size dt, A diagonal (one value a = A[d,n] per state):
 *   SSM_DISC_MAMBA     A_bar = exp(dt a), B_bar = dt B.  The first-order B_bar of
 *                      the Mamba listings (managen.ai "Selective Scan Algorithm";
 *                      skill page MambaBlock._selective_scan).  The default.
 *   SSM_DISC_ZOH       A_bar = exp(dt a), B_bar = (exp(dt a) - 1) / a * B, and dt B
 *                      where a = 0 (zero-order hold: skill page "Discretization"
 *                      docstring; brentwoodlivery "From Continuous to Discrete").
 *   SSM_DISC_BILINEAR  A_bar = (1 + dt a / 2) / (1 - dt a / 2),
 *                      B_bar = dt / (1 - dt a / 2) * B (chipfoundryservices glossary
 *                      "State Space Models & Mamba", Lab 1).  Defined while
 *                      dt a / 2 != 1, i.e. for every dt when a <= 0.
 */
typedef enum ssm_discretization {
    SSM_DISC_MAMBA = 0,
    SSM_DISC_ZOH = 1,
    SSM_DISC_BILINEAR = 2
} ssm_discretization;

/* Optional variant of the recurrence for ssm_scan_fwd and ssm_state_update.  A NULL
 * pointer means { SSM_DISC_MAMBA, 0, NULL }. */
typedef struct ssm_variant {
    int32_t discretization;    /* an ssm_discretization */
    int32_t reserved;          /* must be 0 */
    const float *delta_bias;   /* [dim] fp32 device pointer, added to delta before the
                                  softplus (the bias of the linear map that produces delta:
                                  skill page, MambaBlock listing, dt_proj); NULL = none */
} ssm_variant;

/* Optional tuning of ssm_scan_fwd.  A NULL pointer or a zero field means
 * "choose automatically".  None of these change the result beyond fp32
 * rounding order. */
typedef struct ssm_scan_opts {
    int64_t chunk_len;     /* length of the sequence chunks scanned in parallel (>= 1) */
    int32_t states_per_lane; /* 1, 2, 4, 8 or 16 states of one channel per GPU lane */
    int32_t time_block;    /* time steps staged per block: 8, 16 or 32 (the generic kernel of
                              the ZOH and bilinear variants always stages 8) */
    int32_t one_block_per_cu; /* 0: automatic; 1: reserve LDS so each CU runs one workgroup; -1: never */
    int32_t a_structure;   /* 0: automatic -- with the Mamba discretisation and dstate 16, a
                              workgroup whose channels all satisfy A[d, n + k] - A[d, n] =
                              A[d, k] - A[d, 0] (k = 16 / states_per_lane; e.g. A[d,n] = -(n+1))
                              forms exp(dt A[d, n + k]) as exp(dt A[d, n]) * exp(dt (A[d,k] -
                              A[d,0])): one exp per lane and step instead of one per state.  The
                              check runs on the device.  -1: always one exp per state. */
} ssm_scan_opts;

/* What ssm_scan_fwd will launch for a given shape (host-only query). */
typedef struct ssm_scan_plan {
    int64_t chunk_len;
    int64_t n_chunks;        /* 1 = single pass; > 1 = chunk carries + combine + rescan */
    int32_t states_per_lane;
    int32_t waves_per_block;
    int32_t time_block;
    int32_t specialised;     /* 1: the dstate == 16, dim % 64 == 0 kernel runs; 0: the generic one */
    uint64_t workspace_bytes;
    uint64_t blocks;         /* workgroups of the main scan launch */
    uint64_t lds_reserve;    /* extra LDS bytes per workgroup that keep one workgroup per CU (0 = none) */
} ssm_scan_plan;

/*
 * Issue-rate probe (measurement only; the scan does not call it).  Launches `workgroups`
 * workgroups of `waves_per_workgroup` waves in which every lane runs 8 independent chains of
 * `iters` operations: op 0 an fp32 FMA, op 1 v_exp_f32, op 2 v_rcp_f32.  The caller times the
 * launch on `stream` (e.g. with events) and divides 64 * waves * workgroups * 8 * iters by
 * the time.  Whether the scan is bound by memory (as the skill page "State Space Models
 * Mamba" has it in its "SSM vs Transformer" table and Common Pitfalls) or by the ALU turns
 * on these rates: a state update is one exp plus four multiplies or FMAs.  `sink` is a
 * device buffer of at least 64 * waves_per_workgroup floats that the kernel may write.
 * Returns SSM_EINVAL for out-of-range arguments.
 */
int ssm_issue_probe(int op, int64_t workgroups, int64_t waves_per_workgroup, int64_t iters, float *sink,
                    void *stream);

/* ABI version of the loaded library (SSM_ABI_VERSION at build time). */
int ssm_abi_version(void);

/* Static text for a status code ("ok", "invalid argument", ...). */
const char *ssm_status_str(int status);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char *ssm_last_error(void);

/* Host-only: fill *plan for this shape.  Returns SSM_OK, or the status the
 * same shape would get from ssm_scan_fwd's shape checks. */
int ssm_scan_plan_get(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                      const ssm_scan_opts *opts, ssm_scan_plan *plan);

/* Host-only: bytes of device workspace ssm_scan_fwd needs for this shape and
 * these options (0 when the scan runs in one pass, or the shape is invalid). */
size_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                int dtype, const ssm_scan_opts *opts);

/*
 * Selective scan over a whole sequence (training / prefill form).
 *
 * Defines y[b,t,d] for t in [0, seqlen) by the recurrence above, starting
 * from h = h0[b,d,:] (or zeros when h0 is NULL), and stores the final state
 * in h_last (when not NULL).  The sequence is cut into chunks scanned in
 * parallel; chunk carries (product of dA over the chunk, end state from
 * zero) are combined with the associative operator
 *     (P1, H1) o (P2, H2) = (P2 * P1, P2 * H1 + H2)
 * (the parallel associative scan of the skill page's "Hardware-Efficient
 * Scan" section, with the operator derived from its recurrence).
 *
 *   x, delta  [batch, seqlen, dim]   dtype   required
 *   A         [dim, dstate]          fp32    required; finite, usually <= 0
 *   B, C      [batch, seqlen, dstate] dtype  required
 *   Dskip     [dim]                  fp32    NULL = no skip term
 *   z         [batch, seqlen, dim]   dtype   NULL = no output gate
 *   h0        [batch, dim, dstate]   fp32    NULL = zero start state
 *   h_last    [batch, dim, dstate]   fp32    NULL = not stored; must not overlap h0
 *   y         [batch, seqlen, dim]   dtype   output; must not overlap any input
 *   delta_softplus  0: delta is the step size;  1: step size = log(1 + exp(delta))
 *   variant   NULL (Mamba discretisation, no delta bias) or see ssm_variant; the
 *             step size is then delta + delta_bias[d], before the softplus
 *   opts      NULL or tuning (see ssm_scan_opts)
 *   workspace device memory of ssm_scan_workspace_bytes() bytes (NULL if 0)
 *
 * batch, seqlen or dim == 0 is a valid no-op (with seqlen == 0, h_last
 * receives h0 or zeros).  1 <= dstate <= SSM_MAX_DSTATE (256), else SSM_EINVAL (< 1)
 * or SSM_EUNSUPPORTED (> 256); dstate 16 with dim a multiple of 64 runs the specialised
 * kernel, every other shape the generic one.
 */
int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                 const void *x, const void *delta, const float *A, const void *B,
                 const void *C, const float *Dskip, const void *z, const float *h0,
                 float *h_last, void *y, int delta_softplus, const ssm_variant *variant,
                 const ssm_scan_opts *opts, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssm_scan_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It takes no workspace:
 * its workspace is a fixed device array of ssm_noalloc_scratch_bytes() bytes (64 MiB) that
 * the library holds on every GPU it runs on until the process ends.  The call allocates
 * and frees nothing.  A shape whose workspace (ssm_scan_workspace_bytes with the same
 * opts) exceeds the array returns SSM_EWORKSPACE before any launch.  Every call on one
 * GPU shares that GPU's array, so calls that overlap on one GPU (on different streams, or
 * from threads the caller does not order) race: the caller must serialise them.  All
 * other arguments, results and errors are those of ssm_scan_fwd.
 */
size_t ssm_noalloc_scratch_bytes(void);
int ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                         const void *x, const void *delta, const float *A, const void *B,
                         const void *C, const float *Dskip, const void *z, const float *h0,
                         float *h_last, void *y, int delta_softplus, const ssm_variant *variant,
                         const ssm_scan_opts *opts, void *stream);

/*
 * Single-token recurrent state update (generation form): one step of the
 * recurrence for every (b, d), with the state kept in HBM between calls.
 * brentwoodlivery, "Training vs Inference Modes": keep h_{k-1}, receive x_k,
 * update h_k, emit y_k, constant work per token.
 *
 *   h         [batch, dim, dstate]   fp32    read and overwritten in place
 *   x, delta  [batch, dim]           dtype   required
 *   A         [dim, dstate]          fp32    required
 *   B, C      [batch, dstate]        dtype   required
 *   Dskip     [dim]                  fp32    NULL = no skip term
 *   z         [batch, dim]           dtype   NULL = no output gate
 *   y         [batch, dim]           dtype   output; must not overlap any input or h
 *   delta_softplus, variant          as for ssm_scan_fwd
 *
 * L consecutive calls give the same y and final h as one ssm_scan_fwd over
 * those L tokens (up to fp32 rounding order).
 */
int ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int dtype, float *h,
                     const void *x, const void *delta, const float *A, const void *B,
                     const void *C, const float *Dskip, const void *z, void *y,
                     int delta_softplus, const ssm_variant *variant, void *stream);

/*
 * Host-only: sizes for ssm_scan_fwd_save at this shape: the device workspace it needs
 * (*workspace_bytes, 0 when none) and the bytes of its checkpoint output
 * (*checkpoint_bytes = batch * ceil(seqlen / 8) * 16 * dim * 4).  Both are set to 0 and
 * an ssm_status returned when the shape is invalid or unsupported (dstate must be 16 and
 * dim a multiple of 64, as for ssm_scan_bwd); SSM_EINVAL when either pointer is NULL.
 */
int ssm_scan_save_sizes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                        size_t *workspace_bytes, size_t *checkpoint_bytes);

/*
 * ssm_scan_fwd that also stores what ssm_scan_bwd would otherwise recompute: the state
 * h before every 8th step (t = 0, 8, 16, ...), for the reverse sweep of a training step.
 * Same recurrence, arguments, layouts and results as ssm_scan_fwd (y and h_last agree
 * with it up to the rounding of a different sequence chunking, bit for bit when neither
 * call splits the sequence), without ssm_scan_opts: the sequence is chunked as the
 * backward chunks it.  Additionally
 *   checkpoints  [batch][ceil(seqlen/8)][16][dim] fp32, device memory owned by the
 *                caller, ssm_scan_save_sizes() bytes, 16-byte aligned, overlapping no
 *                other argument; fully overwritten.  Entry [b][k][n][d] is the state
 *                of (b, d, n) before step 8k.
 *   workspace    device memory of ssm_scan_save_sizes() bytes (NULL if 0)
 * dstate must be 16 and dim a multiple of 64, else SSM_EUNSUPPORTED.  seqlen == 0 sets
 * h_last = h0 (or zeros) and stores no checkpoints.
 */
int ssm_scan_fwd_save(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                      const void *x, const void *delta, const float *A, const void *B,
                      const void *C, const float *Dskip, const void *z, const float *h0,
                      float *h_last, void *y, int delta_softplus, const ssm_variant *variant,
                      float *checkpoints, void *workspace, size_t workspace_bytes, void *stream);

/* Host-only: bytes of device workspace ssm_scan_bwd needs for this shape (0 when
 * nothing is computed, or the shape is invalid or unsupported); with
 * saved_checkpoints != 0, for a call given checkpoints (less: no checkpoint pass).  For
 * shapes other than dstate 16 with dim a multiple of 64 it includes the padded copies. */
size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                    int dtype, int saved_checkpoints);

/*
 * Backward pass of ssm_scan_fwd: gradients of a loss with respect to every input,
 * given dy = dLoss/dy and (optionally) dh_last = dLoss/dh_last.  Reverse-mode
 * derivative of the recurrence above (the skill page's Verification Checklist asks
 * for gradients through the step size; the step is the managen.ai page's "Selective
 * Scan Algorithm"): with lam = dLoss/dh after step t, running t backwards,
 *     lam += C_t gy0,  gy0 = dy_t * silu(z_t) (dy_t without a gate)
 *     dC_t += gy0 h_t,   dB_t += lam dt x_t,   dA += lam dt exp(dt A) h_{t-1}
 *     dx_t = D gy0 + dt sum_n lam B_t,  ddelta_t = sum_n lam (A exp(dt A) h_{t-1} + B_t x_t)
 *     lam = exp(dt A) lam,   dh0 = lam after t = 0
 * (ddelta_t is multiplied by sigmoid(delta_t + delta_bias) in softplus mode: the
 * derivative with respect to the raw input).  That is the Mamba discretisation; with
 * SSM_DISC_ZOH or SSM_DISC_BILINEAR the chain rule runs through that map's A_bar(dt, a)
 * and B_bar = f(dt, a) B instead (dB_t += lam f x_t, dx_t = D gy0 + sum_n lam f B_t,
 * ddelta_t = sum_n lam (dA_bar/ddt h_{t-1} + df/ddt B_t x_t),
 * dA += lam (dA_bar/da h_{t-1} + df/da B_t x_t), lam = A_bar lam).
 *
 * Inputs as ssm_scan_fwd (same layouts and dtypes), plus
 *   dy        [batch, seqlen, dim]   dtype   required
 *   dh_last   [batch, dim, dstate]   fp32    NULL = zero
 *   discretization                   an ssm_discretization (as the forward call's
 *             variant); any other value is SSM_EINVAL
 *   delta_bias [dim]                 fp32    NULL = no bias; else the step size is
 *             delta + delta_bias[d] (before the softplus), as in ssm_variant
 * Outputs (device memory owned by the caller; none may overlap an input or another
 * output; each is fully overwritten):
 *   dx, ddelta [batch, seqlen, dim]  dtype   required
 *   dz        [batch, seqlen, dim]   dtype   required when z is given, else ignored
 *   dB, dC    [batch, seqlen, dstate] dtype  required (sums over dim)
 *   dA        [dim, dstate]          fp32    required (sum over batch and time)
 *   dD        [dim]                  fp32    required when Dskip is given, else ignored
 *   dh0       [batch, dim, dstate]   fp32    NULL = not stored
 *   ddelta_bias [dim]                fp32    required when delta_bias is given, else
 *             ignored: the sum of ddelta over batch and time
 *   checkpoints  NULL: the call first runs the forward again, storing the state before
 *             every 8th step in its workspace; else the checkpoints that ssm_scan_fwd_save
 *             stored for these same inputs (x, delta, A, B, C, h0, delta_softplus,
 *             discretisation, delta_bias), read only.  Checkpoints of other inputs give
 *             meaningless gradients; nothing can detect that.
 *   workspace device memory of ssm_scan_bwd_workspace_bytes(..., checkpoints != NULL)
 *             bytes (partial sums, and without saved checkpoints the checkpoints)
 *
 * Any 1 <= dstate <= 256 (more is SSM_EUNSUPPORTED) and any dim.  dstate == 16 with dim a
 * multiple of 64 runs the native kernels in place; dstate < 16 or other dims run them on
 * copies padded (in the workspace) to the next multiple of 64 channels and to 16 states,
 * whose padding carries x = 0 and B = C = 0 and so adds nothing to any gradient; dstate >
 * 16 runs them once per group of 16 states on fp32 copies (the states of one group neither
 * read nor write another's), with dx, ddelta, dz and ddelta_bias summed over the groups in
 * fp32 and D's terms taken in the first group only.  Shapes other than dstate == 16 with
 * dim a multiple of 64 take no saved checkpoints (SSM_EUNSUPPORTED).  dim == 0 is a no-op; batch == 0 or seqlen == 0 sets
 * dA, dD, ddelta_bias to zero (and, with seqlen == 0, dh0 = dh_last or zeros).
 * Deterministic: every reduction runs in a fixed order.
 */
int ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                 const void *x, const void *delta, const float *A, const void *B,
                 const void *C, const float *Dskip, const void *z, const float *h0,
                 const void *dy, const float *dh_last, void *dx, void *ddelta, float *dA,
                 void *dB, void *dC, float *dD, void *dz, float *dh0, int delta_softplus,
                 int discretization, const float *delta_bias, float *ddelta_bias,
                 const float *checkpoints, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Causal depthwise convolution along the sequence, then SiLU: the step before the scan
 * in a Mamba block (skill page "State Space Models Mamba", MambaBlock listing: Conv1d
 * with kernel size d_conv, padding d_conv - 1 and one group per channel, its output cut
 * to the sequence length, then silu).  With W = width and xp the W - 1 inputs before
 * the sequence (state_in, or zeros) followed by x:
 *     y[b,t,d] = silu(bias[d] + sum_{k<W} w[d,k] * xp[b, t+k, d])     (silu = 1)
 *     y[b,t,d] =      bias[d] + sum_{k<W} w[d,k] * xp[b, t+k, d]      (silu = 0)
 *     state_out[b,d,:] = the last W - 1 values of xp[b, :, d]   (oldest first)
 *
 *   x         [batch, seqlen, dim]   dtype   required when seqlen > 0
 *   w         [dim, width]           fp32    required
 *   bias      [dim]                  fp32    NULL = no bias
 *   state_in  [batch, dim, width-1]  dtype   NULL = zeros before the sequence
 *   y         [batch, seqlen, dim]   dtype   output; must not overlap an input
 *   state_out [batch, dim, width-1]  dtype   NULL = not stored; must not overlap an input
 * 1 <= width <= 4 (SSM_EUNSUPPORTED above).  batch or dim == 0 is a no-op; seqlen == 0
 * only passes state_in (or zeros) to state_out.
 */
int ssm_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                   const void *x, const float *w, const float *bias, const void *state_in,
                   void *y, void *state_out, int silu, void *stream);

/* Host-only: bytes of device workspace ssm_conv1d_bwd needs (0 when nothing is
 * computed or the shape is invalid). */
size_t ssm_conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                                      int dtype);

/*
 * Backward of ssm_conv1d_fwd: gradients of a loss given dy = dLoss/dy, by the chain
 * rule through the same definition (the final state is not differentiated):
 *     g = dy * silu'(a) (dy when silu == 0),   silu'(a) = s (1 + a (1 - s)), s = sigmoid(a)
 *     dx[t] = sum_k w[d,k] g[t + W - 1 - k]  (terms with t + W - 1 - k < seqlen)
 *     dw[d,k] = sum_{b,t} g[t] xp[t + k],   dbias[d] = sum_{b,t} g[t]
 *     dstate[b,d,j] = sum_k w[d,k] g[j - k]  (the gradient of state_in, j < width-1)
 *
 * Inputs as ssm_conv1d_fwd (x, w, bias, state_in, silu), plus
 *   dy        [batch, seqlen, dim]   dtype   required
 * Outputs (device memory owned by the caller, fully overwritten, none overlapping an
 * input or another output):
 *   dx        [batch, seqlen, dim]   dtype   required
 *   dw        [dim, width]           fp32    required
 *   dbias     [dim]                  fp32    NULL = not computed (allowed with bias NULL)
 *   dstate    [batch, dim, width-1]  dtype   NULL = not computed (allowed with state_in NULL:
 *             the gradient of a zero starting state)
 *   workspace device memory of ssm_conv1d_bwd_workspace_bytes() bytes (per-tile sums)
 * batch == 0 or seqlen == 0 sets dw, dbias, dstate to zero; dim == 0 is a no-op.
 * Deterministic: the sums run in a fixed order.
 */
int ssm_conv1d_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                   const void *x, const float *w, const float *bias, const void *state_in,
                   const void *dy, void *dx, float *dw, float *dbias, void *dstate, int silu,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * One token of ssm_conv1d_fwd (generation form): state [batch, dim, width-1] (dtype,
 * oldest input first) is read and updated in place, x and y are [batch, dim].
 * L consecutive calls give the same y and final state as one ssm_conv1d_fwd over those
 * L tokens.
 */
int ssm_conv1d_update(int64_t batch, int64_t dim, int64_t width, int dtype, void *state,
                      const void *x, const float *w, const float *bias, void *y, int silu,
                      void *stream);

/*
 * Multi-head SSD scan: the state space model of a Mamba-2 layer (managen.ai, "Mamba:
 * State Space Models Challenge Transformers", Mamba2Block: heads of d_head = 64
 * channels, d_state = 128; brentwoodlivery, "State-space models (Mamba, S4)", section
 * "Mamba 2 and Hybrid Architectures": the SSM as a structured matrix multiplication).
 * For every batch row b, head h, channel p < headdim and state n < dstate:
 *
 *     dt       = delta[b,t,h] (+ delta_bias[h]; log(1 + exp(.)) of it when delta_softplus)
 *     S[p,n]   = exp(dt * A[h]) * S[p,n] + dt * B[b,t,n] * x[b,t,h,p]
 *     y[b,t,h,p] = sum_n C[b,t,n] * S[p,n] + Dskip[h] * x[b,t,h,p],  then * silu(z) if gated
 *
 * i.e. the recurrence of ssm_scan_fwd with one step size and one scalar decay per
 * head.  The heads fall into ngroups groups of nheads / ngroups consecutive heads, and
 * the heads of a group share one B and one C row per token: head h reads group
 * g = h / (nheads / ngroups) (ngroups = 1: every head shares B and C).
 *
 *   x, z      [batch, seqlen, nheads, headdim]  bf16   z NULL = no gate
 *   delta     [batch, seqlen, nheads]           bf16
 *   A, Dskip, delta_bias  [nheads]              fp32   Dskip, delta_bias may be NULL
 *   B, C      [batch, seqlen, ngroups, dstate]  bf16
 *   h0, h_last [batch, nheads, headdim, dstate] fp32   NULL = zero start / not stored
 *   y         [batch, seqlen, nheads, headdim]  bf16   output; must not overlap an input
 *
 * headdim 64, dstate 128, bf16: the matrix-core kernel.  Any other headdim >= 1, dstate <=
 * 256 (more is SSM_EUNSUPPORTED), and fp32 (dtype SSM_DTYPE_F32 for x, z, delta, B, C, y):
 * the generic scan kernel over the nheads * headdim channels, one pass; with ngroups > 1
 * it needs (nheads / ngroups) * headdim to be a multiple of 64 (else SSM_EUNSUPPORTED).
 * ngroups must be >= 1 and divide nheads (else SSM_EINVAL).  No workspace.
 * seqlen == 0 stores h0 (or zeros) in h_last; batch or nheads == 0 is a no-op.
 */
int ssm_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                int64_t ngroups, int dtype, const void *x, const void *delta, const float *A, const void *B,
                const void *C, const float *Dskip, const void *z, const float *delta_bias,
                const float *h0, float *h_last, void *y, int delta_softplus, void *stream);

/* Bytes of device workspace ssm_ssd_bwd needs for this shape (0 when nothing is
 * computed or the shape is invalid). */
size_t ssm_ssd_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                   int64_t dstate, int dtype);

/*
 * Backward pass of ssm_ssd_fwd for one B/C group: gradients of a loss with respect to
 * every input, given dy = dLoss/dy and (optionally) dh_last = dLoss/dh_last.  The layer is
 * the selective scan of ssm_scan_fwd over the nheads * headdim channels (pages: managen.ai
 * Mamba2Block, brentwoodlivery "Mamba 2 and Hybrid Architectures"), with each head's step
 * size delta[b, t, h], decay a_h, D_h and bias tied over its headdim channels and B, C
 * shared by all heads; so the gradients are those of ssm_scan_bwd on the per-channel
 * expansion, with the tied ones (ddelta, dA, dD, ddelta_bias) summed over each head's
 * channels.  The call runs exactly that: fp32 copies of the expansion in the workspace,
 * ssm_scan_bwd on them (up to 256 states: groups of 16), then the per-head sums in a fixed
 * order (deterministic).
 *   inputs   x, delta, A, B, C, Dskip, z, delta_bias, h0, delta_softplus: as for ssm_ssd_fwd
 *            with ngroups == 1 (several groups: SSM_EUNSUPPORTED); dy [B, L, H, P] (dtype),
 *            dh_last [B, H, P, N] fp32 or NULL
 *   outputs  dx, dz [B, L, H, P] and ddelta [B, L, H] and dB, dC [B, L, N] in dtype;
 *            dA, dD, ddelta_bias [H] and dh0 [B, H, P, N] fp32.  dD, dz, ddelta_bias are
 *            required exactly when Dskip, z, delta_bias are given; dh0 may be NULL.
 *   workspace device memory of ssm_ssd_bwd_workspace_bytes(...) bytes
 * Pointers are caller-owned device memory; asynchronous on stream.  batch == 0 or seqlen == 0
 * writes dA, dD, ddelta_bias as zeros and (seqlen == 0) dh0 = dh_last or zeros.
 * Not tuned: it costs ceil(N / 16) scan backwards over the H * P channels plus the copies;
 * a reverse kernel on the matrix cores would be the fast form.
 */
int ssm_ssd_bwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                int64_t ngroups, int dtype, const void *x, const void *delta, const float *A, const void *B,
                const void *C, const float *Dskip, const void *z, const float *delta_bias,
                const float *h0, const void *dy, const float *dh_last, void *dx, void *ddelta, float *dA,
                void *dB, void *dC, float *dD, void *dz, float *ddelta_bias, float *dh0,
                int delta_softplus, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
