/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective-SSM scan library.
 *
 * The operation (page "Mamba 논문 리뷰: Selective State Space Models로
 * Transformer를 넘어서", youngju.dev):
 *   section 3.1  delta_t = softplus(raw_delta_t + delta_bias)   (selection)
 *   section 2.2  Abar = exp(delta A)                            (discretisation)
 *   section 3.3  Bbar x = delta B_t x_t  (Euler input term of the listing)
 *   section 2.2  h_t = Abar o h_{t-1} + Bbar x_t, y_t = C_t . h_t
 *   section 3.4  y_t += D x_t, then y_t *= SiLU(z_t)             (block)
 * per batch row b, channel d and state n, with a diagonal fp32 state of size N
 * per channel.  Tensor contract of the section 3.3 listing: x, delta (B, L, D);
 * A (D, N); B, C (B, L, N); plus D, z and delta_bias of the block.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; every tensor
 *     is dense, row-major, with the last index fastest.  The library never
 *     allocates, frees or retains them, and keeps no global mutable state.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising.  Argument errors are detected on
 *     the host before any HIP call and nothing is enqueued; faults during
 *     execution surface at the caller's next synchronisation.
 *   - Return value: SSM_OK (0) or a negative SSM_ERR_* code.
 */
#ifndef SSM_SCAN_H_
#define SSM_SCAN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_SCAN_ABI_VERSION 4

/* Element type of x, delta, B, C, z and y.  A, D, delta_bias, h0, hT are
 * always fp32, and all arithmetic (state, accumulation) is fp32. */
typedef enum ssm_dtype { SSM_DTYPE_F32 = 0, SSM_DTYPE_BF16 = 1 } ssm_dtype;

enum ssm_status {
  SSM_OK = 0,
  SSM_ERR_NULL = -1,      /* a required pointer (args, x, delta, A, B, C, y) is NULL      */
  SSM_ERR_SHAPE = -2,     /* an extent is negative, or an element count overflows int64   */
  SSM_ERR_DSTATE = -3,    /* dstate N outside 1..64                                       */
  SSM_ERR_DTYPE = -4,     /* dtype not one of ssm_dtype                                   */
  SSM_ERR_ALIGN = -5,     /* a tensor base address is not 16-byte aligned                 */
  SSM_ERR_ALIAS = -6,     /* y overlaps an input, or hT overlaps an input other than h0   */
  SSM_ERR_WORKSPACE = -7, /* time_splits > 1 asked for but workspace is NULL or too small */
  SSM_ERR_LAUNCH = -8,    /* the HIP launch failed (hipGetLastError after the launch)     */
  SSM_ERR_VARIANT = -9,   /* variant / flags / time_splits not valid for this problem     */
};

/* Kernel family (SSM_VARIANT_AUTO picks one from the problem shape). */
enum ssm_variant {
  SSM_VARIANT_AUTO = 0,
  SSM_VARIANT_NSPLIT = 1, /* 8 waves share 64 channels: 4 hold N/4 states each, 4 do the per-token
                             work (N in {4, 8, 16, 32, 64}; time splitting)                      */
  SSM_VARIANT_LANE = 2,   /* one lane owns one channel and all N states; any N <= 64           */
  SSM_VARIANT_DECODE = 3, /* seqlen == 1 only: N/4 lanes per channel (N % 4 == 0)              */
};

/* Option bits. */
enum ssm_flags {
  /* Never take the structured-A fast path (decay of state n computed as the
   * (n+1)-th power of the decay of state 0 when A[d,n] == (n+1) A[d,0] holds
   * exactly for a channel block); every Abar is then its own exp. */
  SSM_FLAG_GENERIC_A = 1,
  /* Zero-order-hold input term (section 2.2: Bbar = (delta A)^-1
   * (exp(delta A) - I) delta B) instead of the Euler term delta B: state n
   * receives (exp(delta A[d,n]) - 1) / A[d,n] * B[n] * x (delta * B[n] * x where
   * A[d,n] == 0).  ssm_scan_bwd takes it too and differentiates that
   * forward (dc/ddelta = exp(delta A), dc/dA = (delta exp(delta A) - c) / A
   * for c the coefficient above). */
  SSM_FLAG_ZOH = 2,
  /* Time-split calls only: compose the segments' summaries with a
   * wave-level associative scan in one extra launch (DPP row shifts and
   * broadcasts over the segments, the operator (a1,b1) o (a2,b2) =
   * (a1 a2, a2 b1 + b2)), so that each segment reads the state entering it,
   * instead of folding the summaries before it one after the other (the
   * default, measured faster for up to 64 segments).  Results agree to
   * rounding. */
  SSM_FLAG_CARRY_SCAN = 4,
};

typedef struct ssm_scan_args {
  int64_t batch;   /* B >= 0                                                     */
  int64_t seqlen;  /* L >= 0                                                     */
  int64_t dim;     /* D >= 0: channels                                           */
  int64_t dstate;  /* N, 1..64                                                   */
  int32_t dtype;   /* ssm_dtype of x, delta, B, C, z, y                          */
  int32_t flags;   /* ssm_flags bits                                             */
  const void *x;           /* (B, L, D) input                          required */
  const void *delta;       /* (B, L, D) raw step size, before bias and softplus, required */
  const float *A;          /* (D, N) fp32, used as given (normally < 0)        required */
  const void *B;           /* (B, L, N) input matrix per token                 required */
  const void *C;           /* (B, L, N) output matrix per token                required */
  const float *D;          /* (D) skip weight; NULL = no skip term                     */
  const void *z;           /* (B, L, D) gate input; NULL = no gate                     */
  const float *delta_bias; /* (D); NULL = zero bias                                    */
  const float *h0;         /* (B, D, N) initial state; NULL = zeros                    */
  float *hT;               /* (B, D, N) final state out; NULL = not returned; may equal h0 (in place) */
  void *y;                 /* (B, L, D) output, same dtype as x                required */
  void *workspace;         /* device scratch for time splitting; may be NULL           */
  int64_t workspace_bytes; /* size of workspace in bytes                               */
  int32_t variant;         /* ssm_variant; 0 = automatic                               */
  int32_t time_splits;     /* segments per sequence: 0 = automatic, 1 = none, >1 = that many (NSPLIT only) */
  float *checkpoints;      /* states for ssm_scan_bwd, or NULL (see below)              */
} ssm_scan_args;

/* Checkpoints.  A training forward can hand the backward the states it
 * passes through, so that ssm_scan_bwd does not run the forward recurrence
 * again (section 3.3's recomputation is then limited to the few tokens
 * inside each chunk).  With T = 8 tokens per chunk (16 when N <= 4), entry
 * i of `checkpoints` holds the state after token (i + 1) T - 1, i.e. the
 * state entering chunk i + 1; the state entering chunk 0 is h0.  The states
 * of an entry are cut into four quarters of M = ceil(N / 4): state n of
 * channel d sits at [b][i][n / M][d][n % M] of a (B, ceil(L / T) - 1, 4, D, M)
 * fp32 array (the layout in which the forward's four state-holding waves each
 * write one contiguous block), ssm_scan_checkpoint_bytes bytes, 16-byte
 * aligned, not overlapping any other tensor.  Every position of a state
 * n < N is written.  The states are the ones the forward computes for y (time
 * splitting included), in the discretisation its flags select. */
int64_t ssm_scan_checkpoint_bytes(const ssm_scan_args *args);

/* Forward selective scan, y (and optionally hT) from the inputs above.
 * With seqlen == 0, y is empty and hT (if given) receives h0 (or zeros).
 * With batch == 0 or dim == 0 there is nothing to compute and SSM_OK is
 * returned.  When time splitting is used (automatic or requested), segment
 * summaries go to `workspace`; with automatic splitting and no (or too small)
 * workspace the call runs unsplit instead.  Deterministic: the same inputs
 * give bitwise the same outputs. */
int ssm_scan_fwd(const ssm_scan_args *args, void *stream);

/* Bytes of workspace ssm_scan_fwd would use for these arguments with a
 * workspace available (0 if the chosen path needs none).  Host-only; makes no
 * HIP call.  Returns a negative SSM_ERR_* code for invalid arguments. */
int64_t ssm_scan_workspace_bytes(const ssm_scan_args *args);

/* ssm_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, plan, kernels and results (bitwise) as ssm_scan_fwd given a
 * workspace of ssm_scan_workspace_bytes bytes, except that the time-split
 * segment summaries live in a device array inside the library, 8 MiB per GPU
 * (held from the library's first such call on that GPU until the process
 * ends).  args->workspace and args->workspace_bytes are ignored.  The call
 * allocates nothing.
 *   - An explicit time_splits > 1 whose summaries need more than 8 MiB
 *     (batch * time_splits * dim * (dstate + 1) * 4 bytes, each part rounded
 *     up to 256 bytes) returns SSM_ERR_WORKSPACE; automatic plans need at
 *     most 4.3 MiB (otherwise they would run unsplit).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (other streams, other threads) race and give wrong
 *     results.  Calls ordered on one stream are safe.  Nothing in the array
 *     needs clearing: each call writes every summary it reads.
 *   - SSM_ERR_LAUNCH if the array's device address cannot be obtained.
 * The caller still owns and passes every input and output. */
int ssm_scan_fwd_noalloc(const ssm_scan_args *args, void *stream);

/* The kernel family and number of time segments ssm_scan_fwd would use, as
 * variant * 65536 + time_splits.  Host-only.  Negative on invalid arguments. */
int64_t ssm_scan_plan(const ssm_scan_args *args);

/* ---- backward -------------------------------------------------------------
 * Gradients of a scalar loss through the forward above, given dL/dy (and
 * optionally dL/dhT): reverse-mode differentiation of the sections 2.2, 3.1,
 * 3.3 and 3.4 operations, walking the recurrence from t = L-1 down to 0 with
 * the state adjoint g (g starts as dL/dhT, each token maps it to
 * exp(delta A) o (gy0 C_t + g), where gy0 = dL/dy_t SiLU(z_t)).
 *
 * The forward's inputs are passed again exactly as they were given to
 * ssm_scan_fwd (the states are recomputed, nothing is saved between the two
 * calls).  Every gradient pointer is optional: NULL skips that output.  Shapes
 * and dtypes of the gradients are those of the matching input: dx, ddelta, dz
 * (B, L, D) and dB, dC (B, L, N) in `dtype`; dA (D, N), dD (D),
 * ddelta_bias (D) and dh0 (B, D, N) fp32.  ddelta is the gradient with
 * respect to the raw step size (before bias and softplus).  dA, dD,
 * ddelta_bias sum over batch rows (and dB, dC over channels) inside the
 * library, in a fixed order: the results are deterministic.  Gradients of
 * inputs that were not given (D, z, delta_bias, h0 NULL) are those of a zero
 * input: dz needs z, the others are still defined.
 *
 * Limits of this version: dstate N in 1..64 (SSM_ERR_DSTATE otherwise). */
typedef struct ssm_scan_bwd_args {
  int64_t batch, seqlen, dim, dstate; /* as ssm_scan_args; N <= 64           */
  int32_t dtype;                      /* ssm_dtype of x, delta, B, C, z, dy and the (B, L, .) gradients */
  int32_t flags;                      /* ssm_flags: SSM_FLAG_GENERIC_A, SSM_FLAG_ZOH as for the forward */
  const void *x;           /* (B, L, D)                                        required */
  const void *delta;       /* (B, L, D) raw step size                          required */
  const float *A;          /* (D, N)                                           required */
  const void *B;           /* (B, L, N)                                        required */
  const void *C;           /* (B, L, N)                                        required */
  const float *D;          /* (D) or NULL                                               */
  const void *z;           /* (B, L, D) or NULL                                         */
  const float *delta_bias; /* (D) or NULL                                               */
  const float *h0;         /* (B, D, N) or NULL                                         */
  const void *dy;          /* (B, L, D) dL/dy                                  required */
  const float *dhT;        /* (B, D, N) dL/dhT, or NULL (= zeros)                       */
  void *dx;                /* (B, L, D) out                                             */
  void *ddelta;            /* (B, L, D) out                                             */
  float *dA;               /* (D, N) out                                                */
  void *dB;                /* (B, L, N) out                                             */
  void *dC;                /* (B, L, N) out                                             */
  float *dD;               /* (D) out                                                   */
  void *dz;                /* (B, L, D) out; requires z                                 */
  float *ddelta_bias;      /* (D) out                                                   */
  float *dh0;              /* (B, D, N) out                                             */
  void *workspace;         /* device scratch of ssm_scan_bwd_workspace_bytes bytes       */
  int64_t workspace_bytes; /* its size                                                  */
  int32_t time_splits;     /* segments per sequence: 0 = automatic, >= 1 = that many    */
  int32_t reserved;        /* must be 0                                                 */
  const float *checkpoints; /* NULL, or the checkpoints ssm_scan_fwd wrote for these same
                               inputs and flags (h0 included): the forward recurrence is
                               then not run again, and the workspace is smaller          */
} ssm_scan_bwd_args;

/* Backward scan.  Errors as for ssm_scan_fwd, plus: SSM_ERR_NULL when a
 * required pointer is NULL or dz is given without z; SSM_ERR_ALIAS when a
 * gradient overlaps an input or another gradient; SSM_ERR_WORKSPACE when the
 * workspace is NULL or smaller than ssm_scan_bwd_workspace_bytes (required
 * whenever B * L * D > 0); SSM_ERR_VARIANT for unknown flags, a negative
 * time_splits or reserved != 0; SSM_ERR_ALIGN / SSM_ERR_ALIAS for checkpoints
 * as for an input.  The workspace is overwritten; its contents
 * on entry do not matter.  Problems with L == 0 give dh0 = dhT (or zeros) and
 * zero dA, dD, ddelta_bias; with B == 0 or D == 0 every non-empty gradient is
 * zero. */
int ssm_scan_bwd(const ssm_scan_bwd_args *args, void *stream);

/* Bytes of workspace ssm_scan_bwd needs for these arguments.  Host-only.
 * Negative SSM_ERR_* code for invalid arguments. */
int64_t ssm_scan_bwd_workspace_bytes(const ssm_scan_bwd_args *args);

/* Number of time segments ssm_scan_bwd would use.  Host-only.  Negative on
 * invalid arguments. */
int64_t ssm_scan_bwd_plan(const ssm_scan_bwd_args *args);

/* ---- conv1d + SiLU prologue -------------------------------------------------
 * The block's prologue on x (section 3.4 listing: a depthwise Conv1d with
 * groups = channels and padding = width - 1, its output cut to the first L
 * positions, then SiLU):
 *   u[b,t,d] = SiLU(bias[d] + sum_{k<W} weight[d,k] * x[b, t-(W-1)+k, d])
 * x at a negative token index is the padding zero or, when `state` is given,
 * row W-1+i of state: the previous call's last W-1 input rows, so that a long
 * sequence can be fed in consecutive calls.  u is the sequence the scan and
 * the caller's projection to B, C and delta consume (section 3.4 derives them
 * from it), so u is materialised; it is not fused into the scan.
 * Layouts: x, u (B, L, D) and state, state_out (B, W-1, D) in `dtype`;
 * weight (D, W) and bias (D) fp32.  Arithmetic is fp32; u is rounded once,
 * to nearest-even. */
typedef struct ssm_conv_args {
  int64_t batch, seqlen, dim; /* B, L, D >= 0                                             */
  int32_t width;              /* W = d_conv, 1..4                                         */
  int32_t dtype;              /* ssm_dtype of x, state, u, state_out                      */
  const void *x;              /* (B, L, D) input                                  required */
  const float *weight;        /* (D, W) taps; tap W-1 multiplies the current token required */
  const float *bias;          /* (D) or NULL (zero)                                        */
  const void *state;          /* (B, W-1, D) previous inputs, or NULL (zero padding)       */
  void *u;                    /* (B, L, D) output                                 required */
  void *state_out;            /* (B, W-1, D) last W-1 input rows out, or NULL              */
} ssm_conv_args;

/* Errors as for ssm_scan_fwd: SSM_ERR_NULL (x, weight, u missing when
 * B*L*D > 0), SSM_ERR_SHAPE, SSM_ERR_DTYPE, SSM_ERR_VARIANT (width outside
 * 1..4), SSM_ERR_ALIGN (16-byte alignment), SSM_ERR_ALIAS (u overlapping an
 * input, or state_out overlapping x, state or u).  With L == 0, state_out
 * receives state (or zeros). */
int ssm_conv1d_silu_fwd(const ssm_conv_args *args, void *stream);

/* ---- Mamba-2 state-space dual (SSD) layer -----------------------------------
 * The multi-head recurrence of section 4.1 (h_t = A_t h_{t-1} + B_t x_t,
 * y_t = C_t h_t) with a scalar decay rate per head and the selection and
 * Euler input term of sections 3.1 and 3.3, per batch row b, head h, head
 * channel p and state n:
 *   delta = softplus(dt[b,t,h] + dt_bias[h]),  a = exp(delta A[h])
 *   S_t[p,n] = a S_{t-1}[p,n] + delta x[b,t,h,p] B[b,t,g,n]
 *   y[b,t,h,p] = sum_n C[b,t,g,n] S_t[p,n] + D[h] x[b,t,h,p]
 * g = h / (H / G): B and C are shared by the H / G heads of a group.  It is
 * evaluated in the chunked matrix (dual) form on the matrix cores.
 * Layouts: x, y (B, L, H, P); dt (B, L, H); B, C (B, L, G, N) in bf16;
 * A, D, dt_bias (H) and the state S0 / ST (B, H, P, N) fp32.
 * One workgroup walks the chunks of one (b, h) in order, so with B*H well
 * under the device's 256 compute units most of them sit idle.  Time
 * splitting cuts the sequence into S segments of whole 64-token chunks: a
 * state-only pass gives each of the first S-1 segments its end state from
 * zero and its total log decay (the same recurrence restricted to the
 * segment, section 4.1's h_t = A_t h_{t-1} + B_t x_t composed over it), and
 * the full pass starts segment s from h0 advanced through segments 0..s-1
 * with those summaries (S_in = exp(sum of log decays) S_prev + S_seg).
 * Results agree with the unsplit call to fp32 rounding.  time_splits: 0
 * picks S from the shape, the most segments for which B*H*S workgroups fit
 * the 256 compute units with segments of at least 4 chunks, at most 64 (so
 * S = 1 once B*H > 128), and S = 1 when workspace is NULL or smaller than
 * ssm_ssd_workspace_bytes reports; 1 never splits; S > 1 asks for S segments
 * (fewer when L has fewer chunks; SSM_ERR_WORKSPACE without a large enough
 * workspace).
 * Limits of this version: dtype SSM_DTYPE_BF16, headdim P = 64,
 * dstate N in {64, 128, 256} (SSM_ERR_VARIANT otherwise). */
typedef struct ssm_ssd_args {
  int64_t batch, seqlen;      /* B <= 65535, L >= 0                                  */
  int64_t nheads, headdim;    /* H >= 1, P = 64                                       */
  int64_t ngroups, dstate;    /* G divides H; N in {64, 128, 256}                     */
  int32_t dtype;              /* SSM_DTYPE_BF16                                       */
  int32_t time_splits;        /* 0 automatic, 1 none, S > 1 segments (see above)       */
  const void *x;              /* (B, L, H, P)                                required */
  const void *dt;             /* (B, L, H) raw step, before bias and softplus required */
  const float *A;             /* (H) decay rate per head (normally < 0)      required */
  const void *B;              /* (B, L, G, N)                                required */
  const void *C;              /* (B, L, G, N)                                required */
  const float *D;             /* (H) or NULL                                           */
  const float *dt_bias;       /* (H) or NULL                                           */
  const float *h0;            /* (B, H, P, N) initial state or NULL (zeros)            */
  float *hT;                  /* (B, H, P, N) final state out or NULL                  */
  void *y;                    /* (B, L, H, P) out                            required */
  void *workspace;            /* device scratch for the segment summaries, or NULL;
                                 16-byte aligned, overwritten, must not overlap any
                                 tensor                                              */
  int64_t workspace_bytes;    /* its size in bytes                                     */
} ssm_ssd_args;

/* Errors as for ssm_scan_fwd; y and hT must not overlap any input or each
 * other (hT may not alias h0); SSM_ERR_VARIANT for time_splits < 0.  With
 * L == 0, hT receives h0 (or zeros). */
int ssm_ssd_fwd(const ssm_ssd_args *args, void *stream);

/* Bytes of workspace ssm_ssd_fwd uses for the segment summaries with these
 * arguments' time_splits (0 when the call would not split): (B, S-1, H, P, N)
 * fp32 end states, then (B, S-1, H) fp32 total log decays, each part starting
 * at a 256-byte boundary.  Host-only; negative SSM_ERR_* for invalid
 * arguments (the workspace fields are not checked here). */
int64_t ssm_ssd_workspace_bytes(const ssm_ssd_args *args);

/* Segments ssm_ssd_fwd would use with these arguments and a workspace of
 * workspace_bytes (1: no split).  Host-only; negative SSM_ERR_* as the call
 * would return them, SSM_ERR_WORKSPACE included. */
int ssm_ssd_plan(const ssm_ssd_args *args);

/* ---- Gated linear attention / mLSTM matrix-state recurrence ----------------
 * Linear attention as a recurrence (HedgeMamba review, stage 2:
 * s_t = s_{t-1} + phi(k_t)^T v_t, read out by phi(q_t), phi = elu + 1 as the
 * example feature map) and its gated form, the mLSTM update of the xLSTM
 * review (the matrix state scaled by a forget coefficient plus the
 * input-gated outer product of value and key).  Per batch row b, head h and
 * group g = h / (H / G):
 *   S_t[p,n] = exp(log_f[b,t,h]) S_{t-1}[p,n] + in_gate[b,t,h] v[b,t,h,p] phi(k[b,t,g,n])
 *   y[b,t,h,p] = sum_n phi(q[b,t,g,n]) S_t[p,n]
 * with log_f = 0 when NULL (no decay: plain linear attention), in_gate = 1
 * when NULL, and phi(u) = u, or elu(u) + 1 with feature_map = 1.  The same
 * chunked matrix form as ssm_ssd_fwd evaluates it (the SSD layer is the case
 * log_f = delta A[h], in_gate = delta, plus D).  log_f is expected <= 0 (a
 * forget gate in (0, 1]); larger values can overflow fp32.
 * Layouts: q, k (B, L, G, N); v, y (B, L, H, P) in bf16; log_f, in_gate
 * (B, L, H) and the state S0 / ST (B, H, P, N) fp32.  feature_map = 1 rounds
 * phi(q) and phi(k) to bf16 before the products.  With feature_map = 1 and a
 * workspace of ssm_gla_workspace_bytes bytes, phi is applied once per call, by
 * an elementwise pass that writes phi(k) and phi(q) to the workspace; without
 * one (NULL or too small) every head's workgroup applies it to its group's
 * keys and queries again.  Both give bitwise the same results.
 * time_splits as for ssm_ssd_fwd: the workspace then also holds the segment
 * summaries, after phi(k) and phi(q) when the feature map is applied once.
 * Limits of this version: dtype SSM_DTYPE_BF16, headdim P = 64,
 * dstate N in {64, 128, 256} (SSM_ERR_VARIANT otherwise). */
typedef struct ssm_gla_args {
  int64_t batch, seqlen;      /* B <= 65535, L >= 0                                  */
  int64_t nheads, headdim;    /* H >= 1, P = 64                                       */
  int64_t ngroups, dstate;    /* G divides H; N in {64, 128, 256}                     */
  int32_t dtype;              /* SSM_DTYPE_BF16                                       */
  int32_t feature_map;        /* 0: phi(u) = u; 1: phi(u) = elu(u) + 1                 */
  const void *q;              /* (B, L, G, N) queries                        required */
  const void *k;              /* (B, L, G, N) keys                           required */
  const void *v;              /* (B, L, H, P) values                         required */
  const float *log_f;         /* (B, L, H) log forget gate or NULL (0)                 */
  const float *in_gate;       /* (B, L, H) input gate or NULL (1)                      */
  const float *h0;            /* (B, H, P, N) initial state or NULL (zeros)            */
  float *hT;                  /* (B, H, P, N) final state out or NULL                  */
  void *y;                    /* (B, L, H, P) out                            required */
  void *workspace;            /* device scratch for phi(k), phi(q) and the segment
                                 summaries, or NULL; 16-byte aligned, overwritten,
                                 must not overlap any tensor                          */
  int64_t workspace_bytes;    /* its size in bytes                                     */
  int32_t time_splits;        /* 0 automatic, 1 none, S > 1 segments (ssm_ssd_args)    */
  int32_t reserved;           /* must be 0                                            */
} ssm_gla_args;

/* Errors as for ssm_ssd_fwd (SSM_ERR_VARIANT also for feature_map outside
 * {0, 1} or reserved != 0); y and hT must not overlap any input or each
 * other.  With L == 0, hT receives h0 (or zeros). */
int ssm_gla_fwd(const ssm_gla_args *args, void *stream);

/* Bytes of workspace ssm_gla_fwd uses: phi(k) and phi(q), each (B, L, G, N)
 * bf16, with the feature map, then the segment summaries laid out as for
 * ssm_ssd_workspace_bytes when the call would split; every part starts at a
 * 256-byte boundary.  With a smaller workspace, an automatic split is dropped
 * first, then the feature-map pass.  Host-only; negative SSM_ERR_* for
 * invalid arguments (the workspace fields are not checked here). */
int64_t ssm_gla_workspace_bytes(const ssm_gla_args *args);

/* Segments ssm_gla_fwd would use (as ssm_ssd_plan). */
int ssm_gla_plan(const ssm_gla_args *args);

/* Static, human-readable text for a status code. */
const char *ssm_scan_strerror(int code);

/* SSM_SCAN_ABI_VERSION of the loaded library. */
int ssm_scan_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H_ */
