/*
 * ssm_mi355x.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * Three entry points, one per path of the Mamba-style selective state space
 * layer described by the pages:
 *
 *   ssm_scan_fwd        full-sequence (prefill) scan: causal depthwise conv1d
 *                       + SiLU, dt = clip(softplus(dt_proj + dt_bias)), the
 *                       diagonal recurrence h_t = exp(dt*A) h_{t-1} + dt*B_t*u_t,
 *                       y_t = C_t . h_t + D*u_t, gate y * SiLU(z).  Page
 *                       "Axon-SSM: selective state space model", sections
 *                       "Algorithm", "SSM scan", "Discretization", "JIT-compiled
 *                       kernels" and "Autoregressive decoding" (prefill,
 *                       cache = None).
 *   ssm_decode_step     one token of autoregressive decoding that updates
 *                       [conv_cache, ssm_state] in place.  Same page, section
 *                       "Autoregressive decoding" (decode, cache =
 *                       [conv_cache, ssm_state]).
 *   ssm_chunk_scan_fwd  multi-head chunked scan (scalar A per head): page "What
 *                       is the Mamba model?", sections "chunkscan" and
 *                       "chunkscan implementation", chunk output formula
 *                       out[l] = sum_{s<=l} cb[l,s] e^{dA[l]-dA[s]} dt[s] x[s]
 *                              + e^{dA[l]} C[l] prev_states + D x[l],
 *                       with the chunk-final state carried to the next chunk.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The scan,
 *    chunked-scan, decode and backward entry points allocate nothing, keep no
 *    per-call state, never copy between host and device and never
 *    synchronise.  The projection entry points (ssm_linear_fwd,
 *    ssm_layer_fwd) are the exception: the first call of a shape on a device
 *    creates that device's hipBLASLt handle and the shape's matmul plan, both
 *    of which allocate host and device memory inside the GEMM library, and
 *    keeps them until the process ends; later calls of the same shape
 *    allocate nothing.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    null stream) and the call returns at once.  Asynchronous kernel faults
 *    surface at the caller's next synchronisation.
 *  - Layouts are dense row-major in the order written next to each field, last
 *    index fastest.  Pointers must be aligned to their element size.
 *  - Every argument error is detected before anything is launched: the call
 *    returns SSM_ERR_INVALID_ARG or SSM_ERR_UNSUPPORTED and writes nothing;
 *    ssm_last_error() then names the field.  A failed launch returns
 *    SSM_ERR_HIP.  NaN/Inf inputs are not checked; they propagate.
 *  - Outputs (y, out) must not overlap any input.  State and cache outputs may
 *    alias their inputs exactly (in-place update).
 *  - Floating point: all arithmetic is fp32; bf16 inputs are widened exactly;
 *    bf16 outputs are rounded to nearest-even.
 */
#ifndef SSM_MI355X_H
#define SSM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 2

/* element types (int32 fields in the structs below) */
typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

/* How B is discretized.  SSM_EULER: dB u = dt B u (the "dB * x_t" of the
 * Axon-SSM page's kernel section and the dt[s] x[s] of the velog page's chunk
 * formula).  SSM_ZOH: the zero-order hold of the molayo page's "Technical
 * details", dB u = ((e^{dt A} - 1) / A) B u.  The decay is e^{dt A} in both. */
typedef enum { SSM_EULER = 0, SSM_ZOH = 1 } ssm_discretization_t;

/* return codes */
typedef enum {
  SSM_OK = 0,
  SSM_ERR_INVALID_ARG = 1, /* a null required pointer, a negative size, bad bounds, wrong struct_size */
  SSM_ERR_UNSUPPORTED = 2, /* a valid request this build does not implement (e.g. d_state != 16) */
  SSM_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_size query */
  SSM_ERR_HIP = 4,         /* the HIP runtime rejected a launch */
  SSM_ERR_INTERNAL = 5     /* debug builds only: a launch plan broke an invariant its kernels rely on */
} ssm_status_t;

/* ------------------------------------------------------------------------
 * Full-sequence scan (prefill).
 *
 * Shapes: Bt = batch, L = seqlen, E = dim (channels), N = d_state.
 *   x             (Bt, L, E) x_dtype     pre-conv x_branch when conv_w != NULL, else u itself
 *   conv_w        (E, K) f32 or NULL     causal depthwise conv; NULL skips conv and SiLU.
 *                                        xc[t] = sum_k conv_w[e,k] * xpad[t+k] (+ conv_b[e]),
 *                                        xpad = (conv_cache_in or zeros, x) along t, so
 *                                        conv_w[e,K-1] multiplies the current token;
 *                                        u = SiLU(xc).  K = conv_k must be 4.
 *   conv_b        (E) f32 or NULL
 *   conv_cache_in (Bt, E, K-1) f32 or NULL (zeros): raw pre-conv inputs before t=0, oldest first
 *   conv_cache_out(Bt, E, K-1) f32 or NULL: the last K-1 raw inputs (including cache_in
 *                                        values when L < K-1), oldest first; may alias conv_cache_in
 *   dt            dt_rank1 != 0: (Bt, L) f32 r, and pre = dt_w[e] * r[b,t] (dt_proj 1 -> E)
 *                 dt_rank1 == 0: (Bt, L, E) dt_dtype, and pre = dt[b,t,e]
 *   dt_w          (E) f32, required iff dt_rank1
 *   dt_bias       (E) f32 or NULL (zero)
 *   dt_softplus   nonzero: dt = clip(softplus(pre + dt_bias), dt_min, dt_max)
 *                 zero:    dt = clip(pre + dt_bias, dt_min, dt_max)
 *   dt_min/dt_max clip bounds (inclusive); -INFINITY / +INFINITY disable a side; dt_min <= dt_max
 *   A             (E, N) f32, the continuous-time diagonal (normally A = -exp(A_log) < 0)
 *   B, C          (Bt, L, N) bc_dtype
 *   D             (E) f32 or NULL (no skip term)
 *   z             (Bt, L, E) z_dtype or NULL (no gate); z_dtype must equal x_dtype
 *   ssm_state_in  (Bt, E, N) f32 or NULL (zeros, the prefill start)
 *   ssm_state_out (Bt, E, N) f32 or NULL; may alias ssm_state_in
 *   y             (Bt, L, E) y_dtype: y_t = (C_t . h_t + D*u_t) * SiLU(z_t)
 *   workspace     device scratch of at least ssm_scan_workspace_size(p) bytes (may be
 *                 NULL when that size is 0); 256-byte aligned; not touched by other calls
 *   time_split    0: the library chooses; >= 1: split the sequence into at most that
 *                 many segments scanned in parallel and combined (at most 32; every
 *                 segment but the last spans a multiple of 8 steps);
 *                 SSM_SCAN_BLOCKED (-1): one pass over 16-step blocks, 16 channels per
 *                 wave, blocks whose dt sits at dt_max in every channel computed as
 *                 matrix-core products of per-block tables (the chunk form of the
 *                 velog page's "chunkscan"); it takes bf16 x and z, an E-wide bf16
 *                 dt, no conv, SSM_EULER, dim % 64 == 0, x/z/dt/bf16 y 8-byte and
 *                 fp32 y and ssm_state_out 16-byte aligned (else SSM_ERR_UNSUPPORTED).
 *                 With 0 the library takes it for such calls when batch * dim / 64 >= 768.
 *   discretization SSM_EULER or SSM_ZOH (see ssm_discretization_t)
 * Supported: N = 16.  L = 0 only copies the state/cache inputs to the outputs.
 * ---------------------------------------------------------------------- */
#define SSM_SCAN_BLOCKED (-1) /* ssm_scan_params_t.time_split: the blocked single-pass scan */

typedef struct ssm_scan_params {
  uint32_t struct_size; /* = sizeof(ssm_scan_params_t) */
  int32_t batch, seqlen, dim, d_state;
  int32_t conv_k;
  const void *x;
  int32_t x_dtype;
  const float *conv_w;
  const float *conv_b;
  const float *conv_cache_in;
  float *conv_cache_out;
  const void *dt;
  int32_t dt_dtype;
  int32_t dt_rank1;
  const float *dt_w;
  const float *dt_bias;
  int32_t dt_softplus;
  float dt_min, dt_max;
  const float *A;
  const void *B;
  const void *C;
  int32_t bc_dtype;
  const float *D;
  const void *z;
  int32_t z_dtype;
  const float *ssm_state_in;
  float *ssm_state_out;
  void *y;
  int32_t y_dtype;
  int32_t time_split;
  void *workspace;
  size_t workspace_bytes;
  int32_t discretization; /* SSM_EULER (0): dB u = dt B u; SSM_ZOH (1): ((e^{dt A} - 1) / A) B u */
} ssm_scan_params_t;

ssm_status_t ssm_scan_fwd(const ssm_scan_params_t *p, void *stream);
size_t ssm_scan_workspace_size(const ssm_scan_params_t *p);
/* Validation only: the status ssm_scan_fwd would return before launching. */
ssm_status_t ssm_scan_check(const ssm_scan_params_t *p);

/* ------------------------------------------------------------------------
 * ssm_scan_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results as ssm_scan_fwd, with the
 * workspace taken from a scratch array inside the library instead of the
 * caller.  p->workspace must be NULL and p->workspace_bytes 0 (else
 * SSM_ERR_INVALID_ARG); every other field is as for ssm_scan_fwd, and the
 * caller still owns the inputs and outputs.  The call allocates nothing and
 * calls no allocating routine.
 *  - The scratch holds SSM_SCAN_NOALLOC_MAX_BYTES (64 MiB).  A call whose
 *    ssm_scan_workspace_size(p) exceeds it returns SSM_ERR_WORKSPACE, with the
 *    size in ssm_last_error(), before anything is launched.  (It covers, for
 *    example, batch 8 x 4096 tokens and batch 1 x 2048 tokens at E 7680 with
 *    the library's own time split.)
 *  - Each GPU the library runs on holds one copy of the scratch for the life
 *    of the process.  Its address on a device is looked up on the first call
 *    made there (with that device current); a failure of that lookup returns
 *    SSM_ERR_HIP.
 *  - Every call on one GPU uses that GPU's single copy: calls that may run at
 *    the same time on one GPU (different streams without ordering between
 *    them, or different threads) race on it and must not overlap.  Calls on
 *    one stream are ordered and safe.  Nothing in the scratch needs to start
 *    at zero; it keeps the last call's contents.
 * ---------------------------------------------------------------------- */
#define SSM_SCAN_NOALLOC_MAX_BYTES ((size_t)64 << 20)
ssm_status_t ssm_scan_fwd_noalloc(const ssm_scan_params_t *p, void *stream);

/* ------------------------------------------------------------------------
 * One decode step, in place.  Shapes as above with L = 1:
 *   x (Bt, E) x_dtype new token (pre-conv when conv_w != NULL); z (Bt, E) or NULL;
 *   dt: dt_rank1 ? (Bt) f32 r : (Bt, E) dt_dtype;  B, C (Bt, N) bc_dtype;
 *   conv_cache (Bt, E, K-1) f32, read then overwritten with the window shifted by one
 *   (required iff conv_w != NULL);  ssm_state (Bt, E, N) f32, read then overwritten;
 *   y (Bt, E) y_dtype.
 * ssm_state, A and conv_w must be 16-byte aligned, B and C aligned to 4
 * elements (16 bytes in f32, 8 in bf16); batch * dim < 2^31.
 * The result equals ssm_scan_fwd with L = 1, conv_cache_in = conv_cache_out =
 * conv_cache and ssm_state_in = ssm_state_out = ssm_state.
 * ---------------------------------------------------------------------- */
typedef struct ssm_decode_params {
  uint32_t struct_size; /* = sizeof(ssm_decode_params_t) */
  int32_t batch, dim, d_state, conv_k;
  const void *x;
  int32_t x_dtype;
  const float *conv_w;
  const float *conv_b;
  float *conv_cache;
  const void *dt;
  int32_t dt_dtype;
  int32_t dt_rank1;
  const float *dt_w;
  const float *dt_bias;
  int32_t dt_softplus;
  float dt_min, dt_max;
  const float *A;
  const void *B;
  const void *C;
  int32_t bc_dtype;
  const float *D;
  const void *z;
  int32_t z_dtype;
  float *ssm_state;
  void *y;
  int32_t y_dtype;
  int32_t discretization; /* as in ssm_scan_params_t */
} ssm_decode_params_t;

ssm_status_t ssm_decode_step(const ssm_decode_params_t *p, void *stream);
ssm_status_t ssm_decode_check(const ssm_decode_params_t *p);

/* ------------------------------------------------------------------------
 * Multi-head chunked scan (SSD form), scalar A per head.
 *   x         (Bt, L, H, P) x_dtype
 *   dt        (Bt, L, H) f32 raw; dt = clip(softplus(dt + dt_bias[h]), dt_min, dt_max)
 *             (softplus skipped when dt_softplus == 0)
 *   dt_bias   (H) f32 or NULL
 *   A         (H) f32 (negative)
 *   B, C      (Bt, L, G, N) bc_dtype; head h reads group h / (H / G)
 *   D         (H) f32 (d_per_channel == 0) or (H, P) f32 (d_per_channel != 0) or NULL
 *   state_in  (Bt, H, P, N) f32 or NULL (zeros); state_out (Bt, H, P, N) f32 or NULL
 *   out       (Bt, L, H, P) out_dtype
 *   dA[l] = sum_{i<=l} dt[i] A_h inside each chunk of chunk_size tokens (inclusive);
 *   state passing: S <- e^{dA[Q-1]} S + sum_s e^{dA[Q-1]-dA[s]} dt[s] x[s] (outer) B[s].
 * A sequence that is not a whole number of chunks ends with a shorter chunk
 * (the same formulas over its own length).
 * Supported: chunk_size up to 256, d_state up to 128, headdim up to 128, x,
 * B/C, z and out each in f32 or bf16, and seqlen * max(nheads * headdim,
 * ngroups * d_state) * 2 bytes (one batch row) below 4 GiB.  Two kernels
 * share the work: N = 64, chunk_size = 128, bf16 x and B/C and headdim a
 * multiple of 16 run the matrix-core kernel (x, B, C, out and z 16-byte
 * aligned; it may cut each sequence into segments, see `segments`); every
 * other shape runs chunk by chunk on the vector ALUs in fp32 (pointers
 * aligned to their element size; `segments` has no effect there: every chunk
 * already starts from the state composed ahead of it).  The result is the
 * same function either way, up to rounding order.
 * Workspace: ssm_chunk_scan_workspace_size() bytes of device memory, 256-byte
 * aligned, owned by the caller (zero for the matrix-core kernel when the
 * sequences are not cut into segments; batch * nchunks * nheads * (headdim *
 * d_state + 1) floats, rounded up, for the vector-ALU kernels); its contents
 * on entry do not matter.
 * ---------------------------------------------------------------------- */
typedef struct ssm_chunk_params {
  uint32_t struct_size; /* = sizeof(ssm_chunk_params_t) */
  int32_t batch, seqlen, nheads, headdim, ngroups, d_state, chunk_size;
  const void *x;
  int32_t x_dtype;
  const float *dt;
  const float *dt_bias;
  int32_t dt_softplus;
  float dt_min, dt_max;
  const float *A;
  const void *B;
  const void *C;
  int32_t bc_dtype;
  const float *D;
  int32_t d_per_channel;
  const float *state_in;
  float *state_out;
  void *out;
  int32_t out_dtype;
  void *workspace;
  size_t workspace_bytes;
  const void *z;        /* (Bt, L, H, P) z_dtype or NULL: out *= SiLU(z) after the D skip */
  int32_t z_dtype;
  int32_t segments;     /* 0: chosen by the library; else cut each sequence into this many
                           runs of whole chunks (at most 16, and at most one per chunk) that
                           start from states composed ahead of them; the result is the same
                           up to rounding order */
} ssm_chunk_params_t;

ssm_status_t ssm_chunk_scan_fwd(const ssm_chunk_params_t *p, void *stream);
size_t ssm_chunk_scan_workspace_size(const ssm_chunk_params_t *p);
ssm_status_t ssm_chunk_scan_check(const ssm_chunk_params_t *p);

/* ------------------------------------------------------------------------
 * Backward of ssm_scan_fwd (Euler form) with recomputation (page "Mamba/SSM
 * basics", the production recipe after "Technical details": intermediate
 * states are recomputed in the backward pass instead of being stored).  Given
 * dy = dL/dy (Bt, L, E) dy_dtype and optionally dstate_out = dL/dh_L
 * (Bt, E, N) f32, writes the gradients of L with respect to the forward's
 * inputs, all f32 and in the inputs' shapes:
 *   dx (Bt, L, E); dz (Bt, L, E) when z was given; ddt: (Bt, L) for a rank-1
 *   dt (gradient of r), else (Bt, L, E); ddt_w (E) for a rank-1 dt; ddt_bias (E);
 *   dA (E, N); dB, dC (Bt, L, N); dD (E); dconv_w (E, 4), dconv_b (E) and
 *   dconv_cache (Bt, E, 3) when there is a conv; dstate_in (Bt, E, N).
 * Any gradient pointer may be NULL (not written).  The forward inputs are the
 * fields of the same names in ssm_scan_params_t with the same rules; the
 * clip passes gradient strictly inside (dt_min, dt_max).  Sums over
 * channels and time are taken in a fixed order (results are deterministic).
 * The workspace holds ssm_scan_bwd_workspace_size(p) bytes (256-byte aligned).
 * Supported: N = 16, Euler discretization; dy_dtype f32 or bf16.
 * ---------------------------------------------------------------------- */
typedef struct ssm_scan_bwd_params {
  uint32_t struct_size; /* = sizeof(ssm_scan_bwd_params_t) */
  int32_t batch, seqlen, dim, d_state, conv_k;
  const void *x;
  int32_t x_dtype;
  const float *conv_w, *conv_b, *conv_cache_in;
  const void *dt;
  int32_t dt_dtype, dt_rank1;
  const float *dt_w, *dt_bias;
  int32_t dt_softplus;
  float dt_min, dt_max;
  const float *A;
  const void *B, *C;
  int32_t bc_dtype;
  const float *D;
  const void *z;
  int32_t z_dtype;
  const float *ssm_state_in;
  const void *dy;
  int32_t dy_dtype;
  const float *dstate_out;
  float *dx, *dz, *ddt, *ddt_w, *ddt_bias, *dA, *dB, *dC, *dD, *dconv_w, *dconv_b, *dconv_cache, *dstate_in;
  void *workspace;
  size_t workspace_bytes;
} ssm_scan_bwd_params_t;

ssm_status_t ssm_scan_bwd(const ssm_scan_bwd_params_t *p, void *stream);
size_t ssm_scan_bwd_workspace_size(const ssm_scan_bwd_params_t *p);
ssm_status_t ssm_scan_bwd_check(const ssm_scan_bwd_params_t *p);

/* ------------------------------------------------------------------------
 * One decode step of the multi-head scan, in place (page "What is the Mamba
 * model?", section "chunkscan": the state that the chunked scan passes from
 * chunk to chunk, advanced by a chunk of one token).  For each (b, h):
 *   dt = clip(softplus(dt_raw[b,h] + dt_bias[h]), dt_min, dt_max)   (softplus
 *        skipped when dt_softplus == 0)
 *   state[b,h,p,n] <- e^{dt A_h} state[b,h,p,n] + dt x[b,h,p] B[b,g,n]
 *   out[b,h,p] = (sum_n C[b,g,n] state[b,h,p,n] + D x[b,h,p]) * SiLU(z[b,h,p])
 * with g = h / (H / G) and the gate only when z != NULL.
 *   x         (Bt, H, P) x_dtype
 *   dt        (Bt, H) f32 raw;  dt_bias (H) f32 or NULL;  A (H) f32
 *   B, C      (Bt, G, N) bc_dtype
 *   D         (H) f32 (d_per_channel == 0) or (H, P) f32 or NULL
 *   z         (Bt, H, P) z_dtype or NULL
 *   state     (Bt, H, P, N) f32, read then overwritten (the layout of the
 *             chunked scan's state_in / state_out)
 *   out       (Bt, H, P) out_dtype; must not overlap any input
 * The result equals ssm_chunk_scan_fwd with L = 1 and state_in = state_out =
 * state.  state must be 16-byte aligned; B and C aligned to 8 elements (32
 * bytes in f32, 16 in bf16).  Supported: N in {16, 32, 64, 128};
 * batch * H * P < 2^31.  All dtypes f32 or bf16.
 * ---------------------------------------------------------------------- */
typedef struct ssm_chunk_decode_params {
  uint32_t struct_size; /* = sizeof(ssm_chunk_decode_params_t) */
  int32_t batch, nheads, headdim, ngroups, d_state;
  const void *x;
  int32_t x_dtype;
  const float *dt;
  const float *dt_bias;
  int32_t dt_softplus;
  float dt_min, dt_max;
  const float *A;
  const void *B;
  const void *C;
  int32_t bc_dtype;
  const float *D;
  int32_t d_per_channel;
  const void *z;
  int32_t z_dtype;
  float *state;
  void *out;
  int32_t out_dtype;
} ssm_chunk_decode_params_t;

ssm_status_t ssm_chunk_decode_step(const ssm_chunk_decode_params_t *p, void *stream);
ssm_status_t ssm_chunk_decode_check(const ssm_chunk_decode_params_t *p);

/* ------------------------------------------------------------------------
 * A projection of the layer (page "Axon-SSM: selective state space model",
 * section "Algorithm": in_proj D -> 2E and out_proj E -> D), no bias:
 *   out[r, o] = sum_i x[r, i] * weight[o, i]
 *   x       (rows, in_features) x_dtype: bf16 is used as it is; f32 enters the
 *           matrix cores as a bf16 pair (value and remainder), which keeps
 *           about 16 mantissa bits
 *   weight  (out_features, in_features) bf16 (the (out, in) layout of a weight)
 *   out     (rows, out_features) out_dtype; must not overlap x or weight
 *   workspace  device scratch of ssm_linear_workspace_size(p) bytes (256-byte
 *           aligned, owned by the caller, contents on entry irrelevant):
 *           none for a bf16 x; for an f32 x its bf16 value and remainder and
 *           an fp32 product.  Missing or short: SSM_ERR_WORKSPACE.
 * fp32 accumulation.  The products run in the ROCm GEMM library (hipBLASLt),
 * the same algorithm for a given shape and device, so results repeat bit for
 * bit.  x, weight and out must be 16-byte aligned; in_features % 8 == 0;
 * out_features % 4 == 0.
 * ---------------------------------------------------------------------- */
typedef struct ssm_linear_params {
  uint32_t struct_size; /* = sizeof(ssm_linear_params_t) */
  int32_t rows, in_features, out_features;
  const void *x;
  int32_t x_dtype;
  const void *weight;
  void *out;
  int32_t out_dtype;
  void *workspace;
  size_t workspace_bytes;
} ssm_linear_params_t;

ssm_status_t ssm_linear_fwd(const ssm_linear_params_t *p, void *stream);
size_t ssm_linear_workspace_size(const ssm_linear_params_t *p);
ssm_status_t ssm_linear_check(const ssm_linear_params_t *p);

/* ------------------------------------------------------------------------
 * The whole layer forward (page "Axon-SSM: selective state space model",
 * section "Algorithm"), T = batch * seqlen tokens:
 *   [x_branch | z] = in_proj(hidden)                   w_in (2E, D) bf16
 *   u = SiLU(causal depthwise conv1d(x_branch))        conv_w (E, K), conv_b (E) or NULL
 *   [B | C | dt_raw] = x_proj(u)                       w_x (2N+1, E) bf16, in that order
 *   dt = clip(softplus(dt_w * dt_raw + dt_bias), dt_min, dt_max)   dt_w, dt_bias (E)
 *   y = scan(u, dt, A, B, C) + D u, gated by SiLU(z)   A (E, N), D (E) or NULL
 *   out = out_proj(y)                                  w_out (D, E) bf16
 * hidden (Bt, L, D) hidden_dtype; out (Bt, L, D) out_dtype; conv caches
 * (Bt, E, K-1) f32 and states (Bt, E, N) f32 as in ssm_scan_fwd (each NULL-able;
 * in and out may be the same buffer).  The activations between the steps
 * (x_branch, z, y: fp32; B, C, dt_raw: fp32) live in the workspace, which
 * must hold ssm_layer_workspace_size(p) bytes (256-byte aligned).
 * Supported: N = 16, K = 4, E % 256 == 0, D % 8 == 0; hidden, the weights,
 * out, conv_w and A 16-byte aligned.
 * Timing events (ssm_set_timing_events) bracket the whole layer.
 * ---------------------------------------------------------------------- */
typedef struct ssm_layer_params {
  uint32_t struct_size; /* = sizeof(ssm_layer_params_t) */
  int32_t batch, seqlen, d_model, dim, d_state, conv_k;
  const void *hidden;
  int32_t hidden_dtype;
  const void *w_in;
  const float *conv_w, *conv_b;
  const void *w_x;
  const float *dt_w, *dt_bias;
  int32_t dt_softplus;
  float dt_min, dt_max;
  const float *A;
  const float *D;
  const void *w_out;
  const float *conv_cache_in;
  float *conv_cache_out;
  const float *ssm_state_in;
  float *ssm_state_out;
  void *out;
  int32_t out_dtype;
  void *workspace;
  size_t workspace_bytes;
} ssm_layer_params_t;

ssm_status_t ssm_layer_fwd(const ssm_layer_params_t *p, void *stream);
size_t ssm_layer_workspace_size(const ssm_layer_params_t *p);
ssm_status_t ssm_layer_check(const ssm_layer_params_t *p);

/* ------------------------------------------------------------------------ */
const char *ssm_status_string(int32_t status);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char *ssm_last_error(void);
int32_t ssm_abi_version(void);
/* sizeof of a params struct: which = 0 scan, 1 decode, 2 chunk, 3 chunk
 * decode, 4 linear, 5 layer, 6 scan backward; 0 otherwise. */
size_t ssm_params_sizeof(int32_t which);

/* Kernel timing for measurement tools.  start and stop are hipEvent_t handles
 * owned by the caller (both NULL switches timing off).  While set, each entry
 * point called on this thread records start on its stream right before the
 * launch of its main kernel (the full-segment scan kernel of ssm_scan_fwd, the
 * only kernel of the others) and stop right after it, so
 * hipEventElapsedTime(start, stop) is that kernel's duration.  The events are
 * only recorded, never created, synchronised or destroyed by the library. */
void ssm_set_timing_events(void *start, void *stop);

/* ---- debug builds (SSM_DEBUG) ---------------------------------------------
 * For callers that want the host-side bounds checks: a build of the library
 * with SSM_DEBUG defined (libssm_mi355x_debug.so, the same kernels) checks,
 * before every launch of ssm_scan_fwd(_noalloc), ssm_chunk_scan_fwd and
 * ssm_scan_bwd, the launch plan against the buffers the call describes: each
 * grid's mapping from block ids to work items is a bijection onto the work,
 * the time segments, chunk segments and summary pieces tile the sequence as
 * the kernels assume, and every workspace region a kernel indexes is
 * 256-byte aligned, lies inside workspace_bytes and overlaps no other.  A
 * failure returns SSM_ERR_INTERNAL (ssm_last_error() names the check) and
 * launches nothing.
 * ssm_debug_checks: launch plans checked so far in this process (-1: a build
 *   without the checks).
 * ssm_debug_check_{scan,chunk,scan_bwd}: validation plus the plan checks of
 *   that entry point without launching anything (runs without a GPU; pointers
 *   are compared, never dereferenced); SSM_ERR_UNSUPPORTED in builds without
 *   the checks. */
long ssm_debug_checks(void);
ssm_status_t ssm_debug_check_scan(const ssm_scan_params_t *p);
ssm_status_t ssm_debug_check_chunk(const ssm_chunk_params_t *p);
ssm_status_t ssm_debug_check_scan_bwd(const ssm_scan_bwd_params_t *p);

#ifdef __cplusplus
}
#endif

#endif /* SSM_MI355X_H */
