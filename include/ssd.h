/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 SSD chunked-scan library (libssd.so).
 *
 * The operation.  For every batch row b and head h (group g = h / (H / G)):
 *     dt'_t = softplus(dt[b,t,h] + dt_bias[h])          softplus(v) = log(1 + e^v)
 *             (then clamped to [dt_min, dt_max] when the dims ask for it)
 *     h_t   = exp(dt'_t * A[h]) * h_{t-1} + dt'_t * x[b,t,h,:]^T B[b,t,g,:]     (P x N state)
 *     y_t   = (h_t C[b,t,g,:]^T + D[h,:] * x[b,t,h,:]) * silu(z[b,t,h,:])    (gate only if z given)
 * with h_{-1} = initial_state (zeros when NULL) and final_state = h_{L-1}; silu(v) = v / (1 + e^-v).
 * Sources: "Agent 228: MAMBA-2 Reference Implementations Comparison", section 2.2 (SSD as a
 * 1-semiseparable masked form, A scalar per head) and section 3.2 (softplus(dt + dt_bias),
 * decay exp(A dt'), input term B dt', chunked evaluation); "Agent 228: MAMBA-2 Implementation
 * Gaps", Gap 1 (diagonal blocks within a chunk plus the carried inter-chunk state), Gap 3
 * (softplus), Gap 4 (D skip term); "MAMBA2 Inference Optimization Report", Step 4 (the last
 * state is kept for stateful inference); the optional gate is the output gating of the
 * reference-comparison page (section 3.1 forward pass, section 6.1) and the optional clamp its
 * dt limits (section 5.2; Implementation Gaps, Gap 3).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are caller-owned DEVICE pointers on the current HIP device, row-major
 *    and contiguous with the layouts given below.  The library never allocates, frees,
 *    synchronises or prints.  Work is enqueued asynchronously on `stream` (0 = null stream).
 *  - Element type of x, dt, B, C and y is dims->dtype (fp32, or bf16 = the upper 16 bits of an
 *    IEEE fp32, stored in 2 bytes).  dt_bias, A, D and every state are always fp32.
 *  - Alignment: x, B, C, y, states and the workspace must be 16-byte aligned; dt, dt_bias, A
 *    and D must be aligned to their element size.
 *  - Validation runs completely before anything is launched.  On any error nothing is
 *    launched and no output is written.  A failure reported by the HIP runtime at launch
 *    is returned as SSD_ERR_HIP.
 *  - Calls are stateless and re-entrant; concurrent calls on different streams need separate
 *    workspaces and outputs.
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1,   /* NULL where a pointer is required, negative size, bad alignment */
  SSD_ERR_UNSUPPORTED = 2,   /* valid but not implemented: chunk size, headdim, dstate, dtype */
  SSD_ERR_DEVICE_PTR = 3,    /* a pointer is not device memory of the current device */
  SSD_ERR_WORKSPACE = 4,     /* workspace NULL or smaller than ssd_fwd_workspace_size() */
  SSD_ERR_HIP = 5,           /* the HIP runtime reported an error when launching */
  SSD_ERR_SCRATCH_LIMIT = 6  /* ssd_fwd_noalloc: the sizes need more than its fixed scratch */
} ssd_status_t;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype_t;

/* Problem sizes.  batch >= 0, seqlen >= 0 (ssd_step ignores it), nheads >= 1,
 * ngroups >= 1 with nheads % ngroups == 0.  Supported (else SSD_ERR_UNSUPPORTED):
 * headdim in {16, 32, 64}; dstate in {16, 32, 64} for SSD_F32 and {32, 64, 128} for SSD_BF16.
 * dt_max > 0 clamps dt' = softplus(dt + dt_bias) to [dt_min, dt_max] (requires
 * 0 <= dt_min <= dt_max, else SSD_ERR_INVALID_ARG); dt_max == 0 means no clamp. */
typedef struct {
  int64_t batch;     /* B */
  int64_t seqlen;    /* L */
  int64_t nheads;    /* H */
  int64_t headdim;   /* P */
  int64_t dstate;    /* N */
  int64_t ngroups;   /* G */
  int32_t dtype;     /* ssd_dtype_t */
  float dt_min;      /* lower clamp of dt' (used when dt_max > 0) */
  float dt_max;      /* upper clamp of dt'; 0 = no clamp */
} ssd_dims_t;

/* Bytes of device workspace ssd_fwd needs for these sizes and chunk size; 0 when the
 * arguments are invalid or unsupported.  Pure host arithmetic.  Layout (each region
 * 256-byte aligned, nc = ceil(L / chunk_size)):
 *   [0] dt'  (B, H, nc, chunk_size) fp32   softplus(dt + dt_bias) (clamped if asked); 0 past the end
 *   [1] dAcs (B, H, nc, chunk_size) fp32   inclusive in-chunk cumulative sum of dt' * A
 *   [2] states (B, nc, H, P, N) fp32       first the state each chunk contributes (decayed to
 *                                          the chunk end), then overwritten in place by the
 *                                          state entering each chunk; on the one-pass path
 *                                          (ssd_fwd_state_path in ssd_tuning.h) fp32 inputs get
 *                                          the entering states only and bf16 inputs leave it
 *                                          unwritten; on the segmented path it holds each
 *                                          segment's end state from a zero start, (B, nseg, H,
 *                                          P, N) fp32, then (256-byte aligned) the states
 *                                          entering the segments in bf16, nseg = ceil(nc / SL)
 *   [3] SSD_F32, and SSD_BF16 with at least 20 heads per group: C B^T, computed once per
 *       group, (B, nc, G, nrb (nrb + 1) / 2) blocks of 16 x 256 fp32, nrb = chunk_size / 64:
 *       the causal 16 x 16 sub-tiles of each pair of 64-row blocks (row block rb, column
 *       block J <= rb), in the scan's register order; 0 bytes otherwise
 *   [4] SSD_BF16 only: the states entering each chunk rounded to bf16, (B, nc, H, P, N); for
 *       bf16 inputs region [2] keeps the per-chunk contributions (state_passing writes the
 *       entering states here instead); on the segmented path, the state each segment alone
 *       carried into its chunks (slots of a segment's first chunk unwritten)
 *   [5] SSD_BF16 only: two (B, H, nc) fp32 arrays (each 256-byte aligned), used on the
 *       segmented path: the segments' total decay exponents (B, H, nseg), then for every chunk
 *       the exponent summed from its segment's start
 * The contents after a call are those intermediates and may be inspected. */
size_t ssd_fwd_workspace_size(const ssd_dims_t* dims, int chunk_size);

/* Chunked SSD forward over a whole sequence (the chunked diagonal-block / carried-state
 * evaluation of the reference-comparison page, section 3.2, and of Gap 1 of the
 * implementation-gaps page).  Three kernels run in order on `stream`: chunk_state (dt', its
 * in-chunk cumsum and the chunk states; where region [3] exists also C B^T once per group),
 * state_passing, chunk_scan.  For SSD_BF16 with P = 64, N = 128 and batch x nheads >= 256 the
 * first two are one kernel instead (chunk_state_seq: one pass over the chunks per (b, h) with
 * the carried state in registers); ssd_fwd_state_path in ssd_tuning.h tells which.  The choice
 * is a pure function of the arguments (ssd_fwd_ex in ssd_tuning.h takes explicit options).
 *   x             (B, L, H, P)  dtype       input sequence
 *   dt            (B, L, H)     dtype       raw step, before bias and softplus
 *   dt_bias, A    (H)           fp32        A is used as given (pass negative values)
 *   B, C          (B, L, G, N)  dtype
 *   D             (H, P)        fp32        NULL means no skip term
 *   z             (B, L, H, P)  dtype       gate; NULL means no gate
 *   chunk_size    64, 128 or 256; the result does not depend on it beyond rounding
 *   initial_state (B, H, P, N)  fp32        NULL means zeros
 *   y             (B, L, H, P)  dtype       output (may not alias an input)
 *   final_state   (B, H, P, N)  fp32        NULL means not wanted; may alias initial_state
 *   workspace     >= ssd_fwd_workspace_size(dims, chunk_size) bytes of device memory
 * batch == 0 is a no-op.  seqlen == 0 writes only final_state (= initial_state or zeros). */
ssd_status_t ssd_fwd(const ssd_dims_t* dims,
                     const void* x, const void* dt, const float* dt_bias, const float* A,
                     const void* B, const void* C, const float* D, const void* z, int chunk_size,
                     const float* initial_state, void* y, float* final_state,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the fixed device scratch that ssd_fwd_noalloc uses as its workspace. */
#define SSD_FWD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* ssd_fwd for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same operation, arguments and results as
 * ssd_fwd, but the workspace is a fixed array of SSD_FWD_NOALLOC_SCRATCH_BYTES inside the library
 * (one per device, held until the process ends), so the call allocates nothing; the caller still
 * passes the inputs and outputs.  Sizes whose ssd_fwd_workspace_size() exceeds the scratch are
 * refused with SSD_ERR_SCRATCH_LIMIT before anything else (nothing launched, nothing written).
 * The first call on a device resolves the array's device address (a host query, no allocation;
 * make that first call outside a graph capture).  Every call on a device shares that device's
 * array and leaves its intermediates there: calls on one device that may run concurrently (on
 * different streams, or from different threads without ordering) race on it and must be
 * serialised by the caller.  Nothing in the scratch needs to start at zero. */
ssd_status_t ssd_fwd_noalloc(const ssd_dims_t* dims,
                             const void* x, const void* dt, const float* dt_bias, const float* A,
                             const void* B, const void* C, const float* D, const void* z, int chunk_size,
                             const float* initial_state, void* y, float* final_state, hipStream_t stream);

/* One recurrent decode step for every (b, h) ("MAMBA2 Inference Optimization Report", Step 4:
 * the carried hidden state; same discretisation as ssd_fwd).  dims->seqlen is ignored.
 *   state  (B, H, P, N) fp32    read and overwritten in place with h_t
 *   x      (B, H, P)    dtype   dt (B, H) dtype   dt_bias, A (H) fp32
 *   B, C   (B, G, N)    dtype   D (H, P) fp32 or NULL   z (B, H, P) dtype or NULL (gate)
 *   y      (B, H, P)    dtype   output, computed from the UPDATED state
 * One kernel; no workspace.  batch == 0 is a no-op. */
ssd_status_t ssd_step(const ssd_dims_t* dims, float* state,
                      const void* x, const void* dt, const float* dt_bias, const float* A,
                      const void* B, const void* C, const float* D, const void* z,
                      void* y, hipStream_t stream);

/* Workspace bytes ssd_bwd needs for these sizes and chunk size, with or without a gate
 * (with_gate != 0 adds room for the pre-gate output and the gated gradient).  0 if the sizes
 * are invalid or unsupported.  The workspace holds the recomputed forward intermediates (for
 * bf16 inputs with a bf16 copy of the entering states, B * nc * H * P * N bf16), the
 * state gradients of every chunk (2 * B * nc * H * P * N fp32), per-head dB and dC
 * (2 * B * L * H * N fp32) and small per-token and per-chunk partials. */
size_t ssd_bwd_workspace_size(const ssd_dims_t* dims, int chunk_size, int with_gate);

/* Gradients of ssd_fwd (y and final_state) with respect to every input: the exact gradient
 * of the recurrence (section 3.2 of "Agent 228: MAMBA-2 Reference Implementations
 * Comparison", D skip of Gap 4 of "Agent 228: MAMBA-2 Implementation Gaps", optional gate and
 * dt clamp), evaluated chunk by chunk as in Gap 1.  Inputs are ssd_fwd's (same dims, chunk
 * size and pointers; the forward intermediates are recomputed, nothing from the forward call
 * is needed) plus:
 *   dout            (B, L, H, P)  dtype   dL/dy (y as ssd_fwd returns it, gate included)
 *   dfinal_state    (B, H, P, N)  fp32    dL/dfinal_state; NULL means zero
 * Outputs (all written, none accumulated into):
 *   dx (B, L, H, P), ddt (B, L, H), dB and dC (B, L, G, N)   dtype
 *   ddt_bias, dA (H)   fp32     dD (H, P) fp32 or NULL (not wanted)
 *   dz (B, L, H, P) dtype: required exactly when z is given
 *   dinitial_state (B, H, P, N) fp32 or NULL (not wanted)
 * ddt is the gradient with respect to the raw dt (before bias and softplus); it is zero where
 * the clamp binds.  Results are deterministic (fixed-order reductions, no atomics).
 * With no tokens (batch == 0 or seqlen == 0) ddt_bias, dA and dD are written as zeros and
 * dinitial_state = dfinal_state (or zeros); the per-token tensors may then be NULL, and so may
 * the workspace when ssd_bwd_workspace_size() is 0.  Nine kernels (two more with a gate). */
ssd_status_t ssd_bwd(const ssd_dims_t* dims,
                     const void* x, const void* dt, const float* dt_bias, const float* A,
                     const void* B, const void* C, const float* D, const void* z, int chunk_size,
                     const float* initial_state, const void* dout, const float* dfinal_state,
                     void* dx, void* ddt, float* ddt_bias, float* dA, void* dB, void* dC, float* dD,
                     void* dz, float* dinitial_state,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gated RMSNorm of the scan output ("Agent 228: MAMBA-2 Reference Implementations Comparison",
 * section 7.3: item 9, the output gate y * silu(z); item 11, an RMSNorm in front of the final
 * projection).  Over each token's channels in groups of norm_heads consecutive heads
 * (norm_heads * P channels; norm_heads = H normalises all of d_inner):
 *     g = y * silu(z)  (g = y when z is NULL),   out = g / sqrt(mean_group(g^2) + eps) * weight
 *   y, z, out  (B, L, H, P)  dtype   16-byte aligned; out is y itself (in place) or disjoint
 *                                    from y and z
 *   weight     (H * P)       fp32    16-byte aligned, channel order h * P + p
 * norm_heads must divide H and eps must be finite and >= 0 (else SSD_ERR_INVALID_ARG); headdim a
 * multiple of 8 (else SSD_ERR_UNSUPPORTED).  dims->dstate, ngroups and dt_min/dt_max are not used
 * (they must still be valid).  batch == 0 or seqlen == 0 is a no-op; for decoding pass one token
 * per sequence (seqlen = 1).  The sum of squares is accumulated in fp32 in a fixed order
 * (deterministic).  One kernel, one pass over y, z and out in HBM. */
ssd_status_t ssd_gated_rmsnorm(const ssd_dims_t* dims, const void* y, const void* z, const float* weight,
                               float eps, int norm_heads, void* out, hipStream_t stream);

/* Causal depthwise conv1d + SiLU that produces the scan's x, B and C ("Agent 228: MAMBA-2
 * Implementation Gaps", Gap 2: one filter of width K = conv_width per channel, causal padding
 * K - 1; SiLU after it as in section 3.1 of "Agent 228: MAMBA-2 Reference Implementations
 * Comparison").  Over the Dc = H*P + 2*G*N channels of xbc = [x | B | C]:
 *     u[t, c] = bias[c] + sum_{k<K} weight[c, k] * xbc[t - (K-1) + k, c],   out = u / (1 + e^-u)
 * and out's channels are written to x, B and C.  Inputs before t = 0 come from conv_state_in.
 *   xbc             (B, L, Dc)    dtype   input (16-byte aligned)
 *   weight          (Dc, K)       fp32    weight[c, K-1] multiplies the current token
 *   bias            (Dc)          fp32    NULL means no bias
 *   conv_state_in   (B, K-1, Dc)  dtype   inputs at times -(K-1) .. -1, oldest first; NULL = zeros
 *   conv_state_out  (B, K-1, Dc)  dtype   NULL = not wanted; receives the inputs at times
 *                                         L-(K-1) .. L-1 (older ones from conv_state_in when
 *                                         L < K-1).  Either conv_state_in itself (updated in
 *                                         place) or disjoint from it
 *   x (B, L, H, P), B and C (B, L, G, N)  dtype   outputs, 16-byte aligned, disjoint from the inputs
 * dims->dt_min/dt_max are not used (must still be valid).  conv_width in 1..4 (else
 * SSD_ERR_UNSUPPORTED).  batch == 0 is a no-op; seqlen == 0 writes only conv_state_out.
 * One kernel. */
ssd_status_t ssd_conv1d_silu(const ssd_dims_t* dims, int conv_width, const void* xbc,
                             const float* weight, const float* bias, const void* conv_state_in,
                             void* conv_state_out, void* x, void* B, void* C, hipStream_t stream);

/* One decode token of ssd_conv1d_silu per sequence: xbc (B, Dc) dtype; conv_state
 * (B, K-1, Dc) dtype is read and shifted in place (required when conv_width > 1); outputs
 * x (B, H, P), B and C (B, G, N) dtype.  dims->seqlen is ignored.  One kernel. */
ssd_status_t ssd_conv1d_silu_step(const ssd_dims_t* dims, int conv_width, void* conv_state,
                                  const void* xbc, const float* weight, const float* bias,
                                  void* x, void* B, void* C, hipStream_t stream);

/* Static English description of a status code; never NULL. */
const char* ssd_status_string(ssd_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
