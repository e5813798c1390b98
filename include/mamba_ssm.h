/*
 * mamba_ssm.h -- C-ABI of the MI355X (gfx950) Mamba-1 selective-scan hot path.
 *
 * Sources: docs.rs source pages of the mamba-rs crate:
 *   [prefill.rs]   mamba-rs 0.6.4, src/mamba_ssm/gpu/prefill.rs   (prefill_body stages F4a-F4d)
 *   [inference.rs] mamba-rs 0.5.1, src/mamba_ssm/gpu/inference.rs (GpuInferenceState; the f32
 *                  step chain F4-F10; the mixed step chain's fused kernels)
 * The pages give launch sites and argument lists; the update rule is the Mamba-1 selective
 * SSM (zero-order hold on A, Euler on B):
 *   delta = softplus(dt + dt_bias),  A = -exp(A_log)
 *   h[n]  = exp(delta*A[n]) * h[n] + delta * B[n] * u
 *   y     = (sum_n C[n]*h[n] + D*u) * silu(z)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller. The library allocates
 *    nothing, never synchronizes, and never reads device memory on the host, so every call
 *    can be captured into a HIP graph. `stream` is a hipStream_t (NULL = default stream);
 *    all work is enqueued on it.
 *  - I/O tensors (x, u, dt, B, C, z, y) share one element type, `io_dtype`: f32 or bf16.
 *    Small parameters (conv_w, conv_b, dt_bias, A_log, D) and both recurrent states are
 *    always f32, whatever io_dtype is ([inference.rs] mixed-precision engine: norms, biases,
 *    a_log, D and conv weights stay f32; the recurrent state stays f32).
 *  - Sizes are element counts; row strides are in elements of io_dtype.
 *  - Recurrent state layout follows GpuInferenceState ([inference.rs]): per layer,
 *    conv state [B][D][K] (d_conv slots, the last K raw inputs, oldest first) and SSM state
 *    [B][D][N] (n fastest). A caller holding [layer][...] arenas passes base + layer offset.
 *  - Errors: every argument is validated before anything is enqueued. A non-zero status
 *    returns with nothing enqueued, and mamba_last_error() (thread-local) names the call
 *    and the argument. Launch failures return MAMBA_EHIP with the HIP error text.
 *    Device faults surface at the caller's next synchronization.
 *  - Empty work: B == 0, D == 0 or (for the prefill calls) T == 0 is valid and leaves
 *    every output untouched, except that a T == 0 scan with distinct in/out state pointers
 *    copies ssm_state_in (or zeros) to ssm_state_out.
 *  - Supported: 1 <= N <= 64, 1 <= K <= 8. N or K outside that returns MAMBA_EUNSUPPORTED
 *    (never a silent early return).
 */
#ifndef MAMBA_SSM_H
#define MAMBA_SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MAMBA_OK = 0,
  MAMBA_EINVAL = 1,       /* bad pointer, size, stride, alignment or aliasing  */
  MAMBA_EUNSUPPORTED = 2, /* N or K beyond what the kernels are built for     */
  MAMBA_EWORKSPACE = 3,   /* workspace missing or smaller than required      */
  MAMBA_EHIP = 4          /* a HIP runtime call or kernel launch failed       */
} mamba_status;

typedef enum { MAMBA_F32 = 0, MAMBA_BF16 = 1 } mamba_dtype;

/* Thread-local description of the last failure on this thread ("" if none). */
const char* mamba_last_error(void);

/* Library version string. */
const char* mamba_version(void);

/*
 * Prefill causal depthwise conv1d + SiLU over T tokens, carrying the conv state.
 * [prefill.rs] prefill_body F4a: the tiled conv reads the x lane strided out of the
 * in_proj output, applies the d_conv taps and bias, fuses SiLU, and reads then
 * updates the persistent conv state. [inference.rs] GpuInferenceState: d_conv slots.
 *
 * Per channel (b, d), with the window X = [conv_state[b,d,0..K-1], x[b,0..T-1,d]]:
 *   u[b,t,d]        = silu(conv_b[d] + sum_k conv_w[d,k] * X[t+1+k])
 *   conv_state[b,d,:] <- X[T..T+K-1]   (the last K entries of the window)
 * The last tap (k = K-1) multiplies the current token.
 *
 *   x            in   [B,T,*] io_dtype; element (b,t,d) at x[(b*T+t)*x_row_stride + d];
 *                     x_row_stride >= D (2*D when x is the lane of an in_proj output).
 *   conv_w       in   [D,K] f32.             conv_b  in  [D] f32, or NULL for zero bias.
 *   conv_state   in/out [B,D,K] f32, updated in place; NULL = zero history, not written.
 *   u            out  [B,T,D] io_dtype, contiguous; must not overlap any input.
 */
mamba_status mamba_conv1d_fwd(const void* x, int64_t x_row_stride, const float* conv_w,
                              const float* conv_b, float* conv_state, void* u,
                              mamba_dtype io_dtype, int B, int T, int D, int K, void* stream);

/*
 * Bytes of device workspace mamba_selective_scan_fwd (and mamba_conv_scan_fwd) needs for
 * this shape (may be 0). The workspace carries chunk summaries and copies of the incoming
 * states between the kernels of one call; its contents on entry do not matter and are
 * garbage on exit.
 */
size_t mamba_selective_scan_workspace_size(int B, int T, int D, int N);

/*
 * Prefill selective scan over T tokens: takes the carried SSM state and returns it.
 * [prefill.rs] prefill_body F4c (delta = softplus of the dt_proj output plus bias) and
 * F4d (the scan over all T, its y gated by silu(z) read from the in_proj output at a
 * row stride, the final state written to the persistent SSM state, which prefill never
 * zeroes); [inference.rs] GpuMambaInference::new (A = -exp(A_log) per layer).
 *
 * Per channel (b, d), h[n] starting from ssm_state_in[b,d,n]:
 *   delta = softplus(dt[b,t,d] + dt_bias[d])   (delta_softplus != 0)
 *         = dt[b,t,d] + dt_bias[d]             (delta_softplus == 0)
 *   h[n]  = exp(delta * A[n]) * h[n] + delta * Bm[b,t,n] * u[b,t,d],  A[n] = -exp(A_log[d,n])
 *   y[b,t,d] = (sum_n Cm[b,t,n]*h[n] + D_skip[d]*u[b,t,d]) * silu(z[b,t,d])
 *   ssm_state_out[b,d,n] = h[n] after the last token
 *
 *   u, dt        in   [B,T,D] io_dtype, contiguous.
 *   dt_bias      in   [D] f32, or NULL for zero.
 *   A_log        in   [D,N] f32 (any values; no structure is assumed).
 *   Bm, Cm       in   io_dtype; row (b,t) starts at (b*T+t)*bc_row_stride; n = 0..N-1 are
 *                     the first N elements of the row (bc_row_stride >= N; e.g. B and C as
 *                     column blocks of an x_proj output row).
 *   D_skip       in   [D] f32, or NULL for zero.
 *   z            in   io_dtype, element (b,t,d) at z[(b*T+t)*z_row_stride + d]
 *                     (z_row_stride >= D), or NULL for no gate (y = the ungated value).
 *   ssm_state_in in   [B,D,N] f32, or NULL for a zero initial state.
 *   ssm_state_out out [B,D,N] f32, or NULL; may equal ssm_state_in (update in place) but
 *                     must not partially overlap it.
 *   y            out  [B,T,D] io_dtype, contiguous; must not overlap any input.
 *   workspace    scratch of at least mamba_selective_scan_workspace_size(B,T,D,N) bytes,
 *                256-byte aligned (NULL allowed when that size is 0).
 */
mamba_status mamba_selective_scan_fwd(const void* u, const void* dt, const float* dt_bias,
                                      int delta_softplus, const float* A_log, const void* Bm,
                                      const void* Cm, int64_t bc_row_stride, const float* D_skip,
                                      const void* z, int64_t z_row_stride,
                                      const float* ssm_state_in, float* ssm_state_out, void* y,
                                      mamba_dtype io_dtype, int B, int T, int D, int N,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The whole prefill of one layer's SSM core in one call: mamba_conv1d_fwd followed by
 * mamba_selective_scan_fwd, fused so that u need not go through memory. [prefill.rs]
 * prefill_body F4a (conv + SiLU from the carried conv state) then F4c/F4d (softplus, scan,
 * gate); the pages fuse the conv with its SiLU and the scan with its gate, this call fuses
 * the two.
 *
 *   x, x_row_stride, conv_w, conv_b, conv_state, K     as mamba_conv1d_fwd (conv_state in
 *                     place; NULL means zeros and no state is written).
 *   dt ... ssm_state_in, ssm_state_out, y, N, workspace as mamba_selective_scan_fwd; the
 *                     workspace size is mamba_selective_scan_workspace_size(B, T, D, N).
 *   u            out  [B,T,D] io_dtype, or NULL to skip writing it. The scan uses u rounded
 *                     to io_dtype, so the result equals the two separate calls exactly.
 * Errors as the two separate calls; u, y, the states and the workspace must not overlap any
 * input. T = 0 leaves the conv state as it is and passes the SSM state through.
 */
mamba_status mamba_conv_scan_fwd(const void* x, int64_t x_row_stride, const float* conv_w,
                                 const float* conv_b, float* conv_state, const void* dt,
                                 const float* dt_bias, int delta_softplus, const float* A_log,
                                 const void* Bm, const void* Cm, int64_t bc_row_stride,
                                 const float* D_skip, const void* z, int64_t z_row_stride,
                                 const float* ssm_state_in, float* ssm_state_out, void* u, void* y,
                                 mamba_dtype io_dtype, int B, int T, int D, int K, int N,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * mamba_conv_scan_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, results and
 * errors as mamba_conv_scan_fwd without the workspace pair: the chunk summaries go to a fixed
 * scratch array inside the library (16 MiB per GPU, held from the library's first use on that
 * GPU until the process ends). Every shape with d_state <= 53 fits; a shape whose workspace
 * (mamba_selective_scan_workspace_size) exceeds 16 MiB fails with MAMBA_EWORKSPACE before
 * anything is enqueued. The call allocates nothing: it neither calls hipMalloc nor lets a
 * library allocate.
 * All calls on one GPU share its scratch, which keeps whatever the last call left there (every
 * call writes the parts it reads before reading them). Calls whose work may overlap on one GPU
 * (on different streams, or from different threads without ordering) race on the scratch and
 * must not be issued; calls ordered on one stream are safe. The current device must be the
 * one the stream and the buffers belong to.
 */
mamba_status mamba_conv_scan_fwd_noalloc(const void* x, int64_t x_row_stride, const float* conv_w,
                                         const float* conv_b, float* conv_state, const void* dt,
                                         const float* dt_bias, int delta_softplus,
                                         const float* A_log, const void* Bm, const void* Cm,
                                         int64_t bc_row_stride, const float* D_skip,
                                         const void* z, int64_t z_row_stride,
                                         const float* ssm_state_in, float* ssm_state_out, void* u,
                                         void* y, mamba_dtype io_dtype, int B, int T, int D, int K,
                                         int N, void* stream);

/*
 * One decode step of the conv for L independent layers in one launch.
 * [inference.rs] step chain F4 (one-token conv on the d_conv-slot shift register, state
 * mutated in place) + F4b (SiLU), fused as in the mixed chain's conv-step-with-SiLU
 * kernel; GpuInferenceState for the layout.
 *
 * Per (l, b, d): shift conv_state[l,b,d,:] left by one, store x in slot K-1, then
 *   u[l,b,d] = silu(conv_b[l,d] + sum_k conv_w[l,d,k] * conv_state[l,b,d,k]).
 *
 *   x            in   io_dtype; element (l,b,d) at x[(l*B+b)*x_row_stride + d], x_row_stride >= D.
 *   conv_w       in   [L,D,K] f32.     conv_b  in  [L,D] f32, or NULL for zero.
 *   conv_state   in/out [L,B,D,K] f32, updated in place.
 *   u            out  [L,B,D] io_dtype, contiguous.
 * L*B above 65535 is MAMBA_EUNSUPPORTED.
 */
mamba_status mamba_conv1d_step(const void* x, int64_t x_row_stride, const float* conv_w,
                               const float* conv_b, float* conv_state, void* u,
                               mamba_dtype io_dtype, int L, int B, int D, int K, void* stream);

/*
 * One decode step of the SSM for L independent layers in one launch, state in place.
 * [inference.rs] step chain F7 (softplus of dt_proj output), F9 (one-token state update
 * and readout with D, state mutated in place), F10 (silu(z) gate), and the mixed chain's
 * fused kernel that reads B and C in place from the x_proj output and gates before the
 * store. Same formula as mamba_selective_scan_fwd with T = 1.
 *
 *   u, dt        in   [L,B,D] io_dtype, contiguous.
 *   dt_bias      in   [L,D] f32, or NULL.          A_log  in  [L,D,N] f32.
 *   Bm, Cm       in   io_dtype, row (l,b) at (l*B+b)*bc_row_stride, n in the first N elements.
 *   D_skip       in   [L,D] f32, or NULL.
 *   z            in   io_dtype, element (l,b,d) at z[(l*B+b)*z_row_stride + d], or NULL.
 *   ssm_state    in/out [L,B,D,N] f32, updated in place.
 *   y            out  [L,B,D] io_dtype, contiguous.
 * L*B above 65535 is MAMBA_EUNSUPPORTED.
 */
mamba_status mamba_ssm_step(const void* u, const void* dt, const float* dt_bias,
                            int delta_softplus, const float* A_log, const void* Bm,
                            const void* Cm, int64_t bc_row_stride, const float* D_skip,
                            const void* z, int64_t z_row_stride, float* ssm_state, void* y,
                            mamba_dtype io_dtype, int L, int B, int D, int N, void* stream);

/*
 * One decode step of the whole SSM core -- conv, SiLU, softplus, state update, readout, D
 * skip and gate -- for L independent layers in one launch: mamba_conv1d_step followed by
 * mamba_ssm_step, fused so that u does not go through memory. [inference.rs] step chain
 * F4/F4b then F7-F10 (the pages fuse each half; this call fuses the two halves).
 *
 *   x, x_row_stride, conv_w, conv_b, conv_state   as mamba_conv1d_step (conv_state in place).
 *   dt, dt_bias, delta_softplus, A_log, Bm, Cm, bc_row_stride, D_skip, z, z_row_stride,
 *   ssm_state                                      as mamba_ssm_step (ssm_state in place).
 *   u            out  [L,B,D] io_dtype, or NULL to skip writing it. In bf16 the SSM half
 *                     uses u rounded to bf16, exactly as the two separate calls do.
 *   y            out  [L,B,D] io_dtype, contiguous.
 * Errors as the two separate calls; y, u and the states must not overlap any input.
 */
mamba_status mamba_decode_step(const void* x, int64_t x_row_stride, const float* conv_w,
                               const float* conv_b, float* conv_state, const void* dt,
                               const float* dt_bias, int delta_softplus, const float* A_log,
                               const void* Bm, const void* Cm, int64_t bc_row_stride,
                               const float* D_skip, const void* z, int64_t z_row_stride,
                               float* ssm_state, void* u, void* y, mamba_dtype io_dtype, int L,
                               int B, int D, int K, int N, void* stream);

/* ======================================================================================
 * Full-backbone prefill (24-layer Mamba-1 stack) and the layer pieces around the SSM core.
 * [prefill.rs] prefill_body: per layer RMSNorm (F1), in_proj (F2), conv + x_proj (F4a-F4b),
 * dt_proj (F4c), scan (F4d), out_proj (F5), residual add (F6); then norm_f and the
 * last-timestep gather. gpu_lm.rs page (mamba-rs 0.7.1): embedding lookup and the tied LM
 * head, one GEMM against the embedding table with the vocabulary padded to a multiple of 64.
 * Precision: weights bf16; GEMM operands bf16 (activations rounded as they enter the GEMM),
 * f32 accumulation; residual stream, norms, conv, scan and states f32.
 * ====================================================================================== */

/*
 * out[r, :] = E[tokens[r], :] as f32. tokens: [rows] int32 (ids outside [0, vocab) are
 * clamped into range); E: [>= vocab, d_model] bf16, row-major; out: [rows, d_model] f32.
 */
mamba_status mamba_embed_gather(const int32_t* tokens, const void* E, float* out, int64_t rows,
                                int vocab, int d_model, void* stream);

/*
 * RMSNorm: out[r, :] = x[r, :] / sqrt(mean(x[r, :]^2) + eps) * w  ([prefill.rs] F1 and norm_f).
 * x: rows at x + r * x_row_stride (f32), d_model contiguous; w: [d_model] f32 or NULL (= 1);
 * out: [rows, d_model] contiguous, f32 (out_dtype MAMBA_F32) or bf16 (MAMBA_BF16, the form
 * a following GEMM takes). The last-token gather is x = h + (T-1)*d_model with
 * x_row_stride = T*d_model.
 */
mamba_status mamba_rmsnorm(const float* x, int64_t x_row_stride, const float* w, float eps,
                           void* out, mamba_dtype out_dtype, int64_t rows, int d_model,
                           void* stream);

/*
 * C[M, N] = A[M, K] * W[N, K]^T   (accumulate == 0)
 * C[M, N] += A[M, K] * W[N, K]^T  (accumulate != 0; the residual add fused into out_proj)
 * A: f32 or bf16 (a_dtype), rows lda apart, rounded to bf16 on the way in; W: bf16, the
 * nn.Linear layout (one row of K per output column), rows ldw apart; C: f32, rows ldc apart.
 * bf16 MFMA (v_mfma_f32_16x16x32_bf16) with f32 accumulation; M <= 8 (with M * K * 4 bytes
 * <= 64 KB) takes a streaming kernel instead (the LM head). accumulate != 0: C += A * W^T.
 */
mamba_status mamba_gemm_bf16(const void* A, mamba_dtype a_dtype, int64_t lda, const void* W,
                             int64_t ldw, float* C, int64_t ldc, int M, int N, int K,
                             int accumulate, void* stream);

/*
 * The two projections between the conv and the scan of a prefill layer ([prefill.rs]
 * prefill_body F4b and F4c: x_proj of the conv output u gives the dt lane, B and C; the
 * low-rank dt lane goes through dt_proj to give the per-channel dt before its softplus):
 *   xdbl[M, xw]     = u[M, d_inner] * W_x[xw, d_inner]^T          (xw = dt_rank + 2 d_state:
 *                     columns dt lane | B | C)
 *   dt[M, d_inner]  = xdbl[:, 0:dt_rank] * W_dt[d_inner, dt_rank]^T, then + dt_bias when
 *                     dt_bias is given, then softplus when delta_softplus != 0: the scan's
 *                     delta, formed as mamba_selective_scan_fwd forms it (same order, same
 *                     bits), for a scan then called without dt_bias and softplus
 * u f32, rows ldu apart; W_x and W_dt bf16 in the nn.Linear layout, contiguous rows; xdbl
 * and dt f32, contiguous. Operands are rounded to bf16 (RNE) as they enter each product
 * (u, and the dt lane of xdbl as computed in f32), with f32 accumulation, as mamba_gemm_bf16
 * does; x_proj is split over d_inner and its partial sums added in a fixed order, so the
 * values do not depend on timing. workspace: at least
 * mamba_xproj_dtproj_workspace_size(M, d_inner, dt_rank, d_state) bytes (the split's
 * partial planes; may be NULL when that is 0). dt_bias: [d_inner] f32 or NULL (zero).
 * Errors: MAMBA_EINVAL for negative sizes or
 * leading dimensions below d_inner, MAMBA_EWORKSPACE for a missing or short workspace; xdbl,
 * dt and the workspace must not overlap each other or the inputs. M == 0 is a no-op.
 */
size_t mamba_xproj_dtproj_workspace_size(int M, int d_inner, int dt_rank, int d_state);
mamba_status mamba_xproj_dtproj(const float* u, int64_t ldu, const void* W_x, const void* W_dt,
                                float* xdbl, float* dt, const float* dt_bias, int delta_softplus,
                                int M, int d_inner, int dt_rank, int d_state, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Stages F4a-F4c of a prefill layer in one call ([prefill.rs] prefill_body F4a, F4b, F4c):
 * the conv + SiLU of mamba_conv1d_fwd over f32 rows, then x_proj of its output u and dt_proj
 * of the dt lane as mamba_xproj_dtproj with M = B*T. u and the conv state come out as
 * mamba_conv1d_fwd leaves them (same bits); xdbl and dt as mamba_xproj_dtproj computes them.
 * Where d_conv == 4 and d_inner is a multiple of 64 the conv runs inside x_proj's product
 * (u is still stored, for the scan).
 *   x, x_row_stride, conv_w, conv_b, conv_state, u   as mamba_conv1d_fwd with MAMBA_F32.
 *   lengths      in   [B] int32 valid tokens per sequence (device, clamped to [0, T]), or
 *                     NULL (all T): the new conv state is taken after each sequence's own
 *                     last valid token.
 *   W_x, W_dt, xdbl, dt, dt_bias, delta_softplus   as mamba_xproj_dtproj.
 *   workspace    mamba_xproj_dtproj_workspace_size(B*T, d_inner, dt_rank, d_state) bytes.
 * Errors as the two calls; every output must be disjoint from every input and each other.
 */
mamba_status mamba_conv_xproj_dtproj(const float* x, int64_t x_row_stride, const float* conv_w,
                                     const float* conv_b, float* conv_state,
                                     const int32_t* lengths, float* u, const void* W_x,
                                     const void* W_dt, float* xdbl, float* dt,
                                     const float* dt_bias, int delta_softplus, int B, int T,
                                     int d_inner, int d_conv, int dt_rank, int d_state,
                                     void* workspace, size_t workspace_bytes, void* stream);

typedef struct mamba_backbone_dims {
  int n_layers;      /* 24 for the 130m shape */
  int d_model;       /* 768 */
  int d_inner;       /* 1536 */
  int d_state;       /* 16 (<= 64) */
  int d_conv;        /* 4 (<= 8) */
  int dt_rank;       /* 48 */
  int vocab;         /* 50280: logits columns */
  int vocab_padded;  /* 50304: rows of the embedding table (multiple of 64) */
  float eps;         /* RMSNorm epsilon, 1e-5 */
} mamba_backbone_dims;

/* Device pointers to layer-stacked weights (index l is layer l, contiguous):
 * embed [vocab_padded, d_model] bf16 (also the tied head; padded rows are never selected),
 * norm_f [d_model] f32, norm_w [L, d_model] f32, in_proj [L, 2*d_inner, d_model] bf16
 * (rows 0..d_inner-1 make the x lane, d_inner..2*d_inner-1 the z lane), conv_w
 * [L, d_inner, d_conv] f32, conv_b [L, d_inner] f32, x_proj [L, dt_rank + 2*d_state, d_inner]
 * bf16 (output columns: dt lane, then B, then C), dt_proj [L, d_inner, dt_rank] bf16,
 * dt_bias [L, d_inner] f32, A_log [L, d_inner, d_state] f32, D_skip [L, d_inner] f32,
 * out_proj [L, d_model, d_inner] bf16. */
typedef struct mamba_backbone_weights {
  const void* embed;
  const float* norm_f;
  const float* norm_w;
  const void* in_proj;
  const float* conv_w;
  const float* conv_b;
  const void* x_proj;
  const void* dt_proj;
  const float* dt_bias;
  const float* A_log;
  const float* D_skip;
  const void* out_proj;
} mamba_backbone_weights;

/* Bytes of workspace mamba_backbone_prefill needs for B sequences of T tokens. */
size_t mamba_backbone_workspace_size(const mamba_backbone_dims* dims, int B, int T);

/*
 * Prefill B prompts of T tokens through the whole backbone and return the logits of the last
 * token of each ([prefill.rs] gpu_forward_inference_prefill; gpu_lm.rs compute_logits).
 * tokens: [B, T] int32; conv_state [L][B][d_inner][d_conv] and ssm_state
 * [L][B][d_inner][d_state] f32 in/out (prefill continues from them, as the pages' prefill
 * never zeroes the state); logits: [B, vocab] f32. The layer loop runs on the host and
 * enqueues every kernel on `stream`; nothing is synchronized or allocated.
 */
mamba_status mamba_backbone_prefill(const mamba_backbone_dims* dims,
                                    const mamba_backbone_weights* weights,
                                    const int32_t* tokens, int B, int T, float* conv_state,
                                    float* ssm_state, float* logits, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Prefill variants of mamba_backbone_prefill (the pages' prefill output and batching
 * options): [prefill.rs] the prefill that returns the norm_f output of every position
 * instead of only the last one, the prefill from raw input rows instead of token ids, and a
 * ragged batch in which each sequence has its own length (the pages fall back to step-by-step
 * decoding for it; here one batched call).
 *
 *   tokens   in   [B, T] int32, or NULL when embeds is given (exactly one of the two).
 *   embeds   in   [B, T, d_model] f32 raw input rows (the residual stream starts there).
 *   lengths  in   [B] int32 device array or NULL (= T for all). Sequences are right-padded to
 *                 T; each one's states are taken after its own last token (a length is
 *                 clamped to [0, T]; 0 leaves that sequence's states unchanged). Outputs at
 *                 padded positions are unspecified.
 *   logits   out  [B, vocab] f32: the head on each sequence's last valid token, or NULL.
 *   hidden   out  [B, T, d_model] f32: norm_f of the residual stream at every position, or NULL.
 * At least one of logits and hidden. Workspace: mamba_backbone_workspace_size(dims, B, T).
 */
typedef struct mamba_prefill_io {
  const int32_t* tokens;
  const float* embeds;
  const int32_t* lengths;
  float* logits;
  float* hidden;
} mamba_prefill_io;
mamba_status mamba_backbone_prefill_ex(const mamba_backbone_dims* dims,
                                       const mamba_backbone_weights* weights,
                                       const mamba_prefill_io* io, int B, int T,
                                       float* conv_state, float* ssm_state, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * One decode step of the whole backbone: one new token per sequence through all layers and
 * the tied head. [inference.rs] the backbone step chain F1-F12 (RMSNorm, in_proj, conv step
 * on the x lane, x_proj, dt_proj, softplus + state update + readout + D skip, silu(z) gate,
 * out_proj, residual) and [gpu_lm.rs] norm_f + the tied head; the conv and SSM states are
 * the ones mamba_backbone_prefill leaves, so a prefill followed by decode steps continues
 * each sequence.
 *
 *   tokens       in   [B] int32, the next token of each sequence.
 *   conv_state, ssm_state  in/out, layouts as mamba_backbone_prefill, updated in place.
 *   logits       out  [B, vocab] f32.
 *   workspace    at least mamba_backbone_decode_workspace_size(dims, B) bytes, 256-byte aligned.
 * dt_rank + 2 d_state above 1024 is MAMBA_EUNSUPPORTED.
 * Nothing is allocated or synchronized: the call can be captured into a HIP graph.
 */
size_t mamba_backbone_decode_workspace_size(const mamba_backbone_dims* dims, int B);
mamba_status mamba_backbone_decode_step(const mamba_backbone_dims* dims,
                                        const mamba_backbone_weights* weights,
                                        const int32_t* tokens, int B, float* conv_state,
                                        float* ssm_state, float* logits, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * The decode step captured once into a HIP graph and replayed (the inference.rs page
 * captures its decode chain the same way, so a step costs one graph launch instead of one
 * launch per kernel). The graph records the pointers given here: before each launch the
 * caller writes the next tokens into the same `tokens` buffer; the states, logits and
 * workspace are the same buffers every time.
 *   mamba_backbone_decode_graph_create  validates as mamba_backbone_decode_step, captures on
 *       a private stream and instantiates; *graph receives the handle (NULL on failure).
 *       Host-side graph objects are created here; no device memory is allocated.
 *   mamba_graph_launch   enqueues one replay on `stream`.
 *   mamba_graph_destroy  frees the handle (NULL is a no-op).
 */
typedef struct mamba_graph mamba_graph;
mamba_status mamba_backbone_decode_graph_create(const mamba_backbone_dims* dims,
                                                const mamba_backbone_weights* weights,
                                                const int32_t* tokens, int B, float* conv_state,
                                                float* ssm_state, float* logits, void* workspace,
                                                size_t workspace_bytes, mamba_graph** graph);
mamba_status mamba_graph_launch(mamba_graph* graph, void* stream);
void mamba_graph_destroy(mamba_graph* graph);

/* ---------------------------------------------------------------- Mamba-3 SISO decode step
 *
 * [mamba3_siso inference.rs] (mamba-rs 0.2.1), phases F3-F7 of every layer for one new token
 * per sequence, given each layer's in_proj output row:
 *   F3 split of the row into z | x | B | C | dt | A | trap | angles (the order of m3_split's
 *      outputs), with dt = softplus(dt + dt_bias), A = -max(softplus(A), a_floor) and
 *      lambda = sigmoid(trap);
 *   F4 BC-norm (RMSNorm over d_state per group, eps 1e-5, [d_state] weight), the per-head bias
 *      (head h reads group h / (nheads / ngroups)), the angle step
 *      theta = angle_state + dt * angles and the rotation of adjacent B/C pairs (2i, 2i+1) by
 *      theta[i] for i < n_angles;
 *   F5 alpha = exp(dt A), beta = (1 - lambda) dt alpha, gamma = lambda dt;
 *   F6 h[p][n] = alpha h[p][n] + beta v_prev[p] k_prev[n] + gamma x[p] k[n] (k, q the
 *      rotated B and C; k_prev, v_prev the K and V states), y[p] = q . h[p] + D x[p];
 *   F7 g = y silu(z), RMS-normalised per head and scaled by gate_norm_w when that is given.
 * The K state then holds k, the V state x, the angle state theta.
 *
 *   proj         in   [L][B] rows, f32, proj_row_stride >= W floats apart, where
 *                     W = 2 nheads headdim + 2 ngroups d_state + 3 nheads + n_angles.
 *   params       in   per-layer f32 parameters (below); gate_norm_w may be NULL.
 *   a_floor      in   the floor of -A.
 *   ssm_state    in/out [L][B][nheads][headdim][d_state] f32, 16-byte aligned.
 *   k_state      in/out [L][B][nheads][d_state] f32 (the previous rotated B).
 *   v_state      in/out [L][B][nheads][headdim] f32 (the previous x).
 *   angle_state  in/out [L][B][nheads][max(n_angles, 1)] f32.
 *   out          out  [L][B][nheads * headdim] f32, the gated output (the input of out_proj).
 * Limits: d_state a multiple of 4 in [4, 256], headdim in [1, 256], nheads a multiple of
 * ngroups, 0 <= n_angles <= d_state / 2, L * B * nheads < 2^31 (MAMBA_EUNSUPPORTED or
 * MAMBA_EINVAL otherwise). L or B = 0 is a no-op. Outputs must not overlap inputs or each
 * other. Nothing is allocated or synchronized.
 */
typedef struct mamba3_siso_params {
  const float* dt_bias;     /* [L][nheads] */
  const float* b_norm_w;    /* [L][d_state] */
  const float* c_norm_w;    /* [L][d_state] */
  const float* b_bias;      /* [L][nheads][d_state] */
  const float* c_bias;      /* [L][nheads][d_state] */
  const float* D;           /* [L][nheads] */
  const float* gate_norm_w; /* [L][nheads * headdim], or NULL for the plain silu gate */
} mamba3_siso_params;
mamba_status mamba3_siso_step(const float* proj, int64_t proj_row_stride,
                              const mamba3_siso_params* params, float a_floor,
                              float* ssm_state, float* k_state, float* v_state,
                              float* angle_state, float* out, int L, int B, int nheads,
                              int headdim, int d_state, int ngroups, int n_angles, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SSM_H */
