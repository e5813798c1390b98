/*
 * mamba_oracle.c -- plain f64 reference for the Mamba-1 selective-scan hot path.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py may load or call this library. The product path never does, and
 * this file shares no code, header or constant with the HIP library.
 *
 * Every function is the plain definition, written out: one sequential loop over
 * time per channel, no blocking, no fusion, no reordering. Channels (b, d) are
 * independent, so an OpenMP loop over channels changes nothing in any result:
 * each channel's arithmetic is the same sequence of IEEE f64 operations whatever
 * the thread count. Build without -ffast-math.
 *
 * Sources (docs.rs source pages of the mamba-rs crate):
 *   [inference.rs]  mamba-rs 0.5.1, src/mamba_ssm/gpu/inference.rs
 *   [prefill.rs]    mamba-rs 0.6.4, src/mamba_ssm/gpu/prefill.rs
 * The pages show host code only (launch sites and argument lists). The update rule
 * itself is the Mamba-1 selective SSM with zero-order-hold A and Euler B:
 *   h_t = exp(delta_t * A) * h_{t-1} + delta_t * B_t * u_t,
 *   y_t = (sum_n C_t[n] h_t[n] + D * u_t) * silu(z_t),   A = -exp(A_log).
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#define _POSIX_C_SOURCE 199309L /* clock_gettime */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <time.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(v) = log(1 + exp(v)), in the overflow-free form.
 * [inference.rs] step chain F7 (dt_proj then softplus); [prefill.rs] prefill_body F4c. */
static double softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }

/* silu(v) = v * sigmoid(v) = v / (1 + exp(-v)).
 * [inference.rs] mixed step chain, fused conv-step + SiLU epilogue (F4 + F4b). */
static double silu(double v) { return v / (1.0 + exp(-v)); }

double oracle_softplus(double v) { return softplus(v); }
double oracle_silu(double v) { return silu(v); }

/* Threads the channel loops run on (for reporting the CPU baseline's core count). */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Prefill causal depthwise conv1d + SiLU over T tokens, carrying the conv state.
 * [prefill.rs] prefill_body F4a (tiled conv over all T with fused SiLU, reading and
 * updating the persistent conv state); [inference.rs] GpuInferenceState (d_conv
 * slots per channel, full window).
 *
 * Per channel (b, d), with the window X = concat(conv_state[b,d,0:K], x[b,0:T,d]):
 *   c[t]    = conv_b[d] + sum_{k<K} conv_w[d,k] * X[t+1+k]
 *   u[b,t,d] = silu(c[t])
 *   conv_state[b,d,k] <- X[T+k]           (the last K entries of the window)
 * Tap K-1 multiplies the current token (cross-correlation with K-1 left padding).
 * conv_state == NULL means a zero history and no state written back.
 * conv_b == NULL means zero bias.
 *   x: element (b,t,d) at (b*T + t)*x_row_stride + d; u: [B,T,D] contiguous.
 */
void oracle_conv1d_fwd(const double* x, int64_t x_row_stride, const double* conv_w,
                       const double* conv_b, double* conv_state, double* u,
                       int B, int T, int D, int K) {
  int64_t nch = (int64_t)B * D;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < nch; ++ch) {
    int b = (int)(ch / D), d = (int)(ch % D);
    double* X = (double*)malloc(sizeof(double) * (size_t)(K + T));
    for (int k = 0; k < K; ++k)
      X[k] = conv_state ? conv_state[((int64_t)b * D + d) * K + k] : 0.0;
    for (int t = 0; t < T; ++t) X[K + t] = x[((int64_t)b * T + t) * x_row_stride + d];
    for (int t = 0; t < T; ++t) {
      double c = conv_b ? conv_b[d] : 0.0;
      for (int k = 0; k < K; ++k) c += conv_w[(int64_t)d * K + k] * X[t + 1 + k];
      u[((int64_t)b * T + t) * D + d] = silu(c);
    }
    if (conv_state)
      for (int k = 0; k < K; ++k) conv_state[((int64_t)b * D + d) * K + k] = X[T + k];
    free(X);
  }
}

/*
 * Prefill selective scan over T tokens, carrying the SSM state.
 * [prefill.rs] prefill_body F4c (delta = softplus(dt_proj output + bias)) and F4d
 * (scan with y gated by silu(z) read from the in_proj output, final state left in
 * the persistent SSM state; the state is not zeroed first);
 * [inference.rs] GpuMambaInference::new (A = -exp(A_log) precomputed per layer).
 *
 * Per channel (b, d), with h[n] starting at ssm_state_in[b,d,n] (NULL: zeros):
 *   A[n]  = -exp(A_log[d,n])
 *   delta = softplus(dt[b,t,d] + dt_bias[d])     if delta_softplus
 *         = dt[b,t,d] + dt_bias[d]               otherwise (dt_bias NULL = 0)
 *   h[n]  = exp(delta*A[n]) * h[n] + delta * Bm[b,t,n] * u[b,t,d]
 *   yv    = sum_n Cm[b,t,n] * h[n] + D_skip[d] * u[b,t,d]     (D_skip NULL = 0)
 *   y[b,t,d] = yv * silu(z[b,t,d])                (z NULL: y = yv)
 *   ssm_state_out[b,d,n] = h[n] after step T-1    (NULL: not written)
 * Layouts: u, dt, y [B,T,D] contiguous; Bm, Cm row (b,t) at (b*T+t)*bc_row_stride;
 * z row (b,t) at (b*T+t)*z_row_stride; A_log [D,N]; states [B,D,N].
 * ssm_state_in may equal ssm_state_out.
 */
void oracle_selective_scan_fwd(const double* u, const double* dt, const double* dt_bias,
                               int delta_softplus, const double* A_log, const double* Bm,
                               const double* Cm, int64_t bc_row_stride, const double* D_skip,
                               const double* z, int64_t z_row_stride, const double* ssm_state_in,
                               double* ssm_state_out, double* y, int B, int T, int D, int N) {
  int64_t nch = (int64_t)B * D;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < nch; ++ch) {
    int b = (int)(ch / D), d = (int)(ch % D);
    double* h = (double*)malloc(sizeof(double) * (size_t)N);
    double* A = (double*)malloc(sizeof(double) * (size_t)N);
    for (int n = 0; n < N; ++n) {
      h[n] = ssm_state_in ? ssm_state_in[((int64_t)b * D + d) * N + n] : 0.0;
      A[n] = -exp(A_log[(int64_t)d * N + n]);
    }
    for (int t = 0; t < T; ++t) {
      int64_t row = (int64_t)b * T + t;
      double ut = u[row * D + d];
      double v = dt[row * D + d] + (dt_bias ? dt_bias[d] : 0.0);
      double delta = delta_softplus ? softplus(v) : v;
      double yv = 0.0;
      for (int n = 0; n < N; ++n) {
        h[n] = exp(delta * A[n]) * h[n] + delta * Bm[row * bc_row_stride + n] * ut;
        yv += Cm[row * bc_row_stride + n] * h[n];
      }
      yv += (D_skip ? D_skip[d] : 0.0) * ut;
      y[row * D + d] = z ? yv * silu(z[row * z_row_stride + d]) : yv;
    }
    if (ssm_state_out)
      for (int n = 0; n < N; ++n) ssm_state_out[((int64_t)b * D + d) * N + n] = h[n];
    free(h);
    free(A);
  }
}

/*
 * One decode step of the conv, for one layer.
 * [inference.rs] step chain F4/F4b (conv step on a d_conv-slot shift register,
 * state mutated in place, then SiLU) and GpuInferenceState (full-window layout).
 * Written separately from oracle_conv1d_fwd: shift the window left by one, put
 * the new token in the last slot, then take the K-tap dot product of the window.
 *   x: element (b,d) at b*x_row_stride + d; conv_state [B,D,K] in place; u [B,D].
 */
void oracle_conv1d_step(const double* x, int64_t x_row_stride, const double* conv_w,
                        const double* conv_b, double* conv_state, double* u, int B, int D, int K) {
  int64_t nch = (int64_t)B * D;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < nch; ++ch) {
    int b = (int)(ch / D), d = (int)(ch % D);
    double* s = conv_state + ((int64_t)b * D + d) * K;
    for (int k = 0; k + 1 < K; ++k) s[k] = s[k + 1];
    s[K - 1] = x[(int64_t)b * x_row_stride + d];
    double c = conv_b ? conv_b[d] : 0.0;
    for (int k = 0; k < K; ++k) c += conv_w[(int64_t)d * K + k] * s[k];
    u[(int64_t)b * D + d] = silu(c);
  }
}

/*
 * One decode step of the SSM, for one layer, state updated in place.
 * [inference.rs] step chain F7 (softplus), F9 (one-token update of the state in
 * place and readout with D), F10 (gate), and the mixed chain's fused
 * gather + step + gate kernel (B and C read in place at a row stride).
 * Same per-channel formula as oracle_selective_scan_fwd with T = 1, written
 * separately.
 *   u, dt, y: [B,D]; Bm, Cm row b at b*bc_row_stride; z row b at b*z_row_stride;
 *   A_log [D,N]; ssm_state [B,D,N] in place.
 */
void oracle_ssm_step(const double* u, const double* dt, const double* dt_bias, int delta_softplus,
                     const double* A_log, const double* Bm, const double* Cm, int64_t bc_row_stride,
                     const double* D_skip, const double* z, int64_t z_row_stride,
                     double* ssm_state, double* y, int B, int D, int N) {
  int64_t nch = (int64_t)B * D;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < nch; ++ch) {
    int b = (int)(ch / D), d = (int)(ch % D);
    double* h = ssm_state + ((int64_t)b * D + d) * N;
    double ut = u[(int64_t)b * D + d];
    double v = dt[(int64_t)b * D + d] + (dt_bias ? dt_bias[d] : 0.0);
    double delta = delta_softplus ? softplus(v) : v;
    double acc = 0.0;
    for (int n = 0; n < N; ++n) {
      double a = exp(delta * (-exp(A_log[(int64_t)d * N + n])));
      h[n] = a * h[n] + delta * Bm[(int64_t)b * bc_row_stride + n] * ut;
      acc += Cm[(int64_t)b * bc_row_stride + n] * h[n];
    }
    acc += (D_skip ? D_skip[d] : 0.0) * ut;
    y[(int64_t)b * D + d] = z ? acc * silu(z[(int64_t)b * z_row_stride + d]) : acc;
  }
}

/*
 * CPU-baseline timing, no arithmetic of its own: the wall time in seconds of
 * oracle_conv1d_fwd followed by oracle_selective_scan_fwd on the given arrays (the conv
 * writes u, which the scan reads), measured with the monotonic clock around the two calls
 * only, with the channel loops on `threads` OpenMP threads (0 = the default team).
 */
double oracle_time_conv_scan(const double* x, int64_t x_row_stride, const double* conv_w,
                             const double* conv_b, double* conv_state, double* u,
                             const double* dt, const double* dt_bias, int delta_softplus,
                             const double* A_log, const double* Bm, const double* Cm,
                             int64_t bc_row_stride, const double* D_skip, const double* z,
                             int64_t z_row_stride, const double* ssm_state_in,
                             double* ssm_state_out, double* y, int B, int T, int D, int N, int K,
                             int threads) {
#ifdef _OPENMP
  const int saved = omp_get_max_threads();
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
  struct timespec t0, t1;
  clock_gettime(CLOCK_MONOTONIC, &t0);
  oracle_conv1d_fwd(x, x_row_stride, conv_w, conv_b, conv_state, u, B, T, D, K);
  oracle_selective_scan_fwd(u, dt, dt_bias, delta_softplus, A_log, Bm, Cm, bc_row_stride, D_skip,
                            z, z_row_stride, ssm_state_in, ssm_state_out, y, B, T, D, N);
  clock_gettime(CLOCK_MONOTONIC, &t1);
#ifdef _OPENMP
  omp_set_num_threads(saved);
#endif
  return (double)(t1.tv_sec - t0.tv_sec) + 1e-9 * (double)(t1.tv_nsec - t0.tv_nsec);
}
