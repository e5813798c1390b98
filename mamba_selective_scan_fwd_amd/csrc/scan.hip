// scan.hip -- prefill selective scan over T tokens with carried SSM state.
//
// prefill.rs page (mamba-rs 0.6.4), prefill_body stages F4c (delta = softplus(dt_proj
// output + bias)) and F4d (scan over all T, y gated by silu(z) read at a row stride, final
// state into the persistent SSM state); inference.rs page (mamba-rs 0.5.1),
// GpuMambaInference::new (A = -exp(A_log)). Softplus, A = -exp(A_log), the D skip and the
// gate are all fused here, so u, dt, z are read once and y is written once.
//
// Layout. Lanes run along d (64 consecutive channels per wave): u/dt/z/y rows are read and
// written coalesced, and the B/C rows of token t are the same for every lane of the wave,
// so they are loaded once as scalars and used as SGPR operands. Each lane keeps its N
// states in registers and walks the tokens of its chunk in order.
//
// T parallelism. T is cut into `chunks` pieces so that B * ceil(D/64) * chunks waves fill
// the chip. A chunk's effect on the state is the affine map h -> P*h + H per (b, d, n), with
// P = exp(A * sum(delta)) and H the state reached from h = 0. Three kernels:
//   1. summary: (P, H) of every chunk but the last;
//   2. prefix:  start state of every chunk, folding the maps in token order from the
//               carried input state (one thread per (b, d, n));
//   3. output:  every chunk rescans its tokens from its start state, writing y; the last
//               chunk writes the final state.
// With one chunk only kernel 3 runs, straight from the carried state.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mamba {

constexpr int kScanWave = 64;

template <int NP, bool EXACT, typename IO>
__device__ __forceinline__ void load_row(float (&dst)[NP], const IO* __restrict__ row, int N) {
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    if constexpr (EXACT) {
      dst[n] = to_f32(row[n]);
    } else {
      const float v = to_f32(row[n < N ? n : N - 1]);
      dst[n] = n < N ? v : 0.0f;
    }
  }
}

// A * log2(e) with A = -exp(A_log); padded states get 0 (decay 1, input 0: they stay 0).
template <int NP, bool EXACT>
__device__ __forceinline__ void load_a2(float (&a2)[NP], const float* __restrict__ A_log, int d,
                                        int N) {
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    if (EXACT || n < N) {
      a2[n] = -expf(A_log[(int64_t)d * N + n]) * kLog2e;
    } else {
      a2[n] = 0.0f;
    }
  }
}

__device__ __forceinline__ float make_delta(float dtv, float bias, bool sp) {
  const float v = dtv + bias;
  return sp ? softplus(v) : v;
}

// Kernel 1: per (b, d, chunk c < chunks-1) the chunk map (P, H).
template <typename IO, int NP, bool EXACT>
__global__ void __launch_bounds__(kScanWave) scan_chunk_summary_kernel(
    const IO* __restrict__ u, const IO* __restrict__ dt, const float* __restrict__ dt_bias,
    int delta_softplus, const float* __restrict__ A_log, const IO* __restrict__ Bm,
    int64_t bc_row_stride, float* __restrict__ P_out, float* __restrict__ H_out, int B, int T,
    int D, int N, int chunk_t) {
  const int d = blockIdx.x * kScanWave + threadIdx.x;
  const int b = blockIdx.y;
  const int c = blockIdx.z;
  if (d >= D) return;
  const int t0 = c * chunk_t;
  const int t1 = min(T, t0 + chunk_t);

  float a2[NP];
  load_a2<NP, EXACT>(a2, A_log, d, N);
  const float bias = dt_bias ? dt_bias[d] : 0.0f;
  const bool sp = delta_softplus != 0;

  float H[NP];
#pragma unroll
  for (int n = 0; n < NP; ++n) H[n] = 0.0f;
  float sum_delta = 0.0f;

  for (int t = t0; t < t1; ++t) {
    const int64_t row = (int64_t)b * T + t;
    const float delta = make_delta(to_f32(dt[row * D + d]), bias, sp);
    const float du = delta * to_f32(u[row * D + d]);
    float bv[NP];
    load_row<NP, EXACT>(bv, Bm + row * bc_row_stride, N);
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      const float a = __builtin_amdgcn_exp2f(delta * a2[n]);
      H[n] = fmaf(a, H[n], du * bv[n]);
    }
    sum_delta += delta;
  }

  float* P = P_out + (((int64_t)c * B + b) * D + d) * N;
  float* Hc = H_out + (((int64_t)c * B + b) * D + d) * N;
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    if (EXACT || n < N) {
      P[n] = __builtin_amdgcn_exp2f(sum_delta * a2[n]);
      Hc[n] = H[n];
    }
  }
}

// Kernel 2: start state of every chunk. One thread per (b, d, n); i indexes [B][D][N].
__global__ void __launch_bounds__(256) scan_chunk_prefix_kernel(
    const float* __restrict__ P, const float* __restrict__ H, const float* state_in,
    float* __restrict__ H_in, int64_t bdn, int chunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= bdn) return;
  float h = state_in ? state_in[i] : 0.0f;
  H_in[i] = h;
  for (int c = 0; c + 1 < chunks; ++c) {
    h = fmaf(P[(int64_t)c * bdn + i], h, H[(int64_t)c * bdn + i]);
    H_in[(int64_t)(c + 1) * bdn + i] = h;
  }
}

// Kernel 3: rescan each chunk from its start state; y for every token, final state at the end.
template <typename IO, int NP, bool EXACT>
__global__ void __launch_bounds__(kScanWave) scan_chunk_output_kernel(
    const IO* __restrict__ u, const IO* __restrict__ dt, const float* __restrict__ dt_bias,
    int delta_softplus, const float* __restrict__ A_log, const IO* __restrict__ Bm,
    const IO* __restrict__ Cm, int64_t bc_row_stride, const float* __restrict__ D_skip,
    const IO* __restrict__ z, int64_t z_row_stride, const float* h_start, int64_t h_start_chunk,
    float* state_out, IO* __restrict__ y, int B, int T, int D, int N, int chunk_t, int chunks) {
  const int d = blockIdx.x * kScanWave + threadIdx.x;
  const int b = blockIdx.y;
  const int c = blockIdx.z;
  if (d >= D) return;
  const int t0 = c * chunk_t;
  const int t1 = min(T, t0 + chunk_t);

  float a2[NP];
  load_a2<NP, EXACT>(a2, A_log, d, N);
  const float bias = dt_bias ? dt_bias[d] : 0.0f;
  const float dskip = D_skip ? D_skip[d] : 0.0f;
  const bool sp = delta_softplus != 0;

  float h[NP];
  const float* hs = h_start ? h_start + (int64_t)c * h_start_chunk + ((int64_t)b * D + d) * N
                            : nullptr;
#pragma unroll
  for (int n = 0; n < NP; ++n) h[n] = (hs && (EXACT || n < N)) ? hs[n] : 0.0f;

  for (int t = t0; t < t1; ++t) {
    const int64_t row = (int64_t)b * T + t;
    const float uv = to_f32(u[row * D + d]);
    const float delta = make_delta(to_f32(dt[row * D + d]), bias, sp);
    const float du = delta * uv;
    float bv[NP], cv[NP];
    load_row<NP, EXACT>(bv, Bm + row * bc_row_stride, N);
    load_row<NP, EXACT>(cv, Cm + row * bc_row_stride, N);
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      const float a = __builtin_amdgcn_exp2f(delta * a2[n]);
      h[n] = fmaf(a, h[n], du * bv[n]);
      acc = fmaf(cv[n], h[n], acc);
    }
    acc = fmaf(dskip, uv, acc);
    if (z) acc *= silu(to_f32(z[row * z_row_stride + d]));
    y[row * D + d] = from_f32<IO>(acc);
  }

  if (c == chunks - 1 && state_out) {
    float* so = state_out + ((int64_t)b * D + d) * N;
#pragma unroll
    for (int n = 0; n < NP; ++n)
      if (EXACT || n < N) so[n] = h[n];
  }
}

// T == 0: the state passes through (copied when out != in; zeros when in is NULL).
__global__ void __launch_bounds__(256) state_copy_kernel(const float* in, float* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = in ? in[i] : 0.0f;
}

// ------------------------------------------------------------------------------ plan/launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

ScanPlan plan_selective_scan(int B, int T, int D, int N) {
  ScanPlan p{1, T, 0};
  if (B <= 0 || T <= 0 || D <= 0 || N <= 0) return p;
  // Aim for ~2 waves per SIMD (256 CUs x 4 SIMDs); chunks of at least 16 tokens.
  const int64_t waves_per_chunk = (int64_t)B * ((D + kScanWave - 1) / kScanWave);
  const int64_t target_waves = 2048;
  int64_t chunks = (target_waves + waves_per_chunk - 1) / waves_per_chunk;
  chunks = std::max<int64_t>(1, std::min<int64_t>(chunks, T / 16));
  const int chunk_t = (int)((T + chunks - 1) / chunks);
  p.chunks = (T + chunk_t - 1) / chunk_t;
  p.chunk_t = chunk_t;
  if (p.chunks > 1) {
    const size_t per = align256(sizeof(float) * (size_t)p.chunks * B * D * N);
    p.workspace_bytes = 3 * per;
  }
  return p;
}

template <typename IO, int NP, bool EXACT>
static hipError_t launch_scan_np(const ScanFwdArgs& a, const ScanPlan& p, hipStream_t s) {
  const dim3 blk(kScanWave);
  const int gx = (a.D + kScanWave - 1) / kScanWave;
  const IO* u = static_cast<const IO*>(a.u);
  const IO* dt = static_cast<const IO*>(a.dt);
  const IO* Bm = static_cast<const IO*>(a.Bm);
  const IO* Cm = static_cast<const IO*>(a.Cm);
  const IO* z = static_cast<const IO*>(a.z);
  IO* y = static_cast<IO*>(a.y);
  if (p.chunks == 1) {
    scan_chunk_output_kernel<IO, NP, EXACT><<<dim3(gx, a.B, 1), blk, 0, s>>>(
        u, dt, a.dt_bias, a.delta_softplus, a.A_log, Bm, Cm, a.bc_row_stride, a.D_skip, z,
        a.z_row_stride, a.state_in, 0, a.state_out, y, a.B, a.T, a.D, a.N, p.chunk_t, 1);
    return hipGetLastError();
  }
  const int64_t bdn = (int64_t)a.B * a.D * a.N;
  const size_t per = align256(sizeof(float) * (size_t)p.chunks * bdn);
  char* ws = static_cast<char*>(a.workspace);
  float* P = reinterpret_cast<float*>(ws);
  float* H = reinterpret_cast<float*>(ws + per);
  float* Hin = reinterpret_cast<float*>(ws + 2 * per);
  scan_chunk_summary_kernel<IO, NP, EXACT><<<dim3(gx, a.B, p.chunks - 1), blk, 0, s>>>(
      u, dt, a.dt_bias, a.delta_softplus, a.A_log, Bm, a.bc_row_stride, P, H, a.B, a.T, a.D,
      a.N, p.chunk_t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  scan_chunk_prefix_kernel<<<dim3((unsigned)((bdn + 255) / 256)), 256, 0, s>>>(
      P, H, a.state_in, Hin, bdn, p.chunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  scan_chunk_output_kernel<IO, NP, EXACT><<<dim3(gx, a.B, p.chunks), blk, 0, s>>>(
      u, dt, a.dt_bias, a.delta_softplus, a.A_log, Bm, Cm, a.bc_row_stride, a.D_skip, z,
      a.z_row_stride, Hin, bdn, a.state_out, y, a.B, a.T, a.D, a.N, p.chunk_t, p.chunks);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_scan_io(const ScanFwdArgs& a, const ScanPlan& p, hipStream_t s) {
  switch (a.N) {
    case 16: return launch_scan_np<IO, 16, true>(a, p, s);
    case 8: return launch_scan_np<IO, 8, true>(a, p, s);
    case 32: return launch_scan_np<IO, 32, true>(a, p, s);
    case 64: return launch_scan_np<IO, 64, true>(a, p, s);
  }
  if (a.N < 8) return launch_scan_np<IO, 8, false>(a, p, s);
  if (a.N < 16) return launch_scan_np<IO, 16, false>(a, p, s);
  if (a.N < 32) return launch_scan_np<IO, 32, false>(a, p, s);
  return launch_scan_np<IO, 64, false>(a, p, s);
}

hipError_t launch_selective_scan_fwd(const ScanFwdArgs& a, hipStream_t s) {
  if (a.T == 0) {
    if (a.state_out && a.state_out != a.state_in) {
      const int64_t n = (int64_t)a.B * a.D * a.N;
      state_copy_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(a.state_in,
                                                                          a.state_out, n);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  const ScanPlan p = plan_selective_scan(a.B, a.T, a.D, a.N);
  return a.bf16 ? launch_scan_io<bf16>(a, p, s) : launch_scan_io<float>(a, p, s);
}

}  // namespace mamba
