// conv1d.hip -- causal depthwise conv1d + SiLU: prefill over T tokens and the decode step.
//
// Prefill: prefill.rs page (mamba-rs 0.6.4), prefill_body stage F4a -- a T-tiled conv that
// reads the x lane strided out of the in_proj output, fuses SiLU, and reads then updates the
// persistent conv state. Decode: inference.rs page (mamba-rs 0.5.1), step chain F4 + F4b and
// the mixed chain's conv-step-with-SiLU kernel -- one token against the d_conv-slot shift
// register held in GpuInferenceState.
//
// Layout: lanes run along d, so every load and store of a [.., T, D] row is coalesced
// (64 consecutive channels per wave). Each thread walks a tile of tokens keeping the last
// K-1 inputs in registers.
#include "common.hpp"
#include "launch.hpp"

namespace mamba {

// One thread per (b, d, token tile). Tile 0 of each channel is the only reader of the old
// conv state (for t < K-1) and the only writer of the new one, so an in-place state update
// never races with another tile.
template <typename IO, int K>
__global__ void __launch_bounds__(256) conv1d_fwd_kernel(
    const IO* __restrict__ x, int64_t x_row_stride, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, float* __restrict__ conv_state, IO* __restrict__ u, int B,
    int T, int D, int tile_t) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  const int t0 = blockIdx.z * tile_t;
  if (d >= D || t0 >= T) return;
  const int t1 = min(T, t0 + tile_t);

  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = conv_w[(int64_t)d * K + k];
  const float bias = conv_b ? conv_b[d] : 0.0f;

  // Window X = [state(K), x(T)]; token t needs X[t+1 .. t+K]. win[j] holds X[t+1+j] for
  // j < K-1 before token t is read.
  float old_state[K];
  float win[K];
  const IO* xb = x + (int64_t)b * T * x_row_stride + d;
  float* st = conv_state ? conv_state + ((int64_t)b * D + d) * K : nullptr;
  if (t0 == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) old_state[k] = st ? st[k] : 0.0f;
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) win[j] = old_state[j + 1];
  } else {
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) {
      const int tt = t0 - (K - 1) + j;  // X index t0+1+j  <->  token t0-(K-1)+j
      win[j] = tt >= 0 ? to_f32(xb[(int64_t)tt * x_row_stride]) : (st ? st[K + tt] : 0.0f);
    }
  }

  IO* ub = u + (int64_t)b * T * D + d;
  for (int t = t0; t < t1; ++t) {
    win[K - 1] = to_f32(xb[(int64_t)t * x_row_stride]);
    float c = bias;
#pragma unroll
    for (int k = 0; k < K; ++k) c = fmaf(w[k], win[k], c);
    ub[(int64_t)t * D] = from_f32<IO>(silu(c));
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) win[j] = win[j + 1];
  }

  if (t0 == 0 && st) {
    // New state: X[T .. T+K-1]. Entries with index >= K are tokens T-K..T-1; the others
    // (only when T < K) are the old state shifted left by T.
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = T + k;
      st[k] = i >= K ? to_f32(xb[(int64_t)(i - K) * x_row_stride]) : old_state[i];
    }
  }
}

// One thread per (l, b, d): shift the K-slot state, insert the token, dot with the taps.
// VEC: the K == 4 state row and taps are 16-byte aligned and move as one float4 each.
template <typename IO, int K, bool VEC>
__global__ void __launch_bounds__(256) conv1d_step_kernel(
    const IO* __restrict__ x, int64_t x_row_stride, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, float* __restrict__ conv_state, IO* __restrict__ u, int L,
    int B, int D) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  const int lb = blockIdx.y;  // l * B + b
  if (d >= D) return;
  const int l = lb / B;
  float* st = conv_state + ((int64_t)lb * D + d) * K;
  const float* w = conv_w + ((int64_t)l * D + d) * K;
  float s[K];
  if constexpr (VEC) {
    static_assert(K == 4, "vector path is for K == 4");
    const float4 v = *reinterpret_cast<const float4*>(st);
    const float4 wv = *reinterpret_cast<const float4*>(w);
    s[0] = v.y; s[1] = v.z; s[2] = v.w;
    s[3] = to_f32(x[(int64_t)lb * x_row_stride + d]);
    float c = conv_b ? conv_b[(int64_t)l * D + d] : 0.0f;
    c = fmaf(wv.x, s[0], c);
    c = fmaf(wv.y, s[1], c);
    c = fmaf(wv.z, s[2], c);
    c = fmaf(wv.w, s[3], c);
    *reinterpret_cast<float4*>(st) = make_float4(s[0], s[1], s[2], s[3]);
    u[(int64_t)lb * D + d] = from_f32<IO>(silu(c));
  } else {
#pragma unroll
    for (int k = 0; k + 1 < K; ++k) s[k] = st[k + 1];
    s[K - 1] = to_f32(x[(int64_t)lb * x_row_stride + d]);
    float c = conv_b ? conv_b[(int64_t)l * D + d] : 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) c = fmaf(w[k], s[k], c);
#pragma unroll
    for (int k = 0; k < K; ++k) st[k] = s[k];
    u[(int64_t)lb * D + d] = from_f32<IO>(silu(c));
  }
}

// ------------------------------------------------------------------------------ launchers

template <typename IO, int K>
static hipError_t launch_conv_fwd_k(const ConvFwdArgs& a, hipStream_t s) {
  const int threads = 64;
  // Enough token tiles to put several waves on every SIMD; at least 16 tokens per tile so
  // the K-1 halo reads stay a small fraction.
  const int64_t waves_per_tile = (int64_t)a.B * ((a.D + threads - 1) / threads);
  int tiles = (int)((4096 + waves_per_tile - 1) / waves_per_tile);
  tiles = max(1, min(tiles, (a.T + 15) / 16));
  // Tiles after the first must start at t0 >= K-1 so that only tile 0 reads the old state.
  const int tile_t = max((a.T + tiles - 1) / tiles, K);
  tiles = (a.T + tile_t - 1) / tile_t;
  dim3 grid((a.D + threads - 1) / threads, a.B, tiles);
  conv1d_fwd_kernel<IO, K><<<grid, threads, 0, s>>>(
      static_cast<const IO*>(a.x), a.x_row_stride, a.conv_w, a.conv_b, a.conv_state,
      static_cast<IO*>(a.u), a.B, a.T, a.D, tile_t);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_conv_fwd_io(const ConvFwdArgs& a, hipStream_t s) {
  switch (a.K) {
    case 1: return launch_conv_fwd_k<IO, 1>(a, s);
    case 2: return launch_conv_fwd_k<IO, 2>(a, s);
    case 3: return launch_conv_fwd_k<IO, 3>(a, s);
    case 4: return launch_conv_fwd_k<IO, 4>(a, s);
    case 5: return launch_conv_fwd_k<IO, 5>(a, s);
    case 6: return launch_conv_fwd_k<IO, 6>(a, s);
    case 7: return launch_conv_fwd_k<IO, 7>(a, s);
    case 8: return launch_conv_fwd_k<IO, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, hipStream_t s) {
  return a.bf16 ? launch_conv_fwd_io<bf16>(a, s) : launch_conv_fwd_io<float>(a, s);
}

template <typename IO, int K>
static hipError_t launch_conv_step_k(const ConvStepArgs& a, hipStream_t s) {
  const int threads = 256;
  dim3 grid((a.D + threads - 1) / threads, a.L * a.B);
  const bool vec = K == 4 && ((reinterpret_cast<uintptr_t>(a.conv_state) |
                               reinterpret_cast<uintptr_t>(a.conv_w)) & 15) == 0;
  if constexpr (K == 4) {
    if (vec) {
      conv1d_step_kernel<IO, K, true><<<grid, threads, 0, s>>>(
          static_cast<const IO*>(a.x), a.x_row_stride, a.conv_w, a.conv_b, a.conv_state,
          static_cast<IO*>(a.u), a.L, a.B, a.D);
      return hipGetLastError();
    }
  }
  conv1d_step_kernel<IO, K, false><<<grid, threads, 0, s>>>(
      static_cast<const IO*>(a.x), a.x_row_stride, a.conv_w, a.conv_b, a.conv_state,
      static_cast<IO*>(a.u), a.L, a.B, a.D);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_conv_step_io(const ConvStepArgs& a, hipStream_t s) {
  switch (a.K) {
    case 1: return launch_conv_step_k<IO, 1>(a, s);
    case 2: return launch_conv_step_k<IO, 2>(a, s);
    case 3: return launch_conv_step_k<IO, 3>(a, s);
    case 4: return launch_conv_step_k<IO, 4>(a, s);
    case 5: return launch_conv_step_k<IO, 5>(a, s);
    case 6: return launch_conv_step_k<IO, 6>(a, s);
    case 7: return launch_conv_step_k<IO, 7>(a, s);
    case 8: return launch_conv_step_k<IO, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv1d_step(const ConvStepArgs& a, hipStream_t s) {
  return a.bf16 ? launch_conv_step_io<bf16>(a, s) : launch_conv_step_io<float>(a, s);
}

}  // namespace mamba
