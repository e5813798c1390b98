// conv1d.hip -- causal depthwise conv1d + SiLU: prefill over T tokens and the decode step.
//
// Prefill: prefill.rs page (mamba-rs 0.6.4), prefill_body stage F4a -- a T-tiled conv that
// reads the x lane strided out of the in_proj output, fuses SiLU, and reads then updates the
// persistent conv state. Decode: inference.rs page (mamba-rs 0.5.1), step chain F4 + F4b and
// the mixed chain's conv-step-with-SiLU kernel -- one token against the d_conv-slot shift
// register held in GpuInferenceState.
//
// Layout: lanes run along d, so every load and store of a [.., T, D] row is coalesced. In the
// prefill a thread owns 4 consecutive channels (16-byte f32 / 8-byte bf16 accesses) when the
// shape allows, and walks a tile of tokens keeping the last K-1 inputs in registers, with the
// next 8 rows already in flight.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mamba {

// V consecutive channels of one row, widened to f32 (V = 4: one 16-byte (f32) or 8-byte
// (bf16) access; V = 1: one element).
template <typename IO, int V>
struct Vec {
  static __device__ __forceinline__ void load(float (&v)[V], const IO* p) {
    if constexpr (V == 1) {
      v[0] = to_f32(p[0]);
    } else if constexpr (sizeof(IO) == 4) {
      // x is read once here (non-temporal: it does not displace reused lines)
      const float4 f = load_stream4(reinterpret_cast<const float*>(p));
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
      typedef unsigned u2 __attribute__((ext_vector_type(2)));
      const u2 rr = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
      const uint2 r = make_uint2(rr[0], rr[1]);
      v[0] = __uint_as_float(r.x << 16);
      v[1] = __uint_as_float(r.x & 0xffff0000u);
      v[2] = __uint_as_float(r.y << 16);
      v[3] = __uint_as_float(r.y & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(IO* p, const float (&v)[V]) {
    if constexpr (V == 1) {
      p[0] = from_f32<IO>(v[0]);
    } else if constexpr (sizeof(IO) == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      IO h[4] = {from_f32<IO>(v[0]), from_f32<IO>(v[1]), from_f32<IO>(v[2]), from_f32<IO>(v[3])};
      *reinterpret_cast<uint2*>(p) = *reinterpret_cast<const uint2*>(h);
    }
  }
};

// Tokens staged ahead: the rows of the next block are loaded while the current block is
// computed, so each thread has one block of loads in flight.
constexpr int kConvTB = 8;

// One thread per (b, V channels, token tile). Tile 0 of each channel group is the only reader
// of the old conv state (tiles after it start at t0 >= K-1) and the only writer of the new
// one, so an in-place state update never races with another tile.
template <typename IO, int K, int V>
__global__ void __launch_bounds__(256) conv1d_fwd_kernel(
    const IO* __restrict__ x, int64_t x_row_stride, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, float* __restrict__ conv_state, IO* __restrict__ u, int B,
    int T, int D, int tile_t, const int32_t* __restrict__ lengths) {
  const int d0 = (blockIdx.x * blockDim.x + threadIdx.x) * V;
  const int b = blockIdx.y;
  const int t0 = blockIdx.z * tile_t;
  if (d0 >= D || t0 >= T) return;
  const int t1 = min(T, t0 + tile_t);

  float w[V][K], bias[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < K; ++k) w[v][k] = conv_w[(int64_t)(d0 + v) * K + k];
    bias[v] = conv_b ? conv_b[d0 + v] : 0.0f;
  }

  // Window X = [state(K), x(T)]; token t needs X[t+1 .. t+K]. win[v][j] holds X[t+1+j] of
  // channel d0+v for j < K-1 before token t is read.
  float old_state[V][K];
  float win[V][K];
  const IO* xb = x + (int64_t)b * T * x_row_stride + d0;
  float* st = conv_state ? conv_state + ((int64_t)b * D + d0) * K : nullptr;
  if (t0 == 0) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
      for (int k = 0; k < K; ++k) old_state[v][k] = st ? st[v * K + k] : 0.0f;
#pragma unroll
      for (int j = 0; j + 1 < K; ++j) win[v][j] = old_state[v][j + 1];
    }
  } else {
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) {
      const int tt = t0 - (K - 1) + j;  // X index t0+1+j  <->  token t0-(K-1)+j
      float r[V];
      if (tt >= 0) {
        Vec<IO, V>::load(r, xb + (int64_t)tt * x_row_stride);
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v) r[v] = st ? st[v * K + K + tt] : 0.0f;
      }
#pragma unroll
      for (int v = 0; v < V; ++v) win[v][j] = r[v];
    }
  }

  IO* ub = u + (int64_t)b * T * D + d0;
  // Two register sets, used in turn: the rows of block tb+kConvTB are loaded before block tb
  // is computed. No load carries a condition (rows past the tile re-read its last row), no
  // loaded register is copied, and the loop has no early exit (tokens past the tile are
  // computed and not stored; the window has served its last token by then): a load under a
  // branch, a copy of a register still being loaded, or paths merging after an exit make the
  // wave wait for the prefetch as well.
  float ra[kConvTB][V], rb[kConvTB][V];
  auto load_block = [&](int tb, float (&r)[kConvTB][V]) {
#pragma unroll
    for (int j = 0; j < kConvTB; ++j) Vec<IO, V>::load(r[j], xb + (int64_t)min(tb + j, t1 - 1) * x_row_stride);
  };
  auto conv_block = [&](int tb, const float (&r)[kConvTB][V]) {
#pragma unroll
    for (int j = 0; j < kConvTB; ++j) {
      const int t = tb + j;
      float out[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        win[v][K - 1] = r[j][v];
        float c = bias[v];
#pragma unroll
        for (int k = 0; k < K; ++k) c = fmaf(w[v][k], win[v][k], c);
        out[v] = silu(c);
#pragma unroll
        for (int i = 0; i + 1 < K; ++i) win[v][i] = win[v][i + 1];
      }
      if (t < t1) Vec<IO, V>::store(ub + (int64_t)t * D, out);
    }
  };
  load_block(t0, ra);
  for (int tb = t0; tb < t1; tb += 2 * kConvTB) {
    load_block(tb + kConvTB, rb);
    conv_block(tb, ra);
    load_block(tb + 2 * kConvTB, ra);
    conv_block(tb + kConvTB, rb);
  }

  if (t0 == 0 && st) {
    // New state: X[Tb .. Tb+K-1] with Tb this sequence's length (T unless lengths are given).
    // Entries with index >= K are tokens Tb-K..Tb-1; the others (Tb < K) are the old state
    // shifted left by Tb.
    const int Tb = lengths ? min(max(lengths[b], 0), T) : T;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = Tb + k;
      float r[V];
      if (i >= K) {
        Vec<IO, V>::load(r, xb + (int64_t)(i - K) * x_row_stride);
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v) r[v] = old_state[v][i];
      }
#pragma unroll
      for (int v = 0; v < V; ++v) st[v * K + k] = r[v];
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
    // (every load first, none under a condition: an absent bias is read from the taps)
    const float4 v = *reinterpret_cast<const float4*>(st);
    const float4 wv = *reinterpret_cast<const float4*>(w);
    const IO xr = x[(int64_t)lb * x_row_stride + d];
    const float cb = *(conv_b ? conv_b + (int64_t)l * D + d : w);
    s[0] = v.y; s[1] = v.z; s[2] = v.w;
    s[3] = to_f32(xr);
    float c = conv_b ? cb : 0.0f;
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

template <typename IO, int K, int V>
static hipError_t launch_conv_fwd_kv(const ConvFwdArgs& a, hipStream_t s, int tile_t, int tiles) {
  const int threads = 256;
  const int lanes = (a.D + V - 1) / V;
  dim3 grid((lanes + threads - 1) / threads, a.B, tiles);
  conv1d_fwd_kernel<IO, K, V><<<grid, threads, 0, s>>>(
      static_cast<const IO*>(a.x), a.x_row_stride, a.conv_w, a.conv_b, a.conv_state,
      static_cast<IO*>(a.u), a.B, a.T, a.D, tile_t, a.lengths);
  return hipGetLastError();
}

// Token tiles: enough (b, channel group, tile) threads for ~16 waves per CU, tiles of at
// least 16 tokens (the K-1 halo stays a small fraction) and at least K tokens (tiles after
// the first never touch the old state). Four channels per thread when that still fills the
// chip and rows are 16-byte aligned; one otherwise.
template <typename IO, int K>
static hipError_t launch_conv_fwd_k(const ConvFwdArgs& a, hipStream_t s) {
  const int64_t target_threads = 256 * 16 * 64;
  const size_t es = sizeof(IO);
  const bool vec_ok = a.D % 4 == 0 && a.x_row_stride % 4 == 0 &&
                      ((reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.u)) % (4 * es)) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.conv_w) % 16) == 0;
  const int max_tiles = std::max(1, (a.T + 15) / 16);
  const bool vec = vec_ok && (int64_t)a.B * (a.D / 4) * max_tiles >= target_threads;
  const int64_t per_tile = (int64_t)a.B * (vec ? a.D / 4 : a.D);
  int tiles = (int)std::min<int64_t>(max_tiles, (target_threads + per_tile - 1) / per_tile);
  tiles = std::min(std::max(tiles, 1), 65535);  // grid z limit
  const int tile_t = std::max((a.T + tiles - 1) / tiles, K);
  tiles = (a.T + tile_t - 1) / tile_t;
  return vec ? launch_conv_fwd_kv<IO, K, 4>(a, s, tile_t, tiles)
             : launch_conv_fwd_kv<IO, K, 1>(a, s, tile_t, tiles);
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
