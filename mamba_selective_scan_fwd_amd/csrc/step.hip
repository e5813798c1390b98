// step.hip -- one decode step of the selective SSM for L independent layers in one launch.
//
// inference.rs page (mamba-rs 0.5.1): the f32 step chain F7 (softplus of the dt_proj
// output), F9 (one-token state update in place and readout with D), F10 (gate), and the
// mixed chain's fused kernel that reads B and C in place from the x_proj output at a row
// stride and applies the silu(z) gate before the store. Here softplus, A = -exp(A_log),
// update, readout, D skip and gate are one kernel and all layers one launch.
//
// The step is HBM-bound: per (l, b, d) it reads and writes N f32 states (128 bytes at
// N = 16) against a handful of flops. Each channel is handled by NQ lanes that own four
// consecutive states apiece, so a wave's state traffic is one contiguous, float4-aligned
// stream; the readout sum over n is finished with a butterfly over the NQ lanes.
#include "common.hpp"
#include "launch.hpp"

namespace mamba {

// Four consecutive B (or C) values of row `row` starting at n0, as f32; VEC loads them as one
// 16-byte (f32) or 8-byte (bf16) access.
template <typename IO, bool VEC>
__device__ __forceinline__ void load4(const IO* row, int n0, int N, float (&v)[4]) {
  if constexpr (VEC) {
    if constexpr (sizeof(IO) == 4) {
      const float4 t = *reinterpret_cast<const float4*>(row + n0);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
      const uint2 t = *reinterpret_cast<const uint2*>(row + n0);
      v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xffff0000u);
      v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = n0 + j < N ? to_f32(row[n0 + j]) : 0.0f;
  }
}

// Grid: x over (channel, lane) pairs of one (layer, batch) row, y = l * B + b.
template <typename IO, int NQ, bool VEC>
__global__ void __launch_bounds__(256) ssm_step_kernel(
    const IO* __restrict__ u, const IO* __restrict__ dt, const float* __restrict__ dt_bias,
    int delta_softplus, const float* __restrict__ A_log, const IO* __restrict__ Bm,
    const IO* __restrict__ Cm, int64_t bc_row_stride, const float* __restrict__ D_skip,
    const IO* __restrict__ z, int64_t z_row_stride, float* __restrict__ state,
    IO* __restrict__ y, int B, int D, int N) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int d = t / NQ;
  const int q = t % NQ;
  if (d >= D) return;  // whole NQ-lane groups drop out together
  const int lb = blockIdx.y;  // l * B + b
  const int l = lb / B;
  const int64_t ch = (int64_t)lb * D + d;
  const int64_t ld = (int64_t)l * D + d;

  // Every load is issued before any value is used, and none under a condition (absent
  // vectors are read from a stand-in address and dropped at the use), so a thread's traffic
  // is in flight at once.
  float* hs = state + ch * N;
  const float* al = A_log + ld * N;
  const int n0 = 4 * q;
  const IO u_raw = u[ch];
  const IO dt_raw = dt[ch];
  const float bias_v = *(dt_bias ? dt_bias + ld : al);
  const float dskip_v = *(D_skip ? D_skip + ld : al);
  const IO z_raw = *(z ? z + (int64_t)lb * z_row_stride + d : u + ch);
  float h[4], alog[4], bv[4], cv[4];
  if constexpr (VEC) {
    const float4 hv = load_stream4(hs + n0);
    const float4 av = *reinterpret_cast<const float4*>(al + n0);
    h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
    alog[0] = av.x; alog[1] = av.y; alog[2] = av.z; alog[3] = av.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = n0 + j < N ? hs[n0 + j] : 0.0f;
      alog[j] = n0 + j < N ? al[n0 + j] : 0.0f;
    }
  }
  load4<IO, VEC>(Bm + (int64_t)lb * bc_row_stride, n0, N, bv);
  load4<IO, VEC>(Cm + (int64_t)lb * bc_row_stride, n0, N, cv);

  const float uv = to_f32(u_raw);
  const float v = to_f32(dt_raw) + (dt_bias ? bias_v : 0.0f);
  const float delta = delta_softplus ? softplus(v) : v;
  const float du = delta * uv;
  float part = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // A * log2(e), A = -exp(A_log); padded states (VEC false, n >= N) have B = C = 0
    const float a2 = -__builtin_amdgcn_exp2f(alog[j] * kLog2e) * kLog2e;
    const float a = __builtin_amdgcn_exp2f(delta * a2);
    h[j] = fmaf(a, h[j], du * bv[j]);
    part = fmaf(cv[j], h[j], part);
  }
  if constexpr (VEC) {
    store_stream4(hs + n0, make_float4(h[0], h[1], h[2], h[3]));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (n0 + j < N) hs[n0 + j] = h[j];
  }
#pragma unroll
  for (int m = NQ / 2; m >= 1; m /= 2) part += __shfl_xor(part, m, NQ);
  if (q == 0) {
    float yv = fmaf(D_skip ? dskip_v : 0.0f, uv, part);
    if (z) yv *= silu(to_f32(z_raw));
    y[ch] = from_f32<IO>(yv);
  }
}

template <typename IO, int NQ>
static hipError_t launch_step_nq(const SsmStepArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(((int64_t)a.D * NQ + 255) / 256), (unsigned)(a.L * a.B));
  const size_t es = sizeof(IO);
  // 16-byte state / A_log rows and 4-element aligned B/C rows
  // (16-byte paths only when the NQ lanes' four states each cover exactly N: with N = 12 or
  // 24, say, NQ rounds up and the last lanes would reach into the next channel's row)
  const bool vec = a.N == 4 * NQ && a.bc_row_stride % 4 == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.state) | reinterpret_cast<uintptr_t>(a.A_log)) & 15) == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.Bm) | reinterpret_cast<uintptr_t>(a.Cm)) % (4 * es)) == 0;
  if (vec) {
    ssm_step_kernel<IO, NQ, true><<<grid, 256, 0, s>>>(
        static_cast<const IO*>(a.u), static_cast<const IO*>(a.dt), a.dt_bias, a.delta_softplus,
        a.A_log, static_cast<const IO*>(a.Bm), static_cast<const IO*>(a.Cm), a.bc_row_stride,
        a.D_skip, static_cast<const IO*>(a.z), a.z_row_stride, a.state, static_cast<IO*>(a.y),
        a.B, a.D, a.N);
  } else {
    ssm_step_kernel<IO, NQ, false><<<grid, 256, 0, s>>>(
        static_cast<const IO*>(a.u), static_cast<const IO*>(a.dt), a.dt_bias, a.delta_softplus,
        a.A_log, static_cast<const IO*>(a.Bm), static_cast<const IO*>(a.Cm), a.bc_row_stride,
        a.D_skip, static_cast<const IO*>(a.z), a.z_row_stride, a.state, static_cast<IO*>(a.y),
        a.B, a.D, a.N);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------- fused step
//
// One decode step of the whole SSM core, conv and SSM fused (the pages' step chain fuses
// the conv with its SiLU and the SSM update with its gate; here the two are one kernel, so
// u never goes through HBM). The NQ lanes of a channel each evaluate the K-tap conv (the
// taps are one 16-byte read for K = 4, shared by the lanes through the cache); lane 0 writes
// the shifted conv state and, when asked, u.
template <typename IO, int NQ, bool VEC, int R>
__global__ void __launch_bounds__(256) decode_step_kernel(const DecodeStepArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int d = t / NQ;
  const int q = t % NQ;
  const int D = a.D, N = a.N, K = a.K;
  if (d >= D) return;  // whole NQ-lane groups drop out together
  // R consecutive (layer, batch) rows of one layer (the launcher ensures B % R == 0): the
  // layer's parameters are read and A is computed once for all R rows, and R rows of state
  // traffic are in flight per thread.
  const int lb0 = blockIdx.y * R;
  const int l = lb0 / a.B;
  const int64_t ld = (int64_t)l * D + d;
  const int n0 = 4 * q;

  const float* w = a.conv_w + ld * K;
  float wk[kMaxConvK];
  if (VEC && K == 4) {
    const float4 wv = *reinterpret_cast<const float4*>(w);
    wk[0] = wv.x; wk[1] = wv.y; wk[2] = wv.z; wk[3] = wv.w;
  } else {
#pragma unroll
    for (int k = 0; k < kMaxConvK; ++k) wk[k] = k < K ? w[k] : 0.0f;
  }
  const float cb = a.conv_b ? a.conv_b[ld] : 0.0f;
  const float bias = a.dt_bias ? a.dt_bias[ld] : 0.0f;
  const float dskip = a.D_skip ? a.D_skip[ld] : 0.0f;
  float a2[4];
  {
    const float* al = a.A_log + ld * N;
    float alog[4];
    if constexpr (VEC) {
      const float4 av = *reinterpret_cast<const float4*>(al + n0);
      alog[0] = av.x; alog[1] = av.y; alog[2] = av.z; alog[3] = av.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) alog[j] = n0 + j < N ? al[n0 + j] : 0.0f;
    }
    // A * log2(e), A = -exp(A_log); padded states (VEC false, n >= N) have B = C = 0
#pragma unroll
    for (int j = 0; j < 4; ++j) a2[j] = -__builtin_amdgcn_exp2f(alog[j] * kLog2e) * kLog2e;
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int lb = lb0 + r;
    const int64_t ch = (int64_t)lb * D + d;

    // conv: shift register of the last K raw inputs, oldest first
    float* cst = a.conv_state + ch * K;
    float sreg[kMaxConvK];
    const float xin = to_f32(static_cast<const IO*>(a.x)[(int64_t)lb * a.x_row_stride + d]);
    float c = cb;
    if (VEC && K == 4) {
      const float4 sv = load_stream4(cst);
      sreg[0] = sv.y; sreg[1] = sv.z; sreg[2] = sv.w; sreg[3] = xin;
#pragma unroll
      for (int k = 0; k < 4; ++k) c = fmaf(wk[k], sreg[k], c);
      if (q == 0) store_stream4(cst, make_float4(sreg[0], sreg[1], sreg[2], sreg[3]));
    } else {
#pragma unroll
      for (int k = 0; k < kMaxConvK; ++k) {
        if (k + 1 < K) sreg[k] = cst[k + 1];
        else if (k + 1 == K) sreg[k] = xin;
      }
#pragma unroll
      for (int k = 0; k < kMaxConvK; ++k)
        if (k < K) c = fmaf(wk[k], sreg[k], c);
      if (q == 0) {
#pragma unroll
        for (int k = 0; k < kMaxConvK; ++k)
          if (k < K) cst[k] = sreg[k];
      }
    }
    const float uv = silu(c);
    if (q == 0 && a.u) static_cast<IO*>(a.u)[ch] = from_f32<IO>(uv);
    // an IO-typed u feeds the SSM, as with the two separate calls
    const float us = to_f32(from_f32<IO>(uv));

    const float v = to_f32(static_cast<const IO*>(a.dt)[ch]) + bias;
    const float delta = a.delta_softplus ? softplus(v) : v;
    const float du = delta * us;

    float* hs = a.ssm_state + ch * N;
    float h[4], bv[4], cv[4];
    if constexpr (VEC) {
      const float4 hv = load_stream4(hs + n0);
      h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = n0 + j < N ? hs[n0 + j] : 0.0f;
    }
    load4<IO, VEC>(static_cast<const IO*>(a.Bm) + (int64_t)lb * a.bc_row_stride, n0, N, bv);
    load4<IO, VEC>(static_cast<const IO*>(a.Cm) + (int64_t)lb * a.bc_row_stride, n0, N, cv);
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float ad = __builtin_amdgcn_exp2f(delta * a2[j]);
      h[j] = fmaf(ad, h[j], du * bv[j]);
      part = fmaf(cv[j], h[j], part);
    }
    if constexpr (VEC) {
      store_stream4(hs + n0, make_float4(h[0], h[1], h[2], h[3]));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < N) hs[n0 + j] = h[j];
    }
#pragma unroll
    for (int m = NQ / 2; m >= 1; m /= 2) part += __shfl_xor(part, m, NQ);
    if (q == 0) {
      float yv = fmaf(dskip, us, part);
      if (a.z) yv *= silu(to_f32(static_cast<const IO*>(a.z)[(int64_t)lb * a.z_row_stride + d]));
      static_cast<IO*>(a.y)[ch] = from_f32<IO>(yv);
    }
  }
}

// The fused step for 4-tap convs with 16-byte state rows (the common case). Every load of the
// thread -- the layer's parameters, then the conv state, x, dt, z, SSM state, B and C of all
// R rows -- is issued before any arithmetic or store, so all of a thread's traffic is in
// flight at once. (In decode_step_kernel the compiler keeps each row's loads behind the
// previous row's state stores, which it cannot prove do not alias them, and waits for each
// group of loads in turn.) Optional inputs are read from a valid stand-in address when absent
// and their values dropped at the use, so no load sits under a branch. The arithmetic is
// decode_step_kernel's, in the same order: the results are the same bits.
template <typename IO, int NQ, int R>
__global__ void __launch_bounds__(256) decode_step_k4_kernel(const DecodeStepArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int d = t / NQ;
  const int q = t % NQ;
  const int D = a.D, N = a.N;
  if (d >= D) return;  // whole NQ-lane groups drop out together
  const int lb0 = blockIdx.y * R;  // R consecutive (layer, batch) rows of one layer
  const int l = lb0 / a.B;
  const int64_t ld = (int64_t)l * D + d;
  const int n0 = 4 * q;
  const IO* __restrict__ x = static_cast<const IO*>(a.x);
  const IO* __restrict__ dt = static_cast<const IO*>(a.dt);
  const IO* __restrict__ zb = a.z ? static_cast<const IO*>(a.z) : x;
  const int64_t zs = a.z ? a.z_row_stride : a.x_row_stride;
  const float* __restrict__ wrow = a.conv_w + ld * 4;

  // the layer's parameters
  const float4 wv = *reinterpret_cast<const float4*>(wrow);
  const float cb_l = *(a.conv_b ? a.conv_b + ld : wrow);
  const float bias_l = *(a.dt_bias ? a.dt_bias + ld : wrow);
  const float dskip_l = *(a.D_skip ? a.D_skip + ld : wrow);
  const float4 av = *reinterpret_cast<const float4*>(a.A_log + ld * N + n0);
  // the rows' inputs and states
  float4 cs[R], hv[R];
  IO xr[R], dtr[R], zr[R];
  float bv[R][4], cv[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int lb = lb0 + r;
    const int64_t ch = (int64_t)lb * D + d;
    cs[r] = load_stream4(a.conv_state + ch * 4);
    xr[r] = x[(int64_t)lb * a.x_row_stride + d];
    dtr[r] = dt[ch];
    zr[r] = zb[(int64_t)lb * zs + d];
    hv[r] = load_stream4(a.ssm_state + ch * N + n0);
    load4<IO, true>(static_cast<const IO*>(a.Bm) + (int64_t)lb * a.bc_row_stride, n0, N, bv[r]);
    load4<IO, true>(static_cast<const IO*>(a.Cm) + (int64_t)lb * a.bc_row_stride, n0, N, cv[r]);
  }

  const float wk[4] = {wv.x, wv.y, wv.z, wv.w};
  const float cb = a.conv_b ? cb_l : 0.0f;
  const float bias = a.dt_bias ? bias_l : 0.0f;
  const float dskip = a.D_skip ? dskip_l : 0.0f;
  float a2[4];
  {
    const float alog[4] = {av.x, av.y, av.z, av.w};
    // A * log2(e), A = -exp(A_log)
#pragma unroll
    for (int j = 0; j < 4; ++j) a2[j] = -__builtin_amdgcn_exp2f(alog[j] * kLog2e) * kLog2e;
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int lb = lb0 + r;
    const int64_t ch = (int64_t)lb * D + d;

    // conv: shift register of the last 4 raw inputs, oldest first
    const float sreg[4] = {cs[r].y, cs[r].z, cs[r].w, to_f32(xr[r])};
    float c = cb;
#pragma unroll
    for (int k = 0; k < 4; ++k) c = fmaf(wk[k], sreg[k], c);
    if (q == 0) store_stream4(a.conv_state + ch * 4, make_float4(sreg[0], sreg[1], sreg[2], sreg[3]));
    const float uv = silu(c);
    if (q == 0 && a.u) static_cast<IO*>(a.u)[ch] = from_f32<IO>(uv);
    // an IO-typed u feeds the SSM, as with the two separate calls
    const float us = to_f32(from_f32<IO>(uv));

    const float v = to_f32(dtr[r]) + bias;
    const float delta = a.delta_softplus ? softplus(v) : v;
    const float du = delta * us;

    float h[4] = {hv[r].x, hv[r].y, hv[r].z, hv[r].w};
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float ad = __builtin_amdgcn_exp2f(delta * a2[j]);
      h[j] = fmaf(ad, h[j], du * bv[r][j]);
      part = fmaf(cv[r][j], h[j], part);
    }
    store_stream4(a.ssm_state + ch * N + n0, make_float4(h[0], h[1], h[2], h[3]));
#pragma unroll
    for (int m = NQ / 2; m >= 1; m /= 2) part += __shfl_xor(part, m, NQ);
    if (q == 0) {
      float yv = fmaf(dskip, us, part);
      if (a.z) yv *= silu(to_f32(zr[r]));
      static_cast<IO*>(a.y)[ch] = from_f32<IO>(yv);
    }
  }
}

#ifndef MAMBA_DECODE_ROWS
#define MAMBA_DECODE_ROWS 2  // (layer, batch) rows per thread when B allows
#endif
#ifndef MAMBA_DECODE_K4
#define MAMBA_DECODE_K4 1  // the 4-tap kernel with every load issued first (1) or the general one (0)
#endif

template <typename IO, int NQ, int R>
static hipError_t launch_decode_nqr(const DecodeStepArgs& a, bool vec, hipStream_t s) {
  const dim3 grid((unsigned)(((int64_t)a.D * NQ + 255) / 256), (unsigned)(a.L * a.B / R));
  if (vec && a.K == 4 && MAMBA_DECODE_K4 != 0)
    decode_step_k4_kernel<IO, NQ, R><<<grid, 256, 0, s>>>(a);
  else if (vec)
    decode_step_kernel<IO, NQ, true, R><<<grid, 256, 0, s>>>(a);
  else
    decode_step_kernel<IO, NQ, false, R><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <typename IO, int NQ>
static hipError_t launch_decode_nq(const DecodeStepArgs& a, hipStream_t s) {
  const size_t es = sizeof(IO);
  // (16-byte paths only when the NQ lanes' four states each cover exactly N: with N = 12 or
  // 24, say, NQ rounds up and the last lanes would reach into the next channel's row)
  const bool vec = a.N == 4 * NQ && a.bc_row_stride % 4 == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.ssm_state) | reinterpret_cast<uintptr_t>(a.A_log) |
                     reinterpret_cast<uintptr_t>(a.conv_state) | reinterpret_cast<uintptr_t>(a.conv_w)) & 15) == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.Bm) | reinterpret_cast<uintptr_t>(a.Cm)) % (4 * es)) == 0;
  if (MAMBA_DECODE_ROWS > 1 && a.B % MAMBA_DECODE_ROWS == 0)
    return launch_decode_nqr<IO, NQ, MAMBA_DECODE_ROWS>(a, vec, s);
  return launch_decode_nqr<IO, NQ, 1>(a, vec, s);
}

template <typename IO>
static hipError_t launch_decode_io(const DecodeStepArgs& a, hipStream_t s) {
  const int nq = (a.N + 3) / 4;
  if (nq <= 1) return launch_decode_nq<IO, 1>(a, s);
  if (nq <= 2) return launch_decode_nq<IO, 2>(a, s);
  if (nq <= 4) return launch_decode_nq<IO, 4>(a, s);
  if (nq <= 8) return launch_decode_nq<IO, 8>(a, s);
  return launch_decode_nq<IO, 16>(a, s);
}

hipError_t launch_decode_step(const DecodeStepArgs& a, hipStream_t s) {
  return a.bf16 ? launch_decode_io<bf16>(a, s) : launch_decode_io<float>(a, s);
}

template <typename IO>
static hipError_t launch_step_io(const SsmStepArgs& a, hipStream_t s) {
  const int nq = (a.N + 3) / 4;
  if (nq <= 1) return launch_step_nq<IO, 1>(a, s);
  if (nq <= 2) return launch_step_nq<IO, 2>(a, s);
  if (nq <= 4) return launch_step_nq<IO, 4>(a, s);
  if (nq <= 8) return launch_step_nq<IO, 8>(a, s);
  return launch_step_nq<IO, 16>(a, s);
}

hipError_t launch_ssm_step(const SsmStepArgs& a, hipStream_t s) {
  return a.bf16 ? launch_step_io<bf16>(a, s) : launch_step_io<float>(a, s);
}

}  // namespace mamba
