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

template <typename IO, int NQ, bool VEC>
__global__ void __launch_bounds__(256) ssm_step_kernel(
    const IO* __restrict__ u, const IO* __restrict__ dt, const float* __restrict__ dt_bias,
    int delta_softplus, const float* __restrict__ A_log, const IO* __restrict__ Bm,
    const IO* __restrict__ Cm, int64_t bc_row_stride, const float* __restrict__ D_skip,
    const IO* __restrict__ z, int64_t z_row_stride, float* __restrict__ state,
    IO* __restrict__ y, int L, int B, int D, int N) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ch = gid / NQ;  // ((l * B + b) * D + d)
  const int q = (int)(gid % NQ);
  const int64_t nch = (int64_t)L * B * D;
  if (ch >= nch) return;  // whole NQ-lane groups drop out together
  const int d = (int)(ch % D);
  const int64_t lb = ch / D;
  const int l = (int)(lb / B);

  const float uv = to_f32(u[ch]);
  const float v = to_f32(dt[ch]) + (dt_bias ? dt_bias[(int64_t)l * D + d] : 0.0f);
  const float delta = delta_softplus ? softplus(v) : v;
  const float du = delta * uv;

  float* hs = state + ch * N;
  const float* al = A_log + ((int64_t)l * D + d) * N;
  const IO* brow = Bm + lb * bc_row_stride;
  const IO* crow = Cm + lb * bc_row_stride;
  const int n0 = 4 * q;

  float h[4], alog[4];
  if constexpr (VEC) {
    const float4 hv = *reinterpret_cast<const float4*>(hs + n0);
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
  float part = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + j;
    if (VEC || n < N) {
      const float a = __builtin_amdgcn_exp2f(delta * (-expf(alog[j]) * kLog2e));
      h[j] = fmaf(a, h[j], du * to_f32(brow[n]));
      part = fmaf(to_f32(crow[n]), h[j], part);
    }
  }
  if constexpr (VEC) {
    *reinterpret_cast<float4*>(hs + n0) = make_float4(h[0], h[1], h[2], h[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (n0 + j < N) hs[n0 + j] = h[j];
  }
#pragma unroll
  for (int m = NQ / 2; m >= 1; m /= 2) part += __shfl_xor(part, m, NQ);
  if (q == 0) {
    float yv = fmaf(D_skip ? D_skip[(int64_t)l * D + d] : 0.0f, uv, part);
    if (z) yv *= silu(to_f32(z[lb * z_row_stride + d]));
    y[ch] = from_f32<IO>(yv);
  }
}

template <typename IO, int NQ>
static hipError_t launch_step_nq(const SsmStepArgs& a, hipStream_t s) {
  const int64_t threads = (int64_t)a.L * a.B * a.D * NQ;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  const bool vec = a.N % 4 == 0 && ((reinterpret_cast<uintptr_t>(a.state) |
                                     reinterpret_cast<uintptr_t>(a.A_log)) & 15) == 0;
  if (vec) {
    ssm_step_kernel<IO, NQ, true><<<blocks, 256, 0, s>>>(
        static_cast<const IO*>(a.u), static_cast<const IO*>(a.dt), a.dt_bias, a.delta_softplus,
        a.A_log, static_cast<const IO*>(a.Bm), static_cast<const IO*>(a.Cm), a.bc_row_stride,
        a.D_skip, static_cast<const IO*>(a.z), a.z_row_stride, a.state, static_cast<IO*>(a.y),
        a.L, a.B, a.D, a.N);
  } else {
    ssm_step_kernel<IO, NQ, false><<<blocks, 256, 0, s>>>(
        static_cast<const IO*>(a.u), static_cast<const IO*>(a.dt), a.dt_bias, a.delta_softplus,
        a.A_log, static_cast<const IO*>(a.Bm), static_cast<const IO*>(a.Cm), a.bc_row_stride,
        a.D_skip, static_cast<const IO*>(a.z), a.z_row_stride, a.state, static_cast<IO*>(a.y),
        a.L, a.B, a.D, a.N);
  }
  return hipGetLastError();
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
