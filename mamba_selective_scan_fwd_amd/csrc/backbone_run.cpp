// backbone_run.cpp -- the native layer loop of the full-backbone prefill.
//
// prefill.rs page (mamba-rs 0.6.4): gpu_forward_inference_prefill and prefill_body -- embed,
// then per layer F1 RMSNorm, F2 in_proj, F4a conv over the x lane of the in_proj output (row
// stride 2*d_inner), F4b x_proj, F4c dt_proj (its bias goes into the scan as dt_bias), F4d the
// scan with B and C read in place from the x_proj output and the gate from the z lane, F5
// out_proj and F6 the residual add (fused here into out_proj as an accumulating GEMM); then
// norm_f on the last timestep of each sequence and the tied LM head (gpu_lm.rs page, mamba-rs
// 0.7.1). The loop runs on the host and only enqueues kernels: no synchronization, no
// allocation, so it can be captured into a HIP graph like every other call.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "../../include/mamba_ssm.h"
#include "launch.hpp"

namespace mamba {

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }


struct BackboneLayout {
  size_t h, xn, proj, u, xdbl, dt, y, last, scan, total;
};

BackboneLayout backbone_layout(const mamba_backbone_dims& d, int B, int T) {
  const size_t bt = (size_t)B * T;
  const size_t xw = (size_t)d.dt_rank + 2 * (size_t)d.d_state;
  BackboneLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += a256(bytes);
    return at;
  };
  l.h = take(bt * d.d_model * 4);
  l.xn = take(bt * d.d_model * 2);
  l.proj = take(bt * 2 * (size_t)d.d_inner * 4);
  l.u = take(bt * d.d_inner * 4);
  l.xdbl = take(bt * xw * 4);
  l.dt = take(bt * d.d_inner * 4);
  l.y = take(bt * d.d_inner * 4);
  l.last = take((size_t)B * d.d_model * 2);
  l.scan = take(plan_selective_scan(B, T, d.d_inner, d.d_state).workspace_bytes);
  l.total = off;
  return l;
}

size_t backbone_workspace_bytes(const mamba_backbone_dims& d, int B, int T) {
  return backbone_layout(d, B, T).total;
}

hipError_t run_backbone_prefill(const mamba_backbone_dims& d, const mamba_backbone_weights& w,
                                const int32_t* tokens, int B, int T, float* conv_state,
                                float* ssm_state, float* logits, void* workspace, hipStream_t s) {
  BackbonePrefillIO io{};
  io.tokens = tokens;
  io.logits = logits;
  return run_backbone_prefill_io(d, w, io, B, T, conv_state, ssm_state, workspace, s);
}

hipError_t run_backbone_prefill_io(const mamba_backbone_dims& d, const mamba_backbone_weights& w,
                                   const BackbonePrefillIO& io, int B, int T, float* conv_state,
                                   float* ssm_state, void* workspace, hipStream_t s) {
  const BackboneLayout lay = backbone_layout(d, B, T);
  char* ws = static_cast<char*>(workspace);
  float* h = reinterpret_cast<float*>(ws + lay.h);
  void* xn = ws + lay.xn;
  float* proj = reinterpret_cast<float*>(ws + lay.proj);
  float* u = reinterpret_cast<float*>(ws + lay.u);
  float* xdbl = reinterpret_cast<float*>(ws + lay.xdbl);
  float* dt = reinterpret_cast<float*>(ws + lay.dt);
  float* y = reinterpret_cast<float*>(ws + lay.y);
  void* last = ws + lay.last;
  void* scan_ws = ws + lay.scan;

  const int64_t bt = (int64_t)B * T;
  const int Dm = d.d_model, D = d.d_inner, N = d.d_state, K = d.d_conv, R = d.dt_rank;
  const int xw = R + 2 * N;
  const auto* in_proj = static_cast<const bf16_storage*>(w.in_proj);
  const auto* x_proj = static_cast<const bf16_storage*>(w.x_proj);
  const auto* dt_proj = static_cast<const bf16_storage*>(w.dt_proj);
  const auto* out_proj = static_cast<const bf16_storage*>(w.out_proj);

  // the residual stream starts at the embedding rows, or at the caller's raw inputs
  hipError_t e = io.embeds ? hipMemcpyAsync(h, io.embeds, sizeof(float) * bt * Dm, hipMemcpyDeviceToDevice, s)
                           : launch_embed_gather(io.tokens, w.embed, h, bt, d.vocab, Dm, s);
  if (e != hipSuccess) return e;
  for (int l = 0; l < d.n_layers; ++l) {
    // F1: normed activations, already bf16 for the in_proj GEMM
    if ((e = launch_rmsnorm(h, Dm, w.norm_w + (int64_t)l * Dm, d.eps, xn, true, bt, Dm, s)) != hipSuccess) return e;
    // F2: proj = xn @ in_proj^T   [bt, 2D]: x lane | z lane
    if ((e = launch_gemm_bf16(xn, true, Dm, in_proj + (int64_t)l * 2 * D * Dm, Dm, proj, 2 * D, (int)bt,
                              2 * D, Dm, false, s)) != hipSuccess) return e;
    // F4a: conv + SiLU over the x lane, carrying this layer's conv state, computed inside
    // F4b: xdbl = u @ x_proj^T   [bt, R + 2N]: dt lane | B | C, split over K, its partial
    // planes in y, which is free until the scan writes it
    // F4c: dt = xdbl[:, :R] @ dt_proj^T   [bt, D], in the kernel that sums x_proj's planes.
    // (The bias and softplus stay in the scan: formed in that kernel's epilogue instead, the
    // 24-layer step measured 6.18 against 6.16 ms.)
    ConvFwdArgs ca{proj, 2 * D, w.conv_w + (int64_t)l * D * K, w.conv_b + (int64_t)l * D,
                   conv_state + (int64_t)l * B * D * K, u, false, B, T, D, K};
    ca.lengths = io.lengths;
    if ((e = launch_conv_xproj_dtproj(ca, x_proj + (int64_t)l * xw * D, xdbl, xw, dt_proj + (int64_t)l * D * R,
                                      R, dt, y, D / xw, DtOut{}, s)) != hipSuccess) return e;
    // F4d: the scan, B/C read in place from xdbl, the gate from the z lane of proj
    ScanFwdArgs sa{u, dt, w.dt_bias + (int64_t)l * D, true, w.A_log + (int64_t)l * D * N,
                   xdbl + R, xdbl + R + N, xw, w.D_skip + (int64_t)l * D, proj + D, 2 * D,
                   ssm_state + (int64_t)l * B * D * N, ssm_state + (int64_t)l * B * D * N, y,
                   false, B, T, D, N, scan_ws};
    sa.lengths = io.lengths;
    // y leaves the scan as bf16: out_proj rounds its operand to bf16 anyway (the same RNE
    // rounding), and a bf16 A is half the bytes and stages straight into LDS
    sa.y_bf16 = true;
    if ((e = launch_selective_scan_fwd(sa, s)) != hipSuccess) return e;
    // F5 + F6: h += y @ out_proj^T
    if ((e = launch_gemm_bf16(y, true, D, out_proj + (int64_t)l * Dm * D, D, h, Dm, (int)bt, Dm, D,
                              true, s)) != hipSuccess) return e;
  }
  // norm_f at every position (the all-T output), and on each sequence's last (valid) token
  // followed by the tied head against the embedding
  if (io.hidden && (e = launch_rmsnorm(h, Dm, w.norm_f, d.eps, io.hidden, false, bt, Dm, s)) != hipSuccess)
    return e;
  if (!io.logits) return hipSuccess;
  if (io.lengths)
    e = launch_rmsnorm_last(h, io.lengths, T, w.norm_f, d.eps, last, true, B, Dm, s);
  else
    e = launch_rmsnorm(h + (int64_t)(T - 1) * Dm, (int64_t)T * Dm, w.norm_f, d.eps, last, true, B, Dm, s);
  if (e != hipSuccess) return e;
  return launch_gemm_bf16(last, true, Dm, w.embed, Dm, io.logits, d.vocab, B, d.vocab, Dm, false, s);
}

// ----------------------------------------------------------------------------- decode step
//
// inference.rs page (mamba-rs 0.5.1), the step chain F1-F12 of the backbone engine: embed one
// token per sequence, then per layer RMSNorm (F1), in_proj (F2), the conv step on the x lane
// (F4, F4b), x_proj (F5), dt_proj (F6), softplus + state update + readout + D skip (F7-F9),
// the silu(z) gate (F10), out_proj (F11) and the residual (F12); then norm_f and the tied head
// (gpu_lm.rs page). Same weights and state layout as the prefill, so a prefill followed by
// decode steps continues one sequence.
//
// Six kernels per layer: RMSNorm with the previous layer's residual add, in_proj, the conv
// step, x_proj, the SSM step (dt_proj, softplus, update, readout, skip, gate), out_proj. The
// projections are split over K for the small batch; their partial planes are summed by the
// kernels that read them (in slice order), not by a reduction kernel of their own.

struct DecodeLayout {
  size_t h, xn, proj, u, xdbl, y, last, part_in, part_x, part_out, total;
};

static DecodeLayout decode_layout(const mamba_backbone_dims& d, int B) {
  const size_t xw = (size_t)d.dt_rank + 2 * (size_t)d.d_state;
  DecodeLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += a256(bytes);
    return at;
  };
  l.h = take((size_t)B * d.d_model * 4);
  l.xn = take((size_t)B * d.d_model * 2);
  l.proj = take((size_t)B * 2 * d.d_inner * 4);
  l.u = take((size_t)B * d.d_inner * 4);
  l.xdbl = take((size_t)B * xw * 4);
  l.y = take((size_t)B * d.d_inner * 4);
  l.last = take((size_t)B * d.d_model * 2);
  // split-K partial planes of in_proj (read by the conv step and, for z, by the SSM step),
  // of x_proj (read by the SSM step) and of out_proj (read by the next RMSNorm): all three
  // are live at once
  auto parts = [&](int N, int K) {
    const int ks = gemm_splitk_slices(B, N, K);
    return ks > 1 ? (size_t)ks * B * N * 4 : 0;
  };
  l.part_in = take(parts(2 * d.d_inner, d.d_model));
  // (the fused conv step + x_proj leaves d_inner / kConvXC planes)
  l.part_x = take(std::max(parts((int)xw, d.d_inner),
                           d.d_inner % kConvXC == 0 ? (size_t)(d.d_inner / kConvXC) * B * xw * 4 : 0));
  l.part_out = take(parts(d.d_model, d.d_inner));
  l.total = off;
  return l;
}

size_t backbone_decode_workspace_bytes(const mamba_backbone_dims& d, int B) {
  return decode_layout(d, B).total;
}

hipError_t run_backbone_decode(const mamba_backbone_dims& d, const mamba_backbone_weights& w,
                               const int32_t* tokens, int B, float* conv_state, float* ssm_state,
                               float* logits, void* workspace, hipStream_t s) {
  const DecodeLayout lay = decode_layout(d, B);
  char* ws = static_cast<char*>(workspace);
  float* h = reinterpret_cast<float*>(ws + lay.h);
  void* xn = ws + lay.xn;
  float* proj = reinterpret_cast<float*>(ws + lay.proj);
  float* u = reinterpret_cast<float*>(ws + lay.u);
  float* xdbl = reinterpret_cast<float*>(ws + lay.xdbl);
  float* y = reinterpret_cast<float*>(ws + lay.y);
  void* last = ws + lay.last;
  float* part_in = reinterpret_cast<float*>(ws + lay.part_in);
  float* part_x = reinterpret_cast<float*>(ws + lay.part_x);
  float* part_out = reinterpret_cast<float*>(ws + lay.part_out);

  const int Dm = d.d_model, D = d.d_inner, N = d.d_state, K = d.d_conv, R = d.dt_rank;
  const int xw = R + 2 * N;
  const auto* in_proj = static_cast<const bf16_storage*>(w.in_proj);
  const auto* x_proj = static_cast<const bf16_storage*>(w.x_proj);
  const auto* dt_proj = static_cast<const bf16_storage*>(w.dt_proj);
  const auto* out_proj = static_cast<const bf16_storage*>(w.out_proj);

  hipError_t e = launch_embed_gather(tokens, w.embed, h, B, d.vocab, Dm, s);
  if (e != hipSuccess) return e;
  const bool fuse_conv_x = D % kConvXC == 0 && B <= kSplitKMaxM;
  PartsView v_out{nullptr, 0, 0, 0};  // the previous layer's out_proj, not yet in h
  for (int l = 0; l < d.n_layers; ++l) {
    // F12 of the previous layer (residual) + F1
    if ((e = launch_residual_rmsnorm(h, v_out, w.norm_w + (int64_t)l * Dm, d.eps, xn, B, Dm, s)) != hipSuccess)
      return e;
    PartsView v_in, v_x;
    if ((e = launch_gemm_bf16_parts(xn, true, Dm, in_proj + (int64_t)l * 2 * D * Dm, Dm, proj, 2 * D, B, 2 * D,
                                    Dm, false, part_in, &v_in, s)) != hipSuccess)
      return e;
    const bf16_storage* wx = x_proj + (int64_t)l * xw * D;
    if (fuse_conv_x && (reinterpret_cast<uintptr_t>(wx) & 15) == 0) {
      // conv step and x_proj in one launch, x_proj left as per-slice partial planes
      if ((e = launch_decode_conv_xproj(v_in, w.conv_w + (int64_t)l * D * K, w.conv_b + (int64_t)l * D,
                                        conv_state + (int64_t)l * B * D * K, u, wx, xw, part_x, &v_x, B, D,
                                        K, s)) != hipSuccess)
        return e;
    } else {
      if ((e = launch_decode_conv(v_in, w.conv_w + (int64_t)l * D * K, w.conv_b + (int64_t)l * D,
                                  conv_state + (int64_t)l * B * D * K, u, B, D, K, s)) != hipSuccess)
        return e;
      if ((e = launch_gemm_bf16_parts(u, false, D, wx, D, xdbl, xw, B, xw, D, false, part_x, &v_x, s)) !=
          hipSuccess)
        return e;
    }
    if ((e = launch_decode_ssm(u, v_x, dt_proj + (int64_t)l * D * R, R, w.dt_bias + (int64_t)l * D,
                               w.A_log + (int64_t)l * D * N, w.D_skip + (int64_t)l * D, v_in, D,
                               ssm_state + (int64_t)l * B * D * N, y, B, D, N, s)) != hipSuccess)
      return e;
    if ((e = launch_gemm_bf16_parts(y, false, D, out_proj + (int64_t)l * Dm * D, D, h, Dm, B, Dm, D, true,
                                    part_out, &v_out, s)) != hipSuccess)
      return e;
  }
  if ((e = launch_residual_rmsnorm(h, v_out, w.norm_f, d.eps, last, B, Dm, s)) != hipSuccess) return e;
  return launch_gemm_bf16(last, true, Dm, w.embed, Dm, logits, d.vocab, B, d.vocab, Dm, false, s);
}

}  // namespace mamba
