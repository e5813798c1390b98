// mamba3.hip -- Mamba-3 SISO decode step on gfx950: phases F3-F7 of a layer for L layers and
// B sequences in one launch (mamba3_siso inference.rs page, mamba-rs 0.2.1: m3_split, BC-norm,
// the per-head bias, the angle step and RoPE, alpha/beta/gamma, the trapezoidal state update
// with its K and V states, and the output gate).
//
// One workgroup (256 threads) per (layer, sequence, head). The head's state is a
// [headdim][d_state] f32 tile, read and written once: it is the bulk of the traffic, so its
// loads are issued first, before the prologue (split, norms, rotation) that they do not depend
// on. Lanes are laid out LPR per state row (LPR = d_state / 4 rounded up to a power of two,
// one float4 of a row per lane), so a wave reads whole rows, contiguous in HBM.
#include "common.hpp"
#include "launch.hpp"

namespace mamba {
namespace {

constexpr int kThreads = 256;
constexpr float kNormEps = 1e-5f;

__device__ __forceinline__ float sigmoid(float v) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp(-v));
}

// Sum of v over the 256 threads of the block, returned to every thread. `red` is 8 floats of
// LDS; the leading barrier lets consecutive calls reuse it.
__device__ __forceinline__ float2 block_sum2(float a, float b, float* red) {
  for (int m = 32; m >= 1; m /= 2) {
    a += __shfl_xor(a, m, 64);
    b += __shfl_xor(b, m, 64);
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[wave] = a;
    red[4 + wave] = b;
  }
  __syncthreads();
  return make_float2((red[0] + red[1]) + (red[2] + red[3]), (red[4] + red[5]) + (red[6] + red[7]));
}

template <int LPR>
__global__ void __launch_bounds__(kThreads) m3_siso_step_kernel(const M3StepArgs a) {
  constexpr int RPW = 64 / LPR;                       // state rows per wave per pass
  constexpr int RPB = 4 * RPW;                        // rows per block per pass
  constexpr int U = RPB >= 64 ? 1 : (64 / RPB > 8 ? 8 : 64 / RPB);  // passes in flight

  const int nh = a.nh, hd = a.hd, ds = a.ds, na = a.na;
  const int h = blockIdx.x % nh;
  const int64_t lb = blockIdx.x / nh;  // l * B + b
  const int l = (int)(lb / a.B);
  const int64_t head = lb * nh + h;    // (l, b, h)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int di = nh * hd, gs = a.ng * ds;
  const float* row = a.proj + lb * a.proj_row_stride;
  float* hs = a.ssm + head * hd * ds;

  const int c = lane % LPR, n0 = 4 * c;
  const int sub = wave * RPW + lane / LPR;
  const bool active = n0 < ds;

  // Every load of the head's prologue, then the first passes' state rows, before any value is
  // used. No load carries a condition: indices are clamped into the tensors (a thread past
  // d_state or headdim, a row past hd, the angle of a head with no angles read an in-bounds
  // slot, or a stand-in address for an absent vector, and the value is dropped at the use).
  // A load under a condition, or a use right after it, makes the wave wait right there; and
  // since loads complete in order, the head's inputs go first, so that waiting for them does
  // not wait for the state rows too.
  const int o_dt = 2 * di + 2 * gs;
  const int g = h / (nh / a.ng);
  const int tds = min(tid, ds - 1), thd = min(tid, hd - 1);
  const int ia = min(tds >> 1, max(na - 1, 0));  // this thread's angle pair (clamped)
  const int64_t pb = ((int64_t)l * nh + h) * ds + tds;
  const float r_dt = row[o_dt + h], r_a = row[o_dt + nh + h], r_lam = row[o_dt + 2 * nh + h];
  const float r_dtb = a.dt_bias[(int64_t)l * nh + h];
  const float r_b = row[2 * di + g * ds + tds], r_c = row[2 * di + gs + g * ds + tds];
  const float r_kp = a.k_state[head * ds + tds];
  const float r_x = row[di + h * hd + thd], r_vp = a.v_state[head * hd + thd], r_z = row[h * hd + thd];
  const float r_bw = a.b_norm_w[(int64_t)l * ds + tds], r_cw = a.c_norm_w[(int64_t)l * ds + tds];
  const float r_bb = a.b_bias[pb], r_cb = a.c_bias[pb];
  float* const ang = a.angle + head * a.angle_stride + ia;
  const float r_ang = *ang;
  const float r_th = *(na > 0 ? row + o_dt + 3 * nh + ia : row + o_dt);
  const float Dh = a.D[(int64_t)l * nh + h];
  const float r_gw = *(a.gate_w ? a.gate_w + (int64_t)l * di + h * hd + thd : row);
  const int n0c = active ? n0 : 0;
  auto row_load = [&](int p) { return load_stream4(hs + (int64_t)min(p, hd - 1) * ds + n0c); };
  float4 hv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) hv[u] = row_load(sub + u * RPB);

  __shared__ float s_braw[256], s_craw[256], s_k[256], s_q[256], s_kp[256];
  __shared__ float s_x[256], s_vp[256], s_y[256], s_red[8];

  // F3: this head's scalars
  const float dt = softplus(r_dt + r_dtb);
  const float A = -fmaxf(softplus(r_a), a.a_floor);
  const float lam = sigmoid(r_lam);
  const float alpha = fast_exp(dt * A);
  const float beta = (1.0f - lam) * dt * alpha, gamma = lam * dt;

  // F4: BC-norm of this head's group, then the head's bias
  float bv = 0.f, cv = 0.f;
  if (tid < ds) {
    bv = r_b;
    cv = r_c;
    s_kp[tid] = r_kp;
  }
  float zr = 0.f;
  if (tid < hd) {
    s_x[tid] = r_x;
    s_vp[tid] = r_vp;
    zr = r_z;
  }
  const float2 ss = block_sum2(bv * bv, cv * cv, s_red);
  if (tid < ds) {
    const float rb = rsqrtf(ss.x / ds + kNormEps), rc = rsqrtf(ss.y / ds + kNormEps);
    s_braw[tid] = bv * rb * r_bw + r_bb;
    s_craw[tid] = cv * rc * r_cw + r_cb;
  }
  __syncthreads();
  // F4: angle step and rotation of adjacent pairs; the K state takes the rotated B
  if (tid < ds) {
    const int i = tid >> 1;
    float kb = s_braw[tid], qc = s_craw[tid];
    if (i < na) {
      const float theta = r_ang + dt * r_th;
      float sn, cs;
      sincosf(theta, &sn, &cs);
      const float kb0 = s_braw[tid & ~1], kb1 = s_braw[tid | 1];
      const float qc0 = s_craw[tid & ~1], qc1 = s_craw[tid | 1];
      if ((tid & 1) == 0) {
        kb = kb0 * cs - kb1 * sn;
        qc = qc0 * cs - qc1 * sn;
        *ang = theta;
      } else {
        kb = kb0 * sn + kb1 * cs;
        qc = qc0 * sn + qc1 * cs;
      }
    }
    s_k[tid] = kb;
    s_q[tid] = qc;
    a.k_state[head * ds + tid] = kb;  // this thread read the old value above
  }
  if (tid < hd) a.v_state[head * hd + tid] = s_x[tid];  // likewise
  __syncthreads();

  // F5/F6: per-lane coefficients of its 4 states
  float kc[4], xc[4], qv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = active ? n0 + j : 0;
    const bool in = active && n0 + j < ds;
    kc[j] = in ? beta * s_kp[n] : 0.f;
    xc[j] = in ? gamma * s_k[n] : 0.f;
    qv[j] = in ? s_q[n] : 0.f;
  }

  for (int p0 = 0; p0 < hd; p0 += U * RPB) {
    if (p0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) hv[u] = row_load(p0 + sub + u * RPB);
    }
    float yp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + sub + u * RPB;
      const bool on = active && p < hd;
      if (!on) hv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      const float vp = on ? s_vp[p] : 0.f, xx = on ? s_x[p] : 0.f;
      float4 hn;
      hn.x = fmaf(alpha, hv[u].x, fmaf(kc[0], vp, xc[0] * xx));
      hn.y = fmaf(alpha, hv[u].y, fmaf(kc[1], vp, xc[1] * xx));
      hn.z = fmaf(alpha, hv[u].z, fmaf(kc[2], vp, xc[2] * xx));
      hn.w = fmaf(alpha, hv[u].w, fmaf(kc[3], vp, xc[3] * xx));
      if (on) store_stream4(hs + (int64_t)p * ds + n0, hn);
      yp[u] = (qv[0] * hn.x + qv[1] * hn.y) + (qv[2] * hn.z + qv[3] * hn.w);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int m = LPR / 2; m >= 1; m /= 2) yp[u] += __shfl_xor(yp[u], m, LPR);
      const int p = p0 + sub + u * RPB;
      if (c == 0 && p < hd) s_y[p] = yp[u] + Dh * s_x[p];
    }
  }
  __syncthreads();

  // F7: gate, optionally RMS-normalised over the head
  float gz = 0.f;
  if (tid < hd) gz = s_y[tid] * silu(zr);
  if (a.gate_w) {
    const float2 sg = block_sum2(gz * gz, 0.f, s_red);
    gz *= rsqrtf(sg.x / hd + kNormEps);
    if (tid < hd) gz *= r_gw;
  }
  if (tid < hd) a.out[lb * di + h * hd + tid] = gz;
}

template <int LPR>
hipError_t launch_lpr(const M3StepArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.L * a.B * a.nh;
  m3_siso_step_kernel<LPR><<<dim3((unsigned)blocks), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_m3_siso_step(const M3StepArgs& a, hipStream_t s) {
  if ((int64_t)a.L * a.B * a.nh == 0 || a.hd == 0) return hipSuccess;
  if (a.ds % 4 != 0 || a.ds > kM3MaxDState || a.hd > kM3MaxHeadDim || a.ds < 4 ||
      a.nh % a.ng != 0 || 2 * a.na > a.ds || (int64_t)a.L * a.B * a.nh > kM3MaxBlocks)
    return hipErrorInvalidValue;
  const int q = a.ds / 4;
  if (q > 32) return launch_lpr<64>(a, s);
  if (q > 16) return launch_lpr<32>(a, s);
  if (q > 8) return launch_lpr<16>(a, s);
  if (q > 4) return launch_lpr<8>(a, s);
  if (q > 2) return launch_lpr<4>(a, s);
  if (q > 1) return launch_lpr<2>(a, s);
  return launch_lpr<1>(a, s);
}

}  // namespace mamba
