// scan.hip -- prefill selective scan over T tokens with carried SSM state.
//
// prefill.rs page (mamba-rs 0.6.4), prefill_body stages F4c (delta = softplus(dt_proj
// output + bias)) and F4d (scan over all T, y gated by silu(z) read at a row stride, final
// state into the persistent SSM state); inference.rs page (mamba-rs 0.5.1),
// GpuMambaInference::new (A = -exp(A_log)). Softplus, A = -exp(A_log), the D skip and the
// gate are all fused here: u, dt, z, B and C are read once and y is written once.
//
// Workgroup = 64 consecutive channels x all NP (padded) states, as kWaves waves. Wave q
// owns states [q*S, (q+1)*S) of every channel (lanes run along d, S = NP / kWaves states
// in registers per lane), so a channel's recurrence is split over the waves by state, not
// by time: there is no rescan and the whole T of a chunk is walked once.
//
// The per-token work that does not depend on the state is shared through LDS, in blocks of
// kWaves tokens: in each block wave q computes delta (softplus) and delta*u for token q of
// the block and silu(z) for the same token, and stages part of the block's B/C rows; every
// wave then reads delta, delta*u and its states' B/C values for the block's tokens from LDS
// and advances its S states, leaving its partial C.h per token in LDS; after the barrier
// wave q adds the kWaves partials of token q, the D skip and the gate, and stores y. The
// block buffers are double-buffered, so one barrier per block orders everything.
//
// T parallelism: when B * ceil(D/64) workgroups cannot fill the chip, T is cut into chunks.
// A chunk acts on the state as h -> P*h + H per (b, d, n), P = exp(A * sum(delta)) and H the
// state it reaches from h = 0. A summary pass computes (sum(delta), H) of every chunk but
// the last; the output pass starts each chunk from the carried state folded through the
// maps of the chunks before it (few chunks, so each workgroup folds them itself).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mamba {

constexpr int kLanes = 64;
constexpr int kWaves = 8;          // waves per workgroup; also tokens per block
constexpr int kThreads = kLanes * kWaves;

struct ScanParams {
  const void* u;
  const void* dt;
  const void* Bm;
  const void* Cm;
  const void* z;
  void* y;
  const float* dt_bias;
  const float* A_log;
  const float* D_skip;
  const float* state_in;   // [B][D][N] or NULL
  float* state_out;        // [B][D][N] or NULL
  float* sum_ws;           // [B][chunks][D]      sum of delta per chunk (chunks > 1)
  float* h_ws;             // [B][chunks][N][D]   chunk end state from h = 0 (chunks > 1)
  float* start_ws;         // [B][N][D]           copy of the carried state (chunks > 1)
  int64_t bc_row_stride;
  int64_t z_row_stride;
  int B, T, D, N;
  int chunk_t, chunks;
  int softplus;
};

// A * log2(e) for A = -exp(A_log) of state n (0 for padded states: decay 1, and their B and
// C are staged as 0, so they stay 0 and add nothing).
__device__ __forceinline__ float a_log2(const float* __restrict__ A_log, int d, int n, int N) {
  return n < N ? -__builtin_amdgcn_exp2f(A_log[(int64_t)d * N + n] * kLog2e) * kLog2e : 0.0f;
}

// OUT = false: summary pass over chunks 0 .. chunks-2 (no y). OUT = true: the output pass.
template <typename IO, int NP, bool OUT, bool GATE>
__global__ void __launch_bounds__(kThreads) scan_kernel(const ScanParams p) {
  constexpr int S = NP / kWaves;  // states per lane
  constexpr int BCW = 2 * NP;     // staged B/C row: per wave group [B(S) | C(S)]
  static_assert(S >= 2 && S * kWaves == NP, "state split");

  __shared__ float2 s_dd[2][kWaves][kLanes];                     // (delta, delta*u)
  __shared__ __attribute__((aligned(16))) float s_bc[2][kWaves][BCW];
  __shared__ float s_yp[OUT ? 2 : 1][OUT ? kWaves : 1][kWaves][kLanes];  // partial C.h

  const int lane = threadIdx.x & (kLanes - 1);
  // wave index, made explicitly wave-uniform so row arithmetic stays scalar
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int d = blockIdx.x * kLanes + lane;
  const bool dval = d < p.D;
  const int dc = dval ? d : p.D - 1;  // clamped channel for loads of masked lanes
  const int b = blockIdx.y;
  const int c = blockIdx.z;
  const int N = p.N, D = p.D;
  const int t0 = c * p.chunk_t;
  const int len = min(p.T, t0 + p.chunk_t) - t0;
  const int nblk = (len + kWaves - 1) / kWaves;
  const int64_t row0 = (int64_t)b * p.T + t0;  // first row of the chunk

  const IO* __restrict__ u = static_cast<const IO*>(p.u);
  const IO* __restrict__ dt = static_cast<const IO*>(p.dt);
  const IO* __restrict__ Bm = static_cast<const IO*>(p.Bm);
  const IO* __restrict__ Cm = static_cast<const IO*>(p.Cm);
  const IO* __restrict__ z = static_cast<const IO*>(p.z);

  float a2[S];
#pragma unroll
  for (int s = 0; s < S; ++s) a2[s] = a_log2(p.A_log, dc, q * S + s, N);
  const float bias = p.dt_bias ? p.dt_bias[dc] : 0.0f;
  const float dskip = p.D_skip ? p.D_skip[dc] : 0.0f;
  const bool sp = p.softplus != 0;

  // ---- start state
  float h[S];
  if constexpr (OUT) {
    if (p.chunks == 1) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = q * S + s;
        h[s] = (p.state_in && n < N) ? p.state_in[((int64_t)b * D + dc) * N + n] : 0.0f;
      }
    } else {
      // carried state, then the maps of chunks 0 .. c-1 in token order
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = q * S + s;
        h[s] = n < N ? p.start_ws[((int64_t)b * N + n) * D + dc] : 0.0f;
      }
      for (int cc = 0; cc < c; ++cc) {
        const int64_t bc_ = (int64_t)b * p.chunks + cc;
        const float sd = p.sum_ws[bc_ * D + dc];
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int n = q * S + s;
          if (n < N) h[s] = fmaf(__builtin_amdgcn_exp2f(a2[s] * sd), h[s], p.h_ws[(bc_ * N + n) * D + dc]);
        }
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < S; ++s) h[s] = 0.0f;
    if (c == 0 && dval) {  // keep the carried state for the output pass (it may be updated in place)
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = q * S + s;
        if (n < N)
          p.start_ws[((int64_t)b * N + n) * D + d] =
              p.state_in ? p.state_in[((int64_t)b * D + d) * N + n] : 0.0f;
      }
    }
  }

  // ---- per-token loads of this wave's token in block k, and its B/C staging values
  // Thread i < kWaves * BCW stages entry i of the block: token i / BCW, slot i % BCW.
  constexpr int BC_PER_T = (kWaves * BCW + kThreads - 1) / kThreads;
  // Loads are never predicated: a token past the chunk re-reads the chunk's last row and a
  // padded state re-reads state N-1 (in bounds; such values are replaced by 0 when staged or
  // never read), so no load result has to be merged with an older value.
  const IO* __restrict__ dt_l = dt + dc;
  const IO* __restrict__ u_l = u + dc;
  const IO* __restrict__ z_l = z + dc;
  auto load_tok = [&](int k, float& rdt, float& ru, float& rz) {
    const int64_t row = row0 + min(k * kWaves + q, len - 1);  // wave-uniform
    rdt = to_f32(dt_l[row * D]);
    ru = to_f32(u_l[row * D]);
    if constexpr (OUT && GATE) rz = to_f32(z_l[row * p.z_row_stride]);
  };
  auto bc_slot = [&](int r, int& j, int& n, bool& isC) {
    const int i = threadIdx.x + r * kThreads;
    j = i / BCW;
    const int slot = i % BCW;
    const int w = slot % (2 * S);
    isC = w >= S;
    n = slot / (2 * S) * S + (isC ? w - S : w);
  };
  auto load_bc = [&](int k, float (&v)[BC_PER_T]) {
#pragma unroll
    for (int r = 0; r < BC_PER_T; ++r) {
      if (threadIdx.x + r * kThreads < kWaves * BCW) {  // whole waves
        int j, n;
        bool isC;
        bc_slot(r, j, n, isC);
        const IO* src = isC ? Cm : Bm;
        v[r] = to_f32(src[(row0 + min(k * kWaves + j, len - 1)) * p.bc_row_stride + min(n, N - 1)]);
      }
    }
  };
  auto store_bc = [&](int k, int buf, const float (&v)[BC_PER_T]) {
#pragma unroll
    for (int r = 0; r < BC_PER_T; ++r) {
      const int i = threadIdx.x + r * kThreads;
      if (i < kWaves * BCW) {
        int j, n;
        bool isC;
        bc_slot(r, j, n, isC);
        const bool ok = k * kWaves + j < len && n < N && (OUT || !isC);
        s_bc[buf][j][i % BCW] = ok ? v[r] : 0.0f;
      }
    }
  };

  // Register sets by block parity: the values of block m live in set m & 1, so the loop,
  // unrolled by two, never copies a register that a load is still filling.
  float pf_dt[2] = {0.0f, 0.0f}, pf_u[2] = {0.0f, 0.0f}, pf_z[2] = {0.0f, 0.0f};
  float pf_bc[2][BC_PER_T];
  float u_blk[2] = {0.0f, 0.0f}, g_blk[2] = {1.0f, 1.0f};  // u, silu(z) of this wave's token

  // stage A: delta, delta*u of this wave's token of block m into LDS; B/C rows of block m
  auto stage_a = [&](int m, auto P) {
    constexpr int st = decltype(P)::value;
    const float delta = sp ? softplus(pf_dt[st] + bias) : pf_dt[st] + bias;
    s_dd[st][q][lane] = make_float2(delta, delta * pf_u[st]);
    u_blk[st] = pf_u[st];
    if constexpr (OUT && GATE) g_blk[st] = silu(pf_z[st]);
    store_bc(m, st, pf_bc[st]);
  };

  float sum_delta = 0.0f;
  // one block: stage A of block k+1, loads of block k+2, stage B of block k, barrier, finish
  auto block = [&](int k, auto P) {
    constexpr int st = decltype(P)::value;  // == k & 1
    constexpr int nx = st ^ 1;
    if (k + 1 < nblk) {
      stage_a(k + 1, std::integral_constant<int, nx>{});
      if (k + 2 < nblk) {
        load_tok(k + 2, pf_dt[st], pf_u[st], pf_z[st]);
        load_bc(k + 2, pf_bc[st]);
      }
    }

    // stage B: every wave advances its S states over the block's tokens
    const int nj = min(kWaves, len - k * kWaves);
    const float* bcg = &s_bc[st][0][q * 2 * S];
#pragma unroll
    for (int j = 0; j < kWaves; ++j) {
      if (j >= nj) break;
      const float2 dd = s_dd[st][j][lane];
      const float* bcr = bcg + j * BCW;
      float bv[S], cv[S];
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) {
        bv[s2] = bcr[s2];
        if constexpr (OUT) cv[s2] = bcr[S + s2];
      }
      float acc = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) {
        const float a = __builtin_amdgcn_exp2f(dd.x * a2[s2]);
        h[s2] = fmaf(a, h[s2], dd.y * bv[s2]);
        if constexpr (OUT) acc = fmaf(cv[s2], h[s2], acc);
      }
      if constexpr (OUT) s_yp[st][j][q][lane] = acc;
      else sum_delta += dd.x;
    }
    __syncthreads();

    // finishing step: token q of the block
    if constexpr (OUT) {
      if (q < nj) {
        float yv = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) yv += s_yp[st][q][w][lane];
        yv = fmaf(dskip, u_blk[st], yv);
        if constexpr (GATE) yv *= g_blk[st];
        if (dval) static_cast<IO*>(p.y)[(row0 + k * kWaves + q) * D + d] = from_f32<IO>(yv);
      }
    }
  };

  // prologue: block 0 staged, block 1 in flight
  load_tok(0, pf_dt[0], pf_u[0], pf_z[0]);
  load_bc(0, pf_bc[0]);
  stage_a(0, std::integral_constant<int, 0>{});
  if (nblk > 1) {
    load_tok(1, pf_dt[1], pf_u[1], pf_z[1]);
    load_bc(1, pf_bc[1]);
  }
  __syncthreads();
  for (int k = 0; k < nblk; k += 2) {
    block(k, std::integral_constant<int, 0>{});
    if (k + 1 < nblk) block(k + 1, std::integral_constant<int, 1>{});
  }

  if (!dval) return;
  if constexpr (OUT) {
    if (c == p.chunks - 1 && p.state_out) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = q * S + s;
        if (n < N) p.state_out[((int64_t)b * D + d) * N + n] = h[s];
      }
    }
  } else {
    const int64_t bc_ = (int64_t)b * p.chunks + c;
    if (q == 0) p.sum_ws[bc_ * D + d] = sum_delta;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int n = q * S + s;
      if (n < N) p.h_ws[(bc_ * N + n) * D + d] = h[s];
    }
  }
}

// T == 0: the state passes through (copied when out != in; zeros when in is NULL).
__global__ void __launch_bounds__(256) state_copy_kernel(const float* in, float* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = in ? in[i] : 0.0f;
}

// ------------------------------------------------------------------------------ plan/launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Launch-plan constants (overridable at build time for tuning sweeps).
#ifndef MAMBA_SCAN_TARGET_WAVES
#define MAMBA_SCAN_TARGET_WAVES 4096  // ~4 waves per SIMD (256 CUs x 4 SIMDs)
#endif
#ifndef MAMBA_SCAN_MIN_CHUNK
#define MAMBA_SCAN_MIN_CHUNK 64  // tokens per chunk, at least
#endif

static int padded_n(int N) { return N <= 16 ? 16 : (N <= 32 ? 32 : 64); }

ScanPlan plan_selective_scan(int B, int T, int D, int N) {
  ScanPlan p{1, T, 0};
  if (B <= 0 || T <= 0 || D <= 0 || N <= 0) return p;
  const int64_t waves_per_chunk = (int64_t)B * ((D + kLanes - 1) / kLanes) * kWaves;
  int64_t chunks = (MAMBA_SCAN_TARGET_WAVES + waves_per_chunk - 1) / waves_per_chunk;
  chunks = std::max<int64_t>(1, std::min<int64_t>(chunks, T / MAMBA_SCAN_MIN_CHUNK));
  // whole blocks of kWaves tokens per chunk
  int chunk_t = (int)((T + chunks - 1) / chunks);
  chunk_t = (chunk_t + kWaves - 1) / kWaves * kWaves;
  p.chunks = (T + chunk_t - 1) / chunk_t;
  p.chunk_t = chunk_t;
  if (p.chunks > 1) {
    const size_t bcd = (size_t)B * p.chunks * D;
    p.workspace_bytes = align256(sizeof(float) * bcd) + align256(sizeof(float) * bcd * N) +
                        align256(sizeof(float) * (size_t)B * N * D);
  }
  return p;
}

template <typename IO, int NP>
static hipError_t launch_scan_np(const ScanFwdArgs& a, const ScanPlan& pl, hipStream_t s) {
  ScanParams p{};
  p.u = a.u;
  p.dt = a.dt;
  p.Bm = a.Bm;
  p.Cm = a.Cm;
  p.z = a.z;
  p.y = a.y;
  p.dt_bias = a.dt_bias;
  p.A_log = a.A_log;
  p.D_skip = a.D_skip;
  p.state_in = a.state_in;
  p.state_out = a.state_out;
  p.bc_row_stride = a.bc_row_stride;
  p.z_row_stride = a.z_row_stride;
  p.B = a.B;
  p.T = a.T;
  p.D = a.D;
  p.N = a.N;
  p.chunk_t = pl.chunk_t;
  p.chunks = pl.chunks;
  p.softplus = a.delta_softplus ? 1 : 0;
  const unsigned gx = (unsigned)((a.D + kLanes - 1) / kLanes);
  if (pl.chunks > 1) {
    char* ws = static_cast<char*>(a.workspace);
    const size_t bcd = (size_t)a.B * pl.chunks * a.D;
    p.sum_ws = reinterpret_cast<float*>(ws);
    ws += align256(sizeof(float) * bcd);
    p.h_ws = reinterpret_cast<float*>(ws);
    ws += align256(sizeof(float) * bcd * a.N);
    p.start_ws = reinterpret_cast<float*>(ws);
    scan_kernel<IO, NP, false, false><<<dim3(gx, a.B, pl.chunks - 1), kThreads, 0, s>>>(p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(gx, a.B, pl.chunks);
  if (a.z)
    scan_kernel<IO, NP, true, true><<<grid, kThreads, 0, s>>>(p);
  else
    scan_kernel<IO, NP, true, false><<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_scan_io(const ScanFwdArgs& a, const ScanPlan& p, hipStream_t s) {
  switch (padded_n(a.N)) {
    case 16: return launch_scan_np<IO, 16>(a, p, s);
    case 32: return launch_scan_np<IO, 32>(a, p, s);
    default: return launch_scan_np<IO, 64>(a, p, s);
  }
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
