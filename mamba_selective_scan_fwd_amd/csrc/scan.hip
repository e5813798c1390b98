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
// Tokens staged in registers ahead of use: u/dt/z of the next block are loaded while the
// current block is computed, so memory latency hides behind one block of work.
constexpr int kTB = 8;
// Third dword of a raw buffer resource on gfx9-family parts (32-bit data, no swizzle).
constexpr int kBufferFlags = 0x00020000;

using rsrc_t = __amdgpu_buffer_rsrc_t;

// The packed B/C rows are read-only for the whole call; reading them through the constant
// address space lets the compiler use scalar loads for these wave-uniform rows regardless of
// what the kernel stores elsewhere.
using cfloat = __attribute__((address_space(4))) const float;
__device__ __forceinline__ cfloat* as_constant(const float* p) {
  return (cfloat*)(p);
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kBufferFlags);
}

template <typename IO>
__device__ __forceinline__ float bload(rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(IO) == 4) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
  } else {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0) << 16);
  }
}

// A * log2(e) with A = -exp(A_log); states padded past N get 0 (decay 1; their B and C
// entries are packed as 0, so they stay 0 and add nothing).
template <int NP>
__device__ __forceinline__ void load_a2(float (&a2)[NP], const float* __restrict__ A_log, int d,
                                        int N) {
#pragma unroll
  for (int n = 0; n < NP; ++n)
    a2[n] = n < N ? -__builtin_amdgcn_exp2f(A_log[(int64_t)d * N + n] * kLog2e) * kLog2e : 0.0f;
}

__device__ __forceinline__ float make_delta(float dtv, float bias, bool sp) {
  const float v = dtv + bias;
  return sp ? softplus(v) : v;
}

// One block of kTB tokens of a [rows, row_stride] tensor for this lane's channel. The
// resource is rebased at the block so 32-bit offsets never overflow; tokens past t_end
// re-read the last valid row (never out of bounds; those values are not used).
template <typename IO>
struct BlockReader {
  const IO* base;       // element (row0 + t0, d0) -- the chunk's first row, wave's channel 0
  int64_t row_stride;   // elements
  uint32_t voff;        // this lane's byte offset in a row

  __device__ __forceinline__ void load(float (&dst)[kTB], int tb_rel, int n_valid) const {
    const IO* p = base + (int64_t)tb_rel * row_stride;
    const uint32_t rs_bytes = (uint32_t)(row_stride * sizeof(IO));
    const rsrc_t r = make_rsrc(p, (uint32_t)(kTB * rs_bytes));
#pragma unroll
    for (int j = 0; j < kTB; ++j) dst[j] = bload<IO>(r, voff, (uint32_t)min(j, n_valid - 1) * rs_bytes);
  }
};

// Pack B and C into f32 rows [B[0..NP), C[0..NP)] per token, zero padded past N, so the
// scan kernels read one contiguous row per token with scalar loads and no conversion.
template <typename IO, int NP>
__global__ void __launch_bounds__(256) pack_bc_kernel(const IO* __restrict__ Bm,
                                                      const IO* __restrict__ Cm,
                                                      int64_t bc_row_stride,
                                                      float* __restrict__ out, int64_t rows,
                                                      int N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * 2 * NP) return;
  const int64_t r = i / (2 * NP);
  const int k = (int)(i % (2 * NP));
  const int n = k < NP ? k : k - NP;
  const IO* src = k < NP ? Bm : Cm;
  out[i] = n < N ? to_f32(src[r * bc_row_stride + n]) : 0.0f;
}

// Chunk c of channel (b, d): the affine map h -> P*h + H it applies to the state, with
// P = exp(A * sum(delta)) and H the state it produces from h = 0. Chunks are disjoint runs of
// chunk_t tokens. Output layout [b][d][c][n] (n fastest), chunks 0 .. chunks-2.
template <typename IO, int NP>
__global__ void __launch_bounds__(kScanWave) scan_chunk_summary_kernel(
    const IO* __restrict__ u, const IO* __restrict__ dt, const float* __restrict__ dt_bias,
    int delta_softplus, const float* __restrict__ A_log, const float* __restrict__ bc,
    float* __restrict__ P_out, float* __restrict__ H_out, int B, int T, int D, int N,
    int chunk_t, int chunks) {
  const int d0 = blockIdx.x * kScanWave;
  const int d = d0 + threadIdx.x;
  const int b = blockIdx.y;
  const int c = blockIdx.z;
  if (d >= D) return;
  const int t0 = c * chunk_t;
  const int t1 = min(T, t0 + chunk_t);
  const int64_t row0 = (int64_t)b * T;

  float a2[NP];
  load_a2<NP>(a2, A_log, d, N);
  const float bias = dt_bias ? dt_bias[d] : 0.0f;
  const bool sp = delta_softplus != 0;

  float H[NP];
#pragma unroll
  for (int n = 0; n < NP; ++n) H[n] = 0.0f;
  float sum_delta = 0.0f;

  const int64_t first = (row0 + t0) * D + d0;
  const uint32_t voff = (uint32_t)(threadIdx.x * sizeof(IO));
  const BlockReader<IO> ru{u + first, D, voff};
  const BlockReader<IO> rdt{dt + first, D, voff};
  cfloat* bcp = as_constant(bc) + (row0 + t0) * (2 * NP);

  float cu[kTB], cdt[kTB], nu[kTB], ndt[kTB];
  ru.load(cu, 0, min(kTB, t1 - t0));
  rdt.load(cdt, 0, min(kTB, t1 - t0));
  float bv[NP];
#pragma unroll
  for (int n = 0; n < NP; ++n) bv[n] = bcp[n];
  for (int tb = t0; tb < t1; tb += kTB) {
    if (tb + kTB < t1) {
      ru.load(nu, tb + kTB - t0, min(kTB, t1 - tb - kTB));
      rdt.load(ndt, tb + kTB - t0, min(kTB, t1 - tb - kTB));
    }
#pragma unroll
    for (int j = 0; j < kTB; ++j) {
      const int t = tb + j;
      if (t >= t1) break;
      cfloat* bcn = t + 1 < t1 ? bcp + 2 * NP : bcp;
      float bn[NP];
#pragma unroll
      for (int n = 0; n < NP; ++n) bn[n] = bcn[n];
      const float delta = make_delta(cdt[j], bias, sp);
      const float du = delta * cu[j];
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        const float a = __builtin_amdgcn_exp2f(delta * a2[n]);
        H[n] = fmaf(a, H[n], du * bv[n]);
      }
      sum_delta += delta;
#pragma unroll
      for (int n = 0; n < NP; ++n) bv[n] = bn[n];
      bcp = bcn;
    }
#pragma unroll
    for (int j = 0; j < kTB; ++j) {
      cu[j] = nu[j];
      cdt[j] = ndt[j];
    }
  }

  const int64_t off = (((int64_t)b * D + d) * chunks + c) * N;
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    if (n < N) {
      P_out[off + n] = __builtin_amdgcn_exp2f(sum_delta * a2[n]);
      H_out[off + n] = H[n];
    }
  }
}

// Start state of every chunk: h_in[c] = map_{c-1}( ... map_0(state_in)). One thread per
// (b, d, n), layout [b][d][c][n]: the threads of a channel read contiguous bytes per chunk.
// Loads are issued kPrefixBatch chunks ahead of the dependent fma chain.
constexpr int kPrefixBatch = 8;

__global__ void __launch_bounds__(256) scan_chunk_prefix_kernel(
    const float* __restrict__ P, const float* __restrict__ H, const float* state_in,
    float* __restrict__ H_in, int64_t bdn, int N, int chunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b*D + d)*N + n
  if (i >= bdn) return;
  const int64_t ch = i / N;
  const int n = (int)(i % N);
  const int64_t base = ch * chunks * N + n;
  float h = state_in ? state_in[i] : 0.0f;
  H_in[base] = h;
  for (int c0 = 0; c0 + 1 < chunks; c0 += kPrefixBatch) {
    float p[kPrefixBatch], q[kPrefixBatch];
#pragma unroll
    for (int j = 0; j < kPrefixBatch; ++j) {
      const int c = min(c0 + j, chunks - 2);
      p[j] = P[base + (int64_t)c * N];
      q[j] = H[base + (int64_t)c * N];
    }
#pragma unroll
    for (int j = 0; j < kPrefixBatch; ++j) {
      if (c0 + j + 1 < chunks) {
        h = fmaf(p[j], h, q[j]);
        H_in[base + (int64_t)(c0 + j + 1) * N] = h;
      }
    }
  }
}

// Rescan each chunk from its start state, writing y for every token; the last chunk writes
// the final state. h_start: [b][d][c][n] start states (chunks > 1) or the carried state
// [b][d][n] (one chunk), or NULL for zeros.
template <typename IO, int NP, bool GATE>
__global__ void __launch_bounds__(kScanWave) scan_chunk_output_kernel(
    const IO* __restrict__ u, const IO* __restrict__ dt, const float* __restrict__ dt_bias,
    int delta_softplus, const float* __restrict__ A_log, const float* __restrict__ bc,
    const float* __restrict__ D_skip, const IO* __restrict__ z, int64_t z_row_stride,
    const float* h_start, float* state_out, IO* __restrict__ y, int B, int T, int D, int N,
    int chunk_t, int chunks) {
  const int d0 = blockIdx.x * kScanWave;
  const int d = d0 + threadIdx.x;
  const int b = blockIdx.y;
  const int c = blockIdx.z;
  if (d >= D) return;
  const int t0 = c * chunk_t;
  const int t1 = min(T, t0 + chunk_t);
  const int64_t row0 = (int64_t)b * T;

  float a2[NP];
  load_a2<NP>(a2, A_log, d, N);
  const float bias = dt_bias ? dt_bias[d] : 0.0f;
  const float dskip = D_skip ? D_skip[d] : 0.0f;
  const bool sp = delta_softplus != 0;

  float h[NP];
  const float* hs = h_start ? h_start + (((int64_t)b * D + d) * chunks + c) * N : nullptr;
#pragma unroll
  for (int n = 0; n < NP; ++n) h[n] = (hs && n < N) ? hs[n] : 0.0f;

  const int64_t first = (row0 + t0) * D + d0;
  const uint32_t voff = (uint32_t)(threadIdx.x * sizeof(IO));
  const BlockReader<IO> ru{u + first, D, voff};
  const BlockReader<IO> rdt{dt + first, D, voff};
  const BlockReader<IO> rz{GATE ? z + (row0 + t0) * z_row_stride + d0 : nullptr, z_row_stride, voff};
  cfloat* bcp = as_constant(bc) + (row0 + t0) * (2 * NP);
  // y goes through the restrict pointer (not a buffer store), so the compiler knows it does
  // not alias the packed B/C rows and keeps those as scalar loads.
  IO* yp = y + (row0 + t0) * D + d;

  float cu[kTB], cdt[kTB], cz[kTB], nu[kTB], ndt[kTB], nz[kTB];
  ru.load(cu, 0, min(kTB, t1 - t0));
  rdt.load(cdt, 0, min(kTB, t1 - t0));
  if constexpr (GATE) rz.load(cz, 0, min(kTB, t1 - t0));
  float bv[NP], cv[NP];
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    bv[n] = bcp[n];
    cv[n] = bcp[NP + n];
  }
  for (int tb = t0; tb < t1; tb += kTB) {
    if (tb + kTB < t1) {
      const int nv = min(kTB, t1 - tb - kTB);
      ru.load(nu, tb + kTB - t0, nv);
      rdt.load(ndt, tb + kTB - t0, nv);
      if constexpr (GATE) rz.load(nz, tb + kTB - t0, nv);
    }
#pragma unroll
    for (int j = 0; j < kTB; ++j) {
      const int t = tb + j;
      if (t >= t1) break;
      cfloat* bcn = t + 1 < t1 ? bcp + 2 * NP : bcp;
      float bn[NP], cn[NP];
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        bn[n] = bcn[n];
        cn[n] = bcn[NP + n];
      }
      const float uv = cu[j];
      const float delta = make_delta(cdt[j], bias, sp);
      const float du = delta * uv;
      float acc = 0.0f;
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        const float a = __builtin_amdgcn_exp2f(delta * a2[n]);
        h[n] = fmaf(a, h[n], du * bv[n]);
        acc = fmaf(cv[n], h[n], acc);
      }
      acc = fmaf(dskip, uv, acc);
      if constexpr (GATE) acc *= silu(cz[j]);
      *yp = from_f32<IO>(acc);
      yp += D;
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        bv[n] = bn[n];
        cv[n] = cn[n];
      }
      bcp = bcn;
    }
#pragma unroll
    for (int j = 0; j < kTB; ++j) {
      cu[j] = nu[j];
      cdt[j] = ndt[j];
      if constexpr (GATE) cz[j] = nz[j];
    }
  }

  if (c == chunks - 1 && state_out) {
    float* so = state_out + ((int64_t)b * D + d) * N;
#pragma unroll
    for (int n = 0; n < NP; ++n)
      if (n < N) so[n] = h[n];
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
#define MAMBA_SCAN_TARGET_WAVES 8192  // ~8 waves per SIMD (256 CUs x 4 SIMDs) to hide latency
#endif
#ifndef MAMBA_SCAN_MIN_CHUNK
#define MAMBA_SCAN_MIN_CHUNK 48  // tokens per chunk, at least (per-chunk setup stays small)
#endif

static int padded_n(int N) { return N <= 16 ? 16 : (N <= 32 ? 32 : 64); }

ScanPlan plan_selective_scan(int B, int T, int D, int N) {
  ScanPlan p{1, T, 0};
  if (B <= 0 || T <= 0 || D <= 0 || N <= 0) return p;
  const int64_t waves_per_chunk = (int64_t)B * ((D + kScanWave - 1) / kScanWave);
  const int64_t target_waves = MAMBA_SCAN_TARGET_WAVES;
  int64_t chunks = (target_waves + waves_per_chunk - 1) / waves_per_chunk;
  chunks = std::max<int64_t>(1, std::min<int64_t>(chunks, T / MAMBA_SCAN_MIN_CHUNK));
  const int chunk_t = (int)((T + chunks - 1) / chunks);
  p.chunks = (T + chunk_t - 1) / chunk_t;
  p.chunk_t = chunk_t;
  // [packed B|C rows: B*T*2*NP f32] then, with several chunks, P, H and start states.
  p.workspace_bytes = align256(sizeof(float) * (size_t)B * T * 2 * padded_n(N));
  if (p.chunks > 1) p.workspace_bytes += 3 * align256(sizeof(float) * (size_t)p.chunks * B * D * N);
  return p;
}

template <typename IO, int NP>
static hipError_t launch_scan_np(const ScanFwdArgs& a, const ScanPlan& p, hipStream_t s) {
  const dim3 blk(kScanWave);
  const int gx = (a.D + kScanWave - 1) / kScanWave;
  const IO* u = static_cast<const IO*>(a.u);
  const IO* dt = static_cast<const IO*>(a.dt);
  const IO* z = static_cast<const IO*>(a.z);
  IO* y = static_cast<IO*>(a.y);
  char* ws = static_cast<char*>(a.workspace);
  const int64_t rows = (int64_t)a.B * a.T;
  float* bc = reinterpret_cast<float*>(ws);
  ws += align256(sizeof(float) * (size_t)rows * 2 * NP);
  pack_bc_kernel<IO, NP><<<dim3((unsigned)((rows * 2 * NP + 255) / 256)), 256, 0, s>>>(
      static_cast<const IO*>(a.Bm), static_cast<const IO*>(a.Cm), a.bc_row_stride, bc, rows, a.N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float* h_start = a.state_in;
  if (p.chunks > 1) {
    const int64_t bdn = (int64_t)a.B * a.D * a.N;
    const size_t per = align256(sizeof(float) * (size_t)p.chunks * bdn);
    float* P = reinterpret_cast<float*>(ws);
    float* H = reinterpret_cast<float*>(ws + per);
    float* Hin = reinterpret_cast<float*>(ws + 2 * per);
    scan_chunk_summary_kernel<IO, NP><<<dim3(gx, a.B, p.chunks - 1), blk, 0, s>>>(
        u, dt, a.dt_bias, a.delta_softplus, a.A_log, bc, P, H, a.B, a.T, a.D, a.N, p.chunk_t,
        p.chunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    scan_chunk_prefix_kernel<<<dim3((unsigned)((bdn + 255) / 256)), 256, 0, s>>>(
        P, H, a.state_in, Hin, bdn, a.N, p.chunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    h_start = Hin;
  }
  if (z) {
    scan_chunk_output_kernel<IO, NP, true><<<dim3(gx, a.B, p.chunks), blk, 0, s>>>(
        u, dt, a.dt_bias, a.delta_softplus, a.A_log, bc, a.D_skip, z, a.z_row_stride, h_start,
        a.state_out, y, a.B, a.T, a.D, a.N, p.chunk_t, p.chunks);
  } else {
    scan_chunk_output_kernel<IO, NP, false><<<dim3(gx, a.B, p.chunks), blk, 0, s>>>(
        u, dt, a.dt_bias, a.delta_softplus, a.A_log, bc, a.D_skip, nullptr, 0, h_start,
        a.state_out, y, a.B, a.T, a.D, a.N, p.chunk_t, p.chunks);
  }
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
