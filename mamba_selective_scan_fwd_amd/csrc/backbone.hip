// backbone.hip -- the layer pieces around the SSM core for the full Mamba-1 backbone prefill:
// embedding gather, RMSNorm, bf16 MFMA GEMMs for the projections, and the tied LM head.
//
// prefill.rs page (mamba-rs 0.6.4), prefill_body: per layer RMSNorm (F1), in_proj GEMM (F2),
// conv + x_proj (F4a/F4b), dt_proj (F4c), scan (F4d), out_proj (F5) and residual add (F6);
// then norm_f and the last-timestep gather; gpu_lm.rs page (mamba-rs 0.7.1) for the tied
// head (one GEMM against the embedding table, vocabulary padded to a multiple of 64) and the
// embedding lookup. inference.rs page (mamba-rs 0.5.1): bf16 weights with f32 compute and an
// f32 residual stream.
//
// Precision: GEMM operands are bf16 (weights stored bf16; activations rounded to bf16 as they
// enter the GEMM), products accumulate in f32, everything else is f32.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mamba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------- embedding

// out[r, :] = E[tokens[r], :] (bf16 -> f32). One block per row. Ids outside [0, vocab) are
// clamped into range, so a bad id can never address outside the table.
__global__ void __launch_bounds__(128) embed_gather_kernel(const int32_t* __restrict__ tokens,
                                                           const bf16* __restrict__ E,
                                                           float* __restrict__ out, int vocab,
                                                           int Dm) {
  const int64_t r = blockIdx.x;
  const int64_t tok = min(max(tokens[r], 0), vocab - 1);
  const bf16* src = E + tok * Dm;
  float* dst = out + r * Dm;
  for (int c = threadIdx.x; c < Dm; c += blockDim.x) dst[c] = to_f32(src[c]);
}

// ------------------------------------------------------------------------- RMSNorm

// out[r, :] = x[r, :] * rsqrt(mean(x[r, :]^2) + eps) * w. One 256-thread block per row; rows
// `x_row_stride` apart (the last-token gather is a row stride of T * Dm).
template <typename OT>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ x,
                                                      int64_t x_row_stride,
                                                      const float* __restrict__ w, float eps,
                                                      OT* __restrict__ out, int Dm) {
  __shared__ float part[8];
  const int64_t r = blockIdx.x;
  const float* xr = x + r * x_row_stride;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < Dm; c += 256) ss = fmaf(xr[c], xr[c], ss);
  for (int m = 32; m >= 1; m /= 2) ss += __shfl_xor(ss, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)Dm + eps);
  OT* o = out + r * Dm;
  for (int c = threadIdx.x; c < Dm; c += 256) o[c] = from_f32<OT>(xr[c] * inv * (w ? w[c] : 1.0f));
}

// ------------------------------------------------------------------------- GEMM (MFMA)
//
// C[M, N] (+)= A[M, K] * W[N, K]^T with A f32 or bf16 (rounded to bf16 when staged), W bf16
// (nn.Linear layout: one row of K per output column), C f32. Block tile BM x BN x 32, four
// waves in a 2 x 2 grid, each wave (BM/2) x (BN/2) as 16 x 16 tiles of
// v_mfma_f32_16x16x32_bf16. Operand fragments: lane l holds row (l % 16) and k = 8*(l/16)+0..7
// of A (of W for B); the result holds rows 4*(l/16)+0..3 of column l % 16.
// LDS rows are 40 bf16 (32 + 8 pad): the 16-byte fragment reads of each group of 8 lanes fall
// on disjoint banks. Double-buffered: the next k-slab is fetched to registers while the
// current one is multiplied.

constexpr int kBK = 32;
constexpr int kLdsK = kBK + 8;

template <typename AT, int BM, int BN>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(const AT* __restrict__ A, int64_t lda,
                                                        const bf16* __restrict__ W, int64_t ldw,
                                                        float* __restrict__ C, int64_t ldc,
                                                        int M, int N, int K, int accumulate) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int A_PER_T = BM * kBK / 256;  // elements of A each thread stages per slab
  constexpr int W_PER_T = BN * kBK / 256;
  static_assert(A_PER_T == 16 || A_PER_T == 8 || A_PER_T == 4, "A staging width");
  static_assert(W_PER_T == 16 || W_PER_T == 8 || W_PER_T == 4, "W staging width");
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * kLdsK];
  __shared__ __attribute__((aligned(16))) bf16 Ws[2][BN * kLdsK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  // staging coordinates: thread -> (row, k offset) of the slab
  constexpr int A_TPR = kBK / A_PER_T;  // threads per row
  constexpr int W_TPR = kBK / W_PER_T;
  const int a_row = tid / A_TPR, a_k = (tid % A_TPR) * A_PER_T;
  const int w_row = tid / W_TPR, w_k = (tid % W_TPR) * W_PER_T;

  float ra[A_PER_T], rw[W_PER_T];
  auto fetch = [&](int k0) {
    const int gm = m0 + a_row;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int gk = k0 + a_k + i;
      ra[i] = (gm < M && gk < K) ? to_f32(A[(int64_t)gm * lda + gk]) : 0.0f;
    }
    const int gn = n0 + w_row;
#pragma unroll
    for (int i = 0; i < W_PER_T; ++i) {
      const int gk = k0 + w_k + i;
      rw[i] = (gn < N && gk < K) ? to_f32(W[(int64_t)gn * ldw + gk]) : 0.0f;
    }
  };
  auto stash = [&](int buf) {
    bf16* a = &As[buf][a_row * kLdsK + a_k];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) a[i] = from_f32<bf16>(ra[i]);
    bf16* w = &Ws[buf][w_row * kLdsK + w_k];
#pragma unroll
    for (int i = 0; i < W_PER_T; ++i) w[i] = from_f32<bf16>(rw[i]);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = (K + kBK - 1) / kBK;
  fetch(0);
  stash(0);
  __syncthreads();
  const int frow = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * kBK);
    bf16x8 af[TM], bfr[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * WM + i * 16 + frow) * kLdsK + fk]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(&Ws[buf][(wn * WN + j * 16 + frow) * kLdsK + fk]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < nk) {
      stash(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+0..3 of column lane%16 of each 16x16 tile
  const int ccol = lane & 15, crow = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int gn = n0 + wn * WN + j * 16 + ccol;
      if (gn >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gm = m0 + wm * WM + i * 16 + crow + r;
        if (gm >= M) continue;
        float* cp = C + (int64_t)gm * ldc + gn;
        *cp = accumulate ? *cp + acc[i][j][r] : acc[i][j][r];
      }
    }
}

// Few-row GEMM (M <= 8, M * K staged floats within 64 KB of LDS): the tied LM head on the last
// token of each sequence, and every projection of a prefill of a handful of tokens. The kernel is
// bound by streaming W (the bf16 embedding table): each wave takes 8 columns; a lane covers
// 8 contiguous k of each column and the A rows sit in LDS (rounded to bf16).
constexpr int kSkinnyMaxM = kSkinnyGemmMaxM;

template <typename AT>
__global__ void __launch_bounds__(256) gemm_skinny_kernel(const AT* __restrict__ A, int64_t lda,
                                                          const bf16* __restrict__ W,
                                                          int64_t ldw, float* __restrict__ C,
                                                          int64_t ldc, int M, int N, int K,
                                                          int accumulate) {
  extern __shared__ float as[];  // M x K, bf16-rounded values held as f32
  for (int i = threadIdx.x; i < M * K; i += 256) {
    const int r = i / K, k = i % K;
    as[i] = to_f32(from_f32<bf16>(to_f32(A[(int64_t)r * lda + k])));
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_base = (blockIdx.x * 4 + wave) * 8;
  for (int cj = 0; cj < 8; ++cj) {
    const int n = n_base + cj;
    if (n >= N) break;
    const bf16* wr = W + (int64_t)n * ldw;
    float part[kSkinnyMaxM];
#pragma unroll
    for (int r = 0; r < kSkinnyMaxM; ++r) part[r] = 0.0f;
    for (int k = lane; k < K; k += 64) {
      const float wv = to_f32(wr[k]);
#pragma unroll
      for (int r = 0; r < kSkinnyMaxM; ++r)
        if (r < M) part[r] = fmaf(as[r * K + k], wv, part[r]);
    }
#pragma unroll
    for (int r = 0; r < kSkinnyMaxM; ++r) {
      if (r >= M) break;
      float v = part[r];
      for (int m = 32; m >= 1; m /= 2) v += __shfl_xor(v, m);
      if (lane == 0) {
        float* cp = C + (int64_t)r * ldc + n;
        *cp = accumulate ? *cp + v : v;
      }
    }
  }
}

// ------------------------------------------------------------------------- launchers

hipError_t launch_embed_gather(const int32_t* tokens, const void* E, float* out, int64_t rows,
                               int vocab, int Dm, hipStream_t s) {
  embed_gather_kernel<<<dim3((unsigned)rows), 128, 0, s>>>(tokens, static_cast<const bf16*>(E), out,
                                                           vocab, Dm);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, int64_t x_row_stride, const float* w, float eps,
                          void* out, bool out_bf16, int64_t rows, int Dm, hipStream_t s) {
  if (out_bf16)
    rmsnorm_kernel<bf16><<<dim3((unsigned)rows), 256, 0, s>>>(x, x_row_stride, w, eps,
                                                              static_cast<bf16*>(out), Dm);
  else
    rmsnorm_kernel<float><<<dim3((unsigned)rows), 256, 0, s>>>(x, x_row_stride, w, eps,
                                                               static_cast<float*>(out), Dm);
  return hipGetLastError();
}

template <typename AT, int BM, int BN>
static hipError_t gemm_tile(const AT* A, int64_t lda, const bf16* W, int64_t ldw, float* C,
                            int64_t ldc, int M, int N, int K, bool acc, hipStream_t s) {
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  gemm_bf16_kernel<AT, BM, BN><<<grid, 256, 0, s>>>(A, lda, W, ldw, C, ldc, M, N, K, acc ? 1 : 0);
  return hipGetLastError();
}

template <typename AT>
static hipError_t gemm_at(const AT* A, int64_t lda, const bf16* W, int64_t ldw, float* C,
                          int64_t ldc, int M, int N, int K, bool acc, hipStream_t s) {
  if (M <= kSkinnyMaxM && (int64_t)M * K * 4 <= kSkinnyGemmMaxLds) {
    const unsigned blocks = (unsigned)((N + 31) / 32);
    gemm_skinny_kernel<AT><<<blocks, 256, sizeof(float) * M * K, s>>>(A, lda, W, ldw, C, ldc, M, N, K,
                                                                     acc ? 1 : 0);
    return hipGetLastError();
  }
  // Wide outputs take 128 x 128 tiles; narrow ones (x_proj's 80 columns) 64 x 32 so that the
  // grid still covers the chip.
  if (N >= 256) return gemm_tile<AT, 128, 128>(A, lda, W, ldw, C, ldc, M, N, K, acc, s);
  return gemm_tile<AT, 64, 32>(A, lda, W, ldw, C, ldc, M, N, K, acc, s);
}

hipError_t launch_gemm_bf16(const void* A, bool a_bf16, int64_t lda, const void* W, int64_t ldw,
                            float* C, int64_t ldc, int M, int N, int K, bool accumulate,
                            hipStream_t s) {
  const bf16* w = static_cast<const bf16*>(W);
  if (a_bf16)
    return gemm_at<bf16>(static_cast<const bf16*>(A), lda, w, ldw, C, ldc, M, N, K, accumulate, s);
  return gemm_at<float>(static_cast<const float*>(A), lda, w, ldw, C, ldc, M, N, K, accumulate, s);
}

}  // namespace mamba
