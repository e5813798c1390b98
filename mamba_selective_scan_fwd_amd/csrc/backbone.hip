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
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mamba {

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

// The same per-row arithmetic with one wave per row, for many rows (a prefill's bt rows):
// lane l plays the four threads w * 64 + l of rmsnorm_kernel's block, keeping their running
// sums apart and reducing each over the wave in the same order, so the result is the same bit
// for bit; the row stays in registers, so it is read once. Rows up to kNormWaveMaxK * 256.
constexpr int kNormWaveMaxK = 8;
template <typename OT, int KMAX>
__global__ void __launch_bounds__(256) rmsnorm_rows_kernel(const float* __restrict__ x, int64_t x_row_stride,
                                                           const float* __restrict__ w, float eps,
                                                           OT* __restrict__ out, int64_t rows, int Dm) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // whole waves
  const float* xr = x + r * x_row_stride;
  float v[4][KMAX], wv[4][KMAX];
  float ss[4];
  // The row and the weights are all loaded before the first use, so the wave waits once; no
  // load carries a condition (columns past Dm re-read the last column, an absent weight
  // vector reads the row, and those values are replaced at the use), since a load under a
  // condition makes the wave wait for it right there.
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int c = min(q * 64 + lane + 256 * k, Dm - 1);
      v[q][k] = xr[c];
      wv[q][k] = *(w ? w + c : xr + c);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ss[q] = 0.0f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const bool in = q * 64 + lane + 256 * k < Dm;
      v[q][k] = in ? v[q][k] : 0.0f;
      wv[q][k] = w && in ? wv[q][k] : 1.0f;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (q * 64 + lane + 256 * k < Dm) ss[q] = fmaf(v[q][k], v[q][k], ss[q]);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    for (int m = 32; m >= 1; m /= 2) ss[q] += __shfl_xor(ss[q], m);
  const float tot = ss[0] + ss[1] + ss[2] + ss[3];
  const float inv = 1.0f / sqrtf(tot / (float)Dm + eps);
  OT* o = out + r * Dm;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int c = q * 64 + lane + 256 * k;
      if (c < Dm) o[c] = from_f32<OT>(v[q][k] * inv * wv[q][k]);
    }
}

// RMSNorm of each sequence's last valid position: row b * T + clamp(lengths[b], 1, T) - 1.
template <typename OT>
__global__ void __launch_bounds__(256) rmsnorm_last_kernel(const float* __restrict__ x,
                                                           const int32_t* __restrict__ lengths,
                                                           int T, const float* __restrict__ w,
                                                           float eps, OT* __restrict__ out,
                                                           int Dm) {
  __shared__ float part[4];
  const int b = blockIdx.x;
  const int t = min(max(lengths[b], 1), T) - 1;
  const float* xr = x + ((int64_t)b * T + t) * Dm;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < Dm; c += 256) ss = fmaf(xr[c], xr[c], ss);
  for (int m = 32; m >= 1; m /= 2) ss += __shfl_xor(ss, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)Dm + eps);
  OT* o = out + (int64_t)b * Dm;
  for (int c = threadIdx.x; c < Dm; c += 256) o[c] = from_f32<OT>(xr[c] * inv * (w ? w[c] : 1.0f));
}

// ------------------------------------------------------------------------- GEMM (MFMA)
//
// C[M, N] (+)= A[M, K] * W[N, K]^T with A f32 or bf16 (rounded to bf16 when staged), W bf16
// (nn.Linear layout: one row of K per output column), C f32.
//
// Block tile BM x BN x BK, WGM x WGN waves, each wave a (BM/WGM) x (BN/WGN) tile made of
// 16 x 16 tiles of v_mfma_f32_16x16x32_bf16. Operand fragments: lane l holds row (l % 16)
// and k = 8*(l/16)+0..7 of A (of W for B); the result holds rows 4*(l/16)+0..3 of column
// l % 16. Global loads move 8 consecutive k (16 bytes of bf16, 32 of f32) per thread and
// chunk, adjacent threads adjacent chunks of a row; staged tiles sit in LDS as bf16 rows of
// BK + 8 elements (the pad spreads the 16-byte fragment reads over the banks). LDS is double
// buffered: the next k-slab is loaded into registers while the current one is multiplied,
// and one barrier per slab orders the buffers. VEC = false is the element-wise path for
// unaligned or ragged operands.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16 bytes from global memory straight into LDS: lane l's bytes land at lds + 16 l (the LDS
// address is the wave's; gfx950 global_load_lds_dwordx4). The builtin exists only for the
// device target, so the host pass of a kernel that calls it sees an empty body.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
#else
  (void)g;
  (void)lds;
#endif
}

template <typename AT>
struct Chunk;  // 8 consecutive elements of a row, as loaded
template <>
struct Chunk<bf16> {
  uint4 v;
};
template <>
struct Chunk<float> {
  float4 lo, hi;
};

template <typename AT>
__device__ __forceinline__ void load_chunk(Chunk<AT>& c, const AT* p);
template <>
__device__ __forceinline__ void load_chunk<bf16>(Chunk<bf16>& c, const bf16* p) {
  c.v = *reinterpret_cast<const uint4*>(p);
}
template <>
__device__ __forceinline__ void load_chunk<float>(Chunk<float>& c, const float* p) {
  c.lo = *reinterpret_cast<const float4*>(p);
  c.hi = *reinterpret_cast<const float4*>(p + 4);
}
template <typename AT>
__device__ __forceinline__ void zero_chunk(Chunk<AT>& c);
template <>
__device__ __forceinline__ void zero_chunk<bf16>(Chunk<bf16>& c) {
  c.v = make_uint4(0, 0, 0, 0);
}
template <>
__device__ __forceinline__ void zero_chunk<float>(Chunk<float>& c) {
  c.lo = c.hi = make_float4(0.f, 0.f, 0.f, 0.f);
}
// 8 elements as bf16 (RNE for f32)
__device__ __forceinline__ bf16x8 to_bf16x8(const Chunk<bf16>& c) {
  return __builtin_bit_cast(bf16x8, c.v);
}
__device__ __forceinline__ bf16x8 to_bf16x8(const Chunk<float>& c) {
  bf16x8 r;
  r[0] = (bf16)c.lo.x; r[1] = (bf16)c.lo.y; r[2] = (bf16)c.lo.z; r[3] = (bf16)c.lo.w;
  r[4] = (bf16)c.hi.x; r[5] = (bf16)c.hi.y; r[6] = (bf16)c.hi.z; r[7] = (bf16)c.hi.w;
  return r;
}
// element-wise chunk load with bounds (ragged K, unaligned rows)
template <typename AT>
__device__ __forceinline__ bf16x8 load_chunk_scalar(const AT* row, int k0, int K) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = k0 + i < K ? (bf16)to_f32(row[k0 + i]) : (bf16)0.0f;
  return r;
}

#ifndef MAMBA_GEMM_WPE
#define MAMBA_GEMM_WPE 2  // waves per SIMD the register allocation must allow
#endif
// large bf16-A products stage their slabs straight into LDS (1) or through registers (0)
#ifndef MAMBA_GEMM_DL
#define MAMBA_GEMM_DL 1
#endif
// 32 x 32 MFMA tiles where the wave tile allows (1) or 16 x 16 everywhere (0)
#ifndef MAMBA_GEMM_MFMA32
#define MAMBA_GEMM_MFMA32 1
#endif
// XOR-swizzled LDS rows for the staged tiles (1) or rows padded by 8 elements (0)
#ifndef MAMBA_GEMM_SWZ
#define MAMBA_GEMM_SWZ 1
#endif
// register sets of staged chunks: 2 (slab kt+2 loads while kt multiplies) or 1 (kt+1)
#ifndef MAMBA_GEMM_SETS
#define MAMBA_GEMM_SETS 2
#endif
// the large-output tile: BM x BN x BK as WGM x WGN waves
#ifndef MAMBA_GEMM_BM
#define MAMBA_GEMM_BM 128
#endif
#ifndef MAMBA_GEMM_BN
#define MAMBA_GEMM_BN 128
#endif
#ifndef MAMBA_GEMM_BK
#define MAMBA_GEMM_BK 64
#endif
#ifndef MAMBA_GEMM_WGM
#define MAMBA_GEMM_WGM 2
#endif
#ifndef MAMBA_GEMM_WGN
#define MAMBA_GEMM_WGN 2
#endif
#ifndef MAMBA_GEMM_CPRE
#define MAMBA_GEMM_CPRE 1  // load the old C tile of an accumulating product before the k loop
#endif
#ifndef MAMBA_GEMM_LDS_EPI
#define MAMBA_GEMM_LDS_EPI 1  // write C through LDS as rows of float4 (1) or from the fragments (0)
#endif

// XCD-aware tile order: the (column tile, row tile) this workgroup takes. See gemm_mfma_kernel.
__device__ __forceinline__ void xcd_tile_order(int& bx, int& by) {
  const int gx = gridDim.x, gy = gridDim.y, G = gx * gy;
  const int L = blockIdx.x + gx * blockIdx.y;
  const int xcd = L % 8, idx = L / 8, base = G / 8, rem = G % 8;
  const int t = xcd * base + min(xcd, rem) + idx;  // a bijection of [0, G)
  constexpr int kGroupN = 8;
  const int full = (gx / kGroupN) * kGroupN * gy;  // tiles in whole groups
  if (t < full) {
    const int g = t / (kGroupN * gy), r = t % (kGroupN * gy);
    by = r / kGroupN;
    bx = g * kGroupN + r % kGroupN;
  } else {
    const int w = gx % kGroupN, r = t - full;  // the last, narrower group
    by = r / w;
    bx = gx - w + r % w;
  }
}

template <typename AT, int BM, int BN, int BK, int WGM, int WGN, bool VEC, bool DL>
__global__ void __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(MAMBA_GEMM_WPE)))
gemm_mfma_kernel(
    const AT* __restrict__ A, int64_t lda, const bf16* __restrict__ W, int64_t ldw,
    float* __restrict__ C, int64_t ldc, int M, int N, int K, int accumulate, int k_chunk,
    int64_t c_split_stride) {
  // XCD-aware tile order. Workgroups are handed to the 8 XCDs (each with its own L2) in
  // round-robin order of their linear id, so neighbouring ids land on different L2s. Here
  // each XCD takes one contiguous run of tiles instead, and the runs follow a grouped
  // order: the column tiles are cut into groups of up to 8, and within a group the tiles go
  // row block by row block (n fastest). The tiles one XCD has in flight then cover a few row
  // blocks of A and at most 8 column blocks of W, which fit its L2 together; with plain
  // row-major order they would span every column block, and W (4.7 MB for in_proj) would be
  // fetched again for each row block.
  // (Split-K launches keep the plain order: their slices share no operand rows.)
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if (gridDim.z == 1) xcd_tile_order(bx, by);
  // split K (gridDim.z > 1): slice z covers k in [z * k_chunk, z * k_chunk + k_chunk) and
  // writes its partial product to its own C plane (C + z * c_split_stride)
  {
    const int k0 = bz * k_chunk;
    A += k0;
    W += k0;
    K = min(K - k0, k_chunk);
    C += bz * c_split_stride;
  }
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  // MFMA tile: 32 x 32 (v_mfma_f32_32x32x16_bf16, 16 k per step) when the wave tile is made
  // of whole 32 x 32 tiles, else 16 x 16 (v_mfma_f32_16x16x32_bf16, 32 k per step)
  constexpr int MT = MAMBA_GEMM_MFMA32 && WTM % 32 == 0 && WTN % 32 == 0 ? 32 : 16;
  constexpr int KSTEP = MT == 32 ? 16 : 32;
  constexpr int TM = WTM / MT, TN = WTN / MT;
  // LDS row layout of the staged tiles. With kSwz, rows are BK elements (no pad) and the
  // 16-byte chunk kc of row r sits at chunk kc ^ swz(r), swz(r) = (r ^ r >> 3) & 7: the 16
  // rows a fragment read touches (and each pair of rows a 16-lane group writes) then fall on
  // distinct bank groups for 32 or 64 four-byte banks. Without it, rows are padded by 8.
  constexpr bool kSwz = (MAMBA_GEMM_SWZ != 0 || DL) && BK == 64;
  static_assert(!DL || (VEC && BK == 64 && std::is_same_v<AT, bf16>), "direct LDS staging: bf16 A, 64-k slabs");
  constexpr int LDK = kSwz ? BK : BK + 8;
  auto swz = [](int r) { return kSwz ? (r ^ (r >> 3)) & 7 : 0; };
  constexpr int CPR = BK / 8;  // chunks per row
  constexpr int A_CH = BM * CPR / NT, W_CH = BN * CPR / NT;
  static_assert(TM * MT == WTM && TN * MT == WTN && BK % 32 == 0, "tile shape");
  static_assert(A_CH * NT == BM * CPR && W_CH * NT == BN * CPR, "staging split");
  static_assert(A_CH <= 32 && W_CH <= 32, "chunk masks");
  // staging buffers for A and W; after the last k-slab the same LDS holds the C tile
  constexpr int LDC = BN + 4;  // (4 rows apart = 16 banks: the fragment writes do not collide)
  constexpr int kStageBytes = 2 * (BM + BN) * LDK * (int)sizeof(bf16);
  // the C tile leaves through LDS in kParts passes of BM / kParts rows (one wave row per
  // pass when the whole tile would need more LDS than the staging buffers)
  constexpr int kParts = BM * LDC * (int)sizeof(float) > kStageBytes ? WGM : 1;
  constexpr int kCBytes = MAMBA_GEMM_LDS_EPI ? BM / kParts * LDC * (int)sizeof(float) : 0;
  __shared__ __attribute__((aligned(16))) char smem[kStageBytes > kCBytes ? kStageBytes : kCBytes];
  auto As = reinterpret_cast<bf16(*)[BM * LDK]>(smem);
  auto Ws = reinterpret_cast<bf16(*)[BN * LDK]>(smem + 2 * BM * LDK * sizeof(bf16));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int m0 = by * BM, n0 = bx * BN;

  // Register sets of staged chunks. With two, the loads of slab kt+2 are issued while slab
  // kt is multiplied and slab kt+1 (loaded one iteration earlier) is written to LDS, so a
  // load has a whole iteration to arrive. On the 16-byte path every chunk load is issued
  // unconditionally (a chunk outside the operands reads an in-bounds address and is zeroed
  // when written to LDS), and chunks stay as loaded (f32 A is rounded to bf16 only then):
  // a load under a branch, or a use right after it, would make the wave wait for every load
  // in flight, the prefetch included. A tile entirely inside the operands skips the checks.
  constexpr int NSET = MAMBA_GEMM_SETS;
  using ARaw = std::conditional_t<VEC, Chunk<AT>, bf16x8>;
  using WRaw = std::conditional_t<VEC, Chunk<bf16>, bf16x8>;
  ARaw ra[NSET][A_CH];
  WRaw rw[NSET][W_CH];
  uint32_t va[NSET] = {}, vw[NSET] = {};  // 16-byte path: bit i set when chunk i is inside
  const bool full = VEC && m0 + BM <= M && n0 + BN <= N && K % BK == 0;
  auto fetch = [&](int k0, auto SET) {
    constexpr int st = decltype(SET)::value;
    if constexpr (VEC) {
      va[st] = 0;
      vw[st] = 0;
    }
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT, r = c / CPR, kc = (c % CPR) * 8;
      const int gm = m0 + r, gk = k0 + kc;
      if constexpr (VEC) {
        const bool ok = full || (gm < M && gk < K);
        load_chunk<AT>(ra[st][i], A + (int64_t)min(gm, M - 1) * lda + (ok ? gk : 0));
        va[st] |= (uint32_t)ok << i;
      } else {
        ra[st][i] = gm < M ? load_chunk_scalar(A + (int64_t)gm * lda, gk, K) : bf16x8{};
      }
    }
#pragma unroll
    for (int i = 0; i < W_CH; ++i) {
      const int c = tid + i * NT, r = c / CPR, kc = (c % CPR) * 8;
      const int gn = n0 + r, gk = k0 + kc;
      if constexpr (VEC) {
        const bool ok = full || (gn < N && gk < K);
        load_chunk<bf16>(rw[st][i], W + (int64_t)min(gn, N - 1) * ldw + (ok ? gk : 0));
        vw[st] |= (uint32_t)ok << i;
      } else {
        rw[st][i] = gn < N ? load_chunk_scalar(W + (int64_t)gn * ldw, gk, K) : bf16x8{};
      }
    }
  };
  auto stash = [&](int buf, auto SET) {
    constexpr int st = decltype(SET)::value;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT;
      const int r = c / CPR;
      bf16x8 v;
      if constexpr (VEC) {
        v = to_bf16x8(ra[st][i]);
        if (!((va[st] >> i) & 1u)) v = bf16x8{};
      } else {
        v = ra[st][i];
      }
      *reinterpret_cast<bf16x8*>(&As[buf][r * LDK + ((c % CPR) ^ swz(r)) * 8]) = v;
    }
#pragma unroll
    for (int i = 0; i < W_CH; ++i) {
      const int c = tid + i * NT;
      const int r = c / CPR;
      bf16x8 v;
      if constexpr (VEC) {
        v = to_bf16x8(rw[st][i]);
        if (!((vw[st] >> i) & 1u)) v = bf16x8{};
      } else {
        v = rw[st][i];
      }
      *reinterpret_cast<bf16x8*>(&Ws[buf][r * LDK + ((c % CPR) ^ swz(r)) * 8]) = v;
    }
  };

  typedef float f32x16 __attribute__((ext_vector_type(16)));
  using AccT = std::conditional_t<MT == 32, f32x16, f32x4>;
  constexpr int NR = MT == 32 ? 16 : 4;  // accumulator registers per lane and tile
  AccT acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.0f;

  // Adding into C (out_proj's residual add) reads the old C tile in the epilogue. When the
  // tile leaves in one pass and a thread's share is at most 12 float4, those reads are
  // issued here, before the first k-slab, in the epilogue's own element order (rows and
  // columns clamped into C; the values of clamped slots are never stored), so that their
  // latency is spent under the k loop instead of after it.
  constexpr int V4 = BN / 4;  // float4 per tile row
  constexpr int kPre = MAMBA_GEMM_CPRE && MAMBA_GEMM_LDS_EPI && kParts == 1 && (BM * V4) % NT == 0 &&
                               BM * V4 / NT <= 12 ? BM * V4 / NT : 0;
  float4 cpre[kPre > 0 ? kPre : 1];
  const bool pre = kPre > 0 && accumulate && N % 4 == 0 && ldc % 4 == 0 &&
                   reinterpret_cast<uintptr_t>(C) % 16 == 0;
  if (pre) {
#pragma unroll
    for (int q = 0; q < kPre; ++q) {
      const int idx = tid + q * NT, r = idx / V4, c4 = (idx % V4) * 4;
      cpre[q] = *reinterpret_cast<const float4*>(C + (int64_t)min(m0 + r, M - 1) * ldc + min(n0 + c4, N - 4));
    }
  }

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int nk = (K + BK - 1) / BK;
  // fragment of lane l: row l % MT of the tile, 8 consecutive k at 8 * (l / MT)
  const int frow = lane & (MT - 1), fk = (lane / MT) * 8;
  auto multiply = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += KSTEP) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WTM + i * MT + frow;
        af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][r * LDK + (((kk + fk) >> 3) ^ swz(r)) * 8]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WTN + j * MT + frow;
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Ws[buf][r * LDK + (((kk + fk) >> 3) ^ swz(r)) * 8]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          if constexpr (MT == 32)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };
  // iteration kt: loads of slab kt+2 into set kt & 1, multiply LDS buffer kt & 1, write slab
  // kt+1 (set (kt+1) & 1) into LDS buffer (kt+1) & 1, barrier
  auto step = [&](int kt, auto SET) {
    constexpr int st = decltype(SET)::value;  // == kt & 1
    if constexpr (NSET == 2) {
      if (kt + 2 < nk) fetch((kt + 2) * BK, SET);
      multiply(st);
      if (kt + 1 < nk) stash(st ^ 1, std::integral_constant<int, st ^ 1>{});
    } else {
      // one register set: slab kt+1 is loaded while slab kt is multiplied
      if (kt + 1 < nk) fetch((kt + 1) * BK, S0{});
      multiply(st);
      if (kt + 1 < nk) stash(st ^ 1, S0{});
    }
    __syncthreads();
  };
  if constexpr (!DL) {
    fetch(0, S0{});
    if constexpr (NSET == 2) {
      if (nk > 1) fetch(BK, S1{});
    }
    stash(0, S0{});
    __syncthreads();
  }
  if constexpr (DL) {
    // Direct staging: each wave moves 1 KB pieces of the next slab from global memory
    // straight into LDS (global_load_lds_dwordx4: lane l's 16 bytes land at the piece's
    // base + 16 l), so no register staging and no LDS store instruction is spent on them.
    // The LDS slot order is the swizzled layout, so lane l of piece i loads the chunk that
    // belongs in slot 64 i + l. Rows past M (N) read the last row; their products are never
    // stored. K is a whole number of slabs on this path.
    constexpr int NW = WGM * WGN;
    constexpr int PA = BM / 8 / NW, PW = BN / 8 / NW;  // 1 KB pieces per wave and tile
    static_assert(PA * NW * 8 == BM && PW * NW * 8 == BN, "piece split");
    auto issue = [&](int k0, int buf) {
#pragma unroll
      for (int j = 0; j < PA; ++j) {
        const int i = wave * PA + j, sl = i * 64 + lane, r = sl >> 3, kc = (sl & 7) ^ swz(r);
        load_lds16(A + (int64_t)min(m0 + r, M - 1) * lda + k0 + 8 * kc, &As[buf][i * 512]);
      }
#pragma unroll
      for (int j = 0; j < PW; ++j) {
        const int i = wave * PW + j, sl = i * 64 + lane, r = sl >> 3, kc = (sl & 7) ^ swz(r);
        load_lds16(W + (int64_t)min(n0 + r, N - 1) * ldw + k0 + 8 * kc, &Ws[buf][i * 512]);
      }
    };
    // the slab's pieces have landed (vector memory counter at zero), then every wave may read
    auto landed = [&]() {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
    };
    issue(0, 0);
    landed();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) issue((kt + 1) * BK, (kt + 1) & 1);
      multiply(kt & 1);
      landed();
    }
  } else {
  // Steady state first: while both slabs of an iteration pair still load a later slab, the
  // fetches carry no condition, so the load counter is known at every point of the loop and
  // each stash waits only for its own slab, not for the prefetch behind it.
  int kt0 = 0;
  if constexpr (NSET == 2) {
    for (; kt0 + 3 < nk; kt0 += 2) {
      fetch((kt0 + 2) * BK, S0{});
      multiply(0);
      stash(1, S1{});
      __syncthreads();
      fetch((kt0 + 3) * BK, S1{});
      multiply(1);
      stash(0, S0{});
      __syncthreads();
    }
  }
  for (int kt = kt0; kt < nk; kt += 2) {
    step(kt, S0{});
    if (kt + 1 < nk) step(kt + 1, S1{});
  }
  }

  // epilogue. Accumulator register r of lane l holds, in a 16 x 16 tile, row 4*(l/16) + r of
  // column l % 16; in a 32 x 32 tile, row 8*(r/4) + 4*(l/32) + r%4 of column l % 32.
  const int ccol = lane & (MT - 1), crow = (lane / MT) * 4;
  auto acc_row = [&](int r) { return MT == 32 ? 8 * (r >> 2) + crow + (r & 3) : crow + r; };
  // A product that adds into C (out_proj's residual) goes through LDS: the tile is read and
  // written back as whole rows. A plain store goes out straight from the fragments (4-byte
  // stores, whole 64- or 128-byte row pieces per instruction), which measured faster for
  // in_proj and dt_proj and slower when C is read first.
  if (MAMBA_GEMM_LDS_EPI != 0 && accumulate) {
    // The tile goes to LDS in that layout (the last k-slab's barrier has freed the staging
    // buffers), then back out as rows: each lane stores 16 contiguous bytes, a wave whole
    // rows, instead of 4-byte stores that cover 64-byte pieces of 4 rows.
    float* Cs = reinterpret_cast<float*>(smem);
    constexpr int PR = BM / kParts;  // tile rows per pass
    for (int part = 0; part < kParts; ++part) {
    if (part > 0) __syncthreads();  // the previous pass's rows have been read
    if (kParts == 1 || wm == part) {
      const int rbase = kParts == 1 ? wm * WTM : 0;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < NR; ++r)
            Cs[(rbase + i * MT + acc_row(r)) * LDC + wn * WTN + j * MT + ccol] = acc[i][j][r];
    }
    __syncthreads();
    constexpr int V = BN / 4;  // float4 per tile row
    if (pre) {
#pragma unroll
      for (int q = 0; q < kPre; ++q) {
        const int idx = tid + q * NT, r = idx / V, c4 = (idx % V) * 4;
        const int gm = m0 + r, gn = n0 + c4;
        const float4 v = *reinterpret_cast<const float4*>(&Cs[r * LDC + c4]);
        if (gm < M && gn < N)
          *reinterpret_cast<float4*>(C + (int64_t)gm * ldc + gn) =
              make_float4(v.x + cpre[q].x, v.y + cpre[q].y, v.z + cpre[q].z, v.w + cpre[q].w);
      }
      return;
    }
    const bool c_vec = ldc % 4 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0;
#pragma unroll 4
    for (int idx = tid; idx < PR * V; idx += NT) {
      const int r = idx / V, c4 = (idx % V) * 4;
      const int gm = m0 + part * PR + r, gn = n0 + c4;
      if (gm >= M) continue;
      const float4 v = *reinterpret_cast<const float4*>(&Cs[r * LDC + c4]);
      float* cp = C + (int64_t)gm * ldc + gn;
      if (c_vec && gn + 4 <= N) {
        float4 o = v;
        if (accumulate) {
          const float4 old = *reinterpret_cast<const float4*>(cp);
          o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
        }
        *reinterpret_cast<float4*>(cp) = o;
      } else {
        const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (gn + q < N) cp[q] = accumulate ? cp[q] + e[q] : e[q];
      }
    }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int gn = n0 + wn * WTN + j * MT + ccol;
      if (gn >= N) continue;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int gm = m0 + wm * WTM + i * MT + acc_row(r);
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

// The same product with 16-byte weight loads (ldw and K multiples of 8, W 16-byte aligned):
// a wave takes 8 columns, and lane l handles column l / 8 and the k-chunks (8 consecutive
// k) l % 8, l % 8 + 8, ... of it, so each load instruction reads 128 contiguous bytes of 8
// weight rows. The 8 lanes of a column add their partial sums with three xor-shuffles.
template <typename AT>
__global__ void __launch_bounds__(256) gemm_skinny_vec_kernel(const AT* __restrict__ A, int64_t lda,
                                                              const bf16* __restrict__ W,
                                                              int64_t ldw, float* __restrict__ C,
                                                              int64_t ldc, int M, int N, int K,
                                                              int accumulate) {
  extern __shared__ float as[];  // M x K, bf16-rounded values held as f32
  for (int r = 0; r < M; ++r)
    for (int k = threadIdx.x; k < K; k += 256)
      as[r * K + k] = to_f32(from_f32<bf16>(to_f32(A[(int64_t)r * lda + k])));
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = (blockIdx.x * 4 + wave) * 8 + (lane >> 3);
  const int kq = lane & 7;
  float part[kSkinnyMaxM];
#pragma unroll
  for (int r = 0; r < kSkinnyMaxM; ++r) part[r] = 0.0f;
  if (n < N) {
    const bf16* wr = W + (int64_t)n * ldw;
#pragma unroll 4
    for (int k0 = kq * 8; k0 < K; k0 += 64) {
      const bf16x8 w8 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(wr + k0));
      float wf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) wf[i] = to_f32(w8[i]);
#pragma unroll
      for (int r = 0; r < kSkinnyMaxM; ++r) {
        if (r < M) {
          const float4 a0 = *reinterpret_cast<const float4*>(&as[r * K + k0]);
          const float4 a1 = *reinterpret_cast<const float4*>(&as[r * K + k0 + 4]);
          float v = part[r];
          v = fmaf(a0.x, wf[0], v); v = fmaf(a0.y, wf[1], v);
          v = fmaf(a0.z, wf[2], v); v = fmaf(a0.w, wf[3], v);
          v = fmaf(a1.x, wf[4], v); v = fmaf(a1.y, wf[5], v);
          v = fmaf(a1.z, wf[6], v); v = fmaf(a1.w, wf[7], v);
          part[r] = v;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kSkinnyMaxM; ++r) {
    if (r >= M) break;
    float v = part[r];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    if (kq == 0 && n < N) {
      float* cp = C + (int64_t)r * ldc + n;
      *cp = accumulate ? *cp + v : v;
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
  // many rows of at most 3 * 256 (or 8 * 256) elements: one wave per row
  if (rows >= 1024 && Dm <= kNormWaveMaxK * 256) {
    const dim3 grid((unsigned)((rows + 3) / 4));
#define MAMBA_NORM_ROWS(KM)                                                                             \
  if (out_bf16)                                                                                         \
    rmsnorm_rows_kernel<bf16, KM><<<grid, 256, 0, s>>>(x, x_row_stride, w, eps, static_cast<bf16*>(out), \
                                                       rows, Dm);                                       \
  else                                                                                                  \
    rmsnorm_rows_kernel<float, KM><<<grid, 256, 0, s>>>(x, x_row_stride, w, eps, static_cast<float*>(out), \
                                                        rows, Dm)
    if (Dm <= 3 * 256) {
      MAMBA_NORM_ROWS(3);
    } else {
      MAMBA_NORM_ROWS(kNormWaveMaxK);
    }
#undef MAMBA_NORM_ROWS
    return hipGetLastError();
  }
  if (out_bf16)
    rmsnorm_kernel<bf16><<<dim3((unsigned)rows), 256, 0, s>>>(x, x_row_stride, w, eps,
                                                              static_cast<bf16*>(out), Dm);
  else
    rmsnorm_kernel<float><<<dim3((unsigned)rows), 256, 0, s>>>(x, x_row_stride, w, eps,
                                                               static_cast<float*>(out), Dm);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_last(const float* x, const int32_t* lengths, int T, const float* w,
                               float eps, void* out, bool out_bf16, int B, int Dm, hipStream_t s) {
  if (out_bf16)
    rmsnorm_last_kernel<bf16><<<dim3((unsigned)B), 256, 0, s>>>(x, lengths, T, w, eps,
                                                                static_cast<bf16*>(out), Dm);
  else
    rmsnorm_last_kernel<float><<<dim3((unsigned)B), 256, 0, s>>>(x, lengths, T, w, eps,
                                                                 static_cast<float*>(out), Dm);
  return hipGetLastError();
}

template <typename AT, int BM, int BN, int BK, int WGM, int WGN>
static hipError_t gemm_tile(const AT* A, int64_t lda, const bf16* W, int64_t ldw, float* C,
                            int64_t ldc, int M, int N, int K, bool acc, bool vec, hipStream_t s,
                            int ks = 1, int k_chunk = 0, int64_t c_split_stride = 0, bool dl = false) {
  if (ks <= 1) k_chunk = K;
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM), (unsigned)ks);
  if constexpr (std::is_same_v<AT, bf16> && BK == 64) {
    if (dl && vec && ks <= 1 && K % BK == 0) {
      gemm_mfma_kernel<AT, BM, BN, BK, WGM, WGN, true, true><<<grid, 64 * WGM * WGN, 0, s>>>(
          A, lda, W, ldw, C, ldc, M, N, K, acc ? 1 : 0, k_chunk, c_split_stride);
      return hipGetLastError();
    }
  }
  if (vec)
    gemm_mfma_kernel<AT, BM, BN, BK, WGM, WGN, true, false><<<grid, 64 * WGM * WGN, 0, s>>>(
        A, lda, W, ldw, C, ldc, M, N, K, acc ? 1 : 0, k_chunk, c_split_stride);
  else
    gemm_mfma_kernel<AT, BM, BN, BK, WGM, WGN, false, false><<<grid, 64 * WGM * WGN, 0, s>>>(
        A, lda, W, ldw, C, ldc, M, N, K, acc ? 1 : 0, k_chunk, c_split_stride);
  return hipGetLastError();
}

template <typename AT>
static hipError_t gemm_at(const AT* A, int64_t lda, const bf16* W, int64_t ldw, float* C,
                          int64_t ldc, int M, int N, int K, bool acc, hipStream_t s) {
  if (M <= kSkinnyMaxM && (int64_t)M * K * 4 <= kSkinnyGemmMaxLds) {
    const unsigned blocks = (unsigned)((N + 31) / 32);
    if (K % 8 == 0 && ldw % 8 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0)
      gemm_skinny_vec_kernel<AT><<<blocks, 256, sizeof(float) * M * K, s>>>(A, lda, W, ldw, C, ldc, M, N,
                                                                             K, acc ? 1 : 0);
    else
      gemm_skinny_kernel<AT><<<blocks, 256, sizeof(float) * M * K, s>>>(A, lda, W, ldw, C, ldc, M, N, K,
                                                                     acc ? 1 : 0);
    return hipGetLastError();
  }
  // 16-byte chunk loads need every row start and the K extent on 8-element boundaries
  // (and K >= 8: on that path a chunk outside the operands still reads 16 in-bounds bytes)
  const bool vec = K >= 8 && K % 8 == 0 && lda % 8 == 0 && ldw % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(A) % 16 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0;
  // Wide outputs: 128 x 128 tiles, 2 x 2 waves. Narrow ones (x_proj's 80 columns): 32 x 80
  // tiles, one column tile, so that the grid still covers the chip. Few rows (a decode step's
  // batch): 64 x 32 tiles, so that streaming the weights is spread over more workgroups.
  if (N < 128) return gemm_tile<AT, 32, 80, 64, 2, 1>(A, lda, W, ldw, C, ldc, M, N, K, acc, vec, s);
  // (very wide outputs with few rows, the tied head of a decode batch: 64 x 64 tiles, which
  // read the weights once per 64 columns with four waves)
  if (M <= 64 && N >= 8192)
    return gemm_tile<AT, 64, 64, 64, 2, 2>(A, lda, W, ldw, C, ldc, M, N, K, acc, vec, s);
  if (M <= 64) return gemm_tile<AT, 64, 32, 64, 2, 1>(A, lda, W, ldw, C, ldc, M, N, K, acc, vec, s);
  // Many rows, at most 1024 columns (out_proj at a prefill's row count): 128 x 128 tiles
  // would give M/128 x N/128 workgroups, 1.5 per CU for the 130m out_proj at 8192 rows;
  // 128 x 96 tiles (4 x 1 waves of 32 x 96, 32 x 32 MFMA) give 2 per CU, and their C tile is
  // small enough for the early read of the old C when the product adds into it. At the
  // 130m prefill: 37 us in the layer chain against 44 us for 128 x 128.
  if (N <= 1024 && M >= 4096)
    return gemm_tile<AT, 128, 96, 64, 4, 1>(A, lda, W, ldw, C, ldc, M, N, K, acc, vec, s, 1, 0, 0,
                                            MAMBA_GEMM_DL != 0);
  // (bf16 A with whole 64-k slabs stages straight into LDS)
  return gemm_tile<AT, MAMBA_GEMM_BM, MAMBA_GEMM_BN, MAMBA_GEMM_BK, MAMBA_GEMM_WGM, MAMBA_GEMM_WGN>(
      A, lda, W, ldw, C, ldc, M, N, K, acc, vec, s, 1, 0, 0, MAMBA_GEMM_DL != 0);
}

// C[m, n] (+)= sum over the ks partial planes P[z, m, n] in order z = 0 .. ks-1.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ P, int ks,
                                                            float* __restrict__ C, int64_t ldc,
                                                            int M, int N, int accumulate) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int m = (int)(i / N), n = (int)(i % N);
  float v = 0.0f;
  for (int z = 0; z < ks; ++z) v += P[(int64_t)z * M * N + i];
  float* cp = C + (int64_t)m * ldc + n;
  *cp = accumulate ? *cp + v : v;
}

// Slices of K for a few-row product (a decode batch), so that streaming W is spread over
// enough workgroups: about 512, each at least one 64-wide k-slab, and at most
// kSplitKMaxSlices slices (their readers add the partial planes one by one).
// k-slices: whole 64-wide slabs per slice, as many slices as needed to cover K
static int splitk_chunk(int K, int want) {
  const int nslab = (K + 63) / 64;
  return (nslab + want - 1) / want * 64;
}

#ifndef MAMBA_SPLITK_TARGET
#define MAMBA_SPLITK_TARGET 512  // workgroups a split-K product aims for
#endif
#ifndef MAMBA_SPLITK_MAX
#define MAMBA_SPLITK_MAX kSplitKMaxSlices
#endif

int gemm_splitk_slices(int M, int N, int K) {
  if (M > kSplitKMaxM || M <= kSkinnyMaxM || K % 8 != 0 || K < 128) return 1;
  const int bm = N < 128 ? 32 : 64, bn = N < 128 ? 80 : 32;
  const int64_t blocks = (int64_t)((N + bn - 1) / bn) * ((M + bm - 1) / bm);
  const int want = (int)std::min<int64_t>(
      std::min<int64_t>(std::max<int64_t>(MAMBA_SPLITK_TARGET / std::max<int64_t>(blocks, 1), 1), (K + 63) / 64),
      MAMBA_SPLITK_MAX);
  const int chunk = splitk_chunk(K, want);
  return (K + chunk - 1) / chunk;
}

hipError_t launch_gemm_bf16_parts(const void* A, bool a_bf16, int64_t lda, const void* W,
                                  int64_t ldw, float* C, int64_t ldc, int M, int N, int K,
                                  bool accumulate, float* partial, PartsView* out, hipStream_t s) {
  const int ks = gemm_splitk_slices(M, N, K);
  const int chunk = ks > 1 ? (K + ks - 1) / ks : K;
  const int k_chunk = (chunk + 63) / 64 * 64;
  const bool aligned = lda % 8 == 0 && ldw % 8 == 0 && reinterpret_cast<uintptr_t>(A) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(W) % 16 == 0;
  if (ks <= 1 || !aligned || M <= kSkinnyMaxM) {
    // one product, written to (or added into) C
    *out = accumulate ? PartsView{nullptr, 0, 0, 0} : PartsView{C, 1, 0, ldc};
    return launch_gemm_bf16(A, a_bf16, lda, W, ldw, C, ldc, M, N, K, accumulate, s);
  }
  const bf16* w = static_cast<const bf16*>(W);
  const int64_t plane = (int64_t)M * N;
  *out = PartsView{partial, ks, plane, N};
  if (N < 128)
    return a_bf16 ? gemm_tile<bf16, 32, 80, 64, 2, 1>(static_cast<const bf16*>(A), lda, w, ldw, partial, N, M, N,
                                                      K, false, true, s, ks, k_chunk, plane)
                  : gemm_tile<float, 32, 80, 64, 2, 1>(static_cast<const float*>(A), lda, w, ldw, partial, N, M,
                                                       N, K, false, true, s, ks, k_chunk, plane);
  return a_bf16 ? gemm_tile<bf16, 64, 32, 64, 2, 1>(static_cast<const bf16*>(A), lda, w, ldw, partial, N, M, N,
                                                    K, false, true, s, ks, k_chunk, plane)
                : gemm_tile<float, 64, 32, 64, 2, 1>(static_cast<const float*>(A), lda, w, ldw, partial, N, M,
                                                     N, K, false, true, s, ks, k_chunk, plane);
}

// Many rows, few columns (x_proj's dt_rank + 2 d_state): 32 x 80 tiles leave too few
// workgroups to stream A at full rate (M / 32 of them), so K is cut into slices: about 1024
// workgroups, whole 64-wide k-slabs per slice, at most max_ks slices.
int gemm_rows_ksplit(int M, int N, int K, int max_ks) {
  if (N >= 128 || M <= kSplitKMaxM || K % 64 != 0) return 1;
  const int64_t blocks = (int64_t)((N + 79) / 80) * ((M + 31) / 32);
  const int want = (int)std::min<int64_t>(
      std::min<int64_t>(std::max<int64_t>(1024 / std::max<int64_t>(blocks, 1), 1), K / 64),
      std::min(max_ks, kSplitKMaxSlices));
  if (want <= 1) return 1;
  const int chunk = splitk_chunk(K, want);
  return (K + chunk - 1) / chunk;
}

hipError_t launch_gemm_bf16_rows(const void* A, bool a_bf16, int64_t lda, const void* W,
                                 int64_t ldw, float* C, int64_t ldc, int M, int N, int K,
                                 bool accumulate, float* partial, int max_ks, hipStream_t s) {
  const int ks = gemm_rows_ksplit(M, N, K, max_ks);
  const bool aligned = lda % 8 == 0 && ldw % 8 == 0 && reinterpret_cast<uintptr_t>(A) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(W) % 16 == 0;
  if (ks <= 1 || !aligned) return launch_gemm_bf16(A, a_bf16, lda, W, ldw, C, ldc, M, N, K, accumulate, s);
  const int k_chunk = splitk_chunk(K, ks);
  const int64_t plane = (int64_t)M * N;
  const bf16* w = static_cast<const bf16*>(W);
  const hipError_t e =
      a_bf16 ? gemm_tile<bf16, 32, 80, 64, 2, 1>(static_cast<const bf16*>(A), lda, w, ldw, partial, N, M, N, K,
                                                 false, true, s, ks, k_chunk, plane)
             : gemm_tile<float, 32, 80, 64, 2, 1>(static_cast<const float*>(A), lda, w, ldw, partial, N, M, N, K,
                                                  false, true, s, ks, k_chunk, plane);
  if (e != hipSuccess) return e;
  splitk_reduce_kernel<<<dim3((unsigned)((plane + 255) / 256)), 256, 0, s>>>(partial, ks, C, ldc, M, N,
                                                                            accumulate ? 1 : 0);
  return hipGetLastError();
}

// x_proj's partial planes summed and dt_proj applied, in one launch (prefill.rs page,
// `prefill_body` stages F4b, the x_proj GEMM, and F4c, the gather of the dt columns and the
// dt_proj GEMM ahead of the softplus, which the scan applies). A workgroup takes 16 MT rows
// and 1/CS of the D output columns; the CS workgroups of a row block run on one XCD (same
// blockIdx % 8), so all but the first find the partial planes in that XCD's L2.
//  1. each row of xdbl (dt lane | B | C) is the sum of the ks partial planes, added in slice
//     order from zero exactly as the reduction kernel above adds them; the column split 0
//     writes the rows out for the scan; every split keeps the dt lane in LDS as bf16 (RNE,
//     the rounding the GEMM applies when it stages an f32 operand), zero-padded to 64 k;
//  2. dt = dt_lane @ W_dt^T by v_mfma_f32_16x16x32_bf16 tiles with W_dt as the first operand
//     (lane l: output column n0 + l % 16, k = 8 (l / 16) + 0..7) and the staged rows as the
//     second, so that the result register r of lane l is dt[m0 + l % 16][n0 + 4 (l / 16) + r].
//     Each wave takes a quarter of the workgroup's columns, G tiles at a time, whose W_dt
//     fragments serve all MT row tiles, and passes each 16 x 16G block through LDS so that
//     it leaves as row runs of 64 G bytes (stored straight from the fragments, each store
//     instruction would cover 16 rows x 64 bytes: 17.5 against 14.9 us at the 130m
//     prefill). W_dt chunks past dt_rank are zero (their loads read the row's first chunk
//     instead, in bounds). The first group of W_dt fragments is loaded before the planes
//     are summed.
// Requires dt_rank % 8 == 0 and <= 64, D % (64 CS) == 0, xw % 4 == 0, 16-byte aligned buffers.
#ifndef MAMBA_XDT_FUSE
#define MAMBA_XDT_FUSE 1  // x_proj's reduction and dt_proj in one kernel (1) or two launches (0)
#endif
#ifndef MAMBA_CONV_XPROJ
#define MAMBA_CONV_XPROJ 1  // the prefill's conv and x_proj in one kernel (1) or two launches (0)
#endif
#ifndef MAMBA_XDT_SPLIT
#define MAMBA_XDT_SPLIT 6  // column splits per row block
#endif
#ifndef MAMBA_XDT_MT
#define MAMBA_XDT_MT 4  // 16-row MFMA tiles per workgroup
#endif
constexpr int kXdtMT = MAMBA_XDT_MT;
constexpr int kXdtRows = 16 * kXdtMT;
constexpr int kXdtMaxRank = 64;
#ifndef MAMBA_XDT_GROUP
#define MAMBA_XDT_GROUP 4
#endif
constexpr int kXdtGroup = MAMBA_XDT_GROUP;  // W_dt tiles whose fragments a wave loads together

template <bool DELTA>
__global__ void __launch_bounds__(256) xproj_sum_dtproj_kernel(const float* __restrict__ P, int ks,
                                                               int64_t plane, float* __restrict__ xdbl,
                                                               int xw, const bf16* __restrict__ Wdt, int R,
                                                               float* __restrict__ dt, int D, int M, int CS,
                                                               const float* __restrict__ dt_bias, int sp) {
  __shared__ __align__(16) bf16 Xs[kXdtRows][kXdtMaxRank + 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrb = (M + kXdtRows - 1) / kXdtRows;
  const int b = blockIdx.x, hi = b / 8, cs = hi % CS, rb = (hi / CS) * 8 + b % 8;
  if (rb >= nrb) return;  // the grid is whole groups of 8 row blocks
  const int m0 = rb * kXdtRows;
  const int fr = lane & 15, fc = lane >> 4;
  const bool v0 = 8 * fc < R, v1 = 32 + 8 * fc < R, two = R > 32;
  const int k0 = v0 ? 8 * fc : 0, k1 = v1 ? 32 + 8 * fc : 0;
  // 16-column tiles per wave, their first, and groups of them
  const int nt = D / (64 * CS), t_beg = (cs * 4 + wave) * nt, ng = (nt + kXdtGroup - 1) / kXdtGroup;
  // W_dt fragments of a group of tiles (indexes past the last tile reload the last one)
  uint4 wa[kXdtGroup], wb[kXdtGroup];
  float4 bias4[kXdtGroup];  // DELTA: dt_bias of the lane's four output columns per tile
  auto fetch = [&](int g) {
#pragma unroll
    for (int i = 0; i < kXdtGroup; ++i) {
      const int t = min(g * kXdtGroup + i, nt - 1);
      const bf16* wr = Wdt + (int64_t)((t_beg + t) * 16 + fr) * R;
      wa[i] = *reinterpret_cast<const uint4*>(wr + k0);
      wb[i] = *reinterpret_cast<const uint4*>(wr + k1);
      if constexpr (DELTA)
        bias4[i] = dt_bias ? *reinterpret_cast<const float4*>(dt_bias + (t_beg + t) * 16 + 4 * fc)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  fetch(0);

  const int qw = cs == 0 ? xw / 4 : R / 4;  // float4 columns this split sums: all, or the dt lane
  for (int q = tid; q < kXdtRows * qw; q += 256) {
    const int r = q / qw, c = 4 * (q % qw);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m0 + r < M) {
      const float* p = P + (int64_t)(m0 + r) * xw + c;
      int z = 0;
      for (; z + 4 <= ks; z += 4) {  // four loads in flight, added in slice order
        float4 t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = *reinterpret_cast<const float4*>(p + (z + i) * plane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v.x += t[i].x; v.y += t[i].y; v.z += t[i].z; v.w += t[i].w;
        }
      }
      for (; z < ks; ++z) {
        const float4 t = *reinterpret_cast<const float4*>(p + z * plane);
        v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
      }
      if (cs == 0) *reinterpret_cast<float4*>(xdbl + (int64_t)(m0 + r) * xw + c) = v;
    }
    if (c < R) {
      Xs[r][c] = (bf16)v.x; Xs[r][c + 1] = (bf16)v.y; Xs[r][c + 2] = (bf16)v.z; Xs[r][c + 3] = (bf16)v.w;
    }
  }
  for (int i = tid; i < kXdtRows * (kXdtMaxRank - R); i += 256)
    Xs[i / (kXdtMaxRank - R)][R + i % (kXdtMaxRank - R)] = (bf16)0.0f;
  __syncthreads();

  // each wave's 16 x 16G blocks of dt, one row tile at a time, are staged in LDS and leave
  // in row order; the W_dt fragments serve every row tile of the workgroup
  constexpr int TP = 16 * kXdtGroup + 4;  // staged row pitch, floats
  __shared__ __align__(16) float Ts[4][16 * TP];
  float* tw = Ts[wave];
  auto group = [&](const uint4* ca, const uint4* cb, int g) {
    const int valid = min(kXdtGroup, nt - g * kXdtGroup) * 4;  // float4 columns that exist
#pragma unroll
    for (int mt = 0; mt < kXdtMT; ++mt) {
      const bf16x8 x0 = *reinterpret_cast<const bf16x8*>(&Xs[16 * mt + fr][8 * fc]);
      const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(&Xs[16 * mt + fr][32 + 8 * fc]);
#pragma unroll
      for (int i = 0; i < kXdtGroup; ++i) {
        const bf16x8 w0 = v0 ? __builtin_bit_cast(bf16x8, ca[i]) : bf16x8{};
        const bf16x8 w1 = v1 ? __builtin_bit_cast(bf16x8, cb[i]) : bf16x8{};
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, x0, acc, 0, 0, 0);
        if (two) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, x1, acc, 0, 0, 0);
        if constexpr (DELTA) {
          // delta = softplus(dt + dt_bias): the scan's own expression, in the same order
          const float bv[4] = {bias4[i].x, bias4[i].y, bias4[i].z, bias4[i].w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = acc[r] + bv[r];
            acc[r] = sp ? softplus(v) : v;
          }
        }
        *reinterpret_cast<f32x4*>(&tw[fr * TP + 16 * i + 4 * fc]) = acc;
      }
      // the wave's 16 x 16G block back in row order (LDS operations of one wave run in
      // issue order): each store instruction covers runs of whole rows
#pragma unroll
      for (int j = 0; j < kXdtGroup; ++j) {
        const int idx = j * 64 + lane, r = idx / (4 * kXdtGroup), c4 = idx % (4 * kXdtGroup);
        const f32x4 v = *reinterpret_cast<const f32x4*>(&tw[r * TP + 4 * c4]);
        const int row = m0 + 16 * mt + r;
        if (row < M && c4 < valid)
          *reinterpret_cast<f32x4*>(dt + (int64_t)row * D + (t_beg + g * kXdtGroup) * 16 + 4 * c4) = v;
      }
    }
  };
  for (int g = 0; g < ng; ++g) {
    if (g > 0) fetch(g);
    group(wa, wb, g);
  }
}

// dt -> softplus(dt + dt_bias) (or dt + dt_bias), elementwise: the two-launch path's epilogue.
__global__ void __launch_bounds__(256) dt_delta_kernel(float* __restrict__ dt, const float* __restrict__ dt_bias,
                                                       int sp, int64_t n, int D) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = dt[i] + (dt_bias ? dt_bias[i % D] : 0.0f);
  dt[i] = sp ? softplus(v) : v;
}

// x_proj's ks partial planes (ks * M * xw floats at `partial`) -> xdbl and dt: one kernel
// when the shapes allow, else the in-order reduction and the dt_proj product.
static hipError_t finish_xproj_dtproj(const float* partial, int ks, float* xdbl, int xw, const void* Wdt,
                                      int R, float* dt, int M, int D, const DtOut& o, hipStream_t s) {
  auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const int64_t plane = (int64_t)M * xw;
  const bool delta = o.bias || o.softplus;
  const bool fuse = MAMBA_XDT_FUSE && a16(Wdt) && a16(xdbl) && a16(dt) && a16(partial) && R % 8 == 0 &&
                    R > 0 && R <= kXdtMaxRank && D % 64 == 0 && xw % 4 == 0 && a16(o.bias);
  hipError_t e;
  if (!fuse) {
    splitk_reduce_kernel<<<dim3((unsigned)((plane + 255) / 256)), 256, 0, s>>>(partial, ks, xdbl, xw, M, xw, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_gemm_bf16(xdbl, false, xw, Wdt, R, dt, D, M, D, R, false, s)) != hipSuccess) return e;
    if (!delta) return hipSuccess;
    const int64_t n = (int64_t)M * D;
    dt_delta_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(dt, o.bias, o.softplus ? 1 : 0, n, D);
    return hipGetLastError();
  }
  int cs = MAMBA_XDT_SPLIT;
  while (cs > 1 && D % (64 * cs) != 0) --cs;
  const int64_t nrb = (M + kXdtRows - 1) / kXdtRows;
  const dim3 grid((unsigned)((nrb + 7) / 8 * 8 * cs));
  if (delta)
    xproj_sum_dtproj_kernel<true><<<grid, 256, 0, s>>>(partial, ks, plane, xdbl, xw, static_cast<const bf16*>(Wdt),
                                                       R, dt, D, M, cs, o.bias, o.softplus ? 1 : 0);
  else
    xproj_sum_dtproj_kernel<false><<<grid, 256, 0, s>>>(partial, ks, plane, xdbl, xw, static_cast<const bf16*>(Wdt),
                                                        R, dt, D, M, cs, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_xproj_dtproj(const float* u, int64_t ldu, const void* Wx, float* xdbl, int xw,
                               const void* Wdt, int R, float* dt, int M, int D, float* partial,
                               int max_ks, const DtOut& o, hipStream_t s) {
  const int ks = gemm_rows_ksplit(M, xw, D, max_ks);
  auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  if (ks <= 1 || ldu % 8 != 0 || D % 8 != 0 || !a16(u) || !a16(Wx)) {
    hipError_t e = launch_gemm_bf16_rows(u, false, ldu, Wx, D, xdbl, xw, M, xw, D, false, partial, max_ks, s);
    if (e != hipSuccess) return e;
    if ((e = launch_gemm_bf16(xdbl, false, xw, Wdt, R, dt, D, M, D, R, false, s)) != hipSuccess) return e;
    if (!o.bias && !o.softplus) return hipSuccess;
    const int64_t n = (int64_t)M * D;
    dt_delta_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(dt, o.bias, o.softplus ? 1 : 0, n, D);
    return hipGetLastError();
  }
  const int k_chunk = splitk_chunk(D, ks);
  const int64_t plane = (int64_t)M * xw;
  const hipError_t e = gemm_tile<float, 32, 80, 64, 2, 1>(u, ldu, static_cast<const bf16*>(Wx), D, partial, xw,
                                                          M, xw, D, false, true, s, ks, k_chunk, plane);
  if (e != hipSuccess) return e;
  return finish_xproj_dtproj(partial, ks, xdbl, xw, Wdt, R, dt, M, D, o, s);
}

// ------------------------------------------------------- conv + x_proj of a prefill layer
//
// prefill.rs page, prefill_body stages F4a (the causal depthwise conv + SiLU over the x lane
// of in_proj's output, carrying the conv state) and F4b (the x_proj GEMM), in one kernel
// whose output is x_proj's split-K partial planes, as the split GEMM leaves them, plus u.
// A workgroup takes 32 tokens of one sequence and one K slice of the channels (the slices
// of the split GEMM), in 64-channel slabs:
//  - lane l of wave q takes channel l of the slab and tokens 8 q .. 8 q + 7, and loads the
//    11 x rows their taps reach itself (256-byte row pieces per wave; the rows shared with
//    the neighbouring wave come from L1/L2); the rows of the next two slabs are in flight
//    while a slab is computed;
//  - u = silu(conv) is formed with the taps added in the order of conv1d_fwd_kernel, so u
//    has the same bits; it is stored for the scan and kept in LDS as bf16 (RNE, the
//    rounding x_proj applies to its operand), double-buffered, so a slab takes one barrier;
//  - the slab goes into the 32 x xw partial product by v_mfma_f32_16x16x32_bf16 tiles
//    (the slab order and k steps of the split GEMM's 32 x 80 tiles). Wave q takes column
//    tiles q and q + 4 for both token tiles, so each W_x fragment is loaded once per
//    workgroup (with two waves per column tile it was loaded twice: 36.7 against 31.6 us
//    at the 130m prefill).
// Workgroup (b, first token block, slice) is the only reader of sequence b's old conv state
// for the slice's channels, and at its end the only writer of the new one (X[Tb .. Tb+K-1]
// of X = [old state, x], Tb the sequence's length), as in conv1d_fwd_kernel. Its loop is a
// copy of its own (FIRST), in which the window rows before the sequence start come from the
// state, so that the other workgroups' loads carry no condition.
constexpr int kCxRows = 32;   // tokens per workgroup
constexpr int kCxK = 4;       // conv taps on this path
constexpr int kCxMaxN = 80;   // x_proj columns: at most 5 tiles of 16

template <bool FIRST>
__device__ __forceinline__ void conv_xproj_body(
    const float* __restrict__ xb, int64_t ldx, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, const float* __restrict__ st_old, float* __restrict__ ub,
    const bf16* __restrict__ Wx, int xw, f32x4 (&acc)[2][2], bf16* As, int t0, int T, int D, int c_beg,
    int nslab) {
  constexpr int SL = 64, W = kCxK - 1 + 8, AP = SL + 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = wave * 8;
  const int ntn = (xw + 15) / 16;
  const int fr = lane & 15, fq = lane >> 4;
  const float* bsrc = conv_b ? conv_b : conv_w;
  // window of slab sl: x rows t0 + r0 - 3 + j (the state before the sequence start);
  // nwin holds the next slab's, nwin2 (two slabs ahead) the one after
  float nwin[W], nwin2[W];
  auto load_window = [&](float (&dst)[W], int sl) {
    const int c = c_beg + sl * SL + lane;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const int tt = t0 + r0 - (kCxK - 1) + j;
      if (FIRST && tt < 0)
        dst[j] = st_old ? st_old[(int64_t)c * kCxK + kCxK + tt] : 0.0f;
      else
        dst[j] = xb[(int64_t)min(tt, T - 1) * ldx + c];
    }
  };
  float4 wnext = *reinterpret_cast<const float4*>(conv_w + (int64_t)(c_beg + lane) * kCxK);
  float bnext = bsrc[c_beg + lane];
  load_window(nwin, 0);
  load_window(nwin2, min(1, nslab - 1));
  for (int sl = 0; sl < nslab; ++sl) {
    const int c0 = c_beg + sl * SL;
    float win[W];
#pragma unroll
    for (int j = 0; j < W; ++j) win[j] = nwin[j];
#pragma unroll
    for (int j = 0; j < W; ++j) nwin[j] = nwin2[j];
    const float4 wt = wnext;
    const float bias = conv_b ? bnext : 0.0f;
    // W_x fragments of this slab: wave q takes column tiles q and q + 4 (when it exists) for
    // both token tiles, so each tile's fragments are loaded once per workgroup; column
    // 16 n + l % 16 (the last column for n >= xw, never stored), k = 8 (l / 16) + 32 kstep
    uint4 wf[2][2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
      wf[0][k2] = *reinterpret_cast<const uint4*>(Wx + (int64_t)min(16 * wave + fr, xw - 1) * D + c0 + 8 * fq +
                                                  32 * k2);
    if (wave + 4 < ntn) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        wf[1][k2] = *reinterpret_cast<const uint4*>(Wx + (int64_t)min(16 * (wave + 4) + fr, xw - 1) * D + c0 +
                                                    8 * fq + 32 * k2);
    }
    {
      const int sn = min(sl + 1, nslab - 1);
      wnext = *reinterpret_cast<const float4*>(conv_w + (int64_t)(c_beg + sn * SL + lane) * kCxK);
      bnext = bsrc[c_beg + sn * SL + lane];
      load_window(nwin2, min(sl + 2, nslab - 1));
    }
    bf16* as = As + (sl & 1) * kCxRows * AP;
    const float w[kCxK] = {wt.x, wt.y, wt.z, wt.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float c = bias;
#pragma unroll
      for (int k = 0; k < kCxK; ++k) c = fmaf(w[k], win[i + k], c);
      const float uv = silu(c);
      if (t0 + r0 + i < T) ub[(int64_t)(t0 + r0 + i) * D + c0 + lane] = uv;
      as[(r0 + i) * AP + lane] = (bf16)uv;
    }
    __syncthreads();
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      bf16x8 a[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) a[m] = *reinterpret_cast<const bf16x8*>(&as[(16 * m + fr) * AP + 32 * k2 + 8 * fq]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (wave + 4 * i < ntn)
#pragma unroll
          for (int m = 0; m < 2; ++m)
            acc[i][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], __builtin_bit_cast(bf16x8, wf[i][k2]),
                                                                acc[i][m], 0, 0, 0);
    }
  }
}

__global__ void __launch_bounds__(256) conv_xproj_kernel(
    const float* __restrict__ x, int64_t ldx, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, float* __restrict__ conv_state, const int32_t* __restrict__ lengths,
    float* __restrict__ u, const bf16* __restrict__ Wx, int xw, float* __restrict__ P, int64_t plane, int T,
    int D, int k_chunk, int ntb) {
  __shared__ __align__(16) bf16 As[2 * kCxRows * (64 + 8)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / ntb, tb = blockIdx.x % ntb, zs = blockIdx.y;
  const int t0 = tb * kCxRows;
  const int c_beg = zs * k_chunk, c_end = min(D, c_beg + k_chunk);
  const int nslab = (c_end - c_beg) / 64;
  const float* xb = x + (int64_t)b * T * ldx;
  float* ub = u + (int64_t)b * T * D;
  const float* st_old = conv_state ? conv_state + (int64_t)b * D * kCxK : nullptr;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m) acc[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (t0 == 0)
    conv_xproj_body<true>(xb, ldx, conv_w, conv_b, st_old, ub, Wx, xw, acc, As, t0, T, D, c_beg, nslab);
  else
    conv_xproj_body<false>(xb, ldx, conv_w, conv_b, st_old, ub, Wx, xw, acc, As, t0, T, D, c_beg, nslab);
  // register r of lane l of tile (i, m) holds token 16 m + 4 (l / 16) + r, column
  // 16 (wave + 4 i) + l % 16
  const int fr = lane & 15, fq = lane >> 4;
  float* pz = P + zs * plane + ((int64_t)b * T + t0) * xw;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = 16 * (wave + 4 * i) + fr;
    if (n >= xw) continue;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 16 * m + 4 * fq + r;
        if (t0 + tr < T) pz[(int64_t)tr * xw + n] = acc[i][m][r];
      }
  }
  if (t0 == 0 && conv_state) {
    // every read of the old state has returned before its thread reached the last barrier
    const int Tb = lengths ? min(max(lengths[b], 0), T) : T;
    float* st = conv_state + (int64_t)b * D * kCxK;
    for (int c = c_beg + tid; c < c_end; c += 256) {
      float v[kCxK];
#pragma unroll
      for (int k = 0; k < kCxK; ++k) {
        const int i = Tb + k;
        v[k] = i >= kCxK ? xb[(int64_t)(i - kCxK) * ldx + c] : st[(int64_t)c * kCxK + i];
      }
#pragma unroll
      for (int k = 0; k < kCxK; ++k) st[(int64_t)c * kCxK + k] = v[k];
    }
  }
}

hipError_t launch_conv_xproj_dtproj(const ConvFwdArgs& ca, const void* Wx, float* xdbl, int xw,
                                    const void* Wdt, int R, float* dt, float* partial, int max_ks,
                                    const DtOut& o, hipStream_t s) {
  const int D = ca.D, T = ca.T;
  const int M = ca.B * T;
  const int ks = gemm_rows_ksplit(M, xw, D, max_ks);
  auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const bool fuse = MAMBA_CONV_XPROJ && ks > 1 && ca.K == kCxK && !ca.bf16 && D % 64 == 0 &&
                    xw <= kCxMaxN && ca.x_row_stride % 4 == 0 && a16(ca.x) && a16(ca.conv_w) && a16(Wx) &&
                    a16(partial);
  hipError_t e;
  if (!fuse) {
    if ((e = launch_conv1d_fwd(ca, s)) != hipSuccess) return e;
    return launch_xproj_dtproj(static_cast<const float*>(ca.u), D, Wx, xdbl, xw, Wdt, R, dt, M, D, partial,
                               max_ks, o, s);
  }
  const int k_chunk = splitk_chunk(D, ks);
  const int ntb = (T + kCxRows - 1) / kCxRows;
  const int64_t plane = (int64_t)M * xw;
  conv_xproj_kernel<<<dim3((unsigned)(ca.B * ntb), (unsigned)ks), 256, 0, s>>>(
      static_cast<const float*>(ca.x), ca.x_row_stride, ca.conv_w, ca.conv_b, ca.conv_state, ca.lengths,
      static_cast<float*>(ca.u), static_cast<const bf16*>(Wx), xw, partial, plane, T, D, k_chunk, ntb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return finish_xproj_dtproj(partial, ks, xdbl, xw, Wdt, R, dt, M, D, o, s);
}

hipError_t launch_gemm_bf16_splitk(const void* A, bool a_bf16, int64_t lda, const void* W,
                                   int64_t ldw, float* C, int64_t ldc, int M, int N, int K,
                                   bool accumulate, float* partial, hipStream_t s) {
  PartsView v;
  hipError_t e = launch_gemm_bf16_parts(A, a_bf16, lda, W, ldw, C, ldc, M, N, K, accumulate, partial, &v, s);
  if (e != hipSuccess || v.p != partial) return e;
  const int64_t plane = (int64_t)M * N;
  splitk_reduce_kernel<<<dim3((unsigned)((plane + 255) / 256)), 256, 0, s>>>(partial, v.ks, C, ldc, M, N,
                                                                            accumulate ? 1 : 0);
  return hipGetLastError();
}

// ------------------------------------------------------- decode step with split-K consumers
//
// In the decode step the split-K partial planes are not reduced by a kernel of their own:
// each consumer adds them up as it reads (PartsView::at, in slice order, so the values are
// those the reduction kernel would have written).

// h[r] += the out_proj partials (if any), then RMSNorm of the new h[r] (bf16 out). The
// arithmetic is that of rmsnorm_kernel applied after a split-K reduction with accumulate.
// A thread's KMAX elements of the row, their partial-plane values and weights are all loaded
// before the first use, so the block waits on memory once.
template <int KMAX>
__global__ void __launch_bounds__(256) residual_rmsnorm_kernel(float* __restrict__ h, PartsView add,
                                                               const float* __restrict__ w, float eps,
                                                               bf16* __restrict__ out, int Dm) {
  __shared__ float part[8];
  const int64_t r = blockIdx.x;
  float* hr = h + r * Dm;
  const int ks = add.ks;
  // Every load is issued unconditionally (addresses clamped into the row, the first plane or
  // the row itself standing in for a missing one) and the values are selected at their use:
  // loads under conditions make the wave wait for each one in turn.
  const float* pp = ks > 0 ? add.p + r * add.ld : hr;
  const int64_t pz = ks > 0 ? add.plane : 0;
  const float* wp = w ? w : hr;
  float v[KMAX], wv[KMAX], pv[kSplitKMaxSlices][KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int c = min((int)threadIdx.x + 256 * k, Dm - 1);
    v[k] = hr[c];
    wv[k] = wp[c];
#pragma unroll
    for (int z = 0; z < kSplitKMaxSlices; ++z) pv[z][k] = pp[min(z, max(ks - 1, 0)) * pz + c];
  }
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int c = threadIdx.x + 256 * k;
    if (c >= Dm) break;
    if (!w) wv[k] = 1.0f;
    if (ks > 0) {
      float sum = 0.0f;  // the planes in slice order, as PartsView::at adds them
#pragma unroll
      for (int z = 0; z < kSplitKMaxSlices; ++z)
        if (z < ks) sum += pv[z][k];
      v[k] = v[k] + sum;
      hr[c] = v[k];
    }
    ss = fmaf(v[k], v[k], ss);
  }
  for (int m = 32; m >= 1; m /= 2) ss += __shfl_xor(ss, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)Dm + eps);
  bf16* o = out + r * Dm;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int c = threadIdx.x + 256 * k;
    if (c < Dm) o[c] = (bf16)(v[k] * inv * wv[k]);
  }
}

// The same for rows wider than 8 * 256: the planes added element by element.
__global__ void __launch_bounds__(256) residual_rmsnorm_wide_kernel(float* __restrict__ h, PartsView add,
                                                                    const float* __restrict__ w, float eps,
                                                                    bf16* __restrict__ out, int Dm) {
  __shared__ float part[8];
  const int64_t r = blockIdx.x;
  float* hr = h + r * Dm;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < Dm; c += 256) {
    float v = hr[c];
    if (add.ks > 0) {
      v = v + add.at(r, c);
      hr[c] = v;
    }
    ss = fmaf(v, v, ss);
  }
  for (int m = 32; m >= 1; m /= 2) ss += __shfl_xor(ss, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)Dm + eps);
  bf16* o = out + r * Dm;
  for (int c = threadIdx.x; c < Dm; c += 256) o[c] = (bf16)(hr[c] * inv * (w ? w[c] : 1.0f));
}

// Conv step on the x lane of the in_proj output (columns 0 .. D-1), the same arithmetic as
// conv1d_step_kernel: shift the K-slot window, append x, taps from the oldest, SiLU.
template <bool K4>
__global__ void __launch_bounds__(256) decode_conv_kernel(PartsView xin, const float* __restrict__ conv_w,
                                                          const float* __restrict__ conv_b,
                                                          float* __restrict__ conv_state,
                                                          float* __restrict__ u, int D, int K) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (d >= D) return;
  float* st = conv_state + ((int64_t)b * D + d) * K;
  const float* w = conv_w + (int64_t)d * K;
  const float xv = xin.at(b, d);
  float c = conv_b ? conv_b[d] : 0.0f;
  if (K4) {  // the 4-slot window and taps as 16-byte accesses
    const float4 v = *reinterpret_cast<const float4*>(st);
    const float4 wv = *reinterpret_cast<const float4*>(w);
    c = fmaf(wv.x, v.y, c);
    c = fmaf(wv.y, v.z, c);
    c = fmaf(wv.z, v.w, c);
    c = fmaf(wv.w, xv, c);
    *reinterpret_cast<float4*>(st) = make_float4(v.y, v.z, v.w, xv);
  } else {
    float sv[kMaxConvK];
    for (int k = 0; k + 1 < K; ++k) sv[k] = st[k + 1];
    sv[K - 1] = xv;
    for (int k = 0; k < K; ++k) c = fmaf(w[k], sv[k], c);
    for (int k = 0; k < K; ++k) st[k] = sv[k];
  }
  u[(int64_t)b * D + d] = silu(c);
}

// Conv step and x_proj of one decode layer in one launch. Workgroup (s, g) takes the
// kConvXC channels of slice s and up to kConvXRows sequences of group g: it runs the conv
// step for them (the arithmetic of decode_conv_kernel: the same u and conv state bit for
// bit), writes u for the SSM step and keeps bf16(u) in LDS, then forms the slice's share of
// every x_proj column: part[s][b][n] = sum over the slice's channels c, in order, of
// bf16(u[b][c]) * W_x[n][c] in f32 (the operands the MFMA product rounds to, f32 sums).
// The SSM step adds the D / kConvXC planes in slice order. Needs D % kConvXC == 0 and 16-byte
// aligned W_x rows.
template <bool K4>
__global__ void __launch_bounds__(256) decode_conv_xproj_kernel(
    PartsView xin, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    float* __restrict__ conv_state, float* __restrict__ u, const bf16* __restrict__ Wx, int xw,
    float* __restrict__ part, int B, int D, int K) {
  __shared__ __align__(16) float s_u[kConvXRows][kConvXC];
  const int sl = blockIdx.x, d0 = sl * kConvXC;
  const int b0 = blockIdx.y * kConvXRows;
  const int rows = min(kConvXRows, B - b0);
  // x_proj: thread n takes output column n for all the group's sequences, so each W_x row
  // slice is loaded once per workgroup; the slice of its first column is loaded here, before
  // the conv step, so that its latency overlaps the conv step's loads
  constexpr int kCh8 = kConvXC / 8;
  uint4 wpre[kCh8];
  {
    const bf16* wr = Wx + (int64_t)min((int)threadIdx.x, xw - 1) * D + d0;
#pragma unroll
    for (int c = 0; c < kCh8; ++c) wpre[c] = *reinterpret_cast<const uint4*>(wr + 8 * c);
  }
  for (int i = threadIdx.x; i < rows * kConvXC; i += 256) {
    const int bl = i / kConvXC, c = i % kConvXC, b = b0 + bl, d = d0 + c;
    float* st = conv_state + ((int64_t)b * D + d) * K;
    const float* w = conv_w + (int64_t)d * K;
    const float xv = xin.at(b, d);
    float cv = conv_b ? conv_b[d] : 0.0f;
    if (K4) {
      const float4 v = *reinterpret_cast<const float4*>(st);
      const float4 wv = *reinterpret_cast<const float4*>(w);
      cv = fmaf(wv.x, v.y, cv);
      cv = fmaf(wv.y, v.z, cv);
      cv = fmaf(wv.z, v.w, cv);
      cv = fmaf(wv.w, xv, cv);
      *reinterpret_cast<float4*>(st) = make_float4(v.y, v.z, v.w, xv);
    } else {
      float sv[kMaxConvK];
      for (int k = 0; k + 1 < K; ++k) sv[k] = st[k + 1];
      sv[K - 1] = xv;
      for (int k = 0; k < K; ++k) cv = fmaf(w[k], sv[k], cv);
      for (int k = 0; k < K; ++k) st[k] = sv[k];
    }
    const float uv = silu(cv);
    u[(int64_t)b * D + d] = uv;
    s_u[bl][c] = to_f32(from_f32<bf16>(uv));
  }
  __syncthreads();
  // each output sums its channels in order
  const int64_t plane = (int64_t)B * xw;
  for (int n = threadIdx.x; n < xw; n += 256) {
    uint4 w8[kCh8];
    if (n == (int)threadIdx.x) {
#pragma unroll
      for (int c = 0; c < kCh8; ++c) w8[c] = wpre[c];
    } else {
      const bf16* wr = Wx + (int64_t)n * D + d0;
#pragma unroll
      for (int c = 0; c < kCh8; ++c) w8[c] = *reinterpret_cast<const uint4*>(wr + 8 * c);
    }
    float acc[kConvXRows];
#pragma unroll
    for (int bl = 0; bl < kConvXRows; ++bl) acc[bl] = 0.0f;
    // (a rolled loop over the 8-channel chunks, the W chunks shifted down the register array,
    // keeps the register count low)
#pragma unroll 1
    for (int c = 0; c < kCh8; ++c) {
      const bf16x8 wv = __builtin_bit_cast(bf16x8, w8[0]);
#pragma unroll
      for (int k = 0; k + 1 < kCh8; ++k) w8[k] = w8[k + 1];
      float uq[kConvXRows][8];
#pragma unroll
      for (int bl = 0; bl < kConvXRows; ++bl) {
        const float4 lo = *reinterpret_cast<const float4*>(&s_u[bl][8 * c]);
        const float4 hi = *reinterpret_cast<const float4*>(&s_u[bl][8 * c + 4]);
        uq[bl][0] = lo.x; uq[bl][1] = lo.y; uq[bl][2] = lo.z; uq[bl][3] = lo.w;
        uq[bl][4] = hi.x; uq[bl][5] = hi.y; uq[bl][6] = hi.z; uq[bl][7] = hi.w;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float wf = to_f32(wv[i]);
#pragma unroll
        for (int bl = 0; bl < kConvXRows; ++bl) acc[bl] = fmaf(uq[bl][i], wf, acc[bl]);
      }
    }
#pragma unroll
    for (int bl = 0; bl < kConvXRows; ++bl)
      if (bl < rows) part[(int64_t)sl * plane + (int64_t)(b0 + bl) * xw + n] = acc[bl];
  }
}

// SSM step of one layer with dt_proj folded in: the x_proj row of sequence b (dt low-rank
// part | B | C, from its partial planes) is summed once into LDS; each channel's NQ lanes
// then form dt = W_dt[d] . bf16(x[0 .. R)) (the projection's bf16 operands, f32 sums), and
// go on as the SSM step (softplus(dt + bias), update, readout, D skip), with z from the
// in_proj partials (columns zcol .. zcol + D - 1).
template <int NQ, bool VEC4>
__global__ void __launch_bounds__(256) decode_ssm_kernel(
    const float* __restrict__ u, PartsView xd, const bf16* __restrict__ Wdt, int R,
    const float* __restrict__ dt_bias, const float* __restrict__ A_log, const float* __restrict__ D_skip,
    PartsView zin, int zcol, float* __restrict__ state, float* __restrict__ y, int D, int N) {
  __shared__ float s_x[kDecodeMaxXProj];
  const int b = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int d = t / NQ, q = t % NQ;
  const int dc = min(d, D - 1);  // (lanes past D load a valid row and drop out below)

  // This lane's loads that do not depend on the x_proj row are issued before the row is
  // staged, so their latency overlaps the staging (the barrier waits only for LDS work):
  // its W_dt run, its four states and A_log entries (16-byte path), u and the parameters.
  // Lane q takes the contiguous columns [q * C, q * C + C) of W_dt's row d.
  const bf16* wr = Wdt + (int64_t)dc * R;
  const int C = (R + NQ - 1) / NQ, r0 = q * C, r1 = min(R, r0 + C);
  constexpr int kPreW = 4;  // W_dt runs of up to 16 columns are loaded up front
  uint2 wpre[kPreW];
  const bool pre_w = VEC4 && C <= 4 * kPreW;
  if (pre_w) {
#pragma unroll
    for (int i = 0; i < kPreW; ++i)
      wpre[i] = *reinterpret_cast<const uint2*>(wr + min(r0 + 4 * i, R - 4));  // used only if inside the run
  }
  const int64_t ch = (int64_t)b * D + dc;
  float* hs = state + ch * N;
  const float* al = A_log + (int64_t)dc * N;
  const int n0 = 4 * q;
  const bool vec_state = VEC4 && N % 4 == 0;
  // (no load under a condition: a lane past N reads the row's last four states and does not
  // use them, absent vectors read a stand-in address; the values are selected at the use)
  float4 hv = make_float4(0.f, 0.f, 0.f, 0.f), av = hv;
  if (vec_state) {
    const int nc = min(n0, N - 4);
    hv = *reinterpret_cast<const float4*>(hs + nc);
    av = *reinterpret_cast<const float4*>(al + nc);
  }
  const float uv = u[ch];
  const float bias_v = *(dt_bias ? dt_bias + dc : u + ch);
  const float dskip_v = *(D_skip ? D_skip + dc : u + ch);
  const float bias = dt_bias ? bias_v : 0.0f;
  const float dskip = D_skip ? dskip_v : 0.0f;

  for (int i = threadIdx.x; i < R + 2 * N; i += 256) s_x[i] = xd.at(b, i);
  __syncthreads();
  if (d >= D) return;  // whole NQ-lane groups drop out together

  float acc = 0.0f;
  if (pre_w) {
#pragma unroll
    for (int i = 0; i < kPreW; ++i) {
      const int r = r0 + 4 * i;
      if (r < r1) {
        const uint2 wv = wpre[i];
        acc = fmaf((float)(bf16)s_x[r], __uint_as_float(wv.x << 16), acc);
        acc = fmaf((float)(bf16)s_x[r + 1], __uint_as_float(wv.x & 0xffff0000u), acc);
        acc = fmaf((float)(bf16)s_x[r + 2], __uint_as_float(wv.y << 16), acc);
        acc = fmaf((float)(bf16)s_x[r + 3], __uint_as_float(wv.y & 0xffff0000u), acc);
      }
    }
  } else if (VEC4) {  // R a multiple of 4 NQ: C is a multiple of 4 and each run is 8-byte aligned
    for (int r = r0; r < r1; r += 4) {
      const uint2 wv = *reinterpret_cast<const uint2*>(wr + r);
      acc = fmaf((float)(bf16)s_x[r], __uint_as_float(wv.x << 16), acc);
      acc = fmaf((float)(bf16)s_x[r + 1], __uint_as_float(wv.x & 0xffff0000u), acc);
      acc = fmaf((float)(bf16)s_x[r + 2], __uint_as_float(wv.y << 16), acc);
      acc = fmaf((float)(bf16)s_x[r + 3], __uint_as_float(wv.y & 0xffff0000u), acc);
    }
  } else {
    for (int r = r0; r < r1; ++r) acc = fmaf((float)(bf16)s_x[r], (float)wr[r], acc);
  }
#pragma unroll
  for (int m = NQ / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m, NQ);

  const float delta = softplus(acc + bias);
  const float du = delta * uv;
  float part = 0.0f;
  if (vec_state) {
    // four states per lane as one 16-byte access (N a multiple of 4: rows 16-byte aligned)
    if (n0 < N) {
      const float hh[4] = {hv.x, hv.y, hv.z, hv.w}, aa[4] = {av.x, av.y, av.z, av.w};
      float hn[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a2 = -__builtin_amdgcn_exp2f(aa[j] * kLog2e) * kLog2e;
        const float a = __builtin_amdgcn_exp2f(delta * a2);
        hn[j] = fmaf(a, hh[j], du * s_x[R + n0 + j]);
        part = fmaf(s_x[R + N + n0 + j], hn[j], part);
      }
      *reinterpret_cast<float4*>(hs + n0) = make_float4(hn[0], hn[1], hn[2], hn[3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = 4 * q + j;
      if (n < N) {
        const float a2 = -__builtin_amdgcn_exp2f(al[n] * kLog2e) * kLog2e;
        const float a = __builtin_amdgcn_exp2f(delta * a2);
        const float hn = fmaf(a, hs[n], du * s_x[R + n]);
        hs[n] = hn;
        part = fmaf(s_x[R + N + n], hn, part);
      }
    }
  }
#pragma unroll
  for (int m = NQ / 2; m >= 1; m /= 2) part += __shfl_xor(part, m, NQ);
  if (q == 0) {
    float yv = fmaf(dskip, uv, part);
    yv *= silu(zin.at(b, zcol + d));
    y[ch] = yv;
  }
}

hipError_t launch_residual_rmsnorm(float* h, const PartsView& add, const float* w, float eps, void* out,
                                   int rows, int Dm, hipStream_t s) {
  const dim3 grid((unsigned)rows);
  if (add.ks > kSplitKMaxSlices || Dm > 8 * 256)
    residual_rmsnorm_wide_kernel<<<grid, 256, 0, s>>>(h, add, w, eps, static_cast<bf16*>(out), Dm);
  else if (Dm <= 3 * 256)
    residual_rmsnorm_kernel<3><<<grid, 256, 0, s>>>(h, add, w, eps, static_cast<bf16*>(out), Dm);
  else
    residual_rmsnorm_kernel<8><<<grid, 256, 0, s>>>(h, add, w, eps, static_cast<bf16*>(out), Dm);
  return hipGetLastError();
}

hipError_t launch_decode_conv(const PartsView& xin, const float* conv_w, const float* conv_b,
                              float* conv_state, float* u, int B, int D, int K, hipStream_t s) {
  const dim3 grid((unsigned)((D + 255) / 256), (unsigned)B);
  if (K == 4 && ((reinterpret_cast<uintptr_t>(conv_w) | reinterpret_cast<uintptr_t>(conv_state)) & 15) == 0)
    decode_conv_kernel<true><<<grid, 256, 0, s>>>(xin, conv_w, conv_b, conv_state, u, D, K);
  else
    decode_conv_kernel<false><<<grid, 256, 0, s>>>(xin, conv_w, conv_b, conv_state, u, D, K);
  return hipGetLastError();
}

hipError_t launch_decode_conv_xproj(const PartsView& xin, const float* conv_w, const float* conv_b,
                                    float* conv_state, float* u, const void* Wx, int xw, float* part,
                                    PartsView* out, int B, int D, int K, hipStream_t s) {
  if (D % kConvXC != 0 || B > kSplitKMaxM || (reinterpret_cast<uintptr_t>(Wx) & 15) != 0)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(D / kConvXC), (unsigned)((B + kConvXRows - 1) / kConvXRows));
  const bf16* w = static_cast<const bf16*>(Wx);
  if (K == 4 && ((reinterpret_cast<uintptr_t>(conv_w) | reinterpret_cast<uintptr_t>(conv_state)) & 15) == 0)
    decode_conv_xproj_kernel<true><<<grid, 256, 0, s>>>(xin, conv_w, conv_b, conv_state, u, w, xw, part, B, D, K);
  else
    decode_conv_xproj_kernel<false><<<grid, 256, 0, s>>>(xin, conv_w, conv_b, conv_state, u, w, xw, part, B, D,
                                                         K);
  *out = PartsView{part, D / kConvXC, (int64_t)B * xw, xw};
  return hipGetLastError();
}

hipError_t launch_decode_ssm(const float* u, const PartsView& xd, const void* Wdt, int R, const float* dt_bias,
                             const float* A_log, const float* D_skip, const PartsView& zin, int zcol,
                             float* state, float* y, int B, int D, int N, hipStream_t s) {
  if (R + 2 * N > kDecodeMaxXProj || N > 64) return hipErrorInvalidValue;
  const int q = (N + 3) / 4;
  const int NQ = q <= 1 ? 1 : q <= 2 ? 2 : q <= 4 ? 4 : q <= 8 ? 8 : 16;
  const dim3 grid((unsigned)(((int64_t)D * NQ + 255) / 256), (unsigned)B);
  const bf16* w = static_cast<const bf16*>(Wdt);
  // 8-byte loads of W_dt when every lane's run of columns is whole groups of four, aligned
  const bool vec4 = R % (4 * NQ) == 0 && reinterpret_cast<uintptr_t>(Wdt) % 8 == 0 && N % 4 == 0 &&
                    ((reinterpret_cast<uintptr_t>(state) | reinterpret_cast<uintptr_t>(A_log)) & 15) == 0;
#define MAMBA_DECODE_SSM(NQV)                                                                         \
  if (vec4)                                                                                           \
    decode_ssm_kernel<NQV, true><<<grid, 256, 0, s>>>(u, xd, w, R, dt_bias, A_log, D_skip, zin, zcol, \
                                                      state, y, D, N);                                \
  else                                                                                                \
    decode_ssm_kernel<NQV, false><<<grid, 256, 0, s>>>(u, xd, w, R, dt_bias, A_log, D_skip, zin, zcol, \
                                                       state, y, D, N)
  switch (NQ) {
    case 1: MAMBA_DECODE_SSM(1); break;
    case 2: MAMBA_DECODE_SSM(2); break;
    case 4: MAMBA_DECODE_SSM(4); break;
    case 8: MAMBA_DECODE_SSM(8); break;
    default: MAMBA_DECODE_SSM(16); break;
  }
#undef MAMBA_DECODE_SSM
  return hipGetLastError();
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
