// launch.hpp -- validated argument bundles passed from the C-ABI layer to the kernel launchers.
// The ABI layer (abi.cpp) checks every field before a launcher sees it; launchers only pick
// a launch shape and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct mamba_backbone_dims;
struct mamba_backbone_weights;

namespace mamba {

// Opaque 2-byte storage unit for bf16 arrays in host code (pointer arithmetic only).
struct bf16_storage {
  unsigned short bits;
};

struct ConvFwdArgs {
  const void* x;
  int64_t x_row_stride;
  const float* conv_w;
  const float* conv_b;
  float* conv_state;
  void* u;
  bool bf16;
  int B, T, D, K;
  // per-sequence valid lengths (device, [B], clamped to [0, T]) or NULL: the new conv state
  // is taken after each sequence's own last token
  const int32_t* lengths = nullptr;
};

struct ConvStepArgs {
  const void* x;
  int64_t x_row_stride;
  const float* conv_w;
  const float* conv_b;
  float* conv_state;
  void* u;
  bool bf16;
  int L, B, D, K;
};

struct ScanFwdArgs {
  const void* u;
  const void* dt;
  const float* dt_bias;
  bool delta_softplus;
  const float* A_log;
  const void* Bm;
  const void* Cm;
  int64_t bc_row_stride;
  const float* D_skip;
  const void* z;
  int64_t z_row_stride;
  const float* state_in;
  float* state_out;
  void* y;
  bool bf16;
  int B, T, D, N;
  void* workspace;
  // fused conv (x != NULL): u is computed from x in the kernel and optionally written
  const void* x = nullptr;
  int64_t x_row_stride = 0;
  const float* conv_w = nullptr;
  const float* conv_b = nullptr;
  float* conv_state = nullptr;
  void* u_out = nullptr;
  int K = 0;
  // per-sequence valid lengths (device, [B], clamped to [0, T]) or NULL: each sequence's
  // states are taken after its own last token; y past it is not written
  const int32_t* lengths = nullptr;
  // f32 I/O with u as an input only: y stored as bf16 (rounded to nearest even), for a
  // consumer that reads it as a bf16 operand (the backbone's out_proj)
  bool y_bf16 = false;
};

struct SsmStepArgs {
  const void* u;
  const void* dt;
  const float* dt_bias;
  bool delta_softplus;
  const float* A_log;
  const void* Bm;
  const void* Cm;
  int64_t bc_row_stride;
  const float* D_skip;
  const void* z;
  int64_t z_row_stride;
  float* state;
  void* y;
  bool bf16;
  int L, B, D, N;
};

// How the prefill scan splits T into chunks for one shape; the workspace size and the
// kernels both derive from this, so they always agree.
struct ScanPlan {
  int chunks;      // number of T chunks (1 = no cross-chunk carry, no workspace)
  int chunk_t;     // tokens per chunk (the last chunk may be shorter)
  size_t workspace_bytes;
};

ScanPlan plan_selective_scan(int B, int T, int D, int N);

// Size of the library's fixed device scratch (noalloc.hip), the workspace of the entry points
// that allocate nothing. The scan planner makes more than one chunk only while B * d_inner is
// at most 24576, with B * chunks * d_inner at most 49152, so its workspace is bounded by
// 983040 + 294912 * d_state bytes: every shape with d_state <= 53 fits.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;

// The fixed scratch's device address on the current device, looked up on the first call per
// device and kept.
hipError_t noalloc_scratch(void** out);

// Largest conv width the kernels take.
constexpr int kMaxConvK = 8;

struct DecodeStepArgs {
  const void* x;
  int64_t x_row_stride;
  const float* conv_w;
  const float* conv_b;
  float* conv_state;
  const void* dt;
  const float* dt_bias;
  bool delta_softplus;
  const float* A_log;
  const void* Bm;
  const void* Cm;
  int64_t bc_row_stride;
  const float* D_skip;
  const void* z;
  int64_t z_row_stride;
  float* ssm_state;
  void* u;  // optional
  void* y;
  bool bf16;
  int L, B, D, K, N;
};
hipError_t launch_decode_step(const DecodeStepArgs& a, hipStream_t s);

// Mamba-3 SISO decode step (phases F3-F7) for L layers and B sequences: one in_proj row per
// (layer, sequence), per-layer parameters, the four states updated in place.
constexpr int kM3MaxDState = 256;
constexpr int kM3MaxHeadDim = 256;
constexpr int64_t kM3MaxBlocks = 0x7fffffff;
struct M3StepArgs {
  const float* proj;        // [L][B] rows of proj_row_stride floats
  int64_t proj_row_stride;
  const float* dt_bias;     // [L][nh]
  const float* b_norm_w;    // [L][ds]
  const float* c_norm_w;    // [L][ds]
  const float* b_bias;      // [L][nh][ds]
  const float* c_bias;      // [L][nh][ds]
  const float* D;           // [L][nh]
  const float* gate_w;      // [L][nh * hd] or NULL (plain silu gate)
  float a_floor;
  float* ssm;               // [L][B][nh][hd][ds], 16-byte aligned
  float* k_state;           // [L][B][nh][ds]
  float* v_state;           // [L][B][nh][hd]
  float* angle;             // [L][B][nh][angle_stride]
  int angle_stride;         // max(na, 1)
  float* out;               // [L][B][nh * hd]
  int L, B, nh, hd, ds, ng, na;
};
hipError_t launch_m3_siso_step(const M3StepArgs& a, hipStream_t s);

hipError_t launch_embed_gather(const int32_t* tokens, const void* E, float* out, int64_t rows,
                               int vocab, int Dm, hipStream_t s);
hipError_t launch_rmsnorm(const float* x, int64_t x_row_stride, const float* w, float eps,
                          void* out, bool out_bf16, int64_t rows, int Dm, hipStream_t s);
// RMSNorm of row (b * T + clamp(lengths[b], 1, T) - 1) of x for b < B: each sequence's last
// valid position.
hipError_t launch_rmsnorm_last(const float* x, const int32_t* lengths, int T, const float* w,
                               float eps, void* out, bool out_bf16, int B, int Dm, hipStream_t s);
hipError_t launch_gemm_bf16(const void* A, bool a_bf16, int64_t lda, const void* W, int64_t ldw,
                            float* C, int64_t ldc, int M, int N, int K, bool accumulate,
                            hipStream_t s);
// Largest M the few-row GEMM takes, and its LDS budget for the staged rows (M * K floats).
constexpr int kSkinnyGemmMaxM = 8;
constexpr int64_t kSkinnyGemmMaxLds = 64 * 1024;
// Split-K GEMM for a decode batch (M <= kSplitKMaxM rows): the number of K slices for a
// shape, and the launcher, which needs gemm_splitk_slices(M, N, K) * M * N floats of scratch.
constexpr int kSplitKMaxM = 64;
constexpr int kSplitKMaxSlices = 8;  // the readers of the partial planes add them one by one
int gemm_splitk_slices(int M, int N, int K);

// The result of a product that may be split over K: value(r, c) = sum over z < ks of
// p[z * plane + r * ld + c], added in order z = 0, 1, ... (ks = 1, plane = 0 for a product
// written whole; ks = 0 when it was added into its destination already).
struct PartsView {
  const float* p;
  int ks;
  int64_t plane, ld;
  __host__ __device__ float at(int64_t r, int64_t c) const {
    const float* q = p + r * ld + c;
    float v = 0.0f;
    int z = 0;
    for (; z + 4 <= ks; z += 4) {  // four loads in flight, added in order
      float t[4];
      for (int i = 0; i < 4; ++i) t[i] = q[(z + i) * plane];
      for (int i = 0; i < 4; ++i) v += t[i];
    }
    for (; z < ks; ++z) v += q[z * plane];
    return v;
  }
};
// C (+)= A W^T for a decode batch, left as split-K partial planes in `partial` (no reduction
// kernel) or, when not split, written to (added into) C; *out describes where the result is.
hipError_t launch_gemm_bf16_parts(const void* A, bool a_bf16, int64_t lda, const void* W,
                                  int64_t ldw, float* C, int64_t ldc, int M, int N, int K,
                                  bool accumulate, float* partial, PartsView* out, hipStream_t s);
// Widest x_proj row (dt_rank + 2 d_state) the decode step's SSM kernel stages in LDS.
constexpr int kDecodeMaxXProj = 1024;
// Decode-step consumers of split-K results: residual add + RMSNorm, conv step on the x lane,
// and the SSM step with dt_proj folded in.
hipError_t launch_residual_rmsnorm(float* h, const PartsView& add, const float* w, float eps, void* out,
                                   int rows, int Dm, hipStream_t s);
hipError_t launch_decode_conv(const PartsView& xin, const float* conv_w, const float* conv_b,
                              float* conv_state, float* u, int B, int D, int K, hipStream_t s);
// Conv step + x_proj of a decode layer in one launch (D a multiple of kConvXC, B <= kSplitKMaxM,
// 16-byte aligned W_x): u and the conv state as launch_decode_conv, and x_proj left as
// D / kConvXC partial planes in `part` (*out describes them).
constexpr int kConvXC = 64;     // channels per x_proj slice
constexpr int kConvXRows = 4;   // sequences per workgroup
constexpr int kConvXOut = 4;    // x_proj outputs a thread accumulates together
hipError_t launch_decode_conv_xproj(const PartsView& xin, const float* conv_w, const float* conv_b,
                                    float* conv_state, float* u, const void* Wx, int xw, float* part,
                                    PartsView* out, int B, int D, int K, hipStream_t s);
hipError_t launch_decode_ssm(const float* u, const PartsView& xd, const void* Wdt, int R, const float* dt_bias,
                             const float* A_log, const float* D_skip, const PartsView& zin, int zcol,
                             float* state, float* y, int B, int D, int N, hipStream_t s);
// C (+)= A W^T for many rows and fewer than 128 columns (a prefill's x_proj): K split into
// up to max_ks slices whose partial planes (ks * M * N floats of `partial`) are summed in
// order into C by a second kernel; one plain product when splitting does not apply.
int gemm_rows_ksplit(int M, int N, int K, int max_ks);
hipError_t launch_gemm_bf16_rows(const void* A, bool a_bf16, int64_t lda, const void* W,
                                 int64_t ldw, float* C, int64_t ldc, int M, int N, int K,
                                 bool accumulate, float* partial, int max_ks, hipStream_t s);
// A prefill's x_proj and dt_proj: xdbl = u @ W_x^T ([M, xw], dt lane | B | C) and
// dt = xdbl[:, :R] @ W_dt^T ([M, D], bias left to the scan); x_proj split over K as
// launch_gemm_bf16_rows does (partial planes in `partial`), its planes summed and dt_proj
// applied by one kernel where the shapes allow, else the two products one after the other.
// What leaves as dt: dt itself (bias NULL, softplus false), or dt + bias, then softplus
// when asked -- the scan's delta, formed in the same order as the scan forms it.
struct DtOut {
  const float* bias = nullptr;  // [D] or NULL
  bool softplus = false;
};
hipError_t launch_xproj_dtproj(const float* u, int64_t ldu, const void* Wx, float* xdbl, int xw,
                               const void* Wdt, int R, float* dt, int M, int D, float* partial,
                               int max_ks, const DtOut& o, hipStream_t s);
// The conv (as launch_conv1d_fwd with a.u f32) followed by launch_xproj_dtproj of its u,
// with the conv computed inside x_proj's split product where the shapes allow (K == 4, f32,
// d_inner a multiple of 64, xw <= 80): u and the conv state as the conv kernel leaves them.
hipError_t launch_conv_xproj_dtproj(const ConvFwdArgs& a, const void* Wx, float* xdbl, int xw,
                                    const void* Wdt, int R, float* dt, float* partial, int max_ks,
                                    const DtOut& o, hipStream_t s);
hipError_t launch_gemm_bf16_splitk(const void* A, bool a_bf16, int64_t lda, const void* W,
                                   int64_t ldw, float* C, int64_t ldc, int M, int N, int K,
                                   bool accumulate, float* partial, hipStream_t s);

hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, hipStream_t s);

size_t backbone_workspace_bytes(const mamba_backbone_dims& d, int B, int T);
// Inputs and outputs of one backbone prefill: token ids or raw input rows, optional
// per-sequence lengths, logits of each last valid token and/or norm_f rows of every position.
struct BackbonePrefillIO {
  const int32_t* tokens = nullptr;   // [B, T]
  const float* embeds = nullptr;     // [B, T, d_model]
  const int32_t* lengths = nullptr;  // [B]
  float* logits = nullptr;           // [B, vocab]
  float* hidden = nullptr;           // [B, T, d_model]
};
hipError_t run_backbone_prefill_io(const mamba_backbone_dims& d, const mamba_backbone_weights& w,
                                   const BackbonePrefillIO& io, int B, int T, float* conv_state,
                                   float* ssm_state, void* workspace, hipStream_t s);
hipError_t run_backbone_prefill(const mamba_backbone_dims& d, const mamba_backbone_weights& w,
                                const int32_t* tokens, int B, int T, float* conv_state,
                                float* ssm_state, float* logits, void* workspace, hipStream_t s);
size_t backbone_decode_workspace_bytes(const mamba_backbone_dims& d, int B);
hipError_t run_backbone_decode(const mamba_backbone_dims& d, const mamba_backbone_weights& w,
                               const int32_t* tokens, int B, float* conv_state, float* ssm_state,
                               float* logits, void* workspace, hipStream_t s);
hipError_t launch_conv1d_step(const ConvStepArgs& a, hipStream_t s);
hipError_t launch_selective_scan_fwd(const ScanFwdArgs& a, hipStream_t s);
hipError_t launch_ssm_step(const SsmStepArgs& a, hipStream_t s);

}  // namespace mamba
