// launch.hpp -- validated argument bundles passed from the C-ABI layer to the kernel launchers.
// The ABI layer (abi.cpp) checks every field before a launcher sees it; launchers only pick
// a launch shape and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mamba {

struct ConvFwdArgs {
  const void* x;
  int64_t x_row_stride;
  const float* conv_w;
  const float* conv_b;
  float* conv_state;
  void* u;
  bool bf16;
  int B, T, D, K;
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

hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, hipStream_t s);
hipError_t launch_conv1d_step(const ConvStepArgs& a, hipStream_t s);
hipError_t launch_selective_scan_fwd(const ScanFwdArgs& a, hipStream_t s);
hipError_t launch_ssm_step(const SsmStepArgs& a, hipStream_t s);

}  // namespace mamba
