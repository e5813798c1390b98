// abi.cpp -- the extern "C" boundary: argument validation, error reporting, dispatch.
//
// Every call checks all of its arguments before anything is enqueued and reports the first
// problem through a thread-local message, in the spirit of the pages' host code, which
// validates buffer sizes before a prefill so that a bad request fails before any work
// (prefill.rs page, mamba-rs 0.6.4, output-length check ahead of prefill_body) and turns
// unsupported d_state into a loud error rather than a silent early return (inference.rs
// page, mamba-rs 0.5.1, mixed chain, fused gather + step + gate guard).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/mamba_ssm.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

constexpr int kMaxN = 64;
constexpr int kMaxK = 8;
constexpr int kMaxGridYZ = 65535;
// Row strides (in elements) the kernels address with 32-bit buffer offsets over 8-row blocks.
constexpr int64_t kMaxRowStride = int64_t(1) << 24;

struct Fail {
  mamba_status status;
};

[[noreturn]] void fail(mamba_status st, const char* fn, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string(fn) + ": " + buf;
  throw Fail{st};
}

size_t elem_size(mamba_dtype t) { return t == MAMBA_BF16 ? 2 : 4; }

void check_dtype(const char* fn, mamba_dtype t) {
  if (t != MAMBA_F32 && t != MAMBA_BF16) fail(MAMBA_EINVAL, fn, "io_dtype %d is not MAMBA_F32 or MAMBA_BF16", (int)t);
}

void check_ptr(const char* fn, const char* name, const void* p, size_t align, bool required) {
  if (!p) {
    if (required) fail(MAMBA_EINVAL, fn, "%s is NULL", name);
    return;
  }
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    fail(MAMBA_EINVAL, fn, "%s (%p) is not %zu-byte aligned", name, p, align);
}

// A tensor's byte range, for overlap checks. rows of `width` elements, `stride` apart.
struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};

Range range(const char* name, const void* p, int64_t rows, int64_t stride, int64_t width,
            size_t esize) {
  if (!p || rows <= 0 || width <= 0) return {name, 0, 0};
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {name, lo, lo + (uintptr_t)(((rows - 1) * stride + width) * (int64_t)esize)};
}

void check_disjoint(const char* fn, const Range& out, std::initializer_list<Range> ins) {
  if (out.lo == out.hi) return;
  for (const Range& r : ins) {
    if (r.lo == r.hi) continue;
    if (out.lo < r.hi && r.lo < out.hi) fail(MAMBA_EINVAL, fn, "%s overlaps %s", out.name, r.name);
  }
}

void check_hip(const char* fn, hipError_t e) {
  if (e != hipSuccess) fail(MAMBA_EHIP, fn, "HIP error %d (%s)", (int)e, hipGetErrorString(e));
}

void check_dim(const char* fn, const char* name, int v) {
  if (v < 0) fail(MAMBA_EINVAL, fn, "%s = %d is negative", name, v);
}

void check_state_dim(const char* fn, const char* name, int v, int max) {
  if (v <= 0) fail(MAMBA_EINVAL, fn, "%s = %d must be at least 1", name, v);
  if (v > max) fail(MAMBA_EUNSUPPORTED, fn, "%s = %d exceeds the supported maximum %d", name, v, max);
}

template <typename F>
mamba_status guarded(F&& f) {
  try {
    f();
    g_last_error.clear();
    return MAMBA_OK;
  } catch (const Fail& e) {
    return e.status;
  }
}

}  // namespace

extern "C" {

const char* mamba_last_error(void) { return g_last_error.c_str(); }

const char* mamba_version(void) { return "mamba_selective_scan_fwd_amd 0.1.0 (gfx950)"; }

mamba_status mamba_conv1d_fwd(const void* x, int64_t x_row_stride, const float* conv_w,
                              const float* conv_b, float* conv_state, void* u,
                              mamba_dtype io_dtype, int B, int T, int D, int K, void* stream) {
  static const char* fn = "mamba_conv1d_fwd";
  return guarded([&] {
    check_dtype(fn, io_dtype);
    check_dim(fn, "B", B);
    check_dim(fn, "T", T);
    check_dim(fn, "D", D);
    check_state_dim(fn, "K", K, kMaxK);
    if (B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "B = %d exceeds %d", B, kMaxGridYZ);
    if ((int64_t)B * T == 0 || D == 0) return;
    const size_t es = elem_size(io_dtype);
    if (x_row_stride < D) fail(MAMBA_EINVAL, fn, "x_row_stride = %lld is less than D = %d", (long long)x_row_stride, D);
    if (x_row_stride > kMaxRowStride) fail(MAMBA_EUNSUPPORTED, fn, "x_row_stride = %lld exceeds %lld", (long long)x_row_stride, (long long)kMaxRowStride);
    check_ptr(fn, "x", x, es, true);
    check_ptr(fn, "conv_w", conv_w, 4, true);
    check_ptr(fn, "conv_b", conv_b, 4, false);
    check_ptr(fn, "conv_state", conv_state, 4, false);
    check_ptr(fn, "u", u, es, true);
    const int64_t rows = (int64_t)B * T;
    const Range rx = range("x", x, rows, x_row_stride, D, es);
    const Range rw = range("conv_w", conv_w, D, K, K, 4);
    const Range rb = range("conv_b", conv_b, 1, D, D, 4);
    const Range rs = range("conv_state", conv_state, (int64_t)B * D, K, K, 4);
    check_disjoint(fn, range("u", u, rows, D, D, es), {rx, rw, rb, rs});
    check_disjoint(fn, rs, {rx, rw, rb});
    mamba::ConvFwdArgs a{x, x_row_stride, conv_w, conv_b, conv_state, u, io_dtype == MAMBA_BF16,
                         B, T, D, K};
    check_hip(fn, mamba::launch_conv1d_fwd(a, static_cast<hipStream_t>(stream)));
  });
}

size_t mamba_selective_scan_workspace_size(int B, int T, int D, int N) {
  return mamba::plan_selective_scan(B, T, D, N).workspace_bytes;
}

mamba_status mamba_selective_scan_fwd(const void* u, const void* dt, const float* dt_bias,
                                      int delta_softplus, const float* A_log, const void* Bm,
                                      const void* Cm, int64_t bc_row_stride, const float* D_skip,
                                      const void* z, int64_t z_row_stride,
                                      const float* ssm_state_in, float* ssm_state_out, void* y,
                                      mamba_dtype io_dtype, int B, int T, int D, int N,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "mamba_selective_scan_fwd";
  return guarded([&] {
    check_dtype(fn, io_dtype);
    check_dim(fn, "B", B);
    check_dim(fn, "T", T);
    check_dim(fn, "D", D);
    check_state_dim(fn, "N", N, kMaxN);
    if (B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "B = %d exceeds %d", B, kMaxGridYZ);
    if (B == 0 || D == 0) return;
    const size_t es = elem_size(io_dtype);
    check_ptr(fn, "ssm_state_in", ssm_state_in, 4, false);
    check_ptr(fn, "ssm_state_out", ssm_state_out, 4, false);
    const int64_t nstate = (int64_t)B * D * N;
    const Range rsi = range("ssm_state_in", ssm_state_in, 1, nstate, nstate, 4);
    const Range rso = range("ssm_state_out", ssm_state_out, 1, nstate, nstate, 4);
    if (ssm_state_in != ssm_state_out) check_disjoint(fn, rso, {rsi});
    if (T == 0) {
      check_hip(fn, mamba::launch_selective_scan_fwd(
                        mamba::ScanFwdArgs{u, dt, dt_bias, delta_softplus != 0, A_log, Bm, Cm,
                                           bc_row_stride, D_skip, z, z_row_stride, ssm_state_in,
                                           ssm_state_out, y, io_dtype == MAMBA_BF16, B, T, D, N,
                                           workspace},
                        static_cast<hipStream_t>(stream)));
      return;
    }
    if (bc_row_stride < N) fail(MAMBA_EINVAL, fn, "bc_row_stride = %lld is less than N = %d", (long long)bc_row_stride, N);
    if (z && z_row_stride < D) fail(MAMBA_EINVAL, fn, "z_row_stride = %lld is less than D = %d", (long long)z_row_stride, D);
    if (D > kMaxRowStride || (z && z_row_stride > kMaxRowStride))
      fail(MAMBA_EUNSUPPORTED, fn, "D or z_row_stride exceeds %lld elements", (long long)kMaxRowStride);
    check_ptr(fn, "u", u, es, true);
    check_ptr(fn, "dt", dt, es, true);
    check_ptr(fn, "dt_bias", dt_bias, 4, false);
    check_ptr(fn, "A_log", A_log, 4, true);
    check_ptr(fn, "Bm", Bm, es, true);
    check_ptr(fn, "Cm", Cm, es, true);
    check_ptr(fn, "D_skip", D_skip, 4, false);
    check_ptr(fn, "z", z, es, false);
    check_ptr(fn, "y", y, es, true);
    const size_t need = mamba::plan_selective_scan(B, T, D, N).workspace_bytes;
    if (need > 0) {
      if (!workspace) fail(MAMBA_EWORKSPACE, fn, "workspace is NULL but %zu bytes are required", need);
      if (workspace_bytes < need) fail(MAMBA_EWORKSPACE, fn, "workspace_bytes = %zu but %zu are required", workspace_bytes, need);
      if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) fail(MAMBA_EINVAL, fn, "workspace is not 256-byte aligned");
    }
    const int64_t rows = (int64_t)B * T;
    const Range ru = range("u", u, rows, D, D, es);
    const Range rdt = range("dt", dt, rows, D, D, es);
    const Range rdb = range("dt_bias", dt_bias, 1, D, D, 4);
    const Range ra = range("A_log", A_log, D, N, N, 4);
    const Range rB = range("Bm", Bm, rows, bc_row_stride, N, es);
    const Range rC = range("Cm", Cm, rows, bc_row_stride, N, es);
    const Range rD = range("D_skip", D_skip, 1, D, D, 4);
    const Range rz = range("z", z, rows, z_row_stride, D, es);
    const Range rws = range("workspace", need ? workspace : nullptr, 1, (int64_t)need, (int64_t)need, 1);
    const Range ry = range("y", y, rows, D, D, es);
    check_disjoint(fn, ry, {ru, rdt, rdb, ra, rB, rC, rD, rz, rsi, rso, rws});
    check_disjoint(fn, rso, {ru, rdt, rdb, ra, rB, rC, rD, rz, rws});
    check_disjoint(fn, rws, {ru, rdt, rdb, ra, rB, rC, rD, rz, rsi});
    mamba::ScanFwdArgs a{u, dt, dt_bias, delta_softplus != 0, A_log, Bm, Cm, bc_row_stride,
                         D_skip, z, z_row_stride, ssm_state_in, ssm_state_out, y,
                         io_dtype == MAMBA_BF16, B, T, D, N, workspace};
    check_hip(fn, mamba::launch_selective_scan_fwd(a, static_cast<hipStream_t>(stream)));
  });
}

}  // extern "C"

namespace {

// mamba_conv_scan_fwd's checks and launch, shared with its no-allocation variant; fn names
// the entry point in error messages.
void conv_scan_fwd(const char* fn, const void* x, int64_t x_row_stride, const float* conv_w,
                   const float* conv_b, float* conv_state, const void* dt, const float* dt_bias,
                   int delta_softplus, const float* A_log, const void* Bm, const void* Cm,
                   int64_t bc_row_stride, const float* D_skip, const void* z,
                   int64_t z_row_stride, const float* ssm_state_in, float* ssm_state_out, void* u,
                   void* y, mamba_dtype io_dtype, int B, int T, int D, int K, int N,
                   void* workspace, size_t workspace_bytes, void* stream) {
  check_dtype(fn, io_dtype);
  check_dim(fn, "B", B);
  check_dim(fn, "T", T);
  check_dim(fn, "D", D);
  check_state_dim(fn, "K", K, kMaxK);
  check_state_dim(fn, "N", N, kMaxN);
  if (B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "B = %d exceeds %d", B, kMaxGridYZ);
  if (B == 0 || D == 0) return;
  const size_t es = elem_size(io_dtype);
  check_ptr(fn, "ssm_state_in", ssm_state_in, 4, false);
  check_ptr(fn, "ssm_state_out", ssm_state_out, 4, false);
  check_ptr(fn, "conv_state", conv_state, 4, false);
  const int64_t nstate = (int64_t)B * D * N;
  const Range rsi = range("ssm_state_in", ssm_state_in, 1, nstate, nstate, 4);
  const Range rso = range("ssm_state_out", ssm_state_out, 1, nstate, nstate, 4);
  const Range rcs = range("conv_state", conv_state, (int64_t)B * D, K, K, 4);
  if (ssm_state_in != ssm_state_out) check_disjoint(fn, rso, {rsi});
  check_disjoint(fn, rcs, {rsi, rso});
  if (T == 0) {  // both states pass through (the conv state is unchanged)
    check_hip(fn, mamba::launch_selective_scan_fwd(
                      mamba::ScanFwdArgs{nullptr, nullptr, dt_bias, delta_softplus != 0, A_log, Bm,
                                         Cm, bc_row_stride, D_skip, z, z_row_stride, ssm_state_in,
                                         ssm_state_out, y, io_dtype == MAMBA_BF16, B, T, D, N,
                                         workspace},
                      static_cast<hipStream_t>(stream)));
    return;
  }
  if (x_row_stride < D) fail(MAMBA_EINVAL, fn, "x_row_stride = %lld is less than D = %d", (long long)x_row_stride, D);
  if (bc_row_stride < N) fail(MAMBA_EINVAL, fn, "bc_row_stride = %lld is less than N = %d", (long long)bc_row_stride, N);
  if (z && z_row_stride < D) fail(MAMBA_EINVAL, fn, "z_row_stride = %lld is less than D = %d", (long long)z_row_stride, D);
  if (D > kMaxRowStride || x_row_stride > kMaxRowStride || (z && z_row_stride > kMaxRowStride))
    fail(MAMBA_EUNSUPPORTED, fn, "D or a row stride exceeds %lld elements", (long long)kMaxRowStride);
  check_ptr(fn, "x", x, es, true);
  check_ptr(fn, "conv_w", conv_w, 4, true);
  check_ptr(fn, "conv_b", conv_b, 4, false);
  check_ptr(fn, "dt", dt, es, true);
  check_ptr(fn, "dt_bias", dt_bias, 4, false);
  check_ptr(fn, "A_log", A_log, 4, true);
  check_ptr(fn, "Bm", Bm, es, true);
  check_ptr(fn, "Cm", Cm, es, true);
  check_ptr(fn, "D_skip", D_skip, 4, false);
  check_ptr(fn, "z", z, es, false);
  check_ptr(fn, "u", u, es, false);
  check_ptr(fn, "y", y, es, true);
  const size_t need = mamba::plan_selective_scan(B, T, D, N).workspace_bytes;
  if (need > 0) {
    if (!workspace) fail(MAMBA_EWORKSPACE, fn, "workspace is NULL but %zu bytes are required", need);
    if (workspace_bytes < need) fail(MAMBA_EWORKSPACE, fn, "workspace_bytes = %zu but %zu are required", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) fail(MAMBA_EINVAL, fn, "workspace is not 256-byte aligned");
  }
  const int64_t rows = (int64_t)B * T;
  const Range rx = range("x", x, rows, x_row_stride, D, es);
  const Range rw = range("conv_w", conv_w, D, K, K, 4);
  const Range rb = range("conv_b", conv_b, 1, D, D, 4);
  const Range rdt = range("dt", dt, rows, D, D, es);
  const Range rdb = range("dt_bias", dt_bias, 1, D, D, 4);
  const Range ra = range("A_log", A_log, D, N, N, 4);
  const Range rB = range("Bm", Bm, rows, bc_row_stride, N, es);
  const Range rC = range("Cm", Cm, rows, bc_row_stride, N, es);
  const Range rD = range("D_skip", D_skip, 1, D, D, 4);
  const Range rz = range("z", z, rows, z_row_stride, D, es);
  const Range rws = range("workspace", need ? workspace : nullptr, 1, (int64_t)need, (int64_t)need, 1);
  const Range ru = range("u", u, rows, D, D, es);
  const Range ry = range("y", y, rows, D, D, es);
  check_disjoint(fn, ry, {rx, rw, rb, rcs, rdt, rdb, ra, rB, rC, rD, rz, rsi, rso, rws, ru});
  check_disjoint(fn, ru, {rx, rw, rb, rcs, rdt, rdb, ra, rB, rC, rD, rz, rsi, rso, rws});
  check_disjoint(fn, rso, {rx, rw, rb, rdt, rdb, ra, rB, rC, rD, rz, rws});
  check_disjoint(fn, rcs, {rx, rw, rb, rdt, rdb, ra, rB, rC, rD, rz, rws});
  check_disjoint(fn, rws, {rx, rw, rb, rdt, rdb, ra, rB, rC, rD, rz, rsi});
  mamba::ScanFwdArgs a{nullptr, dt, dt_bias, delta_softplus != 0, A_log, Bm, Cm, bc_row_stride,
                       D_skip, z, z_row_stride, ssm_state_in, ssm_state_out, y,
                       io_dtype == MAMBA_BF16, B, T, D, N, workspace};
  a.x = x;
  a.x_row_stride = x_row_stride;
  a.conv_w = conv_w;
  a.conv_b = conv_b;
  a.conv_state = conv_state;
  a.u_out = u;
  a.K = K;
  check_hip(fn, mamba::launch_selective_scan_fwd(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

mamba_status mamba_conv_scan_fwd(const void* x, int64_t x_row_stride, const float* conv_w,
                                 const float* conv_b, float* conv_state, const void* dt,
                                 const float* dt_bias, int delta_softplus, const float* A_log,
                                 const void* Bm, const void* Cm, int64_t bc_row_stride,
                                 const float* D_skip, const void* z, int64_t z_row_stride,
                                 const float* ssm_state_in, float* ssm_state_out, void* u, void* y,
                                 mamba_dtype io_dtype, int B, int T, int D, int K, int N,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&] {
    conv_scan_fwd("mamba_conv_scan_fwd", x, x_row_stride, conv_w, conv_b, conv_state, dt, dt_bias,
                  delta_softplus, A_log, Bm, Cm, bc_row_stride, D_skip, z, z_row_stride,
                  ssm_state_in, ssm_state_out, u, y, io_dtype, B, T, D, K, N, workspace,
                  workspace_bytes, stream);
  });
}

mamba_status mamba_conv_scan_fwd_noalloc(const void* x, int64_t x_row_stride, const float* conv_w,
                                         const float* conv_b, float* conv_state, const void* dt,
                                         const float* dt_bias, int delta_softplus,
                                         const float* A_log, const void* Bm, const void* Cm,
                                         int64_t bc_row_stride, const float* D_skip,
                                         const void* z, int64_t z_row_stride,
                                         const float* ssm_state_in, float* ssm_state_out, void* u,
                                         void* y, mamba_dtype io_dtype, int B, int T, int D, int K,
                                         int N, void* stream) {
  static const char* fn = "mamba_conv_scan_fwd_noalloc";
  return guarded([&] {
    check_dim(fn, "B", B);
    check_dim(fn, "T", T);
    check_dim(fn, "D", D);
    check_state_dim(fn, "N", N, kMaxN);
    void* ws = nullptr;
    const size_t need = mamba::plan_selective_scan(B, T, D, N).workspace_bytes;
    if (need > mamba::kNoAllocScratchBytes)
      fail(MAMBA_EWORKSPACE, fn,
           "this shape needs %zu bytes of scratch, more than the %zu of the library's fixed "
           "scratch; call mamba_conv_scan_fwd with a workspace instead",
           need, mamba::kNoAllocScratchBytes);
    if (need > 0) check_hip(fn, mamba::noalloc_scratch(&ws));
    conv_scan_fwd(fn, x, x_row_stride, conv_w, conv_b, conv_state, dt, dt_bias, delta_softplus,
                  A_log, Bm, Cm, bc_row_stride, D_skip, z, z_row_stride, ssm_state_in,
                  ssm_state_out, u, y, io_dtype, B, T, D, K, N, ws, need > 0 ? mamba::kNoAllocScratchBytes : 0,
                  stream);
  });
}

mamba_status mamba_conv1d_step(const void* x, int64_t x_row_stride, const float* conv_w,
                               const float* conv_b, float* conv_state, void* u,
                               mamba_dtype io_dtype, int L, int B, int D, int K, void* stream) {
  static const char* fn = "mamba_conv1d_step";
  return guarded([&] {
    check_dtype(fn, io_dtype);
    check_dim(fn, "L", L);
    check_dim(fn, "B", B);
    check_dim(fn, "D", D);
    check_state_dim(fn, "K", K, kMaxK);
    if ((int64_t)L * B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "L*B = %lld exceeds %d", (long long)L * B, kMaxGridYZ);
    if ((int64_t)L * B == 0 || D == 0) return;
    const size_t es = elem_size(io_dtype);
    if (x_row_stride < D) fail(MAMBA_EINVAL, fn, "x_row_stride = %lld is less than D = %d", (long long)x_row_stride, D);
    check_ptr(fn, "x", x, es, true);
    check_ptr(fn, "conv_w", conv_w, 4, true);
    check_ptr(fn, "conv_b", conv_b, 4, false);
    check_ptr(fn, "conv_state", conv_state, 4, true);
    check_ptr(fn, "u", u, es, true);
    const int64_t rows = (int64_t)L * B;
    const Range rx = range("x", x, rows, x_row_stride, D, es);
    const Range rw = range("conv_w", conv_w, (int64_t)L * D, K, K, 4);
    const Range rb = range("conv_b", conv_b, L, D, D, 4);
    const Range rs = range("conv_state", conv_state, rows * D, K, K, 4);
    check_disjoint(fn, range("u", u, rows, D, D, es), {rx, rw, rb, rs});
    check_disjoint(fn, rs, {rx, rw, rb});
    mamba::ConvStepArgs a{x, x_row_stride, conv_w, conv_b, conv_state, u, io_dtype == MAMBA_BF16,
                          L, B, D, K};
    check_hip(fn, mamba::launch_conv1d_step(a, static_cast<hipStream_t>(stream)));
  });
}

mamba_status mamba_ssm_step(const void* u, const void* dt, const float* dt_bias,
                            int delta_softplus, const float* A_log, const void* Bm,
                            const void* Cm, int64_t bc_row_stride, const float* D_skip,
                            const void* z, int64_t z_row_stride, float* ssm_state, void* y,
                            mamba_dtype io_dtype, int L, int B, int D, int N, void* stream) {
  static const char* fn = "mamba_ssm_step";
  return guarded([&] {
    check_dtype(fn, io_dtype);
    check_dim(fn, "L", L);
    check_dim(fn, "B", B);
    check_dim(fn, "D", D);
    check_state_dim(fn, "N", N, kMaxN);
    if ((int64_t)L * B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "L*B = %lld exceeds %d", (long long)L * B, kMaxGridYZ);
    if ((int64_t)L * B == 0 || D == 0) return;
    const size_t es = elem_size(io_dtype);
    if (bc_row_stride < N) fail(MAMBA_EINVAL, fn, "bc_row_stride = %lld is less than N = %d", (long long)bc_row_stride, N);
    if (z && z_row_stride < D) fail(MAMBA_EINVAL, fn, "z_row_stride = %lld is less than D = %d", (long long)z_row_stride, D);
    check_ptr(fn, "u", u, es, true);
    check_ptr(fn, "dt", dt, es, true);
    check_ptr(fn, "dt_bias", dt_bias, 4, false);
    check_ptr(fn, "A_log", A_log, 4, true);
    check_ptr(fn, "Bm", Bm, es, true);
    check_ptr(fn, "Cm", Cm, es, true);
    check_ptr(fn, "D_skip", D_skip, 4, false);
    check_ptr(fn, "z", z, es, false);
    check_ptr(fn, "ssm_state", ssm_state, 4, true);
    check_ptr(fn, "y", y, es, true);
    const int64_t rows = (int64_t)L * B;
    const Range ru = range("u", u, rows, D, D, es);
    const Range rdt = range("dt", dt, rows, D, D, es);
    const Range rdb = range("dt_bias", dt_bias, L, D, D, 4);
    const Range ra = range("A_log", A_log, (int64_t)L * D, N, N, 4);
    const Range rB = range("Bm", Bm, rows, bc_row_stride, N, es);
    const Range rC = range("Cm", Cm, rows, bc_row_stride, N, es);
    const Range rD = range("D_skip", D_skip, L, D, D, 4);
    const Range rz = range("z", z, rows, z_row_stride, D, es);
    const Range rs = range("ssm_state", ssm_state, rows * D, N, N, 4);
    check_disjoint(fn, range("y", y, rows, D, D, es), {ru, rdt, rdb, ra, rB, rC, rD, rz, rs});
    check_disjoint(fn, rs, {ru, rdt, rdb, ra, rB, rC, rD, rz});
    mamba::SsmStepArgs a{u, dt, dt_bias, delta_softplus != 0, A_log, Bm, Cm, bc_row_stride,
                         D_skip, z, z_row_stride, ssm_state, y, io_dtype == MAMBA_BF16, L, B, D,
                         N};
    check_hip(fn, mamba::launch_ssm_step(a, static_cast<hipStream_t>(stream)));
  });
}

mamba_status mamba_decode_step(const void* x, int64_t x_row_stride, const float* conv_w,
                               const float* conv_b, float* conv_state, const void* dt,
                               const float* dt_bias, int delta_softplus, const float* A_log,
                               const void* Bm, const void* Cm, int64_t bc_row_stride,
                               const float* D_skip, const void* z, int64_t z_row_stride,
                               float* ssm_state, void* u, void* y, mamba_dtype io_dtype, int L,
                               int B, int D, int K, int N, void* stream) {
  static const char* fn = "mamba_decode_step";
  return guarded([&] {
    check_dtype(fn, io_dtype);
    check_dim(fn, "L", L);
    check_dim(fn, "B", B);
    check_dim(fn, "D", D);
    check_state_dim(fn, "K", K, kMaxK);
    check_state_dim(fn, "N", N, kMaxN);
    if ((int64_t)L * B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "L*B = %lld exceeds %d", (long long)L * B, kMaxGridYZ);
    if ((int64_t)L * B == 0 || D == 0) return;
    const size_t es = elem_size(io_dtype);
    if (x_row_stride < D) fail(MAMBA_EINVAL, fn, "x_row_stride = %lld is less than D = %d", (long long)x_row_stride, D);
    if (bc_row_stride < N) fail(MAMBA_EINVAL, fn, "bc_row_stride = %lld is less than N = %d", (long long)bc_row_stride, N);
    if (z && z_row_stride < D) fail(MAMBA_EINVAL, fn, "z_row_stride = %lld is less than D = %d", (long long)z_row_stride, D);
    check_ptr(fn, "x", x, es, true);
    check_ptr(fn, "conv_w", conv_w, 4, true);
    check_ptr(fn, "conv_b", conv_b, 4, false);
    check_ptr(fn, "conv_state", conv_state, 4, true);
    check_ptr(fn, "dt", dt, es, true);
    check_ptr(fn, "dt_bias", dt_bias, 4, false);
    check_ptr(fn, "A_log", A_log, 4, true);
    check_ptr(fn, "Bm", Bm, es, true);
    check_ptr(fn, "Cm", Cm, es, true);
    check_ptr(fn, "D_skip", D_skip, 4, false);
    check_ptr(fn, "z", z, es, false);
    check_ptr(fn, "ssm_state", ssm_state, 4, true);
    check_ptr(fn, "u", u, es, false);
    check_ptr(fn, "y", y, es, true);
    const int64_t rows = (int64_t)L * B;
    const Range rx = range("x", x, rows, x_row_stride, D, es);
    const Range rw = range("conv_w", conv_w, (int64_t)L * D, K, K, 4);
    const Range rb = range("conv_b", conv_b, L, D, D, 4);
    const Range rcs = range("conv_state", conv_state, rows * D, K, K, 4);
    const Range rdt = range("dt", dt, rows, D, D, es);
    const Range rdb = range("dt_bias", dt_bias, L, D, D, 4);
    const Range ra = range("A_log", A_log, (int64_t)L * D, N, N, 4);
    const Range rB = range("Bm", Bm, rows, bc_row_stride, N, es);
    const Range rC = range("Cm", Cm, rows, bc_row_stride, N, es);
    const Range rD = range("D_skip", D_skip, L, D, D, 4);
    const Range rz = range("z", z, rows, z_row_stride, D, es);
    const Range rss = range("ssm_state", ssm_state, rows * D, N, N, 4);
    const Range ru = range("u", u, rows, D, D, es);
    const Range ry = range("y", y, rows, D, D, es);
    check_disjoint(fn, ry, {rx, rw, rb, rcs, rdt, rdb, ra, rB, rC, rD, rz, rss, ru});
    check_disjoint(fn, ru, {rx, rw, rb, rcs, rdt, rdb, ra, rB, rC, rD, rz, rss});
    check_disjoint(fn, rss, {rx, rw, rb, rcs, rdt, rdb, ra, rB, rC, rD, rz});
    check_disjoint(fn, rcs, {rx, rw, rb, rdt, rdb, ra, rB, rC, rD, rz});
    mamba::DecodeStepArgs a{x, x_row_stride, conv_w, conv_b, conv_state, dt, dt_bias,
                            delta_softplus != 0, A_log, Bm, Cm, bc_row_stride, D_skip, z,
                            z_row_stride, ssm_state, u, y, io_dtype == MAMBA_BF16, L, B, D, K, N};
    check_hip(fn, mamba::launch_decode_step(a, static_cast<hipStream_t>(stream)));
  });
}

mamba_status mamba3_siso_step(const float* proj, int64_t proj_row_stride,
                              const mamba3_siso_params* params, float a_floor,
                              float* ssm_state, float* k_state, float* v_state,
                              float* angle_state, float* out, int L, int B, int nheads,
                              int headdim, int d_state, int ngroups, int n_angles, void* stream) {
  static const char* fn = "mamba3_siso_step";
  return guarded([&] {
    check_dim(fn, "L", L);
    check_dim(fn, "B", B);
    check_state_dim(fn, "nheads", nheads, 1 << 20);
    check_state_dim(fn, "headdim", headdim, mamba::kM3MaxHeadDim);
    check_state_dim(fn, "d_state", d_state, mamba::kM3MaxDState);
    if (ngroups < 1) fail(MAMBA_EINVAL, fn, "ngroups = %d must be at least 1", ngroups);
    if (d_state % 4 != 0) fail(MAMBA_EUNSUPPORTED, fn, "d_state = %d is not a multiple of 4", d_state);
    if (nheads % ngroups != 0) fail(MAMBA_EINVAL, fn, "nheads = %d is not a multiple of ngroups = %d", nheads, ngroups);
    if (n_angles < 0 || 2 * n_angles > d_state)
      fail(MAMBA_EINVAL, fn, "n_angles = %d is outside [0, d_state / 2 = %d]", n_angles, d_state / 2);
    const int64_t heads = (int64_t)L * B * nheads;
    if (heads > mamba::kM3MaxBlocks) fail(MAMBA_EUNSUPPORTED, fn, "L*B*nheads = %lld exceeds %lld", (long long)heads, (long long)mamba::kM3MaxBlocks);
    if (!params) fail(MAMBA_EINVAL, fn, "params is NULL");
    if (heads == 0) return;
    const int64_t di = (int64_t)nheads * headdim, gs = (int64_t)ngroups * d_state;
    const int64_t W = 2 * di + 2 * gs + 3 * (int64_t)nheads + n_angles;
    if (proj_row_stride < W) fail(MAMBA_EINVAL, fn, "proj_row_stride = %lld is less than the row width %lld", (long long)proj_row_stride, (long long)W);
    if (proj_row_stride > kMaxRowStride) fail(MAMBA_EUNSUPPORTED, fn, "proj_row_stride = %lld exceeds %lld", (long long)proj_row_stride, (long long)kMaxRowStride);
    check_ptr(fn, "proj", proj, 4, true);
    check_ptr(fn, "params->dt_bias", params->dt_bias, 4, true);
    check_ptr(fn, "params->b_norm_w", params->b_norm_w, 4, true);
    check_ptr(fn, "params->c_norm_w", params->c_norm_w, 4, true);
    check_ptr(fn, "params->b_bias", params->b_bias, 4, true);
    check_ptr(fn, "params->c_bias", params->c_bias, 4, true);
    check_ptr(fn, "params->D", params->D, 4, true);
    check_ptr(fn, "params->gate_norm_w", params->gate_norm_w, 4, false);
    check_ptr(fn, "ssm_state", ssm_state, 16, true);
    check_ptr(fn, "k_state", k_state, 4, true);
    check_ptr(fn, "v_state", v_state, 4, true);
    check_ptr(fn, "angle_state", angle_state, 4, true);
    check_ptr(fn, "out", out, 4, true);
    const int64_t rows = (int64_t)L * B;
    const int na1 = n_angles > 0 ? n_angles : 1;
    const Range rp = range("proj", proj, rows, proj_row_stride, W, 4);
    const Range r1 = range("params->dt_bias", params->dt_bias, L, nheads, nheads, 4);
    const Range r2 = range("params->b_norm_w", params->b_norm_w, L, d_state, d_state, 4);
    const Range r3 = range("params->c_norm_w", params->c_norm_w, L, d_state, d_state, 4);
    const Range r4 = range("params->b_bias", params->b_bias, L, nheads * (int64_t)d_state, nheads * (int64_t)d_state, 4);
    const Range r5 = range("params->c_bias", params->c_bias, L, nheads * (int64_t)d_state, nheads * (int64_t)d_state, 4);
    const Range r6 = range("params->D", params->D, L, nheads, nheads, 4);
    const Range r7 = range("params->gate_norm_w", params->gate_norm_w, L, di, di, 4);
    const Range rh = range("ssm_state", ssm_state, heads * headdim, d_state, d_state, 4);
    const Range rk = range("k_state", k_state, heads, d_state, d_state, 4);
    const Range rv = range("v_state", v_state, heads, headdim, headdim, 4);
    const Range ra = range("angle_state", angle_state, heads, na1, na1, 4);
    const Range ro = range("out", out, rows, di, di, 4);
    check_disjoint(fn, ro, {rp, r1, r2, r3, r4, r5, r6, r7, rh, rk, rv, ra});
    check_disjoint(fn, rh, {rp, r1, r2, r3, r4, r5, r6, r7, rk, rv, ra});
    check_disjoint(fn, rk, {rp, r1, r2, r3, r4, r5, r6, r7, rv, ra});
    check_disjoint(fn, rv, {rp, r1, r2, r3, r4, r5, r6, r7, ra});
    check_disjoint(fn, ra, {rp, r1, r2, r3, r4, r5, r6, r7});
    mamba::M3StepArgs a{proj, proj_row_stride, params->dt_bias, params->b_norm_w, params->c_norm_w,
                        params->b_bias, params->c_bias, params->D, params->gate_norm_w, a_floor,
                        ssm_state, k_state, v_state, angle_state, na1, out, L, B, nheads, headdim,
                        d_state, ngroups, n_angles};
    check_hip(fn, mamba::launch_m3_siso_step(a, static_cast<hipStream_t>(stream)));
  });
}

mamba_status mamba_embed_gather(const int32_t* tokens, const void* E, float* out, int64_t rows,
                                int vocab, int d_model, void* stream) {
  static const char* fn = "mamba_embed_gather";
  return guarded([&] {
    if (rows < 0) fail(MAMBA_EINVAL, fn, "rows = %lld is negative", (long long)rows);
    if (vocab <= 0 || d_model <= 0) fail(MAMBA_EINVAL, fn, "vocab = %d and d_model = %d must be positive", vocab, d_model);
    if (rows == 0) return;
    if (rows > INT32_MAX) fail(MAMBA_EUNSUPPORTED, fn, "rows = %lld exceeds 2^31-1", (long long)rows);
    check_ptr(fn, "tokens", tokens, 4, true);
    check_ptr(fn, "E", E, 2, true);
    check_ptr(fn, "out", out, 4, true);
    check_disjoint(fn, range("out", out, rows, d_model, d_model, 4),
                   {range("tokens", tokens, 1, rows, rows, 4), range("E", E, vocab, d_model, d_model, 2)});
    check_hip(fn, mamba::launch_embed_gather(tokens, E, out, rows, vocab, d_model, static_cast<hipStream_t>(stream)));
  });
}

mamba_status mamba_rmsnorm(const float* x, int64_t x_row_stride, const float* w, float eps,
                           void* out, mamba_dtype out_dtype, int64_t rows, int d_model,
                           void* stream) {
  static const char* fn = "mamba_rmsnorm";
  return guarded([&] {
    check_dtype(fn, out_dtype);
    if (rows < 0 || d_model < 0) fail(MAMBA_EINVAL, fn, "rows and d_model must be non-negative");
    if (rows == 0 || d_model == 0) return;
    if (rows > INT32_MAX) fail(MAMBA_EUNSUPPORTED, fn, "rows = %lld exceeds 2^31-1", (long long)rows);
    if (x_row_stride < d_model) fail(MAMBA_EINVAL, fn, "x_row_stride = %lld is less than d_model = %d", (long long)x_row_stride, d_model);
    if (!(eps >= 0.0f)) fail(MAMBA_EINVAL, fn, "eps must be a non-negative number");
    const size_t es = elem_size(out_dtype);
    check_ptr(fn, "x", x, 4, true);
    check_ptr(fn, "w", w, 4, false);
    check_ptr(fn, "out", out, es, true);
    check_disjoint(fn, range("out", out, rows, d_model, d_model, es),
                   {range("x", x, rows, x_row_stride, d_model, 4), range("w", w, 1, d_model, d_model, 4)});
    check_hip(fn, mamba::launch_rmsnorm(x, x_row_stride, w, eps, out, out_dtype == MAMBA_BF16, rows,
                                        d_model, static_cast<hipStream_t>(stream)));
  });
}

mamba_status mamba_gemm_bf16(const void* A, mamba_dtype a_dtype, int64_t lda, const void* W,
                             int64_t ldw, float* C, int64_t ldc, int M, int N, int K,
                             int accumulate, void* stream) {
  static const char* fn = "mamba_gemm_bf16";
  return guarded([&] {
    check_dtype(fn, a_dtype);
    check_dim(fn, "M", M);
    check_dim(fn, "N", N);
    check_dim(fn, "K", K);
    if (M == 0 || N == 0) return;
    if (lda < K || ldw < K || ldc < N) fail(MAMBA_EINVAL, fn, "leading dimensions must be at least K (A, W) and N (C)");
    if (M > 65535 * 64) fail(MAMBA_EUNSUPPORTED, fn, "M = %d exceeds %d", M, 65535 * 64);
    const size_t es = elem_size(a_dtype);
    check_ptr(fn, "A", A, es, true);
    check_ptr(fn, "W", W, 2, true);
    check_ptr(fn, "C", C, 4, true);
    check_disjoint(fn, range("C", C, M, ldc, N, 4),
                   {range("A", A, M, lda, K, es), range("W", W, N, ldw, K, 2)});
    check_hip(fn, mamba::launch_gemm_bf16(A, a_dtype == MAMBA_BF16, lda, W, ldw, C, ldc, M, N, K,
                                          accumulate != 0, static_cast<hipStream_t>(stream)));
  });
}

// x_proj's K split as the backbone prefill runs it: at most d_inner / xw slices, so that the
// partial planes fit in one [M, d_inner] buffer
static size_t xproj_dtproj_ws(int M, int D, int R, int N) {
  const int xw = R + 2 * N;
  const int ks = mamba::gemm_rows_ksplit(M, xw, D, std::max(D / xw, 1));
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)xw * sizeof(float) : 0;
}

size_t mamba_xproj_dtproj_workspace_size(int M, int d_inner, int dt_rank, int d_state) {
  if (M <= 0 || d_inner <= 0 || dt_rank <= 0 || d_state < 0) return 0;
  return xproj_dtproj_ws(M, d_inner, dt_rank, d_state);
}

mamba_status mamba_xproj_dtproj(const float* u, int64_t ldu, const void* W_x, const void* W_dt,
                                float* xdbl, float* dt, const float* dt_bias, int delta_softplus,
                                int M, int d_inner, int dt_rank, int d_state, void* workspace,
                                size_t workspace_bytes, void* stream) {
  static const char* fn = "mamba_xproj_dtproj";
  return guarded([&] {
    check_dim(fn, "M", M);
    check_dim(fn, "d_inner", d_inner);
    check_dim(fn, "dt_rank", dt_rank);
    check_dim(fn, "d_state", d_state);
    if (M == 0) return;
    if (d_inner == 0 || dt_rank == 0) fail(MAMBA_EINVAL, fn, "d_inner and dt_rank must be positive");
    if (ldu < d_inner) fail(MAMBA_EINVAL, fn, "ldu = %lld is less than d_inner = %d", (long long)ldu, d_inner);
    if (M > 65535 * 16) fail(MAMBA_EUNSUPPORTED, fn, "M = %d exceeds %d", M, 65535 * 16);
    const int xw = dt_rank + 2 * d_state;
    const size_t need = xproj_dtproj_ws(M, d_inner, dt_rank, d_state);
    if (need) {
      if (!workspace) fail(MAMBA_EWORKSPACE, fn, "workspace is NULL but %zu bytes are required", need);
      if (workspace_bytes < need) fail(MAMBA_EWORKSPACE, fn, "workspace_bytes = %zu but %zu are required", workspace_bytes, need);
      check_ptr(fn, "workspace", workspace, 4, true);
    }
    check_ptr(fn, "u", u, 4, true);
    check_ptr(fn, "W_x", W_x, 2, true);
    check_ptr(fn, "W_dt", W_dt, 2, true);
    check_ptr(fn, "xdbl", xdbl, 4, true);
    check_ptr(fn, "dt", dt, 4, true);
    check_ptr(fn, "dt_bias", dt_bias, 4, false);
    const Range ins[] = {range("u", u, M, ldu, d_inner, 4), range("W_x", W_x, xw, d_inner, d_inner, 2),
                         range("W_dt", W_dt, d_inner, dt_rank, dt_rank, 2),
                         range("dt_bias", dt_bias, 1, d_inner, d_inner, 4)};
    const Range rx = range("xdbl", xdbl, M, xw, xw, 4), rd = range("dt", dt, M, d_inner, d_inner, 4);
    check_disjoint(fn, rx, {ins[0], ins[1], ins[2], ins[3], rd});
    check_disjoint(fn, rd, {ins[0], ins[1], ins[2], ins[3]});
    if (need) {
      const Range rw = range("workspace", workspace, 1, need, need, 1);
      check_disjoint(fn, rw, {ins[0], ins[1], ins[2], ins[3], rx, rd});
    }
    mamba::DtOut o;
    o.bias = dt_bias;
    o.softplus = delta_softplus != 0;
    check_hip(fn, mamba::launch_xproj_dtproj(u, ldu, W_x, xdbl, xw, W_dt, dt_rank, dt, M, d_inner,
                                             static_cast<float*>(workspace), std::max(d_inner / xw, 1), o,
                                             static_cast<hipStream_t>(stream)));
  });
}

mamba_status mamba_conv_xproj_dtproj(const float* x, int64_t x_row_stride, const float* conv_w,
                                     const float* conv_b, float* conv_state,
                                     const int32_t* lengths, float* u, const void* W_x,
                                     const void* W_dt, float* xdbl, float* dt,
                                     const float* dt_bias, int delta_softplus, int B, int T,
                                     int d_inner, int d_conv, int dt_rank, int d_state,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "mamba_conv_xproj_dtproj";
  return guarded([&] {
    check_dim(fn, "B", B);
    check_dim(fn, "T", T);
    check_dim(fn, "d_inner", d_inner);
    check_dim(fn, "dt_rank", dt_rank);
    check_dim(fn, "d_state", d_state);
    check_state_dim(fn, "d_conv", d_conv, kMaxK);
    if (B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "B = %d exceeds %d", B, kMaxGridYZ);
    const int64_t rows = (int64_t)B * T;
    if (rows == 0) return;
    if (d_inner == 0 || dt_rank == 0) fail(MAMBA_EINVAL, fn, "d_inner and dt_rank must be positive");
    if (rows > 65535 * 16) fail(MAMBA_EUNSUPPORTED, fn, "B * T = %lld exceeds %d", (long long)rows, 65535 * 16);
    if (x_row_stride < d_inner) fail(MAMBA_EINVAL, fn, "x_row_stride = %lld is less than d_inner = %d", (long long)x_row_stride, d_inner);
    if (x_row_stride > kMaxRowStride) fail(MAMBA_EUNSUPPORTED, fn, "x_row_stride = %lld exceeds %lld", (long long)x_row_stride, (long long)kMaxRowStride);
    const int xw = dt_rank + 2 * d_state;
    const int M = (int)rows;
    const size_t need = xproj_dtproj_ws(M, d_inner, dt_rank, d_state);
    if (need) {
      if (!workspace) fail(MAMBA_EWORKSPACE, fn, "workspace is NULL but %zu bytes are required", need);
      if (workspace_bytes < need) fail(MAMBA_EWORKSPACE, fn, "workspace_bytes = %zu but %zu are required", workspace_bytes, need);
      check_ptr(fn, "workspace", workspace, 4, true);
    }
    check_ptr(fn, "x", x, 4, true);
    check_ptr(fn, "conv_w", conv_w, 4, true);
    check_ptr(fn, "conv_b", conv_b, 4, false);
    check_ptr(fn, "conv_state", conv_state, 4, false);
    check_ptr(fn, "lengths", lengths, 4, false);
    check_ptr(fn, "u", u, 4, true);
    check_ptr(fn, "W_x", W_x, 2, true);
    check_ptr(fn, "W_dt", W_dt, 2, true);
    check_ptr(fn, "xdbl", xdbl, 4, true);
    check_ptr(fn, "dt", dt, 4, true);
    check_ptr(fn, "dt_bias", dt_bias, 4, false);
    const Range rx = range("x", x, rows, x_row_stride, d_inner, 4);
    const Range rcw = range("conv_w", conv_w, d_inner, d_conv, d_conv, 4);
    const Range rcb = range("conv_b", conv_b, 1, d_inner, d_inner, 4);
    const Range rl = range("lengths", lengths, 1, B, B, 4);
    const Range rwx = range("W_x", W_x, xw, d_inner, d_inner, 2);
    const Range rwd = range("W_dt", W_dt, d_inner, dt_rank, dt_rank, 2);
    const Range rdb = range("dt_bias", dt_bias, 1, d_inner, d_inner, 4);
    const Range rs = range("conv_state", conv_state, (int64_t)B * d_inner, d_conv, d_conv, 4);
    const Range ru = range("u", u, rows, d_inner, d_inner, 4);
    const Range rxd = range("xdbl", xdbl, rows, xw, xw, 4);
    const Range rd = range("dt", dt, rows, d_inner, d_inner, 4);
    const Range rw = range("workspace", need ? workspace : nullptr, 1, (int64_t)need, (int64_t)need, 1);
    check_disjoint(fn, rs, {rx, rcw, rcb, rl, rwx, rwd, rdb});
    check_disjoint(fn, ru, {rx, rcw, rcb, rl, rwx, rwd, rdb, rs});
    check_disjoint(fn, rxd, {rx, rcw, rcb, rl, rwx, rwd, rdb, rs, ru});
    check_disjoint(fn, rd, {rx, rcw, rcb, rl, rwx, rwd, rdb, rs, ru, rxd});
    check_disjoint(fn, rw, {rx, rcw, rcb, rl, rwx, rwd, rdb, rs, ru, rxd, rd});
    mamba::ConvFwdArgs a{x, x_row_stride, conv_w, conv_b, conv_state, u, false, B, T, d_inner, d_conv};
    a.lengths = lengths;
    mamba::DtOut o;
    o.bias = dt_bias;
    o.softplus = delta_softplus != 0;
    check_hip(fn, mamba::launch_conv_xproj_dtproj(a, W_x, xdbl, xw, W_dt, dt_rank, dt,
                                                  static_cast<float*>(workspace), std::max(d_inner / xw, 1), o,
                                                  static_cast<hipStream_t>(stream)));
  });
}

static void check_backbone_dims(const char* fn, const mamba_backbone_dims* d) {
  if (!d) fail(MAMBA_EINVAL, fn, "dims is NULL");
  if (d->n_layers < 0) fail(MAMBA_EINVAL, fn, "n_layers = %d is negative", d->n_layers);
  if (d->d_model <= 0 || d->d_inner <= 0 || d->dt_rank <= 0 || d->vocab <= 0)
    fail(MAMBA_EINVAL, fn, "d_model, d_inner, dt_rank and vocab must be positive");
  check_state_dim(fn, "d_state", d->d_state, kMaxN);
  check_state_dim(fn, "d_conv", d->d_conv, kMaxK);
  if (d->vocab_padded < d->vocab) fail(MAMBA_EINVAL, fn, "vocab_padded = %d is less than vocab = %d", d->vocab_padded, d->vocab);
  if (!(d->eps >= 0.0f)) fail(MAMBA_EINVAL, fn, "eps must be a non-negative number");
  if (2LL * d->d_inner > kMaxRowStride) fail(MAMBA_EUNSUPPORTED, fn, "d_inner = %d too large", d->d_inner);
}

size_t mamba_backbone_workspace_size(const mamba_backbone_dims* dims, int B, int T) {
  if (!dims || B <= 0 || T <= 0) return 0;
  return mamba::backbone_workspace_bytes(*dims, B, T);
}

// Shared checks of the backbone calls: weights, tokens [ntok], states, logits [B, vocab] and
// a workspace of at least `need` bytes, all mutually disjoint where written.
static void check_backbone_call(const char* fn, const mamba_backbone_dims& d,
                                const mamba_backbone_weights* w, const int32_t* tokens,
                                int64_t ntok, int B, const float* conv_state,
                                const float* ssm_state, const float* logits, const void* workspace,
                                size_t workspace_bytes, size_t need) {
  if (!w) fail(MAMBA_EINVAL, fn, "weights is NULL");
  check_ptr(fn, "embed", w->embed, 2, true);
  check_ptr(fn, "norm_f", w->norm_f, 4, true);
  check_ptr(fn, "norm_w", w->norm_w, 4, d.n_layers > 0);
  check_ptr(fn, "in_proj", w->in_proj, 2, d.n_layers > 0);
  check_ptr(fn, "conv_w", w->conv_w, 4, d.n_layers > 0);
  check_ptr(fn, "conv_b", w->conv_b, 4, d.n_layers > 0);
  check_ptr(fn, "x_proj", w->x_proj, 2, d.n_layers > 0);
  check_ptr(fn, "dt_proj", w->dt_proj, 2, d.n_layers > 0);
  check_ptr(fn, "dt_bias", w->dt_bias, 4, d.n_layers > 0);
  check_ptr(fn, "A_log", w->A_log, 4, d.n_layers > 0);
  check_ptr(fn, "D_skip", w->D_skip, 4, d.n_layers > 0);
  check_ptr(fn, "out_proj", w->out_proj, 2, d.n_layers > 0);
  check_ptr(fn, "tokens", tokens, 4, true);
  check_ptr(fn, "conv_state", conv_state, 4, d.n_layers > 0);
  check_ptr(fn, "ssm_state", ssm_state, 4, d.n_layers > 0);
  check_ptr(fn, "logits", logits, 4, true);
  if (!workspace) fail(MAMBA_EWORKSPACE, fn, "workspace is NULL but %zu bytes are required", need);
  if (workspace_bytes < need) fail(MAMBA_EWORKSPACE, fn, "workspace_bytes = %zu but %zu are required", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) fail(MAMBA_EINVAL, fn, "workspace is not 256-byte aligned");
  const int64_t L = d.n_layers;
  const Range rws = range("workspace", workspace, 1, (int64_t)need, (int64_t)need, 1);
  const Range rlog = range("logits", logits, B, d.vocab, d.vocab, 4);
  const Range rcs = range("conv_state", conv_state, L * B * d.d_inner, d.d_conv, d.d_conv, 4);
  const Range rss = range("ssm_state", ssm_state, L * B * d.d_inner, d.d_state, d.d_state, 4);
  const Range rtok = range("tokens", tokens, 1, ntok, ntok, 4);
  const Range remb = range("embed", w->embed, d.vocab_padded, d.d_model, d.d_model, 2);
  check_disjoint(fn, rws, {rlog, rcs, rss, rtok, remb});
  check_disjoint(fn, rlog, {rcs, rss, rtok, remb});
  check_disjoint(fn, rcs, {rss, rtok, remb});
  check_disjoint(fn, rss, {rtok, remb});
}

mamba_status mamba_backbone_prefill(const mamba_backbone_dims* dims,
                                    const mamba_backbone_weights* w, const int32_t* tokens,
                                    int B, int T, float* conv_state, float* ssm_state,
                                    float* logits, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  static const char* fn = "mamba_backbone_prefill";
  return guarded([&] {
    check_backbone_dims(fn, dims);
    check_dim(fn, "B", B);
    check_dim(fn, "T", T);
    if (B == 0 || T == 0) return;
    if (B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "B = %d exceeds %d", B, kMaxGridYZ);
    if ((int64_t)B * T > INT32_MAX / 2) fail(MAMBA_EUNSUPPORTED, fn, "B * T too large");
    const mamba_backbone_dims& d = *dims;
    check_backbone_call(fn, d, w, tokens, (int64_t)B * T, B, conv_state, ssm_state, logits, workspace,
                        workspace_bytes, mamba::backbone_workspace_bytes(d, B, T));
    check_hip(fn, mamba::run_backbone_prefill(d, *w, tokens, B, T, conv_state, ssm_state, logits,
                                              workspace, static_cast<hipStream_t>(stream)));
  });
}

mamba_status mamba_backbone_prefill_ex(const mamba_backbone_dims* dims,
                                       const mamba_backbone_weights* w, const mamba_prefill_io* io,
                                       int B, int T, float* conv_state, float* ssm_state,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "mamba_backbone_prefill_ex";
  return guarded([&] {
    check_backbone_dims(fn, dims);
    if (!io) fail(MAMBA_EINVAL, fn, "io is NULL");
    check_dim(fn, "B", B);
    check_dim(fn, "T", T);
    if (B == 0 || T == 0) return;
    if (B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "B = %d exceeds %d", B, kMaxGridYZ);
    if ((int64_t)B * T > INT32_MAX / 2) fail(MAMBA_EUNSUPPORTED, fn, "B * T too large");
    if (!io->tokens == !io->embeds) fail(MAMBA_EINVAL, fn, "exactly one of tokens and embeds must be given");
    if (!io->logits && !io->hidden) fail(MAMBA_EINVAL, fn, "neither logits nor hidden is requested");
    const mamba_backbone_dims& d = *dims;
    const int64_t bt = (int64_t)B * T;
    check_ptr(fn, "embeds", io->embeds, 4, false);
    check_ptr(fn, "lengths", io->lengths, 4, false);
    check_ptr(fn, "hidden", io->hidden, 4, false);
    const size_t need = mamba::backbone_workspace_bytes(d, B, T);
    // the shared checks want a logits buffer and a token array: stand in the ones present
    const float* lg = io->logits ? io->logits : io->hidden;
    const int32_t* tk = io->tokens ? io->tokens : reinterpret_cast<const int32_t*>(io->embeds);
    check_backbone_call(fn, d, w, tk, io->tokens ? bt : bt * d.d_model, io->logits ? B : 0, conv_state,
                        ssm_state, lg, workspace, workspace_bytes, need);
    const Range rws = range("workspace", workspace, 1, (int64_t)need, (int64_t)need, 1);
    const Range rhid = range("hidden", io->hidden, bt, d.d_model, d.d_model, 4);
    const Range rlog = range("logits", io->logits, B, d.vocab, d.vocab, 4);
    const Range rlen = range("lengths", io->lengths, 1, B, B, 4);
    const Range remb = range("embeds", io->embeds, bt, d.d_model, d.d_model, 4);
    const int64_t L = d.n_layers;
    const Range rcs = range("conv_state", conv_state, L * B * d.d_inner, d.d_conv, d.d_conv, 4);
    const Range rss = range("ssm_state", ssm_state, L * B * d.d_inner, d.d_state, d.d_state, 4);
    check_disjoint(fn, rhid, {rws, rlog, rlen, remb, rcs, rss});
    check_disjoint(fn, rws, {rlen, remb});
    check_disjoint(fn, rlog, {rlen, remb});
    check_disjoint(fn, rcs, {rlen, remb});
    check_disjoint(fn, rss, {rlen, remb});
    mamba::BackbonePrefillIO pio{};
    pio.tokens = io->tokens;
    pio.embeds = io->embeds;
    pio.lengths = io->lengths;
    pio.logits = io->logits;
    pio.hidden = io->hidden;
    check_hip(fn, mamba::run_backbone_prefill_io(d, *w, pio, B, T, conv_state, ssm_state, workspace,
                                                 static_cast<hipStream_t>(stream)));
  });
}

size_t mamba_backbone_decode_workspace_size(const mamba_backbone_dims* dims, int B) {
  if (!dims || B <= 0) return 0;
  return mamba::backbone_decode_workspace_bytes(*dims, B);
}

static void check_decode_call(const char* fn, const mamba_backbone_dims* dims,
                              const mamba_backbone_weights* w, const int32_t* tokens, int B,
                              const float* conv_state, const float* ssm_state, const float* logits,
                              const void* workspace, size_t workspace_bytes) {
  check_backbone_dims(fn, dims);
  check_dim(fn, "B", B);
  if (B == 0) fail(MAMBA_EINVAL, fn, "B = 0");
  if ((int64_t)B > kMaxGridYZ) fail(MAMBA_EUNSUPPORTED, fn, "B = %d exceeds %d", B, kMaxGridYZ);
  if ((int64_t)dims->dt_rank + 2LL * dims->d_state > mamba::kDecodeMaxXProj)
    fail(MAMBA_EUNSUPPORTED, fn, "dt_rank + 2 d_state = %lld exceeds %d", (long long)dims->dt_rank + 2LL * dims->d_state,
         mamba::kDecodeMaxXProj);
  check_backbone_call(fn, *dims, w, tokens, B, B, conv_state, ssm_state, logits, workspace,
                      workspace_bytes, mamba::backbone_decode_workspace_bytes(*dims, B));
}

mamba_status mamba_backbone_decode_step(const mamba_backbone_dims* dims,
                                        const mamba_backbone_weights* w, const int32_t* tokens,
                                        int B, float* conv_state, float* ssm_state, float* logits,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "mamba_backbone_decode_step";
  return guarded([&] {
    check_decode_call(fn, dims, w, tokens, B, conv_state, ssm_state, logits, workspace, workspace_bytes);
    check_hip(fn, mamba::run_backbone_decode(*dims, *w, tokens, B, conv_state, ssm_state, logits,
                                             workspace, static_cast<hipStream_t>(stream)));
  });
}

// A captured decode step: the instantiated graph of every kernel launch of one
// mamba_backbone_decode_step with fixed pointers.
struct mamba_graph {
  hipGraphExec_t exec = nullptr;
};

mamba_status mamba_backbone_decode_graph_create(const mamba_backbone_dims* dims,
                                                const mamba_backbone_weights* w,
                                                const int32_t* tokens, int B, float* conv_state,
                                                float* ssm_state, float* logits, void* workspace,
                                                size_t workspace_bytes, mamba_graph** out) {
  static const char* fn = "mamba_backbone_decode_graph_create";
  return guarded([&] {
    if (!out) fail(MAMBA_EINVAL, fn, "out is NULL");
    *out = nullptr;
    check_decode_call(fn, dims, w, tokens, B, conv_state, ssm_state, logits, workspace, workspace_bytes);
    // capture on a private stream (default priority), so the caller's streams are untouched
    hipStream_t cs = nullptr;
    check_hip(fn, hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
      const hipError_t run = mamba::run_backbone_decode(*dims, *w, tokens, B, conv_state, ssm_state,
                                                        logits, workspace, cs);
      e = hipStreamEndCapture(cs, &graph);
      if (run != hipSuccess) e = run;
    }
    hipGraphExec_t exec = nullptr;
    if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(cs);
    check_hip(fn, e);
    *out = new mamba_graph{exec};
  });
}

mamba_status mamba_graph_launch(mamba_graph* g, void* stream) {
  static const char* fn = "mamba_graph_launch";
  return guarded([&] {
    if (!g || !g->exec) fail(MAMBA_EINVAL, fn, "graph is NULL");
    check_hip(fn, hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
  });
}

void mamba_graph_destroy(mamba_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  delete g;
}

}  // extern "C"
