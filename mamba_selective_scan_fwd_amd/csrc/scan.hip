// scan.hip -- prefill selective scan over T tokens with carried SSM state.
//
// prefill.rs page (mamba-rs 0.6.4), prefill_body stages F4c (delta = softplus(dt_proj
// output + bias)) and F4d (scan over all T, y gated by silu(z) read at a row stride, final
// state into the persistent SSM state); inference.rs page (mamba-rs 0.5.1),
// GpuMambaInference::new (A = -exp(A_log)). Softplus, A = -exp(A_log), the D skip and the
// gate are all fused here: u, dt, z, B and C are read once and y is written once.
//
// Workgroup = CH consecutive channels (32; 64 when N > 32) x all NP (padded) states, as W
// waves. Each lane holds one channel and one group of S consecutive states in registers
// (S = 2 at N = 16): lanes 0..CH-1 of a wave take one state group, the next CH lanes the
// next. A channel's recurrence is thus split over lanes and waves by state, not by time:
// there is no rescan and the whole T of a chunk is walked once.
//
// The per-token work that does not depend on the state is shared through LDS, in blocks of
// kTB = 8 tokens. In each block every thread owns one (token, channel) item: it computes
// delta (softplus), delta*u and silu(z) for that item (and, with the conv fused, u itself
// from its K raw inputs) and stages part of the block's B/C rows. Every lane then reads
// delta, delta*u and its states' B/C values for the block's tokens from LDS, advances its S
// states and leaves its partial C.h per token in LDS; after the barrier each item's owner
// adds the partials of its item, the D skip and the gate, and stores y. The block buffers
// are double-buffered, so one barrier per block orders everything, and the global loads of
// a block are issued one block before their use.
//
// T parallelism: when B * ceil(D/CH) workgroups cannot fill the chip, T is cut into chunks.
// A chunk acts on the state as h -> P*h + H per (b, d, n), P = exp(A * sum(delta)) and H the
// state it reaches from h = 0. A summary pass computes (sum(delta), H) of every chunk but
// the last; the output pass starts each chunk from the carried state folded through the
// maps of the chunks before it (at most MAMBA_SCAN_MAX_CHUNKS chunks, so each workgroup folds
// them itself).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mamba {

constexpr int kLanes = 64;
constexpr int kTB = 8;  // tokens per block (one LDS exchange and one barrier per block)

#ifndef MAMBA_SCAN_CH
#define MAMBA_SCAN_CH 32  // channels per workgroup (32 or 64)
#endif
constexpr int kCh = MAMBA_SCAN_CH;
constexpr int kWaves = kTB * kCh / kLanes;  // one per-token item per thread and block

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
  // fused conv (u computed from x in the kernel)
  const void* x;           // x[b,t,d] at (b*T+t)*x_row_stride + d
  const float* conv_w;     // [D][K]
  const float* conv_b;     // [D] or NULL
  float* conv_state;       // [B][D][K] in/out, or NULL (zeros, not written)
  float* conv_ws;          // [B][D][K] copy of the incoming conv state (chunks > 1)
  void* u_out;             // [B][T][D] or NULL
  const int32_t* lengths;  // [B] valid tokens per sequence (clamped to [0, T]) or NULL
  int64_t x_row_stride;
  int64_t bc_row_stride;
  int64_t z_row_stride;
  int B, T, D, N, K;
  int chunk_t, chunks;
  int softplus;
  int y_bf16;  // f32 I/O only: y stored as bf16 (the operand type of the product that reads it)
};

// A * log2(e) for A = -exp(A_log) of state n (0 for padded states: decay 1, and their B and
// C are staged as 0, so they stay 0 and add nothing).
__device__ __forceinline__ float a_log2(const float* __restrict__ A_log, int d, int n, int N) {
  return n < N ? -__builtin_amdgcn_exp2f(A_log[(int64_t)d * N + n] * kLog2e) * kLog2e : 0.0f;
}

// Load one element at byte offset `lane_off` of a row whose address is wave-uniform: the row
// address stays in scalar registers and the load takes the per-lane offset, so no vector
// address arithmetic is spent per token.
template <typename IO>
__device__ __forceinline__ float load_at(const IO* row, uint32_t lane_off) {
  return to_f32(*reinterpret_cast<const IO*>(reinterpret_cast<const char*>(row) + lane_off));
}
// The same, returning the stored element unconverted: a prefetched value stays in its I/O
// type until it is used, so the wait for the load sits at the use, not at the load.
template <typename IO>
__device__ __forceinline__ IO load_raw(const IO* row, uint32_t lane_off) {
  return *reinterpret_cast<const IO*>(reinterpret_cast<const char*>(row) + lane_off);
}

// OUT = false: summary pass over chunks 0 .. chunks-2 (no y). OUT = true: the output pass.
//
// Workgroup: CH channels x NP states as W waves. Lane l of wave q holds channel l % CH and
// state group g = q * H + l / CH (H = 64 / CH groups per wave), i.e. states [g*S, g*S+S) with
// S = NP / (W * H). The per-token work of a block (kTB tokens x CH channels) is one item per
// thread: item i = q * 64 + l is token i / CH, channel i % CH.
// KC = 0: u is an input. KC > 0: the causal depthwise conv + SiLU is fused in -- each
// per-token item reads its K raw inputs (x rows t-K+1 .. t, the carried conv state before
// the sequence start) and computes u itself (rounded to the I/O type, as a stored u would
// be); KC = 4 is the compile-time 4-tap case, KC = kMaxConvK any K <= 8 at run time.
#ifndef MAMBA_SCAN_WPE
#define MAMBA_SCAN_WPE 5  // minimum waves per SIMD the register allocation must allow
#endif

template <typename IO, int NP, int CH, int W, bool OUT, bool GATE, int KC>
__global__ void __launch_bounds__(kLanes * W) __attribute__((amdgpu_waves_per_eu(MAMBA_SCAN_WPE)))
scan_kernel(const ScanParams p) {
  constexpr int H = kLanes / CH;     // state groups per wave
  constexpr int G = W * H;           // state groups per workgroup
  constexpr int S = NP / G;          // states per lane
  constexpr int NT = kLanes * W;
  // staged B/C row: per group [B(S) | C(S)]; the summary pass stages B alone, per group B(S)
  constexpr int BCS = OUT ? 2 * S : S;  // slots per group
  constexpr int BCW = G * BCS;
  static_assert(S >= 1 && S * G == NP, "state split");
  static_assert(kTB * CH == NT, "one per-token item per thread and block");

  __shared__ float2 s_dd[2][kTB][CH];  // (delta, delta*u)
  __shared__ __attribute__((aligned(16))) float s_bc[2][kTB][BCW];
  __shared__ float s_yp[OUT ? 2 : 1][OUT ? kTB : 1][G][CH];  // partial C.h per group
  __shared__ float s_sd[OUT ? 1 : kTB][CH];  // summary pass: sum of delta per token residue

  const int lane = threadIdx.x & (kLanes - 1);
  // wave index, explicitly wave-uniform so that row arithmetic stays scalar
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int ch = lane % CH;          // this lane's channel in the scan
  const int g = q * H + lane / CH;   // this lane's state group
  // Channel group of this workgroup. Workgroups go to the 8 XCDs (each with its own L2) in
  // round-robin order of their linear id. When a group's rows are narrower than a 128-byte
  // line (bf16, 32 channels), groups 2p and 2p+1 -- the two halves of the same lines -- are
  // given workgroup ids 8 apart, so both land on one XCD and the line is fetched once.
  int cgrp = blockIdx.x;
  if constexpr (CH * sizeof(IO) < 128) {
    const int x16 = blockIdx.x & ~15;
    if (x16 + 16 <= (int)gridDim.x) cgrp = x16 + 2 * (blockIdx.x & 7) + ((blockIdx.x >> 3) & 1);
  }
  const int d0 = cgrp * CH;
  const int b = blockIdx.y;
  const int c = blockIdx.z;
  const int N = p.N, D = p.D;
  const int t0 = c * p.chunk_t;
  // this sequence's length (ragged batches: each sequence stops at its own last token)
  const int Tb = p.lengths ? min(max(p.lengths[b], 0), p.T) : p.T;
  const int len = max(min(Tb, t0 + p.chunk_t) - t0, 0);  // 0: the chunk is past the end
  const int nblk = (len + kTB - 1) / kTB;
  const int64_t row0 = (int64_t)b * p.T + t0;  // first row of the chunk
  const int64_t bcs = p.bc_row_stride;
  const int d = d0 + ch;
  const int dc = min(d, D - 1);  // clamped channel for loads of masked lanes

  // per-token item of this thread: token ij of the block (ij = it_wave + it_lane), channel ic
  const int it_wave = q * kLanes / CH;  // wave-uniform part of the token index
  const int it_lane = lane / CH;
  const int ic = lane % CH;
  const int di = d0 + ic;
  const int dic = min(di, D - 1);

  const IO* __restrict__ u = static_cast<const IO*>(p.u);
  const IO* __restrict__ dt = static_cast<const IO*>(p.dt);
  const IO* __restrict__ z = static_cast<const IO*>(p.z);
  // byte offsets of this thread's item in a block's first row (the row address is scalar)
  const uint32_t off_x = ((uint32_t)it_lane * (uint32_t)D + (uint32_t)dic) * (uint32_t)sizeof(IO);
  const uint32_t off_z =
      ((uint32_t)it_lane * (uint32_t)p.z_row_stride + (uint32_t)dic) * (uint32_t)sizeof(IO);
  const uint32_t off_y = ((uint32_t)it_lane * (uint32_t)D + (uint32_t)dic) * (uint32_t)sizeof(IO);

  float a2[S];
#pragma unroll
  for (int s = 0; s < S; ++s) a2[s] = a_log2(p.A_log, dc, g * S + s, N);
  const float bias = p.dt_bias ? p.dt_bias[dic] : 0.0f;
  float dskip = p.D_skip ? p.D_skip[dic] : 0.0f;
  const bool sp = p.softplus != 0;
  const bool dval = d < D;

  // fused conv: taps and bias of this thread's item channel, and where the incoming conv
  // state is read (the output pass of a chunked call reads the copy the summary pass made,
  // since the last chunk overwrites the state in place)
  constexpr int KM = KC > 0 ? KC : 1;
  const int K = KC == kMaxConvK ? p.K : KM;
  float wk[KM];
  float cbias = 0.0f;
  const float* cs_old = nullptr;
  const IO* __restrict__ xin = static_cast<const IO*>(p.x);
  uint32_t off_xx = 0;
  if constexpr (KC > 0) {
#pragma unroll
    for (int kk = 0; kk < KM; ++kk) wk[kk] = kk < K ? p.conv_w[(int64_t)dic * K + kk] : 0.0f;
    cbias = p.conv_b ? p.conv_b[dic] : 0.0f;
    // (a NULL conv state means zeros: the copy is then never made nor read)
    cs_old = !p.conv_state ? nullptr : (OUT && p.chunks > 1) ? p.conv_ws : p.conv_state;
    off_xx = ((uint32_t)it_lane * (uint32_t)p.x_row_stride + (uint32_t)dic) * (uint32_t)sizeof(IO);
  }

  // ---- start state
  float h[S];
  if constexpr (OUT) {
    if (p.chunks == 1) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = g * S + s;
        h[s] = (p.state_in && n < N) ? p.state_in[((int64_t)b * D + dc) * N + n] : 0.0f;
      }
    } else {
      // carried state, then the maps of chunks 0 .. c-1 in token order
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = g * S + s;
        h[s] = n < N ? p.start_ws[((int64_t)b * N + n) * D + dc] : 0.0f;
      }
      // predecessors in groups of kFold: all of a group's loads are issued before its fmas.
      // The lane's part of each index is formed once; per predecessor only a wave-uniform
      // offset is added (one address add per load instead of a 64-bit index product).
      constexpr int kFold = S <= 2 ? 8 : (S <= 4 ? 4 : 1);
      const float* sw_lane = p.sum_ws + (int64_t)b * p.chunks * D + dc;
      const float* hw_lane[S];
#pragma unroll
      for (int s = 0; s < S; ++s)
        hw_lane[s] = p.h_ws + ((int64_t)b * p.chunks * N + min(g * S + s, N - 1)) * D + dc;
      const int64_t chunk_nd = (int64_t)N * D;  // h_ws distance between consecutive chunks
      for (int c0 = 0; c0 < c; c0 += kFold) {
        float sd[kFold], hv[kFold][S];
#pragma unroll
        for (int f = 0; f < kFold; ++f) {
          const int64_t cc = min(c0 + f, c - 1);
          sd[f] = sw_lane[cc * D];
#pragma unroll
          for (int s = 0; s < S; ++s) hv[f][s] = hw_lane[s][cc * chunk_nd];
        }
#pragma unroll
        for (int f = 0; f < kFold; ++f) {
          if (c0 + f < c) {
#pragma unroll
            for (int s = 0; s < S; ++s)
              if (g * S + s < N) h[s] = fmaf(__builtin_amdgcn_exp2f(a2[s] * sd[f]), h[s], hv[f][s]);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < S; ++s) h[s] = 0.0f;
    if (c == 0 && dval) {  // keep the carried state for the output pass (it may be updated in place)
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = g * S + s;
        if (n < N)
          p.start_ws[((int64_t)b * N + n) * D + d] =
              p.state_in ? p.state_in[((int64_t)b * D + d) * N + n] : 0.0f;
      }
      if constexpr (KC > 0) {
        if (g == 0 && p.conv_state) {
          for (int kk = 0; kk < K; ++kk)
            p.conv_ws[((int64_t)b * D + d) * K + kk] = p.conv_state[((int64_t)b * D + d) * K + kk];
        }
      }
    }
  }

  // ---- B/C staging: thread i < kTB * BCW stages entry i of a block (token i / BCW, slot
  // i % BCW; the slots of group g are [B(gS..gS+S) | C(gS..gS+S)], or B(gS..gS+S) alone in
  // the summary pass, which reads no C).
  constexpr int BC_PER_T = (kTB * BCW + NT - 1) / NT;
  const IO* bc_src[BC_PER_T];  // this thread's B or C entry, token bc_j of the chunk's block 0
  int bc_j[BC_PER_T];
  bool bc_use[BC_PER_T];
#pragma unroll
  for (int r = 0; r < BC_PER_T; ++r) {
    const int i = threadIdx.x + r * NT;
    const int slot = i % BCW, w = slot % BCS;
    const bool isC = w >= S;
    const int n = slot / BCS * S + (isC ? w - S : w);
    bc_j[r] = i / BCW;
    bc_use[r] = i < kTB * BCW && n < N;
    bc_src[r] = static_cast<const IO*>(isC ? p.Cm : p.Bm) + (row0 + bc_j[r]) * bcs + min(n, N - 1);
  }

  // Loads are never predicated on the token: a token past the chunk re-reads the chunk's last
  // row (in bounds; such values are never used), so no load result is merged with an older
  // value and nothing waits on a load before its use.
  IO pf_dt[2], pf_u[2], pf_z[2], pf_bc[2][BC_PER_T];  // stored values, converted at use
  float pf_x[2][KM];  // fused conv: the item's K raw inputs, oldest first
  float u_blk[2], g_blk[2];  // u and silu(z) of this thread's item, for the finish
  // fused conv, general case (the sequence start or a partial block): token tg of the
  // sequence needs X[tg+1 .. tg+K] of X = [conv state (K), x (T)]
  auto load_conv_inputs = [&](int k, int st) {
    if constexpr (KC > 0) {
      const int tg = t0 + min(k * kTB + it_wave + it_lane, len - 1);
#pragma unroll
      for (int kk = 0; kk < KM; ++kk) {
        if (kk < K) {
          const int rel = tg + 1 + kk - K;  // x token, or a state slot when negative
          pf_x[st][kk] = rel >= 0 ? to_f32(xin[((int64_t)b * p.T + rel) * p.x_row_stride + dic])
                         : (cs_old ? cs_old[((int64_t)b * D + dic) * K + K + rel] : 0.0f);
        }
      }
    }
  };
  // Row offsets (in elements, wave-uniform) of the next block to load: load_block is called
  // once per block in block order, and each call advances them by one block, so a block's
  // row addresses cost one scalar add per tensor rather than a 64-bit row multiply.
  int64_t ld_xd = (row0 + it_wave) * D;                  // u, dt
  int64_t ld_z = (row0 + it_wave) * p.z_row_stride;      // z
  int64_t ld_x = (row0 + it_wave + 1 - K) * p.x_row_stride;  // oldest conv tap (fused conv)
  int64_t ld_bc = 0;                                     // B/C, from the chunk's first row
  auto load_block = [&](int k, auto P) {
    constexpr int st = decltype(P)::value;
    if (k * kTB + kTB <= len) {
      // full block: scalar row address + the thread's fixed byte offset
      pf_dt[st] = load_raw(dt + ld_xd, off_x);
      if constexpr (KC == 0) {
        pf_u[st] = load_raw(u + ld_xd, off_x);
      } else if (t0 + k * kTB >= K - 1) {
        // every tap of every item in the block is an x row: scalar rows, fixed lane offset
#pragma unroll
        for (int kk = 0; kk < KM; ++kk)
          if (kk < K) pf_x[st][kk] = load_at(xin + ld_x + kk * p.x_row_stride, off_xx);
      } else {
        load_conv_inputs(k, st);
      }
      if constexpr (OUT && GATE) pf_z[st] = load_raw(z + ld_z, off_z);
#pragma unroll
      for (int r = 0; r < BC_PER_T; ++r)
        if (threadIdx.x + r * NT < kTB * BCW) pf_bc[st][r] = bc_src[r][ld_bc];  // whole waves
    } else {
      const int64_t row = row0 + min(k * kTB + it_wave + it_lane, len - 1);
      pf_dt[st] = dt[row * D + dic];
      if constexpr (KC == 0) pf_u[st] = u[row * D + dic];
      else load_conv_inputs(k, st);
      if constexpr (OUT && GATE) pf_z[st] = z[row * p.z_row_stride + dic];
#pragma unroll
      for (int r = 0; r < BC_PER_T; ++r)
        if (threadIdx.x + r * NT < kTB * BCW)
          pf_bc[st][r] = bc_src[r][(int64_t)(min(k * kTB + bc_j[r], len - 1) - bc_j[r]) * bcs];
    }
    ld_xd += (int64_t)kTB * D;
    ld_z += (int64_t)kTB * p.z_row_stride;
    ld_x += (int64_t)kTB * p.x_row_stride;
    ld_bc += (int64_t)kTB * bcs;
  };

  float sum_delta = 0.0f;  // summary pass: this item's share of the chunk's sum of delta
  // stage A: delta and delta*u of this thread's item of block k into LDS, B/C of block k
  auto stage_a = [&](int k, auto P) {
    constexpr int st = decltype(P)::value;
    if constexpr (KC > 0) {
      // conv + SiLU in the order of the stand-alone conv kernel, rounded to the I/O type
      float cv = cbias;
#pragma unroll
      for (int kk = 0; kk < KM; ++kk)
        if (kk < K) cv = fmaf(wk[kk], pf_x[st][kk], cv);
      const IO uo = from_f32<IO>(silu(cv));
      pf_u[st] = uo;
      if constexpr (OUT) {
        const int j = it_wave + it_lane;
        if (p.u_out && di < D && k * kTB + j < len)
          static_cast<IO*>(p.u_out)[(row0 + k * kTB + j) * D + di] = uo;
      }
    }
    const float v = to_f32(pf_dt[st]) + bias;
    const float delta = sp ? softplus(v) : v;
    const float uf = to_f32(pf_u[st]);
    s_dd[st][it_wave + it_lane][ic] = make_float2(delta, delta * uf);
    // summary pass: the chunk's sum of delta, per item (token residue j of channel ic); the
    // residues are added at the end
    if constexpr (!OUT) sum_delta += k * kTB + it_wave + it_lane < len ? delta : 0.0f;
    u_blk[st] = uf;
    if constexpr (OUT && GATE) g_blk[st] = silu(to_f32(pf_z[st]));
    // pin both values here: left to the compiler they sink to their use after the next
    // block's loads, whose wait then covers those loads too
    asm volatile("" : "+v"(u_blk[st]));
    if constexpr (OUT && GATE) asm volatile("" : "+v"(g_blk[st]));
#pragma unroll
    for (int r = 0; r < BC_PER_T; ++r) {
      const int i = threadIdx.x + r * NT;
      if (i < kTB * BCW)
        // (tokens past the chunk's end are never scanned, so only padded states need zeros)
        s_bc[st][bc_j[r]][i % BCW] = bc_use[r] ? to_f32(pf_bc[st][r]) : 0.0f;
    }
  };

  // stage B: the LDS operands of one token (delta, delta*u, and this group's B and C)
  struct TokOps {
    float2 dd;
    float bv[S], cv[S];
  };
  auto read_token = [&](int st, int j, TokOps& o) {
    o.dd = s_dd[st][j][ch];
    const float* bcr = &s_bc[st][j][g * BCS];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      o.bv[s] = bcr[s];
      if constexpr (OUT) o.cv[s] = bcr[S + s];
    }
  };
  // advance the S states by one token; the partial C.h goes to LDS
  auto scan_token = [&](int st, int j, const TokOps& o) {
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float a = __builtin_amdgcn_exp2f(o.dd.x * a2[s]);
      h[s] = fmaf(a, h[s], o.dd.y * o.bv[s]);
      if constexpr (OUT) acc = s == 0 ? o.cv[0] * h[0] : fmaf(o.cv[s], h[s], acc);
    }
    if constexpr (OUT) s_yp[st][j][g][ch] = acc;
  };
  // Token j+1's LDS reads are issued before token j's arithmetic (one token of look-ahead:
  // the read latency hides behind a token of work). A full block is one straight-line
  // region: the compiler pairs the reads of neighbouring tokens into wider LDS instructions
  // and moves the decay factors of a token ahead of the previous token's state update.
  auto scan_block = [&](int st, int nj) {
    TokOps cur, nxt;
    read_token(st, 0, cur);
    if (nj == kTB) {
#pragma unroll
      for (int j = 0; j < kTB; ++j) {
        if (j + 1 < kTB) read_token(st, j + 1, nxt);
        scan_token(st, j, cur);
        cur = nxt;
      }
    } else {
      for (int j = 0; j < nj; ++j) {
        if (j + 1 < nj) read_token(st, j + 1, nxt);
        scan_token(st, j, cur);
        cur = nxt;
      }
    }
  };

  int64_t st_y = (row0 + it_wave) * D;  // y row offset of the block being finished
  // one block: stage A of block k+1, loads of block k+2, stage B of block k, barrier, finish
  auto block = [&](int k, auto P) {
    constexpr int st = decltype(P)::value;  // == k & 1
    if (k + 1 < nblk) {
      stage_a(k + 1, std::integral_constant<int, st ^ 1>{});
      // every use of block k+1's loads stays above the next loads: a use scheduled below
      // them would have to wait for them as well (the load counter drains in order)
      __builtin_amdgcn_sched_barrier(0);
      if (k + 2 < nblk) load_block(k + 2, P);
    }
    const int nj = min(kTB, len - k * kTB);
    scan_block(st, nj);
    __syncthreads();

    // finish: this thread's item of the block
    if constexpr (OUT) {
      const int j = it_wave + it_lane;
      if (j < nj) {
        float part[G];
#pragma unroll
        for (int w = 0; w < G; ++w) part[w] = s_yp[st][j][w][ic];
#pragma unroll
        for (int span = 1; span < G; span *= 2)  // pairwise tree: short dependency chain
#pragma unroll
          for (int w = 0; w + span < G; w += 2 * span) part[w] += part[w + span];
        float yv = part[0];
        yv = fmaf(dskip, u_blk[st], yv);
        if constexpr (GATE) yv *= g_blk[st];
        if (di < D) {
          // (a bf16 y from f32 I/O is taken only with u as an input: the backbone's scan; the
          // fused-conv kernels keep their register budget for the conv)
          if (std::is_same_v<IO, float> && KC == 0 && p.y_bf16) {
            // same element offsets at half the width
            bf16* yrow = static_cast<bf16*>(p.y) + st_y;
            *reinterpret_cast<bf16*>(reinterpret_cast<char*>(yrow) + off_y / 2) = from_f32<bf16>(yv);
          } else {
            // scalar row of the wave's first token + the lane's fixed byte offset
            IO* yrow = static_cast<IO*>(p.y) + st_y;
            // y streams out non-temporally: it is not read again here, and the cache lines it
            // would occupy stay with the inputs (at the 2.8b layer, those the partner workgroup
            // -- the other half of each 128-byte row -- has yet to read: fetch 1.61 -> 1.53 GB
            // per call; at the 130m layer, the inputs the next call finds in the caches)
            __builtin_nontemporal_store(from_f32<IO>(yv),
                                        reinterpret_cast<IO*>(reinterpret_cast<char*>(yrow) + off_y));
          }
        }
      }
      st_y += (int64_t)kTB * D;
    }
  };

  // Wait for the start state and the skip weight here, once: their first uses are inside the
  // block loop, where the wait would be a full drain of the load counter on every block.
  asm volatile("" : "+v"(dskip));
#pragma unroll
  for (int s = 0; s < S; ++s) asm volatile("" : "+v"(h[s]));

  // prologue: block 0 staged, block 1 in flight (an empty chunk loads nothing; its map is
  // the identity and its state passes through)
  if (nblk > 0) {
    load_block(0, std::integral_constant<int, 0>{});
    stage_a(0, std::integral_constant<int, 0>{});
    if (nblk > 1) load_block(1, std::integral_constant<int, 1>{});
  }
  __syncthreads();
  for (int k = 0; k < nblk; k += 2) {
    block(k, std::integral_constant<int, 0>{});
    if (k + 1 < nblk) block(k + 1, std::integral_constant<int, 1>{});
  }

  if constexpr (!OUT) {
    s_sd[it_wave + it_lane][ic] = sum_delta;
    __syncthreads();
  }
  if (!dval) return;
  if constexpr (OUT) {
    if (c == p.chunks - 1 && p.state_out) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = g * S + s;
        if (n < N) p.state_out[((int64_t)b * D + d) * N + n] = h[s];
      }
    }
    if constexpr (KC > 0) {
      // new conv state X[T .. T+K-1]: x tokens T-K .. T-1, or (T < K) the old state shifted
      if (c == p.chunks - 1 && p.conv_state && g == 0) {
        for (int kk = 0; kk < K; ++kk) {
          const int i = Tb + kk;
          p.conv_state[((int64_t)b * D + d) * K + kk] =
              i >= K ? to_f32(xin[((int64_t)b * p.T + i - K) * p.x_row_stride + d])
                     : (cs_old ? cs_old[((int64_t)b * D + d) * K + i] : 0.0f);
        }
      }
    }
  } else {
    const int64_t bc_ = (int64_t)b * p.chunks + c;
    if (g == 0) {
      // the chunk's sum of delta: the kTB token residues of channel ch, in residue order
      float sd = 0.0f;
#pragma unroll
      for (int j = 0; j < kTB; ++j) sd += s_sd[j][ch];
      p.sum_ws[bc_ * D + d] = sd;
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int n = g * S + s;
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
#define MAMBA_SCAN_TARGET_WAVES 6144  // ~6 waves per SIMD (256 CUs x 4 SIMDs)
#endif
#ifndef MAMBA_SCAN_MIN_CHUNK
#define MAMBA_SCAN_MIN_CHUNK 88  // tokens per chunk, at least (11 blocks)
#endif
#ifndef MAMBA_SCAN_MAX_CHUNKS
#define MAMBA_SCAN_MAX_CHUNKS 64  // each output workgroup folds up to this many - 1 chunk maps
#endif

static int padded_n(int N) { return N <= 16 ? 16 : (N <= 32 ? 32 : 64); }

ScanPlan plan_selective_scan(int B, int T, int D, int N) {
  ScanPlan p{1, T, 0};
  if (B <= 0 || T <= 0 || D <= 0 || N <= 0) return p;
  // Chunks are added while the grid stays within the target (rounded down: a grid that
  // already fills most of it runs as one chunk, since every extra chunk count adds a summary
  // pass over the data), and no chunk is shorter than the minimum, where the chunk's fixed
  // start (the fold of its predecessors' maps, the first loads) is no longer amortised.
  const int64_t waves_per_chunk = (int64_t)B * ((D + kCh - 1) / kCh) * kWaves;
  int64_t chunks = MAMBA_SCAN_TARGET_WAVES / waves_per_chunk;
  chunks = std::max<int64_t>(1, std::min<int64_t>(chunks, T / MAMBA_SCAN_MIN_CHUNK));
  // the fold of the chunk maps before a chunk is sequential in the chunk count, so the count
  // is capped: a very long sequence over few channels gets longer chunks instead
  chunks = std::min<int64_t>(chunks, MAMBA_SCAN_MAX_CHUNKS);
  // whole blocks of kTB tokens per chunk
  int chunk_t = (int)((T + chunks - 1) / chunks);
  chunk_t = (chunk_t + kTB - 1) / kTB * kTB;
  p.chunks = (T + chunk_t - 1) / chunk_t;
  p.chunk_t = chunk_t;
  if (p.chunks > 1) {
    // chunk sums, chunk end states, the carried SSM state, and (fused conv) the carried
    // conv state
    const size_t bcd = (size_t)B * p.chunks * D;
    p.workspace_bytes = align256(sizeof(float) * bcd) + align256(sizeof(float) * bcd * N) +
                        align256(sizeof(float) * (size_t)B * N * D) +
                        align256(sizeof(float) * (size_t)B * D * kMaxConvK);
  }
  return p;
}

template <typename IO, int NP, int KC>
static hipError_t launch_scan_npk(const ScanFwdArgs& a, const ScanPlan& pl, hipStream_t s) {
  // 64 states per channel: 64-channel workgroups keep the states per lane at 8
  constexpr int CH = NP == 64 ? 64 : kCh;
  constexpr int W = kTB * CH / kLanes;
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
  p.x = a.x;
  p.conv_w = a.conv_w;
  p.conv_b = a.conv_b;
  p.conv_state = a.conv_state;
  p.u_out = a.u_out;
  p.lengths = a.lengths;
  p.x_row_stride = a.x_row_stride;
  p.bc_row_stride = a.bc_row_stride;
  p.z_row_stride = a.z_row_stride;
  p.B = a.B;
  p.T = a.T;
  p.D = a.D;
  p.N = a.N;
  p.K = a.K;
  p.chunk_t = pl.chunk_t;
  p.chunks = pl.chunks;
  p.softplus = a.delta_softplus ? 1 : 0;
  p.y_bf16 = a.y_bf16 && !a.bf16 && !a.x ? 1 : 0;
  const unsigned gx = (unsigned)((a.D + CH - 1) / CH);
  if (pl.chunks > 1) {
    char* ws = static_cast<char*>(a.workspace);
    const size_t bcd = (size_t)a.B * pl.chunks * a.D;
    p.sum_ws = reinterpret_cast<float*>(ws);
    ws += align256(sizeof(float) * bcd);
    p.h_ws = reinterpret_cast<float*>(ws);
    ws += align256(sizeof(float) * bcd * a.N);
    p.start_ws = reinterpret_cast<float*>(ws);
    ws += align256(sizeof(float) * (size_t)a.B * a.N * a.D);
    p.conv_ws = reinterpret_cast<float*>(ws);
    scan_kernel<IO, NP, CH, W, false, false, KC><<<dim3(gx, a.B, pl.chunks - 1), kLanes * W, 0, s>>>(p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(gx, a.B, pl.chunks);
  if (a.z)
    scan_kernel<IO, NP, CH, W, true, true, KC><<<grid, kLanes * W, 0, s>>>(p);
  else
    scan_kernel<IO, NP, CH, W, true, false, KC><<<grid, kLanes * W, 0, s>>>(p);
  return hipGetLastError();
}

template <typename IO, int NP>
static hipError_t launch_scan_np(const ScanFwdArgs& a, const ScanPlan& pl, hipStream_t s) {
  if (!a.x) return launch_scan_npk<IO, NP, 0>(a, pl, s);
  if (a.K == 4) return launch_scan_npk<IO, NP, 4>(a, pl, s);
  return launch_scan_npk<IO, NP, kMaxConvK>(a, pl, s);
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
