// Ulysses relayouts for one rank, gfx950: sequence-major -> head-major before
// attention and head-major -> sequence-major after it.
//
//   forward: dst[t][b, p*S_loc + s, j, :] = src[t][p][b, s, rank*H_loc + j, :]
//   inverse: dst[t][b, s, r*H_loc + j, :] = src[t][r][b, rank*S_loc + s, j, :]
//
// ("Scaling Video Generation Across NVL72 rack with TensorRT-LLM", "Ulysses
// Parallelism" and its Figure 2: [B, S/P, H, D] -> [B, S, H/P, D] before the
// full-sequence attention and back after it, Q/K/V moved together from the
// fused projection; "CUDA IPC Ulysses" (TeleFuser), "Strided Copy Engine
// scatter": the strided V view is read in place and written straight into the
// final layout; "How 8 GPUs split tokens" (LTX-2 SP), "Precise statement": the
// round trip returns every byte.)  A pure copy of 16-bit patterns.
//
// HBM-bound stream.  The copy is cut into runs: one run is the H_loc*D
// contiguous elements one token contributes to one tensor from one rank's
// head slice (or one head's D elements when a view's head slices are not
// contiguous).  Each wave copies whole runs with 16-byte loads and stores; all
// loads of a run are issued before its stores.  Every byte is touched once, so
// loads and stores are non-temporal: the forward copy 6-8 % faster at the
// LTX-2 and Wan shares' sizes; the inverse 10 % faster on its own (Wan shard,
// 69 -> 76 % of HBM) and 3.5 % faster right after the attention that wrote its
// source at the Cosmos share (74.6 -> 77.2 %), 1.5 % slower there at Wan's
// (76.3 -> 75.1 %).  Run indices are wave-uniform,
// so the per-run address arithmetic (tensor, shard, token) stays in scalar
// registers, in 32 bits (the host keeps the run count at or below 2^30, so a
// wave's run index plus the grid stride cannot overflow).  Runs are numbered so
// that consecutive runs write consecutive destination bytes.  A forward call
// that writes some tensors token-contiguous (below) runs both kinds of
// workgroup in one launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsd_internal.h"

namespace lsd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kUnroll = 4;  // 16-byte vectors per lane in flight per pass

template <bool kInverse>
__device__ __attribute__((always_inline)) void copy_body(const RelayoutArgs& a, int n_runs, int block, int nblocks) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int runs_per_token = a.H_loc / a.heads_per_run;
  const int vpr = a.heads_per_run * a.D / 8;  // vectors per run
  const int stride = nblocks * kWavesPerBlock;

  for (int run = block * kWavesPerBlock + wave; run < n_runs; run += stride) {
    const int jr = run % runs_per_token;
    const int tok = run / runs_per_token;
    const int j0 = jr * a.heads_per_run;
    int p, s, tb;
    if (!kInverse) {  // tok = ((t*B + b)*P + p)*S_loc + s
      s = tok % a.S_loc;
      const int tp = tok / a.S_loc;
      p = tp % a.P;
      tb = tp / a.P;
    } else {          // tok = ((t*B + b)*S_loc + s)*P + r, p = source rank r
      p = tok % a.P;
      const int ts = tok / a.P;
      s = ts % a.S_loc;
      tb = ts / a.S_loc;
    }
    const int b = tb % a.B;
    const int t = tb / a.B;

    const uint16_t* sp;
    uint16_t* dp;
    if (!kInverse) {
      sp = a.src[t][p] + (int64_t)b * a.src_sb[t][p] + (int64_t)s * a.src_ss[t][p] +
           (int64_t)(a.rank * a.H_loc + j0) * a.src_sh[t][p];
      dp = a.dst[t] + (int64_t)b * a.dst_sb[t] + (int64_t)(p * a.S_loc + s) * a.dst_ss[t] +
           (int64_t)j0 * a.dst_sh[t];
    } else {
      sp = a.src[t][p] + (int64_t)b * a.src_sb[t][p] + (int64_t)(a.rank * a.S_loc + s) * a.src_ss[t][p] +
           (int64_t)j0 * a.src_sh[t][p];
      dp = a.dst[t] + (int64_t)b * a.dst_sb[t] + (int64_t)s * a.dst_ss[t] +
           (int64_t)(p * a.H_loc + j0) * a.dst_sh[t];
    }

    for (int v0 = 0; v0 < vpr; v0 += 64 * kUnroll) {
      u32x4 buf[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + u * 64 + lane;
        if (v < vpr) {
          const u32x4* src = (const u32x4*)(sp + 8 * v);
          buf[u] = __builtin_nontemporal_load(src);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + u * 64 + lane;
        if (v < vpr) {
          __builtin_nontemporal_store(buf[u], (u32x4*)(dp + 8 * v));
        }
      }
    }
  }
}

template <bool kInverse>
__global__ void __launch_bounds__(kThreads) relayout_kernel(const RelayoutArgs a, int n_runs) {
  copy_body<kInverse>(a, n_runs, (int)blockIdx.x, (int)gridDim.x);
}

// Forward relayout into a token-contiguous destination (each channel's
// P*S_loc tokens one row of pitch dst_sd):
//   dst[t][b, p*S_loc + s, j, d] = src[t][p][b, s, rank*H_loc + j, d]
// with the destination stored [b][j][d][token].  One wave moves 64 tokens x
// 128 channels (two 64-channel blocks; one when D = 64 or for the last block
// of an odd count) of one head: lane (c = lane % 8, g = lane / 8) loads
// 16 bytes (8 channels) of each block of each of the 8 tokens 8g..8g+7,
// transposes each 8x8 block in registers and stores 16 bytes (8 tokens) of
// each of its channels, so each load instruction reads 8 whole 128-byte lines
// (8 tokens, 64 channels) and each store writes 8 (8 channels, 64 tokens).
// Tokens past the end are neither read nor written; a row's last partial
// 8-token group is stored element by element, so row padding is never touched.
// A wave takes both channel blocks of its tokens, so a token's 256 bytes of
// one head are read together: at the Cosmos share the V part ran at 62 % of
// HBM against 57 % with one block per wave (whole relayout 71.7 % against
// 69.4 %; Wan's share 72.2 % against 71.4 %).  Clusters of 2 or 4 heads in
// consecutive workgroups, heads fastest, and plain (cached) loads or stores
// measured level or slower.
constexpr int kTokWavesPerBlock = 4;

// units of work: 64-token blocks x pairs of 64-channel blocks, per head
__host__ __device__ inline int64_t tok_units(int64_t n_tensors, int64_t B, int64_t H_loc, int64_t S, int64_t D) {
  return n_tensors * B * H_loc * (((S + 63) / 64 + 3) / 4 * 4) * ((D / 64 + 1) / 2);
}

__device__ __attribute__((always_inline)) void tok_body(const RelayoutArgs& a, int n_units, int block) {
  const int lane = threadIdx.x & 63;
  const int unit = block * kTokWavesPerBlock + (int)(threadIdx.x >> 6);
  if (unit >= n_units) return;
  const int S = a.P * a.S_loc;
  const int n_tblk = (S + 63) / 64;
  const int n_dh = a.D / 64;
  const int n_dp = (n_dh + 1) / 2;
  // unit = ((((t * B + b) * H_loc + j) * n_dp + dp) * n_tblk4 + tb4) * 4 + tl:
  // the 4 waves of a workgroup take 4 consecutive 64-token blocks of one
  // (head, channel-block pair), so each of its channel rows gets 512
  // contiguous bytes (0.9 % faster than 2 token blocks x 2 channel blocks)
  const int n_tblk4 = (n_tblk + 3) / 4;
  int rest = unit;
  const int tl = rest % 4; rest /= 4;
  const int tb4 = rest % n_tblk4; rest /= n_tblk4;
  const int dp = rest % n_dp; rest /= n_dp;
  const int j = rest % a.H_loc; rest /= a.H_loc;
  const int b = rest % a.B;
  const int t = rest / a.B;
  const int tb = tb4 * 4 + tl;
  if (tb >= n_tblk) return;
  const int nb = min(2, n_dh - 2 * dp);  // channel blocks of this unit: 1 or 2 (uniform)
  const int c = lane & 7, g = lane >> 3;
  const int tok0 = tb * 64 + 8 * g;

  u32x4 x[2][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int tok = tok0 + k;
    x[0][k] = (u32x4){0u, 0u, 0u, 0u};
    x[1][k] = (u32x4){0u, 0u, 0u, 0u};
    if (tok < S) {
      const int p = tok / a.S_loc, s = tok - p * a.S_loc;
      const uint16_t* sp = a.src[t][p] + (int64_t)b * a.src_sb[t][p] + (int64_t)s * a.src_ss[t][p] +
                           (int64_t)(a.rank * a.H_loc + j) * a.src_sh[t][p] + 128 * dp + 8 * c;
      x[0][k] = __builtin_nontemporal_load((const u32x4*)sp);
      if (nb == 2) x[1][k] = __builtin_nontemporal_load((const u32x4*)(sp + 64));
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h >= nb) break;
    uint16_t* dp_ = a.dst[t] + (int64_t)b * a.dst_sb[t] + (int64_t)j * a.dst_sh[t] +
                    (int64_t)(128 * dp + 64 * h + 8 * c) * a.dst_sd[t] + tok0;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      // tokens 2i, 2i+1 of channel 8c + dd: the 16-bit halves dd%2 of dword dd/2
      const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
      u32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = __builtin_amdgcn_perm(x[h][2 * i + 1][dd >> 1], x[h][2 * i][dd >> 1], sel);
      uint16_t* row = dp_ + (int64_t)dd * a.dst_sd[t];
      if (tok0 + 8 <= S) {
        __builtin_nontemporal_store(y, (u32x4*)row);
      } else if (tok0 < S) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (tok0 + e < S) row[e] = (uint16_t)(y[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

__global__ void __launch_bounds__(64 * kTokWavesPerBlock) relayout_tok_kernel(const RelayoutArgs a, int n_units) {
  tok_body(a, n_units, (int)blockIdx.x);
}

// Both in one launch: the copying workgroups first, then the transposing
// ones (measured faster than spreading the transposing workgroups evenly
// among the copying ones).
__global__ void __launch_bounds__(kThreads) relayout_both_kernel(const RelayoutArgs a, const RelayoutArgs at, int n_runs,
                                                                 int n_units, int n_total, int n_tok) {
  const int i = (int)blockIdx.x;
  const int n_copy = n_total - n_tok;
  if (i < n_copy) copy_body<false>(a, n_runs, i, n_copy);
  else tok_body(at, n_units, i - n_copy);
}

}  // namespace

hipError_t launch_relayout_both(const RelayoutArgs& a, const RelayoutArgs& at, hipStream_t stream) {
  const int64_t n_runs = relayout_runs(a);
  const int64_t S = (int64_t)at.P * at.S_loc;
  const int64_t n_units = tok_units(at.n_tensors, at.B, at.H_loc, S, at.D);
  if (n_runs > 0x7fffffff || n_units > 0x7fffffff || at.D % 64 != 0 || a.inverse || at.inverse)
    return hipErrorInvalidValue;
  const int64_t n_tok = (n_units + kTokWavesPerBlock - 1) / kTokWavesPerBlock;
  int64_t n_copy = (n_runs + kWavesPerBlock - 1) / kWavesPerBlock;
  if (n_copy + n_tok == 0) return hipSuccess;
  hipLaunchKernelGGL(relayout_both_kernel, dim3((unsigned)(n_copy + n_tok)), dim3(kThreads), 0, stream, a, at, (int)n_runs,
                     (int)n_units, (int)(n_copy + n_tok), (int)n_tok);
  return hipGetLastError();
}

hipError_t launch_relayout_tok(const RelayoutArgs& a, hipStream_t stream) {
  const int64_t S = (int64_t)a.P * a.S_loc;
  const int64_t n_units = tok_units(a.n_tensors, a.B, a.H_loc, S, a.D);
  if (n_units == 0) return hipSuccess;
  if (n_units > 0x7fffffff || a.D % 64 != 0 || a.inverse) return hipErrorInvalidValue;
  const int64_t blocks = (n_units + kTokWavesPerBlock - 1) / kTokWavesPerBlock;
  hipLaunchKernelGGL(relayout_tok_kernel, dim3((unsigned)blocks), dim3(64 * kTokWavesPerBlock), 0, stream, a,
                     (int)n_units);
  return hipGetLastError();
}

int64_t relayout_runs(const RelayoutArgs& a) {
  return (int64_t)a.n_tensors * a.B * a.P * a.S_loc * (a.H_loc / a.heads_per_run);
}

hipError_t launch_relayout(const RelayoutArgs& a, hipStream_t stream) {
  const int64_t n_runs = relayout_runs(a);
  if (n_runs == 0) return hipSuccess;
  if (n_runs > 0x7fffffff) return hipErrorInvalidValue;
  int64_t blocks = (n_runs + kWavesPerBlock - 1) / kWavesPerBlock;
  // One run per wave (no grid-stride loop) measured fastest for the forward
  // copy (Wan's Q/K/V share: 0.424 -> 0.379 ms); the inverse prefers about
  // 1.15 runs per wave (0.144 -> 0.139 ms).
  if (a.inverse && blocks > 32768) blocks = 32768;
  if (a.inverse)
    hipLaunchKernelGGL(relayout_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, (int)n_runs);
  else
    hipLaunchKernelGGL(relayout_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, (int)n_runs);
  return hipGetLastError();
}

}  // namespace lsd
