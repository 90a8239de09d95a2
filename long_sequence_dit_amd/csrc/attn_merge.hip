// Exact log-sum-exp merge of n partial attention results, for gfx950.
//
// With M = max_i LSE_i and w_i = exp(LSE_i - M) per (b, h, s):
//   LSE = M + ln sum_i w_i,   O = sum_i (w_i / sum_k w_k) O_i
// ("Scaling Video Generation Across NVL72 rack with TensorRT-LLM", "Context
// Parallelism > Ring Attention" online-softmax merge and "Attention2D
// Parallelism > Merge phase" batched combine).  Rows whose LSEs are all -inf
// (no keys in any partial) give O = 0 and LSE = -inf.
//
// HBM-bound stream (non-temporal loads and stores: each byte is touched
// once).  A workgroup takes 2 consecutive positions s of a group of heads of
// one batch entry, so for contiguous (B, S, H, D) partials it reads and writes
// one contiguous span per partial.  Measured at LTX-2 scale (n = 2) and on the
// Ring share (n = 3): 0.117 ms when a workgroup took 64 positions of one head
// (256-byte rows 8 KB apart); 0.109 and 0.204 ms with 16 positions of all
// heads; 0.105 and 0.188 ms with 2 (4 and 8 fall in between).  Its weights
// take n * heads * 2 floats of LDS, sized at launch: a fixed 64 KB allowed
// only two workgroups per CU and ran 40 % slower.  Workgroups of 512 threads:
// at n = 3 (the Ring share) 0.181 ms against 0.193 ms with 256 threads, at
// n = 2 (LTX-2 scale) 0.108 against 0.111 ms.  For n = 2 to 4 the partial
// count is a template constant and each thread issues its vector's n loads
// before any arithmetic (with a run-time count the compiler issued one load
// at a time and waited for it): 0.181 -> 0.174 ms at n = 3 (72 -> 75 % of
// HBM), 0.108 -> 0.103 ms at n = 2 (71 -> 74 %), bit-identical.  Two vectors
// per thread per pass were slower at n = 2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsd_internal.h"

namespace lsd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kTok = 2;          // consecutive sequence positions per workgroup
constexpr int kThreads = 512;   // 256 measured 5-7 % slower at n = 2 and 3, 1024 15 % slower at n = 3
constexpr int kLdsFloats = 16384;  // at most 64 KB of weights per workgroup

__device__ inline uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// One workgroup: kTok consecutive positions s x a group of hg heads of one
// batch entry.  Phase 1 turns the n LSEs of each (h, s) into normalised
// weights in LDS (per head, kTok consecutive LSEs are read together).  Phase 2
// streams the token rows: for contiguous (B, S, H, D) partials a token's heads
// are adjacent, so the workgroup reads and writes kTok * hg * D * 2 contiguous
// bytes per partial, not scattered 256-byte rows.
// kN: the partial count when it is a compile-time constant (2 to 4), else 0
// (then the partials are read in a run-time loop).
template <int kN>
__global__ void __launch_bounds__(kThreads) attn_merge_kernel(const MergeArgs a, int n_stiles, int hg, int n_hgroups) {
  extern __shared__ float w_s[];  // [n][hg][kTok], sized at launch

  int rest = blockIdx.x;
  const int st = rest % n_stiles; rest /= n_stiles;
  const int g = rest % n_hgroups;
  const int b = rest / n_hgroups;
  const int s0 = st * kTok, h0 = g * hg;
  const int nh = min(hg, a.H - h0);
  const int tid = threadIdx.x;

  for (int p = tid; p < nh * kTok; p += kThreads) {
    const int hl = p / kTok, sl = p % kTok;
    const int s = s0 + sl;
    if (s >= a.S) continue;
    const int64_t li = ((int64_t)b * a.H + h0 + hl) * a.S + s;
    float L[kMaxMerge];
    float M = -INFINITY;
    for (int i = 0; i < a.n; ++i) {
      L[i] = a.lse_in[i][li];
      M = fmaxf(M, L[i]);
    }
    if (M == -INFINITY) {
      for (int i = 0; i < a.n; ++i) w_s[(i * hg + hl) * kTok + sl] = 0.0f;
      if (a.lse_out) a.lse_out[li] = -INFINITY;
    } else {
      float sum = 0.0f;
      for (int i = 0; i < a.n; ++i) {
        L[i] = expf(L[i] - M);
        sum += L[i];
      }
      const float inv = 1.0f / sum;
      for (int i = 0; i < a.n; ++i) w_s[(i * hg + hl) * kTok + sl] = L[i] * inv;
      if (a.lse_out) a.lse_out[li] = M + logf(sum);
    }
  }
  __syncthreads();

  const int vpr = a.D >> 3;          // 16-byte vectors per head row
  const int vpt = nh * vpr;          // per token
  const int ns = min(kTok, a.S - s0);
  auto addr_in = [&](int i, int q) -> const u32x4* {
    const int sl = q / vpt, r = q % vpt;
    const int hl = r / vpr, c = r % vpr;
    return (const u32x4*)(a.o_in[i] + (int64_t)b * a.in_sb[i] + (int64_t)(s0 + sl) * a.in_ss[i] +
                          (int64_t)(h0 + hl) * a.in_sh[i] + 8 * c);
  };
  auto store = [&](int q, const float* acc) {
    const int sl = q / vpt, r = q % vpt;
    const int hl = r / vpr, c = r % vpr;
    const u32x4 out = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
                       pack_bf16(acc[6], acc[7])};
    __builtin_nontemporal_store(out, (u32x4*)(a.o_out + (int64_t)b * a.out_sb + (int64_t)(s0 + sl) * a.out_ss +
                                              (int64_t)(h0 + hl) * a.out_sh + 8 * c));
  };
  auto weight = [&](int i, int q) {
    const int sl = q / vpt, hl = (q % vpt) / vpr;
    return w_s[(i * hg + hl) * kTok + sl];
  };
  auto accumulate = [&](float* acc, float w, const u32x4& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += w * __uint_as_float(v[e] << 16);
      acc[2 * e + 1] += w * __uint_as_float(v[e] & 0xffff0000u);
    }
  };
  const int nq = ns * vpt;
  if constexpr (kN > 0) {
    for (int q = tid; q < nq; q += kThreads) {
      u32x4 v[kN];
#pragma unroll
      for (int i = 0; i < kN; ++i) v[i] = __builtin_nontemporal_load(addr_in(i, q));
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kN; ++i) accumulate(acc, weight(i, q), v[i]);
      store(q, acc);
    }
  } else {
    for (int q = tid; q < nq; q += kThreads) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int i = 0; i < a.n; ++i) accumulate(acc, weight(i, q), __builtin_nontemporal_load(addr_in(i, q)));
      store(q, acc);
    }
  }
}

}  // namespace

hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.D % 8 != 0 || a.n < 1 || a.n > kMaxMerge) return hipErrorInvalidValue;
  const int hg = min(a.H, kLdsFloats / (a.n * kTok));  // heads whose weights fit in LDS
  const int n_hgroups = (a.H + hg - 1) / hg;
  const int n_stiles = (a.S + kTok - 1) / kTok;
  const int64_t nblk = (int64_t)n_stiles * n_hgroups * a.B;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = (size_t)a.n * hg * kTok * sizeof(float);
  switch (a.n) {
    case 2:
      hipLaunchKernelGGL(attn_merge_kernel<2>, dim3((unsigned)nblk), dim3(kThreads), lds, stream, a, n_stiles, hg, n_hgroups);
      break;
    case 3:
      hipLaunchKernelGGL(attn_merge_kernel<3>, dim3((unsigned)nblk), dim3(kThreads), lds, stream, a, n_stiles, hg, n_hgroups);
      break;
    case 4:
      hipLaunchKernelGGL(attn_merge_kernel<4>, dim3((unsigned)nblk), dim3(kThreads), lds, stream, a, n_stiles, hg, n_hgroups);
      break;
    default:
      hipLaunchKernelGGL(attn_merge_kernel<0>, dim3((unsigned)nblk), dim3(kThreads), lds, stream, a, n_stiles, hg, n_hgroups);
  }
  return hipGetLastError();
}

}  // namespace lsd
