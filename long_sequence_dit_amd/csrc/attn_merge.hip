// Exact log-sum-exp merge of n partial attention results, for gfx950.
//
// With M = max_i LSE_i and w_i = exp(LSE_i - M) per (b, h, s):
//   LSE = M + ln sum_i w_i,   O = sum_i (w_i / sum_k w_k) O_i
// ("Scaling Video Generation Across NVL72 rack with TensorRT-LLM", "Context
// Parallelism > Ring Attention" online-softmax merge and "Attention2D
// Parallelism > Merge phase" batched combine).  Rows whose LSEs are all -inf
// (no keys in any partial) give O = 0 and LSE = -inf.
//
// HBM-bound stream.  One workgroup covers 64 consecutive sequence positions of
// one (b, h): the 64 x n LSE values are read coalesced and turned into
// normalised weights in LDS, then each 16-lane group streams one 256-byte
// (D = 128) output row, reading the n partial rows it combines (non-temporal
// loads and stores: each byte is touched once).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsd_internal.h"

namespace lsd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = 64;
constexpr int kThreads = 256;

__device__ inline uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__global__ void __launch_bounds__(kThreads) attn_merge_kernel(const MergeArgs a, int n_stiles) {
  __shared__ float w_s[kMaxMerge][kRows];

  const int st = blockIdx.x % n_stiles;
  const int bh = blockIdx.x / n_stiles;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int s0 = st * kRows;
  const int tid = threadIdx.x;
  const int64_t lse_row = ((int64_t)b * a.H + h) * a.S;

  if (tid < kRows) {
    const int s = s0 + tid;
    if (s < a.S) {
      float L[kMaxMerge];
      float M = -INFINITY;
      for (int i = 0; i < a.n; ++i) {
        L[i] = a.lse_in[i][lse_row + s];
        M = fmaxf(M, L[i]);
      }
      if (M == -INFINITY) {
        for (int i = 0; i < a.n; ++i) w_s[i][tid] = 0.0f;
        if (a.lse_out) a.lse_out[lse_row + s] = -INFINITY;
      } else {
        float sum = 0.0f;
        for (int i = 0; i < a.n; ++i) {
          L[i] = expf(L[i] - M);
          sum += L[i];
        }
        const float inv = 1.0f / sum;
        for (int i = 0; i < a.n; ++i) w_s[i][tid] = L[i] * inv;
        if (a.lse_out) a.lse_out[lse_row + s] = M + logf(sum);
      }
    }
  }
  __syncthreads();

  const int vpr = a.D >> 3;  // 16-byte vectors per row
  const int rows_per_pass = kThreads / vpr;
  const int c = tid % vpr;
  if (tid >= rows_per_pass * vpr) return;
  for (int row = tid / vpr; row < kRows; row += rows_per_pass) {
    const int s = s0 + row;
    if (s >= a.S) break;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < a.n; ++i) {
      const float w = w_s[i][row];
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)(a.o_in[i] + (int64_t)b * a.in_sb[i] +
                                                                 (int64_t)s * a.in_ss[i] + (int64_t)h * a.in_sh[i] + 8 * c));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += w * __uint_as_float(v[e] << 16);
        acc[2 * e + 1] += w * __uint_as_float(v[e] & 0xffff0000u);
      }
    }
    const u32x4 out = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
                       pack_bf16(acc[6], acc[7])};
    __builtin_nontemporal_store(out, (u32x4*)(a.o_out + (int64_t)b * a.out_sb + (int64_t)s * a.out_ss +
                                              (int64_t)h * a.out_sh + 8 * c));
  }
}

}  // namespace

hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t stream) {
  const int n_stiles = (a.S + kRows - 1) / kRows;
  const int64_t nblk = (int64_t)n_stiles * a.H * a.B;
  if (nblk > 0x7fffffff || a.D % 8 != 0 || a.D / 8 > kThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a, n_stiles);
  return hipGetLastError();
}

}  // namespace lsd
