// Pieces shared by the two attention kernels (V in the natural layout,
// attn_fwd.hip; V token-contiguous, attn_fwd_vt.hip): vector types, the
// workgroup shape, bf16 packing, the lane-pair reductions and the output of a
// query row whose (b, h) has no keys.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsd_internal.h"

namespace lsd {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kWaves * 32;       // query rows per workgroup
constexpr int kBlockN = 64;                // keys per LDS tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units

__device__ inline uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// IEEE maximum: lowers to v_maximum3_f32 without the NaN-quieting copies that
// fmaxf needs for MFMA results (NaN inputs are outside the contract anyway).
__device__ inline float vmax(float x, float y) { return __builtin_elementwise_maximum(x, y); }

__device__ inline float partner_max(float x) {
  // lanes l and l^32 hold the two halves of one query row
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ inline float partner_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Output of one query row's 16-byte chunk c when its (b, h) has no keys:
// O = 0 and LSE = -inf; in accumulate mode the running result is unchanged
// and O, if requested, is that running result in bf16 (0 where there is none).
__device__ inline void write_empty(const AttnArgs& a, int b, int s, int h, int c) {
  const int64_t row = ((int64_t)b * a.S_q + s) * a.H + h;
  const int64_t lrow = ((int64_t)b * a.H + h) * a.S_q + s;
  u32x4 out = {0u, 0u, 0u, 0u};
  if (a.o_acc != nullptr) {
    if (a.o == nullptr) return;
    if (a.lse_acc[lrow] != -INFINITY) {
      const f32x4* src = (const f32x4*)(a.o_acc + row * a.D + 8 * c);
      const f32x4 x0 = src[0], x1 = src[1];
      out = (u32x4){pack_bf16(x0[0], x0[1]), pack_bf16(x0[2], x0[3]), pack_bf16(x1[0], x1[1]),
                    pack_bf16(x1[2], x1[3])};
    }
  } else if (a.lse != nullptr && c == 0) {
    a.lse[lrow] = -INFINITY;
  }
  *(u32x4*)(a.o + (int64_t)b * a.o_sb + (int64_t)s * a.o_ss + (int64_t)h * a.o_sh + 8 * c) = out;
}

}  // namespace attn
}  // namespace lsd
