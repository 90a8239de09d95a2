// Dense bidirectional attention forward on FP8 (E4M3) inputs, for gfx950.
//
// Computes the attention of the dequantised inputs q = code_q * s_q,
// k = code_k * s_k, v = code_v * s_v (s = amax / 448 per (b, h), as the FP8
// cast produces them): per query row, LSE = ln sum_j exp(scale q.k_j) and
// O = sum_j exp(scale q.k_j - LSE) v_j, O rounded to bf16
// ("Scaling Video Generation Across NVL72 rack with TensorRT-LLM", "Ulysses
// Parallelism > Fused vs. unfused QKV all-to-all": FP8 inputs for the
// attention kernel, produced by one cast of the stacked QKV; "The Scaling
// Challenge in Video Generation": dense, unmasked attention).  With a key
// count per batch entry (the key-only padding mask of "How 8 GPUs split
// tokens: what LTX-2's sequence-parallel all2all moves", "Data flow") an
// entry attends its first kv_lens[b] keys only.
//
// The structure follows the bf16 kernel (8 waves, 256 query rows per
// workgroup, key tiles double-buffered in LDS, the two waves of a SIMD
// alternating MFMA and softmax phases), with 128-key tiles (the FP8 operands
// leave the registers for them, and each barrier hand-off between the phases
// then serves twice the keys); the products run on
// v_mfma_f32_32x32x64_f8f6f4 (twice the bf16 rate).  In that instruction
// lane l (row or column l % 32) holds 32 codes of the 64-long reduction for
// lane half l / 32, and only the pairing of A and B matters, so the kernel
// chooses the reduction order:
// * QK^T: S^T = K Q^T, reduction over channels; lane half hh holds channels
//   [64 s + 32 hh, +32) of step s in both operands.
// * K rows are stored in LDS permuted (row 8 (r/4) + 4 hh + r % 4 of a 32-key
//   block holds key 16 hh + r), so accumulator register r of lane half hh is
//   the score of key 16 hh + r: each lane half holds 16 consecutive keys.
// * PV: O^T = V^T P^T, reduction over each 64-key half of the tile; byte j of
//   lane half hh is key 32 (j / 16) + 16 hh + j % 16 of the half (64-key
//   blocks of 2 x 32 keys).  The softmax weights, converted to
//   E4M3 in accumulator order, are the B operand as they stand, and the A
//   operand is two 16-byte pieces of a V^T row (V arrives transposed, keys
//   contiguous, from the cast).
// * The dequantisation factors fold into the softmax scale (s_q s_k) and the
//   final normalisation (s_v / l); weights are <= 2^8 (lazy rescaling), well
//   inside E4M3's range of 448.
// * When the logit factor c = scale log2(e) s_q s_k is a power of two (within
//   2^-20, as the cast's scale amax of Q makes the default one), the QK^T
//   products apply it exactly through the instruction's E8M0 block scales,
//   so scores arrive in log2 units.  The reference max m is then kept an
//   integer, and while |m| <= 100 a weight is exp2 of the score alone: the
//   E4M3 conversion divides by 2^m (its scale operand) and the tile's sum is
//   multiplied by 2^-m once, one VALU instruction per score fewer than
//   exp2(s c - m).  The first tile, |m| > 100 and the tiles that raise m use
//   that form.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsd_internal.h"

namespace lsd {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kWaves * 32;       // query rows per workgroup
constexpr int kBlockN = 128;               // keys per LDS tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units; keeps weights <= 2^8
constexpr int kRowK = D + 16;              // K row pitch (bytes): 16-byte skew per row
constexpr int kRowV = kBlockN + 16;        // V^T row pitch (bytes)
constexpr int kLdsK = kBlockN * kRowK;     // bytes per K buffer
constexpr int kLdsV = D * kRowV;           // bytes per V^T buffer
constexpr int kRowO = D + 4;               // output staging pitch (bf16 elements)
constexpr int kLdsO = kWaves * 32 * kRowO * 2;
constexpr int kLds = (2 * (kLdsK + kLdsV) > kLdsO) ? 2 * (kLdsK + kLdsV) : kLdsO;
constexpr int kRowA = D + 4;                // fp32 staging pitch of the accumulate epilogue
constexpr int kLdsA = kWaves * (32 * kRowA + 32) * 4;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// four float32 values -> four E4M3 codes (byte i = value i), nearest even
__device__ inline uint32_t pack4_fp8(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}
// The same, writing over a dword whose old contents do not matter (both
// halves are replaced), so no zero has to be moved in first.  The softmax
// passes the first weight's own bits as that dword: its register is free once
// the conversion has read it, so the conversions write in place.  (Passing the
// previous tile's codes instead tied the new codes to their registers, and the
// compiler then copied all 16 code registers out and back around the slow-path
// test on every tile: 32 moves per tile, 3 % of the kernel's time.)
__device__ inline uint32_t pack4_fp8_over(uint32_t old, float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

__device__ inline float vmax(float x, float y) { return __builtin_elementwise_maximum(x, y); }

__device__ inline float partner_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ inline float partner_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ inline f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// with E8M0 block scales (127 = 2^0) on both operands
__device__ inline f32x16 mfma_fp8_scaled(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
// four float32 values divided by 2^(exponent of scale) -> four E4M3 codes
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack4_fp8_scaled(uint32_t old, float a, float b, float c, float d, float scale) {
  s16x2 v = __builtin_bit_cast(s16x2, old);
  v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, a, b, scale, false);
  v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, c, d, scale, true);
  return __builtin_bit_cast(uint32_t, v);
}

// LDS row of key kk (0..63) in a K tile: within each 32-key block, key
// 16 hh + r sits in row 8 (r / 4) + 4 hh + r % 4.
__device__ inline int k_lds_row(int kk) {
  const int x = kk & 31;
  return (kk & ~31) + 8 * ((x & 15) >> 2) + 4 * (x >> 4) + (x & 3);
}

// kAcc: the fused Ring step - this block's result is merged into the running
// (o_acc, lse_acc) in the epilogue, as in the bf16 kernel.
template <bool kAcc>
__global__ void __launch_bounds__(kThreads) attn_fp8_kernel(const AttnFp8Args a, int n_qtiles) {
  constexpr int kSmem = (kAcc && kLdsA > kLds) ? kLdsA : kLds;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  uint8_t* Ks = smem;               // [2][64][kRowK] bytes, rows permuted
  uint8_t* Vs = smem + 2 * kLdsK;   // [2][D][kRowV] bytes, V^T

  // XCD-aware tile order, batch index fastest (as in the bf16 kernel).
  const int nblk = gridDim.x;
  const int pid = blockIdx.x;
  const int xcd = pid & 7;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = xcd * per + min(xcd, rem) + (pid >> 3);
  const int qt = logical % n_qtiles;
  const int hb = logical / n_qtiles;
  const int b = hb % a.B;
  const int h = hb / a.B;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // valid keys of this batch entry: all S_kv (>= 1 here), or the first
  // kv_lens[b] (the key-only padding mask, clamped to [0, S_kv])
  int skv = a.S_kv;
  if (a.kv_lens != nullptr) skv = min(max(a.kv_lens[b], 0), a.S_kv);
  if (skv == 0) {  // block-uniform: no keys for this (b, h)
    // O = 0, LSE = -inf; in accumulate mode the running result stays and O,
    // if requested, is that result in bf16 (0 where there is none)
    for (int i = tid; i < kBlockM * (D / 8); i += kThreads) {
      const int s = qt * kBlockM + i / (D / 8), c = i % (D / 8);
      if (s >= a.S_q) continue;
      const int64_t lrow = ((int64_t)b * a.H + h) * a.S_q + s;
      u32x4 out = {0u, 0u, 0u, 0u};
      if constexpr (kAcc) {
        if (a.o == nullptr) continue;
        if (a.lse_acc[lrow] != -INFINITY) {
          const f32x4* src = (const f32x4*)(a.o_acc + (((int64_t)b * a.S_q + s) * a.H + h) * D + 8 * c);
          const f32x4 x0 = src[0], x1 = src[1];
          out = (u32x4){pack_bf16(x0[0], x0[1]), pack_bf16(x0[2], x0[3]), pack_bf16(x1[0], x1[1]),
                        pack_bf16(x1[2], x1[3])};
        }
      } else if (a.lse != nullptr && c == 0) {
        a.lse[lrow] = -INFINITY;
      }
      *(u32x4*)(a.o + (int64_t)b * a.o_sb + (int64_t)s * a.o_ss + (int64_t)h * a.o_sh + 8 * c) = out;
    }
    return;
  }
  const int n_tiles = (skv + kBlockN - 1) / kBlockN;
  const float s_q = a.q_amax[b * a.H + h] / 448.0f;
  const float s_k = a.k_amax[b * a.H + h] / 448.0f;
  const float s_v = a.v_amax[b * a.H + h] / 448.0f;
  const float c = a.scale_log2 * s_q * s_k;
  // power-of-two logit factor 2^pe: E8M0 scales 127 + e1 and 127 + e2
  int cex;
  const float cm = frexpf(c, &cex);  // c = cm 2^cex, cm in [0.5, 1)
  int pe = 0;
  bool pow2 = false;
  if (fabsf(cm - 0.5f) <= 0x1p-21f) { pow2 = true; pe = cex - 1; }
  else if (fabsf(cm - 1.0f) <= 0x1p-20f) { pow2 = true; pe = cex; }
  pow2 = pow2 && pe >= -254 && pe <= 254;
  const int qk_sa = pow2 ? 127 + pe / 2 : 127;
  const int qk_sb = pow2 ? 127 + (pe - pe / 2) : 127;
  const float cs = pow2 ? 1.0f : c;  // factor still to apply to a score

  // ---- Q rows of this wave: 32 codes per lane per 64-channel step.
  const int qrow = qt * kBlockM + wave * 32 + l32;
  const bool qvalid = qrow < a.S_q;
  i32x8 qreg[2];
  {
    const uint8_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)min(qrow, a.S_q - 1) * a.q_ss +
                        (int64_t)h * a.q_sh + 32 * hh;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 lo = *(const u32x4*)(qp + 64 * s);
      u32x4 hi = *(const u32x4*)(qp + 64 * s + 16);
      if (!qvalid) lo = hi = (u32x4){0u, 0u, 0u, 0u};
      qreg[s] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  // ---- staging: each thread moves one 16-byte piece of K and of V^T per tile,
  // through buffer loads with a per-tile descriptor.  K rows past the last key
  // read as zero (their scores are masked); V^T rows are padded to a multiple
  // of 64 tokens, so a tile never leaves its rows.
  const uint8_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const uint8_t* vbase = a.vt + (int64_t)b * a.vt_sb + (int64_t)h * a.vt_sh;
  const int k_key = tid >> 3, k_ch = tid & 7;  // pieces: keys k_key and k_key + 64
  const uint32_t k_off0 = (uint32_t)(k_key * a.k_ss + 16 * k_ch);
  const uint32_t k_off1 = (uint32_t)((k_key + 64) * a.k_ss + 16 * k_ch);
  const int k_dst0 = k_lds_row(k_key) * kRowK + 16 * k_ch;
  const int k_dst1 = k_lds_row(k_key + 64) * kRowK + 16 * k_ch;
  const int v_d = tid >> 3, v_q = tid & 7;  // pieces: V^T rows v_d and v_d + 64, keys [16 v_q, +16)
  const uint32_t v_off0 = (uint32_t)(v_d * a.vt_sd + 16 * v_q);
  const uint32_t v_off1 = (uint32_t)((v_d + 64) * a.vt_sd + 16 * v_q);
  const int v_dst0 = v_d * kRowV + 16 * v_q;
  const int v_dst1 = (v_d + 64) * kRowV + 16 * v_q;
  const int v_range = (int)((D - 1) * a.vt_sd + kBlockN);  // < 2^31: row pitch < 2^24
  const uint32_t v_hi_oob = (v_q >= 4) ? 0x80000000u : 0u;  // offsets >= 2^31 lie past the range
  u32x4 kst0, kst1, vst0, vst1;
  auto load_k = [&](int t) {
    const int64_t rows = (int64_t)skv - (int64_t)t * kBlockN;
    const int64_t any = -(int64_t)(rows > 0);
    const int n = (int)(((min(rows, (int64_t)kBlockN) - 1) * a.k_ss + D) & any);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)t * kBlockN * a.k_ss), (short)0, n, 0x00020000);
    kst0 = __builtin_amdgcn_raw_buffer_load_b128(r, k_off0, 0, 0);
    kst1 = __builtin_amdgcn_raw_buffer_load_b128(r, k_off1, 0, 0);
  };
  // V^T rows are readable to S_kv rounded up to 64 tokens: where a tile's
  // second 64 keys lie past that, their pieces take an offset beyond the
  // buffer range and read as zero
  auto load_v = [&](int t) {
    const int n = (t < n_tiles) ? v_range : 0;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)t * kBlockN), (short)0, n, 0x00020000);
    const uint32_t oob = (t * kBlockN + 64 >= skv) ? v_hi_oob : 0u;  // wave-uniform choice
    vst0 = __builtin_amdgcn_raw_buffer_load_b128(r, v_off0 | oob, 0, 0);
    vst1 = __builtin_amdgcn_raw_buffer_load_b128(r, v_off1 | oob, 0, 0);
  };
  auto store_k = [&](int t) {
    *(u32x4*)(Ks + (t & 1) * kLdsK + k_dst0) = kst0;
    *(u32x4*)(Ks + (t & 1) * kLdsK + k_dst1) = kst1;
  };
  auto store_v = [&](int t) {
    *(u32x4*)(Vs + (t & 1) * kLdsV + v_dst0) = vst0;
    *(u32x4*)(Vs + (t & 1) * kLdsV + v_dst1) = vst1;
  };
  auto lds_barrier = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY;  // an integer on the power-of-two path once set
  float m_pow = 0.0f, m_inv = 0.0f, m_lim = 0.0f;  // 2^m, 2^-m, 2^(m+8) for the power-of-two path
  // wave-uniform: the power-of-two path applies (every lane's |m| <= 100);
  // m only changes in the slow path, which updates this (false until the
  // first tile has set m)
  bool fast_ok = false;
  float l_run = 0.0f;
  f32x16 sacc[4];
  uint32_t pk[16] = {};  // this tile's weights as E4M3, in PV operand order (two 64-key halves)

  auto mask_tail = [&](int t) {
    // keys of this lane's scores at or past `lim` (tile-relative) are
    // padding.  Each compare is followed by its select (the fences stop the
    // scheduler from hoisting all 64 compares, whose lane masks would then
    // spill); this runs on the last tile only.
    const int lim = skv - t * kBlockN - 16 * hh;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        __builtin_amdgcn_sched_barrier(0);
        if (32 * kb + r >= lim) sacc[kb][r] = -INFINITY;
      }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Weights E4M3-packed, with the tile's sum.  The tile's 32 weights per lane
  // are summed on their own before joining the running sum (see attn_fwd).
  auto exps = [&]() __attribute__((always_inline)) -> float {
    const float neg_m = -m_run;
    float lt0 = 0.0f, lt1 = 0.0f;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int kb = w >> 2, r = 4 * (w & 3);
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r + 0], cs, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r + 1], cs, neg_m));
      const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r + 2], cs, neg_m));
      const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r + 3], cs, neg_m));
      lt0 = (w == 0) ? p0 + p2 : lt0 + (p0 + p2);  // no 0 + x: the first pair starts the sum
      lt1 = (w == 0) ? p1 + p3 : lt1 + (p1 + p3);
      pk[w] = pack4_fp8_over(__float_as_uint(p0), p0, p1, p2, p3);
    }
    return lt0 + lt1;
  };
  // The power-of-two path's form: p = exp2(s) (scores in log2 units), codes
  // of p / 2^m; returns the tile's sum of p (not yet divided by 2^m).
  auto exps_pow = [&]() __attribute__((always_inline)) -> float {
    float lt0 = 0.0f, lt1 = 0.0f;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int kb = w >> 2, r = 4 * (w & 3);
      const float p0 = __builtin_amdgcn_exp2f(sacc[kb][r + 0]);
      const float p1 = __builtin_amdgcn_exp2f(sacc[kb][r + 1]);
      const float p2 = __builtin_amdgcn_exp2f(sacc[kb][r + 2]);
      const float p3 = __builtin_amdgcn_exp2f(sacc[kb][r + 3]);
      lt0 = (w == 0) ? p0 + p2 : lt0 + (p0 + p2);
      lt1 = (w == 0) ? p1 + p3 : lt1 + (p1 + p3);
      pk[w] = pack4_fp8_scaled(__float_as_uint(p0), p0, p1, p2, p3, m_pow);
    }
    return lt0 + lt1;
  };
  // The row max only matters when a weight against the running max would
  // exceed 2^8 (the lazy-rescale threshold); then the lane's tile sum does
  // too, or is not finite (the first tile).  So the weights are formed
  // against the running max first, and only a wave with such a lane takes
  // the row max, rescales and forms them again: the same result as always
  // taking the max, with about 20 fewer instructions per tile.
  auto softmax = [&]() __attribute__((always_inline)) {
    float lt;
    bool slow;
    // power-of-two path with |m| <= 100 (wave-uniform): exp2(s) cannot
    // overflow while weights stay <= 2^8 relative to m, nor underflow for
    // the row's larger weights
    if (fast_ok) {
      lt = exps_pow();
      slow = __any(!(lt <= m_lim));
      lt *= m_inv;
    } else {
      lt = exps();
      slow = __any(!(lt <= 256.0f));
    }
    if (slow) {
      float mx0 = sacc[0][0], mx1 = sacc[1][0], mx2 = sacc[2][0], mx3 = sacc[3][0];
#pragma unroll
      for (int r = 1; r < 15; r += 2) {
        mx0 = vmax(vmax(mx0, sacc[0][r]), sacc[0][r + 1]);
        mx1 = vmax(vmax(mx1, sacc[1][r]), sacc[1][r + 1]);
        mx2 = vmax(vmax(mx2, sacc[2][r]), sacc[2][r + 1]);
        mx3 = vmax(vmax(mx3, sacc[3][r]), sacc[3][r + 1]);
      }
      mx0 = vmax(vmax(mx0, mx1), vmax(sacc[0][15], sacc[1][15]));
      mx2 = vmax(vmax(mx2, mx3), vmax(sacc[2][15], sacc[3][15]));
      float mx = vmax(mx0, mx2);
      mx = partner_max(mx) * cs;
      const float m_new = vmax(m_run, mx);
      const bool need = m_new > m_run + kRescaleThreshold;
      if (__any(need)) {
        // the power-of-two path keeps m an integer (weights relative to it
        // stay <= 2^8), so 2^m, 2^-m and every rescale factor are exact
        const float m_set = pow2 ? ceilf(m_new) : m_new;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_set) : 1.0f;
        m_run = need ? m_set : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        if (pow2) {
          const int mi = (int)fmaxf(fminf(m_run, 120.0f), -120.0f);
          m_pow = ldexpf(1.0f, mi);
          m_inv = ldexpf(1.0f, -mi);
          m_lim = ldexpf(1.0f, mi + 8);
        }
        fast_ok = pow2 && __all(m_run >= -100.0f && m_run <= 100.0f);
      }
      lt = exps();
    }
    l_run += lt;
  };

  // ---- MFMA phase: PV(t) on 4 d-blocks x 2 key halves, then QK(t+1) on 2
  // channel steps x 4 key blocks.  Each step's A operand is two 16-byte LDS
  // reads, issued two steps ahead; sched_barrier fences keep the order.
  constexpr int kSteps = 16;
  constexpr int kDist = 2;
  auto frag_off = [&](int i, int t) -> const uint8_t* {
    if (i < 8) {  // V^T rows 32 db + l32, keys 64 j + [16 hh, +16) and 64 j + [32 + 16 hh, +16)
      const int db = i & 3, j = i >> 2;
      return Vs + (t & 1) * kLdsV + (32 * db + l32) * kRowV + 64 * j + 16 * hh;
    }
    const int jj = i - 8, s = jj >> 2, kb = jj & 3;
    return Ks + ((t + 1) & 1) * kLdsK + (32 * kb + l32) * kRowK + 64 * s + 32 * hh;
  };
  auto frag_load = [&](int i, int t) -> i32x8 {
    const uint8_t* p = frag_off(i, t);
    const u32x4 lo = *(const u32x4*)p;
    const u32x4 hi = *(const u32x4*)(p + (i < 8 ? 32 : 16));
    return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto mfma_phase = [&](int t) {
    i32x8 fr[kDist];
#pragma unroll
    for (int i = 0; i < kDist; ++i) fr[i] = frag_load(i, t);
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const i32x8 cur = fr[i % kDist];
      if (i + kDist < kSteps) fr[i % kDist] = frag_load(i + kDist, t);
      if (i < 8) {
        const int db = i & 3, j = i >> 2;
        const i32x8 pb = {(int)pk[8 * j + 0], (int)pk[8 * j + 1], (int)pk[8 * j + 2], (int)pk[8 * j + 3],
                          (int)pk[8 * j + 4], (int)pk[8 * j + 5], (int)pk[8 * j + 6], (int)pk[8 * j + 7]};
        oacc[db] = mfma_fp8(cur, pb, oacc[db]);
      } else {
        const int jj = i - 8, s = jj >> 2, kb = jj & 3;
        sacc[kb] = mfma_fp8_scaled(cur, qreg[s], s == 0 ? (f32x16){} : sacc[kb], qk_sa, qk_sb);
      }
      if (i == 1) store_k(t + 2);
      if (i == 3) store_v(t + 1);
      if (i == 6) load_k(t + 3);
      if (i == 8) load_v(t + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- ping-pong schedule (as in the bf16 kernel): group A (waves 0-3) runs
  // one barrier interval ahead of group B (waves 4-7).
  const int group = wave >> 2;
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  load_k(1);
  store_k(1);
  __syncthreads();
  load_k(2);
  load_v(1);
  {  // QK(0)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = (f32x16){};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint8_t* p = Ks + (32 * kb + l32) * kRowK + 64 * s + 32 * hh;
        const u32x4 lo = *(const u32x4*)p;
        const u32x4 hi = *(const u32x4*)(p + 16);
        const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sacc[kb] = mfma_fp8_scaled(kf, qreg[s], sacc[kb], qk_sa, qk_sb);
      }
    }
  }
  if (group == 1) lds_barrier();
  for (int t = 0; t < n_tiles; ++t) {
    if ((t + 1) * kBlockN > skv) mask_tail(t);
    softmax();
    lds_barrier();
    __builtin_amdgcn_s_setprio(1);
    mfma_phase(t);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
  }
  if (group == 0) lds_barrier();

  // ---- epilogue: O = s_v O^T / l, LSE = ln 2 (m + log2 l), O staged through LDS
  const float l_tot = partner_sum(l_run);
  const float osc = s_v / l_tot;
  constexpr float kLn2 = 0.69314718055994530942f;
  if constexpr (kAcc) {
    // Merge with the running result of earlier key blocks (exact LSE merge,
    // fp32): with M = max(LSE_acc, LSE_blk) and w = exp(LSE - M),
    //   O_acc <- (w_acc O_acc + w_blk O_blk) / (w_acc + w_blk),
    //   LSE_acc <- M + ln(w_acc + w_blk).
    // LSE_blk is finite (the block has keys), so M is; rows with no history
    // (LSE_acc = -inf) get w_acc = 0 and their O_acc is not read.  The
    // weighted block rows go through LDS (free once every wave has left the
    // loop), so the fp32 running O is read and written in whole 512-byte rows.
    const int64_t lrow = ((int64_t)b * a.H + h) * a.S_q + qrow;
    const float lse_b = (m_run + __log2f(l_tot)) * kLn2;
    const float lse_a = qvalid ? a.lse_acc[lrow] : -INFINITY;
    const float mx = fmaxf(lse_a, lse_b);
    const float wa = expf(lse_a - mx);
    const float wb = expf(lse_b - mx);
    const float rs = 1.0f / (wa + wb);
    const float ca = wa * rs, cb = wb * rs * osc;
    if (hh == 0 && qvalid) a.lse_acc[lrow] = mx + logf(wa + wb);
    __syncthreads();
    float* Aw = (float*)smem + wave * (32 * kRowA + 32);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 w = {oacc[db][4 * g + 0] * cb, oacc[db][4 * g + 1] * cb, oacc[db][4 * g + 2] * cb,
                         oacc[db][4 * g + 3] * cb};
        *(f32x4*)(Aw + l32 * kRowA + 32 * db + 8 * g + 4 * hh) = w;
      }
    if (hh == 0) Aw[32 * kRowA + l32] = ca;
    __syncthreads();
    // lane -> (row, 16-byte chunk of the row): 2 rows per pass
    constexpr int kCPRA = D / 4;
    constexpr int kRowsPerPassA = 64 / kCPRA;
    const int cha = lane % kCPRA;
    const int row_base_a = qt * kBlockM + wave * 32;
#pragma unroll 4
    for (int r = lane / kCPRA; r < 32; r += kRowsPerPassA) {
      const int row = row_base_a + r;
      if (row >= a.S_q) break;  // rows past S_q only at the end of the wave's range
      const float car = Aw[32 * kRowA + r];
      f32x4 nv = *(const f32x4*)(Aw + r * kRowA + 4 * cha);
      float* gp = a.o_acc + (((int64_t)b * a.S_q + row) * a.H + h) * D + 4 * cha;
      if (car > 0.0f) {  // history exists (w_acc > 0): O_acc holds data
        const f32x4 prev = *(const f32x4*)gp;
#pragma unroll
        for (int e = 0; e < 4; ++e) nv[e] = __builtin_fmaf(prev[e], car, nv[e]);
      }
      *(f32x4*)gp = nv;
      if (a.o != nullptr)
        *(u32x2*)(a.o + (int64_t)b * a.o_sb + (int64_t)row * a.o_ss + (int64_t)h * a.o_sh + 4 * cha) =
            (u32x2){pack_bf16(nv[0], nv[1]), pack_bf16(nv[2], nv[3])};
    }
    return;
  }
  __syncthreads();
  uint16_t* Ow = (uint16_t*)smem + wave * 32 * kRowO;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = {pack_bf16(oacc[db][4 * g + 0] * osc, oacc[db][4 * g + 1] * osc),
                       pack_bf16(oacc[db][4 * g + 2] * osc, oacc[db][4 * g + 3] * osc)};
      *(u32x2*)(Ow + l32 * kRowO + 32 * db + 8 * g + 4 * hh) = w;
    }
  if (a.lse != nullptr && hh == 0 && qvalid)
    a.lse[((int64_t)b * a.H + h) * a.S_q + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  constexpr int kCPR = D / 8;
  constexpr int kRowsPerPass = 64 / kCPR;
  const int ch = lane % kCPR;
  const int r0 = lane / kCPR;
  const int row_base = qt * kBlockM + wave * 32;
  uint16_t* obase = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + 8 * ch;
#pragma unroll
  for (int r = r0; r < 32; r += kRowsPerPass) {
    const u32x4 v = *(const u32x4*)(Ow + r * kRowO + 8 * ch);
    const int row = row_base + r;
    if (row < a.S_q) *(u32x4*)(obase + (int64_t)row * a.o_ss) = v;
  }
}

// S_kv == 0: O = 0, LSE = -inf.
__global__ void attn_fp8_empty_kernel(const AttnFp8Args a) {
  const int64_t n = (int64_t)a.B * a.S_q * a.H * (D / 8);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % (D / 8));
    const int64_t row = i / (D / 8);
    const int h = (int)(row % a.H);
    const int64_t bs = row / a.H;
    const int s = (int)(bs % a.S_q);
    const int b = (int)(bs / a.S_q);
    *(u32x4*)(a.o + (int64_t)b * a.o_sb + (int64_t)s * a.o_ss + (int64_t)h * a.o_sh + 8 * c) = (u32x4){0u, 0u, 0u, 0u};
    if (a.lse != nullptr && c == 0) a.lse[((int64_t)b * a.H + h) * a.S_q + s] = -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_fp8(const AttnFp8Args& a, hipStream_t stream) {
  if (a.S_kv == 0 && a.o_acc == nullptr) {
    const int64_t n = (int64_t)a.B * a.S_q * a.H * (D / 8);
    const int blocks = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
    hipLaunchKernelGGL(attn_fp8_empty_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const int n_qtiles = (a.S_q + kBlockM - 1) / kBlockM;
  const int64_t nblk = (int64_t)n_qtiles * a.H * a.B;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  if (a.o_acc != nullptr)  // accumulate mode (an empty block too: its rows keep the running result)
    hipLaunchKernelGGL(attn_fp8_kernel<true>, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a, n_qtiles);
  else
    hipLaunchKernelGGL(attn_fp8_kernel<false>, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

}  // namespace lsd
