// Dense bidirectional attention forward with log-sum-exp, for gfx950.
//
// Computes, per (batch b, head h, query i):
//   LSE_i = ln sum_j exp(scale * q_i . k_j),   O_i = sum_j exp(scale q_i.k_j - LSE_i) v_j
// ("Scaling Video Generation Across NVL72 rack with TensorRT-LLM", sections
// "The Scaling Challenge in Video Generation" and "Context Parallelism >
// Attention2D Parallelism > Local Attention"), with an online softmax over
// key/value tiles (the same streaming recurrence the Ring section describes
// for merging per-block results).
//
// Design (one workgroup = 8 waves = 256 query rows of one (b, h)):
// * Each wave owns 32 query rows.  Its Q rows stay in VGPRs for the whole
//   kernel as the B operand of v_mfma_f32_32x32x16_bf16.
// * Scores are computed transposed, S^T = K Q^T (A = K tile from LDS), so a
//   lane holds one query row and 16 keys of every 32-key block: the row max and
//   row sum are in-lane, with one permlane32 swap to combine the two lane halves.
// * The same accumulator registers, rounded to bf16, are directly the B operand
//   (P^T) of the PV product O^T = V^T P^T; the key order inside the 16-wide
//   reduction is permuted to match the accumulator layout, and the A operand
//   (V^T) is read from the row-major V tile with ds_read_b64_tr_b16.
// * K/V tiles of 64 keys are staged through LDS, double-buffered: the global
//   loads of tile t+1 are in flight while tile t is computed.
// * The row max is tracked lazily: O and l are rescaled only when a row's max
//   grows by more than 2^8 (in the exp2 domain), which keeps exp2 arguments
//   <= 8; the final O / l and LSE are exact for any reference max.
// * blockIdx is remapped so that consecutive query tiles of one (b, h) land on
//   the same XCD and share its L2 while streaming the same K/V.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsd_internal.h"

namespace lsd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kWaves * 32;  // query rows per workgroup
constexpr int kBlockN = 64;           // keys per LDS tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <int D>
struct Cfg {
  // LDS row pitches (elements).  K rows are skewed by 16 B so that 16 lanes
  // reading one 16-B column of 16 rows hit distinct banks; V rows by 64 B so
  // that the 4-row x 64-B footprint of a transposed read by 32 lanes does.
  static constexpr int kRowK = D + 8;
  static constexpr int kRowV = D + 32;
  static constexpr int kDSteps = D / 16;                  // QK^T reduction steps
  static constexpr int kDBlocks = D / 32;                 // O^T row blocks
  static constexpr int kChunksPerRow = D / 8;             // 16-B chunks per row
  static constexpr int kLoadsPerThread = kBlockN * kChunksPerRow / kThreads;  // per tensor
  static constexpr int kLdsK = kBlockN * kRowK;           // elements per buffer
  static constexpr int kLdsV = kBlockN * kRowV;
};

__device__ inline uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ inline float partner_max(float x) {
  // lanes l and l^32 hold the two halves of one query row
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ inline float partner_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int D>
__global__ void __launch_bounds__(kThreads)
attn_fwd_kernel(const AttnArgs a, int n_qtiles) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (C::kLdsK + C::kLdsV)];
  uint16_t* Ks = smem;                    // [2][kBlockN][kRowK]
  uint16_t* Vs = smem + 2 * C::kLdsK;     // [2][kBlockN][kRowV]

  // ---- XCD-aware tile order: dispatch is round-robin over 8 XCDs; give each
  // XCD a contiguous range of (b, h, q-tile) so its CUs share K/V in L2.
  const int nblk = gridDim.x;
  const int pid = blockIdx.x;
  const int xcd = pid & 7;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = xcd * per + min(xcd, rem) + (pid >> 3);
  const int qt = logical % n_qtiles;
  const int bh = logical / n_qtiles;
  const int h = bh % a.H;
  const int b = bh / a.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;  // lane half

  const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const uint16_t* vbase = a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;

  // ---- Q rows of this wave, as MFMA B operands (k = head channel).
  const int qrow = qt * kBlockM + wave * 32 + l32;
  const bool qvalid = qrow < a.S_q;
  bf16x8 qreg[C::kDSteps];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)qrow * a.q_ss + (int64_t)h * a.q_sh + 8 * hh;
#pragma unroll
    for (int s = 0; s < C::kDSteps; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qvalid) v = *(const u32x4*)(qp + 16 * s);
      qreg[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- global -> register staging of one K/V tile (rows beyond S_kv are zero)
  const int n_tiles = (a.S_kv + kBlockN - 1) / kBlockN;
  u32x4 kst[C::kLoadsPerThread], vst[C::kLoadsPerThread];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < C::kLoadsPerThread; ++u) {
      const int idx = tid + kThreads * u;
      const int row = idx / C::kChunksPerRow;
      const int ch = idx % C::kChunksPerRow;
      const int j = t * kBlockN + row;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (j < a.S_kv) {
        kv = *(const u32x4*)(kbase + (int64_t)j * a.k_ss + 8 * ch);
        vv = *(const u32x4*)(vbase + (int64_t)j * a.v_ss + 8 * ch);
      }
      kst[u] = kv;
      vst[u] = vv;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::kLoadsPerThread; ++u) {
      const int idx = tid + kThreads * u;
      const int row = idx / C::kChunksPerRow;
      const int ch = idx % C::kChunksPerRow;
      *(u32x4*)(Ks + buf * C::kLdsK + row * C::kRowK + 8 * ch) = kst[u];
      *(u32x4*)(Vs + buf * C::kLdsV + row * C::kRowV + 8 * ch) = vst[u];
    }
  };

  f32x16 oacc[C::kDBlocks];
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -INFINITY;  // running reference max, log2 domain
  float l_run = 0.0f;       // this lane's partial row sum
  const float c = a.scale_log2;

  // per-lane constant parts of the transposed V read address
  const int tr_i = lane & 15;
  const int tr_row = 4 * hh + (tr_i >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (tr_i & 3);

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);

    const uint16_t* Kt = Ks + buf * C::kLdsK;
    const uint16_t* Vt = Vs + buf * C::kLdsV;

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
      const uint16_t* kp = Kt + (32 * kb + l32) * C::kRowK + 8 * hh;
#pragma unroll
      for (int s = 0; s < C::kDSteps; ++s) {
        bf16x8 ka = __builtin_bit_cast(bf16x8, *(const u32x4*)(kp + 16 * s));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], sacc[kb], 0, 0, 0);
      }
    }

    // ---- mask keys beyond S_kv (last tile only)
    const int kv0 = t * kBlockN;
    if (kv0 + kBlockN > a.S_kv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (j >= a.S_kv) sacc[kb][r] = -INFINITY;
        }
    }

    // ---- online softmax (exp2 domain, lazy rescale)
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = partner_max(mx) * c;
    const float m_new = fmaxf(m_run, mx);
    const bool need = m_new > m_run + kRescaleThreshold;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = need ? m_new : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float neg_m = -m_run;
    uint32_t pk[2][8];
    // The tile's 32 weights are summed on their own before joining the running
    // sum: added one by one to a sum dominated by a few large weights (outlier
    // keys), the many small ones would fall below half an ulp and be lost.
    float lt0 = 0.0f, lt1 = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r + 1], c, neg_m));
        lt0 += p0;
        lt1 += p1;
        pk[kb][r >> 1] = pack_bf16(p0, p1);
      }
    l_run += lt0 + lt1;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 pv = {pk[kb][4 * ks + 0], pk[kb][4 * ks + 1], pk[kb][4 * ks + 2], pk[kb][4 * ks + 3]};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pv);
        const uint16_t* vp = Vt + (32 * kb + 16 * ks + tr_row) * C::kRowV + tr_col;
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db) {
          s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 32 * db));
          s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * C::kRowV + 32 * db));
          u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          u32x4 av = {lo2[0], lo2[1], hi2[0], hi2[1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb, oacc[db], 0, 0, 0);
        }
      }

    if (t + 1 < n_tiles) {
      store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: O = O^T / l, LSE = ln 2 * (m + log2 l)
  const float l_tot = partner_sum(l_run);
  if (!qvalid) return;
  const float inv = 1.0f / l_tot;
  uint16_t* op = a.o + (int64_t)b * a.o_sb + (int64_t)qrow * a.o_ss + (int64_t)h * a.o_sh + 4 * hh;
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w = {pack_bf16(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                 pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
      *(u32x2*)(op + 32 * db + 8 * g) = w;
    }
  if (a.lse != nullptr && hh == 0)
    a.lse[((int64_t)b * a.H + h) * a.S_q + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
}

// S_kv == 0: no keys, O = 0 and LSE = -inf (one thread per 8 output elements).
__global__ void attn_empty_kernel(const AttnArgs a) {
  const int64_t rows = (int64_t)a.B * a.S_q * a.H;
  const int vecs = a.D / 8;
  const int64_t n = rows * vecs;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / vecs;
    const int c = (int)(i % vecs);
    const int h = (int)(row % a.H);
    const int64_t bs = row / a.H;
    const int s = (int)(bs % a.S_q);
    const int b = (int)(bs / a.S_q);
    *(u32x4*)(a.o + (int64_t)b * a.o_sb + (int64_t)s * a.o_ss + (int64_t)h * a.o_sh + 8 * c) = (u32x4){0u, 0u, 0u, 0u};
    if (a.lse != nullptr && c == 0) a.lse[((int64_t)b * a.H + h) * a.S_q + s] = -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.S_q + kBlockM - 1) / kBlockM;
  const int64_t nblk = (int64_t)n_qtiles * a.H * a.B;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.S_kv == 0) {
    const int64_t n = (int64_t)a.B * a.S_q * a.H * (a.D / 8);
    const int blocks = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
    hipLaunchKernelGGL(attn_empty_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  switch (a.D) {
    case 64: return launch_d<64>(a, stream);
    case 128: return launch_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lsd
