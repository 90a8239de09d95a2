// Dense bidirectional attention forward with log-sum-exp, for gfx950: the
// kernel for V in the natural [B, S, H, D] layout.
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
//   reduction is permuted to match the accumulator layout.
// * V is transposed in registers on its way into LDS (key pairs packed with
//   v_perm), so each PV A operand is one 16-byte LDS read; K is stored
//   row-major.  K/V tiles of 64 keys are double-buffered in LDS and their
//   global loads are issued one iteration ahead.
// * Ping-pong: the two waves that share a SIMD run half an iteration apart, so
//   one streams MFMAs while the other does the softmax arithmetic.
// * The row max is tracked lazily: O and l are rescaled only when a row's max
//   grows by more than 2^8 (in the exp2 domain), which keeps exp2 arguments
//   <= 8; the final O / l and LSE are exact for any reference max.  A tile's
//   max is taken only when its weights against the current reference could
//   exceed 2^8, so most tiles skip it.
// * blockIdx is remapped so that consecutive query tiles of one (b, h) land on
//   the same XCD and share its L2 while streaming the same K/V.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_common.h"
#include "lsd_internal.h"

namespace lsd {
namespace {

using namespace attn;

template <int D>
struct Cfg {
  // K row pitch (elements): 16-byte skew per row, so 16 lanes reading one
  // 16-byte column of 16 consecutive rows hit distinct banks.
  static constexpr int kRowK = D + 8;
  // V is stored transposed, V^T[d][vt_pos(j)], 64 keys per row in the order the
  // PV MFMA consumes them; a pitch of 72 elements (36 dwords) makes both the
  // transposing 4-byte writes and the 16-byte operand reads conflict-free.
  static constexpr int kRowVT = 72;
  static constexpr int kDSteps = D / 16;           // QK^T reduction steps
  static constexpr int kDBlocks = D / 32;          // O^T row blocks
  static constexpr int kChunksPerRow = D / 8;      // 16-byte chunks per row
  static constexpr int kLoadsPerThread = kBlockN * kChunksPerRow / kThreads;  // K chunks per thread
  static constexpr int kLdsK = kBlockN * kRowK;    // elements per K buffer
  static constexpr int kLdsV = D * kRowVT;         // elements per V^T buffer
};

// Position of key j (0..63) inside a V^T row.  The PV MFMA's 16-wide
// reduction slot e of lane half hh carries key 8*(e/4) + 4*hh + e%4 of its
// 16-key group (the order in which the S^T accumulator holds the weights), so
// each lane half's 8 keys are stored contiguously.
__device__ __host__ constexpr int vt_pos(int j) {
  return 16 * (j >> 4) + 8 * ((j >> 2) & 1) + 4 * ((j & 15) >> 3) + (j & 3);
}

// kAcc: accumulate mode - this block's result is merged into the running
// (o_acc, lse_acc) in the epilogue (the Ring step's update, done in place).
template <int D, bool kAcc>
__global__ void __launch_bounds__(kThreads)
attn_fwd_kernel(const AttnArgs a, int n_qtiles) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (C::kLdsK + C::kLdsV)];
  uint16_t* Ks = smem;                 // [2][kBlockN][kRowK]
  uint16_t* Vs = smem + 2 * C::kLdsK;  // [2][D][kRowVT], V transposed

  // ---- XCD-aware tile order: dispatch is round-robin over 8 XCDs; give each
  // XCD a contiguous range of (h, b, q-tile) so its CUs share K/V in L2.  The
  // batch index runs fastest, so with per-batch key lengths every XCD gets
  // the same mix of long and short batch entries.
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
  const int hh = lane >> 5;  // lane half

  // Valid keys of this batch entry: all S_kv, or the first kv_lens[b] (the
  // key-only padding mask; clamped to [0, S_kv]).  Keys past skv get zero
  // weight and are never read.
  int skv = a.S_kv;
  if (a.kv_lens != nullptr) skv = min(max(a.kv_lens[b], 0), a.S_kv);
  if (skv == 0) {  // block-uniform: no keys for this (b, h)
    for (int i = threadIdx.x; i < kBlockM * (D / 8); i += kThreads) {
      const int s = qt * kBlockM + i / (D / 8);
      if (s < a.S_q) write_empty(a, b, s, h, i % (D / 8));
    }
    return;
  }

  const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const uint16_t* vbase = a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  const int n_tiles = (skv + kBlockN - 1) / kBlockN;  // >= 1

  // ---- Q rows of this wave, as MFMA B operands (k = head channel).
  const int qrow = qt * kBlockM + wave * 32 + l32;
  const bool qvalid = qrow < a.S_q;
  bf16x8 qreg[C::kDSteps];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)min(qrow, a.S_q - 1) * a.q_ss + (int64_t)h * a.q_sh + 8 * hh;
#pragma unroll
    for (int s = 0; s < C::kDSteps; ++s) {
      u32x4 v = *(const u32x4*)(qp + 16 * s);
      if (!qvalid) v = (u32x4){0u, 0u, 0u, 0u};
      qreg[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- global -> register -> LDS staging, with buffer loads.  Each tile
  // gets a buffer descriptor (built in scalar registers) whose base is the
  // tile's first row and whose byte range ends with the last valid row, so a
  // lane's offset inside the tile is fixed for the whole kernel and rows past
  // the valid keys read as zero (their scores are masked to -inf, so they get zero
  // weight).  Tiles past the end get an empty range.
  int k_row[C::kLoadsPerThread], k_ch[C::kLoadsPerThread];
  uint32_t k_off[C::kLoadsPerThread];
#pragma unroll
  for (int u = 0; u < C::kLoadsPerThread; ++u) {
    const int idx = tid + kThreads * u;
    k_row[u] = idx / C::kChunksPerRow;
    k_ch[u] = idx % C::kChunksPerRow;
    k_off[u] = (uint32_t)(k_row[u] * a.k_ss + 8 * k_ch[u]) * 2u;
  }
  // V: thread -> (key pair, 16-byte d-chunk); each wave covers all 32 pairs of
  // a tile for two chunks, which keeps the transposing writes conflict-free.
  // For D = 64 only waves 0-3 carry V.
  const int vp_pair = (tid & 63) >> 1;
  const bool v_loader = 2 * (tid >> 6) + (tid & 1) < C::kChunksPerRow;
  const int vp_chunk = v_loader ? 2 * (tid >> 6) + (tid & 1) : 0;
  const uint32_t v_off0 = (uint32_t)(2 * vp_pair * a.v_ss + 8 * vp_chunk) * 2u;
  const uint32_t v_off1 = v_off0 + (uint32_t)a.v_ss * 2u;
  u32x4 kst[2][C::kLoadsPerThread], vst[2][2];  // [tile parity]
  auto tile_bytes = [&](int t, int64_t ss) -> int {
    const int64_t rows = (int64_t)skv - (int64_t)t * kBlockN;
    const int64_t any = -(int64_t)(rows > 0);  // all ones if a row is left
    const int64_t n = ((min(rows, (int64_t)kBlockN) - 1) * ss * 2 + 2 * D) & any;
    return (int)n;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto load_k = [&](int t, auto par) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (int64_t)t * kBlockN * a.k_ss), (short)0, tile_bytes(t, a.k_ss), 0x00020000);
#pragma unroll
    for (int u = 0; u < C::kLoadsPerThread; ++u) kst[par()][u] = __builtin_amdgcn_raw_buffer_load_b128(r, k_off[u], 0, 0);
  };
  auto load_v = [&](int t, auto par) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (int64_t)t * kBlockN * a.v_ss), (short)0, tile_bytes(t, a.v_ss), 0x00020000);
    vst[par()][0] = __builtin_amdgcn_raw_buffer_load_b128(r, v_off0, 0, 0);
    vst[par()][1] = __builtin_amdgcn_raw_buffer_load_b128(r, v_off1, 0, 0);
  };
  // The loop's loads (K of tile t + 4 and V of tile t + 3 in iteration t)
  // take descriptors prepared in the softmax phase, whose wave has issue
  // slots to spare, instead of ahead of the MFMA phase's loads; 32-bit byte
  // counts (the host keeps sequence strides below 2^24 elements), scalar
  // compares, and an empty asm that keeps the work there.
  uint32_t nk_lo = 0, nk_hi = 0, nk_n = 0, nv_lo = 0, nv_hi = 0, nv_n = 0;
  auto tile_bytes32 = [&](int t, int ss) -> uint32_t {
    const int rows = skv - t * kBlockN;
    return rows >= kBlockN ? (uint32_t)((kBlockN - 1) * ss * 2 + 2 * D)
                           : (rows > 0 ? (uint32_t)((rows - 1) * ss * 2 + 2 * D) : 0u);
  };
  auto prep_loads = [&](int t) {
    const uint64_t kp = (uint64_t)(uintptr_t)(kbase + (int64_t)(t + 4) * kBlockN * a.k_ss);
    const uint64_t vp = (uint64_t)(uintptr_t)(vbase + (int64_t)(t + 3) * kBlockN * a.v_ss);
    nk_lo = __builtin_amdgcn_readfirstlane((uint32_t)kp);
    nk_hi = __builtin_amdgcn_readfirstlane((uint32_t)(kp >> 32));
    nk_n = __builtin_amdgcn_readfirstlane(tile_bytes32(t + 4, (int)a.k_ss));
    nv_lo = __builtin_amdgcn_readfirstlane((uint32_t)vp);
    nv_hi = __builtin_amdgcn_readfirstlane((uint32_t)(vp >> 32));
    nv_n = __builtin_amdgcn_readfirstlane(tile_bytes32(t + 3, (int)a.v_ss));
    asm volatile("" : "+s"(nk_lo), "+s"(nk_hi), "+s"(nk_n), "+s"(nv_lo), "+s"(nv_hi), "+s"(nv_n));
  };
  auto load_k_pre = [&](auto par) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(((uint64_t)nk_hi << 32) | nk_lo), (short)0, (int)nk_n, 0x00020000);
#pragma unroll
    for (int u = 0; u < C::kLoadsPerThread; ++u) kst[par()][u] = __builtin_amdgcn_raw_buffer_load_b128(r, k_off[u], 0, 0);
  };
  auto load_v_pre = [&](auto par) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(((uint64_t)nv_hi << 32) | nv_lo), (short)0, (int)nv_n, 0x00020000);
    vst[par()][0] = __builtin_amdgcn_raw_buffer_load_b128(r, v_off0, 0, 0);
    vst[par()][1] = __builtin_amdgcn_raw_buffer_load_b128(r, v_off1, 0, 0);
  };
  auto store_k = [&](int t, auto par) {
#pragma unroll
    for (int u = 0; u < C::kLoadsPerThread; ++u)
      *(u32x4*)(Ks + (t & 1) * C::kLdsK + k_row[u] * C::kRowK + 8 * k_ch[u]) = kst[par()][u];
  };
  // V^T[d][vt_pos(j)]: for each of the 8 channels d of the chunk, one dword
  // holding (V[2p][d], V[2p+1][d]); vt_pos keeps key pairs adjacent.
  const int vt_col = vt_pos(2 * vp_pair);
  auto store_v = [&](int t, auto par) {
    uint16_t* dst = Vs + (t & 1) * C::kLdsV + (8 * vp_chunk) * C::kRowVT + vt_col;
    if (C::kChunksPerRow == 16 || v_loader) {  // every thread carries V when D = 128
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = __builtin_amdgcn_perm(vst[par()][1][e >> 1], vst[par()][0][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
        *(uint32_t*)(dst + e * C::kRowVT) = w;
      }
    }
  };
  // Workgroup barrier that orders LDS only: outstanding global prefetches stay
  // in flight across it.
  auto lds_barrier = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  f32x16 oacc[C::kDBlocks];
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY;  // running reference max, log2 domain
  float l_run = 0.0f;       // this lane's partial row sum
  const float c = a.scale_log2;
  f32x16 sacc[2];           // S^T of the tile being processed
  uint32_t pk[2][8];        // its weights, bf16 pairs

  // ---- VALU phase SM(t): mask, row max, lazy rescale, exp
  auto mask_tail = [&](int t) {
    // Register r of key block kb holds key t kBlockN + 32 kb + 8 (r / 4) +
    // 4 hh + r % 4; it is padding from lim on.  Each select is pinned where
    // it stands (empty asm): left to the compiler, the compares all came
    // first and their lane masks spilled.
    const int lim = skv - t * kBlockN - 4 * hh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[kb][r];
        if (32 * kb + 8 * (r >> 2) + (r & 3) >= lim) x = -INFINITY;
        asm volatile("" : "+v"(x));
        sacc[kb][r] = x;
      }
  };
  // P = exp2(S c - m) rounded to bf16, with m the current reference max.  The
  // tile's 32 weights are summed on their own before joining the running sum:
  // added one by one to a sum dominated by a few large weights (outlier keys),
  // the many small ones would fall below half an ulp and be lost.
  auto exps = [&]() __attribute__((always_inline)) -> float {
    const float neg_m = -m_run;
    float lt0 = 0.0f, lt1 = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r + 1], c, neg_m));
        lt0 = (kb == 0 && r == 0) ? p0 : lt0 + p0;  // no 0 + x: the first weights start the sums
        lt1 = (kb == 0 && r == 0) ? p1 : lt1 + p1;
        pk[kb][r >> 1] = pack_bf16(p0, p1);
      }
    return lt0 + lt1;
  };
  static_assert(kRescaleThreshold == 8.0f, "the fast path bound below is 2^threshold");
  auto softmax = [&]() __attribute__((always_inline)) {
    // Fast path: weights against the current reference max.  Only when some
    // lane's weights may exceed 2^8 (their sum does, or is not finite) is the
    // row max taken: lazy rescale as described above, then the weights again.
    // Either way every weight used is at most 2^8 times the reference.
    float lt = exps();
    if (__any(!(lt <= 256.0f))) {
      // two chains of 3-input maxima (one instruction per two scores)
      float mx0 = sacc[0][0], mx1 = sacc[1][0];
#pragma unroll
      for (int r = 1; r < 15; r += 2) {
        mx0 = vmax(vmax(mx0, sacc[0][r]), sacc[0][r + 1]);
        mx1 = vmax(vmax(mx1, sacc[1][r]), sacc[1][r + 1]);
      }
      float mx = vmax(vmax(mx0, mx1), vmax(sacc[0][15], sacc[1][15]));
      mx = partner_max(mx) * c;
      const float m_new = vmax(m_run, mx);
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
      lt = exps();
    }
    l_run += lt;
    // the weights and the sum are complete here, before the barrier that ends
    // this phase (otherwise the compiler may sink their arithmetic into the
    // MFMA phase)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pk[kb][i]));
    asm volatile("" ::"v"(l_run));
  };

  // ---- MFMA phase G(t) = PV(t) then QK(t+1), as a fixed list of steps.  Step
  // i issues the LDS read of the operand that step i + kDist consumes, then its
  // own MFMA; sched_barrier fences keep this order, so kDist reads are always
  // in flight and one wave streams MFMAs back to back.  The staging of
  // K_{t+2} / V_{t+1} into LDS and the global loads of K_{t+3} / V_{t+2} ride
  // on fixed steps.
  constexpr int kPvSteps = 4 * C::kDBlocks;  // (kb, ks, db)
  constexpr int kQkSteps = 2 * C::kDSteps;   // (kb, s2)
  constexpr int kSteps = kPvSteps + kQkSteps;
  constexpr int kDist = 4;
  auto frag_ptr = [&](int i, int t) -> const uint16_t* {
    if (i < kPvSteps) {
      const int kb = i / (2 * C::kDBlocks), ks = (i / C::kDBlocks) & 1, db = i % C::kDBlocks;
      return Vs + (t & 1) * C::kLdsV + (32 * db + l32) * C::kRowVT + 8 * hh + 16 * (2 * kb + ks);
    }
    const int j = i - kPvSteps;
    const int kb = j / C::kDSteps, s2 = j % C::kDSteps;
    return Ks + ((t + 1) & 1) * C::kLdsK + (32 * kb + l32) * C::kRowK + 8 * hh + 16 * s2;
  };
  auto mfma_phase = [&](int t, auto par) {
    using P = decltype(par);
    using Q = std::integral_constant<int, 1 - P::value>;
    u32x4 fr[kDist];
#pragma unroll
    for (int i = 0; i < kDist; ++i) fr[i] = *(const u32x4*)frag_ptr(i, t);
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 cur = fr[i % kDist];
      if (i + kDist < kSteps) fr[i % kDist] = *(const u32x4*)frag_ptr(i + kDist, t);
      if (i < kPvSteps) {
        const int kb = i / (2 * C::kDBlocks), ks = (i / C::kDBlocks) & 1, db = i % C::kDBlocks;
        const u32x4 pv4 = {pk[kb][4 * ks + 0], pk[kb][4 * ks + 1], pk[kb][4 * ks + 2], pk[kb][4 * ks + 3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur),
                                                            __builtin_bit_cast(bf16x8, pv4), oacc[db], 0, 0, 0);
      } else {
        const int j = i - kPvSteps;
        const int kb = j / C::kDSteps, s2 = j % C::kDSteps;
        const f32x16 acc_in = (s2 == 0) ? (f32x16){} : sacc[kb];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur), qreg[s2], acc_in, 0, 0, 0);
      }
      // staging registers per tile parity: K(t+2) and V(t+1) leave for LDS,
      // and their slots take the loads of K(t+4) and V(t+3), two iterations
      // ahead of their stores
      if (i == 2) store_k(t + 2, P{});
      if (i == 3) store_v(t + 1, Q{});
      if (i == 6) load_k_pre(P{});
      if (i == 8) load_v_pre(Q{});
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- Ping-pong schedule.  Waves w and w+4 share a SIMD; group A (waves
  // 0-3) runs one barrier interval ahead of group B (waves 4-7), so in every
  // interval one wave of each SIMD is in its MFMA phase G(t) while the other is
  // in its VALU phase SM(t):
  //   A: QK(0) SM(0) | G(0) | SM(1) | G(1) | ...
  //   B: QK(0)       | SM(0) | G(0) | SM(1) | ...
  // LDS: K_t lives in K buffer t%2 and is read during intervals 2t-1 (A) and 2t
  // (B); V_t in V buffer t%2 during 2t+1 (A) and 2t+2 (B).  Both groups write
  // their chunks of K_{t+2} and V_{t+1} during their G(t) (intervals 2t+1 and
  // 2t+2), after every reader of those buffers has passed a barrier, and issue
  // the global loads of K_{t+3} and V_{t+2}, in flight for one iteration.  Past
  // the last tile the loads have an empty range (they return zero) and the LDS
  // writes fill buffers whose contents are never used.
  const int group = wave >> 2;
  load_k(0, I0{});
  load_v(0, I0{});
  store_k(0, I0{});
  store_v(0, I0{});
  load_k(1, I1{});
  store_k(1, I1{});
  __syncthreads();
  load_k(2, I0{});
  load_k(3, I1{});
  load_v(1, I1{});
  load_v(2, I0{});

  {  // QK(0)
    const uint16_t* kp = Ks + l32 * C::kRowK + 8 * hh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = (f32x16){};
#pragma unroll
      for (int s2 = 0; s2 < C::kDSteps; ++s2)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, *(const u32x4*)(kp + 32 * kb * C::kRowK + 16 * s2)), qreg[s2], sacc[kb], 0, 0, 0);
    }
  }
  if (group == 1) lds_barrier();
  auto iteration = [&](int t, auto par) {
    if ((t + 1) * kBlockN > skv) mask_tail(t);
    softmax();
    prep_loads(t);
    lds_barrier();
    __builtin_amdgcn_s_setprio(1);
    mfma_phase(t, par);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
  };
  for (int t = 0; t < n_tiles; t += 2) {  // unrolled by two: tile parity is a constant
    iteration(t, I0{});
    if (t + 1 < n_tiles) iteration(t + 1, I1{});
  }
  if (group == 0) lds_barrier();

  // ---- epilogue: O = O^T / l, LSE = ln 2 * (m + log2 l)
  const float l_tot = partner_sum(l_run);
  const float inv = 1.0f / l_tot;
  constexpr float kLn2 = 0.69314718055994530942f;
  if constexpr (kAcc) {
    // Merge with the running result of earlier key blocks (exact LSE merge,
    // fp32): with M = max(LSE_acc, LSE_blk) and w = exp(LSE - M),
    //   O_acc <- (w_acc O_acc + w_blk O_blk) / (w_acc + w_blk),
    //   LSE_acc <- M + ln(w_acc + w_blk).
    // LSE_blk is finite (the block has keys), so M is; rows with no history
    // (LSE_acc = -inf) get w_acc = 0 and their O_acc is not read.
    const int64_t lrow = ((int64_t)b * a.H + h) * a.S_q + qrow;
    const float lse_b = (m_run + __log2f(l_tot)) * kLn2;
    const float lse_a = qvalid ? a.lse_acc[lrow] : -INFINITY;
    const float mx = fmaxf(lse_a, lse_b);
    const float wa = expf(lse_a - mx);
    const float wb = expf(lse_b - mx);
    const float rs = 1.0f / (wa + wb);
    const float ca = wa * rs, cb = wb * rs * inv;
    if (hh == 0 && qvalid) a.lse_acc[lrow] = mx + logf(wa + wb);
    // The block's weighted rows (w_blk O_blk / (w_acc + w_blk)) go through LDS
    // (the K/V buffers are free once every wave has left the loop), half of D
    // at a time (a whole fp32 tile does not fit this kernel's LDS), so that
    // the fp32 running O is read and written in contiguous row pieces (256
    // bytes at D = 128) rather than 16-byte pieces of 32 rows.  Each wave
    // uses its own region; a row's history weight w_acc / (w_acc + w_blk)
    // comes from the lane that holds the row (lane r, r < 32).
    __syncthreads();
    constexpr int kW = D / 2;      // columns per pass
    constexpr int kRowA = kW + 4;  // pitch (floats)
    static_assert(kWaves * 32 * kRowA * 4 <= (int)sizeof(smem), "fp32 staging fits the stage buffers");
    float* Aw = (float*)smem + wave * 32 * kRowA;
    constexpr int kCPR = kW / 4;             // 16-byte chunks per row piece
    constexpr int kRowsPerPass = 64 / kCPR;  // 4 rows per pass at D = 128, 8 at D = 64
    const int ch = lane % kCPR;
    const int row_base = qt * kBlockM + wave * 32;
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
#pragma unroll
      for (int db = hp * kW / 32; db < (hp + 1) * kW / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 w = {oacc[db][4 * g + 0] * cb, oacc[db][4 * g + 1] * cb, oacc[db][4 * g + 2] * cb,
                           oacc[db][4 * g + 3] * cb};
          *(f32x4*)(Aw + l32 * kRowA + 32 * db - hp * kW + 8 * g + 4 * hh) = w;
        }
      // (this wave's LDS operations complete in order: the reads below see
      // the writes above, and the next pass's writes follow these reads)
#pragma unroll
      for (int it = 0; it < 32 / kRowsPerPass; ++it) {
        // the whole wave takes every step, so the lane shuffle reads active lanes
        const int r = it * kRowsPerPass + lane / kCPR;
        const float car = __shfl(ca, r);
        const int row = row_base + r;
        if (row >= a.S_q) continue;
        f32x4 nv = *(const f32x4*)(Aw + r * kRowA + 4 * ch);
        float* gp = a.o_acc + (((int64_t)b * a.S_q + row) * a.H + h) * D + hp * kW + 4 * ch;
        if (car > 0.0f) {  // history exists (w_acc > 0): O_acc holds data
          const f32x4 prev = *(const f32x4*)gp;
#pragma unroll
          for (int e = 0; e < 4; ++e) nv[e] = __builtin_fmaf(prev[e], car, nv[e]);
        }
        *(f32x4*)gp = nv;
        if (a.o != nullptr)
          *(u32x2*)(a.o + (int64_t)b * a.o_sb + (int64_t)row * a.o_ss + (int64_t)h * a.o_sh + hp * kW + 4 * ch) =
              (u32x2){pack_bf16(nv[0], nv[1]), pack_bf16(nv[2], nv[3])};
      }
    }
    return;
  }
  // Stage this wave's 32 x D output tile through LDS (the K/V buffers are free
  // once every wave has left the loop) so that global stores write whole
  // 256-byte rows instead of 8-byte pieces of 32 different rows.
  __syncthreads();
  constexpr int kRowO = D + 4;  // pitch (elements): rows land on distinct bank pairs
  uint16_t* Ow = smem + wave * 32 * kRowO;
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w = {pack_bf16(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                 pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
      *(u32x2*)(Ow + l32 * kRowO + 32 * db + 8 * g + 4 * hh) = w;
    }
  if (a.lse != nullptr && hh == 0 && qvalid)
    a.lse[((int64_t)b * a.H + h) * a.S_q + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  // rows are written by 64 lanes: lane = (row r in 0..64/CPR-1, 16-B chunk)
  constexpr int kCPR = D / 8;  // 16-byte chunks per row
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

// S_kv == 0: no keys anywhere (one thread per 8 output elements).
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
    write_empty(a, b, s, h, c);
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.S_q + kBlockM - 1) / kBlockM;
  const int64_t nblk = (int64_t)n_qtiles * a.H * a.B;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  if (a.o_acc != nullptr)
    hipLaunchKernelGGL((attn_fwd_kernel<D, true>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, a, n_qtiles);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, false>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.S_kv != 0 && a.v_tok) return launch_attn_fwd_vt(a, stream);
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
