// Dense bidirectional attention forward with log-sum-exp, for gfx950: the
// kernel for V given token-contiguous (each channel's keys one row, the
// layout the Ulysses relayout can write), whose K and V tiles are staged with
// direct global->LDS loads.
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
// * K rows are stored in LDS with bits 2 and 3 of the key index swapped, which
//   makes accumulator register r of lane half hh score key 16(r/8) + 8hh + r%8:
//   rounded to bf16, the same registers are directly the B operand (P^T) of the
//   PV product O^T = V^T P^T, and the matching A operand is a plain 16-byte
//   read of a V^T row in natural key order.
// * K and V^T tiles reach LDS with buffer loads that write LDS directly (no
//   VGPR staging, no LDS store instructions); 64-key tiles rotate through four
//   LDS stage buffers, loaded three iterations ahead of use.
// * Ping-pong: the two waves that share a SIMD run half an iteration apart, so
//   one streams MFMAs while the other does the softmax arithmetic.
// * The row max is tracked lazily: O and l are rescaled only when a row's max
//   grows by more than 2^8 (in the exp2 domain), which keeps exp2 arguments
//   <= 8; the final O / l and LSE are exact for any reference max.  A tile's
//   max is taken only when its weights against the current reference could
//   exceed 2^8, so most tiles skip it.
// * The MFMA phase issues the next tiles' direct loads from inline assembly
//   with every operand already scalar (one M0 write per pair of loads, their
//   byte ranges and validity worked out in the softmax phase), because each
//   non-MFMA instruction in that phase delays the MFMA stream; the two
//   phases now take about equally long.
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

constexpr int kStages = 4;                 // LDS stage buffers

template <int D>
struct Cfg {
  static constexpr int kDSteps = D / 16;           // QK^T reduction steps
  static constexpr int kDBlocks = D / 32;          // O^T row blocks
  static constexpr int kCPR = D / 8;               // 16-byte chunks per K row
  static constexpr int kRowsPerLine = 16 / kCPR;   // K rows per 256 bytes
  static constexpr int kDma = D / 64;              // direct loads per thread per K (or V^T) tile
  static constexpr int kTileBytes = kBlockN * D * 2;   // one K or V^T tile (V^T rows of 128 bytes)
  static constexpr int kVBytes = kTileBytes;
  static constexpr int kVRegion = kStages * kTileBytes;  // V^T buffers start here
  // one more V^T-shaped area holds the last tile's chunk that straddles the
  // key count (see the staging notes in the kernel)
  static constexpr int kSide = kVRegion + kStages * kVBytes;
  static constexpr int kLdsBytes = kSide + kVBytes;
};

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer straight into LDS, lane i's bytes at
// lds + 16 i (lds must be wave-uniform; lanes out of the buffer's range write
// zeros).  The builtin exists in the device pass only.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
#endif
}

// The same load issued from inline assembly with M0 computed by a scalar add
// (LDS address = wbase + off): no vector-to-scalar moves on the way to M0.
// One wait state separates the M0 write from the load that reads it.  The
// compiler does not see these loads; their completion is awaited with
// explicit s_waitcnt vmcnt.
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
template <int kOff>
__device__ inline void dma16_asm(const u32x4s& rs, uint32_t wbase, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds"
               :: "s"(wbase), "i"(kOff), "v"(voff), "s"(rs) : "memory", "scc", "m0");
#endif
}

// Two such loads into consecutive 1 KB slots with one M0 write: the second
// takes the immediate offset 1024, which moves its LDS and buffer addresses
// alike, so its lane offsets come in reduced by 1024 (each must be at least
// 1024).  Bit-identical to two single loads and 0.3 % faster (one M0 write
// and wait state fewer per pair in the MFMA phase).
template <int kOff>
__device__ inline void dma16_asm_pair(const u32x4s& rs, uint32_t wbase, uint32_t voff0, uint32_t voff1m) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile(
      "s_add_u32 m0, %0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %4, 0 offen lds\n\t"
      "buffer_load_dwordx4 %3, %4, 0 offen offset:1024 lds"
      :: "s"(wbase), "i"(kOff), "v"(voff0), "v"(voff1m), "s"(rs) : "memory", "scc", "m0");
#endif
}

// Key held by LDS row rho of a K tile: bits 2 and 3 swapped (an involution).
__device__ inline int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// kAcc: accumulate mode - this block's result is merged into the running
// (o_acc, lse_acc) in the epilogue (the Ring step's update, done in place).
// kVPair: the V^T row pitch is at least 64 keys, so the two V^T loads of a
// thread share one M0 write (see dma16_asm_pair).
template <int D, bool kAcc, bool kVPair>
__global__ void __launch_bounds__(kThreads)
attn_fwd_vt_kernel(const AttnArgs a, int n_qtiles) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::kLdsBytes / 2];
  uint8_t* const lds = (uint8_t*)smem;

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS addresses in SGPRs
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

  // ---- Staging.  Stage buffer s (s % kStages) holds K_{s+1} in the K region
  // and V_s in the V region: the two tiles G(s) reads.  Every load goes
  // through a buffer descriptor per tile; lanes out of its range write zeros.
  // K: direct loads, 1 KB of LDS per wave instruction.  A K tile's range ends
  // with the last valid key (rows past it are zero; tiles past the end get an
  // empty range).  LDS row rho holds key swap23(rho); its 16-byte chunks are
  // XOR-swizzled by row so that 16 lanes reading one chunk of 16 rows hit
  // distinct banks.
  uint32_t k_voff[C::kDma];
#pragma unroll
  for (int u = 0; u < C::kDma; ++u) {
    const int g = wave * C::kDma + u;
    const int rho = g * (64 / C::kCPR) + lane / C::kCPR;
    const int kc = (lane % C::kCPR) ^ ((rho / C::kRowsPerLine) % C::kCPR);
    k_voff[u] = (uint32_t)(swap23(rho) * (int)a.k_ss + 8 * kc) * 2u;
  }
  auto tile_bytes = [&](int t, int64_t ss) -> int {
    const int64_t rows = (int64_t)skv - (int64_t)t * kBlockN;
    const int64_t any = -(int64_t)(rows > 0);  // all ones if a row is left
    const int64_t n = ((min(rows, (int64_t)kBlockN) - 1) * ss * 2 + 2 * D) & any;
    return (int)n;
  };
  auto dma_k = [&](int t, uint8_t* dst) {  // K tile t -> dst
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (int64_t)t * kBlockN * a.k_ss), (short)0, tile_bytes(t, a.k_ss), 0x00020000);
#pragma unroll
    for (int u = 0; u < C::kDma; ++u) dma16(r, dst + (wave * C::kDma + u) * 1024, k_voff[u]);
  };
  uint8_t* const vregion = lds + C::kVRegion;
  // V^T: direct loads of 128-byte rows (64 keys of one channel),
  // 16-byte chunks XOR-swizzled by row pair.  A chunk is loaded only when all
  // 8 of its keys are valid.  When the key count is not a multiple of 8, the
  // last tile's chunk that straddles it is written once, before the loop,
  // into a side area of the same shape (valid keys, then zeros), and in the
  // last iteration the lanes that read that chunk are pointed there.
  uint32_t v_voff[C::kDma];
  int v_key[C::kDma];
#pragma unroll
  for (int u = 0; u < C::kDma; ++u) {
    const int d = (wave * C::kDma + u) * 8 + lane / 8;
    const int vc = (lane % 8) ^ ((d >> 1) & 7);
    v_voff[u] = (uint32_t)(d * (int)a.v_sd + 8 * vc) * 2u;
    v_key[u] = 8 * vc;
  }
  const int vt_range = (int)(((int64_t)(D - 1) * a.v_sd + kBlockN) * 2);
  auto dma_v = [&](int t, uint8_t* dst) {  // V^T tile t -> dst
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (int64_t)t * kBlockN), (short)0, vt_range, 0x00020000);
#pragma unroll
    for (int u = 0; u < C::kDma; ++u) {
      const uint32_t off = (t * kBlockN + v_key[u] + 8 <= skv) ? v_voff[u] : 0x7ffffff0u;
      dma16(r, dst + (wave * C::kDma + u) * 1024, off);
    }
  };
  // Inside the loop the loads walk the tiles in order, so their tile pointers
  // and key counts are running scalars, and every LDS destination is a scalar
  // too: no vector-to-scalar moves feed M0 in the MFMA phase.
  const int64_t k_tile_step = (int64_t)kBlockN * a.k_ss;
  // buffer descriptors of the next K and V^T tiles, advanced in place
  const uint64_t k_first = (uint64_t)(uintptr_t)(kbase + kStages * k_tile_step);  // K_{t+4} in iteration t
  u32x4s rk = {(uint32_t)k_first, (uint32_t)(k_first >> 32) & 0xffffu, 0u, 0x00020000u};
  const uint64_t k_step = (uint64_t)k_tile_step * 2;
  int k_rows_next = skv - kStages * kBlockN;
  // byte range of a full K tile (fits in 31 bits: the host keeps k_ss < 2^24)
  const uint32_t k_full = (uint32_t)((kBlockN - 1) * (int)a.k_ss * 2 + 2 * D);
  // this wave's 1 KB slots of a tile (the low 32 bits of a flat pointer into
  // LDS are the LDS address); scalar, since wave is
  const uint32_t wbase = (uint32_t)(uintptr_t)lds + (uint32_t)wave * C::kDma * 1024;
  auto advance = [](u32x4s& r, uint64_t step) {  // 48-bit base: the high word stays below 2^16
    const uint64_t p = (((uint64_t)r[1] << 32) | r[0]) + step;
    r[0] = (uint32_t)p;
    r[1] = (uint32_t)(p >> 32);
  };
  auto dma_k_next = [&](auto off_c) {
    constexpr int kOff = decltype(off_c)::value;
    // (rk[2], the tile's byte range, was set in the softmax phase)
    // (a second slot's K rows lie 8 or more token strides in: offset >= 2048)
    if constexpr (C::kDma > 1) dma16_asm_pair<kOff>(rk, wbase, k_voff[0], k_voff[1] - 1024u);
    else dma16_asm<kOff>(rk, wbase, k_voff[0]);
    advance(rk, k_step);
    k_rows_next -= kBlockN;
  };
  const uint64_t v_first = (uint64_t)(uintptr_t)(vbase + (kStages - 1) * kBlockN);  // V_{t+3} in iteration t
  u32x4s rv = {(uint32_t)v_first, (uint32_t)(v_first >> 32) & 0xffffu, (uint32_t)vt_range, 0x00020000u};
  int v_key_next = (kStages - 1) * kBlockN;
  int v_full = 0;
  // Scalar bookkeeping of the next loads, done in the softmax phase (whose
  // wave has issue slots to spare) rather than ahead of the first MFMA of the
  // MFMA phase; the empty asm keeps it there.
  auto prep_next = [&]() {
    const int rows = k_rows_next;
    rk[2] = __builtin_amdgcn_readfirstlane(
        rows >= kBlockN ? k_full : (rows > 0 ? (uint32_t)((rows - 1) * (int)a.k_ss * 2 + 2 * D) : 0u));
    v_full = __builtin_amdgcn_readfirstlane((v_key_next + kBlockN <= skv) ? 1 : 0);
    asm volatile("" : "+s"(rk[2]), "+s"(v_full));
  };
  auto dma_v_next = [&](auto off_c) {
    constexpr int kOff = decltype(off_c)::value;
    auto issue = [&](uint32_t o0, uint32_t o1) {
      // a second slot's V^T rows lie 8 or more row pitches in: offset >= 1024
      // once the pitch is at least 64 keys
      if constexpr (C::kDma > 1) {
        if constexpr (kVPair) dma16_asm_pair<kOff>(rv, wbase, o0, o1 - 1024u);
        else {
          dma16_asm<kOff>(rv, wbase, o0);
          dma16_asm<kOff + 1024>(rv, wbase, o1);
        }
      } else {
        dma16_asm<kOff>(rv, wbase, o0);
      }
    };
    if (v_full) {  // uniform: every chunk of the tile is valid (set in the softmax phase)
      issue(v_voff[0], C::kDma > 1 ? v_voff[C::kDma - 1] : 0u);
    } else {
      auto voff = [&](int u) { return (v_key_next + v_key[u] + 8 <= skv) ? v_voff[u] : 0x7ffffff0u; };
      issue(voff(0), C::kDma > 1 ? voff(C::kDma - 1) : 0u);
    }
    advance(rv, (uint64_t)kBlockN * 2);
    v_key_next += kBlockN;
  };
  // Each lane's fragment addresses (row l32), before stage and row-block
  // offsets: kfa[s2] for QK step s2, vfa[2 kb + ks] for the PV keys
  // 32 kb + 16 ks + 8 hh .. + 7.
  const uint8_t* kfa[C::kDSteps];
  const uint8_t* vfa[4];
#pragma unroll
  for (int s2 = 0; s2 < C::kDSteps; ++s2)
    kfa[s2] = lds + l32 * (2 * D) + 16 * ((2 * s2 + hh) ^ ((l32 / C::kRowsPerLine) % C::kCPR));
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4)
    vfa[c4] = vregion + l32 * 128 + 16 * ((2 * c4 + hh) ^ ((l32 >> 1) & 7));
  constexpr int kVRowBlock = 32 * 128;  // bytes per 32 V^T rows
  // Workgroup barrier that orders LDS accesses.  Direct loads in flight stay
  // in flight across it: each wave awaits its own with s_waitcnt vmcnt.
  auto lds_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

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
    // Register r of key block kb holds key t kBlockN + 32 kb + 16 (r / 8) +
    // 8 hh + r % 8; it is padding from lim on.  Each select is pinned where
    // it stands (empty asm): left to the compiler, the compares all came
    // first and their lane masks spilled.
    const int lim = skv - t * kBlockN - 8 * hh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[kb][r];
        if (32 * kb + 16 * (r >> 3) + (r & 7) >= lim) x = -INFINITY;
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
  // in flight and one wave streams MFMAs back to back.  Loads for later tiles
  // ride on fixed steps.
  constexpr int kPvSteps = 4 * C::kDBlocks;  // (kb, ks, db)
  constexpr int kQkSteps = 2 * C::kDSteps;   // (kb, s2)
  constexpr int kSteps = kPvSteps + kQkSteps;
  constexpr int kDist = 6;
  auto frag = [&](int i, auto st) -> u32x4 {
    constexpr int S = decltype(st)::value;
    if (i < kPvSteps) {
      const int kb = i / (2 * C::kDBlocks), ks = (i / C::kDBlocks) & 1, db = i % C::kDBlocks;
      return *(const u32x4*)(vfa[2 * kb + ks] + S * C::kVBytes + db * kVRowBlock);
    }
    const int j = i - kPvSteps;
    const int kb = j / C::kDSteps, s2 = j % C::kDSteps;
    return *(const u32x4*)(kfa[s2] + S * C::kTileBytes + 32 * kb * (2 * D));
  };
  // Stage t+3 (K_{t+4}, V_{t+3}) goes into the buffer stage t-1 used, free
  // once both groups have passed G(t-1).  At the end the wave waits for its
  // own loads of stage t+2 (only stage t+3 may stay in flight), so that stage
  // t+2 is published before either group starts SM(t+2): each wave then reads
  // the first kDist fragments of G(t) at the end of SM(t), before the barrier,
  // and G(t) starts without waiting on LDS latency (2 % faster).
  constexpr int kInFlight = (kStages - 3) * 2 * C::kDma;
  u32x4 fr[kDist];
  auto prefetch = [&](auto st) {
#pragma unroll
    for (int i = 0; i < kDist; ++i) fr[i] = frag(i, st);
  };
  auto mfma_phase = [&](int t, auto st) {
    constexpr int S = decltype(st)::value;
    constexpr int kFree = (S + kStages - 1) % kStages;
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 cur = fr[i % kDist];
      if (i + kDist < kSteps) fr[i % kDist] = frag(i + kDist, st);
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
      if (i == 4) dma_k_next(std::integral_constant<int, kFree * C::kTileBytes>{});
      if (i == 12) dma_v_next(std::integral_constant<int, C::kVRegion + kFree * C::kVBytes>{});
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kInFlight) : "memory");
  };

  // ---- Ping-pong schedule.  Waves w and w+4 share a SIMD; group A (waves
  // 0-3) runs one barrier interval ahead of group B (waves 4-7), so in every
  // interval one wave of each SIMD is in its MFMA phase G(t) while the other is
  // in its VALU phase SM(t):
  //   A: QK(0) SM(0) | G(0) | SM(1) | G(1) | ...
  //   B: QK(0)       | SM(0) | G(0) | SM(1) | ...
  // G(t) reads stage t during intervals 2t+1 (A) and 2t+2 (B); each group loads
  // its half of stage t+3 during its G(t) into the buffer of stage t-1, whose
  // last reader finished in interval 2t, and has its half of stage t+2 landed
  // by the end of its G(t) (interval 2t+2 at the latest), before SM(t+2)
  // starts for either group.  K_0, read by QK(0) only, sits in the V buffer
  // of stage 3, first loaded in G(0).
  // Past the last tile the loads have an empty range (they write zeros) into
  // buffers whose contents are never used.
  const int group = wave >> 2;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  static_assert(C::kDma <= 2, "one or two direct loads per wave and tile");
  static_assert(kStages == 4, "the main loop is unrolled for four stage buffers");
  uint8_t* const k0 = vregion + (kStages - 1) * C::kVBytes;
  dma_k(0, k0);
  {
#pragma unroll
    for (int s0 = 0; s0 < kStages - 1; ++s0) {
      dma_k(s0 + 1, lds + s0 * C::kTileBytes);
      dma_v(s0, vregion + s0 * C::kVBytes);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kInFlight) : "memory");  // K_0, stages 0 and 1 landed
    if ((skv & 7) != 0 && tid < D) {  // side chunk of channel d = tid
      const int c_s = (skv & (kBlockN - 1)) >> 3, key0 = skv & ~7;
      const uint16_t* src = vbase + (int64_t)tid * a.v_sd + key0;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (key0 + 2 * e < skv) ? src[2 * e] : 0u;
        const uint32_t hi = (key0 + 2 * e + 1 < skv) ? src[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      *(u32x4*)(lds + C::kSide + tid * 128 + 16 * (c_s ^ ((tid >> 1) & 7))) = (u32x4){w[0], w[1], w[2], w[3]};
    }
  }
  __syncthreads();

  {  // QK(0)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = (f32x16){};
#pragma unroll
      for (int s2 = 0; s2 < C::kDSteps; ++s2)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, *(const u32x4*)(kfa[s2] - lds + k0 + 32 * kb * (2 * D))), qreg[s2], sacc[kb], 0, 0, 0);
    }
  }
  if (group == 1) lds_barrier();
  auto iteration = [&](int t, auto st) {
    if ((t + 1) * kBlockN > skv) {
      mask_tail(t);
      if ((skv & 7) != 0) {  // last tile: the straddling chunk comes from the side area
        const int c_s = (skv & (kBlockN - 1)) >> 3;
        const int delta = C::kSide - C::kVRegion - decltype(st)::value * C::kVBytes;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
          if (2 * c4 + hh == c_s) vfa[c4] += delta;
      }
    }
    softmax();
    prep_next();
    prefetch(st);  // stage t was published before SM(t) began
    // No LDS wait before this barrier: the wave has written no LDS in SM(t),
    // and its prefetch reads of stage t need not land before the other group
    // proceeds (nobody writes that buffer until both groups have left G(t)).
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_s_setprio(1);
    mfma_phase(t, st);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
  };
  for (int t = 0; t < n_tiles; t += kStages) {  // unrolled: the stage buffer is a constant
    iteration(t, I0{});
    if (t + 1 < n_tiles) iteration(t + 1, I1{});
    if (t + 2 < n_tiles) iteration(t + 2, I2{});
    if (t + 3 < n_tiles) iteration(t + 3, I3{});
  }
  if (group == 0) lds_barrier();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads past the end still land in LDS

  // ---- epilogue: O = O^T / l, LSE = ln 2 * (m + log2 l)
  const float l_tot = partner_sum(l_run);
  const float inv = 1.0f / l_tot;
  constexpr float kLn2 = 0.69314718055994530942f;
  const float osc = inv;  // scale from oacc to the output values
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
    // (the K/V stage buffers are free once every wave has left the loop), so
    // that the fp32 running O is read and written in whole 512-byte rows
    // rather than 16-byte pieces of 32 rows.  Per wave: 32 rows of D floats
    // (pitch D + 4) and the rows' history weights w_acc / (w_acc + w_blk).
    __syncthreads();
    constexpr int kRowA = D + 4;
    static_assert(kWaves * (32 * kRowA + 32) * 4 <= C::kLdsBytes, "fp32 staging fits the stage buffers");
    float* Aw = (float*)smem + wave * (32 * kRowA + 32);
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 w = {oacc[db][4 * g + 0] * cb, oacc[db][4 * g + 1] * cb, oacc[db][4 * g + 2] * cb,
                         oacc[db][4 * g + 3] * cb};
        *(f32x4*)(Aw + l32 * kRowA + 32 * db + 8 * g + 4 * hh) = w;
      }
    if (hh == 0) Aw[32 * kRowA + l32] = ca;
    __syncthreads();
    // lane -> (row, 16-byte chunk of the row): 2 rows per pass at D = 128
    constexpr int kCPR = D / 4;
    constexpr int kRowsPerPass = 64 / kCPR;
    const int ch = lane % kCPR;
    const int row_base = qt * kBlockM + wave * 32;
#pragma unroll 4
    for (int r = lane / kCPR; r < 32; r += kRowsPerPass) {
      const int row = row_base + r;
      if (row >= a.S_q) break;  // rows past S_q only at the end of the wave's range
      const float car = Aw[32 * kRowA + r];
      f32x4 nv = *(const f32x4*)(Aw + r * kRowA + 4 * ch);
      float* gp = a.o_acc + (((int64_t)b * a.S_q + row) * a.H + h) * D + 4 * ch;
      if (car > 0.0f) {  // history exists (w_acc > 0): O_acc holds data
        const f32x4 prev = *(const f32x4*)gp;
#pragma unroll
        for (int e = 0; e < 4; ++e) nv[e] = __builtin_fmaf(prev[e], car, nv[e]);
      }
      *(f32x4*)gp = nv;
      if (a.o != nullptr)
        *(u32x2*)(a.o + (int64_t)b * a.o_sb + (int64_t)row * a.o_ss + (int64_t)h * a.o_sh + 4 * ch) =
            (u32x2){pack_bf16(nv[0], nv[1]), pack_bf16(nv[2], nv[3])};
    }
    return;
  }
  // Stage this wave's 32 x D output tile through LDS (the K/V buffers are free
  // once every wave has left the loop) so that global stores write whole
  // 256-byte rows instead of 8-byte pieces of 32 different rows.
  __syncthreads();
  constexpr int kRowO = D + 8;  // pitch (elements): 16-byte aligned rows, 4-bank skew per row
  uint16_t* Ow = smem + wave * 32 * kRowO;
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w = {pack_bf16(oacc[db][4 * g + 0] * osc, oacc[db][4 * g + 1] * osc),
                 pack_bf16(oacc[db][4 * g + 2] * osc, oacc[db][4 * g + 3] * osc)};
      *(u32x2*)(Ow + l32 * kRowO + 32 * db + 8 * g + 4 * hh) = w;
    }
  if (!kAcc && a.lse != nullptr && hh == 0 && qvalid)
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

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.S_q + kBlockM - 1) / kBlockM;
  const int64_t nblk = (int64_t)n_qtiles * a.H * a.B;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (D > 64) {  // one direct load per thread and tile at D = 64: nothing to pair
    if (a.v_sd >= 64) {
      if (a.o_acc != nullptr)
        hipLaunchKernelGGL((attn_fwd_vt_kernel<D, true, true>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, a,
                           n_qtiles);
      else
        hipLaunchKernelGGL((attn_fwd_vt_kernel<D, false, true>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, a,
                           n_qtiles);
      return hipGetLastError();
    }
  }
  if (a.o_acc != nullptr)
    hipLaunchKernelGGL((attn_fwd_vt_kernel<D, true, false>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, a, n_qtiles);
  else
    hipLaunchKernelGGL((attn_fwd_vt_kernel<D, false, false>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_vt(const AttnArgs& a, hipStream_t stream) {
  if (a.S_kv == 0 || !a.v_tok) return hipErrorInvalidValue;  // launch_attn_fwd handles these
  switch (a.D) {
    case 64: return launch_d<64>(a, stream);
    case 128: return launch_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lsd
