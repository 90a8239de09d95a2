// Internal launch interface between the C-ABI validation layer (api.cpp) and
// the HIP kernels.  Not installed; the public interface is include/lsd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsd {

// Attention forward.  Strides are in elements; D (head channels) contiguous.
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;        // may be null in accumulate mode
  float* lse;         // [B, H, S_q] contiguous, may be null
  // Accumulate mode (both non-null): the running result of earlier key
  // blocks, read and replaced by its merge with this block's result.
  float* o_acc;       // [B, S_q, H, D] fp32 contiguous
  float* lse_acc;     // [B, H, S_q] fp32 contiguous
  // Key-only padding mask: batch entry b attends its first kv_lens[b] keys
  // (device array of B values, clamped to [0, S_kv]); null = all S_kv keys.
  const int32_t* kv_lens;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  // v_tok = 1: V is token-contiguous (stride of the sequence dim is 1), each
  // channel's keys a row of pitch v_sd elements (V^T per head); 0: natural.
  int64_t v_sd;
  int v_tok;
  int64_t o_sb, o_ss, o_sh;
  int B, H, S_q, S_kv, D;
  float scale_log2;  // softmax scale * log2(e)
};
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream);
// The kernel for a token-contiguous V (v_tok = 1, S_kv > 0); launch_attn_fwd
// dispatches to it.
hipError_t launch_attn_fwd_vt(const AttnArgs& a, hipStream_t stream);

constexpr int kMaxMerge = 16;

struct MergeArgs {
  const uint16_t* o_in[kMaxMerge];
  int64_t in_sb[kMaxMerge], in_ss[kMaxMerge], in_sh[kMaxMerge];
  const float* lse_in[kMaxMerge];
  uint16_t* o_out;
  int64_t out_sb, out_ss, out_sh;
  float* lse_out;  // may be null
  int n, B, S, H, D;
};
hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t stream);

constexpr int kMaxRelayoutTensors = 3;
constexpr int kMaxRelayoutP = 16;

struct RelayoutArgs {
  const uint16_t* src[kMaxRelayoutTensors][kMaxRelayoutP];
  int64_t src_sb[kMaxRelayoutTensors][kMaxRelayoutP];
  int64_t src_ss[kMaxRelayoutTensors][kMaxRelayoutP];
  int64_t src_sh[kMaxRelayoutTensors][kMaxRelayoutP];
  uint16_t* dst[kMaxRelayoutTensors];
  int64_t dst_sb[kMaxRelayoutTensors], dst_ss[kMaxRelayoutTensors], dst_sh[kMaxRelayoutTensors];
  // Token-contiguous destinations (launch_relayout_tok): dst_ss is 1 and
  // dst_sd the row pitch, each channel's tokens one row.
  int64_t dst_sd[kMaxRelayoutTensors];
  int n_tensors, P, rank, B, S_loc, H_loc, D;
  int heads_per_run;  // H_loc when every head slice is contiguous in src and dst, else 1
  // 0: sequence-major shards -> head-major slice (src[t][p] is shard p of the
  //    sequence, (B, S_loc, H, D); dst[t] is (B, P*S_loc, H_loc, D)).
  // 1: the inverse, head-major slices -> sequence shard (src[t][r] is rank
  //    r's slice, (B, P*S_loc, H_loc, D); dst[t] is (B, S_loc, P*H_loc, D)).
  int inverse;
};
// Number of copy runs (one per token, tensor and head group) of a relayout.
int64_t relayout_runs(const RelayoutArgs& a);
hipError_t launch_relayout(const RelayoutArgs& a, hipStream_t stream);
// Forward relayout into token-contiguous destinations (inverse = 0 only).
hipError_t launch_relayout_tok(const RelayoutArgs& a, hipStream_t stream);
// Both kinds in one launch (forward): a's run copy and at's token-contiguous
// destinations, their workgroups interleaved (1-2 % faster than two launches).
hipError_t launch_relayout_both(const RelayoutArgs& a, const RelayoutArgs& at, hipStream_t stream);

// FP8 cast of Q, K, V (D = 128).  Sources are bf16 (B, S, H, D) views; dst[0]
// and dst[1] are E4M3 (B, S, H, D) views (byte strides, channels contiguous);
// dst[2] is V transposed: element (b, s, h, d) at dst[2] + b*dst_sb[2] +
// h*dst_sh[2] + d*dst_sd_v + s.
struct CastArgs {
  const uint16_t* src[3];
  int64_t src_sb[3], src_ss[3], src_sh[3];
  uint8_t* dst[3];
  int64_t dst_sb[3], dst_ss[3], dst_sh[3];
  int64_t dst_sd_v;
  float* amax;  // [3, B, H]
  // null, or per batch entry the number of valid K/V tokens (clamped to
  // [0, S]): K and V amax over those only, V codes of the rest zero, K codes
  // of the rest not written
  const int32_t* kv_lens;
  // null, or the K/V-only cast: Q (slot 0) is neither read nor written and its
  // amax stays 0; K's scale amax is chosen against these Q scale amaxes [B, H]
  // (the power-of-two rule of Q's scale, with the roles swapped)
  const float* q_scale_in;
  int B, S, H;
};
hipError_t launch_cast_fp8(const CastArgs& a, hipStream_t stream);

// FP8 attention (D = 128).  q, k: E4M3 (B, S, H, D) views with byte strides;
// vt: V transposed, element (b, s, h, d) at vt + b*vt_sb + h*vt_sh + d*vt_sd
// + s, rows readable up to S_kv rounded up to 64 tokens.  amax arrays are
// [B, H]; the dequantisation factor is amax / 448.
struct AttnFp8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* vt;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t vt_sb, vt_sh, vt_sd;
  const float* q_amax;
  const float* k_amax;
  const float* v_amax;
  uint16_t* o;
  int64_t o_sb, o_ss, o_sh;
  float* lse;  // [B, H, S_q], may be null
  const int32_t* kv_lens;  // null, or valid keys per batch entry (clamped to [0, S_kv])
  // accumulate mode (both non-null): running fp32 O [B, S_q, H, D] and LSE
  // [B, H, S_q], merged in place; o may then be null
  float* o_acc;
  float* lse_acc;
  int B, H, S_q, S_kv;
  float scale_log2;
};
hipError_t launch_attn_fp8(const AttnFp8Args& a, hipStream_t stream);

}  // namespace lsd
