// Single-pass FP8 cast of Q, K, V for the FP8 attention path, gfx950.
//
// ("Scaling Video Generation Across NVL72 rack with TensorRT-LLM", "Ulysses
// Parallelism > Fused vs. unfused QKV all-to-all": the stacked QKV buffer gets
// one FP8 cast before the attention kernel, in a layout the kernel reads
// without another copy.)
//
// Per (tensor t, batch b, head h): amax = max |x| over tokens and channels;
// code = E4M3(x * (448 / amax)) with the product rounded to float32 and the
// code rounded to nearest even (v_cvt_pk_fp8_f32); amax == 0 uses factor 1.
// Q is coded with a scale amax instead (stored in place of its amax): the
// smallest value in [amax_q, 2 amax_q) for which the default logit factor
// log2(e)/sqrt(128) * (amax_q'/448) * (amax_k/448) is a power of two, so
// that the attention can apply it exactly through the FP8 matrix cores'
// block scales (q_scale_amax; heads with a zero amax keep amax_q).
// Q and K keep their (B, S, H, D) layout; V is written transposed, keys
// contiguous per (b, h, d), which is the operand layout of the PV product.
// With a key count per batch entry (the key-only padding mask), K's and V's
// tokens from kv_lens[b] on are padding: they take no part in the amax, V's
// codes there are zero and K's are not written.
//
// Four launches on the caller's stream: clear amax, reduce it (integer max
// on the float bits of non-negative values: order-independent, so the result
// is deterministic), quantise Q and K, quantise V.  Bulk loads and stores are
// non-temporal.  Tensors stored [B][S][H][128] contiguously per batch entry
// (the relayout's output) take flat grid-stride passes for the amax and the
// Q/K codes; other strides take per-head passes.  Measured at LTX-2 scale
// (Q, K, V [1,24576,32,128]): 0.251 ms (75 % of 8 TB/s) against 0.286 ms
// (66 %) with per-head passes and 64-token V tiles; amax 90.7 us (83 % of
// HBM, a 604 MB read streams at 87 % at best), Q/K codes 94.9 us (79.5 %, a
// 2:1 read:write stream of that size reaches 80.5 %), V 59.8 us (63 %).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsd_internal.h"

namespace lsd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;  // tokens per wave (amax, Q/K) or per workgroup (V)

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// four float32 values -> four E4M3 codes in one dword (byte i = value i)
__device__ inline uint32_t pack4_fp8(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// Tokens of tensor t of batch entry b that count: all S for Q, the first
// kv_lens[b] (clamped to [0, S]) for K and V under the key-length mask.
__device__ inline int valid_tokens(const CastArgs& a, int t, int b) {
  if (t == 0) return a.q_scale_in != nullptr ? 0 : a.S;  // no Q in the K/V-only cast
  if (a.kv_lens == nullptr) return a.S;
  return min(max(a.kv_lens[b], 0), a.S);
}

__global__ void amax_clear_kernel(float* amax, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax[i] = 0.0f;
}

// Per-head amax pass (any strides; contiguous tensors take the flat pass
// below).  One wave per (t, b, h, run of 512 tokens: shorter runs mean more atomics on
// one word and measured slower, 256 by 2-5 %, 64 by 35 %), heads fastest across
// waves (2 % faster than runs of one head fastest); a pass covers 4 tokens x 256 B
// (16 lanes per token row of D = 128 channels).  The loads of 8 passes are
// issued before any arithmetic; rows past the valid tokens re-read the last
// valid row (harmless for a maximum), so the loop has no branches.
constexpr int kAmaxRun = 512;

__global__ void __launch_bounds__(256) amax_kernel(const CastArgs a, int n_runs) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)3 * a.B * a.H * n_runs;
  if (w >= n_waves) return;
  // heads fastest: waves running together read whole token rows
  const int h = (int)(w % a.H);
  const int64_t rest = w / a.H;
  const int run = (int)(rest % n_runs);
  const int b = (int)((rest / n_runs) % a.B);
  const int t = (int)(rest / ((int64_t)n_runs * a.B));
  const int lim = valid_tokens(a, t, b);
  if (run * kAmaxRun >= lim) return;  // no valid token in this run (wave-uniform)
  const uint16_t* base = a.src[t] + (int64_t)b * a.src_sb[t] + (int64_t)h * a.src_sh[t] + 8 * (lane & 15);
  const int s0 = run * kAmaxRun + (lane >> 4);
  float m = 0.0f;
  for (int i0 = 0; i0 < kAmaxRun; i0 += 32) {
    u32x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + i0 + 4 * u, lim - 1);
      x[u] = __builtin_nontemporal_load((const u32x4*)(base + (int64_t)s * a.src_ss[t]));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf16_lo(x[u][e])), fabsf(bf16_hi(x[u][e]))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) atomicMax((unsigned int*)&a.amax[((int64_t)t * a.B + b) * a.H + h], __float_as_uint(m));
}

__device__ inline float inv_scale(float amax) { return amax > 0.0f ? 448.0f / amax : 1.0f; }

// log2(e) / sqrt(128) in float32 (0x3e0293ee): the attention's default
// logit factor (softmax scale 1/sqrt(D) for D = 128, times log2 e)
constexpr float kScaleLog2D128 = 0x1.0527dcp-3f;

// Q's scale amax, in float32 step by step: base = kScaleLog2D128 *
// (amax_k / 448), t = base * (amax_q / 448), e the smallest integer with
// 2^e >= t, result (2^e / base) * 448, from 2^(e+1) if that falls below
// amax_q; a zero amax, or a result that is not finite, keeps amax_q.
__device__ inline float q_scale_amax(float aq, float ak) {
  if (!(aq > 0.0f) || !(ak > 0.0f)) return aq;
  const float base = kScaleLog2D128 * (ak / 448.0f);
  const float t = base * (aq / 448.0f);
  int ex;
  const float m = frexpf(t, &ex);  // t = m 2^ex, m in [0.5, 1)
  const int e = (m == 0.5f) ? ex - 1 : ex;
  float r = (ldexpf(1.0f, e) / base) * 448.0f;
  if (r < aq) r = (ldexpf(1.0f, e + 1) / base) * 448.0f;
  return (r <= 3.402823466e38f) ? r : aq;
}

// the factor that codes tensor t of (b, h): 448 / amax, Q's from its scale
// amax; in the K/V-only cast K's from its scale amax against the given Q's
// (the logit factor is symmetric in the two scales, so the same rule applies)
__device__ inline float code_factor(const CastArgs& a, int t, int64_t bh) {
  const float am = a.amax[(int64_t)t * a.B * a.H + bh];
  if (t == 0) return inv_scale(q_scale_amax(am, a.amax[(int64_t)a.B * a.H + bh]));
  if (t == 1 && a.q_scale_in != nullptr) return inv_scale(q_scale_amax(am, a.q_scale_in[bh]));
  return inv_scale(am);
}

// Per-head Q and K pass (any strides; contiguous tensors with contiguous code
// outputs take the flat pass below): one wave per (t in {0,1}, b, h, 64 tokens), heads fastest so that
// waves running together read whole token rows; 16-byte bf16 vectors in,
// 8-byte code vectors out.  All 16 loads of a lane are issued before any
// conversion; rows past the valid tokens re-read the last valid row and are
// not stored.
__global__ void __launch_bounds__(256) quant_qk_kernel(const CastArgs a, int n_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)2 * a.B * a.H * n_chunks;
  if (w >= n_waves) return;
  const int h = (int)(w % a.H);
  const int64_t rest = w / a.H;
  const int chunk = (int)(rest % n_chunks);
  const int b = (int)((rest / n_chunks) % a.B);
  const int t = (int)(rest / ((int64_t)n_chunks * a.B));
  const int lim = valid_tokens(a, t, b);  // K codes past it are not written
  if (chunk * kChunk >= lim) return;
  const float inv = code_factor(a, t, (int64_t)b * a.H + h);
  const uint16_t* src = a.src[t] + (int64_t)b * a.src_sb[t] + (int64_t)h * a.src_sh[t] + 8 * (lane & 15);
  uint8_t* dst = a.dst[t] + (int64_t)b * a.dst_sb[t] + (int64_t)h * a.dst_sh[t] + 8 * (lane & 15);
  const int s0 = chunk * kChunk + (lane >> 4);
  u32x4 x[kChunk / 4];
#pragma unroll
  for (int u = 0; u < kChunk / 4; ++u) {
    const int s = min(s0 + 4 * u, lim - 1);
    x[u] = __builtin_nontemporal_load((const u32x4*)(src + (int64_t)s * a.src_ss[t]));
  }
#pragma unroll
  for (int u = 0; u < kChunk / 4; ++u) {
    const int s = s0 + 4 * u;
    if (s < lim) {
      u32x2 c;
      c[0] = pack4_fp8(bf16_lo(x[u][0]) * inv, bf16_hi(x[u][0]) * inv, bf16_lo(x[u][1]) * inv, bf16_hi(x[u][1]) * inv);
      c[1] = pack4_fp8(bf16_lo(x[u][2]) * inv, bf16_hi(x[u][2]) * inv, bf16_lo(x[u][3]) * inv, bf16_hi(x[u][3]) * inv);
      __builtin_nontemporal_store(c, (u32x2*)(dst + (int64_t)s * a.dst_ss[t]));
    }
  }
}

// V: one workgroup per (b, 256 tokens, h).  Thread (token group g of 4
// tokens, channel chunk c of 8 channels) converts, in each of 4 passes of 64
// tokens, a 4 x 8 block and writes, for each of its 8 channels, the 4 tokens'
// codes as one dword of the transposed tile in LDS ([d][256 tokens], pitch
// 272 B); then the tile leaves as 16-byte pieces, 256 contiguous bytes per
// row (1.4 % faster for the whole cast than 64-token tiles; a variant without
// LDS, each lane packing 16 tokens of each of its channels, measured 3-4 %
// slower with 4, 8 or 16 waves per workgroup).  Rows are padded to a multiple
// of 64 tokens: the last tile writes zero codes for tokens S .. the padded
// end, and nothing past it; under the key-length mask the tokens from
// kv_lens[b] on code as zero too.
constexpr int kVTok = 256;
constexpr int kVPitch = kVTok + 16;
__global__ void __launch_bounds__(256) quant_vt_kernel(const CastArgs a, int n_chunks) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * kVPitch];
  // heads fastest: workgroups that run together read whole token rows
  const int h = blockIdx.x % a.H;
  const int chunk = (blockIdx.x / a.H) % n_chunks;
  const int b = blockIdx.x / (a.H * n_chunks);
  const float inv = inv_scale(a.amax[((int64_t)2 * a.B + b) * a.H + h]);
  const uint16_t* src = a.src[2] + (int64_t)b * a.src_sb[2] + (int64_t)h * a.src_sh[2];
  const int s0 = chunk * kVTok;
  const int lim = valid_tokens(a, 2, b);  // tokens past it code as zero
  // Q's stored amax becomes its scale amax; the Q pass (an earlier launch)
  // has finished reading it
  // (in the K/V-only cast K's stored amax becomes its scale amax instead)
  if (chunk == 0 && threadIdx.x == 0) {
    if (a.q_scale_in == nullptr) {
      float* aq = &a.amax[(int64_t)b * a.H + h];
      *aq = q_scale_amax(*aq, a.amax[((int64_t)a.B + b) * a.H + h]);
    } else {
      float* ak = &a.amax[((int64_t)a.B + b) * a.H + h];
      *ak = q_scale_amax(*ak, a.q_scale_in[(int64_t)b * a.H + h]);
    }
  }
  const int tid = threadIdx.x;
  const int g = tid >> 4;      // token group (0..15)
  const int c = tid & 15;      // channel chunk (0..15)
  u32x4 x[4][4];
#pragma unroll
  for (int pass = 0; pass < 4; ++pass)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = s0 + 64 * pass + 4 * g + i;
      x[pass][i] = (u32x4){0u, 0u, 0u, 0u};
      if (s < lim) x[pass][i] = __builtin_nontemporal_load((const u32x4*)(src + (int64_t)s * a.src_ss[2] + 8 * c));
    }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    float v[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[i][2 * e] = bf16_lo(x[pass][i][e]) * inv;
        v[i][2 * e + 1] = bf16_hi(x[pass][i][e]) * inv;
      }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *(uint32_t*)(tile + (8 * c + e) * kVPitch + 64 * pass + 4 * g) = pack4_fp8(v[0][e], v[1][e], v[2][e], v[3][e]);
  }
  __syncthreads();
  // 128 rows x 16 pieces of 16 bytes; 8 per thread; pieces past the row's
  // padded end (a multiple of 64 tokens) are not written
  const int s_end = (a.S + 63) / 64 * 64;
  uint8_t* dst = a.dst[2] + (int64_t)b * a.dst_sb[2] + (int64_t)h * a.dst_sh[2];
  for (int p = tid; p < 128 * 16; p += 256) {
    const int d = p >> 4, q = p & 15;
    if (s0 + 16 * q >= s_end) continue;
    const u32x4 val = *(const u32x4*)(tile + d * kVPitch + 16 * q);   // tokens past lim were loaded as 0
    __builtin_nontemporal_store(val, (u32x4*)(dst + (int64_t)d * a.dst_sd_v + s0 + 16 * q));
  }
}

// Flat passes for tensors stored [B][S][H][128] contiguously per batch entry
// (token stride H*128, head stride 128): a (tensor, batch entry) is one span
// of S*16H 16-byte vectors, streamed by G workgroups in a grid-stride loop.
// G*256*kU is a multiple of 16H, so vector slot u of a thread stays on one
// head, (g*256*kU + 256u + tid)/16 mod H, for the whole loop.
// The amax pass runs about 512 workgroups in all (2 per CU; 256, 768 and 1024
// measured 1-3 % slower, one pass per workgroup 35 % slower: each workgroup
// ends with up to H global atomics) and reduces in LDS before its atomics;
// the Q/K pass gives each workgroup one pass (a grid of 4096 or 8192 measured
// 5-11 % slower).
constexpr int kU = 8;
constexpr int kMaxFlatH = 256;
constexpr int kAmaxGroups = 512;
constexpr int64_t kQkGroups = int64_t(1) << 40;  // capped at one pass per workgroup

__global__ void __launch_bounds__(256) amax_flat_kernel(const CastArgs a, int G) {
  __shared__ unsigned int smax[kMaxFlatH];
  const int tid = threadIdx.x;
  const int seg = blockIdx.x / G, g = blockIdx.x % G;  // seg = t * B + b
  const int t = seg / a.B, b = seg % a.B;
  for (int i = tid; i < a.H; i += 256) smax[i] = 0u;
  const int64_t n = (int64_t)valid_tokens(a, t, b) * 16 * a.H;
  const int64_t stride = (int64_t)G * 256 * kU;
  const int64_t first = (int64_t)g * 256 * kU + tid;
  const u32x4* base = (const u32x4*)(a.src[t] + (int64_t)b * a.src_sb[t]);
  float m[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) m[u] = 0.0f;
  for (int64_t i0 = first; i0 < n; i0 += stride) {
    u32x4 x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + 256 * u;
      x[u] = (u32x4){0u, 0u, 0u, 0u};
      if (i < n) x[u] = __builtin_nontemporal_load(base + i);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) m[u] = fmaxf(m[u], fmaxf(fabsf(bf16_lo(x[u][e])), fabsf(bf16_hi(x[u][e]))));
  }
  __syncthreads();  // smax cleared
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float v = m[u];
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if ((tid & 15) == 0) {
      const int h = (int)(((first + 256 * u) / 16) % a.H);
      atomicMax(&smax[h], __float_as_uint(v));
    }
  }
  __syncthreads();
  // the stored maxima only grow: skip the atomic when a plain read already
  // shows a value at least this large (a stale read only costs an atomic)
  for (int h = tid; h < a.H; h += 256) {
    const unsigned int v = smax[h];
    unsigned int* dst = (unsigned int*)&a.amax[(int64_t)seg * a.H + h];
    if (v > *(volatile unsigned int*)dst) atomicMax(dst, v);
  }
}

__global__ void __launch_bounds__(256) quant_qk_flat_kernel(const CastArgs a, int G) {
  const int tid = threadIdx.x;
  const int seg = blockIdx.x / G, g = blockIdx.x % G;  // seg = t * B + b, t in {0, 1}
  const int t = seg / a.B, b = seg % a.B;
  const int64_t n = (int64_t)valid_tokens(a, t, b) * 16 * a.H;  // K codes past the valid tokens are not written
  const int64_t stride = (int64_t)G * 256 * kU;
  const int64_t first = (int64_t)g * 256 * kU + tid;
  const u32x4* src = (const u32x4*)(a.src[t] + (int64_t)b * a.src_sb[t]);
  u32x2* dst = (u32x2*)(a.dst[t] + (int64_t)b * a.dst_sb[t]);
  float inv[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u)
    inv[u] = code_factor(a, t, (int64_t)b * a.H + (int)(((first + 256 * u) / 16) % a.H));
  for (int64_t i0 = first; i0 < n; i0 += stride) {
    u32x4 x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + 256 * u;
      if (i < n) x[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + 256 * u;
      if (i < n) {
        const float f = inv[u];
        u32x2 c;
        c[0] = pack4_fp8(bf16_lo(x[u][0]) * f, bf16_hi(x[u][0]) * f, bf16_lo(x[u][1]) * f, bf16_hi(x[u][1]) * f);
        c[1] = pack4_fp8(bf16_lo(x[u][2]) * f, bf16_hi(x[u][2]) * f, bf16_lo(x[u][3]) * f, bf16_hi(x[u][3]) * f);
        __builtin_nontemporal_store(c, dst + i);
      }
    }
  }
}

// workgroups per span: about `target` in all, a multiple of 16H / gcd(16H, 256 kU)
static int64_t flat_groups(int H, int64_t n_vec, int n_seg, int64_t target) {
  int a = 16 * H, b = 256 * kU;
  while (b) { const int r = a % b; a = b; b = r; }
  const int64_t m = 16 * H / a;
  int64_t G = target / n_seg;
  const int64_t need = (n_vec + 256 * kU - 1) / (256 * kU);  // no more groups than passes
  if (G > need) G = need;
  G = (G + m - 1) / m * m;
  if (G < m) G = m;
  return G;
}

}  // namespace

hipError_t launch_cast_fp8(const CastArgs& a, hipStream_t stream) {
  const int n = 3 * a.B * a.H;
  hipLaunchKernelGGL(amax_clear_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a.amax, n);
  if (a.S == 0) return hipGetLastError();
  const int n_chunks = (a.S + kChunk - 1) / kChunk;
  const int n_runs = (a.S + kAmaxRun - 1) / kAmaxRun;
  const int64_t amax_waves = (int64_t)3 * a.B * a.H * n_runs;
  const int64_t qk_waves = (int64_t)2 * a.B * a.H * n_chunks;
  const int n_vchunks = (a.S + kVTok - 1) / kVTok;
  const int64_t vt_blocks = (int64_t)a.B * a.H * n_vchunks;
  if ((amax_waves + 3) / 4 > 0x7fffffff || vt_blocks > 0x7fffffff) return hipErrorInvalidValue;
  bool flat_src = a.H <= kMaxFlatH, flat_dst = true;
  for (int t = 0; t < 3; ++t) flat_src = flat_src && a.src_sh[t] == 128 && a.src_ss[t] == (int64_t)128 * a.H;
  for (int t = 0; t < 2; ++t) flat_dst = flat_dst && a.dst_sh[t] == 128 && a.dst_ss[t] == (int64_t)128 * a.H;
  const int64_t n_vec = (int64_t)a.S * 16 * a.H;
  const int64_t g_amax = flat_groups(a.H, n_vec, 3 * a.B, kAmaxGroups);
  const int64_t g_qk = flat_groups(a.H, n_vec, 2 * a.B, kQkGroups);
  flat_src = flat_src && 3 * a.B * g_amax <= 0x7fffffff;
  flat_dst = flat_dst && 2 * a.B * g_qk <= 0x7fffffff;
  if (flat_src) {
    hipLaunchKernelGGL(amax_flat_kernel, dim3((unsigned)(3 * a.B * g_amax)), dim3(256), 0, stream, a, (int)g_amax);
  } else {
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)((amax_waves + 3) / 4)), dim3(256), 0, stream, a, n_runs);
  }
  if (flat_src && flat_dst) {
    hipLaunchKernelGGL(quant_qk_flat_kernel, dim3((unsigned)(2 * a.B * g_qk)), dim3(256), 0, stream, a, (int)g_qk);
  } else {
    hipLaunchKernelGGL(quant_qk_kernel, dim3((unsigned)((qk_waves + 3) / 4)), dim3(256), 0, stream, a, n_chunks);
  }
  hipLaunchKernelGGL(quant_vt_kernel, dim3((unsigned)vt_blocks), dim3(256), 0, stream, a, n_vchunks);
  return hipGetLastError();
}

}  // namespace lsd
