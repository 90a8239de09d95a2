// C-ABI entry points: host-side argument validation, then one kernel launch.
// Every check runs before any HIP call, so a rejected request enqueues nothing
// and touches no device state.  See include/lsd.h for the contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "lsd.h"
#include "lsd_internal.h"

namespace {

thread_local std::string g_err;

lsd_status fail(lsd_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

lsd_status ok() {
  g_err.clear();
  return LSD_OK;
}

bool view_empty(const lsd_view4& v) {
  for (int i = 0; i < 4; ++i)
    if (v.shape[i] == 0) return true;
  return false;
}

// Byte range [lo, hi) touched by a view of elements of `eb` bytes.
struct Span {
  uintptr_t lo = 0, hi = 0;
};

Span span_of(const lsd_view4& v, int eb) {
  Span s;
  if (view_empty(v)) return s;
  int64_t last = 0;
  for (int i = 0; i < 4; ++i) last += (v.shape[i] - 1) * v.stride[i];
  s.lo = (uintptr_t)v.data;
  s.hi = s.lo + (uintptr_t)(last + 1) * (uintptr_t)eb;
  return s;
}

Span span_flat(const void* p, int64_t n, int eb) {
  Span s;
  if (p == nullptr || n <= 0) return s;
  s.lo = (uintptr_t)p;
  s.hi = s.lo + (uintptr_t)n * (uintptr_t)eb;
  return s;
}

bool overlaps(const Span& a, const Span& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Structural checks shared by every bf16 view.  The unit-stride dimension is
// the head channel (unit_dim 3), or the sequence (unit_dim 1) for a V given
// token-contiguous; every other stride is a multiple of 16 bytes.
lsd_status check_view(const char* name, const lsd_view4* v, int unit_dim = 3) {
  if (v == nullptr) return fail(LSD_EINVAL, "%s: null view", name);
  for (int i = 0; i < 4; ++i) {
    if (v->shape[i] < 0) return fail(LSD_EINVAL, "%s: negative shape[%d]", name, i);
    if (v->shape[i] > 0x7fffffff) return fail(LSD_EINVAL, "%s: shape[%d] exceeds 2^31-1", name, i);
    if (v->stride[i] < 0) return fail(LSD_EINVAL, "%s: negative stride[%d]", name, i);
  }
  if (view_empty(*v)) return LSD_OK;
  if (v->data == nullptr) return fail(LSD_EINVAL, "%s: null data pointer", name);
  if (v->stride[unit_dim] != 1 && v->shape[unit_dim] > 1)
    return fail(LSD_EINVAL, "%s: stride[%d] must be 1 (%s contiguous)", name, unit_dim,
                unit_dim == 3 ? "head channels" : "tokens");
  if ((uintptr_t)v->data % 16 != 0) return fail(LSD_EINVAL, "%s: data pointer not 16-byte aligned", name);
  if (v->shape[3] % 8 != 0) return fail(LSD_EINVAL, "%s: D=%lld is not a multiple of 8", name, (long long)v->shape[3]);
  for (int i = 0; i < 4; ++i)
    if (i != unit_dim && v->shape[i] > 1 && v->stride[i] % 8 != 0)
      return fail(LSD_EINVAL, "%s: stride[%d]=%lld is not a multiple of 8 elements (16 bytes)", name, i,
                  (long long)v->stride[i]);
  // the largest element offset must fit comfortably in 64-bit byte arithmetic
  double last = 0;
  for (int i = 0; i < 4; ++i) last += (double)(v->shape[i] - 1) * (double)v->stride[i];
  if (last * 2.0 > 9.0e18) return fail(LSD_EINVAL, "%s: view spans more than 2^62 bytes", name);
  return LSD_OK;
}

// Structural checks of an FP8 (one byte per element) view: the unit stride is
// the channel stride (unit_dim 3) or, for V stored transposed, the sequence
// stride (unit_dim 1); every other stride and the data pointer are multiples
// of 16 bytes.
lsd_status check_view8(const char* name, const lsd_view4* v, int unit_dim) {
  if (v == nullptr) return fail(LSD_EINVAL, "%s: null view", name);
  for (int i = 0; i < 4; ++i) {
    if (v->shape[i] < 0) return fail(LSD_EINVAL, "%s: negative shape[%d]", name, i);
    if (v->shape[i] > 0x7fffffff) return fail(LSD_EINVAL, "%s: shape[%d] exceeds 2^31-1", name, i);
    if (v->stride[i] < 0) return fail(LSD_EINVAL, "%s: negative stride[%d]", name, i);
  }
  if (view_empty(*v)) return LSD_OK;
  if (v->data == nullptr) return fail(LSD_EINVAL, "%s: null data pointer", name);
  if (v->stride[unit_dim] != 1 && v->shape[unit_dim] > 1)
    return fail(LSD_EINVAL, "%s: stride[%d] must be 1 (%s contiguous)", name, unit_dim,
                unit_dim == 3 ? "head channels" : "tokens");
  if ((uintptr_t)v->data % 16 != 0) return fail(LSD_EINVAL, "%s: data pointer not 16-byte aligned", name);
  for (int i = 0; i < 4; ++i)
    if (i != unit_dim && v->shape[i] > 1 && v->stride[i] % 16 != 0)
      return fail(LSD_EINVAL, "%s: stride[%d]=%lld is not a multiple of 16 bytes", name, i, (long long)v->stride[i]);
  double last = 0;
  for (int i = 0; i < 4; ++i) last += (double)(v->shape[i] - 1) * (double)v->stride[i];
  if (last > 9.0e18) return fail(LSD_EINVAL, "%s: view spans more than 2^62 bytes", name);
  return LSD_OK;
}

// Layout of a V view: token-contiguous (V^T rows: stride[1] = 1, channel
// stride = row pitch) when its channels are not unit-stride.
bool v_token_major(const lsd_view4* v) {
  return v != nullptr && v->stride[3] != 1 && v->shape[3] > 1 && v->stride[1] == 1;
}

// A token-contiguous V's rows hold all S keys, do not overlap, and are
// addressed with 32-bit byte offsets.
lsd_status check_vt_rows(const char* name, const lsd_view4* v) {
  if (view_empty(*v)) return LSD_OK;
  const int64_t S = v->shape[1], D = v->shape[3];
  if (D > 1 && v->stride[3] < S)
    return fail(LSD_EINVAL, "%s: token-contiguous rows: pitch stride[3]=%lld is below S=%lld", name,
                (long long)v->stride[3], (long long)S);
  if (v->stride[3] >= (int64_t(1) << 23))
    return fail(LSD_EUNSUPPORTED, "%s: token-contiguous rows: pitch stride[3]=%lld must be below 2^23", name,
                (long long)v->stride[3]);
  return LSD_OK;
}

bool same_shape(const lsd_view4& a, const lsd_view4& b) {
  for (int i = 0; i < 4; ++i)
    if (a.shape[i] != b.shape[i]) return false;
  return true;
}

std::atomic<int> g_dev_ok[64];  // 0 unknown, 1 gfx950, 2 other

lsd_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LSD_EDEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(LSD_EDEVICE, "device index %d out of range", dev);
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(LSD_EDEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(LSD_EUNSUPPORTED, "device %d is not gfx950 (MI355X); the kernels are built for gfx950 only", dev);
  return LSD_OK;
}

lsd_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LSD_EDEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}


// Shared validation and launch of both attention entry points.  In
// accumulate mode o (bf16 output) is optional and lse is unused; o_acc
// ([B,S_q,H,D] fp32) and lse_acc ([B,H,S_q] fp32) are read and written.
lsd_status attention(bool acc, const lsd_view4* q, const lsd_view4* k, const lsd_view4* v, const int32_t* kv_lens,
                     const lsd_view4* o, float* lse, float* o_acc, float* lse_acc, float softmax_scale,
                     void* stream) {
  lsd_status s;
  if ((s = check_view("q", q)) != LSD_OK) return s;
  if ((s = check_view("k", k)) != LSD_OK) return s;
  const bool v_tok = v_token_major(v);
  if ((s = check_view("v", v, v_tok ? 1 : 3)) != LSD_OK) return s;
  if (v_tok && (s = check_vt_rows("v", v)) != LSD_OK) return s;
  if ((!acc || o != nullptr) && (s = check_view("o", o)) != LSD_OK) return s;
  const int64_t B = q->shape[0], S_q = q->shape[1], H = q->shape[2], D = q->shape[3];
  const int64_t S_kv = k->shape[1];
  if (k->shape[0] != B || k->shape[2] != H || k->shape[3] != D)
    return fail(LSD_EINVAL, "k shape (%lld,%lld,%lld,%lld) does not match q (B=%lld, H=%lld, D=%lld)",
                (long long)k->shape[0], (long long)k->shape[1], (long long)k->shape[2], (long long)k->shape[3],
                (long long)B, (long long)H, (long long)D);
  if (!same_shape(*v, *k)) return fail(LSD_EINVAL, "v shape must equal k shape (B, S_kv, H, D)");
  if (o != nullptr && !same_shape(*o, *q)) return fail(LSD_EINVAL, "o shape must equal q shape (B, S_q, H, D)");
  if (D != 64 && D != 128) return fail(LSD_EUNSUPPORTED, "head dim D=%lld unsupported (64 or 128)", (long long)D);
  // a 64-key K/V tile is addressed with 32-bit byte offsets
  if (k->stride[1] >= (int64_t(1) << 24) || (!v_tok && v->stride[1] >= (int64_t(1) << 24)))
    return fail(LSD_EUNSUPPORTED, "k/v sequence stride (%lld, %lld elements) must be below 2^24",
                (long long)k->stride[1], (long long)v->stride[1]);
  if (std::isinf(softmax_scale)) return fail(LSD_EINVAL, "softmax_scale is infinite");
  if (lse != nullptr && (uintptr_t)lse % 4 != 0) return fail(LSD_EINVAL, "lse not 4-byte aligned");
  if (kv_lens != nullptr && (uintptr_t)kv_lens % 4 != 0) return fail(LSD_EINVAL, "kv_lens not 4-byte aligned");
  if (acc) {
    if (o_acc == nullptr || lse_acc == nullptr) return fail(LSD_EINVAL, "null o_acc or lse_acc");
    if ((uintptr_t)o_acc % 16 != 0) return fail(LSD_EINVAL, "o_acc not 16-byte aligned");
    if ((uintptr_t)lse_acc % 4 != 0) return fail(LSD_EINVAL, "lse_acc not 4-byte aligned");
  }
  if (B * S_q * H == 0) return ok();

  const Span sq = span_of(*q, 2), sk = span_of(*k, 2), sv = span_of(*v, 2);
  const Span none = span_flat(nullptr, 0, 1);
  const Span so = o != nullptr ? span_of(*o, 2) : none;
  const Span sl = span_flat(lse, B * H * S_q, 4);
  const Span soa = span_flat(o_acc, B * S_q * H * D, 4);
  const Span sla = span_flat(lse_acc, B * H * S_q, 4);
  const Span skl = span_flat(kv_lens, B, 4);
  const Span ins[4] = {sq, sk, sv, skl};
  const Span outs[4] = {so, sl, soa, sla};
  const char* names[4] = {"o", "lse", "o_acc", "lse_acc"};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(outs[i], ins[j])) return fail(LSD_EINVAL, "%s overlaps an input (q, k, v or kv_lens)", names[i]);
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j])) return fail(LSD_EINVAL, "%s overlaps %s", names[i], names[j]);
  }
  if ((s = check_device()) != LSD_OK) return s;

  const float scale = (softmax_scale > 0.0f) ? softmax_scale : (float)(1.0 / std::sqrt((double)D));
  lsd::AttnArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = (const uint16_t*)q->data;
  a.k = (const uint16_t*)k->data;
  a.v = (const uint16_t*)v->data;
  a.o = o != nullptr ? (uint16_t*)o->data : nullptr;
  a.lse = lse;
  a.o_acc = o_acc;
  a.lse_acc = lse_acc;
  a.kv_lens = kv_lens;
  a.q_sb = q->stride[0]; a.q_ss = q->stride[1]; a.q_sh = q->stride[2];
  a.k_sb = k->stride[0]; a.k_ss = k->stride[1]; a.k_sh = k->stride[2];
  a.v_sb = v->stride[0]; a.v_ss = v->stride[1]; a.v_sh = v->stride[2];
  a.v_sd = v->stride[3];
  a.v_tok = v_tok ? 1 : 0;
  if (o != nullptr) { a.o_sb = o->stride[0]; a.o_ss = o->stride[1]; a.o_sh = o->stride[2]; }
  a.B = (int)B; a.H = (int)H; a.S_q = (int)S_q; a.S_kv = (int)S_kv; a.D = (int)D;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  return launched(lsd::launch_attn_fwd(a, (hipStream_t)stream), acc ? "attn_fwd_accumulate" : "attn_fwd");
}

// q_scale != nullptr: the K/V-only cast (slot 0 repeats slot 1 and is neither
// read nor written; K's scale amax is chosen against the given Q scales).
lsd_status cast_qkv_fp8(const lsd_view4* src, const lsd_view4* dst, float* amax, const int32_t* kv_lens,
                        const float* q_scale, void* stream) {
  if (src == nullptr || dst == nullptr) return fail(LSD_EINVAL, "null src or dst array");
  lsd_status s;
  const int t0 = q_scale != nullptr ? 1 : 0;
  static const char* sn[3] = {"src[0] (q)", "src[1] (k)", "src[2] (v)"};
  static const char* dn[3] = {"dst[0] (q8)", "dst[1] (k8)", "dst[2] (v8, transposed)"};
  static const char* snk[3] = {"", "src[0] (k)", "src[1] (v)"};
  static const char* dnk[3] = {"", "dst[0] (k8)", "dst[1] (v8, transposed)"};
  const char* const* sn_ = t0 ? snk : sn;
  const char* const* dn_ = t0 ? dnk : dn;
  for (int t = t0; t < 3; ++t) {
    if ((s = check_view(sn_[t], &src[t])) != LSD_OK) return s;
    if ((s = check_view8(dn_[t], &dst[t], t == 2 ? 1 : 3)) != LSD_OK) return s;
    if (!same_shape(src[t], src[t0])) return fail(LSD_EINVAL, "%s: the sources must have one shape", sn_[t]);
    if (!same_shape(dst[t], src[t0]))
      return fail(LSD_EINVAL, "%s: shape must equal the sources' (B, S, H, D)", dn_[t]);
  }
  const int64_t B = src[t0].shape[0], S = src[t0].shape[1], H = src[t0].shape[2], D = src[t0].shape[3];
  if (D != 128) return fail(LSD_EUNSUPPORTED, "FP8 path: head dim D=%lld unsupported (128)", (long long)D);
  // V rows are written up to the next multiple of 64 tokens (zero codes)
  const int64_t s_pad = (S + 63) / 64 * 64;
  if (dst[2].stride[3] < s_pad)
    return fail(LSD_EINVAL, "dst[2] (v8): row pitch stride[3]=%lld is below S=%lld rounded up to 64",
                (long long)dst[2].stride[3], (long long)S);
  if (amax == nullptr) return fail(LSD_EINVAL, "null amax");
  if ((uintptr_t)amax % 4 != 0) return fail(LSD_EINVAL, "amax not 4-byte aligned");
  if (kv_lens != nullptr && (uintptr_t)kv_lens % 4 != 0) return fail(LSD_EINVAL, "kv_lens not 4-byte aligned");
  if (q_scale != nullptr && (uintptr_t)q_scale % 4 != 0) return fail(LSD_EINVAL, "q_scale_amax not 4-byte aligned");
  if (B * H == 0) return ok();
  Span ins[5], outs[4];
  const Span none = span_flat(nullptr, 0, 1);
  for (int t = 0; t < 3; ++t) {
    ins[t] = t >= t0 ? span_of(src[t], 2) : none;
    outs[t] = t >= t0 ? span_of(dst[t], 1) : none;
  }
  ins[3] = span_flat(kv_lens, B, 4);
  ins[4] = span_flat(q_scale, B * H, 4);
  outs[2].hi += (uintptr_t)(s_pad - S);  // the last row's padding is written too
  outs[3] = span_flat(amax, 3 * B * H, 4);
  const char* on[4] = {dn_[0], dn_[1], dn_[2], "amax"};
  const char* in_names[5] = {sn_[0], sn_[1], sn_[2], "kv_lens", "q_scale_amax"};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlaps(outs[i], ins[j])) return fail(LSD_EINVAL, "%s overlaps %s", on[i], in_names[j]);
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j])) return fail(LSD_EINVAL, "%s overlaps %s", on[i], on[j]);
  }
  if ((s = check_device()) != LSD_OK) return s;
  lsd::CastArgs a;
  std::memset(&a, 0, sizeof a);
  for (int t = 0; t < 3; ++t) {
    a.src[t] = (const uint16_t*)src[t].data;
    a.src_sb[t] = src[t].stride[0]; a.src_ss[t] = src[t].stride[1]; a.src_sh[t] = src[t].stride[2];
    a.dst[t] = (uint8_t*)dst[t].data;
    a.dst_sb[t] = dst[t].stride[0]; a.dst_ss[t] = dst[t].stride[1]; a.dst_sh[t] = dst[t].stride[2];
  }
  a.dst_sd_v = dst[2].stride[3];
  a.amax = amax;
  a.kv_lens = kv_lens;
  a.q_scale_in = q_scale;
  a.B = (int)B; a.S = (int)S; a.H = (int)H;
  return launched(lsd::launch_cast_fp8(a, (hipStream_t)stream), q_scale ? "cast_kv_fp8" : "cast_qkv_fp8");
}

lsd_status attn_fwd_fp8(const lsd_view4* q8, const lsd_view4* k8, const lsd_view4* v8, const float* q_amax,
                        const float* k_amax, const float* v_amax, const int32_t* kv_lens, const lsd_view4* o,
                        float* lse, float* o_acc, float* lse_acc, bool acc, float softmax_scale, void* stream) {
  lsd_status s;
  if ((s = check_view8("q8", q8, 3)) != LSD_OK) return s;
  if ((s = check_view8("k8", k8, 3)) != LSD_OK) return s;
  if ((s = check_view8("v8 (transposed)", v8, 1)) != LSD_OK) return s;
  if ((!acc || o != nullptr) && (s = check_view("o", o)) != LSD_OK) return s;
  const int64_t B = q8->shape[0], S_q = q8->shape[1], H = q8->shape[2], D = q8->shape[3];
  const int64_t S_kv = k8->shape[1];
  if (k8->shape[0] != B || k8->shape[2] != H || k8->shape[3] != D)
    return fail(LSD_EINVAL, "k8 shape does not match q8 (B=%lld, H=%lld, D=%lld)", (long long)B, (long long)H,
                (long long)D);
  if (!same_shape(*v8, *k8)) return fail(LSD_EINVAL, "v8 shape must equal k8 shape (B, S_kv, H, D)");
  if (o != nullptr && !same_shape(*o, *q8)) return fail(LSD_EINVAL, "o shape must equal q8 shape (B, S_q, H, D)");
  if (D != 128) return fail(LSD_EUNSUPPORTED, "FP8 path: head dim D=%lld unsupported (128)", (long long)D);
  if (acc) {
    if (o_acc == nullptr || lse_acc == nullptr) return fail(LSD_EINVAL, "null o_acc or lse_acc");
    if ((uintptr_t)o_acc % 16 != 0) return fail(LSD_EINVAL, "o_acc not 16-byte aligned");
    if ((uintptr_t)lse_acc % 4 != 0) return fail(LSD_EINVAL, "lse_acc not 4-byte aligned");
  }
  if (k8->stride[1] >= (int64_t(1) << 24) || v8->stride[3] >= (int64_t(1) << 24))
    return fail(LSD_EUNSUPPORTED, "k8 sequence stride / v8 row pitch must be below 2^24 bytes");
  if (S_kv > 0 && v8->stride[3] < (S_kv + 63) / 64 * 64)
    return fail(LSD_EINVAL, "v8: row pitch stride[3]=%lld is below S_kv=%lld rounded up to 64",
                (long long)v8->stride[3], (long long)S_kv);
  if (q_amax == nullptr || k_amax == nullptr || v_amax == nullptr) return fail(LSD_EINVAL, "null amax array");
  if ((uintptr_t)q_amax % 4 || (uintptr_t)k_amax % 4 || (uintptr_t)v_amax % 4)
    return fail(LSD_EINVAL, "amax arrays not 4-byte aligned");
  if (std::isinf(softmax_scale)) return fail(LSD_EINVAL, "softmax_scale is infinite");
  if (lse != nullptr && (uintptr_t)lse % 4 != 0) return fail(LSD_EINVAL, "lse not 4-byte aligned");
  if (kv_lens != nullptr && (uintptr_t)kv_lens % 4 != 0) return fail(LSD_EINVAL, "kv_lens not 4-byte aligned");
  if (B * S_q * H == 0) return ok();
  Span vs = span_of(*v8, 1);
  if (S_kv > 0) vs.hi += (uintptr_t)((S_kv + 63) / 64 * 64 - S_kv);  // the padded tail of the last row
  const Span ins[7] = {span_of(*q8, 1), span_of(*k8, 1), vs, span_flat(q_amax, B * H, 4),
                       span_flat(k_amax, B * H, 4), span_flat(v_amax, B * H, 4), span_flat(kv_lens, B, 4)};
  const Span none = span_flat(nullptr, 0, 1);
  const Span so = o != nullptr ? span_of(*o, 2) : none, sl = span_flat(lse, B * H * S_q, 4);
  const Span soa = span_flat(o_acc, B * S_q * H * D, 4), sla = span_flat(lse_acc, B * H * S_q, 4);
  const Span outs[4] = {so, sl, soa, sla};
  const char* onames[4] = {"o", "lse", "o_acc", "lse_acc"};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], ins[j])) return fail(LSD_EINVAL, "%s overlaps an input", onames[i]);
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j])) return fail(LSD_EINVAL, "%s overlaps %s", onames[i], onames[j]);
  }
  if ((s = check_device()) != LSD_OK) return s;

  const float scale = (softmax_scale > 0.0f) ? softmax_scale : (float)(1.0 / std::sqrt((double)D));
  lsd::AttnFp8Args a;
  std::memset(&a, 0, sizeof a);
  a.q = (const uint8_t*)q8->data;
  a.k = (const uint8_t*)k8->data;
  a.vt = (const uint8_t*)v8->data;
  a.q_sb = q8->stride[0]; a.q_ss = q8->stride[1]; a.q_sh = q8->stride[2];
  a.k_sb = k8->stride[0]; a.k_ss = k8->stride[1]; a.k_sh = k8->stride[2];
  a.vt_sb = v8->stride[0]; a.vt_sh = v8->stride[2]; a.vt_sd = v8->stride[3];
  a.q_amax = q_amax; a.k_amax = k_amax; a.v_amax = v_amax;
  a.o = o != nullptr ? (uint16_t*)o->data : nullptr;
  if (o != nullptr) { a.o_sb = o->stride[0]; a.o_ss = o->stride[1]; a.o_sh = o->stride[2]; }
  a.lse = acc ? nullptr : lse;
  a.kv_lens = kv_lens;
  a.o_acc = acc ? o_acc : nullptr;
  a.lse_acc = acc ? lse_acc : nullptr;
  a.B = (int)B; a.H = (int)H; a.S_q = (int)S_q; a.S_kv = (int)S_kv;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  return launched(lsd::launch_attn_fp8(a, (hipStream_t)stream),
                  acc ? "attn_fwd_fp8_accumulate" : (kv_lens ? "attn_fwd_fp8_masked" : "attn_fwd_fp8"));
}

}  // namespace

extern "C" {

int lsd_abi_version(void) { return LSD_ABI_VERSION; }

const char* lsd_last_error(void) { return g_err.c_str(); }

lsd_status lsd_attn_fwd(const lsd_view4* q, const lsd_view4* k, const lsd_view4* v, const lsd_view4* o,
                        float* lse, float softmax_scale, void* stream) {
  return attention(false, q, k, v, nullptr, o, lse, nullptr, nullptr, softmax_scale, stream);
}

lsd_status lsd_attn_fwd_masked(const lsd_view4* q, const lsd_view4* k, const lsd_view4* v, const int32_t* kv_lens,
                               const lsd_view4* o, float* lse, float softmax_scale, void* stream) {
  if (kv_lens == nullptr) return fail(LSD_EINVAL, "null kv_lens");
  return attention(false, q, k, v, kv_lens, o, lse, nullptr, nullptr, softmax_scale, stream);
}

lsd_status lsd_attn_fwd_accumulate(const lsd_view4* q, const lsd_view4* k, const lsd_view4* v,
                                   const int32_t* kv_lens, float* o_acc, float* lse_acc, const lsd_view4* o,
                                   float softmax_scale, void* stream) {
  return attention(true, q, k, v, kv_lens, o, nullptr, o_acc, lse_acc, softmax_scale, stream);
}

lsd_status lsd_attn_merge(int n, const lsd_view4* o_parts, const float* const* lse_parts, const lsd_view4* o_out,
                          float* lse_out, void* stream) {
  if (n < 1) return fail(LSD_EINVAL, "n=%d: need at least one partial", n);
  if (n > lsd::kMaxMerge) return fail(LSD_EUNSUPPORTED, "n=%d partials: at most %d per call", n, lsd::kMaxMerge);
  if (o_parts == nullptr || lse_parts == nullptr) return fail(LSD_EINVAL, "null o_parts or lse_parts array");
  lsd_status s;
  if ((s = check_view("o_out", o_out)) != LSD_OK) return s;
  char name[32];
  for (int i = 0; i < n; ++i) {
    std::snprintf(name, sizeof name, "o_parts[%d]", i);
    if ((s = check_view(name, &o_parts[i])) != LSD_OK) return s;
    if (!same_shape(o_parts[i], *o_out)) return fail(LSD_EINVAL, "o_parts[%d] shape differs from o_out", i);
  }
  const int64_t B = o_out->shape[0], S = o_out->shape[1], H = o_out->shape[2], D = o_out->shape[3];
  if (D > 8 * 256) return fail(LSD_EUNSUPPORTED, "D=%lld too large for the merge kernel (<= 2048)", (long long)D);
  if (lse_out != nullptr && (uintptr_t)lse_out % 4 != 0) return fail(LSD_EINVAL, "lse_out not 4-byte aligned");
  if (B * S * H * D == 0) return ok();
  for (int i = 0; i < n; ++i) {
    if (lse_parts[i] == nullptr) return fail(LSD_EINVAL, "lse_parts[%d] is null", i);
    if ((uintptr_t)lse_parts[i] % 4 != 0) return fail(LSD_EINVAL, "lse_parts[%d] not 4-byte aligned", i);
  }
  const Span so = span_of(*o_out, 2);
  const Span slo = span_flat(lse_out, B * H * S, 4);
  if (overlaps(so, slo)) return fail(LSD_EINVAL, "o_out overlaps lse_out");
  for (int i = 0; i < n; ++i) {
    const Span si = span_of(o_parts[i], 2), sli = span_flat(lse_parts[i], B * H * S, 4);
    if (overlaps(so, si) || overlaps(so, sli)) return fail(LSD_EINVAL, "o_out overlaps partial %d", i);
    if (overlaps(slo, si) || overlaps(slo, sli)) return fail(LSD_EINVAL, "lse_out overlaps partial %d", i);
  }
  if ((s = check_device()) != LSD_OK) return s;

  lsd::MergeArgs a;
  std::memset(&a, 0, sizeof a);
  for (int i = 0; i < n; ++i) {
    a.o_in[i] = (const uint16_t*)o_parts[i].data;
    a.in_sb[i] = o_parts[i].stride[0];
    a.in_ss[i] = o_parts[i].stride[1];
    a.in_sh[i] = o_parts[i].stride[2];
    a.lse_in[i] = lse_parts[i];
  }
  a.o_out = (uint16_t*)o_out->data;
  a.out_sb = o_out->stride[0]; a.out_ss = o_out->stride[1]; a.out_sh = o_out->stride[2];
  a.lse_out = lse_out;
  a.n = n; a.B = (int)B; a.S = (int)S; a.H = (int)H; a.D = (int)D;
  return launched(lsd::launch_attn_merge(a, (hipStream_t)stream), "attn_merge");
}

}  // extern "C"

namespace {

// Shared validation and launch of both Ulysses relayouts.
//   forward: src (B, S_loc, H, D) x P shards -> dst (B, P*S_loc, H/P, D)
//   inverse: src (B, P*S_loc, H_loc, D) x P rank slices -> dst (B, S_loc, P*H_loc, D)
lsd_status relayout(bool inverse, const char* fn, int n_tensors, int P, int rank, const lsd_view4* src,
                    const lsd_view4* dst, void* stream) {
  if (n_tensors < 1 || n_tensors > lsd::kMaxRelayoutTensors)
    return fail(LSD_EINVAL, "n_tensors=%d: must be 1..%d (Q, K, V)", n_tensors, lsd::kMaxRelayoutTensors);
  if (P < 1) return fail(LSD_EINVAL, "P=%d: sequence-parallel degree must be >= 1", P);
  if (P > lsd::kMaxRelayoutP) return fail(LSD_EUNSUPPORTED, "P=%d: at most %d shards per call", P, lsd::kMaxRelayoutP);
  if (rank < 0 || rank >= P) return fail(LSD_EINVAL, "rank=%d not in [0, P=%d)", rank, P);
  if (src == nullptr || dst == nullptr) return fail(LSD_EINVAL, "null src or dst array");
  lsd_status s;
  char name[48];
  for (int i = 0; i < n_tensors * P; ++i) {
    std::snprintf(name, sizeof name, "src[%d] (tensor %d, %s %d)", i, i / P, inverse ? "rank" : "shard", i % P);
    if ((s = check_view(name, &src[i])) != LSD_OK) return s;
    if (!same_shape(src[i], src[0]))
      return fail(LSD_EINVAL, inverse ? "src[%d]: head slices must all have the same shape (B, S, H_loc, D)"
                                       : "src[%d]: sequence shards must all have the same shape (B, S_loc, H, D)",
                  i);
  }
  const int64_t B = src[0].shape[0], D = src[0].shape[3];
  int64_t S_loc, H_loc;
  if (!inverse) {
    S_loc = src[0].shape[1];
    const int64_t H = src[0].shape[2];
    if (H % P != 0) return fail(LSD_EINVAL, "head count H=%lld is not divisible by P=%d", (long long)H, P);
    H_loc = H / P;
  } else {
    const int64_t S = src[0].shape[1];
    if (S % P != 0)
      return fail(LSD_EINVAL, "sequence length S=%lld is not divisible by P=%d (equal shards)", (long long)S, P);
    S_loc = S / P;
    H_loc = src[0].shape[2];
  }
  if ((int64_t)P * S_loc > 0x7fffffff) return fail(LSD_EINVAL, "P*S_loc exceeds 2^31-1");
  const int64_t want1 = inverse ? S_loc : P * S_loc, want2 = inverse ? P * H_loc : H_loc;
  bool tok[lsd::kMaxRelayoutTensors] = {};
  for (int t = 0; t < n_tensors; ++t) {
    std::snprintf(name, sizeof name, "dst[%d]", t);
    tok[t] = v_token_major(&dst[t]);
    if (tok[t] && inverse)
      return fail(LSD_EINVAL, "%s: the inverse relayout writes sequence shards with channels contiguous", name);
    if ((s = check_view(name, &dst[t], tok[t] ? 1 : 3)) != LSD_OK) return s;
    const lsd_view4& d = dst[t];
    if (d.shape[0] != B || d.shape[1] != want1 || d.shape[2] != want2 || d.shape[3] != D)
      return fail(LSD_EINVAL, "dst[%d] shape must be (B=%lld, %lld, %lld, D=%lld)", t, (long long)B,
                  (long long)want1, (long long)want2, (long long)D);
    if (tok[t]) {
      if ((s = check_vt_rows(name, &d)) != LSD_OK) return s;
      if (D % 64 != 0)
        return fail(LSD_EUNSUPPORTED, "%s: token-contiguous destination needs D a multiple of 64 (D=%lld)", name,
                    (long long)D);
      // rows of one head, heads of one batch entry: disjoint
      if ((H_loc > 1 && d.stride[2] < D * d.stride[3]) || (B > 1 && d.stride[0] < H_loc * d.stride[2]))
        return fail(LSD_EINVAL, "%s: token-contiguous destination rows overlap (need stride[2] >= D*stride[3] "
                                "and stride[0] >= H*stride[2])", name);
    }
  }
  if (B * S_loc * H_loc * D == 0) return ok();
  for (int t = 0; t < n_tensors; ++t) {
    const Span sd = span_of(dst[t], 2);
    for (int i = 0; i < n_tensors * P; ++i)
      if (overlaps(sd, span_of(src[i], 2))) return fail(LSD_EINVAL, "dst[%d] overlaps src[%d]", t, i);
    for (int u = 0; u < t; ++u)
      if (overlaps(sd, span_of(dst[u], 2))) return fail(LSD_EINVAL, "dst[%d] overlaps dst[%d]", t, u);
  }

  // Tensors with channel-contiguous destinations go to the run-copy kernel,
  // token-contiguous ones to the transposing kernel (one launch each).
  lsd::RelayoutArgs a, at;
  std::memset(&a, 0, sizeof a);
  std::memset(&at, 0, sizeof at);
  bool contiguous_heads = true;
  for (int t = 0; t < n_tensors; ++t) {
    lsd::RelayoutArgs& r = tok[t] ? at : a;
    const int u = r.n_tensors++;
    for (int p = 0; p < P; ++p) {
      const lsd_view4& v = src[t * P + p];
      r.src[u][p] = (const uint16_t*)v.data;
      r.src_sb[u][p] = v.stride[0];
      r.src_ss[u][p] = v.stride[1];
      r.src_sh[u][p] = v.stride[2];
      if (!tok[t] && H_loc > 1 && v.stride[2] != D) contiguous_heads = false;
    }
    r.dst[u] = (uint16_t*)dst[t].data;
    r.dst_sb[u] = dst[t].stride[0];
    r.dst_ss[u] = dst[t].stride[1];
    r.dst_sh[u] = dst[t].stride[2];
    r.dst_sd[u] = dst[t].stride[3];
    if (!tok[t] && H_loc > 1 && dst[t].stride[2] != D) contiguous_heads = false;
  }
  for (lsd::RelayoutArgs* r : {&a, &at}) {
    r->P = P; r->rank = rank; r->B = (int)B; r->S_loc = (int)S_loc;
    r->H_loc = (int)H_loc; r->D = (int)D;
    r->inverse = inverse ? 1 : 0;
  }
  a.heads_per_run = contiguous_heads ? (int)H_loc : 1;
  at.heads_per_run = 1;
  // The copy kernel indexes runs in 32-bit signed arithmetic and advances a
  // wave's run index by about the run count (one wave per run), so the count
  // must stay at or below 2^30 for `run + stride` to fit.
  if (lsd::relayout_runs(a) > (int64_t)1 << 30)
    return fail(LSD_EUNSUPPORTED, "%s: %lld copy runs exceed 2^30", fn, (long long)lsd::relayout_runs(a));
  // transposing waves: 64-token blocks, counted in groups of 4 per (tensor, batch, head, 64 channels)
  const int64_t tok_units = (int64_t)at.n_tensors * B * H_loc * (((P * S_loc + 63) / 64 + 3) / 4 * 4) * ((D / 64 + 1) / 2);
  if (tok_units > 0x7fffffff)
    return fail(LSD_EUNSUPPORTED, "%s: %lld token-contiguous tiles exceed 2^31-1", fn, (long long)tok_units);
  if ((s = check_device()) != LSD_OK) return s;
  if (a.n_tensors > 0 && at.n_tensors > 0 && !a.inverse && lsd::relayout_runs(a) > 0)
    return launched(lsd::launch_relayout_both(a, at, (hipStream_t)stream), fn);
  if (a.n_tensors > 0 && (s = launched(lsd::launch_relayout(a, (hipStream_t)stream), fn)) != LSD_OK) return s;
  if (at.n_tensors > 0) return launched(lsd::launch_relayout_tok(at, (hipStream_t)stream), fn);
  return ok();
}

}  // namespace

extern "C" {

lsd_status lsd_cast_qkv_fp8(const lsd_view4* src, const lsd_view4* dst, float* amax, void* stream) {
  return cast_qkv_fp8(src, dst, amax, nullptr, nullptr, stream);
}

lsd_status lsd_cast_kv_fp8(const lsd_view4* src, const lsd_view4* dst, float* amax, const float* q_scale_amax,
                           const int32_t* kv_lens, void* stream) {
  if (src == nullptr || dst == nullptr) return fail(LSD_EINVAL, "null src or dst array");
  if (q_scale_amax == nullptr) return fail(LSD_EINVAL, "null q_scale_amax");
  const lsd_view4 s3[3] = {src[0], src[0], src[1]};
  const lsd_view4 d3[3] = {dst[0], dst[0], dst[1]};
  return cast_qkv_fp8(s3, d3, amax, kv_lens, q_scale_amax, stream);
}

lsd_status lsd_cast_qkv_fp8_masked(const lsd_view4* src, const lsd_view4* dst, float* amax, const int32_t* kv_lens,
                                   void* stream) {
  if (kv_lens == nullptr) return fail(LSD_EINVAL, "null kv_lens");
  return cast_qkv_fp8(src, dst, amax, kv_lens, nullptr, stream);
}

lsd_status lsd_attn_fwd_fp8(const lsd_view4* q8, const lsd_view4* k8, const lsd_view4* v8, const float* q_amax,
                            const float* k_amax, const float* v_amax, const lsd_view4* o, float* lse,
                            float softmax_scale, void* stream) {
  return attn_fwd_fp8(q8, k8, v8, q_amax, k_amax, v_amax, nullptr, o, lse, nullptr, nullptr, false, softmax_scale,
                      stream);
}

lsd_status lsd_attn_fwd_fp8_masked(const lsd_view4* q8, const lsd_view4* k8, const lsd_view4* v8,
                                   const float* q_amax, const float* k_amax, const float* v_amax,
                                   const int32_t* kv_lens, const lsd_view4* o, float* lse, float softmax_scale,
                                   void* stream) {
  if (kv_lens == nullptr) return fail(LSD_EINVAL, "null kv_lens");
  return attn_fwd_fp8(q8, k8, v8, q_amax, k_amax, v_amax, kv_lens, o, lse, nullptr, nullptr, false, softmax_scale,
                      stream);
}

lsd_status lsd_attn_fwd_fp8_accumulate(const lsd_view4* q8, const lsd_view4* k8, const lsd_view4* v8,
                                       const float* q_amax, const float* k_amax, const float* v_amax,
                                       const int32_t* kv_lens, float* o_acc, float* lse_acc, const lsd_view4* o,
                                       float softmax_scale, void* stream) {
  return attn_fwd_fp8(q8, k8, v8, q_amax, k_amax, v_amax, kv_lens, o, nullptr, o_acc, lse_acc, true, softmax_scale,
                      stream);
}

lsd_status lsd_relayout_seq_to_head(int n_tensors, int P, int rank, const lsd_view4* src, const lsd_view4* dst,
                                    void* stream) {
  return relayout(false, "relayout_seq_to_head", n_tensors, P, rank, src, dst, stream);
}

lsd_status lsd_relayout_head_to_seq(int n_tensors, int P, int rank, const lsd_view4* src, const lsd_view4* dst,
                                    void* stream) {
  return relayout(true, "relayout_head_to_seq", n_tensors, P, rank, src, dst, stream);
}

}  // extern "C"
