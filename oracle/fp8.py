"""Float64 CPU oracle for the FP8 attention inputs: the E4M3 code, the cast of
Q, K, V to FP8 with one scale per (tensor, batch, head), and attention over
the FP8 inputs.

Test infrastructure only, like the rest of this package.

Source: [NVL72] "Scaling Video Generation Across NVL72 rack with TensorRT-LLM",
"Ulysses Parallelism > Fused vs. unfused QKV all-to-all": the stacked QKV
buffer gets one FP8 cast pass before the attention kernel, in a layout the
kernel reads directly.

Readings where the pages are silent (also in the design notes):
* Format: OCP FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits;
  largest finite 448; codes 0x7F / 0xFF are NaN; no infinities).
* Scale: one per (tensor, batch, head), from the absolute maximum over that
  head's tokens and channels: the value x is coded as E4M3(x * (448 / amax))
  with the product rounded to float32 and the code rounded to nearest, ties
  to even; a head that is all zero uses the factor 1 (its codes are 0).
  Dequantised value: decode(code) * (amax / 448) in float32 arithmetic.
* For Q the stored amax is a scale amax in [amax_q, 2 amax_q): the smallest
  one at least amax_q for which the logit factor of the default softmax
  scale, log2(e) / sqrt(128) * (amax_q' / 448) * (amax_k / 448), is a power
  of two (``q_scale_amax``); Q is coded with it.  The attention kernel can
  then apply that factor exactly on the matrix cores.
* FP8 attention computes the attention of the dequantised inputs: its
  definition is ``attention`` applied to them.
* Key-length mask (the bf16 path's key-only padding mask, carried over):
  with ``kv_lens``, batch entry b has kv_lens[b] valid keys (clamped to
  [0, S]).  K's and V's amax are taken over the valid tokens only, V's codes
  of the padding tokens are zero, and K's codes of the padding tokens are
  outside the contract (the library leaves them unwritten; the attention
  never reads them).  Q is unaffected: every query row attends to the valid
  keys of its batch entry.
"""

from __future__ import annotations

import numpy as np

from . import ref

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact value of each E4M3 code (NaN for 0x7F / 0xFF), float64."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * np.exp2(e.astype(np.float64) - 10.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# every finite magnitude code 0x00..0x7E with its value, ascending
_MAG_CODES = np.arange(0x7F, dtype=np.int64)
_MAG_VALUES = e4m3_decode(_MAG_CODES)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest E4M3 code, ties to the even code
    (even mantissa); magnitudes above 464 (past the midpoint between 448 and
    the next step, 480) become NaN (0x7F with the sign), as there is no
    infinity.  The sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    # index of the largest code value <= mag
    lo = np.clip(np.searchsorted(_MAG_VALUES, mag, side="right") - 1, 0, 0x7E)
    hi = np.clip(lo + 1, 0, 0x7E)
    d_lo = mag - _MAG_VALUES[lo]
    d_hi = _MAG_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo)
    # beyond 448 the next step would be 480: 464 is the midpoint, which rounds
    # to the even mantissa (448); anything larger overflows to NaN
    code = np.where(mag > 464.0, 0x7F, code)
    code = np.where(np.isnan(x), 0x7F, code)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def head_amax(x) -> np.ndarray:
    """max |x| over tokens and channels for every (batch, head): [B, H]."""
    v = np.abs(ref._as_f64(x))
    return v.max(axis=(1, 3)) if v.shape[1] > 0 else np.zeros((v.shape[0], v.shape[2]))


def valid_lengths(kv_lens, B: int, S: int) -> np.ndarray:
    """kv_lens clamped to [0, S] per batch entry (all S without a mask)."""
    if kv_lens is None:
        return np.full(B, S, dtype=np.int64)
    return np.clip(np.asarray(kv_lens, dtype=np.int64).reshape(B), 0, S)


def head_amax_valid(x, lens) -> np.ndarray:
    """``head_amax`` over the first lens[b] tokens of each batch entry b
    (zero where there are none): [B, H]."""
    x = np.asarray(x)
    out = np.zeros((x.shape[0], x.shape[2]))
    for b in range(x.shape[0]):
        n = int(lens[b])
        if n > 0:
            out[b] = head_amax(x[b:b + 1, :n])[0]
    return out


# log2(e) / sqrt(128) in float32: the default logit factor of the attention
# (the softmax scale 1 / sqrt(D) for D = 128, times log2 e, rounded to float32)
SCALE_LOG2_D128 = np.float32(float(np.float32(1.0 / np.sqrt(128.0))) * 1.4426950408889634074)


def q_scale_amax(amax_q, amax_k) -> np.ndarray:
    """Q's scale amax per (batch, head), in float32 arithmetic step by step:
    base = SCALE_LOG2_D128 * (amax_k / 448), t = base * (amax_q / 448), e the
    smallest integer with 2^e >= t, result (2^e / base) * 448 (from 2^(e+1)
    if that falls below amax_q).  Heads with amax_q or amax_k zero, or a
    result that is not finite, keep amax_q."""
    aq = np.asarray(amax_q, dtype=np.float32)
    ak = np.asarray(amax_k, dtype=np.float32)
    c448 = np.float32(E4M3_MAX)
    base = (SCALE_LOG2_D128 * (ak / c448).astype(np.float32)).astype(np.float32)
    t = (base * (aq / c448).astype(np.float32)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        m, ex = np.frexp(t)                           # t = m 2^ex, m in [0.5, 1)
        e = np.where(m == np.float32(0.5), ex - 1, ex)
        r = ((np.ldexp(np.float32(1.0), e).astype(np.float32) / base).astype(np.float32) * c448).astype(np.float32)
        r2 = ((np.ldexp(np.float32(1.0), e + 1).astype(np.float32) / base).astype(np.float32) * c448).astype(np.float32)
    r = np.where(r < aq, r2, r)
    keep = ~(aq > 0) | ~(ak > 0) | ~np.isfinite(r)
    return np.where(keep, aq, r).astype(np.float32)


def quantize(x, amax: np.ndarray) -> np.ndarray:
    """E4M3 codes of x [B, S, H, D] with the per-(batch, head) factor
    448 / amax, computed in float32 as the scale rule states."""
    a32 = np.asarray(amax, dtype=np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(a32 > 0, np.float32(E4M3_MAX) / np.where(a32 > 0, a32, np.float32(1)), np.float32(1))
    inv = inv.astype(np.float32)
    xf = ref._as_f64(x).astype(np.float32)                         # bf16 values are exact in float32
    prod = (xf * inv[:, None, :, None]).astype(np.float32)         # one float32 rounding
    return e4m3_encode(prod)


def cast_qkv(q, k, v, kv_lens=None):
    """The single FP8 cast pass over Q, K, V: codes for each tensor and the
    amax array [3, B, H] (q's entry the scale amax of ``q_scale_amax``, k, v).
    With ``kv_lens`` (the key-length mask): K's and V's amax over the valid
    tokens, V's codes of the padding tokens zero; K's codes of the padding
    tokens are returned as computed but are outside the contract."""
    if kv_lens is None:
        amax = np.stack([head_amax(q), head_amax(k), head_amax(v)]).astype(np.float32)
    else:
        lens = valid_lengths(kv_lens, np.asarray(k).shape[0], np.asarray(k).shape[1])
        amax = np.stack([head_amax(q), head_amax_valid(k, lens), head_amax_valid(v, lens)]).astype(np.float32)
    amax[0] = q_scale_amax(amax[0], amax[1])
    with np.errstate(invalid="ignore"):
        q8, k8, v8 = quantize(q, amax[0]), quantize(k, amax[1]), quantize(v, amax[2])
    if kv_lens is not None:
        for b in range(v8.shape[0]):
            v8[b, lens[b]:] = 0
    return q8, k8, v8, amax


def cast_kv(k, v, q_scale, kv_lens=None):
    """The FP8 cast of one key/value block for a query cast earlier: codes of K
    and V and the amax array [3, B, H] ([0] zero: no Q; [1] K's scale amax, the
    ``q_scale_amax`` rule with the roles of Q and K swapped, against the given
    Q scale amax [B, H]; [2] V's amax).  ``kv_lens`` as for ``cast_qkv``."""
    if kv_lens is None:
        ak, av = head_amax(k), head_amax(v)
        lens = None
    else:
        lens = valid_lengths(kv_lens, np.asarray(k).shape[0], np.asarray(k).shape[1])
        ak, av = head_amax_valid(k, lens), head_amax_valid(v, lens)
    amax = np.stack([np.zeros_like(ak), ak, av]).astype(np.float32)
    amax[1] = q_scale_amax(amax[1], np.asarray(q_scale, dtype=np.float32))
    with np.errstate(invalid="ignore"):
        k8, v8 = quantize(k, amax[1]), quantize(v, amax[2])
    if lens is not None:
        for b in range(v8.shape[0]):
            v8[b, lens[b]:] = 0
    return k8, v8, amax


def dequantize(codes, amax) -> np.ndarray:
    """decode(code) * (amax / 448), the scale applied in float32."""
    s = (np.asarray(amax, dtype=np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_decode(codes) * s.astype(np.float64)[:, None, :, None]


def attention_fp8(q8, k8, v8, q_amax, k_amax, v_amax, scale=None, kv_lens=None):
    """Attention over the dequantised FP8 inputs (codes [B, S, H, D] and
    per-(batch, head) amax): (O, LSE) float64; ``kv_lens`` is the key-length
    mask of ``ref.attention``."""
    return ref.attention(dequantize(q8, q_amax), dequantize(k8, k_amax), dequantize(v8, v_amax), scale,
                         kv_lens=kv_lens)


def attention_fp8_accumulate(o_acc, lse_acc, q8, k8, v8, q_amax, k_amax, v_amax, scale=None, kv_lens=None):
    """One Ring step on FP8 inputs: ``ref.attention_accumulate`` of the
    dequantised q against this key/value block (its codes and per-(batch,
    head) scales), merged into the running (O_acc, LSE_acc); float64."""
    return ref.attention_accumulate(o_acc, lse_acc, dequantize(q8, q_amax), dequantize(k8, k_amax),
                                    dequantize(v8, v_amax), scale, kv_lens)


def attention_fp8_rows(q8, k8, v8, q_amax, k_amax, v_amax, b: int, h: int, rows, scale=None, kv_len=None):
    """``attention_fp8`` for selected query rows of one (batch, head), over
    the first ``kv_len`` keys (all of them by default)."""
    sq = np.float32(np.float32(q_amax[b, h]) / np.float32(E4M3_MAX))
    sk = np.float32(np.float32(k_amax[b, h]) / np.float32(E4M3_MAX))
    sv = np.float32(np.float32(v_amax[b, h]) / np.float32(E4M3_MAX))
    rows = np.asarray(list(rows), dtype=np.int64)
    qh = e4m3_decode(q8[b, rows, h, :]) * float(sq)
    n = k8.shape[1] if kv_len is None else int(np.clip(kv_len, 0, k8.shape[1]))
    kh = e4m3_decode(k8[b, :n, h, :]) * float(sk)
    vh = e4m3_decode(v8[b, :n, h, :]) * float(sv)
    return ref._attend_block(qh, kh, vh, ref._default_scale(q8.shape[3], scale))
