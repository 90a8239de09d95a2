"""Python binding of liblsd.so, the MI355X long-sequence DiT attention library.

Argument marshalling only: each function turns torch tensors (device memory
and the current stream) into the C-ABI views of ``include/lsd.h`` and calls
the matching entry point; every step of the computation runs in the HIP
kernels.  There is no fallback: if the library is missing, or a tensor is not
on a GPU, or the device is not gfx950, the call raises.

Entry points (same names as the C ABI without the ``lsd_`` prefix):

* ``attn_fwd(q, k, v, o=None, lse=None, scale=None, return_lse=True)``
* ``attn_merge(o_parts, lse_parts, o=None, lse=None, return_lse=True)``
* ``relayout_seq_to_head(src, P, rank, dst=None)``
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsd.so")

LSD_OK, LSD_EINVAL, LSD_EUNSUPPORTED, LSD_EDEVICE = 0, 1, 2, 3


class View4(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p),
                ("shape", ctypes.c_int64 * 4),
                ("stride", ctypes.c_int64 * 4)]


_lib = None


def lib():
    """Load liblsd.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -m long_sequence_dit_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.lsd_abi_version.restype = ctypes.c_int
        L.lsd_last_error.restype = ctypes.c_char_p
        L.lsd_attn_fwd.restype = ctypes.c_int
        L.lsd_attn_fwd.argtypes = [P(View4), P(View4), P(View4), P(View4), ctypes.c_void_p,
                                   ctypes.c_float, ctypes.c_void_p]
        L.lsd_attn_merge.restype = ctypes.c_int
        L.lsd_attn_merge.argtypes = [ctypes.c_int, P(View4), P(ctypes.c_void_p), P(View4),
                                     ctypes.c_void_p, ctypes.c_void_p]
        L.lsd_relayout_seq_to_head.restype = ctypes.c_int
        L.lsd_relayout_seq_to_head.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P(View4),
                                               P(View4), ctypes.c_void_p]
        L.lsd_attn_fwd_masked.restype = ctypes.c_int
        L.lsd_attn_fwd_masked.argtypes = [P(View4), P(View4), P(View4), ctypes.c_void_p, P(View4),
                                          ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
        L.lsd_attn_fwd_accumulate.restype = ctypes.c_int
        L.lsd_attn_fwd_accumulate.argtypes = [P(View4), P(View4), P(View4), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, P(View4), ctypes.c_float, ctypes.c_void_p]
        L.lsd_cast_qkv_fp8.restype = ctypes.c_int
        L.lsd_cast_qkv_fp8.argtypes = [P(View4), P(View4), ctypes.c_void_p, ctypes.c_void_p]
        L.lsd_attn_fwd_fp8.restype = ctypes.c_int
        L.lsd_attn_fwd_fp8.argtypes = [P(View4), P(View4), P(View4), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, P(View4), ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
        L.lsd_cast_qkv_fp8_masked.restype = ctypes.c_int
        L.lsd_cast_qkv_fp8_masked.argtypes = [P(View4), P(View4), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.lsd_attn_fwd_fp8_masked.restype = ctypes.c_int
        L.lsd_attn_fwd_fp8_masked.argtypes = [P(View4), P(View4), P(View4), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, P(View4), ctypes.c_void_p,
                                              ctypes.c_float, ctypes.c_void_p]
        L.lsd_cast_kv_fp8.restype = ctypes.c_int
        L.lsd_cast_kv_fp8.argtypes = [P(View4), P(View4), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
        L.lsd_attn_fwd_fp8_accumulate.restype = ctypes.c_int
        L.lsd_attn_fwd_fp8_accumulate.argtypes = [P(View4), P(View4), P(View4), ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, P(View4), ctypes.c_float, ctypes.c_void_p]
        L.lsd_relayout_head_to_seq.restype = ctypes.c_int
        L.lsd_relayout_head_to_seq.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P(View4),
                                               P(View4), ctypes.c_void_p]
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status == LSD_OK:
        return
    msg = lib().lsd_last_error().decode(errors="replace")
    if status in (LSD_EINVAL, LSD_EUNSUPPORTED):
        raise ValueError(f"{what}: {msg}")
    raise RuntimeError(f"{what}: {msg}")


def _torch():
    import torch
    return torch


_16BIT = None


def _view(t, name: str, any16: bool = False) -> View4:
    """C view of a 4-d GPU tensor.  Attention and merge operands must be
    bfloat16 (the kernels read bf16 bits; an fp16 tensor would be silently
    misread); the relayouts copy bit patterns and accept any 16-bit type
    (``any16``)."""
    torch = _torch()
    global _16BIT
    if _16BIT is None:
        _16BIT = {torch.bfloat16, torch.int16, torch.uint16, torch.float16}
    if t.dim() != 4:
        raise ValueError(f"{name}: expected a 4-d (B, S, H, D) tensor, got {t.dim()}-d")
    if any16 and t.dtype not in _16BIT:
        raise ValueError(f"{name}: expected 16-bit elements, got {t.dtype}")
    if not any16 and t.dtype != torch.bfloat16:
        raise ValueError(f"{name}: expected bfloat16 elements, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor must be in GPU memory (HIP library, no CPU path)")
    v = View4()
    v.data = t.data_ptr()
    for i in range(4):
        v.shape[i] = t.shape[i]
        v.stride[i] = t.stride(i)
    return v


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _f32_ptr(t, name, shape):
    torch = _torch()
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected a contiguous float32 GPU tensor of shape {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _lens_ptr(kv_lens, B):
    torch = _torch()
    if kv_lens is None:
        return None
    if kv_lens.dtype != torch.int32 or not kv_lens.is_cuda or not kv_lens.is_contiguous() or \
            tuple(kv_lens.shape) != (B,):
        raise ValueError(f"kv_lens: expected a contiguous int32 GPU tensor of shape ({B},)")
    return ctypes.c_void_p(kv_lens.data_ptr())


def attn_fwd(q, k, v, o=None, lse=None, scale: Optional[float] = None, return_lse: bool = True, kv_lens=None):
    """O = softmax(scale * Q K^T) V per (batch, head), plus the natural-log LSE.

    q: (B, S_q, H, D) bf16, k/v: (B, S_kv, H, D) bf16 (strided views allowed,
    last dim contiguous; v may instead be token-contiguous, see
    ``v_token_major``).  Returns ``o`` (and ``lse`` [B, H, S_q] float32 when
    ``return_lse``).  ``scale`` defaults to 1/sqrt(D).  ``kv_lens`` (int32 [B]
    on the GPU) is a key-only padding mask: batch entry b attends its first
    kv_lens[b] keys.
    """
    torch = _torch()
    B, S_q, H, D = q.shape
    if o is None:
        o = torch.empty((B, S_q, H, D), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device)
    vq, vk, vv, vo = _view(q, "q"), _view(k, "k"), _view(v, "v"), _view(o, "o")
    lp = _f32_ptr(lse, "lse", (B, H, S_q)) if lse is not None else None
    sc = ctypes.c_float(0.0 if scale is None else float(scale))
    if kv_lens is None:
        st = lib().lsd_attn_fwd(ctypes.byref(vq), ctypes.byref(vk), ctypes.byref(vv), ctypes.byref(vo), lp, sc,
                                _stream(q))
        _check(st, "lsd_attn_fwd")
    else:
        st = lib().lsd_attn_fwd_masked(ctypes.byref(vq), ctypes.byref(vk), ctypes.byref(vv), _lens_ptr(kv_lens, B),
                                       ctypes.byref(vo), lp, sc, _stream(q))
        _check(st, "lsd_attn_fwd_masked")
    return (o, lse) if lse is not None else o


def attn_fwd_accumulate(q, k, v, o_acc, lse_acc, o=None, scale=None, kv_lens=None):
    """One Ring step: attention of q against the key/value block (k, v), merged
    in place into the running float32 result o_acc [B,S_q,H,D] and lse_acc
    [B,H,S_q] (start with lse_acc = -inf).  If ``o`` (bf16 [B,S_q,H,D]) is given,
    the updated running output is also written to it in bf16.  ``kv_lens`` is
    the block's key-only padding mask as in ``attn_fwd``.  Returns o."""
    B, S_q, H, D = q.shape
    qv, kv, vv = _view(q, "q"), _view(k, "k"), _view(v, "v")
    ov = _view(o, "o") if o is not None else None
    if o_acc is None or lse_acc is None:
        raise ValueError("attn_fwd_accumulate: o_acc and lse_acc are required")
    pa = _f32_ptr(o_acc, "o_acc", (B, S_q, H, D))
    pl = _f32_ptr(lse_acc, "lse_acc", (B, H, S_q))
    st = lib().lsd_attn_fwd_accumulate(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), _lens_ptr(kv_lens, B),
                                       pa, pl,
                                       ctypes.byref(ov) if ov is not None else None,
                                       ctypes.c_float(0.0 if scale is None else float(scale)), _stream(q))
    _check(st, "lsd_attn_fwd_accumulate")
    return o


def attn_merge(o_parts: Sequence, lse_parts: Sequence, o=None, lse=None, return_lse: bool = True):
    """Exact log-sum-exp merge of n partial (O_i, LSE_i) over disjoint key spans."""
    torch = _torch()
    n = len(o_parts)
    if n != len(lse_parts) or n == 0:
        raise ValueError("attn_merge: need as many LSE arrays as partial outputs (n >= 1)")
    B, S, H, D = o_parts[0].shape
    if o is None:
        o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=o_parts[0].device)
    if return_lse and lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=o.device)
    views = (View4 * n)(*[_view(t, f"o_parts[{i}]") for i, t in enumerate(o_parts)])
    ptrs = (ctypes.c_void_p * n)(*[_f32_ptr(t, f"lse_parts[{i}]", (B, H, S)).value
                                   for i, t in enumerate(lse_parts)])
    vo = _view(o, "o")
    lp = _f32_ptr(lse, "lse", (B, H, S)) if lse is not None else None
    st = lib().lsd_attn_merge(n, views, ptrs, ctypes.byref(vo), lp, _stream(o))
    _check(st, "lsd_attn_merge")
    return (o, lse) if lse is not None else o


def _view8(t, name):
    """View of a one-byte-per-element tensor (strides in bytes)."""
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor must be in GPU memory")
    if t.element_size() != 1 or t.dim() != 4:
        raise ValueError(f"{name}: expected a 4-d tensor of one-byte elements (FP8 codes)")
    v = View4()
    v.data = t.data_ptr()
    for i in range(4):
        v.shape[i] = t.shape[i]
        v.stride[i] = t.stride(i)
    return v


def v_token_major(B, S, H, D, device="cuda", pitch=None):
    """Allocate a bf16 V stored token-contiguous: a (B, S, H, D) view whose
    storage is [B, H, D, pitch] (each channel's S keys one row; pitch defaults
    to S rounded up to 64, which starts every row on a 128-byte line; any
    multiple of 8 that is at least S is accepted).  Attention stages such a V
    straight from HBM into LDS, and ``relayout_seq_to_head`` writes V in this
    layout when given one."""
    torch = _torch()
    p = (S + 63) // 64 * 64 if pitch is None else int(pitch)
    if p < S or p % 8 != 0:
        raise ValueError(f"v_token_major: pitch {p} must be a multiple of 8 and at least S={S}")
    vt = torch.empty((B, H, D, p), dtype=torch.bfloat16, device=device)
    return vt.permute(0, 3, 1, 2)[:, :S]


def fp8_buffers(B, S, H, D=128, device="cuda"):
    """Allocate the outputs of ``cast_qkv_fp8``: q8, k8 (B, S, H, D) and v8, the
    (B, S, H, D) view of V stored transposed with rows padded to a multiple of
    64 tokens (storage [B, H, D, S_pad]), plus amax [3, B, H]."""
    torch = _torch()
    s_pad = (S + 63) // 64 * 64
    q8 = torch.empty((B, S, H, D), dtype=torch.float8_e4m3fn, device=device)
    k8 = torch.empty((B, S, H, D), dtype=torch.float8_e4m3fn, device=device)
    vt = torch.empty((B, H, D, s_pad), dtype=torch.float8_e4m3fn, device=device)
    v8 = vt.permute(0, 3, 1, 2)[:, :S]
    amax = torch.empty((3, B, H), dtype=torch.float32, device=device)
    return q8, k8, v8, amax


def cast_qkv_fp8(q, k, v, out=None, kv_lens=None):
    """One FP8 (E4M3) cast of Q, K, V (bf16 (B, S, H, D) views) with one scale
    per (tensor, batch, head).  Returns (q8, k8, v8, amax): v8 is a (B, S, H, D)
    view of V stored transposed; amax[t] is tensor t's per-(b, h) scale amax
    (K, V: max |x|; Q: the power-of-two-adjusted value in [amax_q, 2 amax_q)
    described in include/lsd.h).  ``kv_lens`` (int32 [B] on the GPU) is the
    key-length mask: K and V scales from the first kv_lens[b] tokens, V codes
    of the rest zero, K codes of the rest not written."""
    B, S, H, D = q.shape
    if out is None:
        out = fp8_buffers(B, S, H, D, q.device)
    q8, k8, v8, amax = out
    sv = (View4 * 3)(_view(q, "q"), _view(k, "k"), _view(v, "v"))
    dv = (View4 * 3)(_view8(q8, "q8"), _view8(k8, "k8"), _view8(v8, "v8"))
    ap = _f32_ptr(amax, "amax", (3, B, H))
    if kv_lens is None:
        st = lib().lsd_cast_qkv_fp8(sv, dv, ap, _stream(q))
        _check(st, "lsd_cast_qkv_fp8")
    else:
        st = lib().lsd_cast_qkv_fp8_masked(sv, dv, ap, _lens_ptr(kv_lens, B), _stream(q))
        _check(st, "lsd_cast_qkv_fp8_masked")
    return q8, k8, v8, amax


def cast_kv_fp8(k, v, q_scale_amax, out=None, kv_lens=None):
    """The FP8 cast of one K/V block for a query cast earlier: K's scale amax is
    chosen against ``q_scale_amax`` (float32 [B, H], the query cast's amax[0])
    so that the default logit factor is a power of two.  Returns (k8, v8,
    amax) with amax [3, B, H] ([0] zero, [1] K's scale amax, [2] V's);
    ``out`` may be ``fp8_buffers(...)`` (its q8 is left untouched)."""
    B, S, H, D = k.shape
    if out is None:
        out = fp8_buffers(B, S, H, D, k.device)
    _, k8, v8, amax = out
    sv = (View4 * 2)(_view(k, "k"), _view(v, "v"))
    dv = (View4 * 2)(_view8(k8, "k8"), _view8(v8, "v8"))
    st = lib().lsd_cast_kv_fp8(sv, dv, _f32_ptr(amax, "amax", (3, B, H)), _f32_ptr(q_scale_amax, "q_scale_amax", (B, H)),
                               _lens_ptr(kv_lens, B), _stream(k))
    _check(st, "lsd_cast_kv_fp8")
    return k8, v8, amax


def attn_fwd_fp8(q8, k8, v8, q_amax, k_amax, v_amax, o=None, lse=None, scale: Optional[float] = None,
                 return_lse: bool = True, kv_lens=None):
    """Attention over FP8 inputs (as ``cast_qkv_fp8`` produces them): the
    attention of the dequantised values, O in bf16 and the LSE.  ``kv_lens``
    (int32 [B] on the GPU): batch entry b attends only its first kv_lens[b]
    keys."""
    torch = _torch()
    B, S_q, H, D = q8.shape
    if o is None:
        o = torch.empty((B, S_q, H, D), dtype=torch.bfloat16, device=q8.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q8.device)
    qv, kv, vv, ov = _view8(q8, "q8"), _view8(k8, "k8"), _view8(v8, "v8"), _view(o, "o")
    pq, pk, pv = (_f32_ptr(x, n, (B, H)) for x, n in ((q_amax, "q_amax"), (k_amax, "k_amax"), (v_amax, "v_amax")))
    lp = _f32_ptr(lse, "lse", (B, H, S_q)) if lse is not None else None
    sc = ctypes.c_float(0.0 if scale is None else float(scale))
    if kv_lens is None:
        st = lib().lsd_attn_fwd_fp8(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), pq, pk, pv,
                                    ctypes.byref(ov), lp, sc, _stream(q8))
        _check(st, "lsd_attn_fwd_fp8")
    else:
        st = lib().lsd_attn_fwd_fp8_masked(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), pq, pk, pv,
                                           _lens_ptr(kv_lens, B), ctypes.byref(ov), lp, sc, _stream(q8))
        _check(st, "lsd_attn_fwd_fp8_masked")
    return (o, lse) if lse is not None else o


def attn_fwd_fp8_accumulate(q8, k8, v8, q_amax, k_amax, v_amax, o_acc, lse_acc, o=None,
                            scale: Optional[float] = None, kv_lens=None):
    """One Ring step on FP8 inputs: FP8 attention of q8 against this K/V block
    (codes and scales of the block's cast), merged in place into the running
    float32 ``o_acc`` (B, S_q, H, D) and ``lse_acc`` (B, H, S_q); start with
    lse_acc = -inf.  ``o`` (bf16), if given, receives the updated result.
    ``kv_lens`` is the block's key-length mask.  Returns o."""
    B, S_q, H, D = q8.shape
    if o_acc is None or lse_acc is None:
        raise ValueError("attn_fwd_fp8_accumulate: o_acc and lse_acc are required")
    qv, kv, vv = _view8(q8, "q8"), _view8(k8, "k8"), _view8(v8, "v8")
    ov = _view(o, "o") if o is not None else None
    pq, pk, pv = (_f32_ptr(x, n, (B, H)) for x, n in ((q_amax, "q_amax"), (k_amax, "k_amax"), (v_amax, "v_amax")))
    pa = _f32_ptr(o_acc, "o_acc", (B, S_q, H, D))
    pl = _f32_ptr(lse_acc, "lse_acc", (B, H, S_q))
    st = lib().lsd_attn_fwd_fp8_accumulate(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), pq, pk, pv,
                                           _lens_ptr(kv_lens, B), pa, pl,
                                           ctypes.byref(ov) if ov is not None else None,
                                           ctypes.c_float(0.0 if scale is None else float(scale)), _stream(q8))
    _check(st, "lsd_attn_fwd_fp8_accumulate")
    return o


def relayout_seq_to_head(src: Sequence[Sequence], P: int, rank: int, dst: Optional[List] = None):
    """Ulysses seq-major -> head-major relayout for destination ``rank``.

    src: one list per tensor (1 to 3 of them, e.g. Q, K, V), each holding the P
    sequence shards (B, S_loc, H, D).  Returns one (B, P*S_loc, H/P, D) tensor
    per source tensor.  A destination given token-contiguous (``v_token_major``)
    is written in that layout.
    """
    torch = _torch()
    nt = len(src)
    if nt == 0 or any(len(s) != P for s in src):
        raise ValueError("relayout_seq_to_head: src must be n_tensors lists of P shards each")
    B, S_loc, H, D = src[0][0].shape
    if dst is None:
        if H % P != 0:
            raise ValueError(f"relayout_seq_to_head: head count H={H} is not divisible by P={P}")
        dst = [torch.empty((B, P * S_loc, H // P, D), dtype=src[0][0].dtype, device=src[0][0].device)
               for _ in range(nt)]
    sv = (View4 * (nt * P))(*[_view(c, f"src[{t}][{p}]", any16=True) for t, s in enumerate(src)
                              for p, c in enumerate(s)])
    dv = (View4 * nt)(*[_view(d, f"dst[{t}]", any16=True) for t, d in enumerate(dst)])
    st = lib().lsd_relayout_seq_to_head(nt, P, rank, sv, dv, _stream(src[0][0]))
    _check(st, "lsd_relayout_seq_to_head")
    return dst


def relayout_head_to_seq(src: Sequence[Sequence], P: int, rank: int, dst: Optional[List] = None):
    """Ulysses head-major -> seq-major relayout for destination ``rank`` (the
    inverse of ``relayout_seq_to_head``, run on the attention output).

    src: one list per tensor (1 to 3 of them), each holding the P ranks' head
    slices (B, P*S_loc, H_loc, D).  Returns one (B, S_loc, P*H_loc, D) tensor per
    source tensor: sequence shard ``rank`` with every head.
    """
    torch = _torch()
    nt = len(src)
    if nt == 0 or any(len(s) != P for s in src):
        raise ValueError("relayout_head_to_seq: src must be n_tensors lists of P head slices each")
    B, S, H_loc, D = src[0][0].shape
    if dst is None:
        if S % P != 0:
            raise ValueError(f"relayout_head_to_seq: sequence length S={S} is not divisible by P={P}")
        dst = [torch.empty((B, S // P, P * H_loc, D), dtype=src[0][0].dtype, device=src[0][0].device)
               for _ in range(nt)]
    sv = (View4 * (nt * P))(*[_view(c, f"src[{t}][{r}]", any16=True) for t, s in enumerate(src)
                              for r, c in enumerate(s)])
    dv = (View4 * nt)(*[_view(d, f"dst[{t}]", any16=True) for t, d in enumerate(dst)])
    st = lib().lsd_relayout_head_to_seq(nt, P, rank, sv, dv, _stream(src[0][0]))
    _check(st, "lsd_relayout_head_to_seq")
    return dst
