"""The C-ABI library (CPU only): it loads, exports every entry point that
include/lsd.h declares, and rejects invalid requests on the host before any
HIP call.  Pointers here are fake (aligned addresses that are never
dereferenced): validation is pure address arithmetic.

A few cases check that a layout is *accepted*: such a call gets past
validation to the device check, which fails where no GPU is visible.  On a
machine with a GPU that call would go on to launch a kernel on the fake
addresses, so those cases are skipped whenever a GPU is visible (the GPU
parity tests exercise the same layouts with real memory there)."""

import ctypes
import os
import re

import pytest

import long_sequence_dit_amd as lsd
from long_sequence_dit_amd import View4, LSD_EINVAL, LSD_EUNSUPPORTED

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lsd.h")

BASE = 1 << 40  # fake, 16-byte aligned device addresses


def gpu_visible() -> bool:
    """True when a GPU is visible to this process (counting devices does not
    initialise one)."""
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover - torch missing or broken
        return os.path.exists("/dev/kfd")


def skip_if_gpu(what: str) -> None:
    """Guard a call whose arguments pass validation: with fake addresses it
    may only run where the device check stops it (no GPU visible)."""
    if gpu_visible():
        pytest.skip(f"{what}: passes validation and would launch on fake addresses with a GPU visible")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsd_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = lsd.lib()
    syms = declared_symbols()
    assert {"lsd_attn_fwd", "lsd_attn_merge", "lsd_relayout_seq_to_head",
            "lsd_abi_version", "lsd_last_error"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), f"{s} declared in lsd.h but not exported by liblsd.so"
    assert L.lsd_abi_version() == 3


def view(addr, shape, stride=None):
    if stride is None:
        stride = [shape[1] * shape[2] * shape[3], shape[2] * shape[3], shape[3], 1]
    v = View4()
    v.data = addr
    for i in range(4):
        v.shape[i] = shape[i]
        v.stride[i] = stride[i]
    return v


def attn(q, k, v, o, lse=None, scale=0.0):
    L = lsd.lib()
    r = L.lsd_attn_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(o),
                       None if lse is None else ctypes.c_void_p(lse), ctypes.c_float(scale), None)
    return r, L.lsd_last_error().decode()


GB = 1 << 30


def good4(S_q=256, S_kv=256, H=2, D=64, B=1):
    return (view(BASE, (B, S_q, H, D)), view(BASE + GB, (B, S_kv, H, D)),
            view(BASE + 2 * GB, (B, S_kv, H, D)), view(BASE + 3 * GB, (B, S_q, H, D)))


@pytest.mark.parametrize("case,status,needle", [
    ("D=96", LSD_EUNSUPPORTED, "head dim"),
    ("k_heads", LSD_EINVAL, "does not match"),
    ("v_shape", LSD_EINVAL, "v shape"),
    ("o_shape", LSD_EINVAL, "o shape"),
    ("stride3", LSD_EINVAL, "stride[3]"),
    ("misaligned", LSD_EINVAL, "16-byte aligned"),
    ("stride_align", LSD_EINVAL, "multiple of 8"),
    ("null_data", LSD_EINVAL, "null data"),
    ("negative", LSD_EINVAL, "negative"),
    ("alias", LSD_EINVAL, "overlaps"),
    ("lse_alias", LSD_EINVAL, "lse overlaps"),
    ("inf_scale", LSD_EINVAL, "infinite"),
])
def test_attn_fwd_validation(case, status, needle):
    q, k, v, o = good4()
    lse = None
    scale = 0.0
    if case == "D=96":
        q, k, v, o = good4(D=96)
    elif case == "k_heads":
        k = view(BASE + GB, (1, 256, 3, 64))
    elif case == "v_shape":
        v = view(BASE + 2 * GB, (1, 128, 2, 64))
    elif case == "o_shape":
        o = view(BASE + 3 * GB, (1, 255, 2, 64))
    elif case == "stride3":
        q = view(BASE, (1, 256, 2, 64), [256 * 128 * 2, 256, 128, 2])
    elif case == "misaligned":
        q = view(BASE + 8, (1, 256, 2, 64))
    elif case == "stride_align":
        q = view(BASE, (1, 256, 2, 64), [256 * 132, 132, 68, 1])
    elif case == "null_data":
        k = view(0, (1, 256, 2, 64))
    elif case == "negative":
        q = view(BASE, (1, 256, 2, 64), [-1, 128, 64, 1])
    elif case == "alias":
        o = view(BASE + 64, (1, 256, 2, 64))
    elif case == "lse_alias":
        lse = BASE + 3 * GB + 4096
    elif case == "inf_scale":
        scale = float("inf")
    r, msg = attn(q, k, v, o, lse, scale)
    assert r == status and needle in msg, (r, msg)


def test_attn_fwd_zero_size_is_noop():
    q, k, v, o = good4(S_q=0)
    r, msg = attn(q, k, v, o)
    assert r == 0 and msg == ""


def merge(n, parts, lses, out, lse_out=None):
    L = lsd.lib()
    arr = (View4 * max(1, len(parts)))(*parts) if parts else None
    ptrs = (ctypes.c_void_p * max(1, len(lses)))(*lses) if lses else None
    r = L.lsd_attn_merge(n, arr, ptrs, ctypes.byref(out), None if lse_out is None else ctypes.c_void_p(lse_out),
                         None)
    return r, L.lsd_last_error().decode()


def test_attn_merge_validation():
    shp = (1, 100, 4, 128)
    parts = [view(BASE + i * GB, shp) for i in range(3)]
    lses = [BASE + (10 + i) * GB for i in range(3)]
    out = view(BASE + 20 * GB, shp)
    assert merge(0, parts, lses, out)[0] == LSD_EINVAL
    assert merge(17, parts * 6, lses * 6, out)[0] == LSD_EUNSUPPORTED
    bad = [parts[0], view(BASE + GB, (1, 99, 4, 128)), parts[2]]
    r, msg = merge(3, bad, lses, out)
    assert r == LSD_EINVAL and "shape differs" in msg
    r, msg = merge(3, parts, [lses[0], 0, lses[2]], out)
    assert r == LSD_EINVAL and "null" in msg
    r, msg = merge(3, parts, lses, view(BASE + GB + 512, shp))
    assert r == LSD_EINVAL and "overlaps" in msg
    r, msg = merge(3, parts, lses, out, lse_out=lses[1] + 64)
    assert r == LSD_EINVAL and "overlaps" in msg
    r, msg = merge(3, parts, lses, out, lse_out=BASE + 30 * GB + 2)
    assert r == LSD_EINVAL and "aligned" in msg


def relayout(nt, P, rank, src, dst):
    L = lsd.lib()
    sv = (View4 * len(src))(*src)
    dv = (View4 * len(dst))(*dst)
    r = L.lsd_relayout_seq_to_head(nt, P, rank, sv, dv, None)
    return r, L.lsd_last_error().decode()


def test_relayout_validation():
    B, S_loc, H, D, P = 2, 50, 40, 128, 4
    fused = [S_loc * 3 * H * D, 3 * H * D, D, 1]
    src = [view(BASE + t * H * D * 2 + p * GB, (B, S_loc, H, D), fused) for t in range(3) for p in range(P)]
    dst = [view(BASE + (10 + t) * GB, (B, P * S_loc, H // P, D)) for t in range(3)]
    assert relayout(0, P, 0, src, dst)[0] == LSD_EINVAL
    assert relayout(3, 0, 0, src, dst)[0] == LSD_EINVAL
    assert relayout(3, 17, 0, src * 6, dst)[0] == LSD_EUNSUPPORTED
    r, msg = relayout(3, P, 4, src, dst)
    assert r == LSD_EINVAL and "rank" in msg
    # 40 heads cannot be split 3 ways (the pages' divisibility rule)
    src3 = [view(BASE + p * GB, (B, S_loc, H, D), fused) for p in range(3)]
    dst3 = [view(BASE + 10 * GB, (B, 3 * S_loc, 13, D))]
    r, msg = relayout(1, 3, 0, src3, dst3)
    assert r == LSD_EINVAL and "not divisible" in msg
    # unequal shard lengths
    uneq = list(src)
    uneq[1] = view(BASE + GB, (B, S_loc - 1, H, D), fused)
    r, msg = relayout(3, P, 0, uneq, dst)
    assert r == LSD_EINVAL and "same shape" in msg
    r, msg = relayout(3, P, 0, src, [dst[0], view(BASE + 11 * GB, (B, P * S_loc, H // P + 1, D)), dst[2]])
    assert r == LSD_EINVAL and "dst[1] shape" in msg
    r, msg = relayout(3, P, 0, src, [dst[0], dst[0], dst[2]])
    assert r == LSD_EINVAL and "overlaps" in msg
    r, msg = relayout(3, P, 0, src, [view(BASE + 4096, (B, P * S_loc, H // P, D)), dst[1], dst[2]])
    assert r == LSD_EINVAL and "overlaps src" in msg


def relayout_inv(nt, P, rank, src, dst):
    L = lsd.lib()
    sv = (View4 * len(src))(*src)
    dv = (View4 * len(dst))(*dst)
    r = L.lsd_relayout_head_to_seq(nt, P, rank, sv, dv, None)
    return r, L.lsd_last_error().decode()


def test_relayout_head_to_seq_validation():
    B, S_loc, H_loc, D, P = 2, 50, 10, 128, 4
    src = [view(BASE + r * GB, (B, P * S_loc, H_loc, D)) for r in range(P)]
    dst = [view(BASE + 10 * GB, (B, S_loc, P * H_loc, D))]
    assert relayout_inv(0, P, 0, src, dst)[0] == LSD_EINVAL
    assert relayout_inv(1, 0, 0, src, dst)[0] == LSD_EINVAL
    assert relayout_inv(1, 17, 0, src * 5, dst)[0] == LSD_EUNSUPPORTED
    r, msg = relayout_inv(1, P, -1, src, dst)
    assert r == LSD_EINVAL and "rank" in msg
    # the slices' sequence length must split into P equal shards
    odd = [view(BASE + r * GB, (B, P * S_loc + 1, H_loc, D)) for r in range(P)]
    r, msg = relayout_inv(1, P, 0, odd, dst)
    assert r == LSD_EINVAL and "not divisible" in msg
    uneq = list(src)
    uneq[2] = view(BASE + 2 * GB, (B, P * S_loc, H_loc + 1, D))
    r, msg = relayout_inv(1, P, 0, uneq, dst)
    assert r == LSD_EINVAL and "same shape" in msg
    r, msg = relayout_inv(1, P, 0, src, [view(BASE + 10 * GB, (B, S_loc, H_loc, D))])
    assert r == LSD_EINVAL and "dst[0] shape" in msg
    r, msg = relayout_inv(1, P, 0, src, [view(BASE + GB + 4096, (B, S_loc, P * H_loc, D))])
    assert r == LSD_EINVAL and "overlaps src" in msg
    r, msg = relayout_inv(2, P, 0, src + src, dst + dst)
    assert r == LSD_EINVAL and "overlaps" in msg


def test_attn_fwd_masked_and_accumulate_validation():
    L = lsd.lib()
    q, k, v, o = good4()
    lens = BASE + 9 * GB
    r = L.lsd_attn_fwd_masked(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None, ctypes.byref(o), None,
                              ctypes.c_float(0.0), None)
    assert r == LSD_EINVAL and "kv_lens" in L.lsd_last_error().decode()
    r = L.lsd_attn_fwd_masked(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.c_void_p(lens + 2),
                              ctypes.byref(o), None, ctypes.c_float(0.0), None)
    assert r == LSD_EINVAL and "aligned" in L.lsd_last_error().decode()
    # an output overlapping kv_lens
    r = L.lsd_attn_fwd_masked(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.c_void_p(BASE + 3 * GB),
                              ctypes.byref(o), None, ctypes.c_float(0.0), None)
    assert r == LSD_EINVAL and "overlaps" in L.lsd_last_error().decode()
    acc, lacc = BASE + 10 * GB, BASE + 11 * GB
    r = L.lsd_attn_fwd_accumulate(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None, None,
                                  ctypes.c_void_p(lacc), None, ctypes.c_float(0.0), None)
    assert r == LSD_EINVAL and "o_acc" in L.lsd_last_error().decode()
    r = L.lsd_attn_fwd_accumulate(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None,
                                  ctypes.c_void_p(acc + 4), ctypes.c_void_p(lacc), None, ctypes.c_float(0.0), None)
    assert r == LSD_EINVAL and "16-byte" in L.lsd_last_error().decode()
    r = L.lsd_attn_fwd_accumulate(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None,
                                  ctypes.c_void_p(acc), ctypes.c_void_p(acc + 64), None, ctypes.c_float(0.0), None)
    assert r == LSD_EINVAL and "overlaps" in L.lsd_last_error().decode()
    r = L.lsd_attn_fwd_accumulate(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None,
                                  ctypes.c_void_p(BASE + 64), ctypes.c_void_p(lacc), None, ctypes.c_float(0.0), None)
    assert r == LSD_EINVAL and "overlaps" in L.lsd_last_error().decode()


def view8(addr, shape, stride):
    return view(addr, shape, stride)


def test_fp8_cast_and_attention_validation():
    L = lsd.lib()
    B, S, H, D = 2, 100, 3, 128
    bf = [view(BASE + t * GB, (B, S, H, D)) for t in range(3)]
    s_pad = 128
    q8 = view8(BASE + 10 * GB, (B, S, H, D), [S * H * D, H * D, D, 1])
    k8 = view8(BASE + 11 * GB, (B, S, H, D), [S * H * D, H * D, D, 1])
    v8 = view8(BASE + 12 * GB, (B, S, H, D), [H * D * s_pad, 1, D * s_pad, s_pad])
    amax = BASE + 13 * GB

    def cast(src, dst, am):
        r = L.lsd_cast_qkv_fp8((View4 * 3)(*src), (View4 * 3)(*dst), ctypes.c_void_p(am) if am else None, None)
        return r, L.lsd_last_error().decode()

    r, msg = cast(bf, [q8, k8, view8(BASE + 12 * GB, (B, S, H, D), [H * D * 112, 1, D * 112, 112])], amax)
    assert r == LSD_EINVAL and "rounded up to 64" in msg
    r, msg = cast(bf, [q8, k8, view8(BASE + 12 * GB, (B, S, H, D), [S * H * D, H * D, D, 1])], amax)
    assert r == LSD_EINVAL and "stride[1] must be 1" in msg
    r, msg = cast([view(BASE + t * GB, (B, S, H, 64)) for t in range(3)],
                  [view8(BASE + (10 + t) * GB, (B, S, H, 64), [S * H * 64, H * 64, 64, 1]) for t in range(2)]
                  + [view8(BASE + 12 * GB, (B, S, H, 64), [H * 64 * s_pad, 1, 64 * s_pad, s_pad])], amax)
    assert r == LSD_EUNSUPPORTED and "128" in msg
    r, msg = cast(bf, [q8, k8, v8], 0)
    assert r == LSD_EINVAL and "amax" in msg
    r, msg = cast(bf, [q8, q8, v8], amax)
    assert r == LSD_EINVAL and "overlaps" in msg
    r, msg = cast(bf, [q8, k8, v8], BASE + 12 * GB + 64)
    assert r == LSD_EINVAL and "overlaps" in msg

    o = view(BASE + 20 * GB, (B, S, H, D))

    def attn8(qv, kv, vv, ov, lse=None, amaxes=(amax, amax + 64, amax + 128)):
        a = [ctypes.c_void_p(x) if x else None for x in amaxes]
        r = L.lsd_attn_fwd_fp8(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), a[0], a[1], a[2],
                               ctypes.byref(ov), None if lse is None else ctypes.c_void_p(lse),
                               ctypes.c_float(0.0), None)
        return r, L.lsd_last_error().decode()

    r, msg = attn8(q8, k8, view8(BASE + 12 * GB, (B, S, H, D), [H * D * 96, 1, D * 96, 96]), o)
    assert r == LSD_EINVAL and "rounded up to 64" in msg
    r, msg = attn8(q8, k8, v8, o, amaxes=(amax, 0, amax))
    assert r == LSD_EINVAL and "amax" in msg
    r, msg = attn8(q8, k8, v8, view(BASE + 12 * GB + 4096, (B, S, H, D)))
    assert r == LSD_EINVAL and "overlaps" in msg
    r, msg = attn8(q8, k8, v8, o, lse=BASE + 10 * GB + 32)
    assert r == LSD_EINVAL and "overlaps" in msg
    r, msg = attn8(q8, view8(BASE + 11 * GB, (B, S, H + 1, D), [S * (H + 1) * D, (H + 1) * D, D, 1]), v8, o)
    assert r == LSD_EINVAL and "k8 shape" in msg


def test_fp8_masked_entry_points_validation():
    """The key-length variants of the FP8 cast and attention: kv_lens must be
    given, 4-byte aligned and clear of every output; the rest is checked as in
    the unmasked calls (no launch is reached in these cases)."""
    L = lsd.lib()
    B, S, H, D = 2, 100, 3, 128
    bf = [view(BASE + t * GB, (B, S, H, D)) for t in range(3)]
    q8 = view8(BASE + 10 * GB, (B, S, H, D), [S * H * D, H * D, D, 1])
    k8 = view8(BASE + 11 * GB, (B, S, H, D), [S * H * D, H * D, D, 1])
    v8 = view8(BASE + 12 * GB, (B, S, H, D), [H * D * 128, 1, D * 128, 128])
    amax = BASE + 13 * GB
    lens = BASE + 14 * GB
    o = view(BASE + 20 * GB, (B, S, H, D))

    def cast(kl, dst=(q8, k8, v8)):
        r = L.lsd_cast_qkv_fp8_masked((View4 * 3)(*bf), (View4 * 3)(*dst), ctypes.c_void_p(amax),
                                      ctypes.c_void_p(kl) if kl else None, None)
        return r, L.lsd_last_error().decode()

    def attn8(kl, ov=o):
        r = L.lsd_attn_fwd_fp8_masked(ctypes.byref(q8), ctypes.byref(k8), ctypes.byref(v8), ctypes.c_void_p(amax),
                                      ctypes.c_void_p(amax + 64), ctypes.c_void_p(amax + 128),
                                      ctypes.c_void_p(kl) if kl else None, ctypes.byref(ov), None,
                                      ctypes.c_float(0.0), None)
        return r, L.lsd_last_error().decode()

    for fn in (cast, attn8):
        r, msg = fn(0)
        assert r == LSD_EINVAL and "null kv_lens" in msg
        r, msg = fn(lens + 2)
        assert r == LSD_EINVAL and "kv_lens not 4-byte aligned" in msg
    r, msg = cast(BASE + 10 * GB + 16)                      # kv_lens inside q8's codes
    assert r == LSD_EINVAL and "overlaps kv_lens" in msg
    r, msg = attn8(BASE + 20 * GB + 16)                     # kv_lens inside o
    assert r == LSD_EINVAL and "o overlaps an input" in msg
    r, msg = cast(lens, dst=(q8, q8, v8))
    assert r == LSD_EINVAL and "overlaps" in msg


def test_fp8_kv_cast_validation():
    """The K/V-only cast: q_scale_amax must be given and aligned and may not
    overlap an output; K and V must have one shape."""
    L = lsd.lib()
    B, S, H, D = 2, 100, 3, 128
    src = [view(BASE + t * GB, (B, S, H, D)) for t in range(2)]
    k8 = view8(BASE + 11 * GB, (B, S, H, D), [S * H * D, H * D, D, 1])
    v8 = view8(BASE + 12 * GB, (B, S, H, D), [H * D * 128, 1, D * 128, 128])
    amax, qs = BASE + 13 * GB, BASE + 14 * GB

    def cast(sv, dv, q):
        r = L.lsd_cast_kv_fp8((View4 * 2)(*sv), (View4 * 2)(*dv), ctypes.c_void_p(amax),
                              ctypes.c_void_p(q) if q else None, None, None)
        return r, L.lsd_last_error().decode()

    r, msg = cast(src, [k8, v8], 0)
    assert r == LSD_EINVAL and "null q_scale_amax" in msg
    r, msg = cast(src, [k8, v8], qs + 2)
    assert r == LSD_EINVAL and "q_scale_amax not 4-byte aligned" in msg
    r, msg = cast(src, [k8, v8], amax + 8)
    assert r == LSD_EINVAL and "amax overlaps q_scale_amax" in msg
    r, msg = cast([src[0], view(BASE + GB, (B, S + 1, H, D))], [k8, v8], qs)
    assert r == LSD_EINVAL and "one shape" in msg


def test_fp8_accumulate_validation():
    """The FP8 Ring step: o_acc and lse_acc must be given and aligned, and no
    output (o_acc, lse_acc, o) may overlap an input or another output."""
    L = lsd.lib()
    B, S, H, D = 2, 100, 3, 128
    q8 = view8(BASE + 10 * GB, (B, S, H, D), [S * H * D, H * D, D, 1])
    k8 = view8(BASE + 11 * GB, (B, S, H, D), [S * H * D, H * D, D, 1])
    v8 = view8(BASE + 12 * GB, (B, S, H, D), [H * D * 128, 1, D * 128, 128])
    amax = BASE + 13 * GB
    o_acc, lse_acc = BASE + 15 * GB, BASE + 16 * GB

    def acc(oa, la, o=None):
        r = L.lsd_attn_fwd_fp8_accumulate(ctypes.byref(q8), ctypes.byref(k8), ctypes.byref(v8), ctypes.c_void_p(amax),
                                          ctypes.c_void_p(amax + 64), ctypes.c_void_p(amax + 128), None,
                                          ctypes.c_void_p(oa) if oa else None, ctypes.c_void_p(la) if la else None,
                                          None if o is None else ctypes.byref(o), ctypes.c_float(0.0), None)
        return r, L.lsd_last_error().decode()

    r, msg = acc(0, lse_acc)
    assert r == LSD_EINVAL and "null o_acc or lse_acc" in msg
    r, msg = acc(o_acc + 4, lse_acc)
    assert r == LSD_EINVAL and "o_acc not 16-byte aligned" in msg
    r, msg = acc(o_acc, lse_acc + 2)
    assert r == LSD_EINVAL and "lse_acc not 4-byte aligned" in msg
    r, msg = acc(BASE + 10 * GB + 64, lse_acc)
    assert r == LSD_EINVAL and "o_acc overlaps an input" in msg
    r, msg = acc(o_acc, o_acc + 256)
    assert r == LSD_EINVAL and "lse_acc overlaps o_acc" in msg
    r, msg = acc(o_acc, lse_acc, view(o_acc + 1024, (B, S, H, D)))
    assert r == LSD_EINVAL and "overlaps o" in msg


def test_attn_fwd_rejects_huge_kv_stride():
    q, k, v, o = good4()
    k = view(BASE + GB, (1, 256, 2, 64), [256 * (1 << 24), 1 << 24, 64, 1])
    r, msg = attn(q, k, v, o)
    assert r == LSD_EUNSUPPORTED and "2^24" in msg


def vt_view(addr, B, S, H, D, pitch):
    # token-contiguous V: storage [B, H, D, pitch]
    return view(addr, (B, S, H, D), [H * D * pitch, 1, D * pitch, pitch])


def test_attn_fwd_token_major_v_validation():
    q, k, _, o = good4(S_kv=300)
    B, S_kv, H, D = 1, 300, 2, 64
    r, msg = attn(q, k, vt_view(BASE + 2 * GB, B, S_kv, H, D, 296), o)
    assert r == LSD_EINVAL and "below S=300" in msg
    r, msg = attn(q, k, vt_view(BASE + 2 * GB, B, S_kv, H, D, 308), o)
    assert r == LSD_EINVAL and "stride[3]" in msg and "multiple of 8" in msg
    r, msg = attn(q, k, vt_view(BASE + 2 * GB, B, S_kv, H, D, 1 << 23), o)
    assert r == LSD_EUNSUPPORTED and "2^23" in msg
    r, msg = attn(q, k, vt_view(BASE + 2 * GB + 2, B, S_kv, H, D, 304), o)
    assert r == LSD_EINVAL and "16-byte aligned" in msg
    # neither channels nor tokens unit-stride
    r, msg = attn(q, k, view(BASE + 2 * GB, (B, S_kv, H, D), [S_kv * H * D * 2, 2, S_kv * D * 2, 8]), o)
    assert r == LSD_EINVAL and "stride[3] must be 1" in msg
    # overlap with an output is still caught
    r, msg = attn(q, k, vt_view(BASE + 3 * GB, B, S_kv, H, D, 304), o)
    assert r == LSD_EINVAL and "overlaps" in msg


def test_attn_fwd_token_major_v_accepted():
    skip_if_gpu("accepted token-contiguous V layouts")
    q, k, _, o = good4(S_kv=300)
    B, S_kv, H, D = 1, 300, 2, 64
    # accepted layout: validation passes, so the call reaches the device check
    # (no GPU here) instead of failing on the view
    r, msg = attn(q, k, vt_view(BASE + 2 * GB, B, S_kv, H, D, 304), o)
    assert r != 0 and "v:" not in msg and "pitch" not in msg
    # a token-contiguous v may have a huge batch stride (the 2^24 limit is on k and natural v)
    vt = view(BASE + 2 * GB, (B, S_kv, H, D), [1 << 30, 1, D * 304, 304])
    r, msg = attn(q, k, vt, o)
    assert r != 0 and "2^24" not in msg and "v:" not in msg


def test_relayout_token_major_destination_validation():
    B, S_loc, H, D, P = 1, 100, 4, 64, 2
    src = (View4 * (3 * P))(*[view(BASE + i * GB, (B, S_loc, H, D)) for i in range(3 * P)])
    S, Hl = P * S_loc, H // P
    def dsts(vt):
        return (View4 * 3)(view(BASE + 10 * GB, (B, S, Hl, D)), view(BASE + 11 * GB, (B, S, Hl, D)), vt)
    if not gpu_visible():  # accepted: reaches the device check, which stops it without a GPU
        ok_vt = vt_view(BASE + 12 * GB, B, S, Hl, D, 200)
        r, msg = relayout(3, P, 0, src, dsts(ok_vt))
        assert r != 0 and "dst" not in msg
    r, msg = relayout(3, P, 0, src, dsts(vt_view(BASE + 12 * GB, B, S, Hl, D, 192)))
    assert r == LSD_EINVAL and "below S=200" in msg
    r, msg = relayout(3, P, 0, src, dsts(view(BASE + 12 * GB, (B, S, Hl, D), [Hl * D * 200, 1, 104, 200])))
    assert r == LSD_EINVAL and "overlap" in msg
    src32 = (View4 * (3 * P))(*[view(BASE + i * GB, (B, S_loc, H, 32)) for i in range(3 * P)])
    d32 = (View4 * 3)(view(BASE + 10 * GB, (B, S, Hl, 32)), view(BASE + 11 * GB, (B, S, Hl, 32)),
                      vt_view(BASE + 12 * GB, B, S, Hl, 32, 200))
    r, msg = relayout(3, P, 0, src32, d32)
    assert r == LSD_EUNSUPPORTED and "multiple of 64" in msg
    # the inverse writes channel-contiguous shards only
    isrc = (View4 * P)(*[view(BASE + i * GB, (B, S, Hl, D)) for i in range(P)])
    r, msg = relayout_inv(1, P, 0, isrc, (View4 * 1)(vt_view(BASE + 12 * GB, B, S_loc, H, D, 104)))
    assert r == LSD_EINVAL and "inverse" in msg


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros((1, 8, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU memory"):
        lsd.attn_fwd(q, q, q)


def test_python_binding_refuses_non_bf16_attention_and_merge_operands():
    """fp16 (or int16) bits would be read as bf16 and give a silently wrong
    result: attention and merge take bfloat16 only (checked before any device
    work); the relayouts, pure bit copies, accept any 16-bit type."""
    torch = pytest.importorskip("torch")
    b = torch.zeros((1, 8, 1, 64), dtype=torch.bfloat16)
    for dt in (torch.float16, torch.int16):
        h = torch.zeros((1, 8, 1, 64), dtype=dt)
        with pytest.raises(ValueError, match="bfloat16"):
            lsd.attn_fwd(h, b, b)
        with pytest.raises(ValueError, match="bfloat16"):
            lsd.attn_fwd_accumulate(h, b, b, torch.zeros((1, 8, 1, 64)), torch.zeros((1, 1, 8)))
        with pytest.raises(ValueError, match="bfloat16"):
            lsd.attn_merge([h, b], [torch.zeros((1, 1, 8)), torch.zeros((1, 1, 8))])
        with pytest.raises(ValueError, match="GPU memory"):   # passes the dtype check, stops at the device
            lsd.relayout_seq_to_head([[h]], 1, 0, dst=[h.clone()])
