"""The FP8 path on the GPU (through the C ABI): the cast of Q, K, V to E4M3
bit-exact against the oracle (codes and amax), and FP8 attention against the
oracle's attention of the dequantised inputs within the FP8 contract:

  per element  |O - O_ref| <= 2^-4 A + 2^-10 C + 2^-8 |O_ref| + 1e-5
  overall      mean |O - O_ref| <= 0.05 mean |O_ref| + 1e-4
  LSE          |LSE - LSE_ref| <= 1e-3

with A = sum_j p_j |v_j| / l and C = sum_j |v_j| / l (p_j = exp(s_j - max s),
l = sum p): the E4M3 weights carry at most half an ulp (2^-4) of relative
error, or 2^-10 absolute below the normal range; the bf16 output adds 2^-9
relative.  The logits are exact FP8 products summed in float32, so the LSE
keeps the bf16 path's bar."""

import numpy as np
import pytest

import synth
from oracle import fp8, ref
from gpu_util import note, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

lsd = pytest.importorskip("long_sequence_dit_amd")


def codes(x):
    t = torch()
    return np.ascontiguousarray(x.view(t.uint8).cpu().numpy())


def deq_rows(c, amax, b, h, rows=None):
    s = float(np.float32(np.float32(amax[b, h]) / np.float32(448.0)))
    x = c[b, :, h, :] if rows is None else c[b, rows, h, :]
    return fp8.e4m3_decode(x) * s


def check_fp8(o, lse, q8, k8, v8, amax, heads, rows_fn, what, scale=None, lse_tol=1e-3):
    """o, lse on the GPU; q8/k8/v8 host codes (B, S, H, D); amax [3, B, H]."""
    og = to_f64(o)
    lg = lse.cpu().numpy()
    D = q8.shape[3]
    sc = ref._default_scale(D, scale)
    worst = 0.0
    worst_lse = 0.0
    errs, mags = [], []
    for b in range(q8.shape[0]):
        for h in heads:
            rows = rows_fn(b, h)
            qh = deq_rows(q8, amax[0], b, h, rows)
            kh = deq_rows(k8, amax[1], b, h)
            vh = deq_rows(v8, amax[2], b, h)
            O, L = ref._attend_block(qh, kh, vh, sc)
            if kh.shape[0] == 0:
                assert np.all(og[b, rows, h] == 0) and np.all(np.isneginf(lg[b, h, rows])), what
                continue
            s = (qh @ kh.T) * sc
            p = np.exp(s - s.max(axis=1, keepdims=True))
            l = p.sum(axis=1, keepdims=True)
            A = (p @ np.abs(vh)) / l
            C = np.abs(vh).sum(axis=0)[None, :] / l
            bound = 2.0 ** -4 * A + 2.0 ** -10 * C + 2.0 ** -8 * np.abs(O) + 1e-5
            err = np.abs(og[b, rows, h] - O)
            assert np.all(np.isfinite(og[b, rows, h])), f"{what} b={b} h={h}: non-finite"
            ratio = float((err / bound).max())
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"{what} b={b} h={h}: error exceeds the FP8 bound (ratio {ratio:.3f})"
            dl = np.abs(lg[b, h, rows] - L)
            assert dl.max() <= lse_tol, f"{what} b={b} h={h}: LSE max-abs {dl.max():.3e}"
            worst_lse = max(worst_lse, float(dl.max()))
            errs.append(err.ravel())
            mags.append(np.abs(O).ravel())
    if errs:
        e, m = np.concatenate(errs), np.concatenate(mags)
        assert e.mean() <= 0.05 * m.mean() + 1e-4, f"{what}: mean-abs {e.mean():.3e} vs mean|O| {m.mean():.3e}"
        note(f"{what}: worst bound ratio {worst:.3f}, mean-abs {e.mean():.3e} ({e.mean() / max(m.mean(), 1e-30):.2%} "
             f"of mean |O|), worst LSE max-abs {worst_lse:.3e}")


def all_rows(S):
    return lambda b, h: np.arange(S)


@pytest.mark.parametrize("shape", [(2, 100, 3), (1, 64, 2), (1, 1, 1), (2, 257, 2), (2, 1000, 40)])
def test_cast_bit_exact(shape):
    B, S, H = shape
    note(f"fp8 cast B={B} S={S} H={H}")
    t = torch()
    q = synth.normal_bf16((B, S, H, 128), 100, 1)
    k = synth.normal_bf16((B, S, H, 128), 101, 1).copy()
    v = synth.normal_bf16((B, S, H, 128), 102, 1).copy()
    k[0, :, H - 1] = 0                                           # an all-zero head
    v[B - 1, :, 0] = synth.f32_to_bf16_bits(ref.bf16_bits_to_f64(v[B - 1, :, 0]).astype(np.float32) * 300)
    q8, k8, v8, amax = lsd.cast_qkv_fp8(to_dev(q), to_dev(k), to_dev(v))
    t.cuda.synchronize()
    eq8, ek8, ev8, eamax = fp8.cast_qkv(q, k, v)
    assert np.array_equal(amax.cpu().numpy(), eamax), "amax"
    assert np.array_equal(codes(q8), eq8), "q codes"
    assert np.array_equal(codes(k8), ek8), "k codes"
    assert np.array_equal(codes(v8), ev8), "v codes (transposed storage)"
    # the transposed rows are zero-padded up to a multiple of 64 tokens
    store = v8.as_strided((B, H, 128, (S + 63) // 64 * 64), (v8.stride(0), v8.stride(2), v8.stride(3), 1))
    pad = codes(store)[..., S:]
    assert pad.size == 0 or np.all(pad == 0), "v padding"


def test_cast_from_fused_strided_views():
    note("fp8 cast from a fused [B,S,3,H,D] buffer")
    t = torch()
    fused = synth.normal_bf16((2, 150, 3, 4, 128), 103, 1)
    f = to_dev(fused)
    q8, k8, v8, amax = lsd.cast_qkv_fp8(f[:, :, 0], f[:, :, 1], f[:, :, 2])
    t.cuda.synchronize()
    eq8, ek8, ev8, eamax = fp8.cast_qkv(fused[:, :, 0], fused[:, :, 1], fused[:, :, 2])
    assert np.array_equal(amax.cpu().numpy(), eamax)
    assert np.array_equal(codes(q8), eq8) and np.array_equal(codes(k8), ek8) and np.array_equal(codes(v8), ev8)


@pytest.mark.parametrize("S_q,S_kv", [(300, 333), (256, 64), (200, 1), (70, 640), (512, 257)])
def test_attention_within_fp8_contract(S_q, S_kv):
    note(f"fp8 attention S_q={S_q} S_kv={S_kv}")
    t = torch()
    B, H = 2, 3
    q = synth.normal_bf16((B, S_q, H, 128), 104, 1)
    k = synth.normal_bf16((B, S_kv, H, 128), 105, 1)
    v = synth.normal_bf16((B, S_kv, H, 128), 106, 1)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    q8, _, _, aq = lsd.cast_qkv_fp8(dq, dq, dq)
    _, k8, v8, akv = lsd.cast_qkv_fp8(dk, dk, dv)
    o, lse = lsd.attn_fwd_fp8(q8, k8, v8, aq[0], akv[1], akv[2])
    t.cuda.synchronize()
    amax = np.stack([aq[0].cpu().numpy(), akv[1].cpu().numpy(), akv[2].cpu().numpy()])
    check_fp8(o, lse, codes(q8), codes(k8), codes(v8), amax, range(H), all_rows(S_q), f"fp8 {S_q}x{S_kv}")
    # for context only: distance to bf16 attention of the unquantised inputs
    O, _ = ref.attention(q, k, v)
    d = np.abs(to_f64(o) - O)
    note(f"  vs unquantised inputs: max-abs {d.max():.3e} mean-abs {d.mean():.3e}")


@pytest.mark.parametrize("std,scale", [(4.0, None), (15.0, None), (15.0, 0.05)])
def test_logit_factor_paths(std, scale):
    """The default cast makes the logit factor a power of two: weights come
    from exp2 of the score while the row max stays within +-100 log2 units
    (std 4), from exp2(s - m) beyond that (std 15: row maxima of several
    hundred); a custom softmax scale makes the factor arbitrary (the other
    path).  All against the oracle within the FP8 contract, except that the
    LSE bar grows with the logits: the matrix cores sum each logit's 128 FP8
    products in float32, about 2e-5 relative measured (LSE off by 1.6e-3 at
    LSE 70, the same on either path), so the bar is 1e-3 + 2^-14 max|logit|."""
    note(f"fp8 attention: inputs with std {std}, softmax scale {scale}")
    t = torch()
    B, S, H = 1, 1000, 2
    q = synth.f32_to_bf16_bits(synth.normal_f32((B, S, H, 128), 107, 1) * np.float32(std))
    k = synth.f32_to_bf16_bits(synth.normal_f32((B, S, H, 128), 108, 1) * np.float32(std))
    v = synth.normal_bf16((B, S, H, 128), 109, 1)
    q8, k8, v8, amax = lsd.cast_qkv_fp8(to_dev(q), to_dev(k), to_dev(v))
    o, lse = lsd.attn_fwd_fp8(q8, k8, v8, amax[0], amax[1], amax[2], scale=scale)
    t.cuda.synchronize()
    a = amax.cpu().numpy()
    hq, hk = codes(q8), codes(k8)
    if scale is None:  # the factor the cast aimed at is a power of two
        c = (np.log2(np.e) / np.sqrt(128.0)) * (a[0].astype(np.float64) / 448) * (a[1].astype(np.float64) / 448)
        assert np.all(np.abs(np.log2(c) - np.round(np.log2(c))) < 1e-6)
    s_max = max(float(np.abs((deq_rows(hq, a[0], 0, h) @ deq_rows(hk, a[1], 0, h).T)).max()) for h in range(H))
    s_max *= ref._default_scale(128, scale)
    note(f"  largest |logit| {s_max / np.log(2):.1f} log2 units")
    check_fp8(o, lse, hq, hk, codes(v8), a, range(H), lambda b, h: np.arange(0, S, 3), f"fp8 std {std} scale {scale}",
              scale=scale, lse_tol=1e-3 + 2.0 ** -14 * s_max)


def test_outlier_keys_empty_block_and_ring_slice():
    note("fp8 attention: outlier keys, S_kv = 0, 64-aligned key block of the padded V rows")
    t = torch()
    q, k, v, _ = synth.cosmos_qkv(seed=4, S=2000, H=2, D=128)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    q8, k8, v8, amax = lsd.cast_qkv_fp8(dq, dk, dv)
    o, lse = lsd.attn_fwd_fp8(q8, k8, v8, amax[0], amax[1], amax[2])
    t.cuda.synchronize()
    a = amax.cpu().numpy()
    hq, hk, hv = codes(q8), codes(k8), codes(v8)
    check_fp8(o, lse, hq, hk, hv, a, range(2), all_rows(2000), "fp8 outliers")
    # a key block [640, 1400) of the same FP8 tensors, as a Ring step would use
    o2, l2 = lsd.attn_fwd_fp8(q8, k8[:, 640:1400], v8[:, 640:1400], amax[0], amax[1], amax[2])
    t.cuda.synchronize()
    check_fp8(o2, l2, hq, hk[:, 640:1400], hv[:, 640:1400], a, range(2), all_rows(2000), "fp8 key block")
    o3, l3 = lsd.attn_fwd_fp8(q8, k8[:, :0], v8[:, :0], amax[0], amax[1], amax[2])
    t.cuda.synchronize()
    assert (o3.float() == 0).all() and t.isneginf(l3).all()
    # determinism
    o4, l4 = lsd.attn_fwd_fp8(q8, k8, v8, amax[0], amax[1], amax[2])
    t.cuda.synchronize()
    assert t.equal(o4.view(t.int16), o.view(t.int16)) and t.equal(l4, lse)


@pytest.mark.parametrize("lo,n", [(0, 127), (0, 128), (0, 129), (0, 192), (0, 193), (64, 129), (64, 200)])
def test_key_counts_around_tile_halves_with_poisoned_padding(lo, n):
    """Key blocks [lo, lo + n) of cast tensors whose codes past the readable
    end are NaN: K rows past the block's last key, and V^T bytes past lo + n
    rounded up to 64 tokens (all that the ABI asks to be readable).  Key
    counts just under, at and over a 128-key tile and its 64-key halves; the
    output must stay finite and within the FP8 contract."""
    note(f"fp8 attention: key block [{lo}, {lo + n}) with NaN codes past the readable end")
    t = torch()
    B, S_q, H, S = 1, 100, 2, 512
    q = synth.normal_bf16((B, S_q, H, 128), 110, 1)
    kv = synth.normal_bf16((B, S, H, 128), 111, 1)
    vv = synth.normal_bf16((B, S, H, 128), 112, 1)
    q8, _, _, aq = lsd.cast_qkv_fp8(to_dev(q), to_dev(q), to_dev(q))
    _, k8, v8, akv = lsd.cast_qkv_fp8(to_dev(kv), to_dev(kv), to_dev(vv))
    t.cuda.synchronize()
    hk, hv = codes(k8)[:, lo:lo + n], codes(v8)[:, lo:lo + n]
    k8.view(t.uint8)[:, lo + n:] = 0x7F                            # E4M3 NaN
    vt = v8.permute(0, 2, 3, 1)                                     # storage [B, H, D, S]
    vt.view(t.uint8)[..., lo + (n + 63) // 64 * 64:] = 0x7F
    o, lse = lsd.attn_fwd_fp8(q8, k8[:, lo:lo + n], v8[:, lo:lo + n], aq[0], akv[1], akv[2])
    t.cuda.synchronize()
    assert t.isfinite(o.float()).all() and t.isfinite(lse).all()
    amax = np.stack([aq[0].cpu().numpy(), akv[1].cpu().numpy(), akv[2].cpu().numpy()])
    check_fp8(o, lse, codes(q8), hk, hv, amax, range(H), all_rows(S_q), f"fp8 keys [{lo}, {lo + n})")


# ------------------------------------------------ key-length mask (FP8 path)

NAN_BF16 = np.uint16(0x7FC1)
MASK_LENS = [300, 1, 0, 127, 128, 129, 257, 64, 350, -3]   # the last two are clamped to 300 and 0


def _lens_dev(lens):
    t = torch()
    return t.tensor(lens, dtype=t.int32, device="cuda")


def _poisoned_qkv(lens, S, H, seed):
    """Q, K, V [B, S, H, 128] whose K and V tokens from lens[b] on are NaN."""
    B = len(lens)
    q = synth.normal_bf16((B, S, H, 128), seed, 1)
    k = synth.normal_bf16((B, S, H, 128), seed + 1, 1).copy()
    v = synth.normal_bf16((B, S, H, 128), seed + 2, 1).copy()
    for b, n in enumerate(lens):
        k[b, max(0, min(n, S)):] = NAN_BF16
        v[b, max(0, min(n, S)):] = NAN_BF16
    return q, k, v


@pytest.mark.parametrize("layout", ["contiguous", "fused"])
def test_masked_cast_bit_exact(layout):
    """lsd_cast_qkv_fp8_masked: amax and the codes of Q (all tokens), K and V
    (valid tokens) bit-exact against the oracle; V's codes of the padding up
    to the padded row end zero; K's codes of the padding left as they were.
    NaN in the padding; lengths across the 64-token chunks of the passes,
    zero and out of range.  The contiguous layout takes the flat passes, the
    fused [B, S, 3, H, D] views the per-head passes."""
    note(f"fp8 masked cast ({layout})")
    t = torch()
    S, H = 300, 3
    q, k, v = _poisoned_qkv(MASK_LENS, S, H, 120)
    B = len(MASK_LENS)
    if layout == "fused":
        f = to_dev(np.stack([q, k, v], axis=2))
        dq, dk, dv = f[:, :, 0], f[:, :, 1], f[:, :, 2]
    else:
        dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    out = lsd.fp8_buffers(B, S, H)
    out[1].view(t.uint8).fill_(0x5A)                               # K padding must keep this
    q8, k8, v8, amax = lsd.cast_qkv_fp8(dq, dk, dv, out=out, kv_lens=_lens_dev(MASK_LENS))
    t.cuda.synchronize()
    eq8, ek8, ev8, eamax = fp8.cast_qkv(q, k, v, kv_lens=MASK_LENS)
    assert np.array_equal(amax.cpu().numpy(), eamax), "amax"
    assert np.array_equal(codes(q8), eq8), "q codes"
    gk, gv = codes(k8), codes(v8)
    for b, n in enumerate(MASK_LENS):
        n = max(0, min(n, S))
        assert np.array_equal(gk[b, :n], ek8[b, :n]), f"k codes b={b}"
        assert np.all(gk[b, n:] == 0x5A), f"k padding written b={b}"
    assert np.array_equal(gv, ev8), "v codes (padding zero)"
    store = v8.as_strided((B, H, 128, (S + 63) // 64 * 64), (v8.stride(0), v8.stride(2), v8.stride(3), 1))
    assert np.all(codes(store)[..., S:] == 0), "v row padding"


@pytest.mark.parametrize("S,H", [(300, 2), (640, 2)])
def test_masked_attention_within_fp8_contract(S, H):
    """lsd_attn_fwd_fp8_masked on the masked cast of a padded batch: every
    entry within the FP8 contract against the oracle's attention of its valid
    keys (an entry without keys: O = 0, LSE = -inf); the output stays finite
    although the K codes past the valid keys are NaN; with every length at
    S_kv it is bit-identical to lsd_attn_fwd_fp8."""
    note(f"fp8 masked attention S={S} H={H}")
    t = torch()
    lens = [S, 1, 0, 127, 128, 129, 257, 64, S + 50, -3]
    q, k, v = _poisoned_qkv(lens, S, H, 130)
    ld = _lens_dev(lens)
    q8, k8, v8, amax = lsd.cast_qkv_fp8(to_dev(q), to_dev(k), to_dev(v), kv_lens=ld)
    for b, n in enumerate(lens):
        k8.view(t.uint8)[b, max(0, min(n, S)):] = 0x7F                            # E4M3 NaN past the valid keys
    o, lse = lsd.attn_fwd_fp8(q8, k8, v8, amax[0], amax[1], amax[2], kv_lens=ld)
    t.cuda.synchronize()
    assert t.isfinite(o.float()).all()
    cq, ck, cv, am = codes(q8), codes(k8), codes(v8), amax.cpu().numpy()
    for b, n in enumerate(lens):
        n = max(0, min(n, S))
        check_fp8(o[b:b + 1], lse[b:b + 1], cq[b:b + 1], ck[b:b + 1, :n], cv[b:b + 1, :n], am[:, b:b + 1],
                  range(H), all_rows(S), f"fp8 masked b={b} len={n}")
    full = _lens_dev([S] * len(lens))
    qa, ka, va = (to_dev(synth.normal_bf16((len(lens), S, H, 128), 140 + i, 1)) for i in range(3))
    q8a, k8a, v8a, ama = lsd.cast_qkv_fp8(qa, ka, va)
    o1, l1 = lsd.attn_fwd_fp8(q8a, k8a, v8a, ama[0], ama[1], ama[2])
    o2, l2 = lsd.attn_fwd_fp8(q8a, k8a, v8a, ama[0], ama[1], ama[2], kv_lens=full)
    t.cuda.synchronize()
    assert t.equal(o1.view(t.int16), o2.view(t.int16)) and t.equal(l1, l2)


# ------------------------------------------------ fused Ring step (FP8 path)

@pytest.mark.parametrize("layout,masked", [("contiguous", False), ("contiguous", True), ("fused", True)])
def test_kv_cast_bit_exact(layout, masked):
    """lsd_cast_kv_fp8: K's scale amax chosen against a given Q scale, codes
    and all three amax slots bit-exact against the oracle; the q8 buffer of
    ``out`` untouched; with the key-length mask the padding as in the masked
    cast (NaN there, V codes zero, K codes not written)."""
    note(f"fp8 K/V-only cast ({layout}, masked={masked})")
    t = torch()
    S, H = 300, 3
    lens = MASK_LENS if masked else [S] * len(MASK_LENS)
    q, k, v = _poisoned_qkv(lens, S, H, 190)
    B = len(lens)
    dq = to_dev(q)
    _, _, _, aq = lsd.cast_qkv_fp8(dq, dq, dq)
    if layout == "fused":
        f = to_dev(np.stack([k, v, v], axis=2))
        dk, dv = f[:, :, 0], f[:, :, 1]
    else:
        dk, dv = to_dev(k), to_dev(v)
    out = lsd.fp8_buffers(B, S, H)
    out[0].view(t.uint8).fill_(0x33)
    out[1].view(t.uint8).fill_(0x5A)
    k8, v8, amax = lsd.cast_kv_fp8(dk, dv, aq[0], out=out, kv_lens=_lens_dev(lens) if masked else None)
    t.cuda.synchronize()
    ek8, ev8, eamax = fp8.cast_kv(k, v, aq[0].cpu().numpy(), kv_lens=lens if masked else None)
    assert np.array_equal(amax.cpu().numpy(), eamax), "amax"
    assert np.all(codes(out[0]) == 0x33), "q8 written"
    gk = codes(k8)
    for b, n in enumerate(lens):
        n = max(0, min(n, S))
        assert np.array_equal(gk[b, :n], ek8[b, :n]), f"k codes b={b}"
        assert np.all(gk[b, n:] == 0x5A), f"k padding written b={b}"
    assert np.array_equal(codes(v8), ev8), "v codes"


@pytest.mark.parametrize("kv_cast", [False, True])
def test_fp8_ring_steps_within_contract(kv_cast):
    """lsd_attn_fwd_fp8_accumulate over four K/V blocks (each cast with its
    own scales; one with a key-length mask, one whose every entry is empty),
    each step checked from the GPU's own prior state: the merged O within the
    FP8 bound of the block's result weighted by the block's share
    w_b / (w_acc + w_b) (plus float32 merge rounding), the LSE within 1e-3,
    an empty block leaving the running result bit-identical, and the bf16
    output the running O rounded."""
    note(f"fp8 fused Ring steps (blocks cast against the Q scale: {kv_cast})")
    t = torch()
    B, S_q, H = 2, 200, 2
    sc = ref._default_scale(128, None)
    q = synth.normal_bf16((B, S_q, H, 128), 150, 1)
    dq = to_dev(q)
    q8, _, _, aq = lsd.cast_qkv_fp8(dq, dq, dq)
    cq, am_q = codes(q8), aq[0].cpu().numpy()
    o_acc = t.zeros((B, S_q, H, 128), dtype=t.float32, device="cuda")
    lse_acc = t.full((B, H, S_q), float("-inf"), dtype=t.float32, device="cuda")
    o = t.empty((B, S_q, H, 128), dtype=t.bfloat16, device="cuda")
    steps = [(150, None), (77, [77, 30]), (300, None), (64, [0, 0])]
    for i, (n, lens) in enumerate(steps):
        k = synth.normal_bf16((B, n, H, 128), 160 + i, 1)
        v = synth.normal_bf16((B, n, H, 128), 170 + i, 1)
        ld = None if lens is None else _lens_dev(lens)
        if kv_cast:  # each block's K scale chosen against Q's: the power-of-two path
            k8, v8, akv = lsd.cast_kv_fp8(to_dev(k), to_dev(v), aq[0], kv_lens=ld)
        else:
            _, k8, v8, akv = lsd.cast_qkv_fp8(to_dev(k), to_dev(k), to_dev(v), kv_lens=ld)
        prev_o, prev_l = o_acc.cpu().numpy().astype(np.float64), lse_acc.cpu().numpy().astype(np.float64)
        lsd.attn_fwd_fp8_accumulate(q8, k8, v8, aq[0], akv[1], akv[2], o_acc, lse_acc, o=o, kv_lens=ld)
        t.cuda.synchronize()
        new_o, new_l = o_acc.cpu().numpy().astype(np.float64), lse_acc.cpu().numpy().astype(np.float64)
        ck, cv, ak, av = codes(k8), codes(v8), akv[1].cpu().numpy(), akv[2].cpu().numpy()
        for b in range(B):
            nb = n if lens is None else max(0, min(lens[b], n))
            for h in range(H):
                what = f"step {i} b={b} h={h}"
                if nb == 0:
                    assert np.array_equal(new_o[b, :, h], prev_o[b, :, h]) and np.array_equal(new_l[b, h], prev_l[b, h]), what
                    continue
                qh = deq_rows(cq, am_q, b, h)
                kh = deq_rows(ck, ak, b, h)[:nb]
                vh = deq_rows(cv, av, b, h)[:nb]
                O_b, L_b = ref._attend_block(qh, kh, vh, sc)
                s = (qh @ kh.T) * sc
                p = np.exp(s - s.max(axis=1, keepdims=True))
                l = p.sum(axis=1, keepdims=True)
                bound_b = 2.0 ** -4 * (p @ np.abs(vh)) / l + 2.0 ** -10 * np.abs(vh).sum(axis=0)[None, :] / l
                La = prev_l[b, h]
                M = np.maximum(La, L_b)
                with np.errstate(invalid="ignore"):
                    wa = np.where(np.isneginf(La), 0.0, np.exp(La - M))
                wb = np.exp(L_b - M)
                Oa = np.where(np.isneginf(La)[:, None], 0.0, prev_o[b, :, h])
                O_ref = (wa[:, None] * Oa + wb[:, None] * O_b) / (wa + wb)[:, None]
                L_ref = M + np.log(wa + wb)
                beta = (wb / (wa + wb))[:, None]
                err = np.abs(new_o[b, :, h] - O_ref)
                assert np.all(err <= beta * bound_b + 2.0 ** -8 * np.abs(O_ref) + 1e-5), \
                    f"{what}: O outside the bound (ratio {float((err / (beta * bound_b + 2.0 ** -8 * np.abs(O_ref) + 1e-5)).max()):.3f})"
                assert np.abs(new_l[b, h] - L_ref).max() <= 1e-3, f"{what}: LSE"
        ob = o.float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(ob - new_o) <= 2.0 ** -8 * np.abs(new_o) + 1e-30), f"step {i}: bf16 output"
