"""Attention with V given token-contiguous (each channel's keys one row, the
layout staged straight from HBM into LDS), through the C ABI.  That kernel
assigns keys to the MFMA reduction slots in another order than the kernel for
the natural layout, so the two agree to within one bf16 rounding step (fp32
partial sums round differently), and each is checked against the oracle.  The
token-contiguous kernel itself is bit-reproducible across row pitches and
padding contents.  Row padding and masked keys hold NaN bit patterns, so a read
of any of them would poison the output."""

import math

import numpy as np
import pytest

import synth
from oracle import ref
from gpu_util import assert_attention_close, note, to_bits, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

lsd = pytest.importorskip("long_sequence_dit_amd")

NAN_BITS = 0x7FC1


def token_major(v_dev, pitch=None, lens=None):
    """Copy a natural-layout V into a token-contiguous buffer whose padding
    (and keys past lens[b], if given) hold NaN."""
    t = torch()
    B, S, H, D = v_dev.shape
    vt = lsd.v_token_major(B, S, H, D, pitch=pitch)
    base = vt.permute(0, 2, 3, 1)  # [B, H, D, S] view of the storage
    storage = t.as_strided(vt, (B, H, D, vt.stride(3)), (vt.stride(0), vt.stride(2), vt.stride(3), 1))
    storage.view(t.int16).fill_(NAN_BITS)
    base.copy_(v_dev.permute(0, 2, 3, 1))
    if lens is not None:
        for b, n in enumerate(lens):
            base[b, :, :, max(0, min(n, S)):].view(t.int16).fill_(NAN_BITS)
    return vt


def lens_dev(lens):
    t = torch()
    return t.tensor(lens, dtype=t.int32, device="cuda")


CASES = [  # (B, S_q, S_kv, H, D)
    (1, 300, 200, 2, 128),
    (2, 256, 1000, 3, 64),
    (1, 77, 67, 2, 128),     # S_kv not a multiple of 8: the straddling chunk
    (1, 64, 1, 1, 128),
    (1, 130, 8, 2, 64),
    (1, 257, 64, 1, 128),
    (2, 100, 4100, 2, 128),  # many tiles, ragged last one
    (1, 512, 199, 2, 64),
]


def assert_layouts_agree(o1, o2, l1=None, l2=None, what=""):
    """Outputs of the two kernels: equal up to one bf16 rounding step."""
    a, b = to_f64(o1), to_f64(o2)
    assert np.all(np.isfinite(b)), f"{what}: non-finite output"
    bound = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6
    bad = np.abs(a - b) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements differ by more than one bf16 step"
    if l1 is not None:
        d = (l1 - l2).abs()
        d = d[~(l1.isneginf() & l2.isneginf())]
        assert d.numel() == 0 or float(d.max()) <= 1e-5, f"{what}: LSE differs by {float(d.max()):.2e}"


@pytest.mark.parametrize("B,S_q,S_kv,H,D", CASES)
def test_token_major_v(B, S_q, S_kv, H, D):
    note(f"token-major V: B={B} S_q={S_q} S_kv={S_kv} H={H} D={D}")
    t = torch()
    seed = 1000 + S_kv + D
    qh = synth.normal_bf16((B, S_q, H, D), seed, 1)
    kh = synth.normal_bf16((B, S_kv, H, D), seed + 1, 1)
    vh = synth.normal_bf16((B, S_kv, H, D), seed + 2, 1)
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    o1, l1 = lsd.attn_fwd(q, k, v)
    outs = []
    for pitch in (None, (S_kv + 7) // 8 * 8 + 64):
        o2, l2 = lsd.attn_fwd(q, k, token_major(v, pitch))
        t.cuda.synchronize()
        outs.append((to_bits(o2), l2.clone()))
        assert_layouts_agree(o1, o2, l1, l2, f"pitch {pitch}")
    assert np.array_equal(outs[0][0], outs[1][0]) and t.equal(outs[0][1], outs[1][1]), "depends on the pitch"
    O, L = ref.attention(qh, kh, vh)
    assert_attention_close(ref.bf16_bits_to_f64(outs[0][0]), O, outs[0][1].cpu().numpy(), L, "token-major")


@pytest.mark.parametrize("D", [64, 128])
def test_token_major_v_against_oracle(D):
    note(f"token-major V vs oracle D={D}")
    t = torch()
    B, S_q, S_kv, H = 1, 300, 333, 2
    q = synth.normal_bf16((B, S_q, H, D), 1201, 1)
    k = synth.normal_bf16((B, S_kv, H, D), 1202, 1)
    v = synth.normal_bf16((B, S_kv, H, D), 1203, 1)
    o, lse = lsd.attn_fwd(to_dev(q), to_dev(k), token_major(to_dev(v)))
    t.cuda.synchronize()
    O, L = ref.attention(q, k, v)
    assert_attention_close(to_f64(o), O, lse.cpu().numpy(), L, f"token-major D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_token_major_v_masked(D):
    note(f"token-major V with key mask D={D}")
    t = torch()
    lens = [300, 1, 63, 64, 65, 129, 0, 257, 7, 250]
    B, S_q, S_kv, H = len(lens), 120, 300, 2
    qh = synth.normal_bf16((B, S_q, H, D), 1301, 1)
    kh = synth.normal_bf16((B, S_kv, H, D), 1302, 1)
    vh = synth.normal_bf16((B, S_kv, H, D), 1303, 1)
    for b, n in enumerate(lens):
        kh[b, n:] = NAN_BITS
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    ld = lens_dev(lens)
    o1, l1 = lsd.attn_fwd(q, k, v, kv_lens=ld)
    o2, l2 = lsd.attn_fwd(q, k, token_major(v, lens=lens), kv_lens=ld)
    t.cuda.synchronize()
    assert_layouts_agree(o1, o2, l1, l2, "masked")
    O, L = ref.attention(qh, kh, vh, kv_lens=lens)
    assert_attention_close(to_f64(o2), O, l2.cpu().numpy(), L, "masked token-major")
    assert (to_f64(o2)[6] == 0).all() and l2[6].isneginf().all()


@pytest.mark.parametrize("D", [64, 128])
def test_token_major_v_accumulate(D):
    note(f"token-major V in the fused Ring step D={D}")
    t = torch()
    B, S_q, H = 1, 200, 2
    qh = synth.normal_bf16((B, S_q, H, D), 1401, 1)
    q = to_dev(qh)
    host = [(synth.normal_bf16((B, n, H, D), 1410 + n, 1), synth.normal_bf16((B, n, H, D), 1420 + n, 1))
            for n in (150, 77, 300)]
    blocks = [(to_dev(kh), to_dev(vh)) for kh, vh in host]
    res = []
    for tok in (False, True):
        oa = t.zeros((B, S_q, H, D), dtype=t.float32, device="cuda")
        la = t.full((B, H, S_q), float("-inf"), dtype=t.float32, device="cuda")
        o = t.empty((B, S_q, H, D), dtype=t.bfloat16, device="cuda")
        for k, v in blocks:
            lsd.attn_fwd_accumulate(q, k, token_major(v) if tok else v, oa, la, o=o)
        t.cuda.synchronize()
        res.append((oa.clone(), la.clone(), o.clone()))
    assert_layouts_agree(res[0][2], res[1][2], res[0][1], res[1][1], "accumulate")
    assert float((res[0][0] - res[1][0]).abs().max()) <= 1e-5 * max(1.0, float(res[0][0].abs().max()))
    K = np.concatenate([kh for kh, _ in host], axis=1)
    V = np.concatenate([vh for _, vh in host], axis=1)
    O, L = ref.attention(qh, K, V)
    assert_attention_close(to_f64(res[1][2]), O, res[1][1].cpu().numpy(), L, "accumulate token-major")


def growing_logit_keys(S_kv, H, D, steps, seed):
    """Q rows all ones; the keys of tile i (64 keys) are a_i plus small noise in
    every channel, with a_i chosen so that the scaled logit (in log2 units)
    moves by steps[i % len(steps)] from one tile to the next.  Increments above
    8 make the kernels take the row max and rescale (the slow path); smaller
    ones keep the weights below 2^8 against the old reference (the fast path)."""
    scale_log2 = math.log2(math.e) / math.sqrt(D)
    per_unit = scale_log2 * D  # logit per unit of a with Q = 1
    rng = np.random.default_rng(seed)
    level, a = 0.0, np.empty(S_kv, np.float32)
    for i in range((S_kv + 63) // 64):
        level += steps[i % len(steps)]
        a[64 * i:64 * (i + 1)] = level / per_unit
    k = a[None, :, None, None] + rng.normal(0.0, 0.02, (1, S_kv, H, D)).astype(np.float32)
    return synth.f32_to_bf16_bits(k.astype(np.float32))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("steps", [(9.0, 2.0, 12.0, 0.5, 7.5), (-3.0, 10.0, -20.0, 8.5)])
def test_rescale_paths_both_layouts(D, steps):
    """Row maxima that jump by more than 2^8 between tiles (row max taken, O
    and l rescaled) alternating with tiles whose weights stay below 2^8 of the
    old reference (max skipped), and falling maxima: both kernels against the
    oracle."""
    note(f"rescale paths D={D} steps={steps}")
    t = torch()
    B, S_q, S_kv, H = 1, 289, 64 * 12 + 17, 2
    one = synth.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    qh = np.full((B, S_q, H, D), one, dtype=np.uint16)
    kh = growing_logit_keys(S_kv, H, D, steps, 1501 + D)
    vh = synth.normal_bf16((B, S_kv, H, D), 1502 + D, 1)
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    o1, l1 = lsd.attn_fwd(q, k, v)
    o2, l2 = lsd.attn_fwd(q, k, token_major(v))
    t.cuda.synchronize()
    O, L = ref.attention(qh, kh, vh)
    assert_attention_close(to_f64(o1), O, l1.cpu().numpy(), L, "natural V")
    assert_attention_close(to_f64(o2), O, l2.cpu().numpy(), L, "token-major V")


def test_token_major_v_dominant_logit_one_hot_bit_exact():
    """One key per head dominates (logit 4 sqrt(D) above the others), late in
    the sequence: the output is that key's V row, bit for bit."""
    note("token-major V dominant logit")
    S, D, H = 1000, 128, 2
    two = synth.f32_to_bf16_bits(np.array([2.0], np.float32))[0]
    q = np.full((1, 300, H, D), two, dtype=np.uint16)
    k = np.zeros((1, S, H, D), dtype=np.uint16)
    js = [777, 3]
    for h in range(H):
        k[0, js[h], h] = two
    v = synth.normal_bf16((1, S, H, D), 13, 3)
    t = torch()
    o, lse = lsd.attn_fwd(to_dev(q), to_dev(k), token_major(to_dev(v)))
    t.cuda.synchronize()
    ob = to_bits(o)
    for h in range(H):
        assert np.array_equal(ob[0, :, h], np.broadcast_to(v[0, js[h], h], (300, D)))
    assert np.abs(lse.cpu().numpy() - 4.0 * math.sqrt(D)).max() <= 1e-3
