"""Attention with V given token-contiguous (each channel's keys one row, the
layout staged straight from HBM into LDS), through the C ABI.  Both V layouts
run the same arithmetic in the same order, so the token-contiguous path must
match the natural-layout path bit for bit; one case per mode is also checked
against the oracle.  Row padding and masked keys hold NaN bit patterns, so a
read of any of them would poison the output."""

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


@pytest.mark.parametrize("B,S_q,S_kv,H,D", CASES)
def test_token_major_v_matches_natural(B, S_q, S_kv, H, D):
    note(f"token-major V: B={B} S_q={S_q} S_kv={S_kv} H={H} D={D}")
    t = torch()
    seed = 1000 + S_kv + D
    q = to_dev(synth.normal_bf16((B, S_q, H, D), seed, 1))
    k = to_dev(synth.normal_bf16((B, S_kv, H, D), seed + 1, 1))
    v = to_dev(synth.normal_bf16((B, S_kv, H, D), seed + 2, 1))
    o1, l1 = lsd.attn_fwd(q, k, v)
    for pitch in (None, (S_kv + 7) // 8 * 8 + 64):
        vt = token_major(v, pitch)
        o2, l2 = lsd.attn_fwd(q, k, vt)
        t.cuda.synchronize()
        assert np.array_equal(to_bits(o1), to_bits(o2)), f"O differs (pitch {pitch})"
        assert t.equal(l1, l2), f"LSE differs (pitch {pitch})"


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
    q = to_dev(synth.normal_bf16((B, S_q, H, D), 1301, 1))
    kn = synth.normal_bf16((B, S_kv, H, D), 1302, 1)
    for b, n in enumerate(lens):
        kn[b, n:] = NAN_BITS
    k = to_dev(kn)
    v = to_dev(synth.normal_bf16((B, S_kv, H, D), 1303, 1))
    ld = lens_dev(lens)
    o1, l1 = lsd.attn_fwd(q, k, v, kv_lens=ld)
    o2, l2 = lsd.attn_fwd(q, k, token_major(v, lens=lens), kv_lens=ld)
    t.cuda.synchronize()
    assert np.array_equal(to_bits(o1), to_bits(o2)) and t.equal(l1, l2)
    assert np.all(np.isfinite(to_f64(o2)))


@pytest.mark.parametrize("D", [64, 128])
def test_token_major_v_accumulate(D):
    note(f"token-major V in the fused Ring step D={D}")
    t = torch()
    B, S_q, H = 1, 200, 2
    q = to_dev(synth.normal_bf16((B, S_q, H, D), 1401, 1))
    blocks = [(to_dev(synth.normal_bf16((B, n, H, D), 1410 + n, 1)),
               to_dev(synth.normal_bf16((B, n, H, D), 1420 + n, 1))) for n in (150, 77, 300)]
    res = []
    for tok in (False, True):
        oa = t.zeros((B, S_q, H, D), dtype=t.float32, device="cuda")
        la = t.full((B, H, S_q), float("-inf"), dtype=t.float32, device="cuda")
        o = t.empty((B, S_q, H, D), dtype=t.bfloat16, device="cuda")
        for k, v in blocks:
            lsd.attn_fwd_accumulate(q, k, token_major(v) if tok else v, oa, la, o=o)
        t.cuda.synchronize()
        res.append((oa.clone(), la.clone(), to_bits(o)))
    assert t.equal(res[0][0], res[1][0]) and t.equal(res[0][1], res[1][1])
    assert np.array_equal(res[0][2], res[1][2])
