"""Seeded sweep of valid attention inputs against the oracle: batch, query and
key lengths around tile boundaries (64 keys, 256 query rows, 8-key chunks),
head counts, D in {64, 128}, V natural or token-contiguous (with padded row
pitches holding NaN), per-batch key lengths, explicit scales, and the fused
Ring step.  Deterministic: the same cases every run."""

import numpy as np
import pytest

import synth
from oracle import ref
from gpu_util import assert_attention_close, note, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

lsd = pytest.importorskip("long_sequence_dit_amd")

NAN_BITS = 0x7FC1


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    near = lambda m: int(max(1, m + rng.integers(-3, 4)))
    out = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        S_q = near(int(rng.choice([1, 64, 256, 300, 513])))
        S_kv = near(int(rng.choice([8, 64, 128, 200, 449])))
        tok = bool(rng.integers(0, 2))
        masked = bool(rng.integers(0, 2))
        lens = [int(rng.integers(0, S_kv + 2)) for _ in range(B)] if masked else None
        scale = float(rng.choice([0.0, 0.05, 0.3]))
        out.append((i, B, S_q, S_kv, H, D, tok, lens, scale))
    return out


CASES = _cases(24, 20241)


def _token_major(v_dev, extra):
    t = torch()
    B, S, H, D = v_dev.shape
    pitch = (S + 7) // 8 * 8 + extra
    vt = lsd.v_token_major(B, S, H, D, pitch=pitch)
    store = t.as_strided(vt, (B, H, D, vt.stride(3)), (vt.stride(0), vt.stride(2), vt.stride(3), 1))
    store.view(t.int16).fill_(NAN_BITS)
    vt.copy_(v_dev)
    return vt


@pytest.mark.parametrize("i,B,S_q,S_kv,H,D,tok,lens,scale", CASES)
def test_random_case(i, B, S_q, S_kv, H, D, tok, lens, scale):
    note(f"random case {i}: B={B} S_q={S_q} S_kv={S_kv} H={H} D={D} tok={tok} lens={lens} scale={scale}")
    t = torch()
    seed = 7000 + 10 * i
    qh = synth.normal_bf16((B, S_q, H, D), seed, 1)
    kh = synth.normal_bf16((B, S_kv, H, D), seed + 1, 1)
    vh = synth.normal_bf16((B, S_kv, H, D), seed + 2, 1)
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    if tok:
        v = _token_major(v, 8 * (i % 3))
    lsd_lens = None
    if lens is not None:
        lsd_lens = t.tensor(lens, dtype=t.int32, device="cuda")
    sc = None if scale == 0.0 else scale
    o, lse = lsd.attn_fwd(q, k, v, scale=sc, kv_lens=lsd_lens)
    t.cuda.synchronize()
    O, L = ref.attention(qh, kh, vh, scale=sc, kv_lens=lens)
    assert_attention_close(to_f64(o), O, lse.cpu().numpy(), L, f"case {i}")
    # the fused Ring step over the same keys split in two blocks gives the same result
    if lens is None and S_kv >= 2:
        cut = S_kv // 3
        oa = t.zeros((B, S_q, H, D), dtype=t.float32, device="cuda")
        la = t.full((B, H, S_q), float("-inf"), dtype=t.float32, device="cuda")
        o2 = t.empty((B, S_q, H, D), dtype=t.bfloat16, device="cuda")
        for lo, hi in ((0, cut), (cut, S_kv)):
            kb = to_dev(kh[:, lo:hi])
            vb = to_dev(vh[:, lo:hi])
            if tok:
                vb = _token_major(vb, 8)
            lsd.attn_fwd_accumulate(q, kb, vb, oa, la, o=o2, scale=sc)
        t.cuda.synchronize()
        assert_attention_close(to_f64(o2), O, la.cpu().numpy(), L, f"case {i}, two Ring steps")


# A second sweep whose token-contiguous V pitches straddle 64 keys: the kernel
# pairs a thread's two V^T loads per tile only when the pitch is at least 64,
# so both variants run, with padding up to 120 keys past the rounded length.
PITCH_CASES = [(c, int(e)) for c, e in
               zip(_cases(40, 77731), np.random.default_rng(77732).choice([0, 8, 56, 64, 120], 40))]


@pytest.mark.parametrize("case,extra", PITCH_CASES)
def test_random_case_pitches(case, extra):
    i, B, S_q, S_kv, H, D, _, lens, scale = case
    note(f"pitch case {i}: B={B} S_q={S_q} S_kv={S_kv} H={H} D={D} extra={extra} lens={lens} scale={scale}")
    t = torch()
    seed = 8000 + 10 * i
    qh = synth.normal_bf16((B, S_q, H, D), seed, 1)
    kh = synth.normal_bf16((B, S_kv, H, D), seed + 1, 1)
    vh = synth.normal_bf16((B, S_kv, H, D), seed + 2, 1)
    q, k = to_dev(qh), to_dev(kh)
    v = _token_major(to_dev(vh), extra)
    lsd_lens = t.tensor(lens, dtype=t.int32, device="cuda") if lens is not None else None
    sc = None if scale == 0.0 else scale
    o, lse = lsd.attn_fwd(q, k, v, scale=sc, kv_lens=lsd_lens)
    t.cuda.synchronize()
    O, L = ref.attention(qh, kh, vh, scale=sc, kv_lens=lens)
    assert_attention_close(to_f64(o), O, lse.cpu().numpy(), L, f"pitch case {i}")
