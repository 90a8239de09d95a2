"""attn_fwd on the GPU (through the C ABI) against the float64 oracle.

Small shapes spanning several 256-row query tiles and 64-key tiles with
ragged tails, compared element by element; closed forms; strided fused-QKV
views; output guard bands; bitwise determinism."""

import math

import numpy as np
import pytest

import synth
from oracle import ref
from gpu_util import (assert_attention_close, note, to_bits, to_dev, to_f64, torch)

pytestmark = pytest.mark.gpu

lsd = pytest.importorskip("long_sequence_dit_amd")


def run(q, k, v, scale=None):
    t = torch()
    o, lse = lsd.attn_fwd(to_dev(q), to_dev(k), to_dev(v), scale=scale)
    t.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy().astype(np.float64)


def test_tiny_full_parity():
    note("attn tiny: B=1 S=256 H=2 D=64 seed 0")
    q, k, v = synth.tiny_qkv()
    o, lse = run(q, k, v)
    O, L = ref.attention(q, k, v)
    assert_attention_close(o, O, lse, L, "tiny")


SHAPES = [  # (S_q, S_kv, D)
    (1, 1, 64), (17, 63, 128), (64, 64, 64), (65, 127, 128), (129, 255, 64),
    (257, 1000, 128), (1000, 257, 64), (255, 65, 128), (300, 1, 128), (513, 700, 128),
    (600, 129, 64), (256, 4096, 128),
]


@pytest.mark.parametrize("S_q,S_kv,D", SHAPES)
def test_ragged_shapes(S_q, S_kv, D):
    note(f"attn ragged: B=2 H=3 S_q={S_q} S_kv={S_kv} D={D}")
    q, k, v = synth.qkv(2, S_q, S_kv, 3, D, seed=1000 + S_q + 7 * S_kv + D)
    o, lse = run(q, k, v)
    O, L = ref.attention(q, k, v)
    assert_attention_close(o, O, lse, L, f"S_q={S_q} S_kv={S_kv} D={D}")


def test_strided_fused_qkv_views():
    note("attn strided: fused QKV [2,300,3,4,128] views")
    t = torch()
    B, S, H, D = 2, 300, 4, 128
    fused = synth.fused_qkv(B, S, H, D, seed=7)
    f = to_dev(fused)
    q, k, v = f[:, :, 0], f[:, :, 1], f[:, :, 2]
    assert not q.is_contiguous() and q.stride() == (S * 3 * H * D, 3 * H * D, D, 1)
    o, lse = lsd.attn_fwd(q, k, v)
    t.cuda.synchronize()
    O, L = ref.attention(fused[:, :, 0], fused[:, :, 1], fused[:, :, 2])
    assert_attention_close(to_f64(o), O, lse.cpu().numpy(), L, "fused views")
    # a strided output view is written in place and only there
    big = t.full((B, S, 2 * H, D), float("nan"), dtype=t.bfloat16, device="cuda")
    ov = big[:, :, 1::2]
    lsd.attn_fwd(q, k, v, o=ov, return_lse=False)
    t.cuda.synchronize()
    assert_attention_close(to_f64(ov), O, what="strided o")
    assert t.isnan(big[:, :, 0::2].float()).all()


def test_explicit_scale():
    note("attn explicit scale 0.3")
    q, k, v = synth.qkv(1, 200, 333, 2, 128, seed=11)
    o, lse = run(q, k, v, scale=0.3)
    O, L = ref.attention(q, k, v, scale=0.3)
    assert_attention_close(o, O, lse, L, "scale 0.3")


def test_identical_keys_closed_form():
    note("attn identical keys")
    B, Sq, Skv, H, D = 1, 300, 517, 2, 128
    q = synth.normal_bf16((B, Sq, H, D), 12, 1)
    krow = synth.normal_bf16((B, 1, H, D), 12, 2)
    k = np.repeat(krow, Skv, axis=1)
    v = synth.normal_bf16((B, Skv, H, D), 12, 3)
    o, lse = run(q, k, v)
    vm = ref.bf16_bits_to_f64(v).mean(axis=1)
    exp_o = np.broadcast_to(vm[:, None], o.shape)
    qk = np.sum(ref.bf16_bits_to_f64(q) * ref.bf16_bits_to_f64(krow), axis=3) / math.sqrt(D)
    exp_l = np.transpose(qk + math.log(Skv), (0, 2, 1))
    assert_attention_close(o, exp_o, lse, exp_l, "identical keys")


def test_dominant_logit_is_one_hot_bit_exact():
    note("attn dominant logit")
    S, D, H = 1000, 128, 2
    two = synth.f32_to_bf16_bits(np.array([2.0], np.float32))[0]
    q = np.full((1, 300, H, D), two, dtype=np.uint16)
    k = np.zeros((1, S, H, D), dtype=np.uint16)
    js = [777, 3]
    for h in range(H):
        k[0, js[h], h] = two
    v = synth.normal_bf16((1, S, H, D), 13, 3)
    t = torch()
    o, lse = lsd.attn_fwd(to_dev(q), to_dev(k), to_dev(v))
    t.cuda.synchronize()
    ob = to_bits(o)
    for h in range(H):
        assert np.array_equal(ob[0, :, h], np.broadcast_to(v[0, js[h], h], (300, D)))
    s_star = 4.0 * math.sqrt(D)
    assert np.abs(lse.cpu().numpy() - s_star).max() <= 1e-3


def test_constant_values_give_constant_output():
    note("attn V = 1")
    q, k, _ = synth.qkv(1, 400, 900, 2, 128, seed=14)
    ones = np.full(k.shape, 0x3F80, dtype=np.uint16)
    o, _ = run(q, k, ones)
    # every weight sums to one: within one bf16 ulp of 1
    assert np.abs(o - 1.0).max() <= 2.0 ** -8


def test_no_keys():
    note("attn S_kv = 0")
    t = torch()
    q = to_dev(synth.normal_bf16((1, 70, 2, 64), 15, 1))
    k = t.empty((1, 0, 2, 64), dtype=t.bfloat16, device="cuda")
    o, lse = lsd.attn_fwd(q, k, k)
    t.cuda.synchronize()
    assert (o.float() == 0).all() and t.isneginf(lse).all()


def test_guard_bands_and_determinism():
    note("attn guard bands + determinism: S_q=333 S_kv=555 D=128")
    t = torch()
    B, Sq, Skv, H, D = 2, 333, 555, 3, 128
    q, k, v = synth.qkv(B, Sq, Skv, H, D, seed=16)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    outs = []
    for _ in range(2):
        big = t.full((B, Sq + 8, H, D), float("nan"), dtype=t.bfloat16, device="cuda")
        o = big[:, 4:4 + Sq]
        lse_big = t.full((B * H * Sq + 64,), float("nan"), dtype=t.float32, device="cuda")
        lse = lse_big[32:32 + B * H * Sq].view(B, H, Sq)
        lsd.attn_fwd(dq, dk, dv, o=o, lse=lse)
        t.cuda.synchronize()
        assert t.isnan(big[:, :4].float()).all() and t.isnan(big[:, 4 + Sq:].float()).all()
        assert t.isnan(lse_big[:32]).all() and t.isnan(lse_big[32 + B * H * Sq:]).all()
        assert not t.isnan(o.float()).any() and not t.isnan(lse).any()
        outs.append((to_bits(o), lse.cpu().numpy().copy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    O, L = ref.attention(q, k, v)
    assert_attention_close(ref.bf16_bits_to_f64(outs[0][0]), O, outs[0][1], L, "guarded")
