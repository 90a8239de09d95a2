"""attn_fwd_accumulate on the GPU (through the C ABI): Ring steps with the LSE
merge folded into the attention epilogue, against the float64 oracle.

Each step is checked against the oracle applied to the GPU's own previous
running state (so errors do not compound in the comparison), and the final
state against full attention over all keys."""

import numpy as np
import pytest

import synth
from oracle import ref
from gpu_util import assert_attention_close, note, to_bits, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

lsd = pytest.importorskip("long_sequence_dit_amd")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    return synth.f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32))


def run_steps(q, k, v, bounds, what, scale=None, start_garbage=True):
    """Accumulate over key blocks; check every step; return the final state."""
    t = torch()
    B, S_q, H, D = q.shape
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    o_acc = t.full((B, S_q, H, D), float("nan") if start_garbage else 0.0, dtype=t.float32, device="cuda")
    lse_acc = t.full((B, H, S_q), float("-inf"), dtype=t.float32, device="cuda")
    o = t.empty((B, S_q, H, D), dtype=t.bfloat16, device="cuda")
    for i, (lo, hi) in enumerate(bounds):
        note(f"{what}: step {i} keys [{lo}, {hi})")
        prev_o = o_acc.cpu().numpy().astype(np.float64)
        prev_l = lse_acc.cpu().numpy().astype(np.float64)
        lsd.attn_fwd_accumulate(dq, dk[:, lo:hi], dv[:, lo:hi], o_acc, lse_acc, o=o, scale=scale)
        t.cuda.synchronize()
        O_s, L_s = ref.attention_accumulate(prev_o, prev_l, q, k[:, lo:hi], v[:, lo:hi], scale)
        got_o = o_acc.cpu().numpy().astype(np.float64)
        got_l = lse_acc.cpu().numpy()
        acc32 = o_acc.cpu().numpy()
        # rows still without history (LSE = -inf) have no defined O_acc
        empty = np.isneginf(np.transpose(got_l, (0, 2, 1)))[..., None] & np.ones_like(acc32, dtype=bool)
        assert_attention_close(np.where(empty, 0.0, got_o), O_s, got_l, L_s, f"{what} step {i} (o_acc)")
        # the bf16 output is the running result rounded to nearest-even
        want = np.where(empty, np.uint16(0), f32_to_bf16_bits(np.where(empty, 0.0, acc32)))
        assert np.array_equal(to_bits(o), want), f"{what} step {i}: bf16 output != rounded o_acc"
    return o_acc, lse_acc, o


@pytest.mark.parametrize("D", [64, 128])
def test_ring_steps_equal_full_attention(D):
    q = synth.normal_bf16((2, 300, 3, D), 70, 1)
    k = synth.normal_bf16((2, 333, 3, D), 71, 1)
    v = synth.normal_bf16((2, 333, 3, D), 72, 1)
    bounds = [(0, 0), (0, 97), (97, 97), (97, 256), (256, 333)]
    o_acc, lse_acc, o = run_steps(q, k, v, bounds, f"D={D}")
    O, L = ref.attention(q, k, v)
    assert_attention_close(to_f64(o), O, lse_acc.cpu().numpy(), L, f"D={D} final bf16")
    assert_attention_close(o_acc.cpu().numpy().astype(np.float64), O, None, None, f"D={D} final fp32")


def test_tiny_four_chunks_explicit_scale_and_strided_views():
    t = torch()
    q, k, v = synth.tiny_qkv()
    fused = np.stack([q, k, v], axis=2)                         # [1,256,3,2,64]
    f = to_dev(fused)
    dq, dk, dv = f[:, :, 0], f[:, :, 1], f[:, :, 2]             # strided views
    o_acc = t.zeros((1, 256, 2, 64), dtype=t.float32, device="cuda")
    lse_acc = t.full((1, 2, 256), float("-inf"), dtype=t.float32, device="cuda")
    note("tiny accumulate over 4 chunks, scale 0.2, strided views")
    for c in range(4):
        lsd.attn_fwd_accumulate(dq, dk[:, 64 * c:64 * (c + 1)], dv[:, 64 * c:64 * (c + 1)], o_acc, lse_acc,
                                scale=0.2)
    t.cuda.synchronize()
    O, L = ref.attention(q, k, v, scale=0.2)
    assert_attention_close(o_acc.cpu().numpy().astype(np.float64), O, lse_acc.cpu().numpy(), L, "tiny")


def test_matches_separate_attention_and_merge():
    """The fused step and the separate path (attn_fwd per block + attn_merge)
    compute the same result up to the separate path's bf16 partials."""
    t = torch()
    q = synth.normal_bf16((1, 520, 4, 128), 73, 1)
    k = synth.normal_bf16((1, 700, 4, 128), 74, 1)
    v = synth.normal_bf16((1, 700, 4, 128), 75, 1)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    bounds = [(0, 250), (250, 600), (600, 700)]
    note("accumulate vs attn_fwd + attn_merge")
    o_acc = t.zeros((1, 520, 4, 128), dtype=t.float32, device="cuda")
    lse_acc = t.full((1, 4, 520), float("-inf"), dtype=t.float32, device="cuda")
    o_f = t.empty((1, 520, 4, 128), dtype=t.bfloat16, device="cuda")
    for i, (lo, hi) in enumerate(bounds):
        lsd.attn_fwd_accumulate(dq, dk[:, lo:hi], dv[:, lo:hi], o_acc, lse_acc,
                                o=o_f if i == len(bounds) - 1 else None)
    parts = [lsd.attn_fwd(dq, dk[:, lo:hi], dv[:, lo:hi]) for lo, hi in bounds]
    om, lm = lsd.attn_merge([p[0] for p in parts], [p[1] for p in parts])
    t.cuda.synchronize()
    assert_attention_close(to_f64(o_f), to_f64(om), lse_acc.cpu().numpy(), lm.cpu().numpy(), "fused vs separate")
    O, L = ref.attention(q, k, v)
    assert_attention_close(to_f64(o_f), O, lse_acc.cpu().numpy(), L, "fused vs oracle")


def test_empty_block_keeps_state_and_determinism():
    t = torch()
    B, S_q, H, D = 1, 130, 2, 128
    q = synth.normal_bf16((B, S_q, H, D), 76, 1)
    k = synth.normal_bf16((B, 90, H, D), 77, 1)
    v = synth.normal_bf16((B, 90, H, D), 78, 1)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    note("accumulate: empty block, partial history, determinism")
    o_acc = t.zeros((B, S_q, H, D), dtype=t.float32, device="cuda")
    lse_acc = t.full((B, H, S_q), float("-inf"), dtype=t.float32, device="cuda")
    lsd.attn_fwd_accumulate(dq, dk, dv, o_acc, lse_acc)
    lse_acc[0, 1, 5:9] = float("-inf")            # some rows without history
    o_acc[0, 5:9, 1] = float("nan")
    before_o, before_l = o_acc.clone(), lse_acc.clone()
    o = t.empty((B, S_q, H, D), dtype=t.bfloat16, device="cuda")
    lsd.attn_fwd_accumulate(dq, dk[:, :0], dv[:, :0], o_acc, lse_acc, o=o)
    t.cuda.synchronize()
    assert t.equal(lse_acc, before_l)
    assert np.array_equal(o_acc.cpu().numpy(), before_o.cpu().numpy(), equal_nan=True)
    ob = to_bits(o)
    assert (ob[0, 5:9, 1] == 0).all()
    mask = np.ones(ob.shape, dtype=bool)
    mask[0, 5:9, 1] = False
    assert np.array_equal(ob[mask], f32_to_bf16_bits(before_o.cpu().numpy())[mask])
    # rows without history take the next block's result, NaN history ignored
    lsd.attn_fwd_accumulate(dq, dk, dv, o_acc, lse_acc)
    t.cuda.synchronize()
    assert t.isfinite(o_acc).all()
    O, L = ref.attention(q, k, v)
    got = o_acc.cpu().numpy()[0, 5:9, 1].astype(np.float64)
    assert_attention_close(got, O[0, 5:9, 1], lse_acc.cpu().numpy()[0, 1, 5:9], L[0, 1, 5:9], "fresh rows")
    # determinism: the same sequence of steps gives the same bits
    runs = []
    for _ in range(2):
        oa = t.zeros((B, S_q, H, D), dtype=t.float32, device="cuda")
        la = t.full((B, H, S_q), float("-inf"), dtype=t.float32, device="cuda")
        for lo, hi in [(0, 40), (40, 90)]:
            lsd.attn_fwd_accumulate(dq, dk[:, lo:hi], dv[:, lo:hi], oa, la)
        t.cuda.synchronize()
        runs.append((oa.cpu().numpy(), la.cpu().numpy()))
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])
