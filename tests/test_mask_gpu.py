"""Key-only padding mask on the GPU (through the C ABI): batch entry b attends
its first kv_lens[b] keys.  Padding keys are filled with NaN bit patterns, so
any read of them would poison the output."""

import numpy as np
import pytest

import synth
from oracle import ref
from gpu_util import assert_attention_close, note, to_bits, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

lsd = pytest.importorskip("long_sequence_dit_amd")

NAN_BITS = np.uint16(0x7FC1)


def lens_dev(lens):
    t = torch()
    return t.tensor(lens, dtype=t.int32, device="cuda")


def poison(x, lens):
    x = x.copy()
    for b, n in enumerate(lens):
        x[b, max(0, min(n, x.shape[1])):] = NAN_BITS
    return x


@pytest.mark.parametrize("D", [64, 128])
def test_per_batch_lengths_with_nan_padding(D):
    note(f"masked attention D={D}: lengths across tile edges, NaN padding")
    t = torch()
    lens = [300, 1, 63, 64, 65, 129, 0, 257]
    B, S_q, S_kv, H = len(lens), 200, 300, 2
    q = synth.normal_bf16((B, S_q, H, D), 80, 1)
    k = poison(synth.normal_bf16((B, S_kv, H, D), 81, 1), lens)
    v = poison(synth.normal_bf16((B, S_kv, H, D), 82, 1), lens)
    o, lse = lsd.attn_fwd(to_dev(q), to_dev(k), to_dev(v), kv_lens=lens_dev(lens))
    t.cuda.synchronize()
    O, L = ref.attention(q, k, v, kv_lens=lens)
    og, lg = to_f64(o), lse.cpu().numpy()
    assert_attention_close(og, O, lg, L, f"D={D}")
    assert (og[6] == 0).all() and np.isneginf(lg[6]).all()


def test_lengths_are_clamped():
    note("masked attention: lengths clamped to [0, S_kv]")
    t = torch()
    q = synth.normal_bf16((2, 70, 2, 128), 83, 1)
    k = synth.normal_bf16((2, 90, 2, 128), 84, 1)
    v = synth.normal_bf16((2, 90, 2, 128), 85, 1)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    o1, l1 = lsd.attn_fwd(dq, dk, dv, kv_lens=lens_dev([-4, 1000]))
    o2, l2 = lsd.attn_fwd(dq, dk, dv, kv_lens=lens_dev([0, 90]))
    t.cuda.synchronize()
    assert np.array_equal(to_bits(o1), to_bits(o2)) and t.equal(l1, l2)


def test_mask_equals_truncated_views_bit_exact():
    """A length-n mask and a view of the first n keys run the same tiles: the
    results are identical bit for bit."""
    note("masked attention == truncated views, bit-exact")
    t = torch()
    S_kv = 400
    q = synth.normal_bf16((1, 333, 3, 128), 86, 1)
    k = synth.normal_bf16((1, S_kv, 3, 128), 87, 1)
    v = synth.normal_bf16((1, S_kv, 3, 128), 88, 1)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    for n in (1, 64, 150, 399):
        om, lm = lsd.attn_fwd(dq, dk, dv, kv_lens=lens_dev([n]))
        ot, lt = lsd.attn_fwd(dq, dk[:, :n], dv[:, :n])
        t.cuda.synchronize()
        assert np.array_equal(to_bits(om), to_bits(ot)) and t.equal(lm, lt), f"n={n}"


def test_padded_sequence_pad_queries_see_valid_keys():
    """The pages' padding: 1,003 tokens padded to 1,008 (a multiple of 8);
    pad query rows attend every valid key and are finite."""
    note("padded sequence 1003 -> 1008, key-only mask")
    t = torch()
    T, Tp, H, D = 1003, 1008, 4, 128
    q = synth.normal_bf16((1, Tp, H, D), 89, 1)
    q[:, T:] = 0                                               # zero pad rows, as padding does
    k = poison(synth.normal_bf16((1, Tp, H, D), 90, 1), [T])
    v = poison(synth.normal_bf16((1, Tp, H, D), 91, 1), [T])
    o, lse = lsd.attn_fwd(to_dev(q), to_dev(k), to_dev(v), kv_lens=lens_dev([T]))
    t.cuda.synchronize()
    O, L = ref.attention(q, k, v, kv_lens=[T])
    og = to_f64(o)
    assert np.isfinite(og).all()
    assert_attention_close(og, O, lse.cpu().numpy(), L, "padded")
    # a zero query row weighs every valid key equally: O = mean of valid V
    assert_attention_close(og[0, T:], np.broadcast_to(ref.bf16_bits_to_f64(v[0, :T]).mean(axis=0), og[0, T:].shape),
                           None, None, "pad rows")


def test_accumulate_with_block_masks():
    note("accumulate with per-batch block lengths")
    t = torch()
    B, S_q, H, D = 2, 150, 2, 128
    q = synth.normal_bf16((B, S_q, H, D), 92, 1)
    k = synth.normal_bf16((B, 256, H, D), 93, 1)
    v = synth.normal_bf16((B, 256, H, D), 94, 1)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    # two blocks of 128 keys; the second block of batch 1 has only 37 valid keys
    masks = [[128, 128], [128, 37]]
    o_acc = t.zeros((B, S_q, H, D), dtype=t.float32, device="cuda")
    lse_acc = t.full((B, H, S_q), float("-inf"), dtype=t.float32, device="cuda")
    o = t.empty((B, S_q, H, D), dtype=t.bfloat16, device="cuda")
    for i in range(2):
        lsd.attn_fwd_accumulate(dq, dk[:, 128 * i:128 * (i + 1)], dv[:, 128 * i:128 * (i + 1)], o_acc, lse_acc,
                                o=o if i == 1 else None, kv_lens=lens_dev([m[i] for m in masks]))
    t.cuda.synchronize()
    keep = np.concatenate([np.arange(128), 128 + np.arange(37)])
    O0, L0 = ref.attention(q[:1], k[:1], v[:1])
    O1, L1 = ref.attention(q[1:], k[1:, keep], v[1:, keep])
    O = np.concatenate([O0, O1])
    L = np.concatenate([L0, L1])
    assert_attention_close(to_f64(o), O, lse_acc.cpu().numpy(), L, "accumulate + mask")
