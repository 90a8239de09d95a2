"""attn_merge on the GPU (through the C ABI) against the float64 oracle."""

import numpy as np
import pytest

import synth
from oracle import ref
from gpu_util import assert_attention_close, note, to_bits, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

lsd = pytest.importorskip("long_sequence_dit_amd")


def test_tiny_four_way_chunks_equal_full_attention():
    note("merge tiny: 4 x 64-key chunks")
    t = torch()
    q, k, v = synth.tiny_qkv()
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    outs, lses = [], []
    for c in range(4):
        o, l = lsd.attn_fwd(dq, dk[:, 64 * c:64 * (c + 1)], dv[:, 64 * c:64 * (c + 1)])
        outs.append(o)
        lses.append(l)
    om, lm = lsd.attn_merge(outs, lses)
    t.cuda.synchronize()
    O, L = ref.attention(q, k, v)
    assert_attention_close(to_f64(om), O, lm.cpu().numpy(), L, "4-way merge")
    # the merge itself against the oracle's merge of the same bf16 partials
    Om, Lm = ref.merge([to_bits(o) for o in outs], [l.cpu().numpy() for l in lses])
    assert_attention_close(to_f64(om), Om, lm.cpu().numpy(), Lm, "merge of partials")


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 16])
def test_random_partials(n):
    note(f"merge random partials n={n}")
    t = torch()
    B, S, H, D = 2, 333, 3, 128
    parts = [synth.normal_bf16((B, S, H, D), 40 + i, 1) for i in range(n)]
    g = np.random.Generator(np.random.PCG64(50 + n))
    lses = [(g.standard_normal((B, H, S)) * 4 + 10).astype(np.float32) for _ in range(n)]
    if n > 1:
        lses[1][0, 1, :17] = -np.inf               # an empty partial for some rows
        for i in range(n):
            lses[i][1, 2, 100:103] = -np.inf       # rows with no keys at all
    om, lm = lsd.attn_merge([to_dev(p) for p in parts], [t.from_numpy(x).cuda() for x in lses])
    t.cuda.synchronize()
    Om, Lm = ref.merge(parts, lses)
    assert_attention_close(to_f64(om), Om, lm.cpu().numpy(), Lm, f"n={n}")
    if n > 1:
        assert (om[1, 100:103, 2].float() == 0).all() and t.isneginf(lm[1, 2, 100:103]).all()


def test_heads_split_into_groups():
    # 16 partials x 70 heads: the weights of a 16-position tile of all heads do
    # not fit the kernel's LDS budget, so heads are processed in groups
    note("merge n=16, H=70 (head groups), ragged token tail")
    t = torch()
    n, B, S, H, D = 16, 1, 37, 70, 64
    parts = [synth.normal_bf16((B, S, H, D), 70 + i, 1) for i in range(n)]
    g = np.random.Generator(np.random.PCG64(71))
    lses = [(g.standard_normal((B, H, S)) * 3).astype(np.float32) for _ in range(n)]
    om, lm = lsd.attn_merge([to_dev(p) for p in parts], [t.from_numpy(x).cuda() for x in lses])
    t.cuda.synchronize()
    Om, Lm = ref.merge(parts, lses)
    assert_attention_close(to_f64(om), Om, lm.cpu().numpy(), Lm, "head groups")


def test_strided_views_guard_bands_and_determinism():
    note("merge strided + guards")
    t = torch()
    B, S, H, D = 1, 200, 4, 64
    fused = to_dev(synth.normal_bf16((B, S, 3, H, D), 60, 1))
    parts = [fused[:, :, i] for i in range(3)]
    lses = [t.from_numpy((np.random.Generator(np.random.PCG64(61 + i)).standard_normal((B, H, S)) + 5)
                         .astype(np.float32)).cuda() for i in range(3)]
    res = []
    for _ in range(2):
        big = t.full((B, S, 3 * H, D), float("nan"), dtype=t.bfloat16, device="cuda")
        o = big[:, :, H:2 * H]
        lse_big = t.full((B * H * S + 16,), float("nan"), dtype=t.float32, device="cuda")
        lse = lse_big[8:8 + B * H * S].view(B, H, S)
        lsd.attn_merge(parts, lses, o=o, lse=lse)
        t.cuda.synchronize()
        assert t.isnan(big[:, :, :H].float()).all() and t.isnan(big[:, :, 2 * H:].float()).all()
        assert t.isnan(lse_big[:8]).all() and t.isnan(lse_big[8 + B * H * S:]).all()
        res.append((to_bits(o), lse.cpu().numpy().copy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    Om, Lm = ref.merge([to_bits(p) for p in parts], [x.cpu().numpy() for x in lses])
    assert_attention_close(ref.bf16_bits_to_f64(res[0][0]), Om, res[0][1], Lm, "strided merge")


def test_merge_without_lse_output():
    note("merge lse_out = NULL")
    t = torch()
    parts = [to_dev(synth.normal_bf16((1, 64, 2, 128), 70 + i, 1)) for i in range(2)]
    lses = [t.zeros((1, 2, 64), dtype=t.float32, device="cuda") for _ in range(2)]
    o = lsd.attn_merge(parts, lses, return_lse=False)
    t.cuda.synchronize()
    Om, _ = ref.merge([to_bits(p) for p in parts], [x.cpu().numpy() for x in lses])
    assert_attention_close(to_f64(o), Om, what="no lse")
