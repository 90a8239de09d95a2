"""Pins for the CPU oracle: facts fixed by the mathematics or printed on the
pages, independent of the oracle's own code.

Each pin is a function that raises AssertionError when the oracle disagrees.
They look the oracle's functions up through the ``oracle.ref`` module at call
time, so a test can plant a mistake in the oracle (monkeypatch) and check that
some pin catches it.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import synth
from oracle import ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _dec(bits):
    return ref.bf16_bits_to_f64(bits)


def _bits_of(value: float) -> np.uint16:
    return synth.f32_to_bf16_bits(np.array([value], dtype=np.float32))[0]


def _rand(shape, seed, tag=91):
    return synth.normal_bf16(shape, seed, tag)


# ----------------------------------------------------------------- attention

def pin_identical_keys():
    """All keys equal k: every weight is 1/S_kv, so O_i = mean_j v_j and
    LSE_i = scale * q_i.k + ln S_kv (closed form)."""
    B, Sq, Skv, H, D = 2, 37, 53, 3, 64
    q = _rand((B, Sq, H, D), 1)
    krow = _rand((B, 1, H, D), 2)
    k = np.repeat(krow, Skv, axis=1)
    v = _rand((B, Skv, H, D), 3)
    O, L = ref.attention(q, k, v)
    assert O.shape == (B, Sq, H, D) and L.shape == (B, H, Sq)
    vm = _dec(v).mean(axis=1)                                   # [B,H,D]
    exp_o = np.broadcast_to(vm[:, None, :, :], O.shape)
    assert np.allclose(O, exp_o, rtol=0, atol=1e-12), "identical keys: O != mean(V)"
    qk = np.sum(_dec(q) * _dec(krow), axis=3)                   # [B,Sq,H]
    exp_l = np.transpose(qk / math.sqrt(D) + math.log(Skv), (0, 2, 1))
    assert np.allclose(L, exp_l, rtol=0, atol=1e-12), "identical keys: LSE closed form"


def pin_dominant_logit():
    """q = 2*ones, K = 0 except K[j*] = 2*ones (D = 128): the logit of j* is
    s* = 4*sqrt(128) and every other logit is 0, so
    O = (e^{s*} v_{j*} + sum_{j != j*} v_j) / (e^{s*} + S - 1) and
    LSE = s* + ln(1 + (S - 1) e^{-s*})."""
    S, D, H = 300, 128, 2
    two = _bits_of(2.0)
    q = np.full((1, 7, H, D), two, dtype=np.uint16)
    k = np.zeros((1, S, H, D), dtype=np.uint16)
    js = [123, 7]
    for h in range(H):
        k[0, js[h], h, :] = two
    v = _rand((1, S, H, D), 4)
    O, L = ref.attention(q, k, v)
    s_star = 4.0 * math.sqrt(D)
    vf = _dec(v)
    for h in range(H):
        others = vf[0, :, h, :].sum(axis=0) - vf[0, js[h], h, :]
        e = math.exp(s_star)
        exp_o = (e * vf[0, js[h], h, :] + others) / (e + S - 1)
        assert np.allclose(O[0, :, h, :], exp_o[None, :], rtol=0, atol=1e-13), "dominant logit: O"
        exp_l = s_star + math.log1p((S - 1) * math.exp(-s_star))
        assert np.allclose(L[0, h, :], exp_l, rtol=0, atol=1e-12), "dominant logit: LSE"


def pin_rows_sum_to_one():
    """Softmax rows sum to 1: with V = 1 everywhere the output is exactly 1 for
    every row (any weight that is lost, doubled or unnormalised moves it)."""
    B, Sq, Skv, H, D = 1, 19, 41, 2, 64
    q = _rand((B, Sq, H, D), 5)
    k = _rand((B, Skv, H, D), 6)
    ones = np.full((B, Skv, H, D), _bits_of(1.0), dtype=np.uint16)
    O, _ = ref.attention(q, k, ones)
    assert np.allclose(O, 1.0, rtol=0, atol=1e-13), "V = 1 must give O = 1"


def pin_single_key():
    """S_kv = 1: O = v_0 and LSE = scale * q . k_0."""
    B, Sq, H, D = 2, 9, 3, 128
    q = _rand((B, Sq, H, D), 7)
    k = _rand((B, 1, H, D), 8)
    v = _rand((B, 1, H, D), 9)
    O, L = ref.attention(q, k, v)
    assert np.array_equal(O, np.broadcast_to(_dec(v), O.shape)), "S_kv = 1: O = v_0"
    s = np.sum(_dec(q) * _dec(k), axis=3) / math.sqrt(D)        # [B,Sq,H]
    assert np.allclose(L, np.transpose(s, (0, 2, 1)), rtol=0, atol=1e-12)


def pin_no_keys():
    """S_kv = 0 (chosen reading): O = 0 and LSE = -inf, never NaN."""
    q = _rand((1, 5, 2, 64), 10)
    k = np.zeros((1, 0, 2, 64), dtype=np.uint16)
    O, L = ref.attention(q, k, k)
    assert np.all(O == 0) and np.all(np.isneginf(L))


def pin_library_softmax():
    """Against scipy's softmax and logsumexp on an asymmetric shape
    (S_q != S_kv, H != D/..), logits formed with einsum."""
    from scipy.special import logsumexp, softmax
    B, Sq, Skv, H, D = 2, 23, 45, 3, 64
    q = _rand((B, Sq, H, D), 11)
    k = _rand((B, Skv, H, D), 12)
    v = _rand((B, Skv, H, D), 13)
    scale = 0.3
    O, L = ref.attention(q, k, v, scale=scale)
    logits = np.einsum("bqhd,bkhd->bhqk", _dec(q), _dec(k)) * scale
    exp_l = logsumexp(logits, axis=3)
    exp_o = np.einsum("bhqk,bkhd->bqhd", softmax(logits, axis=3), _dec(v))
    assert np.allclose(L, exp_l, rtol=0, atol=1e-12), "LSE vs scipy logsumexp"
    assert np.allclose(O, exp_o, rtol=0, atol=1e-12), "O vs scipy softmax"


def pin_brute_force_tiny():
    """Explicit loops in pure Python (no BLAS) on a tiny case."""
    B, Sq, Skv, H, D = 1, 4, 6, 2, 4
    q = _rand((B, Sq, H, D), 14)
    k = _rand((B, Skv, H, D), 15)
    v = _rand((B, Skv, H, D), 16)
    O, L = ref.attention(q, k, v)
    qf, kf, vf = _dec(q).tolist(), _dec(k).tolist(), _dec(v).tolist()
    sc = 1.0 / math.sqrt(D)
    for h in range(H):
        for i in range(Sq):
            logits = []
            for j in range(Skv):
                acc = 0.0
                for d in range(D):
                    acc += qf[0][i][h][d] * kf[0][j][h][d]
                logits.append(acc * sc)
            tot = sum(math.exp(x) for x in logits)
            assert abs(L[0, h, i] - math.log(tot)) < 1e-12
            for d in range(D):
                o = sum(math.exp(logits[j]) * vf[0][j][h][d] for j in range(Skv)) / tot
                assert abs(O[0, i, h, d] - o) < 1e-12


def pin_permutation_and_scaling():
    """Permuting keys and values together leaves O and LSE unchanged;
    scaling V by 2 scales O by exactly 2."""
    B, Sq, Skv, H, D = 1, 11, 40, 2, 64
    q = _rand((B, Sq, H, D), 17)
    k = _rand((B, Skv, H, D), 18)
    v = _rand((B, Skv, H, D), 19)
    O, L = ref.attention(q, k, v)
    perm = np.random.Generator(np.random.PCG64(5)).permutation(Skv)
    O2, L2 = ref.attention(q, k[:, perm], v[:, perm])
    assert np.allclose(O, O2, rtol=0, atol=1e-13) and np.allclose(L, L2, rtol=0, atol=1e-12)
    O3, L3 = ref.attention(q, k, 2.0 * _dec(v))
    assert np.array_equal(O3, 2.0 * O) and np.array_equal(L3, L)


def pin_scale_argument():
    """An explicit scale equal to 1/sqrt(D) gives the default result; doubling
    the scale equals doubling Q (exact in bf16)."""
    B, S, H, D = 1, 16, 2, 64
    q = _rand((B, S, H, D), 20)
    k = _rand((B, S, H, D), 21)
    v = _rand((B, S, H, D), 22)
    O, L = ref.attention(q, k, v)
    Od, Ld = ref.attention(q, k, v, scale=1.0 / 8.0)
    assert np.array_equal(O, Od) and np.array_equal(L, Ld)
    O2, L2 = ref.attention(q, k, v, scale=0.25)
    O3, L3 = ref.attention(2.0 * _dec(q), k, v)
    assert np.allclose(O2, O3, rtol=0, atol=1e-12) and np.allclose(L2, L3, rtol=0, atol=1e-12)


def pin_key_mask():
    """The key-only padding mask: batch entry b attends its first kv_lens[b]
    keys.  Pads filled with huge values change nothing; the result equals the
    unmasked oracle on the truncated keys, a pure-Python brute force of the
    masked definition on a tiny case, and 0 / -inf for no valid keys; lengths
    are clamped to [0, S_kv]; every query row (padded ones included) gets a
    distribution over the valid keys."""
    B, Sq, Skv, H, D = 3, 11, 23, 2, 64
    q = _rand((B, Sq, H, D), 41)
    k = _rand((B, Skv, H, D), 42).copy()
    v = _rand((B, Skv, H, D), 43).copy()
    lens = [23, 9, 0]
    O, L = ref.attention(q, k, v, kv_lens=lens)
    k[1, 9:] = _bits_of(3.0e4)
    v[1, 9:] = _bits_of(-7.0e3)
    k[2] = _bits_of(1.0e3)
    O2, L2 = ref.attention(q, k, v, kv_lens=lens)
    assert np.array_equal(O, O2) and np.array_equal(L, L2), "padding keys leaked into the result"
    for b, n in enumerate(lens):
        Ot, Lt = ref.attention(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n])
        assert np.allclose(O[b], Ot[0], rtol=0, atol=1e-13) and np.allclose(L[b], Lt[0], rtol=0, atol=1e-13)
    assert np.all(O[2] == 0) and np.all(np.isneginf(L[2]))
    Oc, Lc = ref.attention(q, k, v, kv_lens=[99, -5, 0])
    O0, L0 = ref.attention(q, k, v, kv_lens=[23, 0, 0])
    assert np.array_equal(Oc, O0) and np.array_equal(Lc, L0), "kv_lens not clamped to [0, S_kv]"
    # brute force, tiny: explicit loops over the valid keys only
    qt = _rand((1, 3, 1, 4), 44)
    kt = _rand((1, 5, 1, 4), 45)
    vt = _rand((1, 5, 1, 4), 46)
    Ob, Lb = ref.attention(qt, kt, vt, scale=0.5, kv_lens=[3])
    qf, kf, vf = (_dec(x).tolist() for x in (qt, kt, vt))
    for i in range(3):
        logits = [0.5 * sum(qf[0][i][0][d] * kf[0][j][0][d] for d in range(4)) for j in range(3)]
        m = max(logits)
        ws = [math.exp(x - m) for x in logits]
        tot = sum(ws)
        assert abs(Lb[0, 0, i] - (m + math.log(tot))) < 1e-12
        for d in range(4):
            want = sum(ws[j] * vf[0][j][0][d] for j in range(3)) / tot
            assert abs(Ob[0, i, 0, d] - want) < 1e-12
    # rows_variant agrees and puts no weight on padding
    rows = [0, 5, 10]
    o_r, l_r = ref.attention_rows(q, k, v, 1, 1, rows, kv_lens=lens)
    assert np.allclose(o_r, O[1, rows, 1], rtol=0, atol=1e-13) and np.allclose(l_r, L[1, 1, rows], rtol=0, atol=1e-13)


# ----------------------------------------------------------------- merge

def _partials(q, k, v, bounds):
    outs, lses = [], []
    for lo, hi in bounds:
        o, l = ref.attention(q, k[:, lo:hi], v[:, lo:hi])
        outs.append(o)
        lses.append(l)
    return outs, lses


def pin_merge_equals_full():
    """Merging partials over disjoint key spans (one of them empty) equals
    attention over all keys."""
    B, Sq, Skv, H, D = 1, 256, 256, 2, 64
    q, k, v = synth.tiny_qkv()
    O, L = ref.attention(q, k, v)
    bounds = [(0, 64), (64, 128), (128, 128), (128, 192), (192, 256)]
    outs, lses = _partials(q, k, v, bounds)
    Om, Lm = ref.merge(outs, lses)
    assert np.allclose(Om, O, rtol=0, atol=1e-12) and np.allclose(Lm, L, rtol=0, atol=1e-12)
    # the ragged, asymmetric case: S_q != S_kv, H != S
    q2 = _rand((2, 13, 3, 64), 23)
    k2 = _rand((2, 29, 3, 64), 24)
    v2 = _rand((2, 29, 3, 64), 25)
    O2, L2 = ref.attention(q2, k2, v2)
    outs, lses = _partials(q2, k2, v2, [(0, 5), (5, 17), (17, 29)])
    Om2, Lm2 = ref.merge(outs, lses)
    assert np.allclose(Om2, O2, rtol=0, atol=1e-12) and np.allclose(Lm2, L2, rtol=0, atol=1e-12)


def pin_merge_attention2d_grid():
    """The pages' 2x3 Attention2D example: the row group holding query shards
    {0,1,2} attends key shards {0,3}, {1,4}, {2,5}; merging the three partials
    recovers full attention for those queries."""
    g = _golden()["attention2d_grid"]
    n, shard = g["shards"], 24
    H, D = 2, 64
    q = _rand((1, n * shard, H, D), 26)
    k = _rand((1, n * shard, H, D), 27)
    v = _rand((1, n * shard, H, D), 28)
    rows = np.concatenate([np.arange(s * shard, (s + 1) * shard) for s in g["row_group_queries"]])
    qrow = q[:, rows]
    O, L = ref.attention(qrow, k, v)
    outs, lses = [], []
    for key_shards in g["row_group_key_shards"]:
        keys = np.concatenate([np.arange(s * shard, (s + 1) * shard) for s in key_shards])
        o, l = ref.attention(qrow, k[:, keys], v[:, keys])
        outs.append(o)
        lses.append(l)
    assert len(outs) == g["col_size"]
    Om, Lm = ref.merge(outs, lses)
    assert np.allclose(Om, O, rtol=0, atol=1e-12) and np.allclose(Lm, L, rtol=0, atol=1e-12)


def pin_merge_closed_forms():
    """n identical partials: O unchanged, LSE + ln n.  A -inf partial has no
    effect.  Equal LSEs average.  n = 1 is the identity.  All -inf: O = 0,
    LSE = -inf."""
    B, S, H, D = 1, 10, 3, 64
    o1 = _dec(_rand((B, S, H, D), 29))
    o2 = _dec(_rand((B, S, H, D), 30))
    l1 = _dec(_rand((B, H, S), 31)) * 3.0 + 5.0
    for n in (1, 2, 3, 8):
        O, L = ref.merge([o1] * n, [l1] * n)
        assert np.allclose(O, o1, rtol=0, atol=1e-13)
        assert np.allclose(L, l1 + math.log(n), rtol=0, atol=1e-12)
    ninf = np.full((B, H, S), -np.inf)
    O, L = ref.merge([o1, o2], [l1, ninf])
    assert np.allclose(O, o1, rtol=0, atol=1e-13) and np.array_equal(L, l1)
    O, L = ref.merge([o2, o1], [ninf, l1])
    assert np.allclose(O, o1, rtol=0, atol=1e-13) and np.array_equal(L, l1)
    O, L = ref.merge([o1, o2], [l1, l1])
    assert np.allclose(O, 0.5 * (o1 + o2), rtol=0, atol=1e-13)
    assert np.allclose(L, l1 + math.log(2.0), rtol=0, atol=1e-12)
    O, L = ref.merge([o1, o2], [ninf, ninf])
    assert np.all(O == 0) and np.all(np.isneginf(L))
    # weights are per (b, h, s): an asymmetric LSE pattern picks per row
    lbig = l1.copy()
    lbig[0, 1, 4] = 1e3
    O, L = ref.merge([o1, o2], [lbig, l1])
    assert np.allclose(O[0, 4, 1], o1[0, 4, 1], rtol=0, atol=1e-13)
    assert np.allclose(O[0, 4, 0], 0.5 * (o1[0, 4, 0] + o2[0, 4, 0]), rtol=0, atol=1e-13)


def pin_ring_streaming_merge():
    """The Ring schedule's two-partial sigmoid/logsigmoid update, applied
    block by block, equals the batched merge and full attention."""
    q, k, v = synth.tiny_qkv()
    O, L = ref.attention(q, k, v)
    outs, lses = _partials(q, k, v, [(0, 64), (64, 128), (128, 192), (192, 256)])
    run_o, run_l = outs[0], lses[0]
    for o, l in zip(outs[1:], lses[1:]):
        run_o, run_l = ref.merge_two_logsigmoid(run_o, run_l, o, l)
    assert np.allclose(run_o, O, rtol=0, atol=1e-12) and np.allclose(run_l, L, rtol=0, atol=1e-12)
    ninf = np.full_like(lses[0], -np.inf)
    o, l = ref.merge_two_logsigmoid(outs[0], ninf, outs[1], lses[1])
    assert np.allclose(o, outs[1], rtol=0, atol=1e-13) and np.array_equal(l, lses[1])
    o, l = ref.merge_two_logsigmoid(outs[0], ninf, outs[1], ninf)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def pin_accumulate_streams_to_full():
    """Ring steps with the merge folded in, over disjoint key blocks (one of
    them empty), starting from no history (LSE = -inf, O = NaN garbage), end
    at full attention; the rows variant agrees with the full variant."""
    q, k, v = synth.tiny_qkv()
    O, L = ref.attention(q, k, v)
    B, S, H, D = q.shape
    run_o = np.full((B, S, H, D), np.nan)
    run_l = np.full((B, H, S), -np.inf)
    for lo, hi in [(0, 40), (40, 40), (40, 131), (131, 256)]:
        prev_o, prev_l = run_o, run_l
        run_o, run_l = ref.attention_accumulate(run_o, run_l, q, k[:, lo:hi], v[:, lo:hi])
        rows = [0, 7, 255]
        o_r, l_r = ref.attention_accumulate_rows(prev_o[0, rows, 1], prev_l[0, 1, rows], q, k[:, lo:hi],
                                                 v[:, lo:hi], 0, 1, rows)
        assert np.allclose(o_r, run_o[0, rows, 1], rtol=0, atol=1e-13, equal_nan=True)
        assert np.allclose(l_r, run_l[0, 1, rows], rtol=0, atol=1e-13)
    assert np.allclose(run_o, O, rtol=0, atol=1e-12) and np.allclose(run_l, L, rtol=0, atol=1e-12)
    # the ragged, asymmetric case
    q2 = _rand((2, 13, 3, 64), 33)
    k2 = _rand((2, 29, 3, 64), 34)
    v2 = _rand((2, 29, 3, 64), 35)
    O2, L2 = ref.attention(q2, k2, v2)
    run_o = np.zeros((2, 13, 3, 64))
    run_l = np.full((2, 3, 13), -np.inf)
    for lo, hi in [(0, 1), (1, 17), (17, 29)]:
        run_o, run_l = ref.attention_accumulate(run_o, run_l, q2, k2[:, lo:hi], v2[:, lo:hi])
    assert np.allclose(run_o, O2, rtol=0, atol=1e-12) and np.allclose(run_l, L2, rtol=0, atol=1e-12)


def pin_accumulate_special_cases():
    """A block with no keys leaves the running result unchanged (and gives
    O = 0, LSE = -inf when there is none); with no history the step is plain
    attention; one step equals the Ring schedule's sigmoid/logsigmoid update
    of the same two partials."""
    B, S, H, D = 1, 9, 2, 64
    q = _rand((B, S, H, D), 36)
    k = _rand((B, 21, H, D), 37)
    v = _rand((B, 21, H, D), 38)
    o_a = _dec(_rand((B, S, H, D), 39))
    l_a = _dec(_rand((B, H, S), 40)) + 4.0
    empty_k = k[:, :0]
    o, l = ref.attention_accumulate(o_a, l_a, q, empty_k, empty_k)
    assert np.allclose(o, o_a, rtol=0, atol=1e-14) and np.array_equal(l, l_a)
    ninf = np.full((B, H, S), -np.inf)
    o, l = ref.attention_accumulate(o_a, ninf, q, empty_k, empty_k)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    Ob, Lb = ref.attention(q, k, v)
    o, l = ref.attention_accumulate(np.full_like(o_a, np.nan), ninf, q, k, v)
    assert np.allclose(o, Ob, rtol=0, atol=1e-14) and np.allclose(l, Lb, rtol=0, atol=1e-14)
    o, l = ref.attention_accumulate(o_a, l_a, q, k, v)
    o2, l2 = ref.merge_two_logsigmoid(o_a, l_a, Ob, Lb)
    assert np.allclose(o, o2, rtol=0, atol=1e-12) and np.allclose(l, l2, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- relayout

def pin_relayout_index_map():
    """Element-wise: Y[b, p*S_loc + s, j, d] = X_p[b, s, r*H/P + j, d],
    checked by scalar lookups at random positions."""
    B, S_loc, H, D, P = 2, 7, 8, 16, 4
    chunks = [synth.random_bits16((B, S_loc, H, D), 100 + p) for p in range(P)]
    g = np.random.Generator(np.random.PCG64(9))
    for r in range(P):
        y = ref.relayout_seq_to_head(chunks, P, r)
        assert y.shape == (B, P * S_loc, H // P, D) and y.dtype == np.uint16
        for _ in range(200):
            b, p, s = int(g.integers(B)), int(g.integers(P)), int(g.integers(S_loc))
            j, d = int(g.integers(H // P)), int(g.integers(D))
            assert y[b, p * S_loc + s, j, d] == chunks[p][b, s, r * (H // P) + j, d]


def pin_relayout_identity_and_round_trip():
    """P = 1 is a plain copy; sending every rank its head slice and gathering
    back gives the input bit for bit (NaN payloads included)."""
    B, S_loc, H, D = 1, 5, 12, 8
    x = synth.random_bits16((B, S_loc, H, D), 200)
    assert np.array_equal(ref.relayout_seq_to_head([x], 1, 0), x)
    for P in (2, 3, 4, 6):
        chunks = [synth.random_bits16((B, S_loc, H, D), 300 + 10 * P + p) for p in range(P)]
        ys = [ref.relayout_seq_to_head(chunks, P, r) for r in range(P)]
        for p in range(P):
            back = ref.relayout_head_to_seq(ys, P, p)
            assert np.array_equal(back, chunks[p])


def pin_relayout_inverse_index_map():
    """Element-wise: X_p[b, s, r*H_loc + j, d] = Y_r[b, p*S_loc + s, j, d] for the
    inverse, by scalar lookups at random positions."""
    B, S_loc, H_loc, D, P = 2, 6, 3, 16, 4
    ys = [synth.random_bits16((B, P * S_loc, H_loc, D), 150 + r) for r in range(P)]
    g = np.random.Generator(np.random.PCG64(10))
    for p in range(P):
        x = ref.relayout_head_to_seq(ys, P, p)
        assert x.shape == (B, S_loc, P * H_loc, D) and x.dtype == np.uint16
        for _ in range(200):
            b, r, s = int(g.integers(B)), int(g.integers(P)), int(g.integers(S_loc))
            j, d = int(g.integers(H_loc)), int(g.integers(D))
            assert x[b, s, r * H_loc + j, d] == ys[r][b, p * S_loc + s, j, d]


def pin_relayout_head_limit():
    """Ulysses degree must divide the head count: with 40 heads on 72 GPUs the
    largest usable degree is 8 (the pages' example)."""
    g = _golden()["ulysses_head_limit"]
    H, G = g["num_heads"], g["gpus"]
    ok = []
    for P in range(1, H + 1):
        chunks = [np.zeros((1, 2, H, 4), dtype=np.uint16)] * P
        try:
            ref.relayout_seq_to_head(chunks, P, 0)
        except ValueError:
            continue
        if G % P == 0:
            ok.append(P)
    assert max(ok) == g["largest_ulysses_degree"]


ATTENTION_PINS = [pin_identical_keys, pin_dominant_logit, pin_rows_sum_to_one, pin_single_key,
                  pin_no_keys, pin_library_softmax, pin_brute_force_tiny,
                  pin_permutation_and_scaling, pin_scale_argument, pin_key_mask]
MERGE_PINS = [pin_merge_equals_full, pin_merge_attention2d_grid, pin_merge_closed_forms,
              pin_ring_streaming_merge]
ACCUMULATE_PINS = [pin_accumulate_streams_to_full, pin_accumulate_special_cases]
RELAYOUT_PINS = [pin_relayout_index_map, pin_relayout_identity_and_round_trip, pin_relayout_head_limit,
                 pin_relayout_inverse_index_map]
ALL_PINS = ATTENTION_PINS + MERGE_PINS + ACCUMULATE_PINS + RELAYOUT_PINS


# ----------------------------------------------------------------- fp8

def pin_e4m3_code_table():
    """OCP E4M3 facts: 0x7E = 448 (largest), 0x08 = 2^-6 (smallest normal),
    0x01 = 2^-9 (smallest subnormal), 0x38 = 1, 0xB8 = -1, 0x7F / 0xFF NaN;
    every finite code decodes and re-encodes to itself; values are monotonic
    in the code."""
    from oracle import fp8
    d = fp8.e4m3_decode
    assert d(0x7E) == 448.0 and d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9
    assert d(0x38) == 1.0 and d(0xB8) == -1.0 and d(0x40) == 2.0 and d(0x3C) == 1.5
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF)) and d(0x00) == 0.0
    codes = np.arange(256)
    fin = (codes & 0x7F) != 0x7F
    vals = d(codes)
    assert np.array_equal(fp8.e4m3_encode(vals[fin]), codes[fin].astype(np.uint8))
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)


def pin_e4m3_rounding():
    """Round to nearest, ties to even: midpoints between neighbouring codes
    go to the even mantissa, points just off a midpoint go to the nearer code;
    464 (the midpoint above 448) rounds to 448 and larger values overflow to
    NaN; the sign of zero is kept."""
    from oracle import fp8
    vals = fp8.e4m3_decode(np.arange(0x7F))
    mids = 0.5 * (vals[:-1] + vals[1:])
    got = fp8.e4m3_encode(mids)
    for i, c in enumerate(got):
        even = i if i % 2 == 0 else i + 1
        assert c == even, f"midpoint {mids[i]} -> {c:#x}, want {even:#x}"
    eps = 1e-9
    assert np.array_equal(fp8.e4m3_encode(mids - eps * mids), np.arange(0x7E, dtype=np.uint8))
    assert np.array_equal(fp8.e4m3_encode(mids + eps * mids), np.arange(1, 0x7F, dtype=np.uint8))
    assert fp8.e4m3_encode(np.array([464.0]))[0] == 0x7E
    assert fp8.e4m3_encode(np.array([464.01]))[0] == 0x7F
    assert fp8.e4m3_encode(np.array([-1e9]))[0] == 0xFF
    assert fp8.e4m3_encode(np.array([-0.0]))[0] == 0x80 and fp8.e4m3_encode(np.array([0.0]))[0] == 0x00
    # relative error of normal values is at most half an ulp (2^-4)
    x = np.linspace(2.0 ** -6, 448.0, 10001)
    err = np.abs(fp8.e4m3_decode(fp8.e4m3_encode(x)) - x) / x
    assert err.max() <= 2.0 ** -4 + 1e-15


def pin_fp8_cast():
    """The cast: the largest magnitude of each (tensor, batch, head) codes to
    +-448 exactly (for Q, whose scale amax may be up to twice its amax, to
    at least 224); an all-zero head codes to zeros; values already on the
    FP8 grid of their head's scale are reproduced exactly; every dequantised
    value is within half an FP8 ulp (plus the subnormal step) of the input."""
    from oracle import fp8
    B, S, H, D = 2, 37, 3, 64
    q = _rand((B, S, H, D), 51)
    k = _rand((B, S, H, D), 52).copy()
    v = _rand((B, S, H, D), 53)
    k[1, :, 2, :] = 0                                           # an all-zero head
    q8, k8, v8, amax = fp8.cast_qkv(q, k, v)
    assert amax.shape == (3, B, H)
    for t, (x, c, a) in enumerate(((q, q8, amax[0]), (k, k8, amax[1]), (v, v8, amax[2]))):
        xv = _dec(x)
        for b in range(B):
            for h in range(H):
                if a[b, h] == 0:
                    assert np.all(c[b, :, h] & 0x7F == 0)
                    continue
                i = np.unravel_index(np.argmax(np.abs(xv[b, :, h])), xv[b, :, h].shape)
                if t == 0:
                    assert 224.0 <= fp8.e4m3_decode(c[b, :, h][i] & 0x7F) <= 448.0
                else:
                    assert (c[b, :, h][i] & 0x7F) == 0x7E
        deq = fp8.dequantize(c, a)
        step = (np.asarray(a, np.float64) / 448.0)[:, None, :, None]
        assert np.all(np.abs(deq - xv) <= np.abs(xv) * 2.0 ** -4 + step * 2.0 ** -9 * 1.01)
    # exactly representable inputs: codes times a power-of-two scale
    codes = np.random.Generator(np.random.PCG64(54)).integers(0, 0x7F, size=(1, 16, 1, 32)).astype(np.uint8)
    codes[0, 3, 0, 5] = 0x7E                                    # amax = 448 -> factor 1
    xb = synth.f32_to_bf16_bits(fp8.e4m3_decode(codes).astype(np.float32))
    assert np.array_equal(fp8.quantize(xb, fp8.head_amax(xb)), codes)


def pin_fp8_q_scale():
    """Q's scale amax: at least amax_q and below 2 amax_q, and with it the
    default logit factor log2(e) / sqrt(128) * (amax_q' / 448) * (amax_k / 448)
    is a power of two (checked in float64, to 2^-20); heads whose amax_q or
    amax_k is zero keep amax_q; the cast stores it as Q's amax."""
    from oracle import fp8
    g = np.random.Generator(np.random.PCG64(56))
    aq = np.exp(g.uniform(-25.0, 25.0, size=4000)).astype(np.float32)
    ak = np.exp(g.uniform(-25.0, 25.0, size=4000)).astype(np.float32)
    aq[:8] = [1.0, 448.0, 2.0 ** -10, 3.0, 1.0, 1.5, 7.0, 100.0]
    ak[:8] = [1.0, 448.0, 2.0 ** 10, 3.0, 448.0, 0.75, 7.0, 0.01]
    r = fp8.q_scale_amax(aq, ak).astype(np.float64)
    a64, k64 = aq.astype(np.float64), ak.astype(np.float64)
    assert np.all(r >= a64) and np.all(r < 2.0 * a64 * (1.0 + 2.0 ** -20))
    c = (np.log2(np.e) / np.sqrt(128.0)) * (r / 448.0) * (k64 / 448.0)
    lg = np.log2(c)
    assert np.all(np.abs(lg - np.round(lg)) < 2.0 ** -20 / np.log(2.0))
    z = fp8.q_scale_amax(np.array([0.0, 5.0, 0.0], np.float32), np.array([3.0, 0.0, 0.0], np.float32))
    assert np.array_equal(z, np.array([0.0, 5.0, 0.0], np.float32))
    B, S, H, D = 1, 20, 3, 64
    q, k, v = _rand((B, S, H, D), 57), _rand((B, S, H, D), 58), _rand((B, S, H, D), 59)
    _, _, _, amax = fp8.cast_qkv(q, k, v)
    aq2, ak2 = fp8.head_amax(q).astype(np.float64), fp8.head_amax(k).astype(np.float64)
    a0 = amax[0].astype(np.float64)
    assert np.all(a0 >= aq2) and np.all(a0 < 2.0 * aq2 * (1.0 + 2.0 ** -20))
    lg = np.log2((np.log2(np.e) / np.sqrt(128.0)) * (a0 / 448.0) * (ak2 / 448.0))
    assert np.all(np.abs(lg - np.round(lg)) < 2.0 ** -20 / np.log(2.0))
    assert np.array_equal(amax[1], fp8.head_amax(k).astype(np.float32))


def pin_fp8_attention():
    """FP8 attention is attention of the dequantised inputs: with inputs that
    the cast reproduces exactly it equals attention of the originals, and a
    uniform positive rescaling of one tensor's codes' scale (amax) scales the
    dequantised values and so the logits or outputs accordingly."""
    from oracle import fp8
    g = np.random.Generator(np.random.PCG64(55))
    def on_grid(shape):
        c = g.integers(0, 0x7F, size=shape).astype(np.uint8) | (g.integers(0, 2, size=shape).astype(np.uint8) << 7)
        c[..., 0, :, 0] = 0x7E                                  # amax 448 per (b, h)
        return c
    B, S, H, D = 1, 40, 2, 64
    q8, k8, v8 = on_grid((B, S, H, D)), on_grid((B, S, H, D)), on_grid((B, S, H, D))
    amax = np.full((B, H), 448.0, np.float32)
    O, L = fp8.attention_fp8(q8, k8, v8, amax, amax, amax, scale=1e-4)
    O2, L2 = ref.attention(fp8.e4m3_decode(q8), fp8.e4m3_decode(k8), fp8.e4m3_decode(v8), scale=1e-4)
    assert np.allclose(O, O2, rtol=0, atol=1e-12) and np.allclose(L, L2, rtol=0, atol=1e-12)
    # v scale 2x -> O 2x; q scale 2x with scale/2 -> same result
    O3, L3 = fp8.attention_fp8(q8, k8, v8, amax, amax, 2 * amax, scale=1e-4)
    assert np.allclose(O3, 2 * O, rtol=0, atol=1e-9) and np.allclose(L3, L, rtol=0, atol=1e-12)
    O4, L4 = fp8.attention_fp8(q8, k8, v8, 2 * amax, amax, amax, scale=0.5e-4)
    assert np.allclose(O4, O, rtol=0, atol=1e-12) and np.allclose(L4, L, rtol=0, atol=1e-12)
    rows = [0, 17, 39]
    o_r, l_r = fp8.attention_fp8_rows(q8, k8, v8, amax, amax, amax, 0, 1, rows, scale=1e-4)
    assert np.allclose(o_r, O[0, rows, 1], rtol=0, atol=1e-12) and np.allclose(l_r, L[0, 1, rows], rtol=0, atol=1e-12)


def pin_fp8_key_lengths():
    """The key-length mask on the FP8 path reduces to the unmasked cast and
    attention of the valid keys alone: per batch entry, the masked cast's
    amax and its Q, K and V codes of valid tokens equal the unmasked cast of
    Q with K and V cut to their first kv_lens[b] tokens; V's padding codes
    are zero; an entry without keys has K and V amax 0 (Q keeps its amax);
    NaN in the padding changes nothing; lengths are clamped to [0, S]; with
    every length S the masked cast is the unmasked one; the masked attention
    equals attention over the cut keys."""
    from oracle import fp8
    B, S, H, D = 4, 70, 2, 64
    q = _rand((B, S, H, D), 61)
    k = _rand((B, S, H, D), 62).copy()
    v = _rand((B, S, H, D), 63).copy()
    lens = [70, 33, 0, 1]
    nan_bits = np.uint16(0x7FC1)
    for b, n in enumerate(lens):
        k[b, n:] = nan_bits
        v[b, n:] = nan_bits
    q8, k8, v8, amax = fp8.cast_qkv(q, k, v, kv_lens=lens)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(amax[1:, b] == 0) and np.all(v8[b] == 0)
            assert np.array_equal(amax[0, b], fp8.head_amax(q[b:b + 1])[0].astype(np.float32))
            continue
        tq, tk, tv, ta = fp8.cast_qkv(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n])
        assert np.array_equal(amax[:, b], ta[:, 0])
        assert np.array_equal(q8[b], tq[0]) and np.array_equal(k8[b, :n], tk[0]) and np.array_equal(v8[b, :n], tv[0])
        assert np.all(v8[b, n:] == 0)
    # clamping, and the mask at full length
    _, _, _, a_clamp = fp8.cast_qkv(q, k, v, kv_lens=[100, 33, -5, 1])
    assert np.array_equal(a_clamp, amax)
    kk, vv = _rand((B, S, H, D), 62), _rand((B, S, H, D), 63)
    full = fp8.cast_qkv(q, kk, vv, kv_lens=[S] * B)
    ref_full = fp8.cast_qkv(q, kk, vv)
    assert all(np.array_equal(x, y) for x, y in zip(full, ref_full))
    # attention over the valid keys (entries with keys)
    O, L = fp8.attention_fp8(q8, k8, v8, amax[0], amax[1], amax[2], kv_lens=lens)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(O[b] == 0) and np.all(np.isneginf(L[b]))
            continue
        Ob, Lb = fp8.attention_fp8(q8[b:b + 1], k8[b:b + 1, :n], v8[b:b + 1, :n], amax[0, b:b + 1], amax[1, b:b + 1],
                                   amax[2, b:b + 1])
        assert np.array_equal(O[b], Ob[0]) and np.array_equal(L[b], Lb[0])
        o_r, l_r = fp8.attention_fp8_rows(q8, k8, v8, amax[0], amax[1], amax[2], b, 1, [0, 69], kv_len=n)
        assert np.allclose(o_r, O[b, [0, 69], 1], rtol=0, atol=1e-12) and np.allclose(l_r, L[b, 1, [0, 69]], rtol=0,
                                                                                       atol=1e-12)


def pin_fp8_ring_steps():
    """Ring steps on FP8 inputs: three key/value blocks, each cast with its own
    scales, streamed into a running result from LSE = -inf, give the attention
    of the dequantised query against all dequantised blocks together (the
    exact merge); an empty block leaves the result unchanged."""
    from oracle import fp8
    B, S_q, H, D = 1, 30, 2, 64
    q = _rand((B, S_q, H, D), 71)
    q8, _, _, aq = fp8.cast_qkv(q, q, q)
    blocks = []
    for i, n in enumerate((17, 40, 9)):
        k = synth.f32_to_bf16_bits(_dec(_rand((B, n, H, D), 72 + i)).astype(np.float32) * (1.0 + i))
        v = _rand((B, n, H, D), 80 + i)
        _, k8, v8, a = fp8.cast_qkv(k, k, v)
        blocks.append((k8, v8, a[1], a[2]))
    o = np.zeros((B, S_q, H, D))
    lse = np.full((B, H, S_q), -np.inf)
    for k8, v8, ak, av in blocks:
        o, lse = fp8.attention_fp8_accumulate(o, lse, q8, k8, v8, aq[0], ak, av, scale=0.1)
    K = np.concatenate([fp8.dequantize(k8, ak) for k8, _, ak, _ in blocks], axis=1)
    V = np.concatenate([fp8.dequantize(v8, av) for _, v8, _, av in blocks], axis=1)
    O, L = ref.attention(fp8.dequantize(q8, aq[0]), K, V, scale=0.1)
    assert np.allclose(o, O, rtol=0, atol=1e-12) and np.allclose(lse, L, rtol=0, atol=1e-12)
    k8, v8, ak, av = blocks[0]
    o2, l2 = fp8.attention_fp8_accumulate(o, lse, q8, k8[:, :0], v8[:, :0], aq[0], ak, av, scale=0.1)
    assert np.array_equal(o2, o) and np.array_equal(l2, lse)


def pin_fp8_kv_cast():
    """The K/V-only cast against a given Q scale: K's scale amax lies in
    [amax_k, 2 amax_k) and with it the default logit factor
    log2(e) / sqrt(128) * (q_scale / 448) * (k_scale / 448) is a power of two
    (float64, to 2^-20); K is coded with it, V exactly as the full cast codes
    it; slot 0 is zero; with a key-length mask V's padding codes are zero and
    the scales come from the valid tokens."""
    from oracle import fp8
    B, S, H, D = 2, 45, 3, 64
    q = _rand((B, S, H, D), 91)
    k = _rand((B, S, H, D), 92)
    v = _rand((B, S, H, D), 93)
    _, _, _, aq = fp8.cast_qkv(q, q, q)
    k8, v8, amax = fp8.cast_kv(k, v, aq[0])
    ak = fp8.head_amax(k).astype(np.float64)
    a1 = amax[1].astype(np.float64)
    assert np.all(amax[0] == 0)
    assert np.all(a1 >= ak) and np.all(a1 < 2.0 * ak * (1.0 + 2.0 ** -20))
    lg = np.log2((np.log2(np.e) / np.sqrt(128.0)) * (aq[0].astype(np.float64) / 448.0) * (a1 / 448.0))
    assert np.all(np.abs(lg - np.round(lg)) < 2.0 ** -20 / np.log(2.0))
    assert np.array_equal(k8, fp8.quantize(k, amax[1]))
    _, _, fv8, famax = fp8.cast_qkv(q, k, v)
    assert np.array_equal(v8, fv8) and np.array_equal(amax[2], famax[2])
    lens = [45, 7]
    mk8, mv8, mamax = fp8.cast_kv(k, v, aq[0], kv_lens=lens)
    _, _, mfv8, mfamax = fp8.cast_qkv(q, k, v, kv_lens=lens)
    assert np.array_equal(mv8, mfv8) and np.array_equal(mamax[2], mfamax[2])
    assert np.array_equal(mamax[1], fp8.q_scale_amax(mfamax[1], aq[0]))


FP8_PINS = [pin_e4m3_code_table, pin_e4m3_rounding, pin_fp8_cast, pin_fp8_q_scale, pin_fp8_attention,
            pin_fp8_key_lengths, pin_fp8_ring_steps, pin_fp8_kv_cast]
ALL_PINS = ALL_PINS + FP8_PINS
