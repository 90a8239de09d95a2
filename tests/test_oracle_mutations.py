"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch every one of them: a pin set that a dropped term, a wrong sign, a wrong
index or a transposed operand slips through would not pin anything."""

import math

import numpy as np
import pytest

from oracle import ref
import oracle_pins as pins


def _run(pin_list):
    failed = []
    for pin in pin_list:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


def _block_no_scale(qh, kh, vh, scale):
    return _orig_block(qh, kh, vh, 1.0)


def _block_sqrt_mult(qh, kh, vh, scale):
    return _orig_block(qh, kh, vh, 1.0 / scale)


def _block_log2(qh, kh, vh, scale):
    o, lse = _orig_block(qh, kh, vh, scale)
    return o, lse / math.log(2.0)


def _block_dropped_max(qh, kh, vh, scale):
    s = (qh @ kh.T) * scale
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return (e @ vh) / l[:, None], np.log(l)


def _block_no_normalise(qh, kh, vh, scale):
    s = (qh @ kh.T) * scale
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return e @ vh, m + np.log(e.sum(axis=1))


def _block_wrong_sign(qh, kh, vh, scale):
    return _orig_block(-qh, kh, vh, scale)


def _block_transposed(qh, kh, vh, scale):
    # keys and queries swapped: weights of key j over queries
    s = (kh @ qh.T) * scale                      # [S_kv, n]
    m = s.max(axis=0)
    e = np.exp(s - m[None, :])
    l = e.sum(axis=0)
    w = (e / l[None, :]).T                       # still [n, S_kv] but normalised the wrong way
    return w @ vh, m + np.log(l)


def _block_off_by_one_key(qh, kh, vh, scale):
    return _orig_block(qh, kh[:-1], vh[:-1], scale) if kh.shape[0] > 1 else _orig_block(qh, kh, vh, scale)


def _block_v_shift(qh, kh, vh, scale):
    return _orig_block(qh, kh, np.roll(vh, 1, axis=0), scale)


_orig_block = ref._attend_block

ATTN_MUTANTS = [_block_no_scale, _block_sqrt_mult, _block_log2, _block_dropped_max,
                _block_no_normalise, _block_wrong_sign, _block_transposed,
                _block_off_by_one_key, _block_v_shift]


@pytest.mark.parametrize("mutant", ATTN_MUTANTS, ids=lambda f: f.__name__)
def test_attention_mutant_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(ref, "_attend_block", mutant)
    assert _run(pins.ATTENTION_PINS), f"{mutant.__name__} passed every attention pin"


_orig_merge = ref.merge


def _merge_unnormalised(o_parts, lse_parts):
    O, L = _orig_merge(o_parts, lse_parts)
    n = len(o_parts)
    return O * n, L


def _merge_dropped_max(o_parts, lse_parts):
    O, L = _orig_merge(o_parts, lse_parts)
    M = np.max(np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts]), axis=0)
    with np.errstate(invalid="ignore"):
        return O, np.where(np.isneginf(M), L, L - M)


def _merge_wrong_sign(o_parts, lse_parts):
    return _orig_merge(o_parts, [-np.asarray(x, dtype=np.float64) for x in lse_parts])


def _merge_untransposed(o_parts, lse_parts):
    # weights indexed [B, H, S] applied as if they were [B, S, H]
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])
    M = L.max(axis=0)
    w = np.exp(L - np.where(np.isneginf(M), 0.0, M)[None])
    ws = w.sum(axis=0)
    O = sum(np.reshape(w[i], (w.shape[1], w.shape[3], w.shape[2]))[..., None] * ref._as_f64(o)
            for i, o in enumerate(o_parts))
    O = O / np.reshape(ws, (ws.shape[0], ws.shape[2], ws.shape[1]))[..., None]
    return O, M + np.log(ws)


def _merge_first_only(o_parts, lse_parts):
    return ref._as_f64(o_parts[0]), np.asarray(lse_parts[0], dtype=np.float64)


MERGE_MUTANTS = [_merge_unnormalised, _merge_dropped_max, _merge_wrong_sign,
                 _merge_untransposed, _merge_first_only]


@pytest.mark.parametrize("mutant", MERGE_MUTANTS, ids=lambda f: f.__name__)
def test_merge_mutant_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(ref, "merge", mutant)
    assert _run(pins.MERGE_PINS), f"{mutant.__name__} passed every merge pin"


_orig_relayout = ref.relayout_seq_to_head


def _relayout_next_rank(chunks, P, rank):
    return _orig_relayout(chunks, P, (rank + 1) % P)


def _relayout_reversed_chunks(chunks, P, rank):
    return _orig_relayout(list(chunks)[::-1], P, rank)


def _relayout_no_check(chunks, P, rank):
    B, S_loc, H, D = chunks[0].shape
    hl = max(1, H // P)
    return np.concatenate([c[:, :, rank * hl:(rank + 1) * hl, :] for c in chunks], axis=1)


def _relayout_interleaved(chunks, P, rank):
    y = _orig_relayout(chunks, P, rank)
    B, S, hl, D = y.shape
    S_loc = S // P
    # tokens interleaved across shards instead of concatenated
    return y.reshape(B, P, S_loc, hl, D).transpose(0, 2, 1, 3, 4).reshape(B, S, hl, D)


RELAYOUT_MUTANTS = [_relayout_next_rank, _relayout_reversed_chunks, _relayout_no_check,
                    _relayout_interleaved]


@pytest.mark.parametrize("mutant", RELAYOUT_MUTANTS, ids=lambda f: f.__name__)
def test_relayout_mutant_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(ref, "relayout_seq_to_head", mutant)
    assert _run(pins.RELAYOUT_PINS), f"{mutant.__name__} passed every relayout pin"


_orig_accumulate = ref.attention_accumulate


def _acc_keeps_garbage(o_acc, lse_acc, q, k, v, scale=None):
    # forgets that O_acc is meaningless where there is no history
    O_b, L_b = ref.attention(q, k, v, scale)
    return ref.merge([np.asarray(o_acc, dtype=np.float64), O_b], [np.asarray(lse_acc, dtype=np.float64), L_b])


def _acc_replaces(o_acc, lse_acc, q, k, v, scale=None):
    # the running result is overwritten instead of merged
    O_b, L_b = ref.attention(q, k, v, scale)
    return O_b, L_b


def _acc_unweighted(o_acc, lse_acc, q, k, v, scale=None):
    # averages the two results instead of weighting by their LSEs
    O_b, L_b = ref.attention(q, k, v, scale)
    L_a = np.asarray(lse_acc, dtype=np.float64)
    none = np.transpose(np.isneginf(L_a), (0, 2, 1))[..., None]
    O_a = np.where(none, O_b, np.asarray(o_acc, dtype=np.float64))
    _, L = ref.merge([O_a, O_b], [L_a, L_b])
    return 0.5 * (O_a + O_b), L


ACCUMULATE_MUTANTS = [_acc_keeps_garbage, _acc_replaces, _acc_unweighted]


@pytest.mark.parametrize("mutant", ACCUMULATE_MUTANTS, ids=lambda f: f.__name__)
def test_accumulate_mutant_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(ref, "attention_accumulate", mutant)
    assert _run(pins.ACCUMULATE_PINS), f"{mutant.__name__} passed every accumulate pin"


_orig_inverse = ref.relayout_head_to_seq


def _inverse_next_shard(heads, P, p):
    return _orig_inverse(heads, P, (p + 1) % P)


def _inverse_reversed_ranks(heads, P, p):
    return _orig_inverse(list(heads)[::-1], P, p)


INVERSE_MUTANTS = [_inverse_next_shard, _inverse_reversed_ranks]


@pytest.mark.parametrize("mutant", INVERSE_MUTANTS, ids=lambda f: f.__name__)
def test_inverse_relayout_mutant_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(ref, "relayout_head_to_seq", mutant)
    assert _run(pins.RELAYOUT_PINS), f"{mutant.__name__} passed every relayout pin"


_orig_valid_keys = ref.valid_keys


def _mask_ignored(kv_lens, b, S_kv):
    return S_kv


def _mask_one_extra(kv_lens, b, S_kv):
    return min(_orig_valid_keys(kv_lens, b, S_kv) + 1, S_kv)


def _mask_unclamped(kv_lens, b, S_kv):
    return S_kv if kv_lens is None else int(kv_lens[b])


MASK_MUTANTS = [_mask_ignored, _mask_one_extra, _mask_unclamped]


@pytest.mark.parametrize("mutant", MASK_MUTANTS, ids=lambda f: f.__name__)
def test_key_mask_mutant_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(ref, "valid_keys", mutant)
    assert _run(pins.ATTENTION_PINS), f"{mutant.__name__} passed every attention pin"


from oracle import fp8 as _fp8

_orig_encode = _fp8.e4m3_encode
_orig_decode = _fp8.e4m3_decode


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    c = _orig_encode(x)
    vals = _orig_decode(np.arange(0x7F))
    mids = 0.5 * (vals[:-1] + vals[1:])
    hit = np.isin(np.abs(x), mids)
    up = (np.searchsorted(vals, np.abs(x)) & 0x7F).astype(np.uint8) | (np.signbit(x).astype(np.uint8) << 7)
    return np.where(hit, up, c).astype(np.uint8)


def _encode_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    vals = _orig_decode(np.arange(0x7F))
    lo = np.clip(np.searchsorted(vals, np.abs(x), side="right") - 1, 0, 0x7E)
    return (lo | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def _decode_fnuz_bias(c):
    return _orig_decode(c) * 0.5


_orig_head_amax = _fp8.head_amax


def _amax_per_tensor(x):
    a = _orig_head_amax(x)
    return np.full_like(a, a.max())


_orig_dequant = _fp8.dequantize


def _dequant_no_scale(codes, amax):
    return _orig_decode(codes)


_orig_qscale = _fp8.q_scale_amax


def _qscale_identity(amax_q, amax_k):
    return np.asarray(amax_q, dtype=np.float32)


def _qscale_no_log2e(amax_q, amax_k):
    # the softmax scale without log2(e): a power of two in natural-log units
    return _orig_qscale(amax_q, np.asarray(amax_k, np.float32) / np.float32(np.log2(np.e)))


def _qscale_uses_q(amax_q, amax_k):
    return _orig_qscale(amax_q, amax_q)


def _qscale_power_too_low(amax_q, amax_k):
    return (_orig_qscale(amax_q, amax_k) * np.float32(0.5)).astype(np.float32)


def _qscale_power_too_high(amax_q, amax_k):
    r = _orig_qscale(amax_q, amax_k)
    return np.where(np.asarray(amax_q) > 0, r * np.float32(2.0), r).astype(np.float32)


_orig_amax_valid = _fp8.head_amax_valid


def _amax_valid_ignores_lengths(x, lens):
    return _orig_head_amax(x)


def _amax_valid_one_short(x, lens):
    return _orig_amax_valid(x, np.maximum(np.asarray(lens) - 1, 0))


FP8_MUTANTS = [("head_amax_valid", _amax_valid_ignores_lengths), ("head_amax_valid", _amax_valid_one_short),
               ("e4m3_encode", _encode_ties_away), ("e4m3_encode", _encode_truncate),
               ("e4m3_decode", _decode_fnuz_bias), ("head_amax", _amax_per_tensor),
               ("dequantize", _dequant_no_scale), ("q_scale_amax", _qscale_identity),
               ("q_scale_amax", _qscale_no_log2e), ("q_scale_amax", _qscale_uses_q),
               ("q_scale_amax", _qscale_power_too_low), ("q_scale_amax", _qscale_power_too_high)]


@pytest.mark.parametrize("name,mutant", FP8_MUTANTS, ids=lambda f: getattr(f, "__name__", str(f)))
def test_fp8_mutant_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(_fp8, name, mutant)
    assert _run(pins.FP8_PINS), f"{mutant.__name__} passed every fp8 pin"
