"""Float64 CPU oracle: attention with LSE, LSE merge (batched and folded into a
Ring step), and the Ulysses relayouts in both directions.

Test infrastructure only (see the package docstring): nothing on the product
path may import it.

Sources (page title, then section):

* [NVL72] "Scaling Video Generation Across NVL72 rack with TensorRT-LLM".
  - "The Scaling Challenge in Video Generation": every denoising step runs
    dense, bidirectional self-attention with no causal mask over the whole
    sequence.
  - "Context Parallelism > Attention2D Parallelism > Local Attention": the
    inner backend returns a partial output [B, S_q, H, D] together with a
    log-sum-exp statistic [B, H, S_q], the softmax normaliser of that pass.
  - "Context Parallelism > Ring Attention > Online-softmax merge" and
    "Attention2D > Merge phase": partial (O, LSE) pairs over disjoint key
    spans are merged (streaming, or in one batched combine) into the result
    of one global attention pass.
  - "Ulysses Parallelism": the [B, S/P, H, D] -> [B, S, H/P, D] exchange; P
    must divide the head count.
* [TeleFuser] "CUDA IPC Ulysses: overlapping attention communication on H100",
  sections "Baseline and bottleneck" and "Strided Copy Engine scatter": the
  scatter turns (B, S_local, H_global, D) into (B, S_global, H_local, D), and
  reads the fused-QKV V projection as a strided view.
* [LTX-2 SP] "How 8 GPUs split tokens: what LTX-2's sequence-parallel all2all
  moves", sections "Precise statement" and "How attention is exchanged across
  ranks": a pure byte mover whose round trip gather(send(x)) is byte-exact.

Readings where the pages are silent (each also listed in the design notes):
natural-log LSE over *scaled* logits; scale 1/sqrt(D) unless given; no keys
(S_kv = 0) gives O = 0 and LSE = -inf; a merge whose partials are all -inf gives
O = 0 and LSE = -inf.

Inputs in bfloat16 arrive as ``numpy.uint16`` bit patterns and are decoded
exactly to float64 here; all arithmetic is float64.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

_ROW_CHUNK = 512


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns: the 16 bits are the top half of
    an IEEE binary32 value."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _as_f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


def _default_scale(D: int, scale):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def _attend_block(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float):
    """softmax(scale * q k^T) v for one (batch, head): q [n, D], k/v [S_kv, D].

    Returns (O [n, D], LSE [n]) with LSE_i = ln sum_j exp(scale * q_i . k_j)
    [NVL72, Local Attention].
    """
    n, D = qh.shape
    if kh.shape[0] == 0:
        return np.zeros((n, vh.shape[1])), np.full(n, -np.inf)
    s = (qh @ kh.T) * scale                      # scaled logits, [n, S_kv]
    m = s.max(axis=1)                            # row max (for a stable exp)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    o = (e @ vh) / l[:, None]
    lse = m + np.log(l)
    return o, lse


def valid_keys(kv_lens, b: int, S_kv: int) -> int:
    """Number of keys batch entry b attends: all S_kv, or kv_lens[b] clamped
    to [0, S_kv] (the key-only padding mask)."""
    if kv_lens is None:
        return S_kv
    return int(min(max(int(kv_lens[b]), 0), S_kv))


def attention(q, k, v, scale=None, kv_lens=None):
    """Dense, bidirectional multi-head attention with LSE.

    q: [B, S_q, H, D]; k, v: [B, S_kv, H, D] (bf16 bits or floats, any
    strides).  Returns O float64 [B, S_q, H, D] and LSE float64 [B, H, S_q].
    With ``kv_lens`` (B integers) batch entry b attends only its first
    kv_lens[b] keys: the rest are padding with weight 0, and every query row,
    padded or not, sees all valid keys.
    [NVL72, The Scaling Challenge; Attention2D > Local Attention;
    LTX-2 SP, Data flow (key-only padding mask)]
    """
    B, S_q, H, D = q.shape
    S_kv = k.shape[1]
    assert k.shape == (B, S_kv, H, D) and v.shape[:3] == (B, S_kv, H)
    sc = _default_scale(D, scale)
    O = np.zeros((B, S_q, H, v.shape[3]))
    L = np.full((B, H, S_q), -np.inf)
    for b in range(B):
        n = valid_keys(kv_lens, b, S_kv)
        for h in range(H):
            kh = _as_f64(k[b, :n, h, :])
            vh = _as_f64(v[b, :n, h, :])
            for r0 in range(0, S_q, _ROW_CHUNK):
                qh = _as_f64(q[b, r0:r0 + _ROW_CHUNK, h, :])
                o, lse = _attend_block(qh, kh, vh, sc)
                O[b, r0:r0 + _ROW_CHUNK, h, :] = o
                L[b, h, r0:r0 + _ROW_CHUNK] = lse
    return O, L


def attention_rows(q, k, v, b: int, h: int, rows: Iterable[int], scale=None, kv_lens=None):
    """Attention for selected query rows of one (batch, head), exact against
    the full (valid) key set.  Returns (O [n, D], LSE [n]) float64."""
    rows = np.asarray(list(rows), dtype=np.int64)
    D = q.shape[3]
    sc = _default_scale(D, scale)
    nk = valid_keys(kv_lens, b, k.shape[1])
    kh = _as_f64(k[b, :nk, h, :])
    vh = _as_f64(v[b, :nk, h, :])
    qh = _as_f64(q[b, rows, h, :])
    return _attend_block(qh, kh, vh, sc)


def merge(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """Exact log-sum-exp merge of n partial results over disjoint key spans.

    o_parts: n arrays [B, S, H, D] (bf16 bits or floats); lse_parts: n arrays
    [B, H, S].  With M = max_i LSE_i and w_i = exp(LSE_i - M):
    LSE = M + ln sum_i w_i and O = sum_i w_i O_i / sum_i w_i.  Where every
    LSE_i is -inf the result is O = 0, LSE = -inf.
    [NVL72, Ring Attention > Online-softmax merge; Attention2D > Merge phase]
    """
    n = len(o_parts)
    assert n >= 1 and len(lse_parts) == n
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])   # [n,B,H,S]
    M = L.max(axis=0)
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    w = np.exp(L - Ms[None])                                           # exp(-inf) = 0
    wsum = w.sum(axis=0)
    lse = np.where(empty, -np.inf, Ms + np.log(np.where(empty, 1.0, wsum)))
    wt = np.transpose(w, (0, 1, 3, 2))[..., None]                       # [n,B,S,H,1]
    num = np.zeros(np.asarray(o_parts[0]).shape, dtype=np.float64)
    for i in range(n):
        num += wt[i] * _as_f64(o_parts[i])
    den = np.transpose(np.where(empty, 1.0, wsum), (0, 2, 1))[..., None]
    O = num / den
    return O, lse


def attention_accumulate(o_acc, lse_acc, q, k, v, scale=None, kv_lens=None):
    """One Ring step with the merge folded in: the attention result of q
    against this key/value block, merged into the running result (O_acc,
    LSE_acc) of earlier blocks.  Where LSE_acc = -inf there is no history and
    O_acc is ignored (it may hold anything, NaN included).

    o_acc [B, S_q, H, D] floats, lse_acc [B, H, S_q]; q, k, v as for
    ``attention``.  Returns the new (O, LSE), float64.
    [NVL72, Ring Attention (each step's partial output is merged into the
    running result with the online-softmax recurrence); Limitations and
    Future Work (the combine folded into the attention kernel)]
    """
    O_b, L_b = attention(q, k, v, scale, kv_lens)
    L_a = np.asarray(lse_acc, dtype=np.float64)
    none = np.transpose(np.isneginf(L_a), (0, 2, 1))[..., None]         # [B,S,H,1]
    O_a = np.where(none, 0.0, np.asarray(o_acc, dtype=np.float64))
    return merge([O_a, O_b], [L_a, L_b])


def attention_accumulate_rows(o_acc_rows, lse_acc_rows, q, k, v, b: int, h: int, rows: Iterable[int],
                              scale=None, kv_lens=None):
    """``attention_accumulate`` for selected query rows of one (batch, head):
    o_acc_rows [n, D] and lse_acc_rows [n] are the running result of those
    rows.  Returns (O [n, D], LSE [n]) float64."""
    O_b, L_b = attention_rows(q, k, v, b, h, rows, scale, kv_lens)
    L_a = np.asarray(lse_acc_rows, dtype=np.float64)
    O_a = np.where(np.isneginf(L_a)[:, None], 0.0, np.asarray(o_acc_rows, dtype=np.float64))
    n, D = O_b.shape
    O, L = merge([O_a.reshape(1, n, 1, D), O_b.reshape(1, n, 1, D)], [L_a.reshape(1, 1, n), L_b.reshape(1, 1, n)])
    return O.reshape(n, D), L.reshape(n)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def merge_two_logsigmoid(o_a, lse_a, o_b, lse_b):
    """The two-partial streaming update written with sigmoid / logsigmoid, as
    the Ring schedule describes it: LSE = a - logsigmoid(a - b) and
    O = sigmoid(a - b) O_a + sigmoid(b - a) O_b, with (a, b) the two LSEs
    ordered so that a >= b (which keeps -inf inputs finite).
    [NVL72, Attention2D > Difference from Ring, "Merge schedule"]
    """
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    hi = np.maximum(la, lb)
    lo = np.minimum(la, lb)
    both_empty = np.isneginf(hi)
    with np.errstate(invalid="ignore"):                      # -inf - -inf is masked out
        d = np.where(both_empty, 0.0, hi - lo)               # >= 0, may be +inf
        x = np.where(both_empty, 0.0, la - lb)
    lse = np.where(both_empty, -np.inf, hi - _logsigmoid(d))
    sig_a = np.where(x >= 0, 1.0 / (1.0 + np.exp(-np.abs(x))), np.exp(-np.abs(x)) / (1.0 + np.exp(-np.abs(x))))
    sig_a = np.where(both_empty, 0.0, sig_a)
    sig_b = np.where(both_empty, 0.0, 1.0 - sig_a)
    wa = np.transpose(sig_a, (0, 2, 1))[..., None]
    wb = np.transpose(sig_b, (0, 2, 1))[..., None]
    O = wa * _as_f64(o_a) + wb * _as_f64(o_b)
    return O, lse


def relayout_seq_to_head(chunks: Sequence[np.ndarray], P: int, rank: int) -> np.ndarray:
    """Ulysses seq-major -> head-major relayout for destination ``rank``.

    chunks: the P sequence shards X_p, each (B, S_loc, H, D).  Returns
    Y (B, P*S_loc, H/P, D) with Y[b, p*S_loc + s, j, :] = X_p[b, s, rank*H/P + j, :].
    A pure copy of the 16-bit patterns.
    [NVL72, Ulysses Parallelism; TeleFuser, Baseline and bottleneck]
    """
    assert P >= 1 and len(chunks) == P and 0 <= rank < P
    B, S_loc, H, D = chunks[0].shape
    for c in chunks:
        assert c.shape == (B, S_loc, H, D), "sequence shards must be of equal length"
    if H % P != 0:
        raise ValueError(f"head count {H} is not divisible by P={P}")
    hl = H // P
    return np.concatenate([np.asarray(c)[:, :, rank * hl:(rank + 1) * hl, :] for c in chunks], axis=1)


def relayout_head_to_seq(heads: Sequence[np.ndarray], P: int, p: int) -> np.ndarray:
    """Inverse relayout: rebuild sequence shard ``p`` (B, S_loc, H, D) from the
    P head-major tensors Y_r (B, P*S_loc, H/P, D), r = 0..P-1.
    [LTX-2 SP, Precise statement: the round trip is byte-exact]
    """
    assert len(heads) == P and 0 <= p < P
    B, S, hl, D = heads[0].shape
    assert S % P == 0
    S_loc = S // P
    return np.concatenate([np.asarray(y)[:, p * S_loc:(p + 1) * S_loc, :, :] for y in heads], axis=2)
