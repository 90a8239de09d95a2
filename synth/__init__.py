"""Seeded synthetic inputs for the long-sequence DiT attention hot path.

This module only draws random numbers and stores them as bfloat16 bit
patterns (``numpy.uint16``).  It holds none of the attention, merge or
relayout arithmetic, so that the CPU oracle and the HIP path can both be fed
from it without sharing any code of the method.

Every tensor is drawn from ``numpy.random.PCG64`` streams.  A tensor with
``n`` elements is cut into fixed chunks of ``CHUNK`` elements and chunk ``c``
of a tensor with seed ``s`` and tag ``t`` draws from
``PCG64(SeedSequence([s, t, c]))``; the result is therefore identical however
many threads fill it.

Workloads (token and head counts from the pages; values are synthetic):

* tiny check: B=1, S=256, H=2, D=64, N(0,1) (seed 0);
* LTX-2 scale: B=1, S=24,576, H=32, D=128, Q/K RMS-normalised per head
  (LTX-2 sequence-parallel article, "max_tokens" section: ~24,576 video tokens
  at 1024x1536x121);
* Wan 2.2 A14B Ulysses share: fused QKV [B=2, S=75,600, 3, 40, 128] (Scaling
  Video Generation Across NVL72, "The Scaling Challenge" and "Ulysses
  Parallelism": 40 heads, ~72-75k tokens, stacked [B, S/P, 3, H, D] buffer);
* Ring/Attention2D share: Q [1,25,200,40,128], K/V [1,75,600,40,128];
* Cosmos3-Super share: B=1, S=150,000, H=16, D=128 with 1% of key rows scaled
  by 4 (outlier keys).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22

_TAG_Q, _TAG_K, _TAG_V, _TAG_QKV, _TAG_PERM, _TAG_BITS = 1, 2, 3, 4, 5, 6


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as bfloat16 bit patterns, round to nearest even.

    NaN stays NaN (quiet bit set); overflow past the largest finite bfloat16
    rounds to infinity, as IEEE round-to-nearest-even does.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def _fill_normal(n: int, seed: int, tag: int) -> np.ndarray:
    """n standard-normal float32 values, chunked and threaded, seed-stable."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, c])))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def _encode_threaded(x: np.ndarray) -> np.ndarray:
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = CHUNK

    def work(lo: int) -> None:
        out[lo:lo + step] = f32_to_bf16_bits(flat[lo:lo + step])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(0, flat.size, step)))
    return out.reshape(x.shape)


def normal_f32(shape, seed: int, tag: int) -> np.ndarray:
    n = int(np.prod(shape))
    return _fill_normal(n, seed, tag).reshape(shape)


def normal_bf16(shape, seed: int, tag: int) -> np.ndarray:
    """N(0,1) values rounded (RNE) to bfloat16, returned as uint16 bits."""
    return _encode_threaded(normal_f32(shape, seed, tag))


def random_bits16(shape, seed: int) -> np.ndarray:
    """Uniformly random 16-bit patterns (NaN/Inf/-0 payloads included)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAG_BITS])))
    return g.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def rms_normalised_bf16(shape, seed: int, tag: int, eps: float = 1e-6) -> np.ndarray:
    """N(0,1) rows divided by their RMS over the last axis (float32), as bf16.

    Stands in for a DiT's per-head Q/K RMS norm (no learned weight; eps 1e-6).
    """
    x = normal_f32(shape, seed, tag)
    flat = x.reshape(-1, shape[-1])
    rows = flat.shape[0]
    step = max(1, CHUNK // shape[-1])

    def work(lo: int) -> None:
        blk = flat[lo:lo + step]
        ms = np.mean(blk * blk, axis=1, dtype=np.float32, keepdims=True)
        blk *= (1.0 / np.sqrt(ms + np.float32(eps))).astype(np.float32)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(0, rows, step)))
    return _encode_threaded(x)


# --------------------------------------------------------------------------
# The named workloads.  Shapes are (B, S, H, D); fused QKV is (B, S, 3, H, D).
# --------------------------------------------------------------------------

TINY = dict(B=1, S=256, H=2, D=64, seed=0)
LTX2 = dict(B=1, S=24_576, H=32, D=128, seed=1)
WAN_ULYSSES = dict(B=2, S=75_600, H=40, P=4, D=128, seed=2)
RING_SHARE = dict(B=1, S_q=25_200, n_blocks=3, S_blk=25_200, H=40, D=128, seed=3)
COSMOS_LONG = dict(B=1, S=150_000, H=16, D=128, seed=4, outlier_frac=0.01, outlier_scale=4.0)


def tiny_qkv(seed: int = TINY["seed"], B=1, S=256, H=2, D=64):
    """Q, K, V bf16 bits [B,S,H,D], N(0,1), drawn Q then K then V."""
    shp = (B, S, H, D)
    return (normal_bf16(shp, seed, _TAG_Q), normal_bf16(shp, seed, _TAG_K),
            normal_bf16(shp, seed, _TAG_V))


def qkv(B, S_q, S_kv, H, D, seed):
    """Independent N(0,1) bf16 Q [B,S_q,H,D], K and V [B,S_kv,H,D]."""
    return (normal_bf16((B, S_q, H, D), seed, _TAG_Q),
            normal_bf16((B, S_kv, H, D), seed, _TAG_K),
            normal_bf16((B, S_kv, H, D), seed, _TAG_V))


def ltx2_qkv(seed: int = LTX2["seed"], S: int = LTX2["S"], H: int = LTX2["H"], D: int = 128):
    """LTX-2-scale Q, K (RMS-normalised per head) and V, bf16 [1,S,H,D]."""
    shp = (1, S, H, D)
    return (rms_normalised_bf16(shp, seed, _TAG_Q), rms_normalised_bf16(shp, seed, _TAG_K),
            normal_bf16(shp, seed, _TAG_V))


def fused_qkv(B, S, H, D, seed):
    """Stacked QKV bf16 bits [B, S, 3, H, D] (Q, K, V along axis 2)."""
    return normal_bf16((B, S, 3, H, D), seed, _TAG_QKV)


def outlier_key_rows(S: int, frac: float, seed: int) -> np.ndarray:
    """Sorted positions of round(frac*S) distinct key rows (seeded)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAG_PERM])))
    n = int(round(frac * S))
    return np.sort(g.choice(S, size=n, replace=False))


def cosmos_qkv(seed: int = COSMOS_LONG["seed"], S: int = COSMOS_LONG["S"],
               H: int = COSMOS_LONG["H"], D: int = 128,
               frac: float = COSMOS_LONG["outlier_frac"], scale: float = COSMOS_LONG["outlier_scale"]):
    """Q, K, V bf16 [1,S,H,D]; 1% of key rows (same rows for every head) x4.

    The factor 4 is a power of two, so scaling the bf16 value is exact.
    """
    shp = (1, S, H, D)
    q = normal_bf16(shp, seed, _TAG_Q)
    kf = normal_f32(shp, seed, _TAG_K)
    rows = outlier_key_rows(S, frac, seed)
    kf[:, rows] *= np.float32(scale)
    k = _encode_threaded(kf)
    del kf
    v = normal_bf16(shp, seed, _TAG_V)
    return q, k, v, rows
