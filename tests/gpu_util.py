"""Helpers for the GPU parity tests: moving bf16 bit patterns between numpy
and device memory, and the parity bar.

The bar (spec tolerances): O max-abs <= 2e-2 and mean-abs <= 2e-3 against
the float64 oracle (bf16 output decoded exactly), LSE max-abs <= 1e-3;
relayout bit-exact.
"""

from __future__ import annotations

import sys

import numpy as np

from oracle import ref

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


def torch():
    import torch as _t
    return _t


def to_dev(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).cuda()


def to_bits(x) -> np.ndarray:
    t = torch()
    return x.detach().view(t.int16).contiguous().cpu().numpy().view(np.uint16)


def to_f64(x) -> np.ndarray:
    return ref.bf16_bits_to_f64(to_bits(x))


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def err_stats(o_gpu: np.ndarray, o_ref: np.ndarray):
    d = np.abs(o_gpu - o_ref)
    rel = float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    return float(d.max()), float(d.mean()), rel


def lse_max_abs(lse_gpu, lse_ref, what="") -> float:
    """Largest |LSE_gpu - LSE_ref|; entries that are -inf on both sides agree
    (0), a -inf on one side only is a mismatch (raises)."""
    lg = np.asarray(lse_gpu, dtype=np.float64)
    lr = np.asarray(lse_ref, dtype=np.float64)
    both_inf = np.isneginf(lg) & np.isneginf(lr)
    with np.errstate(invalid="ignore"):   # -inf - -inf is masked out just below
        d = np.where(both_inf, 0.0, np.abs(lg - lr))
    assert np.all(np.isfinite(d)), f"{what}: LSE -inf/finite mismatch"
    return float(d.max()) if d.size else 0.0


def assert_attention_close(o_gpu: np.ndarray, o_ref: np.ndarray, lse_gpu=None, lse_ref=None, what="",
                           with_lse=False):
    """The parity bar; returns (O max-abs, O mean-abs, O relative RMS) and,
    with ``with_lse``, the LSE max-abs as a fourth value."""
    mx, mean, rel = err_stats(o_gpu, o_ref)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    assert mx <= O_MAX_ABS, f"{what}: O max-abs {mx:.3e} > {O_MAX_ABS}"
    assert mean <= O_MEAN_ABS, f"{what}: O mean-abs {mean:.3e} > {O_MEAN_ABS}"
    dl = 0.0
    if lse_gpu is not None:
        dl = lse_max_abs(lse_gpu, lse_ref, what)
        assert dl <= LSE_MAX_ABS, f"{what}: LSE max-abs {dl:.3e} > {LSE_MAX_ABS}"
    return (mx, mean, rel, dl) if with_lse else (mx, mean, rel)
