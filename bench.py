#!/usr/bin/env python3
"""Benchmark of the long-sequence DiT attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM.  Default step (the largest single-GPU workload, the
Cosmos3-Super Ulysses share: 64 heads split 4 ways, S=150,000, D=128):

  fused QKV projection output [1, 150000, 3, 64, 128] (seq-major; heads 0-15
  hold the attention inputs, 1 % of key rows x4; heads 16-63 are seeded
  stand-ins for the other ranks' heads, never read by rank 0)
    -> relayout_seq_to_head (P = 4, rank 0: Q, K, V in one launch, V written
       token-contiguous) -> [1, 150000, 16, 128] each
    -> attn_fwd with fp32 LSE
    -> relayout_head_to_seq of O (this rank's slice and 3 stand-in slices of
       the other ranks) -> sequence shard [1, 37500, 64, 128]

Prints ONE JSON line.  ``value`` is whole-step throughput in attention TFLOP/s
(4*B*H*S_q*S_kv*D per step / step time).  ``roofline`` is measured live for
the dominant kernel (attention) with HIP events on the stream it runs on;
``kernels`` has the same for every kernel of the step.  ``legs`` times the
other workloads' kernels in the same process (attention: 3 warm-up and 10
timed launches; relayout, merge and cast: 20 and 100), each with its median,
minimum and fraction of peak:

  wan   Wan 2.2 Ulysses share: fused QKV [2,75600,3,40,128] -> relayout P=4 for
        every rank 0..3, attention [2,75600,10,128], inverse relayout per shard
  ring  Ring/Attention2D share: Q [1,25200,40,128] vs 3 K/V blocks of 25,200
        -> merge (n=3); the unblocked pass; the fused streaming Ring steps
  ltx2  LTX-2 scale: attention [1,24576,32,128] over all keys
  ltx2_fp8  the same on the FP8 path: one cast, FP8 attention

``cpu_baseline`` times the float64 CPU oracle on a bounded sample of the
step's work on this host and extrapolates it to one step.

Other step workloads (--workload): ltx2, ltx2_fp8, wan, ltx2_varlen, ring,
ring_stream, tiny; ``--legs none`` skips the legs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "attention TFLOP/s + % bf16 MFMA peak (1 GPU); merge/relayout GB/s % HBM"

ATTN_WARMUP, ATTN_ITERS = 3, 10      # timed launches per attention leg
HBM_WARMUP, HBM_ITERS = 20, 100      # per relayout / merge / cast leg

WORKLOADS = {
    "cosmos": dict(desc="Cosmos3-Super Ulysses share (P=4, 16 of 64 heads): fused QKV [1,150000,3,64,128] -> "
                        "relayout rank 0 (V token-contiguous) -> attention [1,150000,16,128] (1% of keys x4) with "
                        "fp32 LSE -> inverse relayout of O -> shard [1,37500,64,128]",
                   B=1, S=150_000, H=64, D=128, P=4, kv_blocks=1, seed=4),
    "ltx2": dict(desc="LTX-2 scale: fused QKV [1,24576,3,32,128] -> relayout (P=1) -> attention over 2 K/V "
                      "blocks with fp32 LSE -> LSE merge", B=1, S=24_576, H=32, D=128, P=1, kv_blocks=2, seed=1),
    "ltx2_fp8": dict(desc="LTX-2 scale on the FP8 path: fused QKV [1,24576,3,32,128] -> relayout (P=1) -> one "
                          "FP8 cast of Q,K,V (per-head scales) -> FP8 attention over all 24576 keys with fp32 LSE",
                     B=1, S=24_576, H=32, D=128, P=1, kv_blocks=1, seed=1, fp8=True),
    "wan": dict(desc="Wan 2.2 A14B Ulysses share: fused QKV [2,75600,3,40,128] -> relayout P=4 rank 0 "
                     "-> attention [2,75600,10,128] with fp32 LSE -> inverse relayout of O (this rank's slice "
                     "and 3 stand-in slices of the other ranks) -> shard [2,18900,40,128]", B=2, S=75_600, H=40,
                D=128, P=4, kv_blocks=1, seed=2),
    "ltx2_varlen": dict(desc="LTX-2 scale, two clips batched with a key-only padding mask: Q,K,V "
                             "[2,24576,32,128], valid keys per clip [24576, 16384] (padding filled with NaN); "
                             "FLOPs count valid keys only", B=2, S=24_576, H=32, D=128, P=None, kv_blocks=1,
                        seed=5, kv_lens=[24_576, 16_384]),
    "ring": dict(desc="Ring/Attention2D share: Q [1,25200,40,128] vs 3 K/V blocks of 25200 with fp32 LSE "
                      "-> LSE merge (n=3)", B=1, S=25_200, H=40, D=128, P=None, kv_blocks=3, seed=3),
    "ring_stream": dict(desc="Ring share with the merge folded into attention: Q [1,25200,40,128] vs 3 K/V "
                             "blocks of 25200, each step attn_fwd_accumulate into a running fp32 (O, LSE); the "
                             "last step also writes bf16 O", B=1, S=25_200, H=40, D=128, P=None, kv_blocks=3,
                        seed=3, stream=True),
    "tiny": dict(desc="tiny: fused QKV [1,256,3,2,64] -> relayout (P=1) -> attention over 4 K/V chunks -> merge",
                 B=1, S=256, H=2, D=64, P=1, kv_blocks=4, seed=0),
}

LEGS = ("wan", "ring", "ltx2", "ltx2_fp8")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="cosmos", choices=sorted(WORKLOADS))
    ap.add_argument("--legs", default="all", help="comma-separated subset of %s, 'all' or 'none'" % ",".join(LEGS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.legs == "all":
        args.legs = list(LEGS)
    elif args.legs == "none":
        args.legs = []
    else:
        args.legs = [x for x in args.legs.split(",") if x]
        bad = [x for x in args.legs if x not in LEGS]
        if bad:
            ap.error(f"unknown legs {bad}; choose from {LEGS}")
    return args


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def token_major(v):
    """The same V values stored token-contiguous (each channel's keys one row)."""
    import long_sequence_dit_amd as lsd
    B, S, H, D = v.shape
    vt = lsd.v_token_major(B, S, H, D)
    vt.copy_(v)
    return vt


def stand_in(shape, seed):
    """Seeded N(0,1) bf16 values drawn on the GPU: data that this rank's
    kernels carry (other ranks' heads or head slices) but never compute on."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


class Pipeline:
    """Device tensors and the launch sequence of one step."""

    def __init__(self, name, w):
        import torch
        import synth
        import long_sequence_dit_amd as lsd
        self.lsd, self.torch, self.name, self.w = lsd, torch, name, w
        B, S, H, D = w["B"], w["S"], w["H"], w["D"]
        self.host = {}
        if name == "cosmos":
            P = w["P"]
            hl = H // P
            q, k, v, _ = synth.cosmos_qkv(seed=w["seed"], S=S, H=hl, D=D)
            self.host.update(q=q, k=k, v=v)
            self.fused = torch.empty((B, S, 3, H, D), dtype=torch.bfloat16, device="cuda")
            for t, x in enumerate((q, k, v)):
                self.fused[:, :, t, :hl] = to_dev(x)
                self.fused[:, :, t, hl:] = stand_in((B, S, H - hl, D), w["seed"] * 100 + t)
            del q, k, v
        elif name in ("ltx2", "ltx2_fp8", "tiny", "wan"):
            if name in ("ltx2", "ltx2_fp8"):
                q, k, v = synth.ltx2_qkv(seed=w["seed"], S=S, H=H, D=D)
                fused = np.stack([q, k, v], axis=2)          # [B,S,3,H,D], the projection's layout
                del q, k, v
            elif name == "tiny":
                q, k, v = synth.tiny_qkv(seed=w["seed"], S=S, H=H, D=D)
                fused = np.stack([q, k, v], axis=2)
            else:
                fused = synth.fused_qkv(B, S, H, D, seed=w["seed"])
            self.host["fused"] = fused
            self.fused = to_dev(fused)
        self.has_relayout = name in ("cosmos", "ltx2", "ltx2_fp8", "tiny", "wan")
        if self.has_relayout:
            P = w["P"]
            S_loc = S // P
            self.src = [[self.fused[:, p * S_loc:(p + 1) * S_loc, t] for p in range(P)] for t in range(3)]
            hl = H // P
            self.qkv = [torch.empty((B, S, hl, D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
            if not w.get("fp8"):  # the relayout writes V token-contiguous, the layout attention stages directly
                self.qkv[2] = lsd.v_token_major(B, S, hl, D)
            self.Hq = hl
        elif name in ("ring", "ring_stream"):
            q, k, v = synth.qkv(B, S, 3 * S, H, D, seed=w["seed"])
            self.host.update(q=q, k=k, v=v)
            self.qkv = [to_dev(q), to_dev(k), token_major(to_dev(v))]
            self.Hq = H
        elif name == "ltx2_varlen":
            q, k, v = synth.qkv(B, S, S, H, D, seed=w["seed"])
            for b, n in enumerate(w["kv_lens"]):
                k[b, n:] = 0x7FC1                               # padding: any read would poison O
                v[b, n:] = 0x7FC1
            self.host.update(q=q, k=k, v=v)
            self.qkv = [to_dev(q), to_dev(k), token_major(to_dev(v))]
            self.Hq = H
        Hq = self.Hq
        self.S_q = self.qkv[0].shape[1]
        self.S_kv = self.qkv[1].shape[1]
        nb = w["kv_blocks"]
        self.bounds = [(i * self.S_kv // nb, (i + 1) * self.S_kv // nb) for i in range(nb)]
        self.o_parts = [torch.empty((B, self.S_q, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(nb)]
        self.lse_parts = [torch.empty((B, Hq, self.S_q), dtype=torch.float32, device="cuda") for _ in range(nb)]
        if nb > 1:
            self.o = torch.empty((B, self.S_q, Hq, D), dtype=torch.bfloat16, device="cuda")
            self.lse = torch.empty((B, Hq, self.S_q), dtype=torch.float32, device="cuda")
        self.fp8 = bool(w.get("fp8"))
        if self.fp8:
            self.fp8_bufs = lsd.fp8_buffers(B, self.qkv[0].shape[1], self.qkv[0].shape[2], D)
            # two passes over the bf16 inputs (amax, then codes) and one byte per element out
            self.cast_bytes = 3 * B * self.qkv[0].shape[1] * self.qkv[0].shape[2] * D * (2 + 2 + 1)
        self.stream = bool(w.get("stream"))
        self.has_merge = nb > 1 and not self.stream
        if self.stream:
            self.o_acc = torch.empty((B, self.S_q, Hq, D), dtype=torch.float32, device="cuda")
            self.lse_acc = torch.empty((B, Hq, self.S_q), dtype=torch.float32, device="cuda")
            self.o = torch.empty((B, self.S_q, Hq, D), dtype=torch.bfloat16, device="cuda")
        # Ulysses output side: with P > 1 the attention output goes back to
        # sequence shard 0; the other ranks' head slices are seeded stand-ins.
        self.has_inverse = self.has_relayout and w["P"] > 1
        if self.has_inverse:
            P = w["P"]
            self.o_final = self.o if nb > 1 else self.o_parts[0]
            others = [stand_in(self.o_final.shape, w["seed"] * 1000 + 7 + r) for r in range(P - 1)]
            self.inv_src = [[self.o_final] + others]
            self.shard = torch.empty((B, self.S_q // P, P * Hq, D), dtype=torch.bfloat16, device="cuda")
            self.inverse_bytes = 2 * 2 * B * (self.S_q // P) * P * Hq * D
        else:
            self.inverse_bytes = 0
        self.kv_lens = w.get("kv_lens")
        self.kv_lens_dev = (torch.tensor(self.kv_lens, dtype=torch.int32, device="cuda")
                            if self.kv_lens is not None else None)
        n_keys = sum(self.kv_lens) if self.kv_lens is not None else B * self.S_kv
        self.flops = 4.0 * Hq * self.S_q * n_keys * D
        n_rel = 3 * B * self.S_q * Hq * D
        self.relayout_bytes = 2 * 2 * n_rel if self.has_relayout else 0
        o_bytes = 2 * B * self.S_q * Hq * D
        l_bytes = 4 * B * Hq * self.S_q
        self.merge_bytes = (nb + 1) * (o_bytes + l_bytes) if self.has_merge else 0
        if self.kv_lens is not None:
            self.attn_flops_per_launch = [self.flops]
        else:
            self.attn_flops_per_launch = [4.0 * B * Hq * self.S_q * (hi - lo) * D for lo, hi in self.bounds]

    def step(self, ev=None):
        """One pass; if ev is given, record start/end events around each kernel."""
        lsd = self.lsd
        k = 0

        def mark():
            nonlocal k
            if ev is not None:
                ev[k].record()
            k += 1
        if self.has_relayout:
            mark()
            lsd.relayout_seq_to_head(self.src, self.w["P"], 0, dst=self.qkv)
            mark()
        q, kk, v = self.qkv
        if self.fp8:
            mark()
            q8, k8, v8, amax = lsd.cast_qkv_fp8(q, kk, v, out=self.fp8_bufs)
            mark()
            mark()
            lsd.attn_fwd_fp8(q8, k8, v8, amax[0], amax[1], amax[2], o=self.o_parts[0], lse=self.lse_parts[0])
            mark()
            return k
        if self.stream:
            self.lse_acc.fill_(float("-inf"))          # no history yet
        for i, (lo, hi) in enumerate(self.bounds):
            mark()
            if self.stream:
                last = i == len(self.bounds) - 1
                lsd.attn_fwd_accumulate(q, kk[:, lo:hi], v[:, lo:hi], self.o_acc, self.lse_acc,
                                        o=self.o if last else None)
            else:
                lsd.attn_fwd(q, kk[:, lo:hi], v[:, lo:hi], o=self.o_parts[i], lse=self.lse_parts[i],
                             kv_lens=self.kv_lens_dev)
            mark()
        if self.has_merge:
            mark()
            lsd.attn_merge(self.o_parts, self.lse_parts, o=self.o, lse=self.lse)
            mark()
        if self.has_inverse:
            mark()
            lsd.relayout_head_to_seq(self.inv_src, self.w["P"], 0, dst=[self.shard])
            mark()
        return k

    def release_device(self):
        """Drop every device tensor of the step (the host inputs stay, for the
        CPU baseline)."""
        import torch

        def on_gpu(x):
            if isinstance(x, torch.Tensor):
                return x.is_cuda
            if isinstance(x, (list, tuple)):
                return any(on_gpu(y) for y in x)
            return False
        for k in [k for k, x in vars(self).items() if on_gpu(x)]:
            setattr(self, k, None)

    def kernel_names(self):
        names = ["relayout"] if self.has_relayout else []
        if self.fp8:
            return names + ["cast_fp8", "attn_fwd"]
        names += ["attn_fwd"] * len(self.bounds)
        if self.has_merge:
            names.append("attn_merge")
        if self.has_inverse:
            names.append("relayout_inv")
        return names

    def n_events(self):
        return 2 * len(self.kernel_names())


# --------------------------------------------------------------------------
# Timing helpers: HIP events recorded on the current stream, which is the
# stream every library call is enqueued on.
# --------------------------------------------------------------------------

def time_launches(fn, warmup, iters):
    """Durations (ms) of `iters` launches of fn after `warmup` untimed ones."""
    import torch
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def rate_entry(ms, work, kind, peak, warmup, **extra):
    """Median/min/mean durations and the rate and fraction of peak at the
    median (and at the fastest launch).  kind 'flop' -> TFLOP/s, 'bytes' -> GB/s."""
    ms = np.asarray(ms, dtype=np.float64)
    med, mn, mean = float(np.median(ms)), float(ms.min()), float(ms.mean())
    if kind == "flop":
        r_med, r_min = work / (med * 1e-3) / 1e12, work / (mn * 1e-3) / 1e12
        d = {"flop": work, "TFLOP/s": round(r_med, 1), "TFLOP/s_best": round(r_min, 1)}
    else:
        r_med, r_min = work / (med * 1e-3) / 1e9, work / (mn * 1e-3) / 1e9
        d = {"bytes": int(work), "GB/s": round(r_med, 1), "GB/s_best": round(r_min, 1)}
    out = {"median_ms": round(med, 4), "min_ms": round(mn, 4), "mean_ms": round(mean, 4),
           "warmup": warmup, "iters": int(ms.size)}
    out.update(d)
    out["frac_peak"] = round(r_med / peak, 4)
    out["frac_peak_best"] = round(r_min / peak, 4)
    out.update(extra)
    return out


def attn_leg(fn, flop, peak=PEAK_BF16_TFLOPS, **extra):
    return rate_entry(time_launches(fn, ATTN_WARMUP, ATTN_ITERS), flop, "flop", peak, ATTN_WARMUP, **extra)


def hbm_leg(fn, nbytes, **extra):
    return rate_entry(time_launches(fn, HBM_WARMUP, HBM_ITERS), nbytes, "bytes", PEAK_HBM_GBS, HBM_WARMUP, **extra)


def free_gpu():
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def leg_wan():
    """Wan 2.2 A14B Ulysses share (B=2, S=75,600, 40 heads, P=4): the forward
    relayout from the strided fused QKV for every rank, attention on rank 0's
    head slice, the inverse relayout for every shard."""
    import torch
    import synth
    import long_sequence_dit_amd as lsd
    B, S, H, D, P = 2, 75_600, 40, 128, 4
    S_loc, hl = S // P, H // P
    f = to_dev(synth.fused_qkv(B, S, H, D, seed=2))
    src = [[f[:, p * S_loc:(p + 1) * S_loc, t] for p in range(P)] for t in range(3)]
    qkv = [torch.empty((B, S, hl, D), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    qkv.append(lsd.v_token_major(B, S, hl, D))
    rel_bytes = 2 * 2 * 3 * B * S * hl * D
    out = {"workload": "fused QKV [2,75600,3,40,128] (seed 2) -> relayout P=4 (Q, K, V in one launch, V "
                       "token-contiguous) per rank -> attention [2,75600,10,128] with fp32 LSE -> inverse relayout "
                       "of O per shard"}
    per_rank = {}
    for r in range(P):
        per_rank[str(r)] = hbm_leg(lambda: lsd.relayout_seq_to_head(src, P, r, dst=qkv), rel_bytes)
    out["relayout"] = {"per_rank": per_rank,
                       "mean_over_ranks_median_ms": round(float(np.mean([v["median_ms"] for v in per_rank.values()])), 4),
                       "worst_rank_frac_peak": min(v["frac_peak"] for v in per_rank.values())}
    lsd.relayout_seq_to_head(src, P, 0, dst=qkv)
    o = torch.empty((B, S, hl, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hl, S), dtype=torch.float32, device="cuda")
    flop = 4.0 * B * hl * S * S * D
    out["attn_fwd"] = attn_leg(lambda: lsd.attn_fwd(*qkv, o=o, lse=lse), flop)
    del f, src, qkv
    free_gpu()
    inv_src = [[o] + [stand_in(o.shape, 2007 + r) for r in range(P - 1)]]
    shard = torch.empty((B, S_loc, P * hl, D), dtype=torch.bfloat16, device="cuda")
    inv_bytes = 2 * 2 * B * S_loc * P * hl * D
    per_shard = {}
    for p in range(P):
        per_shard[str(p)] = hbm_leg(lambda: lsd.relayout_head_to_seq(inv_src, P, p, dst=[shard]), inv_bytes)
    out["relayout_inv"] = {"per_shard": per_shard,
                           "worst_shard_frac_peak": min(v["frac_peak"] for v in per_shard.values())}
    return out


def leg_ring():
    """Ring/Attention2D one-GPU share: Q [1,25200,40,128] against three K/V
    blocks of 25,200; the merge of the three (O, LSE) partials; the unblocked
    pass; the fused streaming Ring steps."""
    import torch
    import synth
    import long_sequence_dit_amd as lsd
    B, Sb, H, D = 1, 25_200, 40, 128
    q, k, v = synth.qkv(B, Sb, 3 * Sb, H, D, seed=3)
    dq, dk, dvn = to_dev(q), to_dev(k), to_dev(v)
    dv = token_major(dvn)
    del q, k, v
    out = {"workload": "Q [1,25200,40,128] vs K/V [1,75600,40,128] (seed 3, V token-contiguous) as 3 blocks of "
                       "25200: 3 x attention with fp32 LSE -> merge (n=3); unblocked attention; 3 fused Ring steps "
                       "(attn_fwd_accumulate into a running fp32 (O, LSE), bf16 O on the last)"}
    parts = [torch.empty((B, Sb, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    lses = [torch.empty((B, H, Sb), dtype=torch.float32, device="cuda") for _ in range(3)]
    flop_blk = 4.0 * B * H * Sb * Sb * D
    blocks = {}
    for i in range(3):
        blocks[str(i)] = attn_leg(lambda: lsd.attn_fwd(dq, dk[:, i * Sb:(i + 1) * Sb], dv[:, i * Sb:(i + 1) * Sb],
                                                       o=parts[i], lse=lses[i]), flop_blk)
    out["attn_fwd_blocks"] = blocks
    om = torch.empty((B, Sb, H, D), dtype=torch.bfloat16, device="cuda")
    lm = torch.empty((B, H, Sb), dtype=torch.float32, device="cuda")
    merge_bytes = 4 * (2 * B * Sb * H * D + 4 * B * H * Sb)
    out["attn_merge"] = hbm_leg(lambda: lsd.attn_merge(parts, lses, o=om, lse=lm), merge_bytes, n=3)
    out["attn_fwd_unblocked"] = attn_leg(lambda: lsd.attn_fwd(dq, dk, dv, o=om, lse=lm), 3 * flop_blk)
    o_acc = torch.empty((B, Sb, H, D), dtype=torch.float32, device="cuda")
    lse_acc = torch.full((B, H, Sb), float("-inf"), dtype=torch.float32, device="cuda")
    steps = {}
    for i in range(3):
        if i == 0:
            def fn():
                lse_acc.fill_(float("-inf"))  # first step: no history (a tiny fill kernel, inside the events)
                lsd.attn_fwd_accumulate(dq, dk[:, :Sb], dv[:, :Sb], o_acc, lse_acc)
        else:
            def fn(i=i):
                lsd.attn_fwd_accumulate(dq, dk[:, i * Sb:(i + 1) * Sb], dv[:, i * Sb:(i + 1) * Sb], o_acc, lse_acc,
                                        o=om if i == 2 else None)
        steps[str(i)] = attn_leg(fn, flop_blk)
    out["attn_fwd_accumulate_steps"] = steps
    ring_ms = sum(b["median_ms"] for b in blocks.values()) + out["attn_merge"]["median_ms"]
    stream_ms = sum(s["median_ms"] for s in steps.values())
    out["ring_step_ms"] = {"blocks_plus_merge": round(ring_ms, 4), "fused_streaming": round(stream_ms, 4),
                           "TFLOP/s_blocks_plus_merge": round(3 * flop_blk / (ring_ms * 1e-3) / 1e12, 1),
                           "TFLOP/s_fused_streaming": round(3 * flop_blk / (stream_ms * 1e-3) / 1e12, 1)}
    # The same share on the FP8 path: Q cast once, each K/V block cast with its
    # own scales, K's chosen against Q's (lsd_cast_kv_fp8) so that every
    # block's logit factor is a power of two, then either three FP8 attentions
    # and the merge, or three fused FP8 Ring steps.
    qb = lsd.fp8_buffers(B, Sb, H, D)
    lsd.cast_qkv_fp8(dq, dq, dq, out=qb)
    kvb = []
    for i in range(3):
        bb = lsd.fp8_buffers(B, Sb, H, D)
        lsd.cast_kv_fp8(dk[:, i * Sb:(i + 1) * Sb], dvn[:, i * Sb:(i + 1) * Sb], qb[3][0], out=bb)
        kvb.append(bb)
    q8, aq = qb[0], qb[3]
    f8_blocks, f8_steps = {}, {}
    for i in range(3):
        bb = kvb[i]
        f8_blocks[str(i)] = attn_leg(lambda bb=bb, i=i: lsd.attn_fwd_fp8(q8, bb[1], bb[2], aq[0], bb[3][1], bb[3][2],
                                                                         o=parts[i], lse=lses[i]),
                                     flop_blk, peak=PEAK_FP8_TFLOPS)
    for i in range(3):
        bb = kvb[i]
        if i == 0:
            def fn(bb=bb):
                lse_acc.fill_(float("-inf"))
                lsd.attn_fwd_fp8_accumulate(q8, bb[1], bb[2], aq[0], bb[3][1], bb[3][2], o_acc, lse_acc)
        else:
            def fn(bb=bb, i=i):
                lsd.attn_fwd_fp8_accumulate(q8, bb[1], bb[2], aq[0], bb[3][1], bb[3][2], o_acc, lse_acc,
                                            o=om if i == 2 else None)
        f8_steps[str(i)] = attn_leg(fn, flop_blk, peak=PEAK_FP8_TFLOPS)
    f8_ring = sum(b["median_ms"] for b in f8_blocks.values()) + out["attn_merge"]["median_ms"]
    f8_stream = sum(x["median_ms"] for x in f8_steps.values())
    out["fp8"] = {"workload": "the same share with Q and each K/V block cast to FP8 (E4M3, per-block scales, K's "
                              "chosen against Q's): 3 x FP8 attention -> merge (n=3), or 3 fused FP8 Ring steps",
                  "attn_fwd_fp8_blocks": f8_blocks, "attn_fwd_fp8_accumulate_steps": f8_steps,
                  "ring_step_ms": {"blocks_plus_merge": round(f8_ring, 4), "fused_streaming": round(f8_stream, 4),
                                   "TFLOP/s_blocks_plus_merge": round(3 * flop_blk / (f8_ring * 1e-3) / 1e12, 1),
                                   "TFLOP/s_fused_streaming": round(3 * flop_blk / (f8_stream * 1e-3) / 1e12, 1)}}
    return out


def leg_ltx2(fp8=False):
    """LTX-2 scale attention [1,24576,32,128] (Q/K RMS-normalised) over all
    24,576 keys, bf16 (V token-contiguous) or on the FP8 path (cast + FP8
    attention)."""
    import torch
    import synth
    import long_sequence_dit_amd as lsd
    B, S, H, D = 1, 24_576, 32, 128
    q, k, v = synth.ltx2_qkv(seed=1, S=S, H=H, D=D)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    del q, k, v
    o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    flop = 4.0 * B * H * S * S * D
    if not fp8:
        dvt = token_major(dv)
        return {"workload": "Q,K,V [1,24576,32,128] (seed 1, Q/K RMS-normalised, V token-contiguous), one pass "
                            "over all keys with fp32 LSE",
                "attn_fwd": attn_leg(lambda: lsd.attn_fwd(dq, dk, dvt, o=o, lse=lse), flop)}
    bufs = lsd.fp8_buffers(B, S, H, D)
    cast_bytes = 3 * B * S * H * D * (2 + 2 + 1)
    cast = hbm_leg(lambda: lsd.cast_qkv_fp8(dq, dk, dv, out=bufs), cast_bytes, launches=4)
    q8, k8, v8, amax = bufs
    att = attn_leg(lambda: lsd.attn_fwd_fp8(q8, k8, v8, amax[0], amax[1], amax[2], o=o, lse=lse), flop,
                   peak=PEAK_FP8_TFLOPS)
    return {"workload": "Q,K,V [1,24576,32,128] (seed 1, Q/K RMS-normalised) -> one FP8 (E4M3) cast with "
                        "per-head scales -> FP8 attention over all keys with fp32 LSE",
            "cast_fp8": cast, "attn_fwd_fp8": att}


def kernel_source_hash(name):
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "long_sequence_dit_amd", "csrc", name), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM traffic per attention launch from committed rocprofv3 counter runs,
    or None when absent or taken on a different attention kernel source."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    src = d.get("source_file")
    if src is None or d.get("attn_source_sha256_16") != kernel_source_hash(src):
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(pipe, budget_s):
    """Time the float64 oracle on a bounded sample of this workload's step and
    extrapolate to one full step (attention rows scale linearly)."""
    from oracle import ref
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    w = pipe.w
    B, D, Hq = w["B"], w["D"], pipe.Hq
    h = pipe.host
    g = np.random.Generator(np.random.PCG64(123))
    t_rel = 0.0
    rel_note = ""
    if "fused" in h:
        f = h["fused"]
        P = w["P"]
        S_loc = w["S"] // P
        # relayout: the oracle's copy over every tensor, timed in full
        t0 = time.perf_counter()
        chunks = [[f[:, p * S_loc:(p + 1) * S_loc, t] for p in range(P)] for t in range(3)]
        qkv = [ref.relayout_seq_to_head(c, P, 0) for c in chunks]
        t_rel = time.perf_counter() - t0
        rel_note = f"; relayout timed in full ({t_rel:.2f} s)"
        q, k, v = qkv
    else:
        q, k, v = h["q"], h["k"], h["v"]
        if pipe.has_relayout:
            # relayout: the oracle's copy over a slab of 4096 tokens of a stand-in
            # fused buffer of the same head count, scaled to the sequence
            P = w["P"]
            slab = 4096
            fs = g.integers(0, 1 << 16, size=(B, slab, 3, w["H"], D), dtype=np.uint16)
            t0 = time.perf_counter()
            for t in range(3):
                ref.relayout_seq_to_head([fs[:, p * slab // P:(p + 1) * slab // P, t] for p in range(P)], P, 0)
            t_rel = (time.perf_counter() - t0) * w["S"] / slab
            rel_note = f"; relayout timed on a {slab}-token slab, scaled ({t_rel:.2f} s)"
            del fs
    # FP8 path: the oracle's cast of two heads (scaled to all heads), whose codes
    # then feed the attention sample
    t_cast = 0.0
    heads = [(b, hh) for b in range(B) for hh in range(Hq)]
    if pipe.fp8:
        from oracle import fp8 as ofp8
        nh = min(2, Hq)
        t0 = time.perf_counter()
        c8 = ofp8.cast_qkv(q[:1, :, :nh], k[:1, :, :nh], v[:1, :, :nh])
        t_cast = (time.perf_counter() - t0) * (B * Hq) / nh
        heads = [(0, hh) for hh in range(nh)]
    # attention: chunks of 256 query rows, cycling over (b, h), until the budget
    rows_done = 0
    t_attn = 0.0
    i = 0
    while t_attn < budget_s and i < 64 * len(heads):
        b, hh = heads[i % len(heads)]
        r0 = int(g.integers(0, max(1, pipe.S_q - 256)))
        rows = np.arange(r0, min(pipe.S_q, r0 + 256))
        t0 = time.perf_counter()
        if pipe.fp8:
            ofp8.attention_fp8_rows(c8[0], c8[1], c8[2], c8[3][0], c8[3][1], c8[3][2], b, hh, rows)
        else:
            ref.attention_rows(q, k, v, b, hh, rows, kv_lens=pipe.kv_lens)
        t_attn += time.perf_counter() - t0
        rows_done += rows.size
        i += 1
    total_rows = B * Hq * pipe.S_q
    t_attn_full = t_attn * total_rows / rows_done
    # merge: the oracle's merge on a slab of sequence positions, scaled
    t_merge_full = 0.0
    if pipe.has_merge:
        nb = len(pipe.bounds)
        S_slab = min(pipe.S_q, 512)
        parts = [np.asarray(g.standard_normal((B, S_slab, Hq, D))) for _ in range(nb)]
        lses = [np.asarray(g.standard_normal((B, Hq, S_slab))) for _ in range(nb)]
        t0 = time.perf_counter()
        ref.merge(parts, lses)
        t_merge_full = (time.perf_counter() - t0) * pipe.S_q / S_slab
    # inverse relayout: the oracle's copy over P stand-in head slices (a slab
    # of at most 16384 tokens, scaled)
    t_inv = 0.0
    if pipe.has_inverse:
        P = w["P"]
        S_slab = min(pipe.S_q, 16384) // P * P
        slices = [np.full((B, S_slab, Hq, D), r, dtype=np.uint16) for r in range(P)]
        t0 = time.perf_counter()
        ref.relayout_head_to_seq(slices, P, 0)
        t_inv = (time.perf_counter() - t0) * pipe.S_q / S_slab
        del slices
    t_step = t_rel + t_cast + t_attn_full + t_merge_full + t_inv
    return {
        "value": pipe.flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(min(cores, blas_threads) if blas_threads > 1 else 1),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle: {rows_done} query rows of attention against all {pipe.S_kv} keys "
                   f"({t_attn:.1f} s), extrapolated to {total_rows} rows"
                   + rel_note
                   + (f"; merge timed on a {min(pipe.S_q, 512)}-position slab, scaled" if pipe.has_merge else "")
                   + (f"; inverse relayout timed on a slab, scaled ({t_inv:.2f} s)" if pipe.has_inverse else "")
                   + (f"; FP8 cast timed on 2 heads, scaled ({t_cast:.2f} s); attention rows on their codes"
                      if pipe.fp8 else "")
                   + f"; extrapolated step {t_step:.1f} s; host has {cores} cores, BLAS threads {blas_threads}"),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py: measures one GPU's share of the sequence-parallel work (asked for --gpus {args.gpus}); "
              "the collectives between GPUs are not implemented, so only --gpus 1 runs", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n}), flush=True)
        return
    import long_sequence_dit_amd as lsd
    lsd.lib()
    w = WORKLOADS[args.workload]
    print(f"bench.py: step workload {args.workload}", file=sys.stderr, flush=True)
    pipe = Pipeline(args.workload, w)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        pipe.step()
    torch.cuda.synchronize()

    ne = pipe.n_events()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ne)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        pipe.step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps

    # per-kernel durations from the events (same stream as the kernels)
    names = pipe.kernel_names()
    dur = {n: [] for n in set(names)}
    attn_flops = []
    for s in range(args.steps):
        ai = 0
        for j, n in enumerate(names):
            ms = evs[s][2 * j].elapsed_time(evs[s][2 * j + 1])
            dur[n].append(ms)
            if n == "attn_fwd":
                attn_flops.append(pipe.attn_flops_per_launch[ai])
                ai += 1
    peak = PEAK_FP8_TFLOPS if pipe.fp8 else PEAK_BF16_TFLOPS
    attn_ms = float(np.mean(dur["attn_fwd"]))
    flops_per_launch = float(np.mean(pipe.attn_flops_per_launch))
    kernels = {"attn_fwd": rate_entry(dur["attn_fwd"], flops_per_launch, "flop", peak, args.warmup,
                                      launches_per_step=len(pipe.bounds))}
    for key, nbytes, extra in (("cast_fp8", getattr(pipe, "cast_bytes", 0), {"launches": 4}),
                               ("relayout", pipe.relayout_bytes, {}), ("attn_merge", pipe.merge_bytes, {}),
                               ("relayout_inv", pipe.inverse_bytes, {})):
        if key in dur:
            kernels[key] = rate_entry(dur[key], nbytes, "bytes", PEAK_HBM_GBS, args.warmup, **extra)

    traffic = load_traffic(args.workload)
    out = {
        "metric": METRIC,
        "value": round(pipe.flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if pipe.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w["desc"], "B": w["B"], "S_q": pipe.S_q, "S_kv": pipe.S_kv, "H": pipe.Hq,
                   "D": w["D"], "kv_blocks": w["kv_blocks"], "fused_merge": pipe.stream,
                   "v_layout": "token-contiguous" if pipe.qkv[2].stride(1) == 1 else "natural",
                   "flop_per_step": pipe.flops},
        "roofline": {"bound": "mfma", "achieved": round(flops_per_launch / (attn_ms * 1e-3) / 1e12, 1),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(flops_per_launch / (attn_ms * 1e-3) / 1e12 / peak, 4),
                     "traffic": traffic, "kernel": "attn_fwd",
                     "flop_per_launch": flops_per_launch, "avg_launch_ms": round(attn_ms, 4)},
        "kernels": kernels,
    }
    if args.legs:
        pipe.release_device()   # the step's buffers go before the legs allocate theirs
        del evs
        free_gpu()
        legs = {}
        for name in args.legs:
            print(f"bench.py: leg {name}", file=sys.stderr, flush=True)
            if name == "wan":
                legs["wan"] = leg_wan()
            elif name == "ring":
                legs["ring"] = leg_ring()
            elif name == "ltx2":
                legs["ltx2"] = leg_ltx2()
            elif name == "ltx2_fp8":
                legs["ltx2_fp8"] = leg_ltx2(fp8=True)
            free_gpu()
        out["legs"] = legs
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(pipe, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
