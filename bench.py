#!/usr/bin/env python3
"""Benchmark of the long-sequence DiT attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM.  Default workload (LTX-2 scale, B=1, S=24,576, H=32,
D=128):

  fused QKV projection output [1, S, 3, 32, 128] (seq-major)
    -> relayout_seq_to_head (Q, K, V in one launch, P = 1: strided views ->
       head-major contiguous tensors)
    -> attn_fwd of Q against the two halves of K/V, each with its fp32 LSE
    -> attn_merge of the two (O, LSE) partials into the exact full result

Prints ONE JSON line.  ``value`` is whole-step throughput in attention TFLOP/s
(4*B*H*S_q*S_kv*D per step / step time).  ``roofline`` is measured live for
the dominant kernel (attention) with HIP events on the stream it runs on;
``kernels`` has the same for the relayout and merge kernels (GB/s against HBM
peak); ``cpu_baseline`` times the float64 CPU oracle on a bounded sample of
the same work on this host and extrapolates it to one step.

Other workloads (--workload): wan (Ulysses share: relayout P=4 -> attention ->
inverse relayout of the output back to this rank's sequence shard), ring
(three K/V blocks + merge), cosmos (S=150,000), tiny.
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

WORKLOADS = {
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
    "cosmos": dict(desc="Cosmos3-Super share: Q,K,V [1,150000,16,128], 1% of keys x4, with fp32 LSE", B=1,
                   S=150_000, H=16, D=128, P=None, kv_blocks=1, seed=4),
    "tiny": dict(desc="tiny: fused QKV [1,256,3,2,64] -> relayout (P=1) -> attention over 4 K/V chunks -> merge",
                 B=1, S=256, H=2, D=64, P=1, kv_blocks=4, seed=0),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ltx2", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (scale for HBM byte counters)")
    return ap.parse_args()


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


class Pipeline:
    """Device tensors and the launch sequence of one step."""

    def __init__(self, name, w):
        import torch
        import synth
        import long_sequence_dit_amd as lsd
        self.lsd, self.torch, self.name, self.w = lsd, torch, name, w
        B, S, H, D = w["B"], w["S"], w["H"], w["D"]
        self.host = {}
        if name in ("ltx2", "ltx2_fp8", "tiny", "wan"):
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
        else:  # cosmos
            q, k, v, _ = synth.cosmos_qkv(seed=w["seed"], S=S, H=H, D=D)
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
        self.has_relayout = name in ("ltx2", "ltx2_fp8", "tiny", "wan")
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
            g = torch.Generator(device="cuda")
            g.manual_seed(w["seed"] * 1000 + 7)
            self.o_final = self.o if nb > 1 else self.o_parts[0]
            others = [torch.randn(self.o_final.shape, generator=g, device="cuda", dtype=torch.float32)
                      .to(torch.bfloat16) for _ in range(P - 1)]
            self.inv_src = [[self.o_final] + others]
            self.shard = torch.empty((B, self.S_q // P, P * Hq, D), dtype=torch.bfloat16, device="cuda")
            self.inverse_bytes = 2 * 2 * B * (self.S_q // P) * P * Hq * D
        else:
            self.inverse_bytes = 0
        B_, D_ = B, D
        self.kv_lens = w.get("kv_lens")
        self.kv_lens_dev = (torch.tensor(self.kv_lens, dtype=torch.int32, device="cuda")
                            if self.kv_lens is not None else None)
        n_keys = sum(self.kv_lens) if self.kv_lens is not None else B_ * self.S_kv
        self.flops = 4.0 * Hq * self.S_q * n_keys * D_
        n_rel = 3 * B_ * self.S_q * Hq * D_
        self.relayout_bytes = 2 * 2 * n_rel if self.has_relayout else 0
        o_bytes = 2 * B_ * self.S_q * Hq * D_
        l_bytes = 4 * B_ * Hq * self.S_q
        self.merge_bytes = (nb + 1) * (o_bytes + l_bytes) if self.has_merge else 0
        if self.kv_lens is not None:
            self.attn_flops_per_launch = [self.flops]
        else:
            self.attn_flops_per_launch = [4.0 * B_ * Hq * self.S_q * (hi - lo) * D_ for lo, hi in self.bounds]

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
    if "fused" in h:
        f = h["fused"]
        P = w["P"]
        S_loc = w["S"] // P
        # relayout: the oracle's copy over every tensor, timed in full
        t0 = time.perf_counter()
        chunks = [[f[:, p * S_loc:(p + 1) * S_loc, t] for p in range(P)] for t in range(3)]
        qkv = [ref.relayout_seq_to_head(c, P, 0) for c in chunks]
        t_rel = time.perf_counter() - t0
        q, k, v = qkv
    else:
        t_rel = 0.0
        q, k, v = h["q"], h["k"], h["v"]
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
    g = np.random.Generator(np.random.PCG64(123))
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
    # inverse relayout: the oracle's copy over P stand-in head slices, timed in full
    t_inv = 0.0
    if pipe.has_inverse:
        P = w["P"]
        slices = [np.full((B, pipe.S_q, Hq, D), r, dtype=np.uint16) for r in range(P)]
        t0 = time.perf_counter()
        ref.relayout_head_to_seq(slices, P, 0)
        t_inv = time.perf_counter() - t0
        del slices
    t_step = t_rel + t_cast + t_attn_full + t_merge_full + t_inv
    return {
        "value": pipe.flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(min(cores, blas_threads) if blas_threads > 1 else 1),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle: {rows_done} query rows of attention against all {pipe.S_kv} keys "
                   f"({t_attn:.1f} s), extrapolated to {total_rows} rows"
                   + (f"; relayout timed in full ({t_rel:.2f} s)" if t_rel else "")
                   + (f"; merge timed on a {min(pipe.S_q, 512)}-position slab, scaled" if pipe.has_merge else "")
                   + (f"; inverse relayout timed in full ({t_inv:.2f} s)" if pipe.has_inverse else "")
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
    attn_tflops = float(np.sum(attn_flops) / (np.sum(dur["attn_fwd"]) * 1e-3)) / 1e12
    kernels = {"attn_fwd": {"launches_per_step": len(pipe.bounds), "avg_ms": round(attn_ms, 4),
                            "TFLOP/s": round(attn_tflops, 1), "frac_mfma_peak": round(attn_tflops / peak, 4)}}
    if pipe.fp8:
        ms = float(np.mean(dur["cast_fp8"]))
        gbs = pipe.cast_bytes / (ms * 1e-3) / 1e9
        kernels["cast_fp8"] = {"avg_ms": round(ms, 4), "bytes": pipe.cast_bytes, "GB/s": round(gbs, 1),
                               "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "launches": 3}
    if pipe.has_relayout:
        ms = float(np.mean(dur["relayout"]))
        gbs = pipe.relayout_bytes / (ms * 1e-3) / 1e9
        kernels["relayout"] = {"avg_ms": round(ms, 4), "bytes": pipe.relayout_bytes, "GB/s": round(gbs, 1),
                               "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    if pipe.has_merge:
        ms = float(np.mean(dur["attn_merge"]))
        gbs = pipe.merge_bytes / (ms * 1e-3) / 1e9
        kernels["attn_merge"] = {"avg_ms": round(ms, 4), "bytes": pipe.merge_bytes, "GB/s": round(gbs, 1),
                                 "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    if pipe.has_inverse:
        ms = float(np.mean(dur["relayout_inv"]))
        gbs = pipe.inverse_bytes / (ms * 1e-3) / 1e9
        kernels["relayout_inv"] = {"avg_ms": round(ms, 4), "bytes": pipe.inverse_bytes, "GB/s": round(gbs, 1),
                                   "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}

    traffic = load_traffic(args.workload)
    flops_per_launch = float(np.mean(pipe.attn_flops_per_launch))
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
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(pipe, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
