"""relayout_seq_to_head and relayout_head_to_seq on the GPU (through the C
ABI): bit-exact against the oracle on random 16-bit patterns (NaN payloads,
infinities and -0 included), and the GPU round trip returns every byte."""

import numpy as np
import pytest

import synth
from oracle import ref
from gpu_util import note, to_bits, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

lsd = pytest.importorskip("long_sequence_dit_amd")


@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("n_tensors", [1, 3])
def test_all_ranks_bit_exact(P, n_tensors):
    note(f"relayout P={P} n_tensors={n_tensors}")
    t = torch()
    B, S_loc, H, D = 2, 37, 8, 128
    host = [[synth.random_bits16((B, S_loc, H, D), 1000 * tt + 10 * P + p) for p in range(P)]
            for tt in range(n_tensors)]
    dev = [[to_dev(x) for x in row] for row in host]
    for r in range(P):
        outs = lsd.relayout_seq_to_head(dev, P, r)
        t.cuda.synchronize()
        for tt in range(n_tensors):
            assert np.array_equal(to_bits(outs[tt]), ref.relayout_seq_to_head(host[tt], P, r))


def test_fused_qkv_strided_source():
    note("relayout fused QKV [2,4*25,3,40,128] -> 3 x [2,100,10,128], P=4")
    t = torch()
    B, S_loc, H, D, P = 2, 25, 40, 128, 4
    host = synth.random_bits16((B, P * S_loc, 3, H, D), 5)
    f = to_dev(host)
    # shard p of tensor t is a strided view into the fused buffer
    src = [[f[:, p * S_loc:(p + 1) * S_loc, tt] for p in range(P)] for tt in range(3)]
    assert src[2][1].stride() == (P * S_loc * 3 * H * D, 3 * H * D, D, 1)
    for r in range(P):
        outs = lsd.relayout_seq_to_head(src, P, r)
        t.cuda.synchronize()
        for tt in range(3):
            chunks = [host[:, p * S_loc:(p + 1) * S_loc, tt] for p in range(P)]
            assert np.array_equal(to_bits(outs[tt]), ref.relayout_seq_to_head(chunks, P, r))


def test_non_contiguous_heads_and_guard_bands():
    note("relayout head-strided destination + guard bands")
    t = torch()
    B, S_loc, H, D, P = 1, 19, 6, 64, 2
    host = [synth.random_bits16((B, S_loc, H, D), 300 + p) for p in range(P)]
    dev = [to_dev(x) for x in host]
    sentinel = -12345
    big = t.full((B, P * S_loc, 2 * (H // P) + 2, D), sentinel, dtype=t.int16, device="cuda")
    dst = big.view(t.bfloat16)[:, :, 1:1 + 2 * (H // P):2]     # every other head slot
    lsd.relayout_seq_to_head([dev], P, 1, dst=[dst])
    t.cuda.synchronize()
    assert np.array_equal(to_bits(dst), ref.relayout_seq_to_head(host, P, 1))
    bb = big.cpu().numpy()
    assert (bb[:, :, 0] == sentinel).all() and (bb[:, :, 2:2 * (H // P) + 1:2] == sentinel).all()
    assert (bb[:, :, -1] == sentinel).all()


def test_round_trip_byte_exact():
    note("relayout round trip (gather(send(x)) == x)")
    t = torch()
    B, S_loc, H, D, P = 2, 33, 12, 128, 4
    host = [synth.random_bits16((B, S_loc, H, D), 400 + p) for p in range(P)]
    dev = [to_dev(x) for x in host]
    ys = []
    for r in range(P):
        ys.append(to_bits(lsd.relayout_seq_to_head([dev], P, r)[0]))
    t.cuda.synchronize()
    for p in range(P):
        assert np.array_equal(ref.relayout_head_to_seq(ys, P, p), host[p])


@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("n_tensors", [1, 3])
def test_inverse_all_ranks_bit_exact(P, n_tensors):
    note(f"relayout_head_to_seq P={P} n_tensors={n_tensors}")
    t = torch()
    B, S_loc, H_loc, D = 2, 23, 3, 128
    host = [[synth.random_bits16((B, P * S_loc, H_loc, D), 5000 + 1000 * tt + 10 * P + r) for r in range(P)]
            for tt in range(n_tensors)]
    dev = [[to_dev(x) for x in row] for row in host]
    for p in range(P):
        outs = lsd.relayout_head_to_seq(dev, P, p)
        t.cuda.synchronize()
        for tt in range(n_tensors):
            assert outs[tt].shape == (B, S_loc, P * H_loc, D)
            assert np.array_equal(to_bits(outs[tt]), ref.relayout_head_to_seq(host[tt], P, p))


def test_gpu_round_trip_byte_exact():
    note("relayout seq->head->seq on the GPU, every rank")
    t = torch()
    B, S_loc, H, D, P = 2, 41, 8, 64, 4
    host = [synth.random_bits16((B, S_loc, H, D), 600 + p) for p in range(P)]
    dev = [to_dev(x) for x in host]
    ys = [lsd.relayout_seq_to_head([dev], P, r)[0] for r in range(P)]
    back = [lsd.relayout_head_to_seq([ys], P, p)[0] for p in range(P)]
    t.cuda.synchronize()
    for p in range(P):
        assert np.array_equal(to_bits(back[p]), host[p])


def test_inverse_strided_views_and_guard_bands():
    note("relayout_head_to_seq strided source + head-strided destination + guard bands")
    t = torch()
    B, S_loc, H_loc, D, P = 1, 17, 2, 64, 3
    # rank slices are views into one wider buffer (every other head slot)
    wide = [to_dev(synth.random_bits16((B, P * S_loc, 2 * H_loc, D), 700 + r)) for r in range(P)]
    src = [w[:, :, ::2] for w in wide]
    host_src = [to_bits(x) for x in src]
    sentinel = -777
    big = t.full((B, S_loc, 2 * P * H_loc + 2, D), sentinel, dtype=t.int16, device="cuda")
    dst = big.view(t.bfloat16)[:, :, 1:1 + 2 * P * H_loc:2]
    lsd.relayout_head_to_seq([src], P, 2, dst=[dst])
    t.cuda.synchronize()
    assert np.array_equal(to_bits(dst), ref.relayout_head_to_seq(host_src, P, 2))
    bb = big.cpu().numpy()
    assert (bb[:, :, 0] == sentinel).all() and (bb[:, :, 2:2 * P * H_loc + 1:2] == sentinel).all()
    assert (bb[:, :, -1] == sentinel).all()


@pytest.mark.parametrize("P,S_loc,D", [(1, 37, 128), (4, 25, 128), (2, 64, 64), (4, 1, 64), (1, 300, 128),
                                         (2, 40, 192), (1, 70, 256)])
def test_token_major_destination(P, S_loc, D):
    note(f"relayout into a token-contiguous V: P={P} S_loc={S_loc} D={D}")
    t = torch()
    B, H = 2, 4 * P
    host = synth.random_bits16((B, P * S_loc, 3, H, D), 77 + P + D)
    f = to_dev(host)
    src = [[f[:, p * S_loc:(p + 1) * S_loc, tt] for p in range(P)] for tt in range(3)]
    S, Hl = P * S_loc, H // P
    sentinel = -4242
    for pitch in ((S + 7) // 8 * 8, (S + 7) // 8 * 8 + 24):
        store = t.full((B, Hl, D, pitch), sentinel, dtype=t.int16, device="cuda")
        vt = store.view(t.bfloat16).permute(0, 3, 1, 2)[:, :S]
        q = t.empty((B, S, Hl, D), dtype=t.bfloat16, device="cuda")
        k = t.empty_like(q)
        for r in range(P):
            lsd.relayout_seq_to_head(src, P, r, dst=[q, k, vt])
            t.cuda.synchronize()
            for tt, out in enumerate((q, k, vt)):
                chunks = [host[:, p * S_loc:(p + 1) * S_loc, tt] for p in range(P)]
                assert np.array_equal(to_bits(out), ref.relayout_seq_to_head(chunks, P, r)), (tt, r, pitch)
            pad = store[..., S:].cpu().numpy()
            assert (pad == sentinel).all(), "row padding written"


def test_token_major_destination_feeds_attention():
    note("relayout with a token-contiguous V, then attention on it")
    t = torch()
    B, S_loc, H, D, P = 1, 200, 4, 128, 2
    f = to_dev(synth.normal_bf16((B, P * S_loc, 3, H, D), 91, 1))
    src = [[f[:, p * S_loc:(p + 1) * S_loc, tt] for p in range(P)] for tt in range(3)]
    q, k, v = lsd.relayout_seq_to_head(src, P, 1)
    vt = lsd.v_token_major(B, P * S_loc, H // P, D)
    q2, k2, vt = lsd.relayout_seq_to_head(src, P, 1, dst=[t.empty_like(q), t.empty_like(k), vt])
    o1, l1 = lsd.attn_fwd(q, k, v)
    o2, l2 = lsd.attn_fwd(q2, k2, vt)
    t.cuda.synchronize()
    assert np.array_equal(to_bits(q), to_bits(q2)) and np.array_equal(to_bits(vt), to_bits(v))
    a, b = to_f64(o1), to_f64(o2)
    assert (np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6).all()
    assert float((l1 - l2).abs().max()) <= 1e-5


@pytest.mark.parametrize("P,S_loc,D", [(2, 19, 64), (4, 33, 128)])
def test_mixed_destinations_one_launch(P, S_loc, D):
    """Q into a head-strided view (one copy run per head), K contiguous and V
    token-contiguous in the same call: the forward call that runs copying and
    transposing workgroups in one launch.  Every destination bit-exact, guard
    slots and row padding untouched."""
    note(f"relayout, mixed destinations in one launch: P={P} S_loc={S_loc} D={D}")
    t = torch()
    B, H = 2, 3 * P
    Hl, S = H // P, P * S_loc
    host = synth.random_bits16((B, S, 3, H, D), 501 + P + D)
    f = to_dev(host)
    src = [[f[:, p * S_loc:(p + 1) * S_loc, tt] for p in range(P)] for tt in range(3)]
    sentinel = -7777
    big = t.full((B, S, 2 * Hl + 2, D), sentinel, dtype=t.int16, device="cuda")
    q = big.view(t.bfloat16)[:, :, 1:1 + 2 * Hl:2]  # every other head slot
    k = t.empty((B, S, Hl, D), dtype=t.bfloat16, device="cuda")
    pitch = (S + 7) // 8 * 8 + 8
    store = t.full((B, Hl, D, pitch), sentinel, dtype=t.int16, device="cuda")
    vt = store.view(t.bfloat16).permute(0, 3, 1, 2)[:, :S]
    for r in range(P):
        lsd.relayout_seq_to_head(src, P, r, dst=[q, k, vt])
        t.cuda.synchronize()
        for tt, out in enumerate((q, k, vt)):
            chunks = [host[:, p * S_loc:(p + 1) * S_loc, tt] for p in range(P)]
            assert np.array_equal(to_bits(out), ref.relayout_seq_to_head(chunks, P, r)), (tt, r)
        bb = big.cpu().numpy()
        assert (bb[:, :, 0] == sentinel).all() and (bb[:, :, 2:2 * Hl + 1:2] == sentinel).all()
        assert (bb[:, :, -1] == sentinel).all()
        assert (store[..., S:].cpu().numpy() == sentinel).all(), "row padding written"
