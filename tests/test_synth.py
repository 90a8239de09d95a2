"""The seeded input generators: bf16 encoding and reproducibility (CPU only)."""

import numpy as np

import synth


def test_rne_encoding_cases():
    f = np.array([1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-40], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(f)
    assert bits[:6].tolist() == [0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80]
    # 3.4e38 rounds past the largest finite bf16 to +inf; 1e-40 stays subnormal
    assert bits[6] == 0x7F80 and 0 < bits[7] < 0x0080
    # exact halfway cases round to the even neighbour
    u = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF], dtype=np.uint32)
    assert synth.f32_to_bf16_bits(u.view(np.float32)).tolist() == [0x3F80, 0x3F82, 0x3F81, 0x3F80]
    nan = synth.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_generation_is_seed_stable_and_chunk_independent():
    a = synth.normal_bf16((3, synth.CHUNK // 2 + 5), 7, 1)
    b = synth.normal_bf16((3, synth.CHUNK // 2 + 5), 7, 1)
    c = synth.normal_bf16((3, synth.CHUNK // 2 + 5), 8, 1)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # the first chunk does not depend on the total size
    d = synth.normal_bf16((synth.CHUNK + 17,), 7, 1)
    e = synth.normal_bf16((synth.CHUNK,), 7, 1)
    assert np.array_equal(d[:synth.CHUNK], e)


def test_distribution_and_workload_structure():
    q, k, v = synth.tiny_qkv()
    assert q.shape == (1, 256, 2, 64) and q.dtype == np.uint16
    x = (q.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(x.mean())) < 0.05 and abs(float(x.std()) - 1.0) < 0.05
    r = synth.rms_normalised_bf16((1, 64, 4, 128), 3, 1)
    rf = (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rms = np.sqrt((rf ** 2).mean(axis=3))
    assert np.allclose(rms, 1.0, atol=1e-2)
    rows = synth.outlier_key_rows(150_000, 0.01, 4)
    assert rows.size == 1500 and np.unique(rows).size == 1500 and rows.max() < 150_000
