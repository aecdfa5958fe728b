"""The seeded input generator: SplitMix64 against its published test vectors, bf16 RNE, determinism."""
import hashlib

import numpy as np

from test_sequence_layers_amd import synth


def test_splitmix64_reference_vectors():
    # Outputs of the reference SplitMix64 (Steele, Lea, Flood 2014; the Java SplittableRandom / Vigna C
    # implementation) for initial states 0 and 1234567.
    assert [int(x) for x in synth.splitmix64(0, 4)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    assert [int(x) for x in synth.splitmix64(1234567, 3)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_splitmix64_is_counter_based():
    full = synth.splitmix64(99, 100)
    assert np.array_equal(full[37:61], synth.splitmix64(99, 24, start=37))


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -7 + 2 ** -8, -2.5, 0.0, -0.0,
                  3.0e38, 1e-40], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-9 rounds up; 1 + 2^-7 + 2^-8 is a tie -> even (1 + 2^-6)
    assert [int(t) for t in b[:5]] == [0x3F80, 0x3F80, 0x3F81, 0x3F82, 0xC020]
    assert int(b[5]) == 0x0000 and int(b[6]) == 0x8000
    back = synth.bf16_bits_to_f32(b)
    assert np.all(np.abs(back[:8] - x[:8]) <= np.abs(x[:8]) * 2.0 ** -8)


def test_bf16_roundtrip_exact_on_representable():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(bits)), bits)


def test_normals_moments():
    n = synth.normals(7, 3, 400001)
    assert abs(n.mean()) < 5e-3 and abs(n.std() - 1.0) < 5e-3
    assert abs(np.mean(n ** 3)) < 2e-2 and abs(np.mean(n ** 4) - 3.0) < 5e-2


def test_inputs_deterministic_and_shaped():
    wl = synth.WORKLOADS["vit3s_fullbatch"].with_(B=2, N=20)
    a, b = synth.make_inputs(wl), synth.make_inputs(wl)
    assert a.q.dtype == np.uint16 and a.q.shape == (2, 20, 6, 64)
    assert a.w0.shape == (6, 64, 64) and a.w0.dtype == np.float32
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.w0, b.w0)]:
        assert np.array_equal(x, y)
    assert not np.array_equal(a.q, a.k)
    # scale: N(0,1)/sqrt(64) and N(0, 0.02^2)
    assert abs(a.q64.std() - 0.125) < 0.01 and abs(a.w0.std() - 0.02) < 0.002


def test_inputs_golden_digest():
    # Bytes of a small draw are frozen so that a change of the generator is noticed.
    wl = synth.WORKLOADS["fullbatch_tiny_fp32"]
    x = synth.make_inputs(wl)
    h = hashlib.sha256(b"".join(t.tobytes() for t in (x.q, x.k, x.v, x.w0))).hexdigest()
    golden = open(__file__.replace("test_synth.py", "golden/synth_fullbatch_tiny_fp32.sha256")).read().split()[0]
    assert h == golden
