"""The seeded input generator: published SplitMix64 outputs, slicing,
determinism and the distribution of its normals."""
import numpy as np

import synth


def test_splitmix64_reference_outputs():
    # First outputs of SplitMix64 seeded with 1234567, as printed with the
    # generator's public reference implementation (Vigna, splitmix64.c).
    ref = [6457827717110365317, 3203168211198807973, 9817491932198370423,
           4593380528125082431, 16408922859458223821]
    assert [synth.splitmix64_at(1234567, n) for n in range(5)] == ref


def test_slices_agree_with_whole_tensor():
    full = synth.normal_bf16((3, 4, 10, 8), 5, 2)
    part = synth.normal_bf16_rows((3, 4, 10, 8), 5, 2, (2, 1))
    np.testing.assert_array_equal(part, full[2, 1])
    np.testing.assert_array_equal(synth.normal_bf16((3, 4, 10, 8), 5, 2), full)
    assert not np.array_equal(synth.normal_bf16((3, 4, 10, 8), 5, 3), full)


def test_normal_moments_and_bf16_rounding():
    f32 = synth.normal_f32((200000,), 9, 1)
    assert abs(f32.mean()) < 0.01 and abs(f32.std() - 1) < 0.01
    bits = synth.normal_bf16((200000,), 9, 1)
    np.testing.assert_array_equal(bits, synth.round_bf16(f32))
    # RNE ties: 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125 -> even (1.0)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, np.inf], dtype=np.float32)
    np.testing.assert_array_equal(synth.round_bf16(x), np.array([0x3F80, 0x3F82, 0xC020, 0x7F80], dtype=np.uint16))
    w = synth.normal_f32((100000,), 9, 7, 0.02)
    assert abs(w.std() - 0.02) < 0.001


def test_uniform_lengths_inclusive_range():
    L = synth.uniform_i32(100000, 1024, 32768, 3, 4)
    assert L.min() >= 1024 and L.max() <= 32768
    assert L.min() < 1100 and L.max() > 32700
    assert abs(L.mean() - (1024 + 32768) / 2) < 200
