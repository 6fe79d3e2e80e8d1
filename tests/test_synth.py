"""The shared seeded input generator (CPU side)."""
import numpy as np

import synth


def test_splitmix64_published_vector():
    # Vigna's splitmix64 seeded with 1234567: its first three outputs.
    s = np.uint64(1234567)
    g = np.uint64(0x9E3779B97F4A7C15)
    with np.errstate(over="ignore"):
        out = [int(synth._mix(s + np.uint64(i) * g)) for i in range(1, 4)]
    assert out == [6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_int9_values_and_balance():
    v = synth.bf16_to_f32(synth.gen_flat(0, 7, synth.INT9, 90000))
    assert set(np.unique(v)) == set(range(-4, 5))
    counts = np.bincount((v + 4).astype(int))
    assert counts.min() > 9000


def test_normal_table_is_a_quantile_table():
    t = synth.bf16_to_f32(synth.ntab())
    assert np.all(np.diff(t) >= 0)
    assert np.array_equal(t, -t[::-1])
    v = synth.bf16_to_f32(synth.gen_flat(0, 9, synth.NORMAL, 200000))
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01


def test_rows_do_not_depend_on_buffer_shape():
    a = synth.gen_rows(3, 11, synth.NORMAL, [0, 5], np.arange(10), 512)
    b = synth.gen_rows(3, 11, synth.NORMAL, [5], np.arange(4, 8), 512)
    assert np.array_equal(a[1, 4:8], b[0])
    assert not np.array_equal(a[0], a[1])


def test_c_generator_equals_numpy_definition():
    rows = np.array([0, 1, 5, 1 << 20, (1 << 24) - 1])
    for kind in (synth.INT9, synth.NORMAL):
        a = synth.gen_rows(7, 123, kind, [0, 3, 15], rows, 64)
        b = synth.gen_rows_numpy(7, 123, kind, [0, 3, 15], rows, 64)
        assert np.array_equal(a, b)
